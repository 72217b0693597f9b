"""GPU parity of the indexer backward at the replayed entries (hytopk_backward)
against the oracle's fp64 chain rule.

* Integer-valued inputs and integer upstream gradients: every product and sum
  is an integer below 2^24, so dq, dw and dk must equal the oracle bit for
  bit (Tiny and ragged shapes: heads not a multiple of 16, k not a multiple of
  the 32-key tile, contexts shorter than k, out-of-range indices as padding).
* Float inputs: per element, |gpu - oracle| <= 1e-4 * A + E, where A is the
  oracle's sum of the absolute values of the terms (the scale a rounding
  bound is stated against: the kernels carry 16 significant bits in every
  bf16-split factor and accumulate in fp32) and E the absolute contribution
  of terms whose ReLU decision lies within 1e-5 * sum_i |q_i k_i| of zero,
  where the kernel's fp32 pre-activation may take the other branch.  dq and
  dw are checked on a query subset; dk on sampled keys (the most selected
  ones and random ones), each recomputed by the oracle from exactly the
  entries that selected it.  Euler's identity <w,dw> = <q,dq> = <k,dk> =
  sum dI * I checks the whole output at once.
"""
import numpy as np
import pytest
import torch

import datagen
import oracle
from gpu_util import say, to_device

pytestmark = pytest.mark.gpu

AMB = 1e-5
REL = 1e-4


@pytest.fixture(scope="module")
def hk():
    import exact_top_token_amd as m
    m.load_library()
    return m


def _grad(shape, seed, integer):
    rng = np.random.default_rng(seed)
    if integer:
        return rng.integers(-3, 4, size=shape).astype(np.float32)
    return rng.standard_normal(shape).astype(np.float32)


def _fmt_kw(inp, dev):
    """Scales and format of a scaled-format problem (empty for bf16)."""
    if inp.dtype == "bf16":
        return {}
    return dict(q_scale=dev["q_scale"], k_scale=dev["k_scale"], fmt=inp.dtype)


def _run(hk, dev, idx, g, want=("dq", "dw", "dk"), kw=None):
    idx_t = torch.from_numpy(np.ascontiguousarray(idx, dtype=np.int32)).cuda()
    g_t = torch.from_numpy(np.ascontiguousarray(g, dtype=np.float32)).cuda()
    res = hk.backward(dev["q"], dev["k"], dev["w"], idx_t, g_t, want=want, **(kw or {}))
    torch.cuda.synchronize()
    return {k: v.cpu().numpy() for k, v in res.items()}


def _assert_equal(name, got, ref):
    if not np.array_equal(got.astype(np.float64), ref):
        bad = np.argwhere(got.astype(np.float64) != ref)
        i = tuple(bad[0])
        raise AssertionError(f"{name}: {len(bad)} mismatches, first at {i}: gpu {got[i]} oracle {ref[i]}")


def _assert_close(name, got, ref, scale, amb):
    tol = REL * scale + amb + 1e-30
    err = np.abs(got.astype(np.float64) - ref)
    if np.any(err > tol):
        i = np.unravel_index(np.argmax(err - tol), err.shape)
        raise AssertionError(f"{name}: |err| {err[i]:.3e} > tol {tol[i]:.3e} at {i} "
                             f"(gpu {got[i]!r}, oracle {ref[i]!r})")


def _integer_case(hk, inp, seed, corrupt=False):
    dev = to_device(inp)
    kw = _fmt_kw(inp, dev)
    idx_t, _ = hk.select(dev["q"], dev["k"], dev["w"], inp.k, **kw)
    idx = idx_t.cpu().numpy()
    if corrupt:  # out-of-range indices are padding
        rng = np.random.default_rng(seed)
        rows = rng.choice(inp.n, size=min(inp.n, 5), replace=False)
        idx[rows, 0] = inp.L + 3
        idx[rows, -1] = -7
    g = _grad(idx.shape, seed, True)
    got = _run(hk, dev, idx, g, kw=kw)
    ref = oracle.backward(inp, idx, g)
    for name in ("dq", "dw", "dk"):
        _assert_equal(name, got[name], ref[name])
    return dev, idx, g, got


def test_tiny_backward_bit_exact(hk):
    inp = datagen.make("tiny")
    say("backward tiny: L=4096 n=256 H=4 d=64 k=256, integer dI")
    _integer_case(hk, inp, 31)


@pytest.mark.parametrize("L,n,H,d,k,seed", [
    (300, 300, 64, 128, 64, 41),     # every query is a tile-multiple k, contexts 1..300
    (200, 200, 20, 64, 150, 42),     # H not a multiple of 16; ctx < k pads early queries
    (1000, 37, 64, 128, 100, 43),    # k not a multiple of 32
    (5000, 130, 8, 128, 1, 44),      # k = 1
    (4100, 33, 64, 64, 2048, 45),    # the largest k, d = 64
])
def test_ragged_backward_bit_exact(hk, L, n, H, d, k, seed):
    say(f"backward ragged: L={L} n={n} H={H} d={d} k={k}")
    inp = datagen.make_custom(f"bw{seed}", L, n, H, d, k, dist="int", seed=seed)
    _integer_case(hk, inp, seed, corrupt=True)


def test_backward_reproducible_and_partial_outputs(hk):
    say("backward: repeated calls bitwise equal; dq/dw without dk, dk alone")
    inp = datagen.make_custom("bwrep", 6000, 300, 64, 128, 256, dist="normal", seed=46)
    dev = to_device(inp)
    idx_t, _ = hk.select(dev["q"], dev["k"], dev["w"], inp.k)
    idx = idx_t.cpu().numpy()
    g = _grad(idx.shape, 46, False)
    a = _run(hk, dev, idx, g)
    b = _run(hk, dev, idx, g)
    c = _run(hk, dev, idx, g, want=("dq", "dw"))
    e = _run(hk, dev, idx, g, want=("dk",))
    for name in ("dq", "dw", "dk"):
        assert np.array_equal(a[name], b[name]), name
    assert np.array_equal(a["dq"], c["dq"]) and np.array_equal(a["dw"], c["dw"])
    assert np.array_equal(a["dk"], e["dk"])


def _float_check(hk, inp, seed, nsub):
    dev = to_device(inp)
    kw = _fmt_kw(inp, dev)
    idx_t, sc_t = hk.select(dev["q"], dev["k"], dev["w"], inp.k, **kw)
    idx, score = idx_t.cpu().numpy(), sc_t.cpu().numpy()
    g = _grad(idx.shape, seed, False)
    got = _run(hk, dev, idx, g, kw=kw)
    # dq, dw on a query subset (first and last query included)
    qs = datagen.subset_queries(inp.n, nsub, seed=7)
    ref = oracle.backward(inp, idx[qs], g[qs], qs, amb=AMB)
    _assert_close("dq", got["dq"][qs], ref["dq"], ref["dq_abs"], ref["dq_amb"])
    _assert_close("dw", got["dw"][qs], ref["dw"], ref["dw_abs"], 0.0)
    # dk on sampled keys, each from every entry that selected it
    valid = idx[idx >= 0]
    cnt = np.bincount(valid, minlength=inp.L)
    rng = np.random.default_rng(seed)
    popular = np.argsort(-cnt, kind="stable")[:8]
    chosen = np.unique(np.concatenate([popular, rng.choice(np.nonzero(cnt)[0], size=24, replace=False)]))
    hit = np.isin(idx, chosen)
    rows = np.nonzero(hit.any(axis=1))[0]
    sub_idx = np.where(hit[rows], idx[rows], -1)
    refk = oracle.backward(inp, sub_idx, g[rows], rows, amb=AMB)
    _assert_close("dk", got["dk"][chosen], refk["dk"][chosen], refk["dk_abs"][chosen],
                  refk["dk_amb"][chosen])
    assert np.all(got["dk"][cnt == 0] == 0.0), "unselected keys must get zero"
    # Euler's identity over the whole output, against sum dI * score (fp32 sums)
    dec = oracle.Decoded(inp)
    ok = idx >= 0
    total = float(np.sum(g[ok].astype(np.float64) * score[ok]))
    scale = float(np.sum(np.abs(g[ok].astype(np.float64) * score[ok])))
    w = inp.w.astype(np.float64)
    lhs_w = float(np.sum(w * got["dw"]))
    lhs_k = float(np.sum(dec.keys * got["dk"]))
    lhs_q = 0.0
    for i in range(0, inp.n, 256):
        qq = np.stack([dec.query(j)[0] for j in range(i, min(inp.n, i + 256))])
        lhs_q += float(np.sum(qq * got["dq"][i:i + 256]))
    for name, lhs in (("w", lhs_w), ("q", lhs_q), ("k", lhs_k)):
        assert abs(lhs - total) <= 1e-4 * scale, (name, lhs, total)


def test_mid_backward_float(hk):
    say("backward mid: L=131072 n=2048 H=64 d=128 k=2048 (one chunk)")
    _float_check(hk, datagen.make("mid"), 51, 64)


def test_glm1m_backward_float(hk):
    say("backward glm1m: L=1048576 n=8192 H=64 d=128 k=2048 (one 8 GiB chunk)")
    _float_check(hk, datagen.make("glm1m"), 52, 32)


# ----------------------------------------------------------- scaled formats

@pytest.mark.parametrize("fmt,H,seed", [("mxfp8", 64, 61), ("mxfp4", 64, 62), ("mxfp4", 8, 63)])
def test_mx_backward_equals_bf16_on_the_same_values(hk, fmt, H, seed):
    """MX integer problems decode to the same values as the bf16 problem of the
    same seed; their backward (with respect to the decoded values) must match
    the oracle and the bf16 backward bit for bit."""
    say(f"backward {fmt}: integer problem L=3000 n=200 H={H} d=128 k=256")
    inp = datagen.make_custom("bwmx", 3000, 200, H, 128, 256, dtype=fmt, dist="int", seed=seed)
    _, idx, g, got = _integer_case(hk, inp, seed, corrupt=True)
    bf = datagen.make_custom("bwbf", 3000, 200, H, 128, 256, dtype="bf16", dist="int", seed=seed)
    ref = _run(hk, to_device(bf), idx, g)
    for name in ("dq", "dw", "dk"):
        assert np.array_equal(got[name], ref[name]), name


@pytest.mark.parametrize("H,k,seed", [(8, 256, 64), (64, 256, 65), (20, 100, 68)])
def test_fp8_backward_exact(hk, H, k, seed):
    """Per-token FP8 with integer codes and power-of-two scales: the scales
    enter as factors (dI k_scale for dq and dw, w q_scale for dk, q_scale on
    dw); every value stays exact, so the gradients equal the oracle's bit for
    bit."""
    from test_gpu_fp8 import _fp8_exact
    say(f"backward fp8: exact problem L=3000 n=200 H={H} d=128 k={k}")
    _integer_case(hk, _fp8_exact(3000, 200, H, k, seed), seed, corrupt=True)


@pytest.mark.parametrize("fmt", ["fp8", "mxfp8", "mxfp4"])
def test_scaled_backward_float(hk, fmt):
    say(f"backward {fmt}: Gaussian problem L=20000 n=256 H=64 d=128 k=512")
    inp = datagen.make_custom("bwsc", 20000, 256, 64, 128, 512, dtype=fmt, dist="normal", seed=66)
    _float_check(hk, inp, 67, 32)


@pytest.mark.parametrize("fmt", ["fp8", "mxfp4"])
def test_scaled_backward_partial_outputs(hk, fmt):
    """dq / dw without dk (the scaled formats still need the workspace for
    their bf16 copies of q and k) and dk alone give the bits of the full call."""
    say(f"backward {fmt}: partial outputs")
    inp = datagen.make_custom("bwpart", 4000, 96, 64, 128, 256, dtype=fmt, dist="normal", seed=69)
    dev = to_device(inp)
    kw = _fmt_kw(inp, dev)
    idx_t, _ = hk.select(dev["q"], dev["k"], dev["w"], inp.k, **kw)
    idx = idx_t.cpu().numpy()
    g = _grad(idx.shape, 69, False)
    full = _run(hk, dev, idx, g, kw=kw)
    part = _run(hk, dev, idx, g, want=("dq", "dw"), kw=kw)
    only_k = _run(hk, dev, idx, g, want=("dk",), kw=kw)
    assert np.array_equal(full["dq"], part["dq"]) and np.array_equal(full["dw"], part["dw"])
    assert np.array_equal(full["dk"], only_k["dk"])
