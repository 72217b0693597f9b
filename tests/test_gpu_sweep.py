"""Seeded sweep of small problems against the oracle, bit for bit.

Each case draws its shape from a fixed seed: H from 1 to 64, d from {64, 128}
(bf16) or 128 (per-token FP8 with power-of-two scales, MXFP8, MXFP4), key
counts with ragged tiles, query counts with ragged groups, k from 1 up to
2,048 (also above the context), and for some cases sequences packed into one
key buffer with shuffled query positions.  Values are integers, exact in
every format, so every selection path must return the oracle's indices and
scores exactly: the candidate path, recovery of a few overflowing queries,
the full rescore, the asynchronous call, the score-table baseline; replay
must return the selected scores, and the backward at the selected entries
(integer upstream gradients) the oracle's dq, dw and dk exactly."""
import numpy as np
import pytest
import torch

import datagen
import oracle
from gpu_util import assert_exact, say, to_device

pytestmark = pytest.mark.gpu

N_CASES = 18


def _as_fp8(base, rng):
    """The same integer values as OCP E4M3 codes with per-token scales drawn
    from 2^-1, 2^0, 2^1 (every product and sum stays exact)."""
    qv = (base.q.astype(np.uint32) << 16).view(np.float32)
    kv = (base.k_.astype(np.uint32) << 16).view(np.float32)
    qs = np.exp2(rng.integers(-1, 2, size=base.n)).astype(np.float32)
    ks = np.exp2(rng.integers(-1, 2, size=base.L)).astype(np.float32)
    inp = datagen.Inputs("sweep", base.L, base.n, base.H, base.d, base.k, "fp8",
                         datagen.f32_to_e4m3(qv), datagen.f32_to_e4m3(kv), base.w, qs, ks)
    inp.q_pos, inp.q_first = base.q_pos, base.q_first
    return inp


def _case(i):
    rng = np.random.default_rng(1000 + i)
    fmt = "fp8" if i >= 14 else ["bf16", "bf16", "bf16", "mxfp8", "mxfp4"][i % 5]
    H = int(rng.integers(1, 65))
    d = int(rng.choice([64, 128])) if fmt == "bf16" else 128
    draw = "bf16" if fmt == "fp8" else fmt  # FP8 codes are made from the bf16 draw below
    packed = i % 3 == 2
    if packed:
        lens = [int(x) for x in rng.integers(40, 1500, size=int(rng.integers(2, 5)))]
        chunks = []
        for s, ln in enumerate(lens):
            cnt = int(rng.integers(1, min(ln, 40) + 1))
            chunks.append((s, int(rng.integers(0, ln - cnt + 1)), cnt))
        L = sum(lens)
    else:
        L = int(rng.integers(16, 4001))
        n = int(rng.integers(1, min(L, 160) + 1))
    kind = i % 4
    k_hi = min(2048, L + 50)
    k = [1, int(rng.integers(2, 65)), int(rng.integers(65, k_hi + 1)) if k_hi > 65 else 64,
         k_hi][kind]
    seed = 2000 + i
    if packed:
        inp = datagen.make_packed("sweep", lens, chunks, H=H, d=d, k=k, dtype=draw, dist="int",
                                  seed=seed)
    else:
        inp = datagen.make_custom("sweep", L, n, H, d, k, dtype=draw, dist="int", seed=seed)
    return _as_fp8(inp, rng) if fmt == "fp8" else inp


@pytest.fixture(scope="module")
def hk():
    import exact_top_token_amd as m
    m.load_library()
    return m


def _np(t):
    return t.cpu().numpy()


@pytest.mark.parametrize("i", range(N_CASES))
def test_sweep_case_every_path_bit_exact(hk, i):
    inp = _case(i)
    packed = inp.q_pos is not None
    say(f"sweep {i}: {inp.dtype} L={inp.L} n={inp.n} H={inp.H} d={inp.d} k={inp.k} "
        f"packed={packed}")
    dv = to_device(inp)
    kw = {}
    if inp.dtype != "bf16":
        kw = dict(q_scale=dv["q_scale"], k_scale=dv["k_scale"], fmt=inp.dtype)
    if packed:
        kw["q_pos"] = torch.from_numpy(np.ascontiguousarray(inp.q_pos, dtype=np.int32)).cuda()
        kw["q_first"] = torch.from_numpy(np.ascontiguousarray(inp.q_first, dtype=np.int32)).cuda()
    ref_idx, ref_val = oracle.select(inp)
    q, k, w = dv["q"], dv["k"], dv["w"]

    idx, sc, st = hk.select(q, k, w, inp.k, with_stats=True, **kw)
    torch.cuda.synchronize()
    assert_exact(inp, range(inp.n), _np(idx), _np(sc), ref_idx, ref_val)
    bits = (_np(idx), _np(sc).view(np.uint32))

    def same(res, what):
        torch.cuda.synchronize()
        assert np.array_equal(_np(res[0]), bits[0]), what
        assert np.array_equal(_np(res[1]).view(np.uint32), bits[1]), what

    # a candidate cap below the largest counts sends those queries to recovery
    dec = oracle.Decoded(inp)
    rows = [oracle.score_row(dec, j) for j in range(inp.n)]
    cnts = sorted(p["cnt"] for p in oracle.predict_paths(rows, inp.k, inp.L,
                                                          cap=6 * inp.k)["per_query"])
    cap = max(1, cnts[-min(len(cnts), 4)] - 1)
    r = hk.select(q, k, w, inp.k, params=dict(cap=cap, rows_chunk=3), with_stats=True, **kw)
    say(f"sweep {i}: cap {cap}: {r[2]['n_failed']} failed, path {r[2]['path']}")
    same(r, "recovery")
    same(hk.select(q, k, w, inp.k, params=dict(force_path=hk.PATH_ROWS_ALL), **kw), "rows")
    same(hk.baseline_select(q, k, w, inp.k, **kw), "baseline")

    ws = torch.empty(hk.select_workspace_bytes(q, k, w, inp.k, params=dict(cap=cap),
                                               q_pos=kw.get("q_pos"), q_first=kw.get("q_first"),
                                               fmt=kw.get("fmt")),
                     dtype=torch.uint8, device="cuda")
    out = (torch.empty_like(idx), torch.empty_like(sc))
    status = torch.zeros(hk.ASYNC_STATUS_WORDS, dtype=torch.int32, device="cuda")
    hk.select_async(q, k, w, inp.k, workspace=ws, out=out, status=status, params=dict(cap=cap),
                    **kw)
    torch.cuda.synchronize()
    if _np(status)[0] == 0:
        same(out, "async")
    else:  # more failures than max_recover: the passing queries' rows are final
        assert _np(status)[1] > 64

    rep = hk.replay(q, k, w, idx, **{x: kw[x] for x in ("q_scale", "k_scale", "fmt") if x in kw})
    torch.cuda.synchronize()
    ok = bits[0] >= 0
    assert np.array_equal(_np(rep).view(np.uint32)[ok], bits[1][ok])
    assert np.all(np.isneginf(_np(rep)[~ok]))

    # the backward at the selected entries, integer upstream gradients: exact
    g = np.random.default_rng(3000 + i).integers(-3, 4, size=bits[0].shape).astype(np.float32)
    fk = {x: kw[x] for x in ("q_scale", "k_scale", "fmt") if x in kw}
    got = hk.backward(q, k, w, idx, torch.from_numpy(g).cuda(), **fk)
    torch.cuda.synchronize()
    ref = oracle.backward(inp, bits[0], g)
    for name in ("dq", "dw", "dk"):
        assert np.array_equal(_np(got[name]).astype(np.float64), ref[name]), name
