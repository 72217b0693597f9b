"""GPU parity for the OCP MX block-scaled formats (MXFP8: E4M3 elements,
MXFP4: E2M1 elements, one E8M0 scale per 32 elements) on integer-valued
inputs: every value is exact after decoding and every score an integer below
2^24, so indices and scores must equal the oracle bit for bit on every
selection path, replay must equal the selected scores, and the MX problem
must return exactly what the bf16 problem with the same values returns."""
import numpy as np
import pytest
import torch

import datagen
import oracle
from gpu_util import assert_exact, say, to_device

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def hk():
    import exact_top_token_amd as m
    m.load_library()
    return m


def _np(t):
    return t.cpu().numpy()


@pytest.mark.parametrize("fmt", ["mxfp8", "mxfp4"])
@pytest.mark.parametrize("H,seed", [(8, 91), (64, 92)])
def test_mx_integer_every_path_bit_exact(hk, fmt, H, seed):
    say(f"mx: {fmt} integer problem L=3000 n=200 H={H} d=128 k=256")
    inp = datagen.make_custom("mxi", 3000, 200, H, 128, 256, dtype=fmt, dist="int", seed=seed)
    ref_idx, ref_val = oracle.select(inp)
    dv = to_device(inp)
    kw = dict(q_scale=dv["q_scale"], k_scale=dv["k_scale"], fmt=fmt)
    idx, sc, st = hk.select(dv["q"], dv["k"], dv["w"], inp.k, with_stats=True, **kw)
    torch.cuda.synchronize()
    assert_exact(inp, range(inp.n), _np(idx), _np(sc), ref_idx, ref_val)
    bits = (_np(idx), _np(sc).view(np.uint32))
    for params in (dict(force_path=1), dict(cap=inp.k, max_recover=8)):
        i2, s2 = hk.select(dv["q"], dv["k"], dv["w"], inp.k, params=params, **kw)
        torch.cuda.synchronize()
        assert np.array_equal(_np(i2), bits[0]) and np.array_equal(_np(s2).view(np.uint32), bits[1])
    rep = hk.replay(dv["q"], dv["k"], dv["w"], idx, **kw)
    bi, bs = hk.baseline_select(dv["q"], dv["k"], dv["w"], inp.k, **kw)
    torch.cuda.synchronize()
    assert np.array_equal(_np(rep).view(np.uint32), bits[1])
    assert np.array_equal(_np(bi), bits[0]) and np.array_equal(_np(bs).view(np.uint32), bits[1])
    # the same integer values stored as bf16 select the same bits
    bf = datagen.make_custom("bfi", 3000, 200, H, 128, 256, dtype="bf16", dist="int", seed=seed)
    db = to_device(bf)
    ib, sb = hk.select(db["q"], db["k"], db["w"], bf.k)
    torch.cuda.synchronize()
    assert np.array_equal(_np(ib), bits[0]) and np.array_equal(_np(sb).view(np.uint32), bits[1])


def test_mx_rejects_missing_scales_and_other_head_dims(hk):
    inp = datagen.make_custom("mxe", 600, 40, 4, 128, 32, dtype="mxfp4", dist="int", seed=93)
    dv = to_device(inp)
    # the binding refuses missing scales (the library's own -1 for them is a CPU ABI test)
    with pytest.raises(ValueError):
        hk.select(dv["q"], dv["k"], dv["w"], inp.k, fmt="mxfp4")
    # d = 64 (32 bytes of E2M1 per row, two scale bytes) is not supported for the MX formats
    q64, k64 = dv["q"][:, :, :32].contiguous(), dv["k"][:, :32].contiguous()
    qs64, ks64 = dv["q_scale"][:, :, :2].contiguous(), dv["k_scale"][:, :2].contiguous()
    with pytest.raises(hk.HytopkError) as e:
        hk.select(q64, k64, dv["w"], inp.k, q_scale=qs64, k_scale=ks64, fmt="mxfp4")
    assert e.value.status == -2


@pytest.mark.parametrize("fmt", ["mxfp8", "mxfp4"])
def test_mx_gaussian_blocks_follow_their_scales(hk, fmt):
    """Gaussian values give every 32-element block its own E8M0 scale, so a
    scale applied to the wrong elements shows up here (integer inputs give
    nearly every block the same scale and cannot)."""
    from gpu_util import assert_float_row
    say(f"mx: {fmt} Gaussian problem L=20000 n=64 H=64 d=128 k=512")
    inp = datagen.make_custom("mxg", 20000, 64, 64, 128, 512, dtype=fmt, dist="normal", seed=94)
    # block maxima of Gaussian values span a few binades: several distinct scales
    assert np.unique(inp.k_scale).size >= 3 and np.unique(inp.q_scale).size >= 3
    dv = to_device(inp)
    kw = dict(q_scale=dv["q_scale"], k_scale=dv["k_scale"], fmt=fmt)
    idx, sc = hk.select(dv["q"], dv["k"], dv["w"], inp.k, **kw)
    rep = hk.replay(dv["q"], dv["k"], dv["w"], idx, **kw)
    torch.cuda.synchronize()
    idx_n, sc_n, rep_n = _np(idx), _np(sc), _np(rep)
    dec = oracle.Decoded(inp)
    for i in range(inp.n):
        assert_float_row(inp.q_start + i, inp.k, oracle.score_row(dec, i), idx_n[i], sc_n[i],
                         f"{fmt} q{i}", rep_n[i])
    assert np.array_equal(rep_n.view(np.uint32), sc_n.view(np.uint32))
