"""GPU parity for per-token FP8 (OCP E4M3 codes, fp32 per-token scales) on
inputs where every value and score is exact: integer codes and power-of-two
scales, so indices and scores must equal the oracle bit for bit on every
selection path, and replay must equal the selected scores.  This pins the
scaled formats' epilogue, which adds the linear part of the weighted ReLU as
one more MFMA row block: its E4M3 pieces of v = sum_h (w_h / 2) q_h carry v
exactly here, and any mistake in their construction or in the per-token
scales changes a score."""
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


def _fp8_exact(L, n, H, k, seed):
    """Integer values in E4M3 codes; q_scale and k_scale drawn from 2^-1, 2^0, 2^1."""
    base = datagen.make_custom("fp8i", L, n, H, 128, k, dtype="bf16", dist="int", seed=seed)
    qv = (base.q.astype(np.uint32) << 16).view(np.float32)
    kv = (base.k_.astype(np.uint32) << 16).view(np.float32)
    rng = np.random.default_rng(seed + 1)
    qs = np.exp2(rng.integers(-1, 2, size=n)).astype(np.float32)
    ks = np.exp2(rng.integers(-1, 2, size=L)).astype(np.float32)
    return datagen.Inputs("fp8i", L, n, H, 128, k, "fp8", datagen.f32_to_e4m3(qv),
                          datagen.f32_to_e4m3(kv), base.w, qs, ks)


@pytest.mark.parametrize("H,seed", [(8, 95), (64, 96)])
def test_fp8_exact_every_path_bit_exact(hk, H, seed):
    say(f"fp8: exact problem L=3000 n=200 H={H} d=128 k=256")
    inp = _fp8_exact(3000, 200, H, 256, seed)
    ref_idx, ref_val = oracle.select(inp)
    dv = to_device(inp)
    kw = dict(q_scale=dv["q_scale"], k_scale=dv["k_scale"], fmt="fp8")
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


def test_fp8_exact_one_split_partial_last_group(hk):
    """8,190 queries fill 512 groups of 16, so the fused kernel runs one key
    split per query (each wave the only writer of its candidates) and the
    last group's last wave has no query; exact FP8 values: the selection
    equals the row baseline on all queries and the oracle on 96 of them."""
    L, n, H, k = 12000, 8190, 64, 256
    say(f"fp8: exact problem, one split, L={L} n={n} H={H} d=128 k={k}")
    inp = _fp8_exact(L, n, H, k, 97)
    dv = to_device(inp)
    kw = dict(q_scale=dv["q_scale"], k_scale=dv["k_scale"], fmt="fp8")
    idx, sc, st = hk.select(dv["q"], dv["k"], dv["w"], k, with_stats=True, **kw)
    bidx, bsc = hk.baseline_select(dv["q"], dv["k"], dv["w"], k, **kw)
    torch.cuda.synchronize()
    assert st["n_failed"] == 0, st
    assert np.array_equal(_np(idx), _np(bidx))
    assert np.array_equal(_np(sc).view(np.uint32), _np(bsc).view(np.uint32))
    qs = np.unique(np.concatenate([np.arange(n - 48, n),
                                   np.random.default_rng(97).choice(n - 48, 48, replace=False)]))
    ref_idx, ref_val = oracle.select(inp, queries=qs)
    for j, i in enumerate(qs):
        assert np.array_equal(_np(idx)[i], ref_idx[j]), f"query {i}"
        assert np.array_equal(_np(sc)[i], ref_val[j].astype(np.float32)), f"query {i}"
