"""GPU parity for per-query key ranges (``hytopk_problem.q_pos`` /
``q_first``): sequences packed back to back in one key buffer, queries in
shuffled order at arbitrary positions (a context-parallel zigzag shard),
contexts shorter than k, and empty contexts.

Integer-valued inputs are compared with the oracle bit for bit on every
selection path; the Gaussian packed problem uses the float comparators of
``gpu_util`` with the query's first key.
"""
import numpy as np
import pytest
import torch

import datagen
import oracle
from gpu_util import assert_exact, assert_float_row, say, to_device

pytestmark = pytest.mark.gpu

SEQS = [700, 300, 1100, 500]
CHUNKS = [(0, 600, 40), (1, 0, 5), (1, 250, 50), (2, 800, 60), (3, 250, 30)]


@pytest.fixture(scope="module")
def hk():
    import exact_top_token_amd as m
    m.load_library()
    return m


def _ranges(inp):
    pos = torch.from_numpy(np.ascontiguousarray(inp.q_pos, dtype=np.int32)).cuda()
    first = None
    if inp.q_first is not None:
        first = torch.from_numpy(np.ascontiguousarray(inp.q_first, dtype=np.int32)).cuda()
    return dict(q_pos=pos, q_first=first)


def _np(t):
    return t.cpu().numpy()


def _counts(inp):
    dec = oracle.Decoded(inp)
    rows = [oracle.score_row(dec, i) for i in range(inp.n)]
    return rows, oracle.predict_paths(rows, inp.k, inp.L, cap=6 * inp.k)


def test_packed_integer_every_path_bit_exact(hk):
    say("ranges: packed integer problem, L=2600 in 4 sequences, n=185 shuffled, H=4 d=64 k=256")
    inp = datagen.make_packed("pk", SEQS, CHUNKS, H=4, d=64, k=256, dist="int", seed=71)
    dv, rg = to_device(inp), _ranges(inp)
    ref_idx, ref_val = oracle.select(inp)
    rows, pred = _counts(inp)
    idx, sc, st = hk.select(dv["q"], dv["k"], dv["w"], inp.k, with_stats=True, **rg)
    torch.cuda.synchronize()
    assert_exact(inp, range(inp.n), _np(idx), _np(sc), ref_idx, ref_val)
    # integer scores: the GPU's candidate counts follow the threshold model exactly
    assert st["cand_total"] == sum(p["cnt"] for p in pred["per_query"])
    assert st["n_failed"] == pred["n_failed"] == 0
    base_bits = (_np(idx), _np(sc).view(np.uint32))

    def same(res, what):
        i, s = res[0], res[1]
        torch.cuda.synchronize()
        assert np.array_equal(_np(i), base_bits[0]), what
        assert np.array_equal(_np(s).view(np.uint32), base_bits[1]), what

    same(hk.select(dv["q"], dv["k"], dv["w"], inp.k, params=dict(force_path=1), **rg), "rows")
    cnts = sorted(p["cnt"] for p in pred["per_query"])
    cap = max(inp.k, cnts[-10] - 1)  # about nine queries overflow: recovery
    r = hk.select(dv["q"], dv["k"], dv["w"], inp.k, params=dict(cap=cap), with_stats=True, **rg)
    assert 1 <= r[2]["n_failed"] <= 64 and r[2]["path"] == 0
    same(r, "recovery")
    r = hk.select(dv["q"], dv["k"], dv["w"], inp.k, params=dict(cap=cap, max_recover=1),
                  with_stats=True, **rg)
    assert r[2]["path"] == 1
    same(r, "full rescore")
    same(hk.baseline_select(dv["q"], dv["k"], dv["w"], inp.k, **rg), "baseline")
    rep = hk.replay(dv["q"], dv["k"], dv["w"], idx)
    torch.cuda.synchronize()
    assert np.array_equal(_np(rep).view(np.uint32), base_bits[1])


def test_zigzag_positions_without_first_key(hk):
    say("ranges: one sequence L=4096, queries at two shuffled runs (zigzag shard), q_pos only")
    inp = datagen.make_custom("zz", 4096, 128, 4, 64, 256, dist="int", seed=72)
    pos = np.concatenate([np.arange(1024, 1088), np.arange(3968, 4032)]).astype(np.int32)
    inp.q_pos = np.random.default_rng(72).permutation(pos).astype(np.int32)
    dv, rg = to_device(inp), _ranges(inp)
    ref_idx, ref_val = oracle.select(inp)
    idx, sc = hk.select(dv["q"], dv["k"], dv["w"], inp.k, **rg)
    torch.cuda.synchronize()
    assert_exact(inp, range(inp.n), _np(idx), _np(sc), ref_idx, ref_val)


def test_empty_and_clamped_contexts(hk):
    say("ranges: empty contexts give padding; positions past the buffer clamp to its end")
    inp = datagen.make_packed("pke", SEQS, CHUNKS, H=4, d=64, k=256, dist="int", seed=73)
    empty = np.array([3, 50, 101])
    inp.q_first = inp.q_first.copy()
    inp.q_first[empty] = inp.q_pos[empty] + 1
    dv, rg = to_device(inp), _ranges(inp)
    ref_idx, ref_val = oracle.select(inp)
    assert np.all(ref_idx[empty] == -1)
    for params in (None, dict(force_path=1)):
        idx, sc = hk.select(dv["q"], dv["k"], dv["w"], inp.k, params=params, **rg)
        torch.cuda.synchronize()
        assert_exact(inp, range(inp.n), _np(idx), _np(sc), ref_idx, ref_val)
    # a position past the end of the buffer behaves as the last key
    moved = np.array([7, 90])
    pos_a, pos_b = inp.q_pos.copy(), inp.q_pos.copy()
    pos_a[moved] = inp.L - 1
    pos_b[moved] = inp.L + 5
    a = hk.select(dv["q"], dv["k"], dv["w"], inp.k, **dict(rg, q_pos=torch.from_numpy(pos_a).cuda()))
    b = hk.select(dv["q"], dv["k"], dv["w"], inp.k, **dict(rg, q_pos=torch.from_numpy(pos_b).cuda()))
    torch.cuda.synchronize()
    assert torch.equal(a[0], b[0]) and torch.equal(a[1].view(torch.int32), b[1].view(torch.int32))


def test_packed_float(hk):
    say("ranges: packed Gaussian problem, L=131072 in 3 sequences, n=1820, H=64 d=128 k=2048")
    inp = datagen.make_packed("pkf", [60000, 40000, 31072],
                              [(0, 59000, 300), (1, 39500, 500), (2, 30000, 1000), (0, 100, 20)],
                              H=64, d=128, k=2048, dist="normal", seed=74)
    dv, rg = to_device(inp), _ranges(inp)
    idx, sc, st = hk.select(dv["q"], dv["k"], dv["w"], inp.k, with_stats=True, **rg)
    rep = hk.replay(dv["q"], dv["k"], dv["w"], idx)
    torch.cuda.synchronize()
    idx_n, sc_n, rep_n = _np(idx), _np(sc), _np(rep)
    assert st["n_failed"] == 0, st
    short = np.nonzero(inp.q_pos - inp.q_first + 1 < inp.k)[0]
    qs = datagen.subset_queries(inp.n, 48, seed=7, must=tuple(short[:8].tolist()))
    dec = oracle.Decoded(inp)
    for i in qs:
        row = oracle.score_row(dec, int(i))
        assert_float_row(int(inp.q_pos[i]), inp.k, row, idx_n[i], sc_n[i], f"pkf q{i}",
                         rep_n[i], first=int(inp.q_first[i]))
    assert np.array_equal(rep_n.view(np.uint32), sc_n.view(np.uint32))
    bidx, bsc = hk.baseline_select(dv["q"], dv["k"], dv["w"], inp.k, **rg)
    torch.cuda.synchronize()
    assert np.array_equal(_np(bidx), idx_n)
    assert np.array_equal(_np(bsc).view(np.uint32), sc_n.view(np.uint32))
