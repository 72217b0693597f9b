"""Pins for the oracle's per-query key ranges (arbitrary query positions and
packed sequences).

A packed buffer is nothing but several independent problems side by side: the
result of a query in sequence s equals the result of the plain problem made
of that sequence's keys up to the query's position (the default layout, which
test_oracle.py pins on its own), shifted by the sequence's first key.
"""
import numpy as np
import pytest

import datagen
import oracle

SEQS = [700, 300, 1100, 500]
CHUNKS = [(0, 600, 40), (1, 0, 5), (1, 250, 50), (2, 800, 60), (3, 250, 30)]


def _packed(dist="int", dtype="bf16", d=64, k=256, seed=61):
    return datagen.make_packed("packed", SEQS, CHUNKS, H=4, d=d, k=k, dtype=dtype, dist=dist,
                               seed=seed)


def _standalone(inp, i):
    """The plain problem of query i: its sequence's keys first..t, the query last."""
    lo, t = int(inp.q_first[i]), int(inp.q_pos[i])
    L = t - lo + 1
    sub = datagen.Inputs("alone", L, 1, inp.H, inp.d, inp.k, inp.dtype, inp.q[i:i + 1],
                         inp.k_[lo:t + 1], inp.w[i:i + 1],
                         None if inp.q_scale is None else inp.q_scale[i:i + 1],
                         None if inp.k_scale is None else inp.k_scale[lo:t + 1])
    return sub, lo


@pytest.mark.parametrize("dtype,dist", [("bf16", "int"), ("bf16", "normal"), ("fp8", "normal")])
def test_packed_queries_equal_independent_problems(dtype, dist):
    inp = _packed(dist, dtype, d=128 if dtype == "fp8" else 64)
    assert inp.q_pos is not None and not np.all(np.diff(inp.q_pos) > 0), "order is shuffled"
    idx, val = oracle.select(inp)
    for i in range(inp.n):
        sub, lo = _standalone(inp, i)
        si, sv = oracle.select(sub)
        want = np.where(si[0] >= 0, si[0] + lo, -1)
        assert np.array_equal(idx[i], want), i
        assert np.array_equal(val[i], sv[0]), i
        # keys stay inside the query's own sequence
        kept = idx[i][idx[i] >= 0]
        assert kept.size == min(inp.k, int(inp.q_pos[i]) - lo + 1)
        assert kept.min() >= lo and kept.max() <= inp.q_pos[i]


def test_explicit_default_positions_change_nothing():
    inp = datagen.make("tiny")
    ref = oracle.select(inp, np.arange(0, inp.n, 17))
    inp.q_pos = (inp.q_start + np.arange(inp.n)).astype(np.int32)
    inp.q_first = np.zeros(inp.n, dtype=np.int32)
    got = oracle.select(inp, np.arange(0, inp.n, 17))
    assert np.array_equal(ref[0], got[0]) and np.array_equal(ref[1], got[1])


def test_packed_threshold_model_uses_the_query_context():
    """The sampled threshold of a packed query is the plain model applied to
    its own context (same L: the number of keys in the call)."""
    inp = _packed()
    dec = oracle.Decoded(inp)
    for i in range(0, inp.n, 7):
        sub, _ = _standalone(inp, i)
        row = oracle.score_row(dec, i)
        alone = oracle.score_row(oracle.Decoded(sub), 0)
        assert np.array_equal(row, alone)
        a = oracle.predict_row(row, inp.k, inp.L, cap=6 * inp.k)
        b = oracle.predict_row(alone, inp.k, inp.L, cap=6 * inp.k)
        assert a == b


def test_replay_and_backward_follow_the_absolute_indices():
    inp = _packed(dist="normal")
    idx, val = oracle.select(inp)
    rep = oracle.replay(inp, idx)
    ok = idx >= 0
    # same fp64 sums, evaluated in differently shaped BLAS calls
    np.testing.assert_allclose(rep[ok], val[ok], rtol=1e-12, atol=1e-15)
    g = np.random.default_rng(3).standard_normal(idx.shape)
    res = oracle.backward(inp, idx, g)
    dec = oracle.Decoded(inp)
    Q = np.stack([dec.query(i)[0] for i in range(inp.n)])
    total = float(np.sum(g[ok] * val[ok]))
    assert abs(float(np.sum(dec.keys * res["dk"])) - total) <= 1e-9 * (np.abs(g[ok] * val[ok]).sum() + 1)
    assert abs(float(np.sum(Q * res["dq"])) - total) <= 1e-9 * (np.abs(g[ok] * val[ok]).sum() + 1)
