"""Pins for the oracle's indexer backward at the replayed entries.

The backward is pinned to things other than its own formula:

* central finite differences of the forward (the forward is pinned on its own
  in test_oracle.py), along random directions, for q, w and k, with several
  queries selecting overlapping keys so the scatter-add onto dk is exercised;
* Euler's identity: the indexer is positively homogeneous of degree 1 in each
  of w[t], q[t] and k[s] separately (ReLU(a x) = a ReLU(x) for a > 0), so
  <w, dw> = <q, dq> = <k, dk> = sum dI * I at the selected entries;
* the one-head, one-key special case, the textbook ReLU derivative;
* exact integers on the integer workload (every value is an integer far
  below 2^53, so fp64 evaluates the sums exactly).
"""
import numpy as np
import pytest

import datagen
import oracle


def _problem(seed, m=5, H=6, d=16, L=40, k=9, wsign=False):
    rng = np.random.default_rng(seed)
    q = rng.standard_normal((m, H, d))
    w = rng.random((m, H)) + 0.1
    if wsign:
        w *= rng.choice([-1.0, 1.0], size=(m, H))
    keys = rng.standard_normal((L, d))
    # overlapping selections, with one padded slot per query
    idx = np.stack([rng.choice(L, size=k, replace=False) for _ in range(m)])
    idx[:, -1] = -1
    g = rng.standard_normal((m, k))
    return q, w, keys, idx, g


def _loss(q, w, keys, idx, g):
    tot = 0.0
    for r in range(q.shape[0]):
        ok = idx[r] >= 0
        tot += float(g[r, ok] @ oracle.indexer_pairs(q[r], w[r], keys[idx[r, ok]]))
    return tot


def _min_abs_c(q, keys, idx):
    v = np.inf
    for r in range(q.shape[0]):
        ok = idx[r] >= 0
        v = min(v, float(np.min(np.abs(q[r] @ keys[idx[r, ok]].T))))
    return v


@pytest.mark.parametrize("seed", [11, 12, 13])
@pytest.mark.parametrize("wsign", [False, True])
def test_backward_matches_finite_differences(seed, wsign):
    q, w, keys, idx, g = _problem(seed, wsign=wsign)
    res = oracle.backward_core(lambda r: (q[r], w[r]), keys, idx, g)
    rng = np.random.default_rng(seed + 100)
    h = 1e-6
    # the step must not carry any c = q . k across the ReLU kink
    assert _min_abs_c(q, keys, idx) > 50 * h * 10
    for name, x, grad in (("q", q, res["dq"]), ("w", w, res["dw"]), ("k", keys, res["dk"])):
        for _ in range(3):
            v = rng.standard_normal(x.shape)
            xp, xm = x + h * v, x - h * v
            args_p = dict(q=q, w=w, keys=keys)
            args_m = dict(q=q, w=w, keys=keys)
            args_p[{"q": "q", "w": "w", "k": "keys"}[name]] = xp
            args_m[{"q": "q", "w": "w", "k": "keys"}[name]] = xm
            fd = (_loss(idx=idx, g=g, **args_p) - _loss(idx=idx, g=g, **args_m)) / (2 * h)
            an = float(np.sum(grad * v))
            assert abs(fd - an) <= 1e-6 * (abs(an) + 1.0), (name, fd, an)


def test_unselected_keys_and_padding_get_no_gradient():
    q, w, keys, idx, g = _problem(21)
    res = oracle.backward_core(lambda r: (q[r], w[r]), keys, idx, g)
    used = np.unique(idx[idx >= 0])
    unused = np.setdiff1d(np.arange(keys.shape[0]), used)
    assert np.all(res["dk"][unused] == 0.0)
    # all-padding query: no dq, no dw
    idx2 = idx.copy()
    idx2[2] = -1
    res2 = oracle.backward_core(lambda r: (q[r], w[r]), keys, idx2, g)
    assert np.all(res2["dq"][2] == 0.0) and np.all(res2["dw"][2] == 0.0)


@pytest.mark.parametrize("name", ["tiny", "mid"])
def test_backward_euler_identity(name):
    inp = datagen.make(name) if name == "tiny" else None
    if inp is None:
        # Mid shape would be slow to select on the CPU: a few queries of a
        # smaller float problem with the same distributions
        inp = datagen.make_custom("euler", L=3000, n=24, H=64, d=128, k=300, dist="normal", seed=77)
    qs = np.arange(min(inp.n, 24))
    idx, val = oracle.select(inp, qs)
    rng = np.random.default_rng(5)
    g = rng.standard_normal(idx.shape)
    res = oracle.backward(inp, idx, g, qs)
    dec = oracle.Decoded(inp)
    Q = np.stack([dec.query(int(i))[0] for i in qs])
    W = np.stack([dec.query(int(i))[1] for i in qs])
    ok = idx >= 0
    total = float(np.sum(g[ok] * val[ok]))
    scale = float(np.sum(np.abs(g[ok] * val[ok]))) + 1.0
    for lhs in (np.sum(W * res["dw"]), np.sum(Q * res["dq"]), np.sum(dec.keys * res["dk"])):
        assert abs(float(lhs) - total) <= 1e-9 * scale


def test_single_head_single_key_is_relu_derivative():
    rng = np.random.default_rng(3)
    for _ in range(20):
        q = rng.standard_normal((1, 8))
        key = rng.standard_normal((1, 8))
        w = np.array([rng.random() + 0.5])
        g = np.array([rng.standard_normal()])
        b = oracle.backward_query(q, w, key, g)
        c = float(q[0] @ key[0])
        on = 1.0 if c > 0 else 0.0
        np.testing.assert_allclose(b["dq"][0], g[0] * w[0] * on * key[0], rtol=1e-15, atol=0)
        np.testing.assert_allclose(b["u"][0], g[0] * w[0] * on * q[0], rtol=1e-15, atol=0)
        assert b["dw"][0] == pytest.approx(g[0] * max(c, 0.0), rel=1e-15)
    # exactly zero pre-activation: derivative 0
    q = np.array([[1.0, -1.0]])
    key = np.array([[2.0, 2.0]])
    b = oracle.backward_query(q, np.array([1.0]), key, np.array([1.0]))
    assert np.all(b["dq"] == 0.0) and np.all(b["u"] == 0.0) and b["dw"][0] == 0.0


def test_backward_integer_workload_is_exact():
    inp = datagen.make("tiny")
    qs = np.arange(0, inp.n, 37)
    idx, _ = oracle.select(inp, qs)
    rng = np.random.default_rng(9)
    g = rng.integers(-3, 4, size=idx.shape).astype(np.float64)
    res = oracle.backward(inp, idx, g, qs)
    for k in ("dq", "dw", "dk"):
        assert np.all(res[k] == np.round(res[k])), k
    # the absolute-term scale bounds every result
    for k in ("dq", "dw", "dk"):
        assert np.all(np.abs(res[k]) <= res[k + "_abs"] + 1e-9)


def test_ambiguity_allowance_covers_only_near_zero_decisions():
    q = np.array([[1.0, -1.0], [1.0, 1.0]])
    key = np.array([[1.0, 1.0 - 1e-9], [3.0, 1.0]])
    b = oracle.backward_query(q, np.array([1.0, 2.0]), key, np.array([1.0, 1.0]), amb=1e-6)
    # c[0, 0] = 1e-9 cancels down from terms of size 1: an fp32 evaluation may
    # take either branch there; every other pre-activation is far from zero
    assert b["dq_amb"][0].sum() > 0 and np.all(b["dq_amb"][1] == 0.0)
    np.testing.assert_allclose(b["dq_amb"][0], 1.0 * key[0], rtol=1e-15)
