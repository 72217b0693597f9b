"""Recovery-stress workloads: clustered keys with planted threshold failures.

Shape of the GLM-5.1 one-GPU shard (L = 1,048,576 keys, n = 8,192 queries at
the last positions, H = 64, d = 128, k = 2,048, bf16).  Keys come from 16
Gaussian clusters (centroid ~ N(0, I)/sqrt(d), member = centroid + 0.5 *
N(0, I)/sqrt(d)); queries ~ N(0, 1)/sqrt(d), weights ~ U(0, 1)/H.  Two groups
of queries are then made to fail the sampled-threshold check on purpose:

* overflow group Q1: queries aligned with a direction u1, and 10,000 keys
  alpha * u1 + noise placed where none of Q1's sampled positions fall, so the
  threshold taken from the samples ignores them and every one of them passes
  it on top of the ~6k ordinary candidates (more than the 6k buffer);
* under-k group Q2: a contiguous run of adjacent queries aligned with u2, and
  keys alpha * u2 + noise planted exactly at the first 200 sampled positions
  of those queries, so the threshold lands inside the planted set and only
  ~100 keys pass (fewer than k).

Planting needs the positions the sampler looks at.  The HyScale explainer
(HyTopK and worked-example paragraphs) takes M = min(max(4096, L/128), 8192)
evenly spaced samples of the query's own context; this module restates that
position rule (floor(j * ctx / M_q)) only to place adversarial keys -- it
computes no scores and no thresholds.  Which queries actually fail is decided
independently by the oracle's threshold model in the tests.

stress_a (seed 1005): |Q1| = 32, |Q2| = 16 -> 48 failures  -> recovery.
stress_b (seed 1006): |Q1| = 96, |Q2| = 32 -> 128 failures -> full rescore.
"""
from __future__ import annotations

import math

import numpy as np

from . import Inputs, f32_to_bf16_bits

STRESS = {
    "stress_a": dict(seed=1005, n_over=32, n_under=16),
    "stress_b": dict(seed=1006, n_over=96, n_under=32),
}
L, N, H, D, K = 1048576, 8192, 64, 128, 2048
N_PLANT_OVER = 10000
J_UNDER = 200


def _grid(ctx: int, L_: int = L) -> np.ndarray:
    """Sampled positions of a query with context ctx (see the module notes)."""
    M = min(max(4096, L_ // 128), 8192)
    mq = min(M, ctx)
    return (np.arange(mq, dtype=np.int64) * ctx) // mq


def _unit(rng, d):
    v = rng.standard_normal(d)
    return v / np.linalg.norm(v)


def make(name: str) -> Inputs:
    cfg = STRESS[name]
    rng = np.random.default_rng(cfg["seed"])
    s = np.float32(1.0 / math.sqrt(D))
    q_start = L - N
    # background
    q = rng.standard_normal((N, H, D), dtype=np.float32) * s
    cent = rng.standard_normal((16, D), dtype=np.float32) * s
    member = rng.integers(0, 16, size=L)
    k = cent[member] + rng.standard_normal((L, D), dtype=np.float32) * (np.float32(0.5) * s)
    w = rng.random((N, H), dtype=np.float32) / np.float32(H)
    u1, u2 = _unit(rng, D).astype(np.float32), _unit(rng, D).astype(np.float32)

    # under-k group: a contiguous run of adjacent queries near the end
    n_under, n_over = cfg["n_under"], cfg["n_over"]
    under = np.arange(N - 1000, N - 1000 + n_under)
    # overflow group: spread over the remaining queries
    pool = np.setdiff1d(np.arange(0, N - 1100), under)
    over = np.sort(rng.choice(pool, size=n_over, replace=False))

    def align(rows, u):
        for i in rows:
            q[i] = u[None, :] + rng.standard_normal((H, D)).astype(np.float32) * (np.float32(0.3) * s)

    align(over, u1)
    align(under, u2)

    # plants for the under-k group: their first J_UNDER sampled positions
    p2 = np.unique(np.concatenate([_grid(q_start + int(i) + 1)[:J_UNDER] for i in under]))
    k[p2] = 1.0 * u2[None, :] + rng.standard_normal((p2.size, D)).astype(np.float32) * (np.float32(0.2) * s)

    # plants for the overflow group: positions no Q1 query samples, below every
    # Q1 context, away from the under-k plants
    lo = int(p2.max()) + 1
    hi = q_start + int(over.min()) + 1
    sampled = np.zeros(hi, dtype=bool)
    for i in over:
        g = _grid(q_start + int(i) + 1)
        sampled[g[g < hi]] = True
    free = np.nonzero(~sampled[lo:hi])[0] + lo
    p1 = np.sort(rng.choice(free, size=N_PLANT_OVER, replace=False))
    k[p1] = 1.0 * u1[None, :] + rng.standard_normal((p1.size, D)).astype(np.float32) * (np.float32(0.2) * s)

    inp = Inputs(name, L, N, H, D, K, "bf16", f32_to_bf16_bits(q), f32_to_bf16_bits(k), w)
    inp.planted_over = over          # queries meant to overflow
    inp.planted_under = under        # queries meant to get fewer than k candidates
    return inp
