"""Recovery stress at the GLM-5.1 shard shape (L = 1,048,576, n = 8,192,
H = 64, d = 128, k = 2,048, bf16): clustered keys with planted queries that
overflow the candidate buffer or get fewer than k candidates.

stress_a plants 32 + 16 failures (the recovery path), stress_b 96 + 32
(more than 64: the full rescore).  The GPU's failure counts by kind must equal
the planted groups, which the oracle's threshold model predicts to fail with a
margin of at least 1,024 candidates.  Other queries may fail too (neighbours of
the under-k run share its sample positions); every flagged query beyond the
planted groups must be one the oracle's model also fails, and queries the
model decides with a clear margin must agree with the GPU.  The recovered
queries must match the oracle; the result must equal the score-table baseline
bit for bit."""
import numpy as np
import pytest
import torch

import datagen
import oracle
from gpu_util import assert_float_row, oracle_rows, say, to_device

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def hk():
    import exact_top_token_amd as m
    m.load_library()
    return m


@pytest.mark.parametrize("name,path", [("stress_a", 0), ("stress_b", 1)])
def test_stress_paths(hk, name, path):
    say(f"{name}: generating inputs")
    inp = datagen.make(name)
    over, under = inp.planted_over, inp.planted_under
    dv = to_device(inp)
    say(f"{name}: hytopk_select")
    idx, sc, st = hk.select(dv["q"], dv["k"], dv["w"], inp.k, with_stats=True)
    torch.cuda.synchronize()
    say(f"{name}: stats {st}")
    failed = np.array(st["failed"], dtype=np.int64)
    planted = set(over.tolist()) | set(under.tolist())
    assert len(failed) == st["n_failed"] == st["n_overflow"] + st["n_underk"]
    assert planted <= set(failed.tolist()), "a planted query was not flagged"
    assert st["path"] == path
    extra = sorted(set(failed.tolist()) - planted)
    say(f"{name}: {len(failed)} flagged, {len(extra)} beyond the planted groups: {extra}")
    # oracle: every flagged query beyond the planted groups, a sample of the
    # planted ones, neighbours of the under-k run and a few ordinary queries
    rng = np.random.default_rng(11)
    check = list(under[:12]) + list(rng.choice(over, size=min(12, over.size), replace=False)) + extra
    check += [int(under[0]) - 1, int(under[-1]) + 1, 0, inp.n - 1]
    check = np.array(sorted(set(int(c) for c in check)))
    say(f"{name}: oracle rows for {check.size} queries")
    rows = oracle_rows(inp, check)
    pred = oracle.predict_paths(rows, inp.k, inp.L, cap=6 * inp.k)
    idx_n, sc_n = idx.cpu().numpy(), sc.cpu().numpy()
    flagged = set(failed.tolist())
    for r, i in enumerate(check):
        p = pred["per_query"][r]
        robust = min(abs(p["margin_cap"]), abs(p["margin_k"])) >= 64 and p["near_tau"] < 8
        if robust:
            assert p["fail"] == (i in flagged), (i, p)
        if i in planted:
            assert p["fail"] and min(abs(p["margin_cap"]), abs(p["margin_k"])) >= 1024, (i, p)
        assert_float_row(inp.L - inp.n + int(i), inp.k, rows[r], idx_n[i], sc_n[i], f"{name} q{i}")
    say(f"{name}: baseline (score table) for bitwise equality")
    bidx, bsc = hk.baseline_select(dv["q"], dv["k"], dv["w"], inp.k)
    torch.cuda.synchronize()
    assert np.array_equal(bidx.cpu().numpy(), idx_n)
    assert np.array_equal(bsc.cpu().numpy().view(np.uint32), sc_n.view(np.uint32))
