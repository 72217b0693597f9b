"""Pins for the CPU oracle: what the pages and the mathematics fix, checked
without reusing the oracle's own code paths.

* the worked-example figures of the HyScale explainer (GLM-5.1 at L = 1M);
* brute force in exact rational arithmetic on tiny inputs (pairwise ranking,
  no sort library), including many ties and ctx < k padding;
* the bf16 and OCP E4M3 decoders against their format definitions' special
  values and against an independent decoder (numpy / torch dtypes);
* invariants on the Tiny workload;
* the soundness of the sampled threshold (candidates give the exact top-k
  whenever the check passes) and its statistical law on i.i.d. scores.
"""
import json
import math
import os
from fractions import Fraction

import numpy as np
import pytest

import datagen
import oracle

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "worked_example.json")


# ---------------------------------------------------------------- worked example

def test_worked_example_figures():
    g = json.load(open(GOLDEN))
    L, n, k = g["L"], g["n"], g["k"]
    M = oracle.sample_count(L)
    assert M == g["sample_count_M"]
    pos = oracle.sample_positions(L, M)
    assert pos.size == M
    assert np.all(np.diff(pos) == g["keys_per_sample"])
    r = oracle.threshold_rank(L, k, M, g["oversample_factor"])
    assert r == g["threshold_rank"]
    assert r * g["keys_per_sample"] == g["keys_represented_by_threshold"] == g["oversample_factor"] * k
    assert n * L * 4 == g["score_table_bytes_per_layer"] == g["score_table_gib"] << 30
    assert n * k * 4 == g["index_bytes"] == g["index_mib"] << 20
    assert (n * L) // (n * k) == g["ratio_table_to_indices"]
    assert g["full_rescore_keys_per_query"] // g["replay_rescored_keys_per_query"] == g["replay_reduction"]
    lo, hi = g["sample_count_bounds"]
    assert oracle.sample_count(1000) == lo and oracle.sample_count(1 << 30) == hi
    assert oracle.DEFAULTS["max_recover"] == g["max_failed_queries_before_full_rescore"]


def test_sample_positions_shape():
    for ctx, M in [(1, 4096), (17, 4096), (4096, 4096), (4097, 4096), (131072, 4096),
                   (1040385, 8192), (1048576, 8192)]:
        p = oracle.sample_positions(ctx, M)
        assert p.size == min(ctx, M)
        assert p[0] == 0 and p[-1] < ctx
        assert np.all(np.diff(p) >= 1)                       # distinct, increasing
        assert np.all(np.diff(p) <= -(-ctx // min(ctx, M)))  # evenly spaced
        if ctx <= M:
            assert np.array_equal(p, np.arange(ctx))


def test_threshold_rank_clamps():
    assert oracle.threshold_rank(10, 256, 10) == 10           # ctx < 3k: every sample
    assert oracle.threshold_rank(4096, 256, 4096) == 768      # Tiny: M_q = ctx
    assert oracle.threshold_rank(131072, 2048, 4096) == 192
    assert oracle.threshold_rank(131071, 2048, 4096) == 193   # ceil, not floor
    assert oracle.threshold_rank(1040385, 2048, 8192) == 49


THRESHOLD_CASES = os.path.join(os.path.dirname(__file__), "golden", "threshold_cases.json")


def _threshold_case_row(case) -> np.ndarray:
    if "row" in case:
        return np.array(case["row"], dtype=np.float64)
    ctx = case["ctx"]
    if case["row_rule"].startswith("ctx = 8192"):
        row = np.full(ctx, -1.0)
        row[0::2] = np.arange(ctx // 2) // 4
        return row
    return np.arange(ctx, dtype=np.float64)


@pytest.mark.parametrize("case", json.load(open(THRESHOLD_CASES))["cases"],
                         ids=lambda c: c["name"])
def test_threshold_hand_computed(case):
    """tau, rank, sample count and candidate count against values derived by
    hand from the sampling rule (duplicates counted separately; M from L)."""
    row = _threshold_case_row(case)
    tau, r, mq = oracle.threshold(row, case["k"], case["L"])
    assert (mq, r, tau) == (case["M_q"], case["r"], case["tau"])
    assert oracle.candidates(row, tau).size == case["count"]
    p = oracle.predict_row(row, case["k"], case["L"], cap=10 ** 6)
    assert (p["tau"], p["cnt"]) == (case["tau"], case["count"])
    for wrong_tau, wrong_count in case["wrong"].values():
        assert (tau, case["count"]) != (wrong_tau, wrong_count)


# ---------------------------------------------------------------- codecs

def test_bf16_decode_special_values():
    cases = {0x3F80: 1.0, 0xC000: -2.0, 0x0000: 0.0, 0x4049: 3.140625,
             0x7F7F: 3.3895313892515355e38, 0x0080: 2.0 ** -126, 0x0001: 2.0 ** -133,
             0x7F80: math.inf, 0xFF80: -math.inf}
    got = oracle.decode_bf16(np.array(list(cases), dtype=np.uint16))
    assert list(got) == list(cases.values())
    assert math.copysign(1.0, oracle.decode_bf16(np.array([0x8000], np.uint16))[0]) == -1.0
    assert np.isnan(oracle.decode_bf16(np.array([0x7FC0], np.uint16))[0])


def test_bf16_decode_all_patterns_vs_float32_view():
    bits = np.arange(1 << 16, dtype=np.uint32)
    with np.errstate(invalid="ignore"):  # signalling-NaN patterns quieten in the cast
        ref = (bits << 16).view(np.float32).astype(np.float64)
    got = oracle.decode_bf16(bits.astype(np.uint16))
    fin = np.isfinite(ref)
    assert np.array_equal(got[fin], ref[fin])
    assert np.array_equal(np.isnan(got), np.isnan(ref))


def test_e4m3_decode_special_values():
    cases = {0x38: 1.0, 0x7E: 448.0, 0xFE: -448.0, 0x01: 2.0 ** -9, 0x08: 2.0 ** -6,
             0x07: 7 * 2.0 ** -9, 0x40: 2.0, 0x3C: 1.5, 0x00: 0.0}
    got = oracle.decode_e4m3(np.array(list(cases), dtype=np.uint8))
    assert list(got) == list(cases.values())
    assert math.copysign(1.0, oracle.decode_e4m3(np.array([0x80], np.uint8))[0]) == -1.0
    assert np.isnan(oracle.decode_e4m3(np.array([0x7F, 0xFF], np.uint8))).all()


def test_e4m3_decode_all_codes_vs_torch():
    torch = pytest.importorskip("torch")
    codes = np.arange(256, dtype=np.uint8)
    ref = torch.from_numpy(codes.copy()).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    got = oracle.decode_e4m3(codes)
    assert np.array_equal(np.isnan(got), np.isnan(ref))
    fin = ~np.isnan(ref)
    assert np.array_equal(got[fin], ref[fin])


def test_datagen_encoders_round_to_nearest_even():
    torch = pytest.importorskip("torch")
    rng = np.random.default_rng(5)
    x = (rng.standard_normal(200000) * 10.0 ** rng.uniform(-8, 8, 200000)).astype(np.float32)
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(datagen.f32_to_bf16_bits(x), ref)
    y = np.clip(rng.standard_normal(200000) * 40, -448, 448)
    y[:6] = [0.0, -0.0, 2.0 ** -10, -(2.0 ** -10), 2.0 ** -9, 3.0]  # zeros, subnormals
    ref8 = torch.from_numpy(y).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(datagen.f32_to_e4m3(y), ref8)
    assert datagen.f32_to_e4m3(np.array([1e6, -1e6]))[0] == 0x7E  # saturates
    assert datagen.f32_to_e4m3(np.array([1e6, -1e6]))[1] == 0xFE


# ---------------------------------------------------------------- brute force

def _exact_bf16(bits):
    """Exact rational value of bf16 bit patterns via numpy's float32 view."""
    f = (np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)
    return [[Fraction(float(v)) for v in row] for row in f.reshape(f.shape[0], -1)]


def _brute_select(inp, i):
    """Scores and top-k of query i from the definition, in exact rationals, with
    ranking by explicit pairwise comparison."""
    H, d, k = inp.H, inp.d, inp.k
    t = inp.L - inp.n + i
    if inp.dtype == "bf16":
        qv = _exact_bf16(inp.q[i].reshape(H, d))
        kv = _exact_bf16(inp.k_[: t + 1])
    else:
        import torch
        dec = lambda c: torch.from_numpy(np.ascontiguousarray(c)).view(torch.float8_e4m3fn).to(torch.float64).numpy()
        qs = Fraction(float(inp.q_scale[i]))
        qv = [[Fraction(float(v)) * qs for v in row] for row in dec(inp.q[i].reshape(H, d))]
        kd = dec(inp.k_[: t + 1])
        kv = [[Fraction(float(v)) * Fraction(float(inp.k_scale[s])) for v in kd[s]] for s in range(t + 1)]
    w = [Fraction(float(x)) for x in inp.w[i]]
    S = []
    for s in range(t + 1):
        tot = Fraction(0)
        for h in range(H):
            dot = sum((qv[h][c] * kv[s][c] for c in range(d)), Fraction(0))
            tot += w[h] * max(dot, Fraction(0))
        S.append(tot)
    ctx = t + 1

    def beats(a, b):  # a ranks before b
        return S[a] > S[b] or (S[a] == S[b] and a < b)

    rank = [sum(1 for b in range(ctx) if beats(b, a)) for a in range(ctx)]
    order = [None] * ctx
    for a, r in enumerate(rank):
        order[r] = a
    keep = order[: min(k, ctx)]
    return S, keep


@pytest.mark.parametrize("seed,L,n,H,d,k", [
    (11, 40, 8, 3, 4, 8),      # heavy ties (values in -3..3, d=4)
    (12, 48, 6, 2, 3, 5),
    (13, 20, 20, 1, 2, 7),     # first queries have ctx < k: padding
    (14, 33, 5, 3, 4, 40),     # k > every ctx
])
def test_brute_force_integer_inputs(seed, L, n, H, d, k):
    inp = datagen.make_custom("bf", L, n, H, d, k, dist="int", seed=seed)
    idx, val = oracle.select(inp)
    for i in range(n):
        S, keep = _brute_select(inp, i)
        m = len(keep)
        assert list(idx[i, :m]) == keep
        assert all(idx[i, m:] == -1) and np.all(np.isneginf(val[i, m:]))
        assert [Fraction(v) for v in val[i, :m]] == [S[a] for a in keep]


@pytest.mark.parametrize("seed", [21, 22])
def test_brute_force_float_inputs(seed):
    inp = datagen.make_custom("bf", 36, 6, 3, 5, 6, dist="normal", seed=seed)
    idx, val = oracle.select(inp)
    for i in range(inp.n):
        S, keep = _brute_select(inp, i)
        assert list(idx[i, : len(keep)]) == keep
        for j, a in enumerate(keep):
            assert abs(Fraction(val[i, j]) - S[a]) <= abs(S[a]) * Fraction(1, 10 ** 12)


def test_brute_force_fp8_inputs():
    pytest.importorskip("torch")
    inp = datagen.make_custom("bf8", 30, 5, 2, 6, 6, dtype="fp8", dist="normal", seed=31)
    idx, val = oracle.select(inp)
    for i in range(inp.n):
        S, keep = _brute_select(inp, i)
        assert list(idx[i, : len(keep)]) == keep
        for j, a in enumerate(keep):
            assert abs(Fraction(val[i, j]) - S[a]) <= abs(S[a]) * Fraction(1, 10 ** 12)


def test_replay_equals_row_scores():
    inp = datagen.make_custom("rp", 300, 16, 4, 8, 12, dist="normal", seed=41)
    idx, val = oracle.select(inp)
    rep = oracle.replay(inp, idx)
    ok = idx >= 0
    assert np.allclose(rep[ok], val[ok], rtol=1e-13, atol=0)
    assert np.all(np.isneginf(rep[~ok]))
    # replay at arbitrary positions against the full rows
    dec = oracle.Decoded(inp)
    rng = np.random.default_rng(3)
    for i in range(inp.n):
        row = oracle.score_row(dec, i)
        pos = rng.integers(0, row.size, 10)
        assert np.allclose(oracle.score_pairs(dec, i, pos), row[pos], rtol=1e-13, atol=0)


# ---------------------------------------------------------------- Tiny invariants

def test_tiny_invariants_and_ties():
    inp = datagen.make("tiny")
    qs = [0, 1, 127, 255]
    idx, val = oracle.select(inp, qs)
    n_tied = 0
    for r, i in enumerate(qs):
        t = inp.L - inp.n + i
        assert len(set(idx[r])) == inp.k and idx[r].min() >= 0 and idx[r].max() <= t
        assert np.all(np.diff(val[r]) <= 0)
        same = np.diff(val[r]) == 0
        assert np.all(np.diff(idx[r])[same] > 0)       # ties by ascending position
        assert np.all(val[r] == np.round(val[r]))      # integer scores
        row = oracle.score_row(oracle.Decoded(inp), i)
        kth = val[r, -1]
        n_tied += int(np.count_nonzero(row == kth)) > int(np.count_nonzero(val[r] == kth))
    assert n_tied > 0, "Tiny should break ties at the k-th score"


# ---------------------------------------------------------------- threshold model

def test_soundness_of_candidate_selection():
    """Whenever the check passes, exact top-k over {score >= tau} equals the
    exact top-k over the whole context [Explainer, HyTopK paragraph]."""
    rng = np.random.default_rng(51)
    passed = 0
    for trial in range(60):
        ctx = int(rng.integers(50, 20000))
        k = int(rng.integers(1, 300))
        if trial % 3 == 0:
            row = rng.integers(0, 30, ctx).astype(np.float64)      # many ties
        else:
            row = rng.standard_normal(ctx)
        tau, r, mq = oracle.threshold(row, k, ctx)
        cap = 6 * k
        got = oracle.select_from_candidates(row, tau, cap, k)
        cnt = oracle.candidates(row, tau).size
        if cnt > cap or cnt < min(k, ctx):
            assert got is None
            continue
        passed += 1
        ref = oracle.exact_topk(row, k)
        assert np.array_equal(got[0], ref[0]) and np.array_equal(got[1], ref[1])
    assert passed > 20


def test_check_flags_overflow_and_underk():
    row = np.arange(1000, dtype=np.float64)
    tau, r, mq = oracle.threshold(row, 10, 1000)
    assert oracle.select_from_candidates(row, tau, cap=5, k=10) is None      # overflow
    assert oracle.select_from_candidates(row, float(row.max()), cap=60, k=10) is None  # under-k
    p = oracle.predict_row(row, 10, 1000, cap=5)
    assert p["overflow"] and p["fail"] and not p["underk"]


def test_threshold_law_iid():
    """On i.i.d. scores the mean candidate count is r + (ctx - M_q) r / (M_q + 1)
    (each non-sampled key beats the r-th of M_q samples with prob r/(M_q+1))."""
    rng = np.random.default_rng(61)
    ctx, k, L = 65536, 256, 65536
    cnts = []
    for _ in range(300):
        row = rng.standard_normal(ctx)
        tau, r, mq = oracle.threshold(row, k, L)
        cnts.append(np.count_nonzero(row >= tau))
    exp = oracle.expected_candidates(ctx, mq, r)
    assert r == 48 and mq == 4096
    assert abs(np.mean(cnts) / exp - 1.0) < 0.02
    assert abs(exp / (3 * k) - 1.0) < 0.01


def test_predict_paths_decides_recovery_vs_full_rescore():
    rows = [np.arange(500, dtype=np.float64) for _ in range(70)]
    few = oracle.predict_paths(rows[:64], k=10, L=500, cap=5)
    assert few["n_failed"] == 64 and not few["full_rescore"]
    many = oracle.predict_paths(rows, k=10, L=500, cap=5)
    assert many["n_failed"] == 70 and many["full_rescore"]


def test_scoring_flops_figures():
    assert oracle.scoring_flops(4096, 256, 4, 64) == 2 * 4 * 64 * 1015936
    assert oracle.scoring_flops(131072, 2048, 64, 128) == 2 * 64 * 128 * 266339328
    assert abs(oracle.scoring_flops(1 << 20, 8192, 64, 128) - 1.4019e14) / 1.4019e14 < 1e-4


def test_brute_force_signed_weights():
    """Negative head weights separate w * ReLU(q.k) from ReLU(w * q.k): the pin
    for where the weight enters the indexer."""
    inp = datagen.make_custom("bw", 30, 6, 3, 4, 6, dist="int", seed=71)
    rng = np.random.default_rng(72)
    inp.w = (rng.integers(-2, 3, size=inp.w.shape)).astype(np.float32)
    inp.w[:, 0] = -1.0
    idx, val = oracle.select(inp)
    for i in range(inp.n):
        S, keep = _brute_select(inp, i)
        assert list(idx[i, : len(keep)]) == keep
        assert [Fraction(v) for v in val[i, : len(keep)]] == [S[a] for a in keep]


def test_stress_generator_failures_match_threshold_model():
    """The planted groups of the recovery-stress workload fail the check with a
    margin >= 1,024 under the oracle's threshold model; their neighbours and
    ordinary queries do not."""
    inp = datagen.make("stress_a")
    dec = oracle.Decoded(inp)
    over, under = inp.planted_over, inp.planted_under
    qs = [int(over[0]), int(over[-1]), int(under[0]), int(under[-1]),
          int(under[0]) - 1, int(under[-1]) + 1, 0, inp.n - 1]
    rows = [oracle.score_row(dec, i) for i in qs]
    pred = oracle.predict_paths(rows, inp.k, inp.L, cap=6 * inp.k)["per_query"]
    assert pred[0]["overflow"] and pred[1]["overflow"]
    assert pred[2]["underk"] and pred[3]["underk"]
    assert min(-pred[0]["margin_cap"], -pred[1]["margin_cap"]) >= 1024
    assert min(-pred[2]["margin_k"], -pred[3]["margin_k"]) >= 1024
    assert not any(p["fail"] for p in pred[4:])
