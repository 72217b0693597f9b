"""GPU parity on integer-valued inputs, where every fp32 score is exact, so the
HIP path must equal the fp64 oracle bit for bit: the Tiny workload (L = 4,096,
n = 256, H = 4, d = 64, k = 256, many ties), ragged shapes, every selection
path (candidates, recovery, full rescore, forced rows, the baseline), replay,
reproducibility and the threshold statistics."""
import numpy as np
import pytest
import torch

import datagen
import oracle
from gpu_util import assert_exact, oracle_rows, say, to_device

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def hk():
    import exact_top_token_amd as m
    m.load_library()
    return m


@pytest.fixture(scope="module")
def tiny():
    inp = datagen.make("tiny")
    rows = oracle_rows(inp, range(inp.n))
    ref = [oracle.exact_topk(r, inp.k) for r in rows]
    return dict(inp=inp, dev=to_device(inp), rows=rows,
                idx=np.stack([r[0] for r in ref]), val=np.stack([r[1] for r in ref]))


def _np(t):
    return t.cpu().numpy()


def test_tiny_select_bit_exact(hk, tiny):
    say("tiny: hytopk_select, L=4096 n=256 H=4 d=64 k=256")
    d, inp = tiny["dev"], tiny["inp"]
    idx, sc, st = hk.select(d["q"], d["k"], d["w"], inp.k, with_stats=True)
    torch.cuda.synchronize()
    assert_exact(inp, range(inp.n), _np(idx), _np(sc), tiny["idx"], tiny["val"])
    assert st["path"] == 0 and st["n_failed"] == 0


def test_tiny_stats_equal_threshold_prediction(hk, tiny):
    """Integer scores: the GPU's thresholds and candidate counts must equal the
    oracle's threshold model exactly."""
    say("tiny: stats vs oracle.predict_paths")
    d, inp = tiny["dev"], tiny["inp"]
    _, _, st = hk.select(d["q"], d["k"], d["w"], inp.k, with_stats=True)
    pred = oracle.predict_paths(tiny["rows"], inp.k, inp.L, cap=6 * inp.k)
    assert st["cand_total"] == sum(p["cnt"] for p in pred["per_query"])
    assert st["cand_max"] == max(p["cnt"] for p in pred["per_query"])
    assert st["n_failed"] == pred["n_failed"]


def test_tiny_replay_and_baseline_bit_exact(hk, tiny):
    say("tiny: hytopk_replay + hytopk_baseline_select")
    d, inp = tiny["dev"], tiny["inp"]
    idx, sc = hk.select(d["q"], d["k"], d["w"], inp.k)
    rep = hk.replay(d["q"], d["k"], d["w"], idx)
    bidx, bsc = hk.baseline_select(d["q"], d["k"], d["w"], inp.k)
    torch.cuda.synchronize()
    assert np.array_equal(_np(rep), _np(sc))
    assert_exact(inp, range(inp.n), _np(bidx), _np(bsc), tiny["idx"], tiny["val"])
    ref_rep = oracle.replay(inp, tiny["idx"])
    assert np.array_equal(_np(rep).astype(np.float64), ref_rep)


def test_tiny_every_path_is_identical(hk, tiny):
    """Forced rows, forced overflow (full rescore) and a cap that sends a few
    queries to recovery all return the same bits as the candidate path."""
    d, inp = tiny["dev"], tiny["inp"]
    base = [_np(t) for t in hk.select(d["q"], d["k"], d["w"], inp.k)]
    cnts = np.array([p["cnt"] for p in oracle.predict_paths(tiny["rows"], inp.k, inp.L,
                                                             cap=6 * inp.k)["per_query"]])
    cap_few = int(np.sort(cnts)[-10])  # the 9 queries above it overflow
    cases = [("rows_all", dict(force_path=hk.PATH_ROWS_ALL), 2, None),
             ("overflow_all", dict(cap=inp.k + 1), 1, inp.n),
             ("recovery", dict(cap=cap_few), 0, int(np.count_nonzero(cnts > cap_few))),
             ("recovery_chunks", dict(cap=cap_few, rows_chunk=2, max_recover=64), 0, None),
             ("full_rescore_chunks", dict(cap=inp.k + 1, rows_chunk=50), 1, inp.n)]
    for name, prm, path, nfail in cases:
        say(f"tiny: path {name} params {prm}")
        idx, sc, st = hk.select(d["q"], d["k"], d["w"], inp.k, params=prm, with_stats=True)
        torch.cuda.synchronize()
        assert st["path"] == path, (name, st)
        if nfail is not None:
            assert st["n_failed"] == nfail, (name, st)
        assert np.array_equal(_np(idx), base[0]), name
        assert np.array_equal(_np(sc), base[1]), name


def test_tiny_reproducible(hk, tiny):
    say("tiny: three identical calls")
    d, inp = tiny["dev"], tiny["inp"]
    runs = [[_np(t) for t in hk.select(d["q"], d["k"], d["w"], inp.k)] for _ in range(3)]
    for r in runs[1:]:
        assert np.array_equal(r[0], runs[0][0]) and np.array_equal(r[1].view(np.uint32),
                                                                   runs[0][1].view(np.uint32))


@pytest.mark.parametrize("L,n,H,d,k,seed", [
    (300, 300, 64, 128, 64, 5),     # q_start = 0: the first 63 queries have ctx < k
    (1000, 37, 64, 128, 100, 6),    # ragged query group and key tile
    (777, 77, 4, 64, 700, 7),       # k close to ctx, small heads
    (5000, 130, 8, 128, 1, 8),      # k = 1
    (4100, 33, 64, 64, 2048, 9),    # k = 2048 at H = 64, d = 64
    (64, 5, 4, 64, 16, 10),         # fewer queries than XCDs (sampling workgroup map)
])
def test_ragged_shapes_bit_exact(hk, L, n, H, d, k, seed):
    say(f"ragged: L={L} n={n} H={H} d={d} k={k} seed={seed}")
    inp = datagen.make_custom("ragged", L, n, H, d, k, dist="int", seed=seed)
    dv = to_device(inp)
    rows = oracle_rows(inp, range(n))
    ref = [oracle.exact_topk(r, k) for r in rows]
    ridx, rval = np.stack([r[0] for r in ref]), np.stack([r[1] for r in ref])
    idx, sc = hk.select(dv["q"], dv["k"], dv["w"], k)
    bidx, bsc = hk.baseline_select(dv["q"], dv["k"], dv["w"], k)
    rep = hk.replay(dv["q"], dv["k"], dv["w"], idx)
    torch.cuda.synchronize()
    assert_exact(inp, range(n), _np(idx), _np(sc), ridx, rval)
    assert_exact(inp, range(n), _np(bidx), _np(bsc), ridx, rval)
    ok = ridx >= 0
    assert np.array_equal(_np(rep)[ok], _np(sc)[ok])
    assert np.all(np.isneginf(_np(rep)[~ok]))


@pytest.mark.parametrize("fmt,L,n", [("bf16", 12000, 8190), ("mxfp8", 12000, 8190),
                                     ("mxfp4", 8000, 4094)])
def test_one_split_with_partial_last_group(hk, fmt, L, n):
    """n queries fill 512 query groups (16 per group, 8 for MXFP4), so the
    fused kernel runs one key split per query -- each wave
    the only writer of its queries' candidates -- and the last group is
    partial: its last wave has no query.  Integer inputs (exact in every
    format): the selection equals the oracle bit for bit on 96 queries (the
    last 48 and 48 random ones) and the row baseline on all."""
    H, d, k = 64, 128, 256
    say(f"one split, partial last group: {fmt} L={L} n={n} H={H} d={d} k={k}")
    inp = datagen.make_custom("onesplit", L, n, H, d, k, dtype=fmt, dist="int", seed=11)
    dv = to_device(inp)
    kw = {}
    if fmt != "bf16":
        kw = dict(q_scale=dv["q_scale"], k_scale=dv["k_scale"], fmt=fmt)
    idx, sc, st = hk.select(dv["q"], dv["k"], dv["w"], k, with_stats=True, **kw)
    bidx, bsc = hk.baseline_select(dv["q"], dv["k"], dv["w"], k, **kw)
    torch.cuda.synchronize()
    assert st["n_failed"] == 0, st
    assert np.array_equal(_np(idx), _np(bidx))
    assert np.array_equal(_np(sc).view(np.uint32), _np(bsc).view(np.uint32))
    qs = np.unique(np.concatenate([np.arange(n - 48, n),
                                   np.random.default_rng(11).choice(n - 48, 48, replace=False)]))
    rows = oracle_rows(inp, qs)
    ref = [oracle.exact_topk(r, k) for r in rows]
    for j, i in enumerate(qs):
        assert np.array_equal(_np(idx)[i], ref[j][0]), f"query {i}"
        assert np.array_equal(_np(sc)[i], ref[j][1].astype(np.float32)), f"query {i}"


def test_explicit_q_start(hk):
    """Queries need not sit at the end: q_start + n < L."""
    say("q_start: L=2000 n=40 q_start=900")
    inp = datagen.make_custom("qs", 2000, 40, 8, 64, 50, dist="int", seed=3)
    dv = to_device(inp)
    qs = 900
    dec = oracle.Decoded(inp)
    dec.q_start = qs
    ref = [oracle.exact_topk(oracle.score_row(dec, i), inp.k) for i in range(inp.n)]
    idx, sc = hk.select(dv["q"], dv["k"], dv["w"], inp.k, q_start=qs)
    torch.cuda.synchronize()
    assert_exact(inp, range(inp.n), _np(idx), _np(sc), np.stack([r[0] for r in ref]),
                 np.stack([r[1] for r in ref]))


def test_api_errors_do_not_launch(hk, tiny):
    say("api errors")
    d, inp = tiny["dev"], tiny["inp"]
    with pytest.raises(hk.HytopkError) as e:
        hk.select(d["q"], d["k"], d["w"], 5000)
    assert e.value.status == -2
    ws = torch.empty(16, dtype=torch.uint8, device="cuda")
    with pytest.raises(hk.HytopkError) as e:
        hk.baseline_select(d["q"], d["k"], d["w"], inp.k, workspace=ws[1:])
    assert e.value.status == -3


@pytest.mark.parametrize("shape", ["tiny", "one_split"])
def test_reversed_key_walk_gives_the_same_bits(hk, tiny, shape, monkeypatch):
    """The scoring kernel walks key tiles last-to-first under the
    HYTOPK_REVERSE_KEY_WALK knob, so candidates reach the buffer in another
    order (several key splits: staged flushes; one split: direct stores); the
    selection, the scores and the candidate counts must not change."""
    if shape == "tiny":
        inp, d = tiny["inp"], tiny["dev"]
    else:
        inp = datagen.make_custom("rev", 12000, 8190, 8, 128, 64, dist="int", seed=5)
        d = to_device(inp)
    say(f"reversed key walk: {shape} L={inp.L} n={inp.n} H={inp.H} k={inp.k}")
    monkeypatch.delenv("HYTOPK_REVERSE_KEY_WALK", raising=False)
    idx0, sc0, st0 = hk.select(d["q"], d["k"], d["w"], inp.k, with_stats=True)
    b0 = [_np(t) for t in hk.baseline_select(d["q"], d["k"], d["w"], inp.k)]
    monkeypatch.setenv("HYTOPK_REVERSE_KEY_WALK", "1")
    idx1, sc1, st1 = hk.select(d["q"], d["k"], d["w"], inp.k, with_stats=True)
    b1 = [_np(t) for t in hk.baseline_select(d["q"], d["k"], d["w"], inp.k)]
    torch.cuda.synchronize()
    assert np.array_equal(_np(idx0), _np(idx1))
    assert np.array_equal(_np(sc0).view(np.uint32), _np(sc1).view(np.uint32))
    assert st0 == st1
    assert np.array_equal(b0[0], b1[0]) and np.array_equal(b0[1].view(np.uint32), b1[1].view(np.uint32))
    assert np.array_equal(b0[0], _np(idx0))


@pytest.mark.parametrize("fmt,L,n,H,d,k,prm", [
    # 64 sample scores per thread, one row block
    ("bf16", 20000, 48, 8, 128, 64, dict(m_min=16384, m_max=16384)),
    # 64 per thread, four row blocks
    ("bf16", 12000, 32, 64, 128, 128, dict(m_min=12000, m_max=12000)),
    # scores in LDS: 64 KB of them
    ("mxfp8", 20000, 32, 64, 128, 64, dict(m_min=16384, m_max=16384)),
    # fewer samples than threads x 4, a larger oversampling factor
    ("bf16", 6000, 40, 64, 64, 32, dict(m_min=1000, m_max=1000, oversample=5)),
    # M from L / m_div (20000 / 4 = 5000), oversampling by one
    ("bf16", 20000, 40, 16, 128, 100, dict(m_min=100, m_div=4, oversample=1)),
])
def test_threshold_parameters_away_from_the_default(hk, fmt, L, n, H, d, k, prm):
    """The sample count M = min(max(m_min, L / m_div), m_max) above 8,192 (the
    register path with 64 scores per thread, the LDS path at its largest) and
    far below it, and other oversampling factors.  Integer scores:
    thresholds and candidate counts equal the oracle's threshold model with
    the same parameters, and the selection equals the oracle."""
    say(f"threshold parameters {prm}: {fmt} L={L} n={n} H={H} d={d} k={k}")
    inp = datagen.make_custom("mq", L, n, H, d, k, dtype=fmt, dist="int", seed=L + n)
    dv = to_device(inp)
    kw = {}
    if fmt != "bf16":
        kw = dict(q_scale=dv["q_scale"], k_scale=dv["k_scale"], fmt=fmt)
    idx, sc, st = hk.select(dv["q"], dv["k"], dv["w"], k, params=prm, with_stats=True, **kw)
    torch.cuda.synchronize()
    rows = oracle_rows(inp, range(n))
    pred = oracle.predict_paths(rows, k, L, cap=6 * k, params=prm)
    assert st["cand_total"] == sum(p["cnt"] for p in pred["per_query"])
    assert st["cand_max"] == max(p["cnt"] for p in pred["per_query"])
    assert st["n_failed"] == pred["n_failed"]
    ref = [oracle.exact_topk(r, k) for r in rows]
    assert_exact(inp, range(n), _np(idx), _np(sc), np.stack([r[0] for r in ref]),
                 np.stack([r[1] for r in ref]))
