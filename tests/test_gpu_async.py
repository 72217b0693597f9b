"""hytopk_select_async: the selection without a host synchronisation.

Integer-valued Tiny inputs make every score exact, so the asynchronous call
must return the bits hytopk_select returns (which the Tiny tests pin to the
oracle) on the candidate path, with recovery in one or several passes, and
with the rows of the passing queries when the failures exceed max_recover
(status[0] then reads 1).  The last test records the call in a graph and
checks every replay against an eager call on the same inputs, with eager
work and synchronisations between the replays."""
import numpy as np
import pytest
import torch

import datagen
import oracle
from gpu_util import oracle_rows, say, to_device

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
    cnts = np.array([p["cnt"] for p in oracle.predict_paths(rows, inp.k, inp.L,
                                                             cap=6 * inp.k)["per_query"]])
    return dict(inp=inp, dev=to_device(inp), cnts=cnts)


def _np(t):
    return t.cpu().numpy()


def _run_async(hk, d, inp, params=None):
    need = hk.select_workspace_bytes(d["q"], d["k"], d["w"], inp.k, params=params)
    ws = torch.empty(need, dtype=torch.uint8, device="cuda")
    idx = torch.full((inp.n, inp.k), -7, dtype=torch.int32, device="cuda")
    sc = torch.full((inp.n, inp.k), -7.0, dtype=torch.float32, device="cuda")
    status = torch.full((hk.ASYNC_STATUS_WORDS,), -1, dtype=torch.int32, device="cuda")
    hk.select_async(d["q"], d["k"], d["w"], inp.k, workspace=ws, out=(idx, sc), status=status,
                    params=params)
    torch.cuda.synchronize()
    return _np(idx), _np(sc), _np(status)


def test_async_equals_select_on_every_recoverable_path(hk, tiny):
    d, inp, cnts = tiny["dev"], tiny["inp"], tiny["cnts"]
    cap_few = int(np.sort(cnts)[-10])  # the 9 queries above it overflow
    cases = [("candidates", None),
             ("recovery", dict(cap=cap_few)),
             ("recovery_passes", dict(cap=cap_few, rows_chunk=2, max_recover=64)),
             ("rows_all", dict(force_path=hk.PATH_ROWS_ALL))]
    for name, prm in cases:
        say(f"async: {name} params {prm}")
        ref_idx, ref_sc, st = hk.select(d["q"], d["k"], d["w"], inp.k, params=prm,
                                        with_stats=True)
        idx, sc, status = _run_async(hk, d, inp, prm)
        assert np.array_equal(idx, _np(ref_idx)), name
        assert np.array_equal(sc.view(np.uint32), _np(ref_sc).view(np.uint32)), name
        assert status[0] == 0, (name, status)
        if name != "rows_all":
            assert status[1] == st["n_failed"], (name, status, st)
            assert status[2] == st["n_overflow"] and status[3] == st["n_underk"], (name, status)
            assert status[4] == st["cand_max"], (name, status)
            assert int(np.uint32(status[5])) + (int(np.uint32(status[6])) << 32) == st["cand_total"]
        assert status[7] == 0


@pytest.mark.parametrize("max_recover", [4, 1])
def test_async_reports_unrecovered_failures(hk, tiny, max_recover):
    """More failures than max_recover (4 rows in two passes, or 1 row):
    status[0] is 1, the passing queries' rows are the exact ones, and the
    failed queries' rows are left untouched."""
    d, inp, cnts = tiny["dev"], tiny["inp"], tiny["cnts"]
    cap_few = int(np.sort(cnts)[-10])
    prm = dict(cap=cap_few, max_recover=max_recover, rows_chunk=3)
    say(f"async: failures beyond max_recover, params {prm}")
    ref_idx, ref_sc, st = hk.select(d["q"], d["k"], d["w"], inp.k, params=prm, with_stats=True)
    assert st["path"] == 1 and st["n_failed"] > max_recover
    idx, sc, status = _run_async(hk, d, inp, prm)
    assert status[0] == 1 and status[1] == st["n_failed"], status
    failed = set(st["failed"])
    ok = np.array([i not in failed for i in range(inp.n)])
    assert np.array_equal(idx[ok], _np(ref_idx)[ok])
    assert np.array_equal(sc[ok].view(np.uint32), _np(ref_sc)[ok].view(np.uint32))
    # the failed queries' rows were left as the caller filled them (no pass ran)
    assert (idx[~ok] == -7).all()


def test_async_graph_replays_match_eager_calls(hk, tiny):
    d, inp, cnts = tiny["dev"], tiny["inp"], tiny["cnts"]
    cap_few = int(np.sort(cnts)[-10])
    prm = dict(cap=cap_few)  # candidates plus one recovery pass
    say("async: graph capture with recovery, three replays")
    q, k = d["q"], d["k"]
    w = d["w"].clone()
    need = hk.select_workspace_bytes(q, k, w, inp.k, params=prm)
    ws = torch.empty(need, dtype=torch.uint8, device="cuda")
    idx = torch.empty((inp.n, inp.k), dtype=torch.int32, device="cuda")
    sc = torch.empty((inp.n, inp.k), dtype=torch.float32, device="cuda")
    status = torch.zeros(hk.ASYNC_STATUS_WORDS, dtype=torch.int32, device="cuda")
    # warm-up outside the capture, then record
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        hk.select_async(q, k, w, inp.k, workspace=ws, out=(idx, sc), status=status, params=prm)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        hk.select_async(q, k, w, inp.k, workspace=ws, out=(idx, sc), status=status, params=prm)
    torch.cuda.synchronize()
    scales = [1.0, 2.0, 1.0]  # the weights change between replays (integers stay exact)
    w0 = d["w"].clone()
    for rep, f in enumerate(scales):
        w.copy_(w0 * f)
        idx.fill_(-3)
        sc.zero_()
        status.fill_(-1)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        got = (_np(idx), _np(sc), _np(status))
        ref_idx, ref_sc, st = hk.select(q, k, w, inp.k, params=prm, with_stats=True)
        torch.cuda.synchronize()
        say(f"async: replay {rep} (w x {f}): failures {st['n_failed']}")
        assert st["n_failed"] > 0 and st["path"] == 0
        assert np.array_equal(got[0], _np(ref_idx)), rep
        assert np.array_equal(got[1].view(np.uint32), _np(ref_sc).view(np.uint32)), rep
        assert got[2][0] == 0 and got[2][1] == st["n_failed"], (rep, got[2])


def test_binding_rejects_short_outputs_before_any_launch(hk, tiny):
    d, inp = tiny["dev"], tiny["inp"]
    ws = torch.empty(hk.select_workspace_bytes(d["q"], d["k"], d["w"], inp.k), dtype=torch.uint8,
                     device="cuda")
    status = torch.zeros(hk.ASYNC_STATUS_WORDS, dtype=torch.int32, device="cuda")
    short = (torch.empty((inp.n - 1, inp.k), dtype=torch.int32, device="cuda"),
             torch.empty((inp.n - 1, inp.k), dtype=torch.float32, device="cuda"))
    with pytest.raises(ValueError):
        hk.select_async(d["q"], d["k"], d["w"], inp.k, workspace=ws, out=short, status=status)
    with pytest.raises(ValueError):
        hk.select_noalloc(d["q"], d["k"], d["w"], inp.k, short)
    with pytest.raises(ValueError):
        hk.replay(d["q"], d["k"], d["w"], short[0])
