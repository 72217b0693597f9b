"""Two host threads, each with its own stream, inputs and workspace, call the
library at the same time: every result must equal the same call made alone
(the library keeps no per-call state outside the caller's buffers; its
per-kernel LDS limits and tracer are shared and guarded)."""
import threading

import numpy as np
import pytest
import torch

import datagen
from gpu_util import say, to_device

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def hk():
    import exact_top_token_amd as m
    m.load_library()
    return m


def _problems():
    a = datagen.make("tiny")
    b = datagen.make_custom("streams_b", 6000, 300, 64, 128, 512, dist="int", seed=41)
    return [a, b]


def _run(hk, dv, inp, reps, out, err):
    try:
        res = []
        for _ in range(reps):
            idx, sc = hk.select(dv["q"], dv["k"], dv["w"], inp.k)
            rep = hk.replay(dv["q"], dv["k"], dv["w"], idx)
            res.append((idx, sc, rep))
        torch.cuda.current_stream().synchronize()
        out.extend((i.cpu().numpy(), s.cpu().numpy(), r.cpu().numpy()) for i, s, r in res)
    except Exception as e:  # reported by the main thread
        err.append(e)


def test_concurrent_calls_on_two_streams_equal_the_calls_alone(hk):
    probs = _problems()
    devs = [to_device(p) for p in probs]
    alone = []
    for p, dv in zip(probs, devs):
        idx, sc = hk.select(dv["q"], dv["k"], dv["w"], p.k)
        rep = hk.replay(dv["q"], dv["k"], dv["w"], idx)
        torch.cuda.synchronize()
        alone.append((idx.cpu().numpy(), sc.cpu().numpy(), rep.cpu().numpy()))
    say("streams: two threads x 4 select + replay calls, each on its own stream")
    streams = [torch.cuda.Stream(), torch.cuda.Stream()]
    outs, errs = [[], []], []

    def worker(j):
        with torch.cuda.stream(streams[j]):
            _run(hk, devs[j], probs[j], 4, outs[j], errs)

    ths = [threading.Thread(target=worker, args=(j,)) for j in range(2)]
    for t in ths:
        t.start()
    for t in ths:
        t.join(timeout=120)
    assert not any(t.is_alive() for t in ths), "a worker did not finish"
    torch.cuda.synchronize()
    assert not errs, errs
    for j in range(2):
        assert len(outs[j]) == 4
        for idx, sc, rep in outs[j]:
            assert np.array_equal(idx, alone[j][0])
            assert np.array_equal(sc.view(np.uint32), alone[j][1].view(np.uint32))
            assert np.array_equal(rep.view(np.uint32), alone[j][2].view(np.uint32))
