"""hytopk_select_noalloc through the C ABI: the select entry point for callers
that cannot allocate device memory, with the library's static scratch as its
workspace.  Two calls in a row (the second on a smaller problem, so stale
scratch contents from the first call are present) must return the bits that
hytopk_select returns with a caller-allocated workspace; a problem that needs
more than the static scratch is refused before any launch."""
import ctypes

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


def _both(hk, inp, params):
    d = to_device(inp)
    ws_need = hk.select_workspace_bytes(d["q"], d["k"], d["w"], inp.k, params=params)
    assert 0 < ws_need <= hk.NOALLOC_SCRATCH_BYTES
    ref_idx, ref_sc, ref_st = hk.select(d["q"], d["k"], d["w"], inp.k, params=params,
                                        with_stats=True)
    idx = torch.full((inp.n, inp.k), 7, dtype=torch.int32, device="cuda")
    sc = torch.full((inp.n, inp.k), 7.0, dtype=torch.float32, device="cuda")
    _, _, st = hk.select_noalloc(d["q"], d["k"], d["w"], inp.k, (idx, sc), params=params,
                                 with_stats=True)
    torch.cuda.synchronize()
    assert np.array_equal(idx.cpu().numpy(), ref_idx.cpu().numpy())
    assert np.array_equal(sc.cpu().numpy().view(np.uint32), ref_sc.cpu().numpy().view(np.uint32))
    assert st == ref_st
    return st


def test_noalloc_matches_select_on_two_calls(hk):
    # first call: the Tiny workload with a candidate cap that sends some
    # queries through recovery (their score rows and the split row top-k
    # live in the static scratch)
    say("noalloc: tiny L=4096 n=256 H=4 d=64 k=256, cap 785")
    big = datagen.make("tiny")
    st1 = _both(hk, big, {"cap": 785})  # about 20 of the 256 counts exceed it
    say(f"noalloc: first call stats {st1}")
    assert st1["n_failed"] > 0 and st1["path"] == 0
    # second call: a smaller problem on the same scratch
    say("noalloc: L=1500 n=40 H=64 d=128 k=64")
    small = datagen.make_custom("noalloc_small", L=1500, n=40, H=64, d=128, k=64, dist="int",
                                seed=23)
    st2 = _both(hk, small, None)
    say(f"noalloc: second call stats {st2}")
    assert st2["n_failed"] == 0


def test_noalloc_refuses_problems_beyond_the_scratch(hk):
    lib = hk.load_library()
    prob = hk.Problem(1 << 20, 8192, (1 << 20) - 8192, 64, 128, 2048, hk.BF16, None, None)
    assert lib.hytopk_select_workspace(ctypes.byref(prob), None) > hk.NOALLOC_SCRATCH_BYTES
    fake = ctypes.c_void_p(0x1000)
    rc = lib.hytopk_select_noalloc(ctypes.byref(prob), None, fake, None, fake, None, fake, fake,
                                   None, None, None)
    assert rc == -3
    assert "static scratch" in lib.hytopk_last_error().decode()
