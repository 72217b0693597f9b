"""The C ABI without a GPU: the library loads, exports every entry point that
include/hytopk.h declares, and rejects bad arguments before touching HIP."""
import ctypes
import os
import re
import subprocess

import pytest

import exact_top_token_amd as hk

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "hytopk.h")


def _declared():
    src = open(HEADER).read()
    return sorted(set(re.findall(r"\b(hytopk_[a-z_]+)\s*\(", src)))


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(hk.library_path()):
        pytest.fail("libhytopk.so is not built: run `python -m exact_top_token_amd.build`")
    return hk.load_library()


def test_header_declares_the_binding_exports():
    assert _declared() == sorted(hk.EXPORTS)


def test_library_exports_every_declared_symbol(lib):
    out = subprocess.run(["nm", "-D", "--defined-only", hk.library_path()],
                         capture_output=True, text=True, check=True).stdout
    syms = {line.split()[-1] for line in out.splitlines() if line.strip()}
    for name in _declared():
        assert name in syms, name
        assert getattr(lib, name) is not None


def _prob(**kw):
    base = dict(L=1 << 20, n=8192, q_start=(1 << 20) - 8192, H=64, d=128, k=2048, dtype=hk.BF16)
    base.update(kw)
    return hk.Problem(**base)


def test_workspace_sizes_match_the_worked_example(lib):
    p = _prob()
    # the conventional table: 8192 x 1,048,576 fp32 = 32 GiB per layer
    assert lib.hytopk_baseline_workspace(ctypes.byref(p)) == 32 << 30
    ws = lib.hytopk_select_workspace(ctypes.byref(p), None)
    # candidates at cap = 6k: 8192 x 12288 x 8 bytes (768 MiB), plus the
    # recovery rows (max_recover = 64 rows of 2^20 fp32 scores: 256 MiB) and
    # the split row top-k's scratch; the score table (32 GiB) is what the
    # method avoids
    cand, rows = 8192 * 12288 * 8, 64 * (1 << 20) * 4
    assert cand + rows <= ws < int(1.1 * (1 << 30))
    assert ws % 256 == 0
    # the rows buffer follows rows_chunk
    prm = hk.Params(rows_chunk=16)
    ws16 = lib.hytopk_select_workspace(ctypes.byref(p), ctypes.byref(prm))
    assert cand + 16 * (1 << 20) * 4 <= ws16 < ws - 48 * (1 << 20) * 4 + (1 << 20)


@pytest.mark.parametrize("kw,code", [
    (dict(n=0), -1), (dict(q_start=(1 << 20) - 8191), -1), (dict(k=0), -1),
    (dict(k=4097), -2), (dict(H=65), -2), (dict(d=96), -2), (dict(dtype=1, d=64), -2),
    (dict(dtype=7), -1), (dict(L=1 << 31, q_start=(1 << 31) - 8192), -2),
    (dict(n=1 << 31, q_start=0, L=(1 << 31) - 1, q_pos=0x1000), -2),  # q_pos: no q_start + n check
])
def test_invalid_problems_are_rejected_before_any_launch(lib, kw, code):
    p = _prob(**kw)
    assert lib.hytopk_select_workspace(ctypes.byref(p), None) == 0
    rc = lib.hytopk_select(ctypes.byref(p), None, *([None] * 8), 0, None, None)
    assert rc == code
    assert lib.hytopk_last_error().decode()
    rc = lib.hytopk_replay(ctypes.byref(p), *([None] * 8))
    assert rc == code


def test_null_pointers_and_workspace_errors(lib):
    p = _prob()
    fake = ctypes.c_void_p(0x1000)
    assert lib.hytopk_select(ctypes.byref(p), None, None, None, fake, None, fake, fake, None,
                             fake, 1 << 40, None, None) == -1
    # workspace too small / misaligned -> -3, checked before any HIP call
    assert lib.hytopk_select(ctypes.byref(p), None, fake, None, fake, None, fake, fake, None,
                             fake, 16, None, None) == -3
    assert lib.hytopk_select(ctypes.byref(p), None, fake, None, fake, None, fake, fake, None,
                             ctypes.c_void_p(0x1001), 1 << 40, None, None) == -3
    assert lib.hytopk_baseline_select(ctypes.byref(p), fake, None, fake, None, fake, fake, None,
                                      fake, 1 << 20, None) == -3
    # fp8 without scales -> -1
    p8 = _prob(dtype=hk.FP8_E4M3)
    assert lib.hytopk_replay(ctypes.byref(p8), fake, None, fake, None, fake, fake, fake, None) == -1
    pmx4 = _prob(dtype=hk.MXFP4_E2M1)
    assert lib.hytopk_select(ctypes.byref(pmx4), None, fake, None, fake, fake, fake, fake, None,
                             fake, 1 << 40, None, None) == -1
    assert "scale" in lib.hytopk_last_error().decode()
    assert lib.hytopk_status_string(-3).decode() == "bad workspace"
    # misaligned inputs -> -1, before any HIP call: q and k 16-byte aligned,
    # w and the scale arrays 4-byte aligned
    odd16, odd4 = ctypes.c_void_p(0x1008), ctypes.c_void_p(0x1002)
    assert lib.hytopk_select(ctypes.byref(p), None, odd16, None, fake, None, fake, fake, None,
                             fake, 1 << 40, None, None) == -1
    assert lib.hytopk_replay(ctypes.byref(p), fake, None, odd16, None, fake, fake, fake, None) == -1
    assert lib.hytopk_replay(ctypes.byref(p), fake, None, fake, None, odd4, fake, fake, None) == -1
    pmx = _prob(dtype=hk.MXFP8_E4M3)
    assert lib.hytopk_replay(ctypes.byref(pmx), fake, fake, fake, odd4, fake, fake, fake, None) == -1
    assert "aligned" in lib.hytopk_last_error().decode()
    # the asynchronous select needs a 4-byte aligned device status array
    assert lib.hytopk_select_async(ctypes.byref(p), None, fake, None, fake, None, fake, fake, None,
                                   fake, 1 << 40, None, None) == -1
    assert "status" in lib.hytopk_last_error().decode()
    assert lib.hytopk_select_async(ctypes.byref(p), None, fake, None, fake, None, fake, fake, None,
                                   fake, 1 << 40, None, odd4) == -1
    assert lib.hytopk_select_async(ctypes.byref(p), None, fake, None, fake, None, fake, fake, None,
                                   fake, 16, None, fake) == -3


def test_bad_params_are_rejected(lib):
    p = _prob()
    for kw in (dict(cap=20000), dict(m_max=1 << 15), dict(force_path=5), dict(oversample=-1)):
        prm = hk.Params(**kw)
        assert lib.hytopk_select_workspace(ctypes.byref(p), ctypes.byref(prm)) == 0


def test_backward_workspace_and_argument_errors(lib):
    p = _prob()
    ws = lib.hytopk_backward_workspace(ctypes.byref(p))
    # one chunk of 8 GiB of dk rows (all 8192 queries x 2048 entries x 128
    # fp32) plus the key-grouping buffers (4 x 64 MiB and the digit counts)
    assert (8 << 30) <= ws < (8 << 30) + (320 << 20) and ws % 256 == 0
    fake = ctypes.c_void_p(0x1000)
    args = [fake, None, fake, None, fake, fake, fake, fake, fake, fake, fake, 1 << 40, None]
    # fp8 without its scales -> invalid; fp8 needs the workspace (its bf16
    # copies of q and k) even without dk -> -3; both before any launch.
    # NULL idx / d_score -> invalid; small workspace with dk -> -3
    p8 = _prob(dtype=hk.FP8_E4M3)
    assert lib.hytopk_backward(ctypes.byref(p8), *args) == -1
    a = list(args); a[1] = fake; a[3] = fake; a[9] = None; a[10] = None; a[11] = 0
    assert lib.hytopk_backward(ctypes.byref(p8), *a) == -3
    assert lib.hytopk_backward_workspace(ctypes.byref(p8)) == ws + (8192 * 64 + (1 << 20)) * 128 * 2
    a = list(args); a[5] = None
    assert lib.hytopk_backward(ctypes.byref(p), *a) == -1
    a = list(args); a[11] = 16
    assert lib.hytopk_backward(ctypes.byref(p), *a) == -3
    bad = _prob(k=4097)
    assert lib.hytopk_backward_workspace(ctypes.byref(bad)) == 0
    assert lib.hytopk_backward(ctypes.byref(bad), *args) == -2


def test_binding_rejects_mis_sized_caller_buffers():
    """The binding checks every caller-given buffer against the problem's
    sizes before a pointer reaches the library (which cannot see sizes)."""
    import torch
    prob = hk.Problem(L=100, n=4, q_start=96, H=2, d=128, k=8, dtype=hk.FP8_E4M3)
    cpu = torch.device("cpu")
    good = (torch.empty((4, 8), dtype=torch.int32), torch.empty((4, 8), dtype=torch.float32))
    hk._outputs(good, prob, cpu)
    for bad in ((torch.empty((4, 7), dtype=torch.int32), good[1]),
                (good[0], torch.empty((4, 8), dtype=torch.float64)),
                (torch.empty((8, 4), dtype=torch.int32).t(), good[1])):
        with pytest.raises(ValueError):
            hk._outputs(bad, prob, cpu)
    q = torch.empty((4, 2, 128), dtype=torch.uint8)
    hk._scales(prob, q, torch.ones(4), torch.ones(100))
    with pytest.raises(ValueError):
        hk._scales(prob, q, torch.ones(4), torch.ones(99))
    with pytest.raises(ValueError):
        hk._scales(prob, q, None, torch.ones(100))
    prob.dtype = hk.MXFP8_E4M3
    hk._scales(prob, q, torch.ones((4, 2, 4), dtype=torch.uint8), torch.ones((100, 4), dtype=torch.uint8))
    with pytest.raises(ValueError):
        hk._scales(prob, q, torch.ones((4, 2, 4)), torch.ones((100, 4), dtype=torch.uint8))
    prob.dtype = hk.BF16
    with pytest.raises(ValueError):
        hk._scales(prob, q, torch.ones(4), None)
    hk._workspace(torch.empty(64, dtype=torch.uint8), cpu)
    with pytest.raises(ValueError):
        hk._workspace(torch.empty(16, dtype=torch.float32), cpu)
