"""Exact top-k indexer selection (HyTopK) and selection replay on MI355X.

A thin ctypes binding over ``libhytopk.so`` (``include/hytopk.h``): it only
marshals torch tensors into pointers and sizes; every step of the selection
runs in the library's HIP kernels on the caller's current stream.  The
library must be built (``python -m exact_top_token_amd.build``); nothing here
falls back to a CPU or PyTorch implementation.
"""
from __future__ import annotations

import ctypes
import os

__all__ = [
    "Problem", "Params", "Stats", "load_library", "library_path", "select", "replay",
    "baseline_select", "select_workspace_bytes", "baseline_workspace_bytes", "HytopkError",
    "EXPORTS", "BF16", "FP8_E4M3", "MXFP8_E4M3", "MXFP4_E2M1", "PATH_AUTO", "PATH_ROWS_ALL", "trace_enable", "trace_read",
    "backward", "backward_workspace_bytes", "select_noalloc", "NOALLOC_SCRATCH_BYTES",
    "select_async", "ASYNC_STATUS_WORDS",
]

BF16, FP8_E4M3, MXFP8_E4M3, MXFP4_E2M1 = 0, 1, 2, 3
_FMT = {"bf16": BF16, "fp8": FP8_E4M3, "mxfp8": MXFP8_E4M3, "mxfp4": MXFP4_E2M1}
PATH_AUTO, PATH_ROWS_ALL = 0, 1
EXPORTS = (
    "hytopk_select_workspace", "hytopk_baseline_workspace", "hytopk_select", "hytopk_replay",
    "hytopk_baseline_select", "hytopk_backward_workspace", "hytopk_backward",
    "hytopk_status_string", "hytopk_last_error", "hytopk_trace_enable", "hytopk_trace_read",
    "hytopk_select_noalloc", "hytopk_select_async",
)
NOALLOC_SCRATCH_BYTES = 64 << 20  # HYTOPK_NOALLOC_SCRATCH_BYTES


class Problem(ctypes.Structure):
    _fields_ = [("L", ctypes.c_int64), ("n", ctypes.c_int64), ("q_start", ctypes.c_int64),
                ("H", ctypes.c_int32), ("d", ctypes.c_int32), ("k", ctypes.c_int32),
                ("dtype", ctypes.c_int32), ("q_pos", ctypes.c_void_p), ("q_first", ctypes.c_void_p)]


class Params(ctypes.Structure):
    _fields_ = [(f, ctypes.c_int32) for f in
                ("m_min", "m_max", "m_div", "oversample", "cap", "max_recover", "force_path",
                 "rows_chunk")]


class Stats(ctypes.Structure):
    _fields_ = [("n_overflow", ctypes.c_int32), ("n_underk", ctypes.c_int32),
                ("n_failed", ctypes.c_int32), ("full_rescore", ctypes.c_int32),
                ("cand_total", ctypes.c_int64), ("cand_max", ctypes.c_int32),
                ("path", ctypes.c_int32), ("failed_queries", ctypes.POINTER(ctypes.c_int32)),
                ("failed_capacity", ctypes.c_int32), ("reserved", ctypes.c_int32)]

    def as_dict(self) -> dict:
        return {f: getattr(self, f) for f, _ in self._fields_
                if f not in ("failed_queries", "failed_capacity", "reserved")}


class TraceEntry(ctypes.Structure):
    _fields_ = [("name", ctypes.c_char * 32), ("launches", ctypes.c_int32),
                ("total_ms", ctypes.c_double)]


class HytopkError(RuntimeError):
    def __init__(self, status: int, msg: str):
        super().__init__(f"hytopk status {status}: {msg}")
        self.status = status


_LIB = None


def library_path() -> str:
    return os.environ.get("HYTOPK_LIBRARY",
                          os.path.join(os.path.dirname(os.path.abspath(__file__)), "libhytopk.so"))


def load_library():
    """Load libhytopk.so (raises if it has not been built)."""
    global _LIB
    if _LIB is not None:
        return _LIB
    path = library_path()
    if not os.path.exists(path):
        raise RuntimeError(f"{path} is missing: build it with `python -m exact_top_token_amd.build`")
    lib = ctypes.CDLL(path)
    P, vp, sz = ctypes.POINTER, ctypes.c_void_p, ctypes.c_size_t
    lib.hytopk_select_workspace.argtypes = [P(Problem), P(Params)]
    lib.hytopk_select_workspace.restype = sz
    lib.hytopk_baseline_workspace.argtypes = [P(Problem)]
    lib.hytopk_baseline_workspace.restype = sz
    lib.hytopk_select.argtypes = [P(Problem), P(Params), vp, vp, vp, vp, vp, vp, vp, vp, sz, vp,
                                  P(Stats)]
    lib.hytopk_select.restype = ctypes.c_int
    lib.hytopk_select_noalloc.argtypes = [P(Problem), P(Params), vp, vp, vp, vp, vp, vp, vp, vp,
                                          P(Stats)]
    lib.hytopk_select_noalloc.restype = ctypes.c_int
    lib.hytopk_select_async.argtypes = [P(Problem), P(Params), vp, vp, vp, vp, vp, vp, vp, vp, sz,
                                        vp, vp]
    lib.hytopk_select_async.restype = ctypes.c_int
    lib.hytopk_replay.argtypes = [P(Problem), vp, vp, vp, vp, vp, vp, vp, vp]
    lib.hytopk_replay.restype = ctypes.c_int
    lib.hytopk_baseline_select.argtypes = [P(Problem), vp, vp, vp, vp, vp, vp, vp, vp, sz, vp]
    lib.hytopk_baseline_select.restype = ctypes.c_int
    lib.hytopk_backward_workspace.argtypes = [P(Problem)]
    lib.hytopk_backward_workspace.restype = sz
    lib.hytopk_backward.argtypes = [P(Problem), vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, sz, vp]
    lib.hytopk_backward.restype = ctypes.c_int
    lib.hytopk_status_string.argtypes = [ctypes.c_int]
    lib.hytopk_status_string.restype = ctypes.c_char_p
    lib.hytopk_last_error.argtypes = []
    lib.hytopk_last_error.restype = ctypes.c_char_p
    lib.hytopk_trace_enable.argtypes = [ctypes.c_int]
    lib.hytopk_trace_enable.restype = ctypes.c_int
    lib.hytopk_trace_read.argtypes = [P(TraceEntry), ctypes.c_int]
    lib.hytopk_trace_read.restype = ctypes.c_int
    _LIB = lib
    return lib


def _check(rc: int) -> None:
    if rc != 0:
        lib = load_library()
        raise HytopkError(rc, lib.hytopk_last_error().decode() or lib.hytopk_status_string(rc).decode())


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _need(t, name: str, shape, dtype, device) -> None:
    """The library writes or reads these buffers by the problem's sizes, so
    a caller-given tensor must have exactly that shape and dtype, be
    contiguous and sit on the inputs' device."""
    if (tuple(t.shape) != tuple(shape) or t.dtype != dtype or not t.is_contiguous()
            or t.device != device):
        raise ValueError(f"{name} must be a contiguous {dtype} tensor of shape {tuple(shape)} "
                         f"on {device}, got {t.dtype} {tuple(t.shape)} on {t.device}")


def _workspace(t, device):
    """Workspace: contiguous uint8 on the inputs' device (its size is checked by the library)."""
    import torch
    if t.dtype != torch.uint8 or t.dim() != 1 or not t.is_contiguous() or t.device != device:
        raise ValueError(f"workspace must be a contiguous 1-D uint8 tensor on {device}")
    return t


def _scales(prob, q, q_scale, k_scale) -> None:
    """Per-token fp32 scales (FP8) or E8M0 bytes per 32 elements (MX)."""
    import torch
    if prob.dtype == BF16:
        if q_scale is not None or k_scale is not None:
            raise ValueError("bf16 inputs take no q_scale / k_scale")
        return
    if q_scale is None or k_scale is None:
        raise ValueError("fp8 and MX inputs need q_scale and k_scale")
    if prob.dtype == FP8_E4M3:
        _need(q_scale, "q_scale", (prob.n,), torch.float32, q.device)
        _need(k_scale, "k_scale", (prob.L,), torch.float32, q.device)
    else:
        _need(q_scale, "q_scale", (prob.n, prob.H, prob.d // 32), torch.uint8, q.device)
        _need(k_scale, "k_scale", (prob.L, prob.d // 32), torch.uint8, q.device)


def _outputs(out, prob, device):
    import torch
    idx, score = out
    _need(idx, "out[0] (indices)", (prob.n, prob.k), torch.int32, device)
    if score is not None:
        _need(score, "out[1] (scores)", (prob.n, prob.k), torch.float32, device)
    return idx, score


def _dtype_code(q, fmt=None) -> int:
    """Storage format: ``fmt`` ("bf16", "fp8", "mxfp8", "mxfp4") when given,
    else bf16 or per-token FP8 from the tensor dtype."""
    import torch
    if fmt is not None:
        return _FMT[fmt]
    if q.dtype == torch.bfloat16:
        return BF16
    if q.dtype in (torch.float8_e4m3fn, torch.uint8):
        return FP8_E4M3
    raise TypeError(f"q/k must be bfloat16 or float8_e4m3fn, got {q.dtype}")


def _problem(q, k, w, topk: int, q_start, q_pos=None, q_first=None, fmt=None) -> Problem:
    """q [n][H][d] and k [L][d] (MXFP4: the last axis holds d/2 bytes)."""
    import torch
    code = _dtype_code(q, fmt)
    n, H, dq = q.shape
    d = 2 * dq if code == MXFP4_E2M1 else dq
    L = k.shape[0]
    if k.shape[1] != dq or tuple(w.shape) != (n, H):
        raise ValueError("shapes must be q [n][H][d], k [L][d], w [n][H]")
    for t in (q, k, w):
        if not t.is_cuda or not t.is_contiguous() or t.device != q.device:
            raise ValueError("q, k and w must be contiguous and on the same GPU")
    if w.dtype != torch.float32:
        raise ValueError("w must be float32")
    if k.dtype != q.dtype or (code in (MXFP8_E4M3, MXFP4_E2M1) and q.dtype != torch.uint8):
        raise ValueError("q and k must share a dtype (uint8 codes for the MX formats)")
    for t in (q_pos, q_first):
        if t is not None and (t.dtype != torch.int32 or tuple(t.shape) != (n,)
                              or t.device != q.device or not t.is_contiguous()):
            raise ValueError("q_pos / q_first must be contiguous int32 [n] tensors on the GPU")
    if q_start is None:
        q_start = 0 if q_pos is not None else L - n
    return Problem(L, n, int(q_start), H, d, int(topk), code,
                   None if q_pos is None else q_pos.data_ptr(),
                   None if q_first is None else q_first.data_ptr())


def _params(params) -> Params | None:
    if params is None:
        return None
    if isinstance(params, Params):
        return params
    p = Params()
    for key, val in dict(params).items():
        setattr(p, key, int(val))
    return p


def _stream(t):
    import torch
    return ctypes.c_void_p(torch.cuda.current_stream(t.device).cuda_stream)


def trace_enable(on: bool = True) -> bool:
    """Bracket every library launch with hipEvents (clears the totals)."""
    return bool(load_library().hytopk_trace_enable(1 if on else 0))


def trace_read() -> dict:
    """{phase: (launches, total_ms)} accumulated since tracing was enabled."""
    lib = load_library()
    n = lib.hytopk_trace_read(None, 0)
    if n < 0:
        _check(n)
    arr = (TraceEntry * max(n, 1))()
    n = lib.hytopk_trace_read(arr, n)
    if n < 0:
        _check(n)
    return {arr[i].name.decode(): (arr[i].launches, arr[i].total_ms) for i in range(n)}


def select_workspace_bytes(q, k, w, topk: int, q_start=None, params=None, q_pos=None,
                           q_first=None, fmt=None) -> int:
    lib = load_library()
    prob = _problem(q, k, w, topk, q_start, q_pos, q_first, fmt)
    prm = _params(params)
    return int(lib.hytopk_select_workspace(ctypes.byref(prob), ctypes.byref(prm) if prm else None))


def baseline_workspace_bytes(q, k, w, topk: int, q_start=None, fmt=None) -> int:
    lib = load_library()
    return int(lib.hytopk_baseline_workspace(ctypes.byref(_problem(q, k, w, topk, q_start,
                                                                   fmt=fmt))))


def select(q, k, w, topk: int, *, q_scale=None, k_scale=None, q_start=None, params=None,
           workspace=None, out=None, with_stats: bool = False, q_pos=None, q_first=None,
           fmt=None):
    """Exact top-k per query (HyTopK).  Returns (idx int32 [n][k], score fp32
    [n][k]) and, with ``with_stats``, a dict of what the call did.  q_pos /
    q_first (int32 [n] on the GPU, optional) give each query's position and
    the first key of its context (packed sequences).  ``fmt`` selects the MX
    formats ("mxfp8", "mxfp4"; q_scale / k_scale then hold E8M0 bytes)."""
    import torch
    lib = load_library()
    prob = _problem(q, k, w, topk, q_start, q_pos, q_first, fmt)
    _scales(prob, q, q_scale, k_scale)
    prm = _params(params)
    need = int(lib.hytopk_select_workspace(ctypes.byref(prob), ctypes.byref(prm) if prm else None))
    if need == 0:
        _check(lib.hytopk_select(ctypes.byref(prob), ctypes.byref(prm) if prm else None,
                                 *([None] * 8), 0, None, None))
    if workspace is None:
        workspace = torch.empty(need, dtype=torch.uint8, device=q.device)
    _workspace(workspace, q.device)
    if out is None:
        idx = torch.empty((prob.n, prob.k), dtype=torch.int32, device=q.device)
        score = torch.empty((prob.n, prob.k), dtype=torch.float32, device=q.device)
    else:
        idx, score = _outputs(out, prob, q.device)
    st = Stats()
    failed_buf = None
    if with_stats:
        failed_buf = (ctypes.c_int32 * int(prob.n))()
        st.failed_queries = ctypes.cast(failed_buf, ctypes.POINTER(ctypes.c_int32))
        st.failed_capacity = int(prob.n)
    _check(lib.hytopk_select(ctypes.byref(prob), ctypes.byref(prm) if prm else None, _ptr(q),
                             _ptr(q_scale), _ptr(k), _ptr(k_scale), _ptr(w), _ptr(idx), _ptr(score),
                             _ptr(workspace), workspace.numel(), _stream(q), ctypes.byref(st)))
    if not with_stats:
        return idx, score
    d = st.as_dict()
    d["failed"] = [failed_buf[i] for i in range(min(st.n_failed, int(prob.n)))]
    return idx, score, d


def select_noalloc(q, k, w, topk: int, out, *, q_scale=None, k_scale=None, q_start=None,
                   params=None, q_pos=None, q_first=None, fmt=None, with_stats: bool = False):
    """hytopk_select_noalloc: select into the caller's ``out`` = (idx, score)
    tensors with the library's static scratch as workspace (no allocation on
    the device).  Returns ``out`` and, with ``with_stats``, the stats dict."""
    lib = load_library()
    prob = _problem(q, k, w, topk, q_start, q_pos, q_first, fmt)
    _scales(prob, q, q_scale, k_scale)
    prm = _params(params)
    idx, score = _outputs(out, prob, q.device)
    st = Stats()
    failed_buf = None
    if with_stats:
        failed_buf = (ctypes.c_int32 * int(prob.n))()
        st.failed_queries = ctypes.cast(failed_buf, ctypes.POINTER(ctypes.c_int32))
        st.failed_capacity = int(prob.n)
    _check(lib.hytopk_select_noalloc(ctypes.byref(prob), ctypes.byref(prm) if prm else None,
                                     _ptr(q), _ptr(q_scale), _ptr(k), _ptr(k_scale), _ptr(w),
                                     _ptr(idx), _ptr(score), _stream(q), ctypes.byref(st)))
    if not with_stats:
        return idx, score
    d = st.as_dict()
    d["failed"] = [failed_buf[i] for i in range(min(st.n_failed, int(prob.n)))]
    return idx, score, d


ASYNC_STATUS_WORDS = 8


def select_async(q, k, w, topk: int, *, workspace, out, status, q_scale=None, k_scale=None,
                 q_start=None, params=None, q_pos=None, q_first=None, fmt=None):
    """hytopk_select_async: select into ``out`` = (idx, score) with the caller's
    ``workspace`` (select_workspace_bytes) and no host synchronisation, so the
    call can be recorded in a CUDA/HIP graph.  ``status`` (int32
    [ASYNC_STATUS_WORDS] on the GPU) receives the device status words:
    status[0] == 1 means more than max_recover queries failed and their rows
    are not final.  Returns ``out``."""
    import torch
    lib = load_library()
    prob = _problem(q, k, w, topk, q_start, q_pos, q_first, fmt)
    _scales(prob, q, q_scale, k_scale)
    prm = _params(params)
    idx, score = _outputs(out, prob, q.device)
    _workspace(workspace, q.device)
    if (status.dtype != torch.int32 or status.numel() < ASYNC_STATUS_WORDS
            or not status.is_contiguous() or status.device != q.device):
        raise ValueError("status must be a contiguous int32 tensor of ASYNC_STATUS_WORDS entries "
                         "on the inputs' device")
    _check(lib.hytopk_select_async(ctypes.byref(prob), ctypes.byref(prm) if prm else None,
                                   _ptr(q), _ptr(q_scale), _ptr(k), _ptr(k_scale), _ptr(w),
                                   _ptr(idx), _ptr(score), _ptr(workspace), workspace.numel(),
                                   _stream(q), _ptr(status)))
    return idx, score


def replay(q, k, w, idx, *, q_scale=None, k_scale=None, q_start=None, out=None, fmt=None):
    """Selection replay: scores of the saved indices idx [n][k] (-inf at idx < 0)."""
    import torch
    lib = load_library()
    prob = _problem(q, k, w, idx.shape[1], q_start, fmt=fmt)
    _scales(prob, q, q_scale, k_scale)
    _need(idx, "idx", (prob.n, prob.k), torch.int32, q.device)
    if out is None:
        out = torch.empty(idx.shape, dtype=torch.float32, device=q.device)
    _need(out, "out", (prob.n, prob.k), torch.float32, q.device)
    _check(lib.hytopk_replay(ctypes.byref(prob), _ptr(q), _ptr(q_scale), _ptr(k), _ptr(k_scale),
                             _ptr(w), _ptr(idx), _ptr(out), _stream(q)))
    return out


def baseline_select(q, k, w, topk: int, *, q_scale=None, k_scale=None, q_start=None,
                    workspace=None, out=None, q_pos=None, q_first=None, fmt=None):
    """The materialise-then-top-k route (writes the n x L fp32 score table)."""
    import torch
    lib = load_library()
    prob = _problem(q, k, w, topk, q_start, q_pos, q_first, fmt)
    _scales(prob, q, q_scale, k_scale)
    need = int(lib.hytopk_baseline_workspace(ctypes.byref(prob)))
    if workspace is None:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=q.device)
    _workspace(workspace, q.device)
    if out is None:
        idx = torch.empty((prob.n, prob.k), dtype=torch.int32, device=q.device)
        score = torch.empty((prob.n, prob.k), dtype=torch.float32, device=q.device)
    else:
        idx, score = _outputs(out, prob, q.device)
    _check(lib.hytopk_baseline_select(ctypes.byref(prob), _ptr(q), _ptr(q_scale), _ptr(k),
                                      _ptr(k_scale), _ptr(w), _ptr(idx), _ptr(score),
                                      _ptr(workspace), workspace.numel(), _stream(q)))
    return idx, score


def backward_workspace_bytes(q, k, w, topk: int, q_start=None, fmt=None) -> int:
    lib = load_library()
    return int(lib.hytopk_backward_workspace(ctypes.byref(_problem(q, k, w, topk, q_start,
                                                                   fmt=fmt))))


def backward(q, k, w, idx, d_score, *, q_scale=None, k_scale=None, q_start=None,
             want=("dq", "dw", "dk"), workspace=None, out=None, fmt=None):
    """Indexer backward at the replayed entries idx [n][k] with upstream
    gradient d_score [n][k] (fp32).  Returns a dict with the requested fp32
    gradients: dq [n][H][d], dw [n][H], dk [L][d] (for FP8 / MX inputs, with
    respect to the decoded values)."""
    import torch
    lib = load_library()
    prob = _problem(q, k, w, idx.shape[1], q_start, fmt=fmt)
    _scales(prob, q, q_scale, k_scale)
    _need(idx, "idx", (prob.n, prob.k), torch.int32, q.device)
    _need(d_score, "d_score", (prob.n, prob.k), torch.float32, q.device)
    res = dict(out or {})
    shapes = {"dq": (prob.n, prob.H, prob.d), "dw": (prob.n, prob.H), "dk": (prob.L, prob.d)}
    if set(res) - set(shapes):
        raise ValueError(f"unknown gradient names in out: {sorted(set(res) - set(shapes))}")
    for name in want:
        if name not in res:
            res[name] = torch.empty(shapes[name], dtype=torch.float32, device=q.device)
    for name, t in res.items():
        _need(t, name, shapes[name], torch.float32, q.device)
    if ("dk" in res or prob.dtype != BF16) and workspace is None:
        need = int(lib.hytopk_backward_workspace(ctypes.byref(prob)))
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=q.device)
    if workspace is not None:
        _workspace(workspace, q.device)
    _check(lib.hytopk_backward(ctypes.byref(prob), _ptr(q), _ptr(q_scale), _ptr(k), _ptr(k_scale),
                               _ptr(w), _ptr(idx), _ptr(d_score), _ptr(res.get("dq")),
                               _ptr(res.get("dw")), _ptr(res.get("dk")), _ptr(workspace),
                               0 if workspace is None else workspace.numel(), _stream(q)))
    return res
