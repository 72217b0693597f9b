"""Helpers of the GPU parity tests: device transfer of datagen inputs and the
comparators against the fp64 oracle.

Float comparators, per verified query, with S the oracle's fp64 score row,
v its k-th score and tol = 1e-4 * (|v| + 1):
  1. structure: min(k, ctx) distinct indices in [0, t]; scores non-increasing;
     equal scores in ascending position; padding -1 / -inf;
  2. scores: |out[j] - S[idx[j]]| <= 1e-4 * (|S[idx[j]]| + 1);
  3. set: every index the GPU kept but the oracle did not has S >= v - tol,
     and every index the oracle kept but the GPU did not has S <= v + tol.
Integer-valued inputs are compared bit for bit instead.
"""
from __future__ import annotations

import sys

import numpy as np
import torch

import datagen
import oracle

REL = 1e-4


def say(msg: str) -> None:
    print(msg, flush=True)
    sys.stdout.flush()


def to_device(inp: datagen.Inputs, device: str = "cuda") -> dict:
    if inp.dtype == "bf16":
        q = torch.from_numpy(inp.q.view(np.int16)).to(device).view(torch.bfloat16)
        k = torch.from_numpy(inp.k_.view(np.int16)).to(device).view(torch.bfloat16)
        qs = ks = None
    elif inp.dtype == "fp8":
        q = torch.from_numpy(inp.q).to(device).view(torch.float8_e4m3fn)
        k = torch.from_numpy(inp.k_).to(device).view(torch.float8_e4m3fn)
        qs = torch.from_numpy(inp.q_scale).to(device)
        ks = torch.from_numpy(inp.k_scale).to(device)
    else:  # MX: raw code bytes and E8M0 scale bytes; the format goes as fmt=
        q = torch.from_numpy(inp.q).to(device)
        k = torch.from_numpy(inp.k_).to(device)
        qs = torch.from_numpy(inp.q_scale).to(device)
        ks = torch.from_numpy(inp.k_scale).to(device)
    w = torch.from_numpy(inp.w).to(device)
    out = dict(q=q, k=k, w=w, q_scale=qs, k_scale=ks)
    if inp.dtype in ("mxfp8", "mxfp4"):
        out["fmt"] = inp.dtype
    return out


def oracle_rows(inp: datagen.Inputs, queries) -> list:
    dec = oracle.Decoded(inp)
    return [oracle.score_row(dec, int(i)) for i in queries]


def assert_exact(inp, queries, idx_gpu: np.ndarray, score_gpu: np.ndarray, ref_idx, ref_val):
    """Bit-exact comparison (integer-valued inputs: fp32 scores are exact)."""
    for r, i in enumerate(queries):
        if not np.array_equal(idx_gpu[r], ref_idx[r]):
            bad = np.nonzero(idx_gpu[r] != ref_idx[r])[0]
            raise AssertionError(f"query {i}: {bad.size} index mismatches, first at {bad[0]}: "
                                 f"gpu {idx_gpu[r, bad[0]]} oracle {ref_idx[r, bad[0]]}")
        ok = ref_idx[r] >= 0
        assert np.array_equal(score_gpu[r][ok].astype(np.float64), ref_val[r][ok]), f"query {i}"
        assert np.all(np.isneginf(score_gpu[r][~ok])), f"query {i} padding"


def assert_structure(t: int, k: int, idx: np.ndarray, score: np.ndarray, where: str,
                     first: int = 0):
    """Structure of one output row; the query sees keys first..t."""
    ctx = max(0, t - first + 1)
    m = min(k, ctx)
    kept = idx[:m]
    assert np.all(idx[m:] == -1) and np.all(np.isneginf(score[m:])), f"{where}: padding"
    if m == 0:
        return
    assert kept.min() >= first and kept.max() <= t, f"{where}: index out of range"
    assert np.unique(kept).size == m, f"{where}: duplicate indices"
    sc = score[:m]
    assert np.all(np.diff(sc) <= 0), f"{where}: scores not non-increasing"
    same = np.diff(sc) == 0
    assert np.all(np.diff(kept)[same] > 0), f"{where}: ties not in ascending position"


def assert_float_row(t: int, k: int, row: np.ndarray, idx: np.ndarray, score: np.ndarray,
                     where: str, replay: np.ndarray | None = None, first: int = 0):
    """Float comparators for one query seeing keys first..t; ``row`` is the
    oracle's score row over that context (entry j = key first + j)."""
    assert_structure(t, k, idx, score, where, first)
    m = min(k, t - first + 1)
    kept = idx[:m].astype(np.int64) - first
    ref = row[kept]
    err = np.abs(score[:m].astype(np.float64) - ref)
    assert np.all(err <= REL * (np.abs(ref) + 1.0)), f"{where}: score error {err.max():.3g}"
    if replay is not None:
        rerr = np.abs(replay[:m].astype(np.float64) - ref)
        assert np.all(rerr <= REL * (np.abs(ref) + 1.0)), f"{where}: replay error {rerr.max():.3g}"
    oidx, oval = oracle.exact_topk(row, k)
    v = oval[m - 1]
    tol = REL * (abs(v) + 1.0)
    g, o = set(kept.tolist()), set(oidx[:m].tolist())
    extra = np.fromiter(g - o, dtype=np.int64)
    missing = np.fromiter(o - g, dtype=np.int64)
    assert np.all(row[extra] >= v - tol), f"{where}: kept a key below the k-th score"
    assert np.all(row[missing] <= v + tol), f"{where}: dropped a key above the k-th score"
    return len(extra)
