"""Seeded synthetic inputs for exact top-k indexer selection and selection replay.

This module draws random numbers and encodes them into the storage formats the
selection path reads (bf16 bit patterns, OCP FP8 E4M3 bytes with per-token fp32
scales, fp32 head weights).  It holds none of the method's arithmetic: no
scoring, no thresholds, no selection.  Both the CPU oracle (``oracle/``) and the
HIP path (``exact_top_token_amd``) consume exactly the arrays produced here, so
the two sides read identical bytes.

Workloads (HyScale pages: the GLM-5.1 worked example on the learnaivisually
explainer gives L = 1,048,576 keys, n = 8,192 queries per GPU, k = 2,048; the
smaller shapes keep the same causal structure):

==========  =========  =====  ==  ===  =====  =====================================
name        L          n      H   d    k      values
==========  =========  =====  ==  ===  =====  =====================================
tiny        4,096      256    4   64   256    q,k ints U{-3..3} (bf16), w ints U{1,2}
mid         131,072    2,048  64  128  2,048  q,k ~ N(0,1)/sqrt(d) bf16, w ~ U(0,1)/H
glm1m       1,048,576  8,192  64  128  2,048  as mid
glm1m_fp8   1,048,576  8,192  64  128  2,048  glm1m's fp32 draws, per-token E4M3
glm1m_mxfp8 1,048,576  8,192  64  128  2,048  glm1m's fp32 draws, MX: E4M3 + E8M0 / 32
glm1m_mxfp4 1,048,576  8,192  64  128  2,048  glm1m's fp32 draws, MX: E2M1 + E8M0 / 32
stress_a    1,048,576  8,192  64  128  2,048  clustered keys + planted failures
stress_b    1,048,576  8,192  64  128  2,048  clustered keys + >64 planted failures
==========  =========  =====  ==  ===  =====  =====================================

By default the queries sit at the last n positions: query i has position
``q_start + i`` with ``q_start = L - n`` and sees keys ``0 .. q_start + i``.
``make_packed`` builds the general form: several sequences packed into one key
buffer, queries at chosen positions in any order, each seeing the keys from
its own sequence's first key through its position (``q_pos``, ``q_first``).

Draw order for every config: q, then k, then w, from
``numpy.random.default_rng(seed)``; fp32 draws are rounded to bf16 with
round-to-nearest-even.
"""
from __future__ import annotations

import dataclasses
import math

import numpy as np

__all__ = [
    "CONFIGS", "Inputs", "make", "make_custom", "make_packed", "f32_to_bf16_bits",
    "f32_to_e4m3", "f32_to_e2m1", "quantize_e4m3_per_row", "quantize_mx", "subset_queries",
]

CONFIGS = {
    "tiny": dict(L=4096, n=256, H=4, d=64, k=256, dtype="bf16", dist="int", seed=1001),
    "mid": dict(L=131072, n=2048, H=64, d=128, k=2048, dtype="bf16", dist="normal", seed=1002),
    "glm1m": dict(L=1048576, n=8192, H=64, d=128, k=2048, dtype="bf16", dist="normal", seed=1003),
    "glm1m_fp8": dict(L=1048576, n=8192, H=64, d=128, k=2048, dtype="fp8", dist="normal", seed=1003),
    "glm1m_mxfp8": dict(L=1048576, n=8192, H=64, d=128, k=2048, dtype="mxfp8", dist="normal", seed=1003),
    "glm1m_mxfp4": dict(L=1048576, n=8192, H=64, d=128, k=2048, dtype="mxfp4", dist="normal", seed=1003),
}
STRESS_NAMES = ("stress_a", "stress_b")   # built by datagen.stress


@dataclasses.dataclass
class Inputs:
    """One selection problem in storage form.

    ``q`` is ``[n][H][d]`` and ``k`` is ``[L][d]``: uint16 bf16 bit patterns, or
    uint8 OCP E4M3 codes when ``dtype == "fp8"`` (then ``q_scale[n]`` and
    ``k_scale[L]`` are the fp32 per-token dequantisation scales).  For the MX
    formats ``dtype == "mxfp8"`` / ``"mxfp4"`` the codes are E4M3 bytes or
    E2M1 nibbles packed two per byte (last axis d / 2), and ``q_scale``
    ``[n][H][d/32]`` / ``k_scale`` ``[L][d/32]`` hold E8M0 block scales.  ``w`` is
    ``[n][H]`` fp32.  Query ``i`` sits at position ``q_start + i`` and sees
    keys ``0 ..`` that position, unless ``q_pos`` / ``q_first`` (int32 ``[n]``)
    give its position and the first key of its context explicitly.
    """
    name: str
    L: int
    n: int
    H: int
    d: int
    k: int
    dtype: str
    q: np.ndarray
    k_: np.ndarray
    w: np.ndarray
    q_scale: np.ndarray | None = None
    k_scale: np.ndarray | None = None
    q_pos: np.ndarray | None = None
    q_first: np.ndarray | None = None

    @property
    def q_start(self) -> int:
        return self.L - self.n


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round fp32 values to bf16 (round to nearest, ties to even); return the
    16-bit patterns.  Inputs are finite, so the 32-bit sum cannot wrap."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    lsb = (u >> np.uint32(16)) & np.uint32(1)
    return ((u + np.uint32(0x7FFF) + lsb) >> np.uint32(16)).astype(np.uint16)


def f32_to_e4m3(x: np.ndarray) -> np.ndarray:
    """Encode values to OCP E4M3 codes: round to nearest, ties to even,
    saturating to +-448 (code 0x7E)."""
    x = np.asarray(x, dtype=np.float64)
    a = np.minimum(np.abs(x), 448.0)
    f, E = np.frexp(a)                      # a = f * 2^E, f in [0.5, 1)
    e = E.astype(np.int64) - 1              # a = (2f) * 2^e, 2f in [1, 2)
    normal = (e >= -6) & (a > 0)            # zero takes the subnormal branch
    m = np.rint((2.0 * f - 1.0) * 8.0).astype(np.int64)   # ties to even
    carry = m == 8
    e = np.where(carry, e + 1, e)
    m = np.where(carry, 0, m)
    code_n = ((e + 7) << 3) | m
    code_s = np.rint(a * 512.0).astype(np.int64)            # subnormal: m * 2^-9
    code = np.where(normal, code_n, code_s)
    code = np.minimum(code, 0x7E)
    sign = np.signbit(x).astype(np.int64) << 7
    return (code | sign).astype(np.uint8)


def quantize_e4m3_per_row(x32: np.ndarray) -> tuple[np.ndarray, np.ndarray]:
    """Per-token quantisation: the leading axis is the token.  scale = amax/448
    in fp32 (1 for an all-zero token); codes = E4M3(x / scale)."""
    rows = x32.reshape(x32.shape[0], -1).astype(np.float32)
    amax = np.abs(rows).max(axis=1)
    scale = np.where(amax > 0, amax / np.float32(448.0), np.float32(1.0)).astype(np.float32)
    codes = np.empty(rows.shape, dtype=np.uint8)
    step = max(1, (1 << 24) // max(1, rows.shape[1]))
    for a in range(0, rows.shape[0], step):
        b = min(rows.shape[0], a + step)
        codes[a:b] = f32_to_e4m3(rows[a:b].astype(np.float64) / scale[a:b, None].astype(np.float64))
    return codes.reshape(x32.shape), scale


# OCP Microscaling (MX) formats: blocks of 32 consecutive elements along the
# head dimension share one E8M0 scale 2^(e - 127).  The block scale follows
# the format's recipe: shared exponent = floor(log2(amax)) - emax, where emax
# is the exponent of the element format's largest normal value (E4M3: 448 =
# 1.75 * 2^8, emax 8; E2M1: 6 = 1.5 * 2^2, emax 2); elements are x / 2^shared
# rounded to nearest (ties to even) and saturated.
MX_BLOCK = 32
_MX_EMAX = {"mxfp8": 8, "mxfp4": 2}


def f32_to_e2m1(x: np.ndarray) -> np.ndarray:
    """Encode values to E2M1 codes (0..15: sign bit 3, magnitudes 0, 0.5, 1,
    1.5, 2, 3, 4, 6 for codes 0..7), round to nearest, ties to even code,
    saturating to 6."""
    x = np.asarray(x, dtype=np.float64)
    a = np.minimum(np.abs(x), 6.0)
    code = np.where(a < 2.0, np.rint(2.0 * a),
                    np.where(a < 4.0, np.rint(a) + 2.0, np.rint(a / 2.0) + 4.0)).astype(np.int64)
    sign = np.where(np.signbit(x), 8, 0)
    return (code | sign).astype(np.uint8)


def quantize_mx(x32: np.ndarray, fmt: str) -> tuple[np.ndarray, np.ndarray]:
    """MX quantisation along the last axis (a multiple of 32).  Returns
    (codes, scales): E4M3 bytes (same shape) or E2M1 codes packed two per byte
    (element 2i in the low nibble of byte i; last axis halved), and the E8M0
    scale bytes [..., last / 32]."""
    x = np.asarray(x32, dtype=np.float32)
    shp = x.shape
    if shp[-1] % MX_BLOCK:
        raise ValueError("the last axis must be a multiple of 32")
    nb = shp[-1] // MX_BLOCK
    flat = x.reshape(-1, nb, MX_BLOCK)
    codes = np.empty(flat.shape, dtype=np.uint8)
    scales = np.empty(flat.shape[:2], dtype=np.uint8)
    step = max(1, (1 << 22) // (nb * MX_BLOCK))
    for a in range(0, flat.shape[0], step):
        blk = flat[a:a + step].astype(np.float64)
        amax = np.abs(blk).max(axis=2)
        with np.errstate(divide="ignore"):
            e = np.where(amax > 0, np.floor(np.log2(np.where(amax > 0, amax, 1.0))) - _MX_EMAX[fmt], -127)
        e = np.clip(e, -127, 127).astype(np.int64)
        scales[a:a + step] = (e + 127).astype(np.uint8)
        v = blk / np.exp2(e.astype(np.float64))[:, :, None]
        codes[a:a + step] = f32_to_e4m3(v) if fmt == "mxfp8" else f32_to_e2m1(v)
    codes = codes.reshape(shp)
    if fmt == "mxfp4":
        codes = (codes[..., 0::2] | (codes[..., 1::2] << 4)).astype(np.uint8)
    return codes, scales.reshape(shp[:-1] + (nb,))


def _draw(cfg: dict, rng: np.random.Generator):
    L, n, H, d = cfg["L"], cfg["n"], cfg["H"], cfg["d"]
    if cfg["dist"] == "int":
        q = rng.integers(-3, 4, size=(n, H, d)).astype(np.float32)
        k = rng.integers(-3, 4, size=(L, d)).astype(np.float32)
        w = rng.integers(1, 3, size=(n, H)).astype(np.float32)
    elif cfg["dist"] == "normal":
        s = np.float32(1.0 / math.sqrt(d))
        q = rng.standard_normal((n, H, d), dtype=np.float32) * s
        k = rng.standard_normal((L, d), dtype=np.float32) * s
        w = rng.random((n, H), dtype=np.float32) / np.float32(H)
    else:
        raise ValueError(cfg["dist"])
    return q, k, w


def make_custom(name: str, L: int, n: int, H: int, d: int, k: int, dtype: str = "bf16",
                dist: str = "normal", seed: int = 0) -> Inputs:
    """Draw a problem of any shape with one of the two value recipes."""
    cfg = dict(L=L, n=n, H=H, d=d, k=k, dtype=dtype, dist=dist, seed=seed)
    if not (0 < n <= L):
        raise ValueError("need 0 < n <= L")
    rng = np.random.default_rng(seed)
    q32, k32, w = _draw(cfg, rng)
    if dtype == "bf16":
        return Inputs(name, L, n, H, d, k, dtype, f32_to_bf16_bits(q32), f32_to_bf16_bits(k32), w)
    if dtype == "fp8":
        qc, qs = quantize_e4m3_per_row(q32)
        kc, ks = quantize_e4m3_per_row(k32)
        return Inputs(name, L, n, H, d, k, dtype, qc, kc, w, qs, ks)
    if dtype in ("mxfp8", "mxfp4"):
        qc, qs = quantize_mx(q32, dtype)
        kc, ks = quantize_mx(k32, dtype)
        return Inputs(name, L, n, H, d, k, dtype, qc, kc, w, qs, ks)
    raise ValueError(dtype)


def make(name: str) -> Inputs:
    """The named workload (see the module table)."""
    if name.startswith("stress"):
        from . import stress
        return stress.make(name)
    cfg = CONFIGS[name]
    return make_custom(name, cfg["L"], cfg["n"], cfg["H"], cfg["d"], cfg["k"],
                       cfg["dtype"], cfg["dist"], cfg["seed"])


def make_packed(name: str, seq_lens, chunks, H: int, d: int, k: int, dtype: str = "bf16",
                dist: str = "normal", seed: int = 0, shuffle: bool = True) -> Inputs:
    """Sequences of the given lengths packed back to back into one key buffer.
    ``chunks`` lists (sequence, first local position, count) runs of query
    positions; query order is shuffled (seeded) unless ``shuffle`` is False.
    Values follow ``make_custom``'s recipes; draw order q, k, w, then the
    shuffle."""
    seq_lens = [int(x) for x in seq_lens]
    starts = np.concatenate([[0], np.cumsum(seq_lens)[:-1]]).astype(np.int64)
    pos, first = [], []
    for sq, lp, cnt in chunks:
        if not (0 <= lp and lp + cnt <= seq_lens[sq]):
            raise ValueError("query run outside its sequence")
        pos.extend(starts[sq] + lp + np.arange(cnt))
        first.extend([starts[sq]] * cnt)
    L, n = int(sum(seq_lens)), len(pos)
    cfg = dict(L=L, n=n, H=H, d=d, k=k, dtype=dtype, dist=dist, seed=seed)
    rng = np.random.default_rng(seed)
    q32, k32, w = _draw(cfg, rng)
    order = rng.permutation(n) if shuffle else np.arange(n)
    q_pos = np.asarray(pos, dtype=np.int32)[order]
    q_first = np.asarray(first, dtype=np.int32)[order]
    if dtype == "bf16":
        inp = Inputs(name, L, n, H, d, k, dtype, f32_to_bf16_bits(q32), f32_to_bf16_bits(k32), w)
    elif dtype == "fp8":
        qc, qs = quantize_e4m3_per_row(q32)
        kc, ks = quantize_e4m3_per_row(k32)
        inp = Inputs(name, L, n, H, d, k, dtype, qc, kc, w, qs, ks)
    elif dtype in ("mxfp8", "mxfp4"):
        qc, qs = quantize_mx(q32, dtype)
        kc, ks = quantize_mx(k32, dtype)
        inp = Inputs(name, L, n, H, d, k, dtype, qc, kc, w, qs, ks)
    else:
        raise ValueError(dtype)
    inp.q_pos, inp.q_first = q_pos, q_first
    return inp


def subset_queries(n: int, count: int = 64, seed: int = 7, must: tuple[int, ...] = ()) -> np.ndarray:
    """A seeded sorted subset of query indices that always holds the first and
    last query and every index in ``must``."""
    base = {0, n - 1, *[int(m) for m in must if 0 <= m < n]}
    rng = np.random.default_rng(seed)
    pool = np.setdiff1d(np.arange(n), np.fromiter(base, dtype=np.int64))
    extra = max(0, min(count - len(base), pool.size))
    pick = rng.choice(pool, size=extra, replace=False) if extra else np.empty(0, np.int64)
    return np.sort(np.concatenate([np.fromiter(base, dtype=np.int64), pick.astype(np.int64)]))
