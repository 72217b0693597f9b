"""CPU fp64 oracle for exact top-k indexer selection and selection replay.

TEST INFRASTRUCTURE ONLY.  Nothing on the product path may import, call or link
this module: only ``tests/``, ``__graft_entry__.smoke()`` and the CPU-baseline
leg of ``bench.py`` use it.  It shares no code, tables or helpers with the HIP
path; both sides read the same input bytes from ``datagen``.

Sources, cited by page title and passage:

* [Explainer] "HyScale sparse-attention training -- Selection without a score
  table -- What does it mean?" (learnaivisually.com).  Paragraphs: *contest*
  (the score table and the two-kernel baseline), *key observation* (selection
  outputs indices; top-k is not differentiable), *HyTopK* (sampled threshold,
  candidate buffer, check, recovery, fallback above 64 failures, radix select
  over positions, radix sort), *selection replay*, *worked example* (the
  GLM-5.1 figures at L = 1,048,576).
* [Summary] "HyScale: Scaling Long-Context Training for Learned Sparse
  Attention" (neuraltrendhub.com), section *What the paper found*.
* [Abstract] the paper's abstract (reproduced on zhuanzhiai.com and in the
  Summary's *Original abstract* section).

What this oracle computes is the plain definition, because the method reaches
exactly that result ([Abstract]: HyTopK returns the exact top-k of every
query without materialising a table of scores):

1. decode the stored inputs exactly to fp64 (bf16 bits; OCP E4M3 codes times
   their per-token fp32 scales; OCP MX block-scaled E4M3 / E2M1 elements times
   their E8M0 scale per 32 elements; fp32 head weights);
2. score every causal pair (query position t sees keys 0..t; with packed
   sequences, the keys from its own sequence's first key through t) with the
   learned-sparse-attention indexer I(t,s) = sum_h w[t,h] * ReLU(q[t,h] . k[s]).
   The pages do not print the indexer's formula; they liken the cost of its
   scores to that of attention scores [Explainer, contest] and say that the
   architecture descends from DeepSeek-V3.2 [Abstract].  This is the standard
   form of that indexer: the head weight applies after the ReLU;
3. order the context by score descending, then position ascending (lower
   position wins a tie) and keep the first min(k, ctx); pad with -1 / -inf;
4. replay: I(t, idx) at the saved indices [Explainer, selection replay];
5. backward at the replayed entries: given an upstream gradient dI[t, j] for
   the score at idx[t, j], the gradients of sum_{t,j} dI[t,j] * I(t, idx[t,j])
   with respect to q, w and k.  The choice itself carries no gradient (top-k
   is not differentiable) and the indexer's loss depends on the selected
   entries' scores alone, so nothing else enters [Explainer, key observation].

The threshold model (``sample_count`` .. ``predict_paths``) is not part of the
result.  It restates the HyTopK paragraph and the worked example so tests can
pin the GPU's statistics, failure sets and path choice.
"""
from __future__ import annotations

import math

import numpy as np

NEG_INF = float("-inf")

# ---------------------------------------------------------------------------
# 1. Exact decoding of the storage formats.
# ---------------------------------------------------------------------------


def decode_bf16(bits: np.ndarray) -> np.ndarray:
    """bf16 bit patterns -> fp64, from the format: 1 sign bit, 8 exponent bits
    (bias 127), 7 fraction bits; exponent 0 is subnormal (f/128 * 2^-126),
    exponent 255 is inf/NaN."""
    b = np.asarray(bits, dtype=np.uint16).astype(np.int64)
    sign = np.where((b >> 15) & 1, -1.0, 1.0)
    e = (b >> 7) & 0xFF
    f = (b & 0x7F).astype(np.float64)
    normal = sign * (1.0 + f / 128.0) * np.exp2(e.astype(np.float64) - 127.0)
    sub = sign * (f / 128.0) * 2.0 ** -126
    out = np.where(e == 0, sub, normal)
    special = e == 0xFF
    if np.any(special):
        out = np.where(special & (f == 0), sign * np.inf, out)
        out = np.where(special & (f != 0), np.nan, out)
    return out


def decode_e4m3(codes: np.ndarray) -> np.ndarray:
    """OCP FP8 E4M3 codes -> fp64, from the format: 1 sign bit, 4 exponent bits
    (bias 7), 3 mantissa bits; exponent 0 is subnormal (m/8 * 2^-6); the codes
    with all exponent and mantissa bits set (0x7F, 0xFF) are NaN; there is no
    infinity, so the largest finite value is 1.75 * 2^8 = 448."""
    c = np.asarray(codes, dtype=np.uint8).astype(np.int64)
    sign = np.where((c >> 7) & 1, -1.0, 1.0)
    e = (c >> 3) & 0xF
    m = (c & 0x7).astype(np.float64)
    normal = sign * (1.0 + m / 8.0) * np.exp2(e.astype(np.float64) - 7.0)
    sub = sign * (m / 8.0) * 2.0 ** -6
    out = np.where(e == 0, sub, normal)
    return np.where((c & 0x7F) == 0x7F, np.nan, out)


def decode_e2m1(codes: np.ndarray) -> np.ndarray:
    """OCP FP4 E2M1 codes (0..15) -> fp64, from the format: 1 sign bit, 2
    exponent bits (bias 1), 1 mantissa bit; exponent 0 is subnormal (m/2);
    no infinity or NaN, largest value 1.5 * 2^2 = 6."""
    c = np.asarray(codes, dtype=np.uint8).astype(np.int64) & 0xF
    sign = np.where((c >> 3) & 1, -1.0, 1.0)
    e = (c >> 1) & 0x3
    m = (c & 0x1).astype(np.float64)
    normal = sign * (1.0 + m / 2.0) * np.exp2(e.astype(np.float64) - 1.0)
    return np.where(e == 0, sign * m / 2.0, normal)


def decode_e8m0(b: np.ndarray) -> np.ndarray:
    """OCP E8M0 scale bytes -> fp64: 2^(b - 127); 0xFF is NaN."""
    x = np.asarray(b, dtype=np.uint8).astype(np.float64)
    return np.where(x == 255, np.nan, np.exp2(x - 127.0))


def decode_mx(codes: np.ndarray, scales: np.ndarray, fmt: str) -> np.ndarray:
    """MX block-scaled values -> fp64: every 32 consecutive elements of the
    last axis share one E8M0 scale.  ``mxfp8``: E4M3 bytes; ``mxfp4``: E2M1
    codes two per byte, element 2i in the low nibble of byte i."""
    c = np.asarray(codes, dtype=np.uint8)
    if fmt == "mxfp8":
        v = _e4m3_lookup(c)
    elif fmt == "mxfp4":
        v = np.empty(c.shape[:-1] + (2 * c.shape[-1],), dtype=np.float64)
        v[..., 0::2] = decode_e2m1(c & 0xF)
        v[..., 1::2] = decode_e2m1(c >> 4)
    else:
        raise ValueError(fmt)
    sc = np.repeat(decode_e8m0(scales), 32, axis=-1)
    return v * sc


_BF16_TABLE = None
_E4M3_TABLE = None


def _bf16_lookup(bits: np.ndarray) -> np.ndarray:
    """decode_bf16 applied through a table of all 65,536 patterns (fast path
    for large arrays; the table is decode_bf16 itself)."""
    global _BF16_TABLE
    if _BF16_TABLE is None:
        _BF16_TABLE = decode_bf16(np.arange(1 << 16, dtype=np.uint16))
    return _BF16_TABLE[np.asarray(bits, dtype=np.uint16)]


def _e4m3_lookup(codes: np.ndarray) -> np.ndarray:
    """decode_e4m3 applied through a table of all 256 codes."""
    global _E4M3_TABLE
    if _E4M3_TABLE is None:
        _E4M3_TABLE = decode_e4m3(np.arange(256, dtype=np.uint8))
    return _E4M3_TABLE[np.asarray(codes, dtype=np.uint8)]


class Decoded:
    """Exact fp64 view of one problem.  Queries are decoded on demand (the
    1M-key shapes hold 8,192 x 64 x 128 query values)."""

    def __init__(self, inp):
        self.inp = inp
        self.L, self.n, self.H, self.d, self.k = inp.L, inp.n, inp.H, inp.d, inp.k
        self.q_start = inp.L - inp.n
        if inp.dtype == "bf16":
            self.keys = _bf16_lookup(inp.k_)
        elif inp.dtype == "fp8":
            self.keys = _e4m3_lookup(inp.k_)
            self.keys *= inp.k_scale.astype(np.float64)[:, None]
        elif inp.dtype in ("mxfp8", "mxfp4"):
            self.keys = decode_mx(inp.k_, inp.k_scale, inp.dtype)
        else:
            raise ValueError(inp.dtype)

    def query(self, i: int) -> tuple[np.ndarray, np.ndarray]:
        """(q[i] as [H][d] fp64, w[i] as [H] fp64)."""
        inp = self.inp
        if inp.dtype == "bf16":
            q = _bf16_lookup(inp.q[i])
        elif inp.dtype == "fp8":
            q = _e4m3_lookup(inp.q[i]) * float(inp.q_scale[i])
        else:
            q = decode_mx(inp.q[i], inp.q_scale[i], inp.dtype)
        return q, inp.w[i].astype(np.float64)

    def position(self, i: int) -> int:
        """Position t of query i: the explicit ``q_pos`` when given, else the
        default q_start + i."""
        if self.inp.q_pos is not None:
            return int(self.inp.q_pos[i])
        return self.q_start + int(i)

    def first(self, i: int) -> int:
        """First key of query i's context (packed sequences), default 0."""
        if self.inp.q_first is not None:
            return int(self.inp.q_first[i])
        return 0


# ---------------------------------------------------------------------------
# 2. Indexer scores.
# ---------------------------------------------------------------------------


def score_row(dec: Decoded, i: int, chunk: int = 32768) -> np.ndarray:
    """I(t, s) for query i (position t) and every key s of its context,
    first..t (first = 0 unless the query's sequence starts later), in fp64.
    Entry j of the row is key first + j."""
    q, w = dec.query(i)
    lo = dec.first(i)
    ctx = max(0, dec.position(i) + 1 - lo)
    out = np.empty(ctx, dtype=np.float64)
    for a in range(0, ctx, chunk):
        b = min(ctx, a + chunk)
        dots = q @ dec.keys[lo + a:lo + b].T  # [H][b-a]  q[t,h] . k[s]
        np.maximum(dots, 0.0, out=dots)       # ReLU
        out[a:b] = w @ dots                   # sum_h w[t,h] * ...
    return out


def score_pairs(dec: Decoded, i: int, keys: np.ndarray) -> np.ndarray:
    """I(t, s) for query i at the given key positions (any order)."""
    q, w = dec.query(i)
    return indexer_pairs(q, w, dec.keys[np.asarray(keys, dtype=np.int64)])


# ---------------------------------------------------------------------------
# 3. Exact top-k under the tie rule, and replay.
# ---------------------------------------------------------------------------


def exact_topk(row: np.ndarray, k: int) -> tuple[np.ndarray, np.ndarray]:
    """Keep the min(k, ctx) best keys of one score row: score descending, then
    position ascending.  Returns (idx int64 [k], score fp64 [k]) padded with
    -1 / -inf."""
    ctx = row.shape[0]
    order = np.lexsort((np.arange(ctx), -row))   # last key is the primary key
    keep = order[: min(k, ctx)]
    idx = np.full(k, -1, dtype=np.int64)
    val = np.full(k, NEG_INF, dtype=np.float64)
    idx[: keep.size] = keep
    val[: keep.size] = row[keep]
    return idx, val


def select(inp, queries=None) -> tuple[np.ndarray, np.ndarray]:
    """Exact top-k for the given query indices (default: all n).
    Returns (idx [m][k] int64, score [m][k] fp64)."""
    dec = Decoded(inp)
    qs = np.arange(inp.n) if queries is None else np.asarray(queries, dtype=np.int64)
    idx = np.empty((qs.size, inp.k), dtype=np.int64)
    val = np.empty((qs.size, inp.k), dtype=np.float64)
    for r, i in enumerate(qs):
        idx[r], val[r] = exact_topk(score_row(dec, int(i)), inp.k)
        idx[r][idx[r] >= 0] += dec.first(int(i))   # row entry j is key first + j
    return idx, val


def replay(inp, idx: np.ndarray, queries=None) -> np.ndarray:
    """Selection replay: rescore only the saved indices.  idx < 0 is padding
    and scores -inf.  Returns fp64 [m][k]."""
    dec = Decoded(inp)
    qs = np.arange(inp.n) if queries is None else np.asarray(queries, dtype=np.int64)
    idx = np.asarray(idx)
    out = np.full(idx.shape, NEG_INF, dtype=np.float64)
    for r, i in enumerate(qs):
        ok = idx[r] >= 0
        if np.any(ok):
            out[r, ok] = score_pairs(dec, int(i), idx[r, ok])
    return out


# ---------------------------------------------------------------------------
# 3b. Backward at the replayed entries (plain chain rule, fp64).
# ---------------------------------------------------------------------------


def indexer_pairs(q: np.ndarray, w: np.ndarray, keys: np.ndarray) -> np.ndarray:
    """I = sum_h w[h] * ReLU(q[h] . key) for one query (q [H][d], w [H]) and
    the rows of ``keys`` ([m][d]); fp64 arrays in, fp64 [m] out."""
    return w @ np.maximum(q @ keys.T, 0.0)


def backward_query(q: np.ndarray, w: np.ndarray, keys: np.ndarray, g: np.ndarray,
                   amb: float = 0.0) -> dict:
    """Gradients of sum_j g[j] * I(q, w, keys[j]) for one query.

    With c[h, j] = q[h] . keys[j] and the ReLU derivative taken as 1 where
    c > 0 and 0 elsewhere (including c == 0):
      dw[h]     = sum_j g[j] * max(c[h, j], 0)
      dq[h, :]  = w[h] * sum_j g[j] * [c[h, j] > 0] * keys[j, :]
      u[j, :]   = sum_h g[j] * w[h] * [c[h, j] > 0] * q[h, :]   (row j's share of dk)
    Also returns the same sums over absolute values of every term (the scale
    against which a rounding-error bound is stated) and, for ``amb`` > 0, the
    absolute contribution of the terms whose ReLU decision is within
    amb * sum_i |q[h, i] * keys[j, i]| of zero, where a lower-precision
    evaluation of c may take the other branch.
    """
    c = q @ keys.T                                  # [H][m]
    on = c > 0.0
    dw = np.where(on, c, 0.0) @ g
    G = np.where(on, g[None, :], 0.0)               # dI[j] * ReLU'(c)
    dq = w[:, None] * (G @ keys)
    u = (G * w[:, None]).T @ q
    ag, aw, aq, ak = np.abs(g), np.abs(w), np.abs(q), np.abs(keys)
    Ga = np.where(on, ag[None, :], 0.0)
    out = dict(dw=dw, dq=dq, u=u,
               dw_abs=np.where(on, c, 0.0) @ ag,
               dq_abs=aw[:, None] * (Ga @ ak),
               u_abs=(Ga * aw[:, None]).T @ aq)
    if amb > 0.0:
        near = np.abs(c) <= amb * (aq @ ak.T)
        Gn = np.where(near, ag[None, :], 0.0)
        out["dq_amb"] = aw[:, None] * (Gn @ ak)
        out["u_amb"] = (Gn * aw[:, None]).T @ aq
    return out


def backward_core(query_fn, keys: np.ndarray, idx: np.ndarray, d_score: np.ndarray,
                  amb: float = 0.0) -> dict:
    """Backward over m queries: ``query_fn(r)`` gives query r's (q [H][d],
    w [H]) in fp64, ``keys`` is [L][d] fp64, idx [m][k] key positions
    (outside [0, L) = padding, no contribution), d_score [m][k] the upstream
    gradient.  dk is the scatter-add of every entry's u row onto its key."""
    idx = np.asarray(idx)
    g_all = np.asarray(d_score, dtype=np.float64)
    L, d = keys.shape
    m = idx.shape[0]
    res = None
    for r in range(m):
        q, w = query_fn(r)
        if res is None:
            H = q.shape[0]
            res = {k: np.zeros((m, H, d)) for k in ("dq", "dq_abs")}
            res.update({k: np.zeros((m, H)) for k in ("dw", "dw_abs")})
            res.update({k: np.zeros((L, d)) for k in ("dk", "dk_abs")})
            if amb > 0.0:
                res["dq_amb"] = np.zeros((m, H, d))
                res["dk_amb"] = np.zeros((L, d))
        ok = (idx[r] >= 0) & (idx[r] < L)
        if not np.any(ok):
            continue
        sel = idx[r, ok].astype(np.int64)
        b = backward_query(q, w, keys[sel], g_all[r, ok], amb)
        res["dq"][r], res["dq_abs"][r] = b["dq"], b["dq_abs"]
        res["dw"][r], res["dw_abs"][r] = b["dw"], b["dw_abs"]
        np.add.at(res["dk"], sel, b["u"])           # scatter-add by key position
        np.add.at(res["dk_abs"], sel, b["u_abs"])
        if amb > 0.0:
            res["dq_amb"][r] = b["dq_amb"]
            np.add.at(res["dk_amb"], sel, b["u_amb"])
    return res


def backward(inp, idx: np.ndarray, d_score: np.ndarray, queries=None, amb: float = 0.0) -> dict:
    """Indexer backward at the replayed entries for the given query indices
    (default: all n).  idx [m][k] holds key positions (negative = padding, no
    contribution); d_score [m][k] the upstream gradient of each replayed
    score.  FP8 inputs are differentiated with respect to their decoded
    values (code times per-token scale).

    Returns fp64 dq [m][H][d], dw [m][H], dk [L][d] (the queries' summed
    contributions; keys no query selected get 0), their absolute-term scales
    (*_abs) and, for amb > 0, the ambiguous-decision allowances (*_amb)."""
    dec = Decoded(inp)
    qs = np.arange(inp.n) if queries is None else np.asarray(queries, dtype=np.int64)
    return backward_core(lambda r: dec.query(int(qs[r])), dec.keys, idx, d_score, amb)


# ---------------------------------------------------------------------------
# 4. The sampled-threshold model (statistics and path prediction only).
# ---------------------------------------------------------------------------

DEFAULTS = dict(m_min=4096, m_max=8192, m_div=128, oversample=3, max_recover=64)


def sample_count(L: int, m_min: int = 4096, m_max: int = 8192, m_div: int = 128) -> int:
    """M = min(max(4096, L/128), 8192) [Explainer, worked example], with L the
    number of keys in the call and integer division."""
    return min(max(m_min, L // m_div), m_max)


def sample_positions(ctx: int, M: int) -> np.ndarray:
    """Evenly spaced samples of that query's context [Explainer, HyTopK]:
    M_q = min(M, ctx) positions floor(j * ctx / M_q), j = 0..M_q-1."""
    mq = min(M, ctx)
    j = np.arange(mq, dtype=np.int64)
    return (j * ctx) // mq


def threshold_rank(ctx: int, k: int, mq: int, oversample: int = 3) -> int:
    """The threshold is the ceil(3k * M / ctx)-th best sample [Explainer, worked
    example: 48 at ctx = 1,048,576, k = 2,048, M = 8,192], clamped to [1, M_q]."""
    r = -(-(oversample * k * mq) // ctx)
    return max(1, min(mq, r))


def threshold(row: np.ndarray, k: int, L: int, params: dict | None = None) -> tuple[float, int, int]:
    """tau = the r-th largest sample score (duplicates count separately).
    Returns (tau, r, M_q)."""
    p = dict(DEFAULTS, **(params or {}))
    ctx = row.shape[0]
    M = sample_count(L, p["m_min"], p["m_max"], p["m_div"])
    pos = sample_positions(ctx, M)
    r = threshold_rank(ctx, k, pos.size, p["oversample"])
    s = np.sort(row[pos])[::-1]
    return float(s[r - 1]), r, pos.size


def candidates(row: np.ndarray, tau: float) -> np.ndarray:
    """Keys that pass the on-chip compare (score >= tau), in position order."""
    return np.nonzero(row >= tau)[0]


def predict_row(row: np.ndarray, k: int, L: int, cap: int, params: dict | None = None) -> dict:
    """Threshold, candidate count and check verdict for one query, with the
    margins that make a prediction robust to fp32-vs-fp64 rounding."""
    tau, r, mq = threshold(row, k, L, params)
    ctx = row.shape[0]
    cnt = int(np.count_nonzero(row >= tau))
    need = min(k, ctx)
    near = int(np.count_nonzero(np.abs(row - tau) <= 1e-6 * (abs(tau) + 1.0)))
    return dict(tau=tau, r=r, mq=mq, cnt=cnt, overflow=cnt > cap, underk=cnt < need,
                fail=(cnt > cap) or (cnt < need), margin_cap=cap - cnt,
                margin_k=cnt - need, near_tau=near)


def predict_paths(rows: list, k: int, L: int, cap: int, params: dict | None = None) -> dict:
    """Per-query predictions for one selection call plus the call's path:
    recovery if 1..64 queries fail, full rescore above 64 [Explainer, HyTopK]."""
    p = dict(DEFAULTS, **(params or {}))
    per = [predict_row(r, k, L, cap, p) for r in rows]
    failed = [i for i, x in enumerate(per) if x["fail"]]
    return dict(per_query=per, failed=failed, n_failed=len(failed),
                full_rescore=len(failed) > p["max_recover"])


def select_from_candidates(row: np.ndarray, tau: float, cap: int, k: int):
    """The method's own route for one query, modelled on the CPU: keep only keys
    with score >= tau; if that set overflowed ``cap`` or holds fewer than
    min(k, ctx) keys the query is flagged (returns None); otherwise the exact
    top-k of the candidates.  Used only to pin the soundness claim."""
    cand = candidates(row, tau)
    if cand.size > cap or cand.size < min(k, row.shape[0]):
        return None
    sub = row[cand]
    order = np.lexsort((cand, -sub))[: min(k, cand.size)]
    idx = np.full(k, -1, dtype=np.int64)
    val = np.full(k, NEG_INF)
    idx[: order.size] = cand[order]
    val[: order.size] = sub[order]
    return idx, val


def expected_candidates(ctx: int, mq: int, r: int) -> float:
    """Mean candidate count for i.i.d. continuous scores: the r passing samples
    plus each of the ctx - M_q other keys exceeding the r-th largest of M_q
    i.i.d. samples with probability r / (M_q + 1)."""
    return r + (ctx - mq) * r / (mq + 1)


def scoring_flops(L: int, n: int, H: int, d: int) -> float:
    """2*H*d per causal pair, summed over queries at the last n positions."""
    pairs = n * L - n * (n - 1) // 2
    return 2.0 * H * d * pairs


def log2_ceil(x: int) -> int:
    return int(math.ceil(math.log2(x))) if x > 1 else 0
