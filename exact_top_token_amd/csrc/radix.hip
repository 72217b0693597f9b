// Check, exact selection and ordering ("HyScale sparse-attention training --
// Selection without a score table", HyTopK paragraph).
//
// * check: a query fails when its candidates overflowed the buffer (count >
//   cap) or number fewer than min(k, ctx).
// * cand_select: for every query that passed, the exact top-k of its
//   candidates.  Candidates arrive in whatever order the scoring kernel left
//   them, so every step below depends only on the candidate multiset, which
//   makes the output bitwise reproducible:
//     1. radix select of the k-th largest order-preserving score key;
//     2. at that score, radix select over positions keeps the lowest-position
//        ties (the pages break ties at the k-th score by position, with a
//        radix select);
//     3. LSD radix sort of the kept k by (score descending, position
//        ascending) (the pages sort the k survivors by radix).
// * row_topk: the same result from materialised score rows (the conventional
//   two-kernel route, recovery and full rescore): radix select over the row,
//   emission of the kept entries in position order (ties: first ones win),
//   then a stable radix sort by score descending.
#include "common.h"
#include "launch.h"

namespace hk {

constexpr int kSelThreads = 512;
constexpr int kSelWaves = kSelThreads / kWave;
constexpr int kMaxRounds = 4;  // k <= 2048 = kMaxRounds * kSelThreads

// ----------------------------------------------------------------- helpers

struct SortScratch {
  int cnt[kSelWaves][256];  // per (wave, digit) running counts, then offsets
  int wsum[kSelWaves];
  int skip;
};

// Stable LSD radix sort, ascending by key bits [lo, hi), of the N <= 2048
// (key, val) pairs in (k0, v0); (k1, v1) is scratch of the same size.
// Digits are up to 8 bits wide (the passes split [lo, hi) evenly).  Wave w
// ranks entries 256 w .. 256 w + 255 in four rounds of 64: the lanes holding
// the same digit are found with one ballot per digit bit, and a running
// count per (wave, digit) in LDS (each wave its own row, so lanes with
// different digits hit different banks) carries the rank across rounds, so
// entries with equal digits keep their order.  Offsets follow (digit, wave)
// order.  Returns true when the result ended in (k1, v1).
__device__ __forceinline__ bool block_sort_pairs(uint32_t* k0, uint32_t* v0, uint32_t* k1, uint32_t* v1, int N,
                                 int lo, int hi, SortScratch& ss) {
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const uint64_t lt = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
  bool flipped = false;
  const int passes = (hi - lo + 7) / 8;
  int sh = lo;
  for (int p = 0; p < passes; ++p) {
    const int w = (hi - sh + (passes - p) - 1) / (passes - p);  // digit bits of this pass
    const int nd = 1 << w;
    const uint32_t dmask = (uint32_t)nd - 1u;
    for (int b = lane; b < nd; b += kWave) ss.cnt[wave][b] = 0;  // this wave's row
    if (tid == 0) ss.skip = 0;
    uint32_t myd[kMaxRounds];
    int myrank[kMaxRounds];
#pragma unroll
    for (int j = 0; j < kMaxRounds; ++j) {
      const int i = wave * (kMaxRounds * kWave) + j * kWave + lane;
      const bool ok = i < N;
      const uint32_t d = ok ? (k0[i] >> sh) & dmask : 0u;
      uint64_t m = __ballot(ok);
      for (int b = 0; b < w; ++b) {
        const bool bit = (d >> b) & 1u;
        const uint64_t bb = __ballot(bit);
        m &= bit ? bb : ~bb;
      }
      int rank = 0;
      if (ok) {
        const int before = ss.cnt[wave][d];
        rank = before + __popcll(m & lt);
        // the lowest lane of each digit group advances the running count
        if ((m & lt) == 0ull) ss.cnt[wave][d] = before + __popcll(m);
      }
      myd[j] = d;
      myrank[j] = rank;
    }
    __syncthreads();
    // digit totals, their exclusive scan (digits in threads 0..255), then the
    // offset of each (digit, wave) in (digit, wave) order
    int tot = 0, pre = 0;
    if (tid < 256) {
      if (tid < nd) {
#pragma unroll
        for (int v = 0; v < kSelWaves; ++v) tot += ss.cnt[v][tid];
      }
      pre = wave_prefix_excl(tot);
      if (lane == kWave - 1) ss.wsum[wave] = pre + tot;
      if (tot == N) ss.skip = 1;  // one digit for all entries: order unchanged
    }
    __syncthreads();
    const bool skip = ss.skip != 0;
    if (!skip && tid < nd) {
      int base = pre;
      for (int v = 0; v < wave; ++v) base += ss.wsum[v];
#pragma unroll
      for (int v = 0; v < kSelWaves; ++v) {
        const int c = ss.cnt[v][tid];
        ss.cnt[v][tid] = base;
        base += c;
      }
    }
    __syncthreads();  // offsets ready; every thread has read the skip flag
    sh += w;
    if (skip) continue;  // uniform
#pragma unroll
    for (int j = 0; j < kMaxRounds; ++j) {
      const int i = wave * (kMaxRounds * kWave) + j * kWave + lane;
      if (i < N) {
        const int dst = ss.cnt[wave][myd[j]] + myrank[j];
        k1[dst] = k0[i];
        v1[dst] = v0[i];
      }
    }
    __syncthreads();
    uint32_t* t;
    t = k0; k0 = k1; k1 = t;
    t = v0; v0 = v1; v1 = t;
    flipped = !flipped;
  }
  return flipped;
}

__device__ __forceinline__ int bits_for(int L) {
  int b = 0;
  while ((1 << b) < L && b < 31) ++b;
  return (b + 3) & ~3;
}

// ----------------------------------------------------------------- zero / check

__global__ void zero_kernel(int* cnt, int n, DevStats* st) {
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) cnt[i] = 0;
  if (i == 0) {
    st->n_overflow = 0;
    st->n_underk = 0;
    st->n_failed = 0;
    st->cand_max = 0;
    st->cand_total = 0ull;
  }
}

hipError_t launch_zero(int* cnt, int n, DevStats* st, hipStream_t s) {
  const int nb = (n + 255) / 256;
  hipLaunchKernelGGL(zero_kernel, dim3(nb > 0 ? nb : 1), dim3(256), 0, s, cnt, n, st);
  return hipGetLastError();
}

__global__ void check_kernel(const int* cnt, int n, const int* qpos, const int* qfirst, int q_start,
                             int L, int topk, int cap, DevStats* st, int* failed) {
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= n) return;
  const int c = cnt[i];
  const QRange rg = query_range(qpos, qfirst, q_start, L, i);
  const int need = min(topk, max(0, rg.hi - rg.lo + 1));
  const bool over = c > cap, under = c < need;
  atomicAdd(&st->cand_total, (unsigned long long)c);
  atomicMax(&st->cand_max, c);
  if (over) atomicAdd(&st->n_overflow, 1);
  if (under) atomicAdd(&st->n_underk, 1);
  if (over || under) failed[atomicAdd(&st->n_failed, 1)] = i;
}

hipError_t launch_check(const int* cnt, int n, const int* qpos, const int* qfirst, int q_start,
                        int L, int topk, int cap, DevStats* st, int* failed, hipStream_t s) {
  hipLaunchKernelGGL(check_kernel, dim3((n + 255) / 256), dim3(256), 0, s, cnt, n, qpos, qfirst,
                     q_start, L, topk, cap, st, failed);
  return hipGetLastError();
}

__global__ void async_status_kernel(const DevStats* st, int max_recover, int32_t* out) {
  if (threadIdx.x != 0) return;
  out[0] = st->n_failed > max_recover ? 1 : 0;
  out[1] = st->n_failed;
  out[2] = st->n_overflow;
  out[3] = st->n_underk;
  out[4] = st->cand_max;
  out[5] = (int32_t)(uint32_t)(st->cand_total & 0xFFFFFFFFull);
  out[6] = (int32_t)(uint32_t)(st->cand_total >> 32);
  out[7] = 0;
}

hipError_t launch_async_status(const DevStats* st, int max_recover, int32_t* out, hipStream_t s) {
  hipLaunchKernelGGL(async_status_kernel, dim3(1), dim3(64), 0, s, st, max_recover, out);
  return hipGetLastError();
}

// ----------------------------------------------------------------- output

// Sort the `need` selected (key, pos) pairs by (score desc, pos asc) and write
// the output row; entries need..topk-1 are padding.  pos_sorted: the pairs
// are already in ascending position order, so a stable sort by score suffices.
__device__ __forceinline__ void sort_and_emit(uint32_t* sk, uint32_t* sp, uint32_t* tk, uint32_t* tp, int need,
                              int topk, int L, bool pos_sorted, int* out_idx, float* out_score,
                              SortScratch& ss) {
  const int tid = threadIdx.x;
  // Ascending by (~key, pos): LSD, position bits first.
  for (int i = tid; i < need; i += kSelThreads) sk[i] = ~sk[i];
  __syncthreads();
  bool fl = false;
  if (!pos_sorted) {
    // sort by position: use the position as the key temporarily
    fl = block_sort_pairs(sp, sk, tp, tk, need, 0, bits_for(L), ss);
    if (fl) { uint32_t* t = sk; sk = tk; tk = t; t = sp; sp = tp; tp = t; }
  }
  fl = block_sort_pairs(sk, sp, tk, tp, need, 0, 32, ss);
  if (fl) { sk = tk; sp = tp; }
  for (int i = tid; i < topk; i += kSelThreads) {
    if (i < need) {
      out_idx[i] = (int)sp[i];
      if (out_score) out_score[i] = key_score(~sk[i]);
    } else {
      out_idx[i] = -1;
      if (out_score) out_score[i] = -__builtin_inff();
    }
  }
}

// ----------------------------------------------------------------- candidates

constexpr int kTieRun = 8;  // longest run of equal kept scores ordered in registers

// Ascending order of the len (2 .. kTieRun) distinct positions at p, by
// odd-even transposition in registers (the padding sorts last).
__device__ __forceinline__ void sort_short_run(uint32_t* p, int len) {
  uint32_t v[kTieRun];
#pragma unroll
  for (int j = 0; j < kTieRun; ++j) v[j] = j < len ? p[j] : 0xFFFFFFFFu;
#pragma unroll
  for (int r = 0; r < kTieRun; ++r) {
#pragma unroll
    for (int j = r & 1; j + 1 < kTieRun; j += 2) {
      const uint32_t a = v[j], b = v[j + 1];
      v[j] = min(a, b);
      v[j + 1] = max(a, b);
    }
  }
#pragma unroll
  for (int j = 0; j < kTieRun; ++j)
    if (j < len) p[j] = v[j];
}

struct CandShared {
  RadixScratch rs;
  SortScratch ss;
  uint32_t red[2 * kSelWaves];
  int nsel;
  int tie;
};

size_t cand_select_lds_bytes(int cap, int topk) {
  // candidate score keys (reused as the sort's scratch pairs), then the
  // selected pairs (key + position)
  return (size_t)(cap > 2 * topk ? cap : 2 * topk) * 4 + (size_t)topk * 8;
}

// One workgroup per query that passed the check.  Only the candidates' score
// keys are staged in LDS (positions stay in the candidate buffer and are read
// for the kept entries only), so two workgroups fit on a CU.  The scores of a
// query's candidates span a narrow range, so the radix digits start at the
// highest bit in which two candidate keys differ.
__global__ void __launch_bounds__(kSelThreads) cand_select_kernel(const int* cnt, const uint2* cand,
                                                                  const int* qpos,
                                                                  const int* qfirst, int q_start,
                                                                  int topk, int cap, int L,
                                                                  int* out_idx, float* out_score) {
  extern __shared__ uint32_t dyn[];
  __shared__ CandShared sh;
  const int q = blockIdx.x, tid = threadIdx.x, lane = tid & 63;
  const int c = cnt[q];
  const QRange rg = query_range(qpos, qfirst, q_start, L, q);
  const int need = min(topk, max(0, rg.hi - rg.lo + 1));
  if (c > cap || c < need) return;  // failed: recovered on the row path
  int* oi = out_idx + (int64_t)q * topk;
  float* os = out_score ? out_score + (int64_t)q * topk : nullptr;
  if (need == 0) {  // empty context: all padding (uniform)
    for (int i = tid; i < topk; i += kSelThreads) {
      oi[i] = -1;
      if (os) os[i] = -__builtin_inff();
    }
    return;
  }
  uint32_t* ck = dyn;               // [cap] candidate score keys (later: sort scratch)
  uint32_t* sk = dyn + max(cap, 2 * topk);  // [topk] kept keys
  uint32_t* sp = sk + topk;         // [topk] kept positions
  const uint2* src = cand + (int64_t)q * cap;
  uint32_t lo = 0xFFFFFFFFu, hi = 0u;
  constexpr int kU = 4;  // candidate loads in flight per thread
  for (int i0 = tid; i0 < c; i0 += kU * kSelThreads) {
    uint32_t y[kU];
#pragma unroll
    for (int u = 0; u < kU; ++u) {
      const int i = i0 + u * kSelThreads;
      y[u] = i < c ? src[i].y : 0u;
    }
#pragma unroll
    for (int u = 0; u < kU; ++u) {
      const int i = i0 + u * kSelThreads;
      if (i < c) {
        const uint32_t kk = score_key(__uint_as_float(y[u]));
        ck[i] = kk;
        lo = min(lo, kk);
        hi = max(hi, kk);
      }
    }
  }
  if (tid == 0) sh.nsel = 0;
  uint32_t kmin, kmax;
  block_minmax(lo, hi, sh.red, kmin, kmax);  // includes the barrier after the loads
  // k-th largest key, as an offset above kmin
  int rem, mult;
  const uint32_t v = kmin + block_select_largest(
      c, need, [&](int i) { return ck[i] - kmin; }, [](int) { return true; }, sh.rs, rem, mult,
      bit_width(kmax - kmin));
  // rem of the mult entries equal to v belong to the top k: keep the rem
  // lowest positions among them (radix select over positions).
  uint32_t pmax = 0xFFFFFFFFu;
  if (rem < mult) {
    int rr, mm;
    const uint32_t pb = (uint32_t)bit_width((uint32_t)(L - 1));
    const uint32_t top = pb >= 32 ? 0xFFFFFFFFu : ((1u << pb) - 1u);
    pmax = top - block_select_largest(
        c, rem, [&](int i) { return top - src[i].x; }, [&](int i) { return ck[i] == v; }, sh.rs,
        rr, mm, (int)pb);
  }
  // compaction: one slot reservation per wave and sweep
  for (int j0 = 0; j0 < c; j0 += kU * kSelThreads) {
    uint32_t px[kU];  // positions, loaded ahead of the sweeps that use them
#pragma unroll
    for (int u = 0; u < kU; ++u) {
      const int i = j0 + u * kSelThreads + tid;
      px[u] = i < c ? src[i].x : 0u;
    }
#pragma unroll
    for (int u = 0; u < kU; ++u) {
      const int i = j0 + u * kSelThreads + tid;
      bool keep = false;
      uint32_t kk = 0u;
      if (i < c) {
        kk = ck[i];
        keep = kk > v || (kk == v && (pmax == 0xFFFFFFFFu || px[u] <= pmax));
      }
      const uint64_t m = __ballot(keep);
      int base = 0;
      if (lane == 0 && m) base = atomicAdd(&sh.nsel, __popcll(m));
      base = __shfl(base, 0);
      if (keep) {
        const int slot = base + __popcll(m & ((lane == 0) ? 0ull : (~0ull >> (64 - lane))));
        if (slot < need) {  // exactly `need` entries qualify; the guard keeps LDS writes in bounds
          sk[slot] = kk;
          sp[slot] = px[u];
        }
      }
    }
  }
  __syncthreads();
  // Order by (score desc, position asc).  Sort on the offset of the key below
  // the largest kept key (only its significant bits); equal scores then sit
  // in runs, each ordered by position on its own when it is short; only a
  // run longer than kTieRun sends the whole row through a position pass and
  // a stable key pass.
  const uint32_t krange = kmax - v;
  uint32_t* tk = ck;
  uint32_t* tp = ck + topk;
  for (int i = tid; i < need; i += kSelThreads) sk[i] = kmax - sk[i];
  __syncthreads();
  const int kbits = (bit_width(krange) + 3) & ~3;
  const int pbits = (bit_width((uint32_t)(L - 1)) + 3) & ~3;
  // One sort call site (stage 0: by key; after a long run of ties, stage 1:
  // by position, stage 2: stable by key again), so the sort is inlined once.
  uint32_t *rk = sk, *rp = sp, *xk = tk, *xp = tp;
  for (int stage = 0;; ++stage) {
    const bool byp = stage == 1;
    const bool fl = block_sort_pairs(byp ? rp : rk, byp ? rk : rp, byp ? xp : xk, byp ? xk : xp,
                                     need, 0, byp ? pbits : kbits, sh.ss);
    if (fl) {
      uint32_t* t = rk; rk = xk; xk = t;
      t = rp; rp = xp; xp = t;
    }
    if (stage == 2) break;
    if (stage == 0) {
      // The thread at the start of each run of equal keys orders the run's
      // positions (runs are disjoint; keys are not written here).
      if (tid == 0) sh.tie = 0;
      __syncthreads();
      for (int i = tid; i + 1 < need; i += kSelThreads) {
        if (rk[i] != rk[i + 1] || (i > 0 && rk[i - 1] == rk[i])) continue;  // not a run start
        int len = 2;
        while (len <= kTieRun && i + len < need && rk[i + len] == rk[i]) ++len;
        if (len > kTieRun)
          sh.tie = 1;
        else
          sort_short_run(rp + i, len);
      }
      __syncthreads();
      if (!sh.tie) break;  // uniform
    }
  }
  for (int i = tid; i < topk; i += kSelThreads) {
    if (i < need) {
      oi[i] = (int)rp[i];
      if (os) os[i] = key_score(kmax - rk[i]);
    } else {
      oi[i] = -1;
      if (os) os[i] = -__builtin_inff();
    }
  }
}

hipError_t launch_cand_select(const int* cnt, const uint2* cand, int n, const int* qpos,
                              const int* qfirst, int q_start, int topk, int cap, int L,
                              int* out_idx, float* out_score, hipStream_t s) {
  const size_t lds = cand_select_lds_bytes(cap, topk);
  static LdsLimit lim;
  hipError_t e = raise_dynamic_lds((const void*)cand_select_kernel, (int)lds, lim);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(cand_select_kernel, dim3((unsigned)n), dim3(kSelThreads), lds, s, cnt, cand,
                     qpos, qfirst, q_start, topk, cap, L, out_idx, out_score);
  return hipGetLastError();
}

// ----------------------------------------------------------------- score rows

struct RowShared {
  RadixScratch rs;
  SortScratch ss;
  int gt[kSelWaves];
  int eq[kSelWaves];
  uint32_t sk[2][4096];
  uint32_t sp[2][4096];
};

__global__ void __launch_bounds__(kSelThreads) row_topk_kernel(const float* rows, int64_t row_stride,
                                                               const int* qlist, int q_offset,
                                                               int nq, const int* qpos,
                                                               const int* qfirst, int q_start,
                                                               int topk, int L, int* out_idx,
                                                               float* out_score, RowGate gate) {
  __shared__ RowShared sh;
  const int e = blockIdx.x, tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  if (e >= gate.live(nq)) return;  // uniform: not a live entry of this pass
  const int q = qlist ? qlist[e] : q_offset + e;
  const QRange rg = query_range(qpos, qfirst, q_start, L, q);
  const int ctx = max(0, rg.hi - rg.lo + 1);
  const int need = min(topk, ctx);
  if (need == 0) {  // empty context: all padding (uniform)
    for (int i = tid; i < topk; i += kSelThreads) {
      out_idx[(int64_t)q * topk + i] = -1;
      if (out_score) out_score[(int64_t)q * topk + i] = -__builtin_inff();
    }
    return;
  }
  // the row holds the scores of keys lo..hi at their key positions
  const float* row = rows + (int64_t)e * row_stride + rg.lo;
  int rem, mult;
  const uint32_t v = block_select_largest(
      ctx, need, [&](int i) { return score_key(row[i]); }, [](int) { return true; }, sh.rs, rem,
      mult);
  // Emit in position order: every key > v, and the first `rem` keys == v.
  const int seg = ((ctx + kSelWaves - 1) / kSelWaves + kWave - 1) / kWave * kWave;
  const int s0 = min(ctx, wave * seg), s1 = min(ctx, s0 + seg);
  int ngt = 0, neq = 0;
  for (int i = s0 + lane; i < s1; i += kWave) {
    const uint32_t kk = score_key(row[i]);
    ngt += kk > v;
    neq += kk == v;
  }
  for (int off = 32; off > 0; off >>= 1) {
    ngt += __shfl_xor(ngt, off);
    neq += __shfl_xor(neq, off);
  }
  if (lane == 0) { sh.gt[wave] = ngt; sh.eq[wave] = neq; }
  __syncthreads();
  int gt_before = 0, eq_before = 0;
  for (int w = 0; w < wave; ++w) { gt_before += sh.gt[w]; eq_before += sh.eq[w]; }
  int out = gt_before + min(eq_before, rem);  // kept entries before this segment
  int ties = eq_before;                         // ties before the current element
  const uint64_t lt = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
  for (int i0 = s0; i0 < s1; i0 += kWave) {
    const int i = i0 + lane;
    const uint32_t kk = i < s1 ? score_key(row[i]) : 0u;
    const bool isgt = i < s1 && kk > v;
    const bool iseq = i < s1 && kk == v;
    const uint64_t meq = __ballot(iseq);
    const int tie_rank = ties + __popcll(meq & lt);
    const bool keep = isgt || (iseq && tie_rank < rem);
    const uint64_t mk = __ballot(keep);
    if (keep) {
      const int slot = out + __popcll(mk & lt);
      if (slot < need) {  // exactly `need` entries qualify; the guard keeps LDS writes in bounds
        sh.sk[0][slot] = kk;
        sh.sp[0][slot] = (uint32_t)(rg.lo + i);
      }
    }
    out += __popcll(mk);
    ties += __popcll(meq);
  }
  __syncthreads();
  sort_and_emit(sh.sk[0], sh.sp[0], sh.sk[1], sh.sp[1], need, topk, L, true,
                out_idx + (int64_t)q * topk, out_score ? out_score + (int64_t)q * topk : nullptr,
                sh.ss);
}

hipError_t launch_row_topk(const float* rows, int64_t row_stride, const int* qlist, int q_offset,
                           int nq, const int* qpos, const int* qfirst, int q_start, int topk, int L,
                           int* out_idx, float* out_score, RowGate gate, hipStream_t s) {
  if (nq <= 0) return hipSuccess;
  hipLaunchKernelGGL(row_topk_kernel, dim3((unsigned)nq), dim3(kSelThreads), 0, s, rows,
                     row_stride, qlist, q_offset, nq, qpos, qfirst, q_start, topk, L, out_idx,
                     out_score, gate);
  return hipGetLastError();
}

// ----------------------------------------------------------------- split rows

// Top-k of a few long rows (recovery of the flagged queries, the full
// rescore in passes of rows): one workgroup per row would leave most of the
// chip idle, so each row is split into `nchunk` chunks of `chunk_len`
// entries.  Three radix passes over the 32-bit order-preserving keys (digits
// of 11, 11 and 10 bits) find the row's k-th largest key v: in each pass
// every chunk's workgroup counts the digits of its entries that match the
// prefix chosen so far into a histogram of its own, and one workgroup per row
// sums the chunk histograms and picks the digit that holds the remaining
// rank.  Emission then keeps every entry above v and, of the entries equal
// to v, the lowest positions (the entries' rank by position among the ties
// comes from the last pass's per-chunk counts of v), which is the tie rule;
// a last workgroup per row sorts the kept entries by (score descending,
// position ascending).  The result is a function of the row contents only.

constexpr int kSplitThreads = 256;
constexpr int kSplitBins = 2048;  // bins of the widest digit
constexpr int kSplitUnroll = 8;   // loads in flight per thread

struct SplitState {
  uint32_t prefix;  // key bits chosen so far (after the last pass: v)
  uint32_t pmask;   // the bits the prefix covers
  int r;            // rank sought among the entries matching the prefix (1-based)
  int mult;         // entries whose key matches the prefix
  int need;         // min(k, ctx)
  int nout;         // entries emitted
  int pad[2];
};

struct SplitLayout {
  size_t state, tiebase, hist, staging, total;
};

static size_t align256(size_t x) { return (x + 255) / 256 * 256; }

static SplitLayout split_layout(int nrows, int nchunk, int topk) {
  SplitLayout l{};
  size_t off = 0;
  l.state = off; off = align256(off + (size_t)nrows * sizeof(SplitState));
  l.tiebase = off; off = align256(off + (size_t)nrows * nchunk * 4);
  l.hist = off; off = align256(off + (size_t)nrows * nchunk * kSplitBins * 4);
  l.staging = off; off = align256(off + (size_t)nrows * topk * 8);
  l.total = off;
  return l;
}

size_t row_select_scratch_bytes(int nrows, int nchunk, int topk) {
  return split_layout(nrows, nchunk, topk).total;
}

int row_select_max_chunks(int64_t L) {
  const int64_t c = (L + 16383) / 16384;
  return (int)(c < 1 ? 1 : (c > 64 ? 64 : c));
}

void row_select_chunks(int nq, int64_t maxctx, int64_t L, int& nchunk, int& chunk_len) {
  const int cmax = row_select_max_chunks(L);
  int64_t target = (1024 + nq - 1) / (nq > 0 ? nq : 1);  // about 1,024 workgroups per pass
  target = target < 1 ? 1 : (target > cmax ? cmax : target);
  if (maxctx < 1) maxctx = 1;
  int64_t len = (maxctx + target - 1) / target;
  len = (len + 1023) / 1024 * 1024;
  nchunk = (int)((maxctx + len - 1) / len);
  chunk_len = (int)len;
}

template <int PASS>
struct SplitPass {
  static constexpr int SHIFT = PASS == 0 ? 21 : (PASS == 1 ? 10 : 0);
  static constexpr int BINS = PASS == 2 ? 1024 : 2048;
  static constexpr uint32_t DMASK = (uint32_t)BINS - 1u;
};

__device__ __forceinline__ int split_query(const RowSelArgs& a, int e) {
  return a.qlist ? a.qlist[e] : a.q_offset + e;
}

// Digit histogram of chunk blockIdx.x of row blockIdx.y over the entries that
// match the prefix of the earlier passes; written whole (zeros included).
template <int PASS>
__global__ void __launch_bounds__(kSplitThreads) split_hist_kernel(RowSelArgs a,
                                                                   const SplitState* st,
                                                                   uint32_t* hist) {
  using P = SplitPass<PASS>;
  __shared__ int lh[P::BINS];
  const int c = blockIdx.x, e = blockIdx.y, tid = threadIdx.x;
  if (e >= a.gate.live(a.nq)) return;  // uniform: not a live row of this pass
  const QRange rg = query_range(a.qpos, a.qfirst, a.q_start, a.L, split_query(a, e));
  const int ctx = max(0, rg.hi - rg.lo + 1);
  for (int b = tid; b < P::BINS; b += kSplitThreads) lh[b] = 0;
  uint32_t prefix = 0u, pmask = 0u;
  if constexpr (PASS > 0) {
    prefix = st[e].prefix;
    pmask = st[e].pmask;
  }
  __syncthreads();
  const int64_t c0 = (int64_t)c * a.chunk_len;
  const int64_t c1 = min<int64_t>(ctx, c0 + a.chunk_len);
  const float* row = a.rows + (int64_t)e * a.row_stride + rg.lo;
  // runs of equal digits per thread are added with one LDS atomic each (in
  // the first pass most entries share a few digits)
  uint32_t run_d = 0u;
  int run_n = 0;
  for (int64_t i0 = c0; i0 < c1; i0 += kSplitUnroll * kSplitThreads) {
    uint32_t kk[kSplitUnroll];
#pragma unroll
    for (int u = 0; u < kSplitUnroll; ++u) {
      const int64_t i = i0 + u * kSplitThreads + tid;
      kk[u] = i < c1 ? score_key(row[i]) : 0u;
    }
#pragma unroll
    for (int u = 0; u < kSplitUnroll; ++u) {
      const int64_t i = i0 + u * kSplitThreads + tid;
      if (i < c1 && (kk[u] & pmask) == prefix) {
        const uint32_t d = (kk[u] >> P::SHIFT) & P::DMASK;
        if (run_n > 0 && d != run_d) {
          atomicAdd(&lh[run_d], run_n);
          run_n = 0;
        }
        run_d = d;
        ++run_n;
      }
    }
  }
  if (run_n > 0) atomicAdd(&lh[run_d], run_n);
  __syncthreads();
  uint32_t* out = hist + ((int64_t)e * a.nchunk + c) * kSplitBins;
  for (int b = tid; b < P::BINS; b += kSplitThreads) out[b] = (uint32_t)lh[b];
}

// One workgroup per row: sums the chunk histograms and picks the digit that
// holds the remaining rank.  After the last pass it also stores, per chunk,
// how many entries equal to v the earlier chunks hold (the tie ranks).
template <int PASS>
__global__ void __launch_bounds__(kSplitThreads) split_pick_kernel(RowSelArgs a, SplitState* st,
                                                                   const uint32_t* hist,
                                                                   uint32_t* tiebase) {
  using P = SplitPass<PASS>;
  constexpr int BPT = P::BINS / kSplitThreads;  // bins per thread
  __shared__ int wsum[kSplitThreads / kWave];
  const int e = blockIdx.x, tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  if (e >= a.gate.live(a.nq)) return;  // uniform: not a live row of this pass
  int r, need;
  uint32_t prefix = 0u, pmask = 0u;
  if constexpr (PASS == 0) {
    const QRange rg = query_range(a.qpos, a.qfirst, a.q_start, a.L, split_query(a, e));
    need = min(a.topk, max(0, rg.hi - rg.lo + 1));
    r = need;
  } else {
    const SplitState s0 = st[e];
    need = s0.need;
    r = s0.r;
    prefix = s0.prefix;
    pmask = s0.pmask;
  }
  if (need == 0) {  // empty context (uniform): nothing to select
    if (PASS == 0 && tid == 0) st[e] = SplitState{0u, 0u, 0, 0, 0, 0, {0, 0}};
    return;
  }
  // thread t holds bins BINS-1 - (BPT t + j), j = 0 .. BPT-1: descending
  int cnt[BPT];
#pragma unroll
  for (int j = 0; j < BPT; ++j) cnt[j] = 0;
  const uint32_t* h = hist + (int64_t)e * a.nchunk * kSplitBins;
  for (int c = 0; c < a.nchunk; ++c) {
#pragma unroll
    for (int j = 0; j < BPT; ++j) cnt[j] += (int)h[(int64_t)c * kSplitBins + P::BINS - 1 - (BPT * tid + j)];
  }
  int tot = 0;
#pragma unroll
  for (int j = 0; j < BPT; ++j) tot += cnt[j];
  int above = wave_prefix_excl(tot);
  if (lane == kWave - 1) wsum[wave] = above + tot;
  __syncthreads();
  for (int w = 0; w < wave; ++w) above += wsum[w];
#pragma unroll
  for (int j = 0; j < BPT; ++j) {
    if (above < r && r <= above + cnt[j]) {  // exactly one thread and bin
      const uint32_t digit = (uint32_t)(P::BINS - 1 - (BPT * tid + j));
      SplitState ns;
      ns.prefix = prefix | (digit << P::SHIFT);
      ns.pmask = pmask | (P::DMASK << P::SHIFT);
      ns.r = r - above;
      ns.mult = cnt[j];
      ns.need = need;
      ns.nout = 0;
      ns.pad[0] = ns.pad[1] = 0;
      st[e] = ns;
      if constexpr (PASS == 2) {
        uint32_t acc = 0u;
        for (int c = 0; c < a.nchunk; ++c) {
          tiebase[(int64_t)e * a.nchunk + c] = acc;
          acc += h[(int64_t)c * kSplitBins + digit];
        }
      }
    }
    above += cnt[j];
  }
}

// Emission: chunk blockIdx.x of row blockIdx.y appends its entries above v
// and its kept ties (rank by position < the remaining rank) to the row's
// staging list, in any order.
__global__ void __launch_bounds__(kSplitThreads) split_emit_kernel(RowSelArgs a, SplitState* st,
                                                                   const uint32_t* hist,
                                                                   const uint32_t* tiebase,
                                                                   uint2* staging) {
  __shared__ int wcnt[kSplitThreads / kWave];
  const int c = blockIdx.x, e = blockIdx.y, tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  if (e >= a.gate.live(a.nq)) return;  // uniform: not a live row of this pass
  const int need = st[e].need;
  if (need == 0) return;  // uniform
  const uint32_t v = st[e].prefix;
  const int rem = st[e].r;
  const QRange rg = query_range(a.qpos, a.qfirst, a.q_start, a.L, split_query(a, e));
  const int ctx = max(0, rg.hi - rg.lo + 1);
  const int64_t c0 = (int64_t)c * a.chunk_len;
  const int64_t c1 = min<int64_t>(ctx, c0 + a.chunk_len);
  if (c0 >= c1) return;  // uniform
  const float* row = a.rows + (int64_t)e * a.row_stride + rg.lo;
  // entries equal to v in this chunk (the last pass's digit of v) and in the
  // chunks before it
  const uint32_t ties = hist[((int64_t)e * a.nchunk + c) * kSplitBins + (v & SplitPass<2>::DMASK)];
  const int tb = (int)tiebase[(int64_t)e * a.nchunk + c];
  const bool ordered = ties > 0u && tb < rem;  // some tie of this chunk may be kept (uniform)
  uint2* dst = staging + (int64_t)e * a.topk;
  int* nout = &st[e].nout;
  const uint64_t lt = lane == 0 ? 0ull : (~0ull >> (64 - lane));
  auto emit = [&](bool keep, uint32_t kk, int64_t i) {
    const uint64_t mk = __ballot(keep);
    if (mk == 0ull) return;  // uniform over the wave
    int base = 0;
    if (lane == 0) base = atomicAdd(nout, __popcll(mk));
    base = __shfl(base, 0);
    if (keep) {
      const int slot = base + __popcll(mk & lt);
      if (slot < a.topk) dst[slot] = make_uint2(kk, (uint32_t)(rg.lo + i));  // exactly need qualify
    }
  };
  if (!ordered) {
    for (int64_t i0 = c0; i0 < c1; i0 += kSplitUnroll * kSplitThreads) {
      uint32_t kk[kSplitUnroll];
#pragma unroll
      for (int u = 0; u < kSplitUnroll; ++u) {
        const int64_t i = i0 + u * kSplitThreads + tid;
        kk[u] = i < c1 ? score_key(row[i]) : 0u;
      }
#pragma unroll
      for (int u = 0; u < kSplitUnroll; ++u) {
        const int64_t i = i0 + u * kSplitThreads + tid;
        emit(i < c1 && kk[u] > v, kk[u], i);
      }
    }
    return;
  }
  // Ties of this chunk may be kept: walk the chunk in position order, 256
  // entries a round, ranking the ties by position.
  int run = tb;  // ties before the current round
  for (int64_t i0 = c0; i0 < c1; i0 += kSplitThreads) {
    const int64_t i = i0 + tid;
    const bool ok = i < c1;
    const uint32_t kk = ok ? score_key(row[i]) : 0u;
    const bool eq = ok && kk == v;
    const uint64_t me = __ballot(eq);
    if (lane == 0) wcnt[wave] = __popcll(me);
    __syncthreads();
    int before = run;
    for (int w = 0; w < wave; ++w) before += wcnt[w];
    int total = 0;
#pragma unroll
    for (int w = 0; w < kSplitThreads / kWave; ++w) total += wcnt[w];
    const int rank = before + __popcll(me & lt);
    emit((ok && kk > v) || (eq && rank < rem), kk, i);
    run += total;
    __syncthreads();  // wcnt is rewritten by the next round
  }
}

// One workgroup per row: order the kept entries and write the output row.
__global__ void __launch_bounds__(kSelThreads) split_sort_kernel(RowSelArgs a, const SplitState* st,
                                                                 const uint2* staging) {
  __shared__ SortScratch ss;
  __shared__ uint32_t sk[2][kMaxRounds * kSelThreads];
  __shared__ uint32_t sp[2][kMaxRounds * kSelThreads];
  const int e = blockIdx.x, tid = threadIdx.x;
  if (e >= a.gate.live(a.nq)) return;  // uniform: not a live row of this pass
  const int q = split_query(a, e);
  const int need = st[e].need;
  const uint2* src = staging + (int64_t)e * a.topk;
  for (int i = tid; i < need; i += kSelThreads) {
    const uint2 x = src[i];
    sk[0][i] = x.x;
    sp[0][i] = x.y;
  }
  __syncthreads();
  sort_and_emit(sk[0], sp[0], sk[1], sp[1], need, a.topk, a.L, false,
                a.out_idx + (int64_t)q * a.topk,
                a.out_score ? a.out_score + (int64_t)q * a.topk : nullptr, ss);
}

hipError_t launch_row_select_split(const RowSelArgs& a, hipStream_t s) {
  if (a.nq <= 0) return hipSuccess;
  if (a.topk > kMaxRounds * kSelThreads || a.nchunk < 1 || a.chunk_len < 1) return hipErrorInvalidValue;
  const SplitLayout l = split_layout(a.nq, a.nchunk, a.topk);
  uint8_t* ws = static_cast<uint8_t*>(a.scratch);
  SplitState* st = reinterpret_cast<SplitState*>(ws + l.state);
  uint32_t* tiebase = reinterpret_cast<uint32_t*>(ws + l.tiebase);
  uint32_t* hist = reinterpret_cast<uint32_t*>(ws + l.hist);
  uint2* staging = reinterpret_cast<uint2*>(ws + l.staging);
  const dim3 chunks((unsigned)a.nchunk, (unsigned)a.nq), rows((unsigned)a.nq);
  const dim3 blk(kSplitThreads);
  hipLaunchKernelGGL(split_hist_kernel<0>, chunks, blk, 0, s, a, st, hist);
  hipLaunchKernelGGL(split_pick_kernel<0>, rows, blk, 0, s, a, st, hist, tiebase);
  hipLaunchKernelGGL(split_hist_kernel<1>, chunks, blk, 0, s, a, st, hist);
  hipLaunchKernelGGL(split_pick_kernel<1>, rows, blk, 0, s, a, st, hist, tiebase);
  hipLaunchKernelGGL(split_hist_kernel<2>, chunks, blk, 0, s, a, st, hist);
  hipLaunchKernelGGL(split_pick_kernel<2>, rows, blk, 0, s, a, st, hist, tiebase);
  hipLaunchKernelGGL(split_emit_kernel, chunks, blk, 0, s, a, st, hist, tiebase, staging);
  hipLaunchKernelGGL(split_sort_kernel, rows, dim3(kSelThreads), 0, s, a, st, staging);
  return hipGetLastError();
}

}  // namespace hk
