// Internal host-side launch interface between the C ABI (api.hip) and the
// kernel translation units.  Every launcher enqueues on `s` and returns the
// hipError_t of the launch.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <algorithm>
#include <atomic>
#include <mutex>

namespace hk {

// Per-device record of the dynamic-LDS limit a kernel was given.
struct LdsLimit {
  static constexpr int kDevices = 64;
  std::atomic<int> bytes[kDevices];
  std::mutex mu;  // orders the raises, so the recorded limit is the one in force
};

// Raises `fn`'s dynamic-LDS limit to at least `bytes` on the current device,
// once: later launches that fit the limit make no runtime call (so a launch
// recorded in a stream capture after a first call outside it makes none).
// Raises never lower the limit, also when threads race.
inline hipError_t raise_dynamic_lds(const void* fn, int bytes, LdsLimit& lim) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= LdsLimit::kDevices)
    return hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize, bytes);
  if (lim.bytes[dev].load(std::memory_order_acquire) >= bytes) return hipSuccess;
  std::lock_guard<std::mutex> g(lim.mu);
  const int want = std::max(bytes, lim.bytes[dev].load(std::memory_order_relaxed));
  e = hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize, want);
  if (e != hipSuccess) return e;
  lim.bytes[dev].store(want, std::memory_order_release);
  return hipSuccess;
}

// Device-side row count of a row-path pass enqueued without a host
// synchronisation (recovery in hytopk_select_async): the pass covers list
// entries base .. base + nq - 1 of a list whose length the device holds in
// *count; entries at or beyond that length do nothing, and a length above
// max_count (too many failures for recovery) makes the whole pass empty.
// count == null: every entry of the pass is live.
struct RowGate {
  const int* count;
  int max_count;
  int base;
  __device__ __forceinline__ int live(int nq) const {
    if (!count) return nq;
    const int c = *count;
    if (c > max_count) return 0;
    const int r = c - base;
    return r < 0 ? 0 : (r < nq ? r : nq);
  }
};

// Fused indexer scoring over causal key ranges.
//   COMPACT (rows == nullptr): keys with score >= tau[q] go to the candidate
//     buffer cand[q][0..cap) as {position, fp32 bits}; cnt[q] counts every
//     passing key, including those beyond cap.
//   ROWS (rows != nullptr): the score of every causal key is written to
//     rows[e * row_stride + key] for launch entry e.
// Launch entry e scores query qlist[e] (or q_offset + e when qlist is null).
struct ScoreArgs {
  const uint8_t* q;
  const uint8_t* k;
  const float* w;
  const void* q_scale;   // fp32 [n] (FP8) or E8M0 [n][H][d/32] (MX)
  const void* k_scale;   // fp32 [L] (FP8) or E8M0 [L][d/32] (MX)
  const float* tau;
  int* cnt;
  uint2* cand;
  float* rows;
  const int* qlist;
  const int* qpos;     // [n] query positions, or null (q_start + i)
  const int* qfirst;   // [n] first key of each query's context, or null (0)
  int64_t row_stride;
  int L;
  int q_start;
  int q_offset;
  int nq;
  int H;
  int cap;
  int nsplit;
  int split_len;
  int reverse;         // 1: walk each launch entry's key tiles from last to first
  RowGate gate;        // ROWS: device-side count of live entries (count null: all nq)
};

hipError_t launch_score(const ScoreArgs& a, int d, int fmt, hipStream_t s);
int score_group_queries(int fmt);  // queries per workgroup of the score kernel

// Per-query sampled threshold: tau[q] = the r-th largest of the M_q sample
// scores at positions floor(j * ctx / M_q).
struct SampleArgs {
  const uint8_t* q;
  const uint8_t* k;
  const float* w;
  const void* q_scale;   // fp32 [n] (FP8) or E8M0 [n][H][d/32] (MX)
  const void* k_scale;   // fp32 [L] (FP8) or E8M0 [L][d/32] (MX)
  float* tau;
  const int* qpos;
  const int* qfirst;
  int L;
  int q_start;
  int n;
  int H;
  int topk;
  int M;
  int oversample;
};

hipError_t launch_sample_tau(const SampleArgs& a, int d, int fmt, hipStream_t s);

// Replay: out[q][j] = I(q_start + q, idx[q][j]) (-inf where idx is outside [0, L)).
struct ReplayArgs {
  const uint8_t* q;
  const uint8_t* k;
  const float* w;
  const void* q_scale;   // fp32 [n] (FP8) or E8M0 [n][H][d/32] (MX)
  const void* k_scale;   // fp32 [L] (FP8) or E8M0 [L][d/32] (MX)
  const int* idx;
  float* out;
  int L;
  int n;
  int H;
  int topk;
};

hipError_t launch_replay(const ReplayArgs& a, int d, int fmt, hipStream_t s);

// Device counters of one selection call.
struct DevStats {
  int n_overflow;
  int n_underk;
  int n_failed;
  int cand_max;
  unsigned long long cand_total;
  int pad[2];
};

hipError_t launch_zero(int* cnt, int n, DevStats* st, hipStream_t s);

// The device status words of hytopk_select_async (HYTOPK_ASYNC_STATUS_WORDS
// int32): [0] 1 when more than max_recover queries failed (their rows were
// not recovered), [1] failures, [2] overflows, [3] under-k queries, [4] the
// largest candidate count, [5], [6] the candidate total (low, high 32 bits),
// [7] 0.
hipError_t launch_async_status(const DevStats* st, int max_recover, int32_t* out, hipStream_t s);

// Check: flags queries whose candidate count is above cap or below
// min(k, ctx) and appends them to `failed`.
hipError_t launch_check(const int* cnt, int n, const int* qpos, const int* qfirst, int q_start,
                        int L, int topk, int cap, DevStats* st, int* failed, hipStream_t s);

// Exact top-k of each passing query's candidates (failed queries are skipped).
hipError_t launch_cand_select(const int* cnt, const uint2* cand, int n, const int* qpos,
                              const int* qfirst, int q_start, int topk, int cap, int L,
                              int* out_idx, float* out_score, hipStream_t s);

// Exact top-k of score rows: entry e is row rows[e * row_stride] of query
// qlist[e] (or q_offset + e).
hipError_t launch_row_topk(const float* rows, int64_t row_stride, const int* qlist, int q_offset,
                           int nq, const int* qpos, const int* qfirst, int q_start, int topk, int L,
                           int* out_idx, float* out_score, RowGate gate, hipStream_t s);

// Exact top-k of a few long score rows, each row split over `nchunk`
// workgroups of `chunk_len` entries (recovery and the full rescore): three
// radix passes over the rows find each row's k-th largest key, an emission
// pass keeps the entries above it and the lowest-position entries equal to
// it, and one workgroup per row sorts the kept entries.  Same result as
// launch_row_topk.
struct RowSelArgs {
  const float* rows;
  int64_t row_stride;
  const int* qlist;    // entry e is query qlist[e] (or q_offset + e)
  int q_offset;
  int nq;
  const int* qpos;
  const int* qfirst;
  int q_start;
  int topk;
  int L;
  int nchunk;          // workgroups per row
  int chunk_len;       // entries per workgroup (a multiple of 1024)
  void* scratch;       // row_select_scratch_bytes(nq, nchunk, topk) bytes, 256-byte aligned
  int* out_idx;
  float* out_score;
  RowGate gate;        // device-side count of live entries (count null: all nq)
};

hipError_t launch_row_select_split(const RowSelArgs& a, hipStream_t s);
size_t row_select_scratch_bytes(int nrows, int nchunk, int topk);
int row_select_max_chunks(int64_t L);
// Chunking of rows of up to maxctx entries for nq rows (nchunk <= row_select_max_chunks(L)).
void row_select_chunks(int nq, int64_t maxctx, int64_t L, int& nchunk, int& chunk_len);
constexpr int kRowSplitMaxRows = 128;  // more rows than this fill the GPU one workgroup per row

// LDS bytes cand_select needs for this cap / k (the host checks the limit).
size_t cand_select_lds_bytes(int cap, int topk);


// Indexer backward at the replayed entries (backward.hip).
struct BwdArgs {
  const uint16_t* q;   // bf16 bits [n][H][d]
  const uint16_t* k;   // bf16 bits [L][d]
  const float* w;      // [n][H]
  const int* idx;      // [n][topk]
  const float* dsc;    // [n][topk] upstream gradient of each replayed score
  float* dq;           // [n][H][d] or null
  float* dw;           // [n][H] or null
  float* u;            // [nq * bwd_padded_k(topk)][d] dk rows of the chunk's entries, or null
  const float* q_scale;  // [n] per-token FP8 scales of q and k (q, k then hold the codes
  const float* k_scale;  // [L] as bf16), or null for bf16 / dequantized MX inputs
  int L;
  int H;
  int topk;
  int q0;              // first query of the chunk
  int nq;              // queries in the chunk
};

hipError_t launch_bwd_query(const BwdArgs& a, int d, hipStream_t s);
// Scaled-format q or k ([rows][d] elements) as bf16 bits for the backward.
hipError_t launch_bwd_dequant(const void* x, const void* scale, int64_t rows, int d, int fmt,
                              uint16_t* out, hipStream_t s);

struct DkArgs {
  const int* idx;      // the chunk's [nq][topk] indices (entry e = row-major position)
  int L;
  int N;               // entries in the chunk (nq * topk)
  int topk;
  uint32_t* k0;        // [N] sort ping-pong buffers
  uint32_t* v0;
  uint32_t* k1;
  uint32_t* v1;
  uint32_t* hist;      // [bwd_sort_hist_count(N)]: per-tile digit counts, digit totals
};

// Groups the chunk's entries by key: stable sort of (key position, u row)
// by key (padding last); returns the sorted keys and rows.
hipError_t launch_bwd_sort(const DkArgs& a, const uint32_t** sorted_keys,
                           const uint32_t** sorted_rows, hipStream_t s);
// dk[s] = (or +=) the sum of the u rows of key s's run, in sorted order.
hipError_t launch_bwd_segments(const uint32_t* sorted_keys, const uint32_t* sorted_rows, int N,
                               int L, const float* u, float* dk, bool accumulate, int d,
                               hipStream_t s);
int bwd_padded_k(int topk);  // key slots per query in the u buffer
hipError_t launch_fill_zero(float* p, int64_t n, hipStream_t s);
size_t bwd_sort_hist_count(int64_t N);

}  // namespace hk
