// Gather-dot kernels: score each query against its own list of key positions.
//
// * Replay ("HyScale sparse-attention training -- Selection without a score
//   table", selection-replay paragraph): rescore only the k saved indices of
//   each query, bit-identical to the scores selection returned (see
//   replay_kernel).
// * Sampled threshold (same page, HyTopK and worked-example paragraphs): score
//   M_q = min(M, ctx) evenly spaced keys floor(j * ctx / M_q) of the query's
//   own context and take the ceil(3k * M_q / ctx)-th best as the threshold.
//   One query per workgroup; its 64 heads fill four 16-row MFMA blocks, and a
//   block-wide radix select over the samples (held in LDS) gives tau.
#include "launch.h"
#include "tile.h"

namespace hk {

// ----------------------------------------------------------------- replay

constexpr int kReplayThreads = 256;  // 4 waves, one query each
constexpr int kReplayDepth = 3;      // column blocks of keys in flight per wave

// One query per wave, RB4 row blocks of 16 heads against 16 keys: the tile
// shared by replay and the sampled threshold.  Row block rb holds heads
// 16 rb .. 16 rb + 15, so lane group g holds heads 16 rb + 4 g + i: exactly
// the heads that half (g & 1) of the pair tile holds in its row blocks of
// parity (g >> 1).  Each lane forms the same partial sum the pair tile forms
// for that half and parity, then the partials are combined in the pair
// tile's order ((even + odd), then the other half), which makes every score
// bit-identical to the one the selection kernels compute.
template <int RB4, int D, int FMT>
struct QueryTile {
  using F = Fmt<FMT>;
  using Frag = typename F::Frag;
  static constexpr int RBYTES = D * F::BITS / 8;
  static constexpr int FB = F::FB;
  static constexpr int KS = D / F::KMMA;
  static constexpr int NBLK = D / 32;
  static_assert(KS >= 1 && D % F::KMMA == 0, "unsupported head dimension");

  Frag qa[RB4][KS];
  int sa[RB4][KS];
  float wf[RB4][4];
  i32x8 lin;  // scaled formats: the linear row block (pieces of v in rows 0..5)
  int lsa;

  // lds: this wave's kLinWords dwords of LDS (16-byte aligned) for the linear
  // row block of the scaled formats; unused for bf16.
  __device__ __forceinline__ void load(const uint8_t* q, const float* w, const void* q_scale, int H,
                                       int qi, uint32_t* lds) {
    const int lane = lane_id(), r = lane & 15, g = lane >> 4;
    if constexpr (F::SCALED) {
      static_assert(KS == 1, "the linear row block covers one k-step");
      // two elements of v per lane (the pair tile takes four per lane of a
      // half wave; every element's arithmetic is the same either way)
      float v[2];
      uint32_t code[kLinPieces];
      int scale[kLinPieces];
      lin_v<FMT, D, 2>(q, w, q_scale, H, qi, 2 * lane, v);
      lin_split<FMT, 2, 64>(v, code, scale);
      lin_store<2>(lds, lane, code, scale);
      wave_lds_sync();
      lin_frag<FMT>(lds, r, g, lin, lsa);
    }
    float qs = 1.0f;
    if constexpr (FMT == kFP8) qs = static_cast<const float*>(q_scale)[qi];
#pragma unroll
    for (int rb = 0; rb < RB4; ++rb) {
      const int h = 16 * rb + r;
      const int64_t hr = (int64_t)qi * H + (h < H ? h : 0);
      const uint8_t* src = q + hr * RBYTES;
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        qa[rb][ks] = h < H ? F::frag(src + ks * F::SLICE, g) : Frag{};
        sa[rb][ks] = 127;
        if constexpr (F::MX) {
          if (h < H) sa[rb][ks] = static_cast<const uint8_t*>(q_scale)[hr * NBLK + 4 * ks + g];
        }
      }
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int hw = 16 * rb + 4 * g + i;
        wf[rb][i] = hw < H ? w[(int64_t)qi * H + hw] * qs * (F::SCALED ? 0.5f : 1.0f) : 0.0f;
      }
    }
  }

  // The lane's fragments of key row `key` (-1: zeros) and their MX scales.
  __device__ __forceinline__ static void key(const uint8_t* k, const void* k_scale, int key,
                                             Frag (&b)[KS], int (&sb)[KS]) {
    const int g = lane_id() >> 4;
    const uint8_t* row = k + (int64_t)(key >= 0 ? key : 0) * RBYTES;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      b[ks] = key >= 0 ? F::frag(row + ks * F::SLICE, g) : Frag{};
      sb[ks] = 127;
      if constexpr (F::MX) {
        if (key >= 0) sb[ks] = static_cast<const uint8_t*>(k_scale)[(int64_t)key * NBLK + 4 * ks + g];
      }
    }
  }

  // Score of (query, key lane % 16), in every lane, before the FP8 key scale.
  __device__ __forceinline__ float score(const Frag (&b)[KS], const int (&sb)[KS]) const {
    // one row block at a time (row blocks ascending: the canonical order);
    // for the scaled formats lane groups 0 and 1 start from their rows of the
    // linear term (pieces 0..3 and 4, 5), groups 2 and 3 from zero rows
    float p = 0.0f;
    if constexpr (F::SCALED) {
      const f32x4 l = F::mma_lin(lin, b[0], f32x4{0.f, 0.f, 0.f, 0.f}, lsa, sb[0]);
      p = (l[0] + l[1]) + (l[2] + l[3]);
    }
#pragma unroll
    for (int rb = 0; rb < RB4; ++rb) {
      f32x4 acc = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) acc = F::mma(qa[rb][ks], b[ks], acc, sa[rb][ks], sb[ks]);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float x = F::SCALED ? __builtin_fabsf(acc[i]) : __builtin_fmaxf(acc[i], 0.0f);
        p = __builtin_fmaf(x, wf[rb][i], p);
      }
    }
    const float t = p + __shfl_xor(p, 32);  // even + odd row blocks of this half
    return t + __shfl_xor(t, 16);           // + the other half
  }
};

// Replay: each 16-key column block holds the query's own indices, so no MFMA
// work is wasted; kReplayDepth column blocks of gathers are kept in flight.
template <int RB4, int D, int FMT>
__global__ void __launch_bounds__(kReplayThreads) replay_kernel(ReplayArgs a) {
  using T = QueryTile<RB4, D, FMT>;
  using Frag = typename T::Frag;
  constexpr int KS = T::KS;
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  __shared__ __attribute__((aligned(16))) uint32_t lin_lds[kReplayThreads / kWave][kLinWords];
  const int q = blockIdx.x * (kReplayThreads / kWave) + wave;
  if (q >= a.n) return;  // wave-uniform; no workgroup barrier in this kernel
  const int K = a.topk;

  T qt;
  qt.load(a.q, a.w, a.q_scale, a.H, q, lin_lds[wave]);

  const int* ids = a.idx + (int64_t)q * K;
  float* out = a.out + (int64_t)q * K;
  const int nblk = (K + 15) / 16;

  Frag buf[kReplayDepth][KS];
  int sbuf[kReplayDepth][KS];
  int kid[kReplayDepth];
  float ksc[kReplayDepth];
  auto fetch = [&](int blk, int slot) {
    const int j = blk * 16 + (lane & 15);
    int key = (blk < nblk && j < K) ? ids[j] : -1;
    if (key >= a.L) key = -1;  // out-of-range indices are padding, never dereferenced
    kid[slot] = key;
    T::key(a.k, a.k_scale, key, buf[slot], sbuf[slot]);
    if constexpr (FMT == kFP8) ksc[slot] = key >= 0 ? static_cast<const float*>(a.k_scale)[key] : 0.0f;
  };
#pragma unroll
  for (int d = 0; d < kReplayDepth - 1; ++d) fetch(d, d);

  for (int blk = 0; blk < nblk; blk += kReplayDepth) {
#pragma unroll
    for (int d = 0; d < kReplayDepth; ++d) {
      const int b = blk + d;
      if (b >= nblk) break;  // wave-uniform
      fetch(b + kReplayDepth - 1, (d + kReplayDepth - 1) % kReplayDepth);
      float s = qt.score(buf[d], sbuf[d]);
      if constexpr (FMT == kFP8) s *= ksc[d];
      const int j = b * 16 + lane;
      if (lane < 16 && j < K) out[j] = kid[d] >= 0 ? s : -__builtin_inff();
    }
  }
}

template <int RB4, int D, int FMT>
static hipError_t replay_rb(const ReplayArgs& a, hipStream_t s) {
  constexpr int per = kReplayThreads / kWave;
  dim3 grid((unsigned)((a.n + per - 1) / per)), block(kReplayThreads);
  hipLaunchKernelGGL((replay_kernel<RB4, D, FMT>), grid, block, 0, s, a);
  return hipGetLastError();
}

template <int FMT>
static hipError_t replay_d128(const ReplayArgs& a, bool small, hipStream_t s) {
  return small ? replay_rb<1, 128, FMT>(a, s) : replay_rb<4, 128, FMT>(a, s);
}

hipError_t launch_replay(const ReplayArgs& a, int d, int fmt, hipStream_t s) {
  if (a.n <= 0) return hipSuccess;
  // row blocks of 16 heads: 1 for the narrow pair tile (H <= 8), else 4
  const bool small = a.H <= 8;
  if (fmt == kBF16) {
    if (d == 64) return small ? replay_rb<1, 64, kBF16>(a, s) : replay_rb<4, 64, kBF16>(a, s);
    if (d == 128) return replay_d128<kBF16>(a, small, s);
    return hipErrorInvalidValue;
  }
  if (d != 128) return hipErrorInvalidValue;
  if (fmt == kFP8) return replay_d128<kFP8>(a, small, s);
  if (fmt == kMXFP8) return replay_d128<kMXFP8>(a, small, s);
  if (fmt == kMXFP4) return replay_d128<kMXFP4>(a, small, s);
  return hipErrorInvalidValue;
}

// ----------------------------------------------------------------- threshold

constexpr int kSampleThreads = 256;  // 4 waves share one query's samples
constexpr int kSampleDepth = 3;      // column blocks of gathers in flight per wave

// One query per workgroup.  Row block rb of the A operand holds heads
// 16 rb .. 16 rb + 15 of the query; output lane group g holds heads
// 16 rb + 4 g + i, summed in-lane, then across the four lane groups.
template <int RB4, int D, int FMT>
__global__ void __launch_bounds__(kSampleThreads) sample_tau_kernel(SampleArgs a) {
  using T = QueryTile<RB4, D, FMT>;
  using Frag = typename T::Frag;
  constexpr int KS = T::KS;
  extern __shared__ float S[];  // sample scores, M_q entries
  __shared__ RadixScratch sc;
  __shared__ __attribute__((aligned(16))) uint32_t lin_lds[kSampleThreads / kWave][kLinWords];

  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  // Workgroups are dispatched to the 8 XCDs round-robin; each XCD takes a
  // contiguous run of queries instead, whose sample positions nearly
  // coincide, so that their key gathers hit that XCD's own L2.
  const int q = [] {
    const int nx = 8, b = blockIdx.x, x = b % nx;
    const int base = (int)gridDim.x / nx, extra = (int)gridDim.x % nx;
    return x * base + min(x, extra) + b / nx;
  }();
  const QRange rg = query_range(a.qpos, a.qfirst, a.q_start, a.L, q);
  const int ctx = rg.hi - rg.lo + 1;
  if (ctx <= 0) {  // empty context: nothing passes, nothing is needed (uniform)
    if (tid == 0) a.tau[q] = __builtin_inff();
    return;
  }
  const int mq = min(a.M, ctx);
  const int64_t num = (int64_t)a.oversample * a.topk * mq;
  int r = (int)((num + ctx - 1) / ctx);
  r = max(1, min(mq, r));

  T qt;
  qt.load(a.q, a.w, a.q_scale, a.H, q, lin_lds[wave]);

  // Wave w scores column blocks w, w + 4, ... of 16 samples, with the
  // gathers of the next kSampleDepth - 1 of its blocks in flight while it
  // scores one (the gathers, served from L2 and beyond, are the latency to
  // hide).  Blocks past the last one fetch nothing.
  const int ncb = (mq + 15) / 16;
  constexpr int kStride = kSampleThreads / kWave;
  Frag buf[kSampleDepth][KS];
  int sbuf[kSampleDepth][KS];
  int kpos[kSampleDepth];
  float ksc[kSampleDepth];
  auto fetch = [&](int i, int slot) {  // the wave's i-th block into ring slot `slot`
    const int j = (wave + i * kStride) * 16 + (lane & 15);
    const int pos = j < mq ? rg.lo + (int)(((int64_t)j * ctx) / mq) : -1;
    kpos[slot] = pos;
    T::key(a.k, a.k_scale, pos, buf[slot], sbuf[slot]);
    if constexpr (FMT == kFP8) ksc[slot] = pos >= 0 ? static_cast<const float*>(a.k_scale)[pos] : 0.0f;
  };
  const int nmine = wave < ncb ? (ncb - wave + kStride - 1) / kStride : 0;  // wave-uniform
#pragma unroll
  for (int d = 0; d < kSampleDepth - 1; ++d) fetch(d, d);
  for (int i0 = 0; i0 < nmine; i0 += kSampleDepth) {
#pragma unroll
    for (int d = 0; d < kSampleDepth; ++d) {
      const int i = i0 + d;
      if (i >= nmine) break;  // wave-uniform
      fetch(i + kSampleDepth - 1, (d + kSampleDepth - 1) % kSampleDepth);
      // The selection kernels' head-sum order: a sampled key's score is
      // bit-identical to the score the fused kernel compares with tau, so the
      // r sampled keys at or above tau always pass.
      float s = qt.score(buf[d], sbuf[d]);
      if constexpr (FMT == kFP8) s *= ksc[d];
      const int j = (wave + i * kStride) * 16 + (lane & 15);
      if (lane < 16 && kpos[d] >= 0) S[j] = s;
    }
  }
  __syncthreads();
  int rem, mult;
  const uint32_t v = block_select_largest(
      mq, r, [&](int i) { return score_key(S[i]); }, [](int) { return true; }, sc, rem, mult);
  if (tid == 0) a.tau[q] = key_score(v);
}

template <int RB4, int D, int FMT>
static hipError_t sample_rb(const SampleArgs& a, hipStream_t s) {
  const int mmax = a.M < a.L ? a.M : a.L;
  const size_t lds = (size_t)mmax * sizeof(float);
  hipError_t e = hipFuncSetAttribute((const void*)sample_tau_kernel<RB4, D, FMT>,
                                     hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
  if (e != hipSuccess) return e;
  dim3 grid((unsigned)a.n), block(kSampleThreads);
  hipLaunchKernelGGL((sample_tau_kernel<RB4, D, FMT>), grid, block, lds, s, a);
  return hipGetLastError();
}

template <int FMT>
static hipError_t sample_d128(const SampleArgs& a, bool small, hipStream_t s) {
  return small ? sample_rb<1, 128, FMT>(a, s) : sample_rb<4, 128, FMT>(a, s);
}

hipError_t launch_sample_tau(const SampleArgs& a, int d, int fmt, hipStream_t s) {
  if (a.n <= 0) return hipSuccess;
  const bool small = a.H <= 16;
  if (fmt == kBF16) {
    if (d == 64) return small ? sample_rb<1, 64, kBF16>(a, s) : sample_rb<4, 64, kBF16>(a, s);
    if (d == 128) return sample_d128<kBF16>(a, small, s);
    return hipErrorInvalidValue;
  }
  if (d != 128) return hipErrorInvalidValue;
  if (fmt == kFP8) return sample_d128<kFP8>(a, small, s);
  if (fmt == kMXFP8) return sample_d128<kMXFP8>(a, small, s);
  if (fmt == kMXFP4) return sample_d128<kMXFP4>(a, small, s);
  return hipErrorInvalidValue;
}

}  // namespace hk
