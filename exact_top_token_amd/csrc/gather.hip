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

// One query per wave.  Row block rb holds heads 16 rb .. 16 rb + 15, so lane
// group g holds heads 16 rb + 4 g + i: exactly the heads that half (g & 1) of
// the pair tile holds in its row blocks of parity (g >> 1).  Each lane forms
// the same partial sum the pair tile forms for that half and parity, then the
// partials are combined in the pair tile's order ((even + odd), then the
// other half), which makes every replayed score bit-identical to the selected
// one.  The keys of a column block are the query's own, so no MFMA work is
// wasted, and kReplayDepth column blocks of gathers are kept in flight.
template <int RB4, int D, bool FP8>
__global__ void __launch_bounds__(kReplayThreads) replay_kernel(ReplayArgs a) {
  constexpr int ESIZE = FP8 ? 1 : 2;
  constexpr int RBYTES = D * ESIZE;
  constexpr int FB = FP8 ? 32 : 16;
  constexpr int KS = RBYTES / (4 * FB);
  using Frag = typename std::conditional<FP8, i32x8, bf16x8>::type;
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63, g = lane >> 4;
  const int q = blockIdx.x * (kReplayThreads / kWave) + wave;
  if (q >= a.n) return;  // wave-uniform; no workgroup barrier in this kernel
  const int K = a.topk;

  Frag qa[RB4][KS];
  float wf[RB4][4];
  {
    const int r = lane & 15;
    const float qs = FP8 ? a.q_scale[q] : 1.0f;
#pragma unroll
    for (int rb = 0; rb < RB4; ++rb) {
      const int h = 16 * rb + r;
      const uint8_t* src = a.q + ((int64_t)q * a.H + (h < a.H ? h : 0)) * RBYTES;
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        if (h < a.H) {
          qa[rb][ks] = *reinterpret_cast<const Frag*>(src + (4 * ks + g) * FB);
        } else {
          qa[rb][ks] = Frag{};
        }
      }
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int hw = 16 * rb + 4 * g + i;
        wf[rb][i] = hw < a.H ? a.w[(int64_t)q * a.H + hw] * qs : 0.0f;
      }
    }
  }

  const int* ids = a.idx + (int64_t)q * K;
  float* out = a.out + (int64_t)q * K;
  const int nblk = (K + 15) / 16;

  Frag buf[kReplayDepth][KS];
  int kid[kReplayDepth];
  float ksc[kReplayDepth];
  auto fetch = [&](int blk, int slot) {
    const int j = blk * 16 + (lane & 15);
    int key = (blk < nblk && j < K) ? ids[j] : -1;
    if (key >= a.L) key = -1;  // out-of-range indices are padding, never dereferenced
    kid[slot] = key;
    const uint8_t* row = a.k + (int64_t)(key >= 0 ? key : 0) * RBYTES;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      if (key >= 0) {
        buf[slot][ks] = *reinterpret_cast<const Frag*>(row + (4 * ks + g) * FB);
      } else {
        buf[slot][ks] = Frag{};
      }
    }
    if constexpr (FP8) ksc[slot] = key >= 0 ? a.k_scale[key] : 0.0f;
  };
#pragma unroll
  for (int d = 0; d < kReplayDepth - 1; ++d) fetch(d, d);

  for (int blk = 0; blk < nblk; blk += kReplayDepth) {
#pragma unroll
    for (int d = 0; d < kReplayDepth; ++d) {
      const int b = blk + d;
      if (b >= nblk) break;  // wave-uniform
      fetch(b + kReplayDepth - 1, (d + kReplayDepth - 1) % kReplayDepth);
      f32x4 acc[RB4];
#pragma unroll
      for (int rb = 0; rb < RB4; ++rb) acc[rb] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
#pragma unroll
        for (int rb = 0; rb < RB4; ++rb) {
          if constexpr (FP8) {
            acc[rb] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(qa[rb][ks], buf[d][ks], acc[rb],
                                                                        0, 0, 0, 127, 0, 127);
          } else {
            acc[rb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(qa[rb][ks], buf[d][ks], acc[rb], 0, 0, 0);
          }
        }
      }
      float p = 0.0f;
#pragma unroll
      for (int rb = 0; rb < RB4; ++rb) {
#pragma unroll
        for (int i = 0; i < 4; ++i) p = __builtin_fmaf(__builtin_fmaxf(acc[rb][i], 0.0f), wf[rb][i], p);
      }
      const float t = p + __shfl_xor(p, 32);   // even + odd row blocks of this half
      float s = t + __shfl_xor(t, 16);         // + the other half
      if constexpr (FP8) s *= ksc[d];
      const int j = b * 16 + lane;
      if (lane < 16 && j < K) out[j] = kid[d] >= 0 ? s : -__builtin_inff();
    }
  }
}

template <int RB4, int D, bool FP8>
static hipError_t replay_rb(const ReplayArgs& a, hipStream_t s) {
  constexpr int per = kReplayThreads / kWave;
  dim3 grid((unsigned)((a.n + per - 1) / per)), block(kReplayThreads);
  hipLaunchKernelGGL((replay_kernel<RB4, D, FP8>), grid, block, 0, s, a);
  return hipGetLastError();
}

hipError_t launch_replay(const ReplayArgs& a, int d, bool fp8, hipStream_t s) {
  if (a.n <= 0) return hipSuccess;
  // row blocks of 16 heads: 1 for the narrow pair tile (H <= 8), else 4
  const bool small = a.H <= 8;
  if (fp8) {
    if (d != 128) return hipErrorInvalidValue;
    return small ? replay_rb<1, 128, true>(a, s) : replay_rb<4, 128, true>(a, s);
  }
  if (d == 64) return small ? replay_rb<1, 64, false>(a, s) : replay_rb<4, 64, false>(a, s);
  if (d == 128) return small ? replay_rb<1, 128, false>(a, s) : replay_rb<4, 128, false>(a, s);
  return hipErrorInvalidValue;
}

// ----------------------------------------------------------------- threshold

constexpr int kSampleThreads = 256;  // 4 waves share one query's samples

// One query per workgroup.  Row block rb of the A operand holds heads
// 16 rb .. 16 rb + 15 of the query; output lane group g holds heads
// 16 rb + 4 g + i, summed in-lane, then across the four lane groups.
template <int RB4, int D, bool FP8>
__global__ void __launch_bounds__(kSampleThreads) sample_tau_kernel(SampleArgs a) {
  constexpr int ESIZE = FP8 ? 1 : 2;
  constexpr int RBYTES = D * ESIZE;
  constexpr int FB = FP8 ? 32 : 16;
  constexpr int KS = RBYTES / (4 * FB);
  using Frag = typename std::conditional<FP8, i32x8, bf16x8>::type;
  extern __shared__ float S[];  // sample scores, M_q entries
  __shared__ RadixScratch sc;

  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63, g = lane >> 4;
  const int q = blockIdx.x;
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

  Frag qa[RB4][KS];
  float wf[RB4][4];
  {
    const int rr = lane & 15;
    float qs = 1.0f;
    if (FP8) qs = a.q_scale[q];
#pragma unroll
    for (int rb = 0; rb < RB4; ++rb) {
      const int h = 16 * rb + rr;
      const uint8_t* src = a.q + ((int64_t)q * a.H + (h < a.H ? h : 0)) * RBYTES;
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        if (h < a.H) {
          qa[rb][ks] = *reinterpret_cast<const Frag*>(src + (4 * ks + g) * FB);
        } else {
          qa[rb][ks] = Frag{};
        }
      }
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int hw = 16 * rb + 4 * g + i;
        wf[rb][i] = hw < a.H ? a.w[(int64_t)q * a.H + hw] * qs : 0.0f;
      }
    }
  }

  for (int cb = wave; cb * 16 < mq; cb += kSampleThreads / kWave) {
    const int j = cb * 16 + (lane & 15);
    const int pos = j < mq ? rg.lo + (int)(((int64_t)j * ctx) / mq) : -1;
    Frag b[KS];
    const uint8_t* row = a.k + (int64_t)(pos >= 0 ? pos : 0) * RBYTES;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      if (pos >= 0) {
        b[ks] = *reinterpret_cast<const Frag*>(row + (4 * ks + g) * FB);
      } else {
        b[ks] = Frag{};
      }
    }
    f32x4 acc[RB4];
#pragma unroll
    for (int rb = 0; rb < RB4; ++rb) acc[rb] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
#pragma unroll
      for (int rb = 0; rb < RB4; ++rb) {
        if constexpr (FP8) {
          acc[rb] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(qa[rb][ks], b[ks], acc[rb], 0, 0,
                                                                      0, 127, 0, 127);
        } else {
          acc[rb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(qa[rb][ks], b[ks], acc[rb], 0, 0, 0);
        }
      }
    }
    // The selection kernels' head-sum order (as in replay_kernel): a lane's
    // partial over its heads, then lane ^ 32 (the other row-block parity of
    // the pair tile), then lane ^ 16 (the other half).  A sampled key's score
    // is then bit-identical to the score the fused kernel compares with tau,
    // so the r sampled keys at or above tau always pass.
    float p = 0.0f;
#pragma unroll
    for (int rb = 0; rb < RB4; ++rb) {
#pragma unroll
      for (int i = 0; i < 4; ++i) p = __builtin_fmaf(__builtin_fmaxf(acc[rb][i], 0.0f), wf[rb][i], p);
    }
    const float t = p + __shfl_xor(p, 32);
    float s = t + __shfl_xor(t, 16);
    if constexpr (FP8) s *= pos >= 0 ? a.k_scale[pos] : 0.0f;
    if (lane < 16 && j < mq) S[j] = s;
  }
  __syncthreads();
  int rem, mult;
  const uint32_t v = block_select_largest(
      mq, r, [&](int i) { return score_key(S[i]); }, [](int) { return true; }, sc, rem, mult);
  if (tid == 0) a.tau[q] = key_score(v);
}

template <int RB4, int D, bool FP8>
static hipError_t sample_rb(const SampleArgs& a, hipStream_t s) {
  const int mmax = a.M < a.L ? a.M : a.L;
  const size_t lds = (size_t)mmax * sizeof(float);
  hipError_t e = hipFuncSetAttribute((const void*)sample_tau_kernel<RB4, D, FP8>,
                                     hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
  if (e != hipSuccess) return e;
  dim3 grid((unsigned)a.n), block(kSampleThreads);
  hipLaunchKernelGGL((sample_tau_kernel<RB4, D, FP8>), grid, block, lds, s, a);
  return hipGetLastError();
}

hipError_t launch_sample_tau(const SampleArgs& a, int d, bool fp8, hipStream_t s) {
  if (a.n <= 0) return hipSuccess;
  const bool small = a.H <= 16;
  if (fp8) {
    if (d != 128) return hipErrorInvalidValue;
    return small ? sample_rb<1, 128, true>(a, s) : sample_rb<4, 128, true>(a, s);
  }
  if (d == 64) return small ? sample_rb<1, 64, false>(a, s) : sample_rb<4, 64, false>(a, s);
  if (d == 128) return small ? sample_rb<1, 128, false>(a, s) : sample_rb<4, 128, false>(a, s);
  return hipErrorInvalidValue;
}

}  // namespace hk
