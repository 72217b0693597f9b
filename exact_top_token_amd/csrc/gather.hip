// Gather-dot kernels: score each query against its own list of key positions.
//
// * Replay ("HyScale sparse-attention training -- Selection without a score
//   table", selection-replay paragraph): rescore only the k saved indices of
//   each query.  It uses the pair tile of the fused scoring kernel, so the
//   replayed scores are bit-identical to the scores selection returned.  The
//   16 keys of one column block belong to ONE query of the pair, so each
//   column block is scored twice (once with query A's keys, once with B's) and
//   the other half of the tile is discarded: replay moves k key rows per query
//   and is bound by that traffic, not by the doubled MFMA work.
// * Sampled threshold (same page, HyTopK and worked-example paragraphs): score
//   M_q = min(M, ctx) evenly spaced keys floor(j * ctx / M_q) of the query's
//   own context and take the ceil(3k * M_q / ctx)-th best as the threshold.
//   One query per workgroup; its 64 heads fill four 16-row MFMA blocks, and a
//   block-wide radix select over the samples (held in LDS) gives tau.
#include "launch.h"
#include "tile.h"

namespace hk {

// ----------------------------------------------------------------- replay

constexpr int kReplayThreads = 512;  // 8 waves = 8 query pairs

template <int RB, int D, bool FP8>
__global__ void __launch_bounds__(kReplayThreads) replay_kernel(ReplayArgs a) {
  using T = PairTile<RB, D, FP8>;
  using Frag = typename T::Frag;
  constexpr int RBYTES = T::RBYTES, KS = T::KS, FB = T::FB;
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63, g = lane >> 4;
  const int e0 = blockIdx.x * 16 + wave * 2;
  const int qa = e0 < a.n ? e0 : -1;
  const int qb = e0 + 1 < a.n ? e0 + 1 : -1;
  if (qa < 0) return;  // wave-uniform; no workgroup barrier below
  T qt;
  qt.load(a.q, a.w, a.q_scale, a.H, qa, qb);
  const int K = a.topk;

  auto fetch = [&](const int* ids, int j0, Frag (&b)[KS], int& key) {
    const int j = j0 + (lane & 15);
    key = j < K ? ids[j] : -1;
    if (key >= a.L) key = -1;  // out-of-range indices are padding, never dereferenced
    const uint8_t* row = a.k + (int64_t)(key >= 0 ? key : 0) * RBYTES;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      if (key >= 0) {
        b[ks] = *reinterpret_cast<const Frag*>(row + (4 * ks + g) * FB);
      } else {
        b[ks] = Frag{};
      }
    }
  };

  for (int pass = 0; pass < 2; ++pass) {
    const int qp = pass ? qb : qa;
    if (qp < 0) break;
    const int* ids = a.idx + (int64_t)qp * K;
    float* out = a.out + (int64_t)qp * K;
    const bool mine = pass ? (lane >= 32 && lane < 48) : (lane < 16);
    Frag bc[KS], bn[KS];
    int kc, kn = -1;
    fetch(ids, 0, bc, kc);
    for (int j0 = 0; j0 < K; j0 += 16) {
      if (j0 + 16 < K) fetch(ids, j0 + 16, bn, kn);
      float s = qt.score(bc);
      if constexpr (FP8) s *= kc >= 0 ? a.k_scale[kc] : 0.0f;
      const int j = j0 + (lane & 15);
      if (mine && j < K) out[j] = kc >= 0 ? s : -__builtin_inff();
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) bc[ks] = bn[ks];
      kc = kn;
    }
  }
}

template <int RB, int D, bool FP8>
static hipError_t replay_rb(const ReplayArgs& a, hipStream_t s) {
  dim3 grid((unsigned)((a.n + 15) / 16)), block(kReplayThreads);
  hipLaunchKernelGGL((replay_kernel<RB, D, FP8>), grid, block, 0, s, a);
  return hipGetLastError();
}

hipError_t launch_replay(const ReplayArgs& a, int d, bool fp8, hipStream_t s) {
  if (a.n <= 0) return hipSuccess;
  const bool small = a.H <= 8;
  if (fp8) {
    if (d != 128) return hipErrorInvalidValue;
    return small ? replay_rb<1, 128, true>(a, s) : replay_rb<8, 128, true>(a, s);
  }
  if (d == 64) return small ? replay_rb<1, 64, false>(a, s) : replay_rb<8, 64, false>(a, s);
  if (d == 128) return small ? replay_rb<1, 128, false>(a, s) : replay_rb<8, 128, false>(a, s);
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
  const int ctx = a.q_start + q + 1;
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
    const int pos = j < mq ? (int)(((int64_t)j * ctx) / mq) : -1;
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
    float s = 0.0f;
#pragma unroll
    for (int rb = 0; rb < RB4; ++rb) {
#pragma unroll
      for (int i = 0; i < 4; ++i) s = __builtin_fmaf(__builtin_fmaxf(acc[rb][i], 0.0f), wf[rb][i], s);
    }
    s += __shfl_xor(s, 16);
    s += __shfl_xor(s, 32);
    if constexpr (FP8) s *= pos >= 0 ? a.k_scale[pos] : 0.0f;
    if (lane < 16 && j < mq) S[j] = s;
  }
  __syncthreads();
  int rem;
  const uint32_t v = block_select_largest(
      mq, r, [&](int i) { return score_key(S[i]); }, [](int) { return true; }, sc, rem);
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
