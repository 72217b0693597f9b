// The indexer tile: one wave scores a PAIR of queries against 16 keys at a
// time with v_mfma_f32_16x16x32_bf16 (bf16) or v_mfma_scale_f32_16x16x128_f8f6f4
// (OCP FP8 E4M3), then applies ReLU and the weighted head sum in registers.
//
// Indexer: I(t,s) = sum_h w[t,h] * ReLU(q[t,h] . k[s]).
//
// MFMA operand layout (16x16 output tile, 64 lanes, lane group g = lane / 16):
//   A (16 rows x K): lane holds row (lane % 16); rows 0..7 are heads of query A
//     and rows 8..15 heads of query B, so row block rb covers heads 8rb..8rb+7
//     of both queries.  The K slice of lane group g at k-step ks is byte range
//     [(4 ks + g) * FB, +FB) of the head's row (FB = 16 bytes for bf16,
//     32 bytes for FP8); B uses the same slices, so every pair (row, key)
//     meets the full d-dimension exactly once over the k-steps.
//   B (K x 16 keys): lane holds key column (lane % 16).
//   D: lane holds rows 4g..4g+3 of column (lane % 16): lanes 0..31 therefore
//     hold 32 heads of query A (heads 8rb + 4(g & 1) + i), lanes 32..63 the
//     same heads of query B.
// Epilogue: each lane sums w * max(acc, 0) over its 32 heads in a fixed order
// (two partials, see epilogue()), then adds its partner lane (lane ^ 16).  A
// (query, key) score is bit-identical whichever kernel, tile position or query
// pairing computed it.
#pragma once

#include "common.h"

namespace hk {

template <int RB, int D, bool FP8>
struct PairTile {
  static constexpr int ESIZE = FP8 ? 1 : 2;              // bytes per element
  static constexpr int RBYTES = D * ESIZE;                // bytes per head row / key row
  static constexpr int FB = FP8 ? 32 : 16;                // fragment bytes per lane per k-step
  static constexpr int KS = RBYTES / (4 * FB);            // k-steps over the d-dimension
  static constexpr int NCH = RBYTES / 16;                 // 16-byte chunks per key row
  static constexpr int HMAX = 8 * RB;                     // heads covered (zero-padded)
  using Frag = typename std::conditional<FP8, i32x8, bf16x8>::type;
  static_assert(KS >= 1 && RBYTES % (4 * FB) == 0, "unsupported head dimension");

  Frag a[RB][KS];   // query pair, A operand
  float wf[RB][4];  // head weights of this lane's 32 heads (times q_scale for FP8)

  // Load the A operand and weights of query indices qa / qb (-1 = absent).
  __device__ __forceinline__ void load(const uint8_t* __restrict__ q, const float* __restrict__ w,
                                       const float* __restrict__ q_scale, int H, int qa, int qb) {
    const int lane = lane_id();
    const int r = lane & 15, g = lane >> 4;
    const int qrow = (r >> 3) ? qb : qa;
#pragma unroll
    for (int rb = 0; rb < RB; ++rb) {
      const int h = 8 * rb + (r & 7);
      const bool ok = qrow >= 0 && h < H;
      const uint8_t* src = q + ((int64_t)(ok ? qrow : 0) * H + (ok ? h : 0)) * RBYTES;
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        if (ok) {
          a[rb][ks] = *reinterpret_cast<const Frag*>(src + (4 * ks + g) * FB);
        } else {
          a[rb][ks] = Frag{};
        }
      }
    }
    const int qw = (lane >> 5) ? qb : qa;
    const int hb = 4 * (g & 1);
    float qs = 1.0f;
    if (FP8 && qw >= 0) qs = q_scale[qw];
#pragma unroll
    for (int rb = 0; rb < RB; ++rb) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int h = 8 * rb + hb + i;
        wf[rb][i] = (qw >= 0 && h < H) ? w[(int64_t)qw * H + h] * qs : 0.0f;
      }
    }
  }

  __device__ __forceinline__ static f32x4 mfma(const Frag& a, const Frag& b, const f32x4& c) {
    if constexpr (FP8) {
      // cbsz = blgp = 0: both operands OCP FP8 E4M3; scale exponents 127 = 2^0.
      return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, c, 0, 0, 0, 127, 0, 127);
    } else {
      return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
    }
  }

  // Scores of both queries against 16 keys whose B fragments are b[ks].
  // Returns this lane's score: query (lane < 32 ? A : B), key (lane % 16),
  // before the per-key FP8 scale.
  __device__ __forceinline__ float score(const Frag (&b)[KS]) const {
    f32x4 acc[RB];
#pragma unroll
    for (int rb = 0; rb < RB; ++rb) acc[rb] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
#pragma unroll
      for (int rb = 0; rb < RB; ++rb) acc[rb] = mfma(a[rb][ks], b[ks], acc[rb]);
    }
    return epilogue(acc);
  }

  // Canonical head-sum order (every kernel that produces a score follows it):
  // per lane, one partial over the even row blocks and one over the odd row
  // blocks (row block ascending, register ascending), t = even + odd, then
  // t + t(lane ^ 16).  A tile holding one query per MFMA (16 heads per row
  // block) sees the same four partials in its four lane groups.
  __device__ __forceinline__ float epilogue(const f32x4 (&acc)[RB]) const {
    float se = 0.0f, so = 0.0f;
#pragma unroll
    for (int rb = 0; rb < RB; ++rb) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float r = __builtin_fmaxf(acc[rb][i], 0.0f);
        if (rb & 1) {
          so = __builtin_fmaf(r, wf[rb][i], so);
        } else {
          se = __builtin_fmaf(r, wf[rb][i], se);
        }
      }
    }
    const float t = se + so;
    return t + __shfl_xor(t, 16);
  }
};

}  // namespace hk
