// The indexer tile: one wave scores a PAIR of queries against 16 keys at a
// time with 16x16 MFMAs (see Fmt in common.h for the per-format
// instruction), then applies ReLU and the weighted head sum in registers.
//
// Indexer: I(t,s) = sum_h w[t,h] * ReLU(q[t,h] . k[s]).
//
// MFMA operand layout (16x16 output tile, 64 lanes, lane group g = lane / 16):
//   A (16 rows x K): lane holds row (lane % 16); rows 0..7 are heads of query A
//     and rows 8..15 heads of query B, so row block rb covers heads 8rb..8rb+7
//     of both queries.  Lane group g holds, at k-step ks, the chunks of the
//     row's k-step slice that Fmt::frag names (one FB-byte run for bf16, E2M1
//     and per-token E4M3); B uses the same chunks, so every pair (row, key)
//     meets the full d-dimension exactly once over the k-steps.  For the MX
//     formats lane group g's elements are the instruction's K block g, which
//     is the row's 32-element block 4 ks + g, and the lane passes that
//     block's E8M0 scale with its operand.
//   B (K x 16 keys): lane holds key column (lane % 16).
//   D: lane holds rows 4g..4g+3 of column (lane % 16): lanes 0..31 therefore
//     hold 32 heads of query A (heads 8rb + 4(g & 1) + i), lanes 32..63 the
//     same heads of query B.
// Epilogue: each lane sums w * max(acc, 0) over its 32 heads in a fixed order
// (two partials, see score()), then adds its partner lane (lane ^ 16).  A
// (query, key) score is bit-identical whichever kernel, tile position or query
// pairing computed it.
#pragma once

#include "common.h"

namespace hk {

template <int RB, int D, int FMT>
struct PairTile {
  using F = Fmt<FMT>;
  using Frag = typename F::Frag;
  static constexpr int RBYTES = D * F::BITS / 8;          // bytes per head row / key row
  static constexpr int FB = F::FB;                        // fragment bytes per lane per k-step
  static constexpr int KS = D / F::KMMA;                  // k-steps over the d-dimension
  static constexpr int NCH = RBYTES / 16;                 // 16-byte chunks per key row
  static constexpr int NBLK = D / 32;                     // MX blocks per row
  static constexpr int HMAX = 8 * RB;                     // heads covered (zero-padded)
  static_assert(KS >= 1 && D % F::KMMA == 0, "unsupported head dimension");

  Frag a[RB][KS];   // query pair, A operand
  int sa[RB][KS];   // E8M0 scale of each A fragment's block (MX; 127 otherwise)
  float wf[RB][4];  // head weights of this lane's 32 heads (times q_scale for FP8)

  // Load the A operand and weights of query indices qa / qb (-1 = absent).
  // q_scale: fp32 [n] (FP8) or E8M0 bytes [n][H][D/32] (MX).
  __device__ __forceinline__ void load(const uint8_t* __restrict__ q, const float* __restrict__ w,
                                       const void* __restrict__ q_scale, int H, int qa, int qb) {
    const int lane = lane_id();
    const int r = lane & 15, g = lane >> 4;
    const int qrow = (r >> 3) ? qb : qa;
#pragma unroll
    for (int rb = 0; rb < RB; ++rb) {
      const int h = 8 * rb + (r & 7);
      const bool ok = qrow >= 0 && h < H;
      const int64_t hr = (int64_t)(ok ? qrow : 0) * H + (ok ? h : 0);
      const uint8_t* src = q + hr * RBYTES;
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        a[rb][ks] = ok ? F::frag(src + ks * F::SLICE, g) : Frag{};
        sa[rb][ks] = 127;
        if constexpr (F::MX) {
          if (ok) sa[rb][ks] = static_cast<const uint8_t*>(q_scale)[hr * NBLK + 4 * ks + g];
        }
      }
    }
    const int qw = (lane >> 5) ? qb : qa;
    const int hb = 4 * (g & 1);
    float qs = 1.0f;
    if constexpr (FMT == kFP8) {
      if (qw >= 0) qs = static_cast<const float*>(q_scale)[qw];
    }
#pragma unroll
    for (int rb = 0; rb < RB; ++rb) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int h = 8 * rb + hb + i;
        wf[rb][i] = (qw >= 0 && h < H) ? w[(int64_t)qw * H + h] * qs : 0.0f;
      }
    }
  }

  // Scores of both queries against 16 keys whose B fragments are b[ks] (with
  // E8M0 scales sb[ks] for MX).  Returns this lane's score: query (lane < 32 ?
  // A : B), key (lane % 16), before the per-key FP8 scale.
  //
  // Canonical head-sum order (every kernel that produces a score follows it):
  // per lane, one partial over the even row blocks and one over the odd row
  // blocks (row block ascending, register ascending), t = even + odd, then
  // t + t(lane ^ 16).  A tile holding one query per MFMA (16 heads per row
  // block) sees the same four partials in its four lane groups.
  __device__ __forceinline__ float score(const Frag (&b)[KS], const int (&sb)[KS]) const {
    // one row block at a time: its k-steps, then its share of the head sum
    // (row blocks ascending, so the partials follow the canonical order)
    float se = 0.0f, so = 0.0f;
#pragma unroll
    for (int rb = 0; rb < RB; ++rb) {
      f32x4 acc = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) acc = F::mma(a[rb][ks], b[ks], acc, sa[rb][ks], sb[ks]);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float r = __builtin_fmaxf(acc[i], 0.0f);
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
