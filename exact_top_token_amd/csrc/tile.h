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
//
// The scaled formats (FP8, MXFP8, MXFP4) take the weighted ReLU apart as
// w * ReLU(x) = (w/2) * |x| + (w/2) * x.  Summed over the heads, the second
// part is a single dot product v . k with v = sum_h (w_h / 2) q_h, which one
// more MFMA row block computes; the per-head work left for the vector ALUs is
// one fma with |acc| (an input modifier) instead of a max and an fma.  On
// these formats the epilogue costs about as much as the MFMAs, and this takes
// 4-5% off the scoring time at the 1M shape for FP8 and MXFP8, about 9% for
// MXFP4 (bf16 keeps max + fma: there the extra row block costs more than it
// saves and its registers do not fit).  v is
// fp32; the MFMA operand carries it as kLinPieces rows of 4-significant-bit
// elements with one E8M0 scale each, piece j being the rounding of what pieces
// 0..j-1 left over (see lin_split), so that the pieces sum to v within 2^-24
// of its largest element and exactly whenever v has fewer significant bits
// than that.  The elements are E4M3 against E4M3 keys and FP6 E2M3 against
// MXFP4's E2M1 keys: the MFMA runs at the rate of its wider operand, and an
// E4M3 row block costs an E2M1 key tile twice what an E2M3 one does.
#pragma once

#include "common.h"

namespace hk {

// ------------------------------------------------------------ linear term

constexpr int kLinPieces = 6;   // pieces of v (E4M3 or E2M3, about 4 bits each)
constexpr int kLinWords = 200;  // LDS dwords per query: 32 per piece, the scales, padding

// Element decoders.  fp32 denormals are kept (the kernels' float mode), so
// a code's exponent and mantissa bits placed at the top of an fp32 mantissa
// and scaled by a power of two give its value, subnormal codes included.
// Finite OCP FP8 E4M3 code in bits 24..31 of t -> value (bias 7).
__device__ __forceinline__ float e4m3_top(uint32_t t) {
  return __uint_as_float((t & 0x80000000u) | ((t >> 4) & 0x07F00000u)) * 0x1p120f;
}

// OCP FP4 E2M1 code in bits 28..31 of t -> value (bias 1).
__device__ __forceinline__ float e2m1_top(uint32_t t) {
  return __uint_as_float((t & 0x80000000u) | ((t >> 6) & 0x01C00000u)) * 0x1p126f;
}

// E8M0 scale byte (< 255) -> 2^(s - 127).
__device__ __forceinline__ float e8m0_value(uint32_t s) {
  return s ? __uint_as_float(s << 23) : 0x1p-127f;
}

// E2M3 code (6 bits: sign, 2 exponent bits with bias 1, 3 mantissa bits) of
// a value that E2M3 holds exactly (|p| <= 7.5).
__device__ __forceinline__ uint32_t e2m3_code(float p) {
  const uint32_t u = __float_as_uint(p), a = u & 0x7FFFFFFFu;
  const float m = __uint_as_float(a);
  const uint32_t mag = m >= 1.0f ? ((((a >> 23) - 126u) << 3) | ((a >> 20) & 7u))
                                 : (uint32_t)(m * 8.0f);
  return ((u >> 26) & 0x20u) | mag;
}

// E4M3 byte of a value that E4M3 holds exactly (|p| <= 448).
__device__ __forceinline__ uint32_t e4m3_code(float p) {
  const uint32_t u = __float_as_uint(p), a = u & 0x7FFFFFFFu;
  const float m = __uint_as_float(a);
  const uint32_t mag = m >= 0x1p-6f ? ((((a >> 23) - 120u) << 3) | ((a >> 20) & 7u))
                                    : (uint32_t)(m * 512.0f);
  return ((u >> 24) & 0x80u) | mag;
}

// NE consecutive elements d0 .. d0 + NE - 1 of v = sum_h (w_h q_scale / 2) q_h
// for query qi (qi < 0: zeros), heads in ascending order, each element its
// own fma chain (so any split of the elements over lanes gives the same
// bits).  The head weights are formed exactly as the tiles form theirs; MX
// elements are decoded with their block's scale.
template <int FMT, int D, int NE>
__device__ __forceinline__ void lin_v(const uint8_t* __restrict__ q, const float* __restrict__ w,
                                      const void* __restrict__ q_scale, int H, int qi, int d0,
                                      float (&v)[NE]) {
  using F = Fmt<FMT>;
  constexpr int RBYTES = D * F::BITS / 8;
  static_assert(NE == 2 || NE == 4, "two or four elements per lane");
#pragma unroll
  for (int i = 0; i < NE; ++i) v[i] = 0.0f;
  if (qi < 0) return;
  float qs = 1.0f;
  if constexpr (FMT == kFP8) qs = static_cast<const float*>(q_scale)[qi];
#pragma unroll 4
  for (int h = 0; h < H; ++h) {
    const int64_t hr = (int64_t)qi * H + h;
    const float hw = w[hr] * qs * 0.5f;
    const uint8_t* row = q + hr * RBYTES;
    float e[NE];
    if constexpr (FMT == kMXFP4) {  // element 2i in the low nibble of byte i
      const uint32_t x = NE == 4 ? *reinterpret_cast<const uint16_t*>(row + d0 / 2) : row[d0 / 2];
#pragma unroll
      for (int i = 0; i < NE; ++i) e[i] = e2m1_top(x << (28 - 4 * i));
    } else {
      const uint32_t x = NE == 4 ? *reinterpret_cast<const uint32_t*>(row + d0)
                                 : *reinterpret_cast<const uint16_t*>(row + d0);
#pragma unroll
      for (int i = 0; i < NE; ++i) e[i] = e4m3_top(x << (24 - 8 * i));
    }
    if constexpr (F::MX) {
      const float sc = e8m0_value(static_cast<const uint8_t*>(q_scale)[hr * (D / 32) + d0 / 32]);
#pragma unroll
      for (int i = 0; i < NE; ++i) e[i] *= sc;
    }
#pragma unroll
    for (int i = 0; i < NE; ++i) v[i] = __builtin_fmaf(hw, e[i], v[i]);
  }
}

// Splits v into kLinPieces pieces of the linear row block's element format
// (E2M3 for MXFP4, else E4M3): NE elements per lane, one query per LANES
// consecutive lanes (32: a half wave, 64: the whole wave).  code[j] packs
// this lane's codes of piece j (element i in byte i); scale[j] is piece j's
// E8M0 scale byte, the same in all the query's lanes.  Piece j's scale 2^e
// puts the largest remaining magnitude m in the format's top binades below
// its largest value ([128, 256) for E4M3, [2, 4) for E2M3; e at least -127);
// each element is rounded to the format at that scale (ties to even: 4
// significant bits, or the subnormal step: 2^-9 for E4M3, 2^-3 for E2M3) and
// the exact rounding error is what piece j + 1 splits.
template <int FMT, int NE, int LANES>
__device__ __forceinline__ void lin_split(const float (&v)[NE], uint32_t (&code)[kLinPieces],
                                          int (&scale)[kLinPieces]) {
  constexpr bool FP6 = FMT == kMXFP4;
  constexpr int TOP = FP6 ? 1 : 7;      // floor(log2 m) - e
  constexpr int MIN_EX = FP6 ? 0 : -6;  // smallest normal binade
  float res[NE];
#pragma unroll
  for (int i = 0; i < NE; ++i) res[i] = v[i];
#pragma unroll
  for (int j = 0; j < kLinPieces; ++j) {
    float m = __builtin_fabsf(res[0]);
#pragma unroll
    for (int i = 1; i < NE; ++i) m = __builtin_fmaxf(m, __builtin_fabsf(res[i]));
#pragma unroll
    for (int off = 1; off < LANES; off <<= 1) m = __builtin_fmaxf(m, __shfl_xor(m, off));
    const int e = max((int)((__float_as_uint(m) >> 23) & 0xFFu) - 127 - TOP, -127);  // <= 126
    scale[j] = e + 127;
    const float down = __uint_as_float((uint32_t)(127 - e) << 23);               // 2^-e
    const float up = e >= -126 ? __uint_as_float((uint32_t)(127 + e) << 23) : 0x1p-127f;
    uint32_t c = 0;
#pragma unroll
    for (int i = 0; i < NE; ++i) {
      const float x = res[i] * down;  // |x| < 2^(TOP + 1)
      const int ex = max((int)((__float_as_uint(x) >> 23) & 0xFFu) - 127, MIN_EX);
      // x + 1.5 * 2^(ex + 20) has unit 2^(ex - 3): adding and removing it
      // rounds x to the format's step at x's binade
      const float magic = __uint_as_float(((uint32_t)(ex + 147) << 23) | 0x400000u);
      const float p = (x + magic) - magic;
      res[i] -= p * up;  // exact
      c |= (FP6 ? e2m3_code(p) : e4m3_code(p)) << (8 * i);
    }
    code[j] = c;
  }
}

// Publishes this lane's pieces (NE codes each, elements NE * l ..) in LDS
// region `reg` (kLinWords dwords, 16-byte aligned; piece j's element d is
// byte 128 j + d), l being the lane's index among its query's lanes.
template <int NE>
__device__ __forceinline__ void lin_store(uint32_t* reg, int l, const uint32_t (&code)[kLinPieces],
                                          const int (&scale)[kLinPieces]) {
#pragma unroll
  for (int j = 0; j < kLinPieces; ++j) {
    if constexpr (NE == 4) {
      reg[32 * j + l] = code[j];
    } else {
      reinterpret_cast<uint16_t*>(reg + 32 * j)[l] = (uint16_t)code[j];
    }
  }
  if (l < kLinPieces) {
    int s = scale[0];
#pragma unroll
    for (int j = 1; j < kLinPieces; ++j) s = l == j ? scale[j] : s;
    reg[32 * kLinPieces + l] = s;
  }
}

// The linear row block's A fragment of lane group g holding piece j of the
// query in `reg` (j >= kLinPieces: a zero row), in the order the format's
// k-step takes its elements, and its scale.  E4M3: elements d 32g .. 32g + 31
// for per-token FP8 (the key fragments' order), d 16g .. 16g + 15 and 64 + 16g
// .. 64 + 16g + 15 for MXFP8 (the instruction's K order).  E2M3 against E2M1
// keys: elements d 32g .. 32g + 31, element p in bits 6p .. 6p + 5 of the
// first six registers (the instruction's FP6 operand layout, measured on
// gfx950 with single-element operands).
template <int FMT>
__device__ __forceinline__ void lin_frag(const uint32_t* reg, int j, int g, i32x8& a, int& sa) {
  a = i32x8{0, 0, 0, 0, 0, 0, 0, 0};
  sa = 127;
  if (j < kLinPieces) {
    const uint32_t* p = reg + 32 * j;
    const int o0 = FMT == kMXFP8 ? 4 * g : 8 * g, o1 = FMT == kMXFP8 ? 16 + 4 * g : 8 * g + 4;
    const u32x4 lo = *reinterpret_cast<const u32x4*>(p + o0);
    const u32x4 hi = *reinterpret_cast<const u32x4*>(p + o1);
    if constexpr (FMT == kMXFP4) {
      const uint32_t w[8] = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
      uint32_t b[6] = {0, 0, 0, 0, 0, 0};
#pragma unroll
      for (int e = 0; e < 32; ++e) {
        const uint32_t c = (w[e >> 2] >> (8 * (e & 3))) & 0x3Fu;
        const int bit = 6 * e;
        b[bit >> 5] |= c << (bit & 31);
        if ((bit & 31) > 26) b[(bit >> 5) + 1] |= c >> (32 - (bit & 31));
      }
      a = i32x8{(int)b[0], (int)b[1], (int)b[2], (int)b[3], (int)b[4], (int)b[5], 0, 0};
    } else {
      a = i32x8{(int)lo[0], (int)lo[1], (int)lo[2], (int)lo[3], (int)hi[0], (int)hi[1], (int)hi[2], (int)hi[3]};
    }
    sa = (int)reg[32 * kLinPieces + j];
  }
}

// t + t(lane ^ 16) and t + t(lane ^ 32) in every lane, through the VALU.
// v_permlane16_swap exchanges rows 1 and 3 (16-lane rows) of its first
// operand with rows 0 and 2 of its second, v_permlane32_swap the upper half
// of the first with the lower half of the second; given two copies of t,
// the two results hold t of the lane's own row (half) and t of the partner
// row (half).  IEEE addition is commutative, so the sum is bit for bit the
// one t + __shfl_xor(t, 16 or 32) gives, without a shuffle's LDS round trip.
__device__ __forceinline__ float add_lane_xor16(float t) {
  const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(t), __float_as_uint(t), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}
__device__ __forceinline__ float add_lane_xor32(float t) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(t), __float_as_uint(t), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// Orders this wave's LDS writes before its later LDS reads.
__device__ __forceinline__ void wave_lds_sync() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

// ------------------------------------------------------------ key stages
// Key rows staged in LDS by direct-to-LDS loads (global_load_lds_dwordx4):
// one load moves 1 KB, lane j's 16 bytes landing at byte 16 j of the
// wave-uniform destination, so a stage holds whole key rows in order.

#define HK_LDS(x) ((__attribute__((address_space(3))) void*)(x))
// s_waitcnt that only bounds the vector-memory counter (gfx9 encoding:
// vmcnt[3:0] | expcnt[6:4] | lgkmcnt[11:8] | vmcnt[15:14]).
#define HK_WAIT_VM(n) __builtin_amdgcn_s_waitcnt(((n) & 0xF) | (((n) >> 4) << 14) | (7 << 4) | (0xF << 8))

// One direct-to-LDS load: each lane fetches 16 bytes at src into bytes
// 16 lane .. 16 lane + 15 from the wave-uniform LDS address dst.  (A
// non-template wrapper: templates that call the builtin directly have had
// their host-side kernel stubs dropped without a diagnostic.)
__device__ __forceinline__ void lds_dma16(const uint8_t* src, uint8_t* dst) {
  __builtin_amdgcn_global_load_lds(src, HK_LDS(dst), 16, 0, 0);
}
// The same with 4 bytes per lane (lane l's dword lands at byte 4 l).
__device__ __forceinline__ void lds_dma4(const uint8_t* src, uint8_t* dst) {
  __builtin_amdgcn_global_load_lds(src, HK_LDS(dst), 4, 0, 0);
}

// XOR swizzle of the 16-byte chunks of staged key row kk (NCH chunks per
// row), so that B-fragment reads (16 bytes per lane) are free of LDS bank
// conflicts.  The LDS counters on gfx950 fit this model of such a read, and
// only this one among the lane groupings tried: 64 four-byte banks, eight
// lanes at a time, the lanes that agree in bits 0, 3 and 5 of the lane index
// (keys kk = lane % 16 of one parity and one half, in two adjacent lane
// groups).  Those eight lanes must reach eight distinct 16-byte bank groups
// for every chunk pattern the formats read: chunk g (and 4 + g) of 8-chunk
// MX rows, 2g and 2g + 1 of per-token E4M3 rows, 4 ks + g of bf16 rows, g of
// E2M1 rows.  A bank simulation of this model gives zero conflicts for all
// of them with the swizzles below, and the counters read zero for the
// formats measured.  The chunk stored at slot c of row kk is chunk
// c ^ key_swz(kk) of the key's row.
template <int NCH>
__host__ __device__ __forceinline__ constexpr int key_swz(int kk) {
  static_assert(NCH == 4 || NCH == 8 || NCH == 16, "key rows of 4, 8 or 16 chunks");
  if constexpr (NCH == 16) return kk & 15;
  else if constexpr (NCH == 8) return (kk & 6) ^ ((kk >> 1) & 1);
  else return (kk >> 1) & (NCH - 1);
}

// LDS byte address of a pointer into a __shared__ array.
__device__ __forceinline__ uint32_t lds_addr(const uint8_t* p) {
  return (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) uint8_t*)p;
}

// Lane group g's B fragment, k-step ks, of staged key row kt (at `krow`,
// swizzled by key_swz): the chunks Fmt::frag names, at their stage slots,
// read with ordinary LDS loads (the compiler schedules each k-step's wait).
template <int FMT, int D>
__device__ __forceinline__ typename Fmt<FMT>::Frag stage_frag(const uint8_t* krow, int kt, int g,
                                                              int ks) {
  using F = Fmt<FMT>;
  constexpr int NCH = D * F::BITS / 8 / 16;
  constexpr int CPS = F::SLICE / 16;  // chunks per k-step slice
  const int sw = key_swz<NCH>(kt);
  if constexpr (F::FB == 32) {  // E4M3: two 16-byte chunks
    const int c0 = CPS * ks + F::chunk0(g), c1 = CPS * ks + F::chunk1(g);
    const u32x4 lo = *reinterpret_cast<const u32x4*>(krow + ((c0 ^ sw) * 16));
    const u32x4 hi = *reinterpret_cast<const u32x4*>(krow + ((c1 ^ sw) * 16));
    return i32x8{(int)lo[0], (int)lo[1], (int)lo[2], (int)lo[3],
                 (int)hi[0], (int)hi[1], (int)hi[2], (int)hi[3]};
  } else {  // bf16 or E2M1: one 16-byte chunk (frag reads chunk g of its slice)
    const int c = CPS * ks + g;
    return F::frag(krow + ((c ^ sw) * 16) - 16 * g, g);
  }
}


// Reads N 16-byte chunks from LDS in one asm block that also waits for
// them.  The compiler does not see these reads, so it does not make them
// wait for direct-to-LDS loads still in flight -- its own analysis cannot
// tell a ring's stages apart and made every read wait for all of them --
// and the kernel waits for a stage's loads explicitly before reading it.
// Outputs are early-clobber, and the asm waits for its loads before it
// ends.  (The score kernel reads with ordinary loads: there one asm block
// per column block measured slower, since each k-step's MFMAs could no
// longer start on their own fragment.)
template <int N>
__device__ __forceinline__ void lds_read_chunks(const uint32_t (&ad)[N], u32x4 (&r)[N]) {
  static_assert(N == 2 || N == 4, "two or four chunks");
  if constexpr (N == 4) {
    asm volatile(
        "ds_read_b128 %0, %4\n\t"
        "ds_read_b128 %1, %5\n\t"
        "ds_read_b128 %2, %6\n\t"
        "ds_read_b128 %3, %7\n\t"
        "s_waitcnt lgkmcnt(0)"
        : "=&v"(r[0]), "=&v"(r[1]), "=&v"(r[2]), "=&v"(r[3])
        : "v"(ad[0]), "v"(ad[1]), "v"(ad[2]), "v"(ad[3])
        : "memory");
  } else {
    asm volatile(
        "ds_read_b128 %0, %2\n\t"
        "ds_read_b128 %1, %3\n\t"
        "s_waitcnt lgkmcnt(0)"
        : "=&v"(r[0]), "=&v"(r[1])
        : "v"(ad[0]), "v"(ad[1])
        : "memory");
  }
}

// bf16 B fragments (every k-step) of staged key row kt (at `krow`, swizzled
// by key_swz), read with lds_read_chunks: chunk CPS ks + g of the row for
// k-step ks.
template <int D>
__device__ __forceinline__ void stage_frags_bf16(const uint8_t* krow, int kt, int g,
                                                 bf16x8 (&b)[D / Fmt<kBF16>::KMMA]) {
  using F = Fmt<kBF16>;
  constexpr int KS = D / F::KMMA;
  constexpr int NCH = D * F::BITS / 8 / 16;
  constexpr int CPS = F::SLICE / 16;  // chunks per k-step slice
  const int sw = key_swz<NCH>(kt);
  uint32_t ad[KS];
#pragma unroll
  for (int ks = 0; ks < KS; ++ks) ad[ks] = lds_addr(krow + (((CPS * ks + g) ^ sw) * 16));
  u32x4 ch[KS];
  lds_read_chunks<KS>(ad, ch);
#pragma unroll
  for (int ks = 0; ks < KS; ++ks) b[ks] = __builtin_bit_cast(bf16x8, ch[ks]);
}

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
  float wf[RB][4];  // head weights of this lane's 32 heads (times q_scale for FP8; halved
                    // for the scaled formats)
  i32x8 lin;        // scaled formats: the linear row block (pieces of v, rows 0..5: A, 8..13: B)
  int lsa;          // its E8M0 scale

  // Load the A operand and weights of query indices qa / qb (-1 = absent).
  // q_scale: fp32 [n] (FP8) or E8M0 bytes [n][H][D/32] (MX).  lds: this
  // wave's 2 * kLinWords dwords of LDS (16-byte aligned) for building the
  // linear row block of the scaled formats; unused for bf16.
  __device__ __forceinline__ void load(const uint8_t* __restrict__ q, const float* __restrict__ w,
                                       const void* __restrict__ q_scale, int H, int qa, int qb,
                                       uint32_t* lds) {
    const int lane = lane_id();
    if constexpr (F::SCALED) {
      static_assert(KS == 1, "the linear row block covers one k-step");
      float v[4];
      uint32_t code[kLinPieces];
      int scale[kLinPieces];
      lin_v<FMT, D, 4>(q, w, q_scale, H, (lane >> 5) ? qb : qa, 4 * (lane & 31), v);
      lin_split<FMT, 4, 32>(v, code, scale);
      lin_store<4>(lds + (lane >> 5) * kLinWords, lane & 31, code, scale);
      wave_lds_sync();
      const int r = lane & 15;
      lin_frag<FMT>(lds + (r >> 3) * kLinWords, r & 7, lane >> 4, lin, lsa);
    }
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
        wf[rb][i] = (qw >= 0 && h < H) ? w[(int64_t)qw * H + h] * qs * (F::SCALED ? 0.5f : 1.0f) : 0.0f;
      }
    }
  }

  // Scores of both queries against 16 keys whose B fragments are b[ks] (with
  // E8M0 scales sb[ks] for MX), in two steps: mma_phase fills the
  // accumulators, epilogue returns this lane's score: query (lane < 32 ?
  // A : B), key (lane % 16), before the per-key FP8 scale.  Between the two
  // the caller may reuse the B-fragment registers (the next block's reads).
  // half_sum is the epilogue without the partner add, for callers that
  // exchange the halves later.
  //
  // Canonical head-sum order (every kernel that produces a score follows it):
  // per lane, one partial over the even row blocks and one over the odd row
  // blocks (row block ascending, register ascending), t = even + odd, then
  // t + t(lane ^ 16).  For the scaled formats the even partial starts from
  // the lane's share of the linear term, (l0 + l1) + (l2 + l3) over its four
  // rows of the linear row block (pieces 0..3 in lane group 0, pieces 4, 5 in
  // lane group 1), and the heads contribute (w/2) * |acc|.  A tile holding
  // one query per MFMA (16 heads per row block) sees the same four partials
  // in its four lane groups.
  //
  // The MFMAs run as one phase at raised wave priority, the epilogue after
  // it at normal priority: of the two waves sharing a SIMD, the one in its
  // MFMA phase then wins every issue conflict with the other's epilogue, so
  // the matrix pipe is refilled as soon as it frees (measured on gfx950:
  // 2.5-5% less score time across the formats; the same order without the
  // priority change gains nothing).
  struct Acc {
    f32x4 h[RB];
    f32x4 l;
  };
  __device__ __forceinline__ void mma_phase(const Frag (&b)[KS], const int (&sb)[KS], Acc& c) const {
    c.l = f32x4{0.f, 0.f, 0.f, 0.f};
    __builtin_amdgcn_s_setprio(1);
    if constexpr (F::SCALED) c.l = F::mma_lin(lin, b[0], c.l, lsa, sb[0]);
#pragma unroll
    for (int rb = 0; rb < RB; ++rb) {
      c.h[rb] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) c.h[rb] = F::mma(a[rb][ks], b[ks], c.h[rb], sa[rb][ks], sb[ks]);
    }
    __builtin_amdgcn_s_setprio(0);
  }
  // This lane's half of the score (its 32 heads), before the partner add.
  __device__ __forceinline__ float half_sum(const Acc& c) const {
    float se = 0.0f, so = 0.0f;
    if constexpr (F::SCALED) se = (c.l[0] + c.l[1]) + (c.l[2] + c.l[3]);
#pragma unroll
    for (int rb = 0; rb < RB; ++rb) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float r = F::SCALED ? __builtin_fabsf(c.h[rb][i]) : __builtin_fmaxf(c.h[rb][i], 0.0f);
        if (rb & 1) {
          so = __builtin_fmaf(r, wf[rb][i], so);
        } else {
          se = __builtin_fmaf(r, wf[rb][i], se);
        }
      }
    }
    return se + so;
  }
  __device__ __forceinline__ float epilogue(const Acc& c) const {
    const float t = half_sum(c);
    return t + __shfl_xor(t, 16);
  }
};

}  // namespace hk
