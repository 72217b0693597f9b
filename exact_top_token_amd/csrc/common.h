// Internal device helpers shared by the selection kernels (gfx950, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

namespace hk {

constexpr int kWave = 64;

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef int i32x8 __attribute__((ext_vector_type(8)));
typedef unsigned u32x4 __attribute__((ext_vector_type(4)));

// Storage formats of q and k (the values of hytopk_dtype).
constexpr int kBF16 = 0;   // bf16
constexpr int kFP8 = 1;    // OCP FP8 E4M3 with fp32 per-token scales
constexpr int kMXFP8 = 2;  // OCP MX: E4M3 elements, one E8M0 scale per 32
constexpr int kMXFP4 = 3;  // OCP MX: E2M1 elements (two per byte), E8M0 per 32

// Per-format constants of the 16x16 MFMA tiles.  bf16 uses
// v_mfma_f32_16x16x32_bf16 (K = 32, 8 elements = 16 bytes per lane per
// k-step); the other formats use v_mfma_scale_f32_16x16x128_f8f6f4 (K = 128,
// 32 elements per lane per k-step: 32 bytes of E4M3 or 16 bytes of E2M1, the
// latter in the low four registers of the operand).  The scaled MFMA takes
// one E8M0 scale per lane for A and one for B: the scale of the lane's row
// (A) or column (B) over its 32 elements -- exactly one MX block.
template <int FMT>
struct Fmt {
  static constexpr bool SCALED = FMT != kBF16;                 // f8f6f4 MFMA
  static constexpr bool MX = FMT == kMXFP8 || FMT == kMXFP4;   // block scales
  static constexpr int BITS = FMT == kBF16 ? 16 : (FMT == kMXFP4 ? 4 : 8);
  static constexpr int KMMA = FMT == kBF16 ? 32 : 128;         // K per MFMA
  static constexpr int FB = FMT == kBF16 ? 16 : (FMT == kMXFP4 ? 16 : 32);
  static constexpr int CODE = FMT == kMXFP4 ? 4 : 0;           // f8f6f4 operand format
  using Frag = typename std::conditional<FMT == kBF16, bf16x8, i32x8>::type;

  // D += A x B with per-lane E8M0 scales sa, sb (127 = 2^0; ignored for bf16).
  __device__ __forceinline__ static f32x4 mma(const Frag& a, const Frag& b, const f32x4& c, int sa,
                                              int sb) {
    if constexpr (FMT == kBF16) {
      return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
    } else {
      return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, c, CODE, CODE, 0, sa, 0, sb);
    }
  }

  // D += A x B where A is the linear row block (E2M3 against E2M1 keys, else
  // E4M3) and B this format.
  static constexpr int LIN_CODE = FMT == kMXFP4 ? 2 : 0;  // f8f6f4 code of E2M3 / E4M3
  __device__ __forceinline__ static f32x4 mma_lin(const i32x8& a, const Frag& b, const f32x4& c,
                                                  int sa, int sb) {
    static_assert(SCALED, "bf16 has no linear row block");
    return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, c, LIN_CODE, CODE, 0, sa, 0, sb);
  }

  // Bytes of one k-step slice of a row (KMMA elements).
  static constexpr int SLICE = KMMA * BITS / 8;

  // 16-byte chunks of a k-step slice that lane group g holds, in operand
  // order (chunk c = bytes [16c, 16c + 16) of the slice).  bf16 and E2M1
  // hold one chunk, g.  Per-token E4M3 holds the contiguous chunks 2g and
  // 2g + 1 (any layout shared by A and B gives the same sums).  Under MX
  // block scales E4M3 must follow the instruction's K order: the operand's
  // first 16 bytes are K = 16g .. 16g + 15 and its last 16 bytes K = 64 + 16g
  // .. 64 + 16g + 15, and lane group b's scale applies to K = 32b .. 32b + 31,
  // so lane group g holds chunks g and 4 + g (measured on gfx950 with
  // single-element operands).
  __device__ __forceinline__ static int chunk0(int g) {
    return FMT == kFP8 ? 2 * g : g;
  }
  __device__ __forceinline__ static int chunk1(int g) {
    return FMT == kFP8 ? 2 * g + 1 : 4 + g;
  }

  // Lane group g's fragment of the k-step slice starting at `slice`
  // (E2M1 fragments fill the low four registers).
  __device__ __forceinline__ static Frag frag(const uint8_t* slice, int g) {
    if constexpr (FMT == kBF16) {
      return *reinterpret_cast<const Frag*>(slice + 16 * g);
    } else if constexpr (FMT == kMXFP4) {
      const u32x4 v = *reinterpret_cast<const u32x4*>(slice + 16 * g);
      return i32x8{(int)v[0], (int)v[1], (int)v[2], (int)v[3], 0, 0, 0, 0};
    } else {
      const u32x4 lo = *reinterpret_cast<const u32x4*>(slice + 16 * chunk0(g));
      const u32x4 hi = *reinterpret_cast<const u32x4*>(slice + 16 * chunk1(g));
      return i32x8{(int)lo[0], (int)lo[1], (int)lo[2], (int)lo[3],
                   (int)hi[0], (int)hi[1], (int)hi[2], (int)hi[3]};
    }
  }
};

// Order-preserving 32-bit key of an fp32 score: larger score <=> larger key.
// -0.0 is folded onto +0.0 so that equal scores always have equal keys.
__device__ __forceinline__ uint32_t score_key(float f) {
  uint32_t u = __float_as_uint(f);
  if (u == 0x80000000u) u = 0u;
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

__device__ __forceinline__ float key_score(uint32_t k) {
  uint32_t u = (k & 0x80000000u) ? (k & 0x7fffffffu) : ~k;
  return __uint_as_float(u);
}

__device__ __forceinline__ int lane_id() { return __lane_id(); }

// Keys of query q's context: lo..hi inclusive (empty when lo > hi).  The
// explicit per-query position / first key when given (packed sequences,
// arbitrary query positions), else position q_start + q and first key 0;
// clamped to the key buffer [0, L).
struct QRange {
  int lo, hi;
};

__device__ __forceinline__ QRange query_range(const int* qpos, const int* qfirst, int q_start,
                                              int L, int q) {
  int hi = qpos ? qpos[q] : q_start + q;
  int lo = qfirst ? qfirst[q] : 0;
  return QRange{max(lo, 0), min(hi, L - 1)};
}

// Inclusive suffix sum across the 64 lanes of a wave: lane i gets sum_{j>=i} x_j.
__device__ __forceinline__ int wave_suffix_sum(int x) {
  const int lane = lane_id();
#pragma unroll
  for (int off = 1; off < kWave; off <<= 1) {
    int v = __shfl_down(x, off);
    if (lane + off < kWave) x += v;
  }
  return x;
}

// Exclusive prefix sum across the 64 lanes of a wave.
__device__ __forceinline__ int wave_prefix_excl(int x) {
  const int lane = lane_id();
  int incl = x;
#pragma unroll
  for (int off = 1; off < kWave; off <<= 1) {
    int v = __shfl_up(incl, off);
    if (lane >= off) incl += v;
  }
  return incl - x;
}

// Shared scratch of the block radix select: 256 histogram bins, 4 wave
// totals, and the chosen digit / remaining rank / multiplicity.
struct RadixScratch {
  int hist[256];
  int wtot[4];
  uint32_t digit;
  int rank;
  int mult;
};

// Block-wide radix select: the r-th largest (1-based, duplicates counted)
// value of key(i) over the i in [0, m) with take(i).  Keys must lie below
// 2^bits (bits <= 32); MSB-first passes of 8-bit digits cover only those bits.
// Requires blockDim.x >= 256 and a multiple of 64; all threads must call it.
// On return `rem` is the rank of the result among the entries equal to it
// (1 <= rem <= mult), and `mult` how many taken entries equal it.
template <typename KeyF, typename TakeF>
__device__ uint32_t block_select_largest(int m, int r, KeyF key, TakeF take, RadixScratch& sc,
                                          int& rem, int& mult, int bits = 32) {
  const int tid = threadIdx.x, nt = blockDim.x;
  uint32_t prefix = 0u, pmask = 0u;
  const int npass = bits <= 0 ? 1 : (bits + 7) / 8;
  for (int pass = npass - 1; pass >= 0; --pass) {
    const int shift = 8 * pass;
    for (int b = tid; b < 256; b += nt) sc.hist[b] = 0;
    __syncthreads();
    // Each thread counts runs of equal digits among its entries and adds a
    // run with one atomic: in the passes where most entries share a digit
    // this avoids serialising every lane on one LDS address.
    uint32_t run_d = 0u;
    int run_n = 0;
    for (int i = tid; i < m; i += nt) {
      if (!take(i)) continue;
      const uint32_t kk = key(i);
      if ((kk & pmask) != prefix) continue;
      const uint32_t d = (kk >> shift) & 255u;
      if (run_n > 0 && d != run_d) {
        atomicAdd(&sc.hist[run_d], run_n);
        run_n = 0;
      }
      run_d = d;
      ++run_n;
    }
    if (run_n > 0) atomicAdd(&sc.hist[run_d], run_n);
    __syncthreads();
    int h = 0, suf = 0;
    if (tid < 256) {
      h = sc.hist[tid];
      suf = wave_suffix_sum(h);
      if (lane_id() == 0) sc.wtot[tid >> 6] = suf;
    }
    __syncthreads();
    if (tid < 256) {
      for (int v = (tid >> 6) + 1; v < 4; ++v) suf += sc.wtot[v];
      // suf = entries (matching the prefix) whose digit is >= tid
      if (suf >= r && suf - h < r) {
        sc.digit = (uint32_t)tid;
        sc.rank = r - (suf - h);
        sc.mult = h;
      }
    }
    __syncthreads();
    prefix |= sc.digit << shift;
    pmask |= 255u << shift;
    r = sc.rank;
    __syncthreads();
  }
  rem = r;
  mult = sc.mult;
  return prefix;
}

// Number of bits needed for values in [0, x].
__device__ __forceinline__ int bit_width(uint32_t x) { return x ? 32 - __clz(x) : 0; }

// Block-wide min and max of one value per thread (all threads must call).
__device__ __forceinline__ void block_minmax(uint32_t lo, uint32_t hi, uint32_t* red,
                                             uint32_t& gmin, uint32_t& gmax) {
  const int tid = threadIdx.x, nw = blockDim.x / kWave;
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) {
    lo = min(lo, (uint32_t)__shfl_xor((int)lo, off));
    hi = max(hi, (uint32_t)__shfl_xor((int)hi, off));
  }
  if (lane_id() == 0) { red[tid >> 6] = lo; red[nw + (tid >> 6)] = hi; }
  __syncthreads();
  gmin = red[0];
  gmax = red[nw];
  for (int w = 1; w < nw; ++w) { gmin = min(gmin, red[w]); gmax = max(gmax, red[nw + w]); }
  __syncthreads();
}

}  // namespace hk
