// Internal device helpers shared by the selection kernels (gfx950, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace hk {

constexpr int kWave = 64;

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef int i32x8 __attribute__((ext_vector_type(8)));
typedef unsigned u32x4 __attribute__((ext_vector_type(4)));

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
    for (int i = tid; i < m; i += nt) {
      if (!take(i)) continue;
      const uint32_t kk = key(i);
      if ((kk & pmask) == prefix) atomicAdd(&sc.hist[(kk >> shift) & 255u], 1);
    }
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
