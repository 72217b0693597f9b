// Indexer backward at the replayed entries ("HyScale sparse-attention
// training -- Selection without a score table", key-observation paragraph:
// the indexer's loss depends on the scores of the selected entries alone, and the
// top-k choice carries no gradient).  Given dI[t, j], the upstream gradient
// of the replayed score I(t, idx[t, j]), with c[h, j] = q[t, h] . k[idx[t, j]]
// and ReLU'(c) = [c > 0]:
//   dw[t, h]    = sum_j dI[t, j] * max(c[h, j], 0)
//   dq[t, h, :] = w[t, h] * sum_j dI[t, j] [c[h, j] > 0] k[idx[t, j], :]
//   u[t, j, :]  = sum_h dI[t, j] w[t, h] [c[h, j] > 0] q[t, h, :]
//   dk[s, :]    = sum over the entries (t, j) with idx[t, j] = s of u[t, j, :]
//
// bwd_query_kernel: one workgroup (4 waves) per query, the query's keys in
// tiles of 32.  Wave w owns heads 16w .. 16w + 15.  It forms c with the query
// as the A operand (lane: 4 heads x 1 key) and c^T with the same registers
// swapped (lane: 1 head x 4 keys), so each layout feeds the next MFMA without
// a transpose:
//   * c^T's layout is dq's A operand (head rows, keys along K); dq's B
//     operand reads the tile transposed in LDS (dims x keys);
//   * c's layout gives G = dI w [c > 0] per (key, 4 heads), stored to LDS as
//     key rows; every wave then forms u for its quarter of the dims with
//     Q^T (dims x heads, held in registers) as the A operand.
// The MFMA operands in the gradient products are bf16, so each fp32 factor
// is split into a round-to-nearest bf16 high part and the bf16 of the
// remainder (hi + lo carries 16 significant bits); both parts are
// multiplied against exact bf16 key / query values and accumulated in fp32.
//
// dk: the u rows of a chunk of queries go to a buffer (query-major); a stable
// LSD radix sort of (key position, row) pairs groups them by key with entries
// in query-then-slot order; waves sum each key's rows in that order and add
// the sum to dk.  Chunks run in order, so dk is bitwise reproducible.
//
// Scaled formats: the gradients are taken with respect to the decoded values.
// A first pass writes q and k as bf16 (bwd_dequant_kernel): MX elements times
// their block's E8M0 scale, exact in bf16; per-token FP8 codes without their
// scales (also exact).  The per-token scales qs[t], ks[s] then enter as
// factors, since c = qs ks c8 with c8 the product of the codes (same sign):
//   dw[t, h]    = qs[t] * sum_j (dI ks[s_j]) max(c8, 0)
//   dq[t, h, :] = w * sum_j (dI ks[s_j]) [c8 > 0] k8[s_j, :]
//   u[t, j, :]  = sum_h dI (w qs[t]) [c8 > 0] q8[t, h, :]
#include <algorithm>
#include <type_traits>

#include "common.h"
#include "launch.h"
#include "tile.h"

namespace hk {

constexpr int kBwdThreads = 256;
constexpr int kBwdTK = 32;     // keys per tile
constexpr int kBwdDepth = 2;   // tiles of key rows in flight (registers)
constexpr int kKtW = kBwdTK + 4;  // transposed tile row (bf16), padded

// Transposed tile: row i (a dim) holds the 32 keys in 8 groups of 4; group
// kg sits at slot kg ^ kt_swz(i).  With 36-element rows this makes both the
// staging writes (32 dim quads x 2 key groups per wave) and the dq operand
// reads (16 dims x 2 groups per lane group) free of LDS bank conflicts.
__device__ __forceinline__ int kt_swz(int i) { return ((i >> 4) ^ (i >> 5)) & 7; }
constexpr int kGtW = 64 + 8;      // G row (bf16): 64 heads, padded

__device__ __forceinline__ void split_bf16(float x, uint32_t& hi, uint32_t& lo) {
  const __bf16 h = (__bf16)x;
  const __bf16 l = (__bf16)(x - (float)h);
  hi = __builtin_bit_cast(uint16_t, h);
  lo = __builtin_bit_cast(uint16_t, l);
}

__device__ __forceinline__ bf16x8 pack8(const uint32_t (&v)[8]) {
  u32x4 p;
  p[0] = v[0] | (v[1] << 16);
  p[1] = v[2] | (v[3] << 16);
  p[2] = v[4] | (v[5] << 16);
  p[3] = v[6] | (v[7] << 16);
  return __builtin_bit_cast(bf16x8, p);
}

__device__ __forceinline__ f32x4 mfma_bf16(const bf16x8& a, const bf16x8& b, const f32x4& c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

// TOK: per-token FP8 scales a.q_scale / a.k_scale applied as factors.
template <int D, bool WITH_U, bool TOK>
__global__ void __launch_bounds__(kBwdThreads) __attribute__((amdgpu_waves_per_eu(3)))
bwd_query_kernel(BwdArgs a) {
  constexpr int NCH = D / 8;   // 16-byte chunks per key row
  constexpr int KS = D / 32;   // k-steps of the c products
  constexpr int NDB = D / 16;  // dim blocks of dq
  constexpr int UDB = D / 64;  // dim blocks of u per wave (a wave owns D / 4 dims)

  // krow and gt are single buffers: every read of krow (the c products) and
  // of gt (the u products) of tile t comes before a barrier that all waves
  // pass before tile t + 1 writes them.  kt is read after tile t's second
  // barrier, so it alternates.  (LDS of three workgroups fits one CU.)
  __shared__ __attribute__((aligned(16))) uint16_t krow[kBwdTK * D];
  __shared__ __attribute__((aligned(16))) uint16_t kt[2][D * kKtW];
  __shared__ __attribute__((aligned(16))) uint16_t gt[2][kBwdTK * kGtW];
  extern __shared__ int dyn[];

  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63, g = lane >> 4, c16 = lane & 15;
  const int qi = a.q0 + blockIdx.x;  // query index in [0, n)
  const int K = a.topk, H = a.H;
  const int ntile = (K + kBwdTK - 1) / kBwdTK;
  // tiles processed: an even count (two LDS buffers, two register slots),
  // plus kBwdDepth tiles of padding that the prefetch reads past the end
  const int ntile2 = (ntile + 1) & ~1;
  const int nslot = (ntile2 + kBwdDepth) * kBwdTK;
  int* ids = dyn;                                   // [nslot] key or -1
  float* dI = reinterpret_cast<float*>(dyn + nslot);  // [nslot] (u's factor)
  // dw's and dq's factor dI * ks[key] (TOK), else dI itself
  float* dIk = TOK ? reinterpret_cast<float*>(dyn + 2 * nslot) : dI;

  for (int j = tid; j < nslot; j += kBwdThreads) {
    int key = j < K ? a.idx[(int64_t)qi * K + j] : -1;
    if (key < 0 || key >= a.L) key = -1;  // padding, never dereferenced
    ids[j] = key;
    dI[j] = key >= 0 ? a.dsc[(int64_t)qi * K + j] : 0.0f;
    if constexpr (TOK) dIk[j] = key >= 0 ? dI[j] * a.k_scale[key] : 0.0f;
  }
  const float qs = TOK ? a.q_scale[qi] : 1.0f;

  // Query fragments of this wave's heads: A operand of c, B operand of c^T.
  bf16x8 qa[KS];
  {
    const int h = 16 * wave + c16;
    const uint16_t* src = a.q + ((int64_t)qi * H + (h < H ? h : 0)) * D;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks)
      qa[ks] = h < H ? *reinterpret_cast<const bf16x8*>(src + (4 * ks + g) * 8) : bf16x8{};
  }
  // Q^T fragments for u: dim rows wave * D/4 + 16 udb + c16, heads 8g + 32hs + e.
  bf16x8 qt[UDB][2];
#pragma unroll
  for (int udb = 0; udb < UDB; ++udb) {
    const int i = wave * (D / 4) + 16 * udb + c16;
#pragma unroll
    for (int hs = 0; hs < 2; ++hs) {
      uint32_t v[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const int h = 8 * g + 32 * hs + e;
        v[e] = h < H ? a.q[((int64_t)qi * H + h) * D + i] : 0u;
      }
      qt[udb][hs] = pack8(v);
    }
  }
  float wv[4], wu[4];  // dq's head weights; u's (times qs for TOK)
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    const int h = 16 * wave + 4 * g + r;
    wv[r] = h < H ? a.w[(int64_t)qi * H + h] : 0.0f;
    wu[r] = TOK ? wv[r] * qs : wv[r];
  }
  f32x4 dqa[NDB];
#pragma unroll
  for (int db = 0; db < NDB; ++db) dqa[db] = f32x4{0.f, 0.f, 0.f, 0.f};
  float dwa[4] = {0.f, 0.f, 0.f, 0.f};
  __syncthreads();  // ids / dI staged

  // Staging: thread t < NBLK moves a 4 keys x 4 dims block of the tile:
  // keys 4 kg .. 4 kg + 3, dims 4 q4 .. 4 q4 + 3 (8-byte global loads; a row's
  // 256 bytes come from 32 consecutive lanes).
  constexpr int NQ4 = D / 4;
  constexpr int NBLK = (kBwdTK / 4) * NQ4;
  static_assert(NBLK <= kBwdThreads, "one block per thread");
  const bool stager = NBLK == kBwdThreads || tid < NBLK;
  const int kg = tid / NQ4, q4 = tid % NQ4;
  uint2 pf[kBwdDepth][4];
  auto gather = [&](int tile, int slot) {
    if (!stager) return;
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      // unconditional load (padding reads row 0 and is zeroed when staged):
      // no branch around the load and no use of it before the stage keeps
      // the wait counts of the pipeline exact
      const int key = ids[tile * kBwdTK + 4 * kg + v];
      pf[slot][v] = *reinterpret_cast<const uint2*>(a.k + (int64_t)(key >= 0 ? key : 0) * D + 4 * q4);
    }
  };
  auto stage = [&](int tile, int slot, int buf) {
    if (!stager) return;
    uint2 x[4];
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      const int j = 4 * kg + v;
      x[v] = pf[slot][v];
      if (ids[tile * kBwdTK + j] < 0) x[v] = uint2{0u, 0u};
      *reinterpret_cast<uint2*>(&krow[j * D + (((q4 >> 1) ^ (j & (NCH - 1))) * 8) + 4 * (q4 & 1)]) = x[v];
    }
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int i = 4 * q4 + e;
      const int sh = 16 * (e & 1);
      uint32_t b[4];
#pragma unroll
      for (int v = 0; v < 4; ++v) b[v] = ((e < 2 ? x[v].x : x[v].y) >> sh) & 0xFFFFu;
      *reinterpret_cast<uint2*>(&kt[buf][i * kKtW + ((kg ^ kt_swz(i)) * 4)]) =
          uint2{b[0] | (b[1] << 16), b[2] | (b[3] << 16)};
    }
  };

#pragma unroll
  for (int s = 0; s < kBwdDepth; ++s) gather(s, s);

  static_assert(kBwdDepth == 2, "slot and LDS buffer share the tile parity");
  auto tile_body = [&](const int t, auto slotc) {
    constexpr int slot = decltype(slotc)::value, buf = slot;
    stage(t, slot, buf);
    gather(t + kBwdDepth, slot);
    __syncthreads();  // key tile t in krow / kt

    f32x4 c[2], ct[2];
#pragma unroll
    for (int blk = 0; blk < 2; ++blk) {
      c[blk] = f32x4{0.f, 0.f, 0.f, 0.f};
      ct[blk] = f32x4{0.f, 0.f, 0.f, 0.f};
      const int j = 16 * blk + c16;
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        const bf16x8 kb = *reinterpret_cast<const bf16x8*>(
            &krow[j * D + (((4 * ks + g) ^ (j & (NCH - 1))) * 8)]);
        c[blk] = mfma_bf16(qa[ks], kb, c[blk]);   // lane: heads 4g + r, key j
        ct[blk] = mfma_bf16(kb, qa[ks], ct[blk]);  // lane: keys 16 blk + 4g + r, head c16
      }
    }
    // dw partials and G = dI w [c > 0] (key rows, for u)
#pragma unroll
    for (int blk = 0; blk < 2; ++blk) {
      const int j = 16 * blk + c16;
      const float di = dI[t * kBwdTK + j], dik = dIk[t * kBwdTK + j];
      uint32_t hi[4], lo[4];
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const float cv = c[blk][r];
        dwa[r] = __builtin_fmaf(dik, __builtin_fmaxf(cv, 0.0f), dwa[r]);
        split_bf16(cv > 0.0f ? di * wu[r] : 0.0f, hi[r], lo[r]);
      }
      uint2* dh = reinterpret_cast<uint2*>(&gt[0][j * kGtW + 16 * wave + 4 * g]);
      uint2* dl = reinterpret_cast<uint2*>(&gt[1][j * kGtW + 16 * wave + 4 * g]);
      *dh = uint2{hi[0] | (hi[1] << 16), hi[2] | (hi[3] << 16)};
      *dl = uint2{lo[0] | (lo[1] << 16), lo[2] | (lo[3] << 16)};
    }
    // G' = dI [c > 0] in c^T's layout: dq's A operand (K slot 4 blk + r of
    // lane group g is key 16 blk + 4g + r)
    bf16x8 gqh, gql;
    {
      uint32_t vh[8], vl[8];
#pragma unroll
      for (int blk = 0; blk < 2; ++blk) {
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          uint32_t h, l;
          split_bf16(dIk[t * kBwdTK + 16 * blk + 4 * g + r], h, l);
          const bool on = ct[blk][r] > 0.0f;
          vh[4 * blk + r] = on ? h : 0u;
          vl[4 * blk + r] = on ? l : 0u;
        }
      }
      gqh = pack8(vh);
      gql = pack8(vl);
    }
    __syncthreads();  // G rows of all heads in gt

    // dq[h, i] += sum_j G'[h, j] k[j, i]; B operand: dims x keys from kt
#pragma unroll
    for (int db = 0; db < NDB; ++db) {
      const int i = 16 * db + c16;
      const uint16_t* row = &kt[buf][i * kKtW];
      const uint2 p0 = *reinterpret_cast<const uint2*>(row + ((g ^ kt_swz(i)) * 4));
      const uint2 p1 = *reinterpret_cast<const uint2*>(row + (((4 + g) ^ kt_swz(i)) * 4));
      const bf16x8 kb = __builtin_bit_cast(bf16x8, u32x4{p0.x, p0.y, p1.x, p1.y});
      dqa[db] = mfma_bf16(gqh, kb, dqa[db]);
      dqa[db] = mfma_bf16(gql, kb, dqa[db]);
    }
    // u^T[i, j] = sum_h Q^T[i, h] G[h, j] for this wave's dims
    if constexpr (WITH_U) {
#pragma unroll
      for (int blk = 0; blk < 2; ++blk) {
        const int j = 16 * blk + c16;
        bf16x8 gh[2], gl[2];
#pragma unroll
        for (int hs = 0; hs < 2; ++hs) {
          gh[hs] = *reinterpret_cast<const bf16x8*>(&gt[0][j * kGtW + 8 * g + 32 * hs]);
          gl[hs] = *reinterpret_cast<const bf16x8*>(&gt[1][j * kGtW + 8 * g + 32 * hs]);
        }
        const int jg = t * kBwdTK + j;
#pragma unroll
        for (int udb = 0; udb < UDB; ++udb) {
          f32x4 acc = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
          for (int hs = 0; hs < 2; ++hs) {
            acc = mfma_bf16(qt[udb][hs], gh[hs], acc);
            acc = mfma_bf16(qt[udb][hs], gl[hs], acc);
          }
          // lane: dims wave * D/4 + 16 udb + 4g + r of key slot jg; every
          // slot of the padded tiles has a row (padding rows are never read)
          *reinterpret_cast<f32x4*>(a.u + ((int64_t)blockIdx.x * ntile2 * kBwdTK + jg) * D +
                                    wave * (D / 4) + 16 * udb + 4 * g) = acc;
        }
      }
    }
  };
  for (int t0 = 0; t0 < ntile2; t0 += kBwdDepth) {
    tile_body(t0, std::integral_constant<int, 0>{});
    tile_body(t0 + 1, std::integral_constant<int, 1>{});
  }

  if (a.dq) {
#pragma unroll
    for (int db = 0; db < NDB; ++db) {
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int h = 16 * wave + 4 * g + r;
        if (h < H) a.dq[((int64_t)qi * H + h) * D + 16 * db + c16] = wv[r] * dqa[db][r];
      }
    }
  }
  if (a.dw) {
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      float v = dwa[r];
      v += __shfl_xor(v, 1);
      v += __shfl_xor(v, 2);
      v += __shfl_xor(v, 4);
      v += __shfl_xor(v, 8);
      const int h = 16 * wave + 4 * g + r;
      if constexpr (TOK) v *= qs;
      if (c16 == 0 && h < H) a.dw[(int64_t)qi * H + h] = v;
    }
  }
}

template <int D, bool WITH_U, bool TOK>
static hipError_t bwd_query_d(const BwdArgs& a, hipStream_t s) {
  const int ntile = (a.topk + kBwdTK - 1) / kBwdTK;
  const size_t dyn = (size_t)(((ntile + 1) & ~1) + kBwdDepth) * kBwdTK * (TOK ? 12 : 8);
  static LdsLimit lim;
  hipError_t e = raise_dynamic_lds((const void*)bwd_query_kernel<D, WITH_U, TOK>, (int)dyn, lim);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL((bwd_query_kernel<D, WITH_U, TOK>), dim3((unsigned)a.nq), dim3(kBwdThreads),
                     dyn, s, a);
  return hipGetLastError();
}

hipError_t launch_bwd_query(const BwdArgs& a, int d, hipStream_t s) {
  if (a.nq <= 0) return hipSuccess;
  const bool u = a.u != nullptr;
  if (d == 64) return u ? bwd_query_d<64, true, false>(a, s) : bwd_query_d<64, false, false>(a, s);
  if (d != 128) return hipErrorInvalidValue;
  if (a.q_scale && a.k_scale)
    return u ? bwd_query_d<128, true, true>(a, s) : bwd_query_d<128, false, true>(a, s);
  return u ? bwd_query_d<128, true, false>(a, s) : bwd_query_d<128, false, false>(a, s);
}

// q or k of a scaled format as bf16 bits, 8 elements per thread and step:
// MX elements times their block's E8M0 scale, per-token FP8 codes as they
// are (their scales are applied by the query kernel).  Both are exact in
// bf16 (an MX product unless it falls below bf16's normal range, where it is
// rounded to nearest).  x: rows of d elements (E2M1: d / 2 bytes); scale:
// E8M0 bytes [rows][d / 32] (MX only).
template <int FMT>
__global__ void bwd_dequant_kernel(const uint8_t* __restrict__ x, const uint8_t* __restrict__ scale,
                                   int64_t rows, int d, uint16_t* __restrict__ out) {
  const int64_t n8 = rows * d / 8;
  for (int64_t i = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; i < n8;
       i += (int64_t)gridDim.x * blockDim.x) {
    const int64_t e0 = 8 * i;  // first element; 8 elements never straddle a row or a block
    float v[8];
    if constexpr (FMT == kMXFP4) {
      const uint32_t w = *reinterpret_cast<const uint32_t*>(x + e0 / 2);
#pragma unroll
      for (int j = 0; j < 8; ++j) v[j] = e2m1_top(w << (28 - 4 * j));
    } else {
      const uint2 w = *reinterpret_cast<const uint2*>(x + e0);
#pragma unroll
      for (int j = 0; j < 8; ++j) v[j] = e4m3_top((j < 4 ? w.x : w.y) << (24 - 8 * (j & 3)));
    }
    if constexpr (FMT == kMXFP8 || FMT == kMXFP4) {
      const int64_t row = e0 / d;
      const float sc = e8m0_value(scale[row * (d / 32) + (e0 % d) / 32]);
#pragma unroll
      for (int j = 0; j < 8; ++j) v[j] *= sc;
    }
    uint32_t b[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const uint32_t u = __float_as_uint(v[j]);
      b[j] = (u + 0x7FFFu + ((u >> 16) & 1u)) >> 16;  // nearest, ties to even
    }
    *reinterpret_cast<u32x4*>(out + e0) =
        u32x4{b[0] | (b[1] << 16), b[2] | (b[3] << 16), b[4] | (b[5] << 16), b[6] | (b[7] << 16)};
  }
}

hipError_t launch_bwd_dequant(const void* x, const void* scale, int64_t rows, int d, int fmt,
                              uint16_t* out, hipStream_t s) {
  const int64_t n8 = rows * d / 8;
  if (n8 <= 0) return hipSuccess;
  const int nb = (int)std::min<int64_t>((n8 + 255) / 256, 16384);
  const auto* xb = static_cast<const uint8_t*>(x);
  const auto* sb = static_cast<const uint8_t*>(scale);
  if (fmt == kFP8) {
    hipLaunchKernelGGL(bwd_dequant_kernel<kFP8>, dim3(nb), dim3(256), 0, s, xb, sb, rows, d, out);
  } else if (fmt == kMXFP8) {
    hipLaunchKernelGGL(bwd_dequant_kernel<kMXFP8>, dim3(nb), dim3(256), 0, s, xb, sb, rows, d, out);
  } else if (fmt == kMXFP4) {
    hipLaunchKernelGGL(bwd_dequant_kernel<kMXFP4>, dim3(nb), dim3(256), 0, s, xb, sb, rows, d, out);
  } else {
    return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

// ----------------------------------------------------------------- dk

constexpr int kRsThreads = 256;
constexpr int kRsItems = 16;
constexpr int kRsTile = kRsThreads * kRsItems;  // entries per sort tile

int rs_tiles(int64_t N) { return (int)((N + kRsTile - 1) / kRsTile); }

// (key position, entry) pairs of a chunk; positions outside [0, L) become L
// (they sort last and are skipped).
// The value is the entry's u row: query-major, slots padded to an even
// number of key tiles.
__global__ void bwd_pairs_kernel(const int* idx, int L, int N, int topk, int kpad, uint32_t* keys,
                                 uint32_t* vals) {
  const int e = blockIdx.x * blockDim.x + threadIdx.x;
  if (e >= N) return;
  const int s = idx[e];
  keys[e] = (s >= 0 && s < L) ? (uint32_t)s : (uint32_t)L;
  vals[e] = (uint32_t)((e / topk) * kpad + e % topk);
}

// Digit counts of one tile, stored digit-major: hist[d * ntiles + tile].
__global__ void __launch_bounds__(kRsThreads) rs_hist_kernel(const uint32_t* keys, int N, int shift,
                                                             int ntiles, uint32_t* hist) {
  __shared__ int cnt[256];
  const int tid = threadIdx.x;
  cnt[tid] = 0;
  __syncthreads();
  const int base = blockIdx.x * kRsTile;
  for (int it = 0; it < kRsItems; ++it) {
    const int e = base + it * kRsThreads + tid;
    if (e < N) atomicAdd(&cnt[(keys[e] >> shift) & 255u], 1);
  }
  __syncthreads();
  hist[(int64_t)tid * ntiles + blockIdx.x] = (uint32_t)cnt[tid];
}

// Exclusive scan of one digit's per-tile counts (workgroup d scans
// hist[d][0..ntiles) in place) and that digit's total in tot[d].
__global__ void __launch_bounds__(kRsThreads) rs_scan_kernel(uint32_t* hist, int ntiles,
                                                             uint32_t* tot) {
  __shared__ uint32_t wsum[kRsThreads / kWave];
  __shared__ uint32_t carry;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  uint32_t* v = hist + (int64_t)blockIdx.x * ntiles;
  if (tid == 0) carry = 0u;
  __syncthreads();
  for (int b0 = 0; b0 < ntiles; b0 += kRsThreads) {
    const int i = b0 + tid;
    const uint32_t x = i < ntiles ? v[i] : 0u;
    const uint32_t pre = (uint32_t)wave_prefix_excl((int)x);
    if (lane == 63) wsum[wave] = pre + x;
    __syncthreads();
    uint32_t off = carry;
    for (int w = 0; w < wave; ++w) off += wsum[w];
    if (i < ntiles) v[i] = off + pre;
    __syncthreads();
    if (tid == kRsThreads - 1) carry = off + pre + x;
    __syncthreads();
  }
  if (tid == 0) tot[blockIdx.x] = carry;
}

// Stable scatter of one tile by its 8-bit digit.  Entries are taken in
// rounds of 256 (round, wave, lane order = input order); within a wave the
// entries with the same digit are found with 8 bit-plane ballots.  The tile
// is first arranged by digit in LDS and then written out run by run, so
// consecutive lanes store consecutive addresses of a digit's run instead of
// every round scattering single elements over up to 256 runs.
__global__ void __launch_bounds__(kRsThreads) rs_scatter_kernel(const uint32_t* kin,
                                                                const uint32_t* vin, uint32_t* kout,
                                                                uint32_t* vout, int N, int shift,
                                                                int ntiles, const uint32_t* hist,
                                                                const uint32_t* tot) {
  __shared__ uint32_t base[256];    // output position of this tile's first entry of digit d
  __shared__ uint32_t lbase[256];   // LDS position of digit d's next entries
  __shared__ uint32_t lstart[256];  // LDS position of digit d's first entry
  __shared__ uint32_t wc[kRsThreads / kWave][256];
  __shared__ uint32_t tk[kRsTile], tv[kRsTile];
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const uint64_t lt = lane == 0 ? 0ull : (~0ull >> (64 - lane));
  const int t0 = blockIdx.x * kRsTile;
  {
    // entries of smaller digits (exclusive scan of the 256 digit totals)
    const uint32_t x = tot[tid];
    const uint32_t pre = (uint32_t)wave_prefix_excl((int)x);
    if (lane == 63) wc[0][wave] = pre + x;
    __syncthreads();
    uint32_t off = 0u;
    for (int w = 0; w < wave; ++w) off += wc[0][w];
    __syncthreads();
    base[tid] = off + pre + hist[(int64_t)tid * ntiles + blockIdx.x];
    wc[1][tid] = 0u;
  }
  __syncthreads();
  // this tile's digit counts, then their exclusive scan: where each digit's
  // entries start in the LDS copy
  for (int it = 0; it < kRsItems; ++it) {
    const int e = t0 + it * kRsThreads + tid;
    if (e < N) atomicAdd(&wc[1][(kin[e] >> shift) & 255u], 1u);
  }
  __syncthreads();
  {
    const uint32_t x = wc[1][tid];
    const uint32_t pre = (uint32_t)wave_prefix_excl((int)x);
    if (lane == 63) wc[0][wave] = pre + x;
    __syncthreads();
    uint32_t off = 0u;
    for (int w = 0; w < wave; ++w) off += wc[0][w];
    lstart[tid] = off + pre;
    lbase[tid] = off + pre;
  }
  __syncthreads();
#pragma unroll
  for (int w = 0; w < kRsThreads / kWave; ++w) wc[w][tid] = 0u;
  __syncthreads();
  for (int it = 0; it < kRsItems; ++it) {
    const int e = t0 + it * kRsThreads + tid;
    const bool valid = e < N;
    const uint32_t key = valid ? kin[e] : 0u;
    const uint32_t val = valid ? vin[e] : 0u;
    const uint32_t dg = (key >> shift) & 255u;
    uint64_t peers = __ballot(valid);
#pragma unroll
    for (int bit = 0; bit < 8; ++bit) {
      const bool on = (dg >> bit) & 1u;
      const uint64_t bb = __ballot(on);
      peers &= on ? bb : ~bb;
    }
    const int rank = __popcll(peers & lt);
    if (valid && rank == 0) wc[wave][dg] = (uint32_t)__popcll(peers);
    __syncthreads();
    if (valid) {
      uint32_t off = lbase[dg] + (uint32_t)rank;
      for (int w = 0; w < wave; ++w) off += wc[w][dg];
      tk[off] = key;
      tv[off] = val;
    }
    __syncthreads();
    uint32_t s = 0;
#pragma unroll
    for (int w = 0; w < kRsThreads / kWave; ++w) {
      s += wc[w][tid];
      wc[w][tid] = 0u;
    }
    lbase[tid] += s;
    __syncthreads();
  }
  // the tile in digit order: entry i goes to its digit's output run
  const int n = min(kRsTile, N - t0);
  for (int i = tid; i < n; i += kRsThreads) {
    const uint32_t key = tk[i];
    const uint32_t dg = (key >> shift) & 255u;
    const uint32_t o = base[dg] + ((uint32_t)i - lstart[dg]);
    kout[o] = key;
    vout[o] = tv[i];
  }
}

// dk[s] (+)= the u rows of key s's run, summed in sorted (entry) order.  Wave
// w owns the runs that START at sorted positions [64w, 64w + 64); the last of
// them may continue past the window.  The wave walks its rows in order,
// kDkBatch row loads in flight at a time, and flushes a run's sum when the
// key changes (stored on the first chunk, added on later ones).
constexpr int kDkBatch = 8;

template <int D>
__global__ void __launch_bounds__(256) dk_segments_kernel(const uint32_t* keys, const uint32_t* vals,
                                                          int N, uint32_t L, const float* u,
                                                          float* dk, int accumulate) {
  constexpr int V = D / 64;  // floats per lane per row
  const int lane = threadIdx.x & 63;
  const int p0 = (blockIdx.x * (blockDim.x >> 6) + (threadIdx.x >> 6)) * 64;
  if (p0 >= N) return;  // wave-uniform; no barrier in this kernel
  const int p = p0 + lane;
  const uint32_t kp = p < N ? keys[p] : 0xFFFFFFFFu;
  const uint32_t kprev = p == 0 ? 0xFFFFFFFFu : (p <= N ? keys[p - 1] : 0xFFFFFFFFu);
  const uint32_t myval = p < N ? vals[p] : 0u;
  const uint64_t heads = __ballot(p < N && kp < L && kp != kprev);
  if (!heads) return;
  const int first = __builtin_ctzll(heads);
  const uint32_t s_last = __shfl(kp, 63 - __builtin_clzll(heads));
  uint32_t cur = __shfl(kp, first);
  float acc[V];
#pragma unroll
  for (int v = 0; v < V; ++v) acc[v] = 0.0f;
  auto flush = [&](uint32_t key) {
    float* out = dk + (int64_t)key * D + V * lane;
#pragma unroll
    for (int v = 0; v < V; ++v) out[v] = accumulate ? out[v] + acc[v] : acc[v];
  };
  for (int x = p0 + first;; x += kDkBatch) {
    uint32_t kb[kDkBatch], vb[kDkBatch];
    bool own[kDkBatch];
#pragma unroll
    for (int b = 0; b < kDkBatch; ++b) {
      const int xb = x + b;
      if (xb - p0 < 64) {  // uniform: inside the window, from registers
        kb[b] = __shfl(kp, xb - p0);
        vb[b] = __shfl(myval, xb - p0);
        own[b] = kb[b] < L;  // every valid run here started in the window
      } else {             // past the window: only the last run continues
        kb[b] = xb < N ? keys[xb] : 0xFFFFFFFFu;
        own[b] = kb[b] == s_last;
        vb[b] = own[b] ? vals[xb] : 0u;
      }
    }
    float r[kDkBatch][V];
#pragma unroll
    for (int b = 0; b < kDkBatch; ++b) {
      const float* row = u + (int64_t)(own[b] ? vb[b] : 0u) * D + V * lane;
#pragma unroll
      for (int v = 0; v < V; ++v) r[b][v] = own[b] ? row[v] : 0.0f;
    }
#pragma unroll
    for (int b = 0; b < kDkBatch; ++b) {
      if (!own[b]) continue;  // uniform
      if (kb[b] != cur) {
        flush(cur);
        cur = kb[b];
#pragma unroll
        for (int v = 0; v < V; ++v) acc[v] = 0.0f;
      }
#pragma unroll
      for (int v = 0; v < V; ++v) acc[v] += r[b][v];
    }
    if (!own[kDkBatch - 1]) break;  // uniform: the wave's last run has ended
  }
  flush(cur);
}

__global__ void fill_zero_kernel(float* p, int64_t n) {
  for (int64_t i = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; i < n;
       i += (int64_t)gridDim.x * blockDim.x)
    p[i] = 0.0f;
}

size_t bwd_sort_hist_count(int64_t N) { return (size_t)256 * rs_tiles(N) + 256; }

hipError_t launch_fill_zero(float* p, int64_t n, hipStream_t s) {
  if (n <= 0) return hipSuccess;
  const int64_t want = (n + 255) / 256;
  const int nb = (int)(want < 8192 ? want : 8192);
  hipLaunchKernelGGL(fill_zero_kernel, dim3(nb), dim3(256), 0, s, p, n);
  return hipGetLastError();
}

hipError_t launch_bwd_sort(const DkArgs& a, const uint32_t** sorted_keys,
                           const uint32_t** sorted_rows, hipStream_t s) {
  const int N = a.N;
  *sorted_keys = a.k0;
  *sorted_rows = a.v0;
  if (N <= 0) return hipSuccess;
  const int nb = (N + 255) / 256;
  hipLaunchKernelGGL(bwd_pairs_kernel, dim3(nb), dim3(256), 0, s, a.idx, a.L, N, a.topk,
                     bwd_padded_k(a.topk), a.k0, a.v0);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const int ntiles = rs_tiles(N);
  int bits = 0;
  while (bits < 32 && ((uint64_t)a.L >> bits) != 0) ++bits;  // keys lie in [0, L]
  uint32_t *ki = a.k0, *vi = a.v0, *ko = a.k1, *vo = a.v1;
  uint32_t* tot = a.hist + (size_t)256 * ntiles;
  for (int shift = 0; shift < bits; shift += 8) {
    hipLaunchKernelGGL(rs_hist_kernel, dim3(ntiles), dim3(kRsThreads), 0, s, ki, N, shift, ntiles,
                       a.hist);
    hipLaunchKernelGGL(rs_scan_kernel, dim3(256), dim3(kRsThreads), 0, s, a.hist, ntiles, tot);
    hipLaunchKernelGGL(rs_scatter_kernel, dim3(ntiles), dim3(kRsThreads), 0, s, ki, vi, ko, vo, N,
                       shift, ntiles, a.hist, tot);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    uint32_t* t = ki; ki = ko; ko = t;
    t = vi; vi = vo; vo = t;
  }
  *sorted_keys = ki;
  *sorted_rows = vi;
  return hipSuccess;
}

hipError_t launch_bwd_segments(const uint32_t* sorted_keys, const uint32_t* sorted_rows, int N,
                               int L, const float* u, float* dk, bool accumulate, int d,
                               hipStream_t s) {
  if (N <= 0) return hipSuccess;
  const int grid = (N + 255) / 256;  // 4 waves of 64 sorted positions each
  if (d == 64) {
    hipLaunchKernelGGL(dk_segments_kernel<64>, dim3(grid), dim3(256), 0, s, sorted_keys,
                       sorted_rows, N, (uint32_t)L, u, dk, accumulate ? 1 : 0);
  } else if (d == 128) {
    hipLaunchKernelGGL(dk_segments_kernel<128>, dim3(grid), dim3(256), 0, s, sorted_keys,
                       sorted_rows, N, (uint32_t)L, u, dk, accumulate ? 1 : 0);
  } else {
    return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

int bwd_padded_k(int topk) { return (((topk + kBwdTK - 1) / kBwdTK + 1) & ~1) * kBwdTK; }

}  // namespace hk
