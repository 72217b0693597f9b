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
//   block-wide radix select over the sample scores (in registers for bf16, in
//   LDS for the scaled formats) gives tau.
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
    const float t = add_lane_xor32(p);  // even + odd row blocks of this half
    return add_lane_xor16(t);           // + the other half
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
constexpr int kSampleWaves = kSampleThreads / kWave;
constexpr int kSampleDepth = 3;      // scaled formats: column blocks of gathers in flight per wave

// Loads the key rows at rowpos[p] (load p: rows p * KPI .. p * KPI + KPI - 1
// of a 16-sample block, lane l taking row p * KPI + dkk at byte offset
// dsw[p]) into the wave's stage `dst`: OPS direct-to-LDS loads of 1 KB.
template <int OPS, int RBYTES>
__device__ __forceinline__ void stage_rows(const uint8_t* k, const int (&rowpos)[OPS],
                                           const int (&dsw)[OPS], uint8_t* dst) {
#pragma unroll
  for (int p = 0; p < OPS; ++p) lds_dma16(k + (int64_t)rowpos[p] * RBYTES + dsw[p], dst + p * 1024);
}

// Block radix select of the r-th largest of the m sample scores held in
// registers: thread t holds sample t + 256 k in sv[N - K + k], k < K (the
// slots below N - K are unused).  The same counting as block_select_largest
// over the same multiset, so the same result.
template <int N>
__device__ uint32_t select_largest_regs(const float (&sv)[N], int K, int m, int r, RadixScratch& sc,
                                        int& rem, int& mult) {
  const int tid = threadIdx.x;
  uint32_t prefix = 0u, pmask = 0u;
  for (int pass = 3; pass >= 0; --pass) {
    const int shift = 8 * pass;
    for (int b = tid; b < 256; b += kSampleThreads) sc.hist[b] = 0;
    __syncthreads();
    uint32_t run_d = 0u;
    int run_n = 0;
#pragma unroll
    for (int sl = 0; sl < N; ++sl) {
      const int k = sl - (N - K);
      const int i = tid + k * kSampleThreads;
      if (k >= 0 && i < m) {
        const uint32_t kk = score_key(sv[sl]);
        if ((kk & pmask) == prefix) {
          const uint32_t d = (kk >> shift) & 255u;
          if (run_n > 0 && d != run_d) {
            atomicAdd(&sc.hist[run_d], run_n);
            run_n = 0;
          }
          run_d = d;
          ++run_n;
        }
      }
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

// bf16 samples: the sampled key rows reach the waves through LDS.
// Direct-to-LDS loads fetch each row whole (16 consecutive lanes per row,
// four lanes to each 64-byte piece), where loading the MFMA operand layout
// straight from memory gives every lane its own 16-byte piece of a
// different row: four times the address-unit work per byte, which bounded
// the gathers (the address path stalled on the cache 62% of the time).
// Each wave owns two stages (the block it scores and the next one's loads)
// and waits for a stage's loads by count.  The scores stay in registers
// (sv, N per thread) and the sample positions are carried per lane, so the
// workgroup's only LDS is the row ring: measured against keeping positions
// and scores in 32 KB of LDS per workgroup, the threshold takes 1.68 ->
// 1.35 ms at the 1M shape.
template <int RB4, int D, int N>
__device__ __forceinline__ void sample_scores_staged(const SampleArgs& a, const QueryTile<RB4, D, kBF16>& qt,
                                                     QRange rg, int ctx, int mq, float (&sv)[N]) {
  using T = QueryTile<RB4, D, kBF16>;
  constexpr int KS = T::KS, RBYTES = T::RBYTES, NCH = RBYTES / 16;
  constexpr int CB_BYTES = 16 * RBYTES;  // a column block's 16 key rows
  constexpr int DEPTH = 2;               // stages per wave: the block scored and the next
  constexpr int OPS = CB_BYTES / 1024;   // 1 KB loads per column block (= its vector-memory ops)
  constexpr int KPI = 1024 / RBYTES;     // key rows per load
  constexpr int SLOT = kSampleWaves * CB_BYTES;
  static_assert(CB_BYTES % 1024 == 0, "stage ring shape");
  __shared__ __attribute__((aligned(1024))) uint8_t ring_lds[DEPTH * SLOT];
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63, g = lane >> 4;

  // Wave w scores blocks 16 k + 4 w + b (b = 0..3) of 16 samples, so that
  // sample t + 256 k belongs to thread t (lane group b keeps block b's
  // scores); K rounds of four blocks cover the mq samples.
  const int K = (mq + kSampleThreads - 1) / kSampleThreads;
  uint8_t* const ring0 = ring_lds + __builtin_amdgcn_readfirstlane(wave) * CB_BYTES;  // stage s: + s * SLOT
  const int dkk = lane / NCH;
  int dsw[OPS];  // the stage's swizzle: load p fetches this chunk of its row
#pragma unroll
  for (int p = 0; p < OPS; ++p) dsw[p] = 16 * ((lane % NCH) ^ key_swz<NCH>(p * KPI + dkk));
  // Positions lo + floor(j * ctx / mq) of this lane's rows, carried from
  // block to block: the next block is 16 samples on, or 208 from the last
  // block of a round to the first of the next.
  // Only load 0's row is carried (position and remainder); the rows of
  // loads 1.. are KPI samples apart and derived from it at each issue.
  const int q16 = (int)((int64_t)16 * ctx / mq), r16 = (int)((int64_t)16 * ctx % mq);
  const int q208 = (int)((int64_t)208 * ctx / mq), r208 = (int)((int64_t)208 * ctx % mq);
  const int qk = (int)((int64_t)KPI * ctx / mq), rk = (int)((int64_t)KPI * ctx % mq);
  int jb = __builtin_amdgcn_readfirstlane(wave * 64);  // first sample of the next block (uniform)
  int pos0, rem0;
  {
    const int64_t n0 = (int64_t)(jb + dkk) * ctx;
    pos0 = (int)(n0 / mq);
    rem0 = (int)(n0 % mq);
  }
  int nissued = 0;
  auto issue = [&](int slot) {  // the wave's next block into ring slot `slot`
    int rowpos[OPS];
    int pp = pos0, rr = rem0;
#pragma unroll
    for (int p = 0; p < OPS; ++p) {
      rowpos[p] = rg.lo + (jb + p * KPI + dkk < mq ? pp : 0);  // past the samples: row lo, never scored
      pp += qk;
      rr += rk;
      if (rr >= mq) {
        rr -= mq;
        ++pp;
      }
    }
    const bool round_end = (nissued & 3) == 3;
    jb += round_end ? 208 : 16;
    pos0 += round_end ? q208 : q16;
    rem0 += round_end ? r208 : r16;
    if (rem0 >= mq) {
      rem0 -= mq;
      ++pos0;
    }
    ++nissued;
    stage_rows<OPS, RBYTES>(a.k, rowpos, dsw, ring0 + slot * SLOT);
  };
  issue(0);
  for (int k = 0; k < K; ++k) {
    float mine = 0.0f;
#pragma unroll
    for (int bq = 0; bq < 4; ++bq) {
      const int d = bq & 1;  // ring slot of this block (blocks alternate)
      issue(d ^ 1);          // the next block (past the last one: row lo, unscored)
      HK_WAIT_VM(OPS);       // this block's loads have landed
      const int kt = lane & 15;
      typename T::Frag b[KS];
      int sb[KS];
      stage_frags_bf16<D>(ring0 + d * SLOT + kt * RBYTES, kt, g, b);
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) sb[ks] = 127;
      // the selection kernels' head-sum order (see the kernel)
      const float s = qt.score(b, sb);
      if (g == bq) mine = s;
    }
    // keep this round's score: the slots shift down by one per round
#pragma unroll
    for (int sl = 0; sl < N - 1; ++sl) sv[sl] = sv[sl + 1];
    sv[N - 1] = mine;
  }
  HK_WAIT_VM(0);  // the load ahead has landed before the wave leaves its stages
}

// Scaled formats: the operand layout gathered straight into registers, the
// next kSampleDepth - 1 blocks of the wave in flight while it scores one.
// (Their rows are half or a quarter of bf16's, and the staged form measured
// slower for them: its LDS halves the waves per CU.)  Blocks past the last
// one fetch nothing.
template <int RB4, int D, int FMT>
__device__ __forceinline__ void sample_scores_direct(const SampleArgs& a, const QueryTile<RB4, D, FMT>& qt,
                                                     QRange rg, int ctx, int mq, float* S) {
  using T = QueryTile<RB4, D, FMT>;
  constexpr int KS = T::KS;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int ncb = (mq + 15) / 16;
  typename T::Frag buf[kSampleDepth][KS];
  int sbuf[kSampleDepth][KS];
  int kpos[kSampleDepth];
  float ksc[kSampleDepth];
  // This lane's sample position, carried from block to block (the wave's
  // blocks are 16 * waves samples apart): no division per fetch.
  constexpr int STEP = 16 * kSampleWaves;
  const int sq = (int)((int64_t)STEP * ctx / mq), sr = (int)((int64_t)STEP * ctx % mq);
  int jc = wave * 16 + (lane & 15), pc, rc;
  {
    const int64_t n0 = (int64_t)jc * ctx;
    pc = (int)(n0 / mq);
    rc = (int)(n0 % mq);
  }
  auto fetch = [&](int i, int slot) {  // the wave's i-th block (fetched in order) into `slot`
    const int pos = jc < mq ? rg.lo + pc : -1;
    jc += STEP;
    pc += sq;
    rc += sr;
    if (rc >= mq) {
      rc -= mq;
      ++pc;
    }
    kpos[slot] = pos;
    T::key(a.k, a.k_scale, pos, buf[slot], sbuf[slot]);
    if constexpr (FMT == kFP8) ksc[slot] = pos >= 0 ? static_cast<const float*>(a.k_scale)[pos] : 0.0f;
  };
  const int nmine = wave < ncb ? (ncb - wave + kSampleWaves - 1) / kSampleWaves : 0;  // wave-uniform
#pragma unroll
  for (int d = 0; d < kSampleDepth - 1; ++d) fetch(d, d);
  for (int i0 = 0; i0 < nmine; i0 += kSampleDepth) {
#pragma unroll
    for (int d = 0; d < kSampleDepth; ++d) {
      const int i = i0 + d;
      if (i >= nmine) break;  // wave-uniform
      fetch(i + kSampleDepth - 1, (d + kSampleDepth - 1) % kSampleDepth);
      float s = qt.score(buf[d], sbuf[d]);
      if constexpr (FMT == kFP8) s *= ksc[d];
      const int j = (wave + i * kSampleWaves) * 16 + (lane & 15);
      if (lane < 16 && kpos[d] >= 0) S[j] = s;
    }
  }
}

// One query per workgroup.  Row block rb of the A operand holds heads
// 16 rb .. 16 rb + 15 of the query; output lane group g holds heads
// 16 rb + 4 g + i, summed in-lane, then across the four lane groups.  Every
// sample's score follows the selection kernels' head-sum order, so it is
// bit-identical to the score the fused kernel compares with tau and the r
// sampled keys at or above tau always pass.
template <int RB4, int D, int FMT, int N>
// (Three waves per SIMD: the bf16 path fits 168 registers with its 32 sample
// scores per thread, and its row ring leaves the LDS for three workgroups;
// with 64 scores per thread, for sample counts above 8,192, two waves, so
// that they fit without spilling.)
__global__ void __launch_bounds__(kSampleThreads) __attribute__((amdgpu_waves_per_eu(N > 32 ? 2 : 3)))
sample_tau_kernel(SampleArgs a) {
  using T = QueryTile<RB4, D, FMT>;
  extern __shared__ float S[];  // sample scores, M_q entries
  __shared__ RadixScratch sc;
  __shared__ __attribute__((aligned(16))) uint32_t lin_lds[kSampleWaves][kLinWords];

  const int tid = threadIdx.x, wave = tid >> 6;
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
  int rem, mult;
  uint32_t v;
  if constexpr (FMT == kBF16) {
    // bf16: the sample scores stay in registers (N per thread), so the
    // workgroup's LDS is only its row ring
    float sv[N];
#pragma unroll
    for (int i = 0; i < N; ++i) sv[i] = 0.0f;
    sample_scores_staged<RB4, D, N>(a, qt, rg, ctx, mq, sv);
    __syncthreads();
    v = select_largest_regs<N>(sv, (mq + kSampleThreads - 1) / kSampleThreads, mq, r, sc, rem, mult);
  } else {
    sample_scores_direct<RB4, D, FMT>(a, qt, rg, ctx, mq, S);
    __syncthreads();
    v = block_select_largest(
        mq, r, [&](int i) { return score_key(S[i]); }, [](int) { return true; }, sc, rem, mult);
  }
  if (tid == 0) a.tau[q] = key_score(v);
}

template <int RB4, int D, int FMT, int N>
static hipError_t sample_launch(const SampleArgs& a, size_t lds, hipStream_t s) {
  static LdsLimit lim;
  if (lds) {
    hipError_t e = raise_dynamic_lds((const void*)sample_tau_kernel<RB4, D, FMT, N>, (int)lds, lim);
    if (e != hipSuccess) return e;
  }
  dim3 grid((unsigned)a.n), block(kSampleThreads);
  hipLaunchKernelGGL((sample_tau_kernel<RB4, D, FMT, N>), grid, block, lds, s, a);
  return hipGetLastError();
}

template <int RB4, int D, int FMT>
static hipError_t sample_rb(const SampleArgs& a, hipStream_t s) {
  const int mmax = a.M < a.L ? a.M : a.L;
  if constexpr (FMT == kBF16) {  // scores in registers: 32 or 64 per thread
    if (mmax <= 32 * kSampleThreads) return sample_launch<RB4, D, FMT, 32>(a, 0, s);
    return sample_launch<RB4, D, FMT, 64>(a, 0, s);
  } else {
    return sample_launch<RB4, D, FMT, 1>(a, (size_t)mmax * sizeof(float), s);
  }
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
