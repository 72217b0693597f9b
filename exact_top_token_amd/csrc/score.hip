// Fused indexer scoring over causal key ranges (the hot loop of HyTopK).
//
// A workgroup of 8 waves (4 for MXFP4) owns 16 (8) queries, one
// query pair per wave held in registers as MFMA A operands, and streams key
// tiles of 128 keys through LDS; every key tile is read from memory once per
// workgroup.
// Per 16-key column block each wave runs 8 x 4 MFMAs (bf16, H = 64, d = 128),
// applies ReLU and the weighted head sum in registers and then either
//   COMPACT: tests every score against the query's sampled threshold in
//     registers and emits only the passing keys into the query's bounded
//     candidate buffer, so no score table is written (HyScale explainer,
//     HyTopK paragraph);
//   ROWS: writes the score to a full score row (the conventional table of the
//     explainer's contest paragraph; also the recovery and full-rescore path).
// Both modes share the scoring code, so a query's scores are bit-identical on
// every path.
#include <type_traits>

#include "launch.h"
#include "tile.h"

namespace hk {

constexpr int kTK = 64;          // keys per scoring pass (a stage holds two)
// Waves per workgroup, one query pair each: 8 (one group per CU, 16 queries
// sharing each key tile) except for MXFP4, which keeps 4: its registers
// allow three waves per SIMD, so three independent groups of 4 share a CU
// and drift out of phase, one group's epilogue overlapping another's MFMAs.
// Measured at the 1M shape: 8 waves take FP8 and MXFP8 2.7-2.8% under 4 (with
// the linear row block; before it, 4 were faster), MXFP4 is 0.9% slower with
// 8, and bf16 4.5% slower with 4.
template <int FMT>
struct Group {
  static constexpr int WAVES = FMT == kMXFP4 ? 4 : 8;
  static constexpr int THREADS = 64 * WAVES;
  static constexpr int QUERIES = 2 * WAVES;
};
constexpr int kSB = 128;         // staged candidates per query before a flush

// Key tiles stream through four LDS stages filled by direct-to-LDS loads
// (global_load_lds_dwordx4), three tiles ahead of the one being scored, with
// one workgroup barrier per tile.  (The compiler cannot tell a stage being
// refilled from the one being read and waits for every outstanding tile
// load before a tile's first LDS read; the refills come from L2, so that
// wait costs little.)
// OWN (COMPACT with one key split): each wave is the only writer of its two
// queries' candidates, so it keeps their counts in registers and every
// passing lane stores its candidate straight to its slot; with several
// splits per query, candidates are staged per wave in LDS and flushed with
// one atomicAdd on the query's count.
template <int RB, int D, int FMT, bool ROWS, bool OWN>
__global__ void __launch_bounds__(Group<FMT>::THREADS) __attribute__((amdgpu_waves_per_eu(2)))
score_tile_kernel(ScoreArgs a) {
  constexpr int kWaves = Group<FMT>::WAVES, kThreads = Group<FMT>::THREADS;
  constexpr int kGroupQ = Group<FMT>::QUERIES;
  using T = PairTile<RB, D, FMT>;
  using F = Fmt<FMT>;
  using Frag = typename T::Frag;
  constexpr int RBYTES = T::RBYTES, NCH = T::NCH, KS = T::KS;
  // keys per stage: 128 (32 KB of bf16 rows, 16 KB of E4M3, 8 KB of E2M1),
  // scored in passes of four 16-key column blocks
  constexpr int TK = 2 * kTK;
  static_assert(!F::MX || KS == 1, "MX scales are loaded for one k-step");
  constexpr int TILE_BYTES = TK * RBYTES;
  constexpr int OPS = TILE_BYTES / (kThreads * 16);  // 16-byte DMA loads per lane per tile
  constexpr int KPB = 1024 / RBYTES;                  // keys per 1 KB DMA block
  constexpr int NCB = TK / 16;                        // 16-key column blocks per tile
  static_assert(TILE_BYTES % (kThreads * 16) == 0, "tile must split evenly over the workgroup");
  // The scaled formats' key scales travel with their tile: one dword per key
  // (FP8: its fp32 scale; MX: its four E8M0 block bytes) after the rows,
  // TK / kWaves keys loaded by each wave, so that no scale is a register
  // load in flight when a stage is read.
  constexpr int SC_BYTES = F::SCALED ? TK * 4 : 0;
  constexpr int SKW = TK / kWaves;                     // scale dwords per wave per tile
  static_assert(!F::SCALED || (T::NBLK == 4 && SKW <= 64), "one dword of scales per key");
  constexpr int VMT = OPS + (F::SCALED ? 1 : 0);       // vector-memory operations per tile and wave

  __shared__ __attribute__((aligned(1024))) uint8_t t0[TILE_BYTES + SC_BYTES];
  __shared__ __attribute__((aligned(1024))) uint8_t t1[TILE_BYTES + SC_BYTES];
  __shared__ __attribute__((aligned(1024))) uint8_t t2[TILE_BYTES + SC_BYTES];
  __shared__ __attribute__((aligned(1024))) uint8_t t3[TILE_BYTES + SC_BYTES];
  __shared__ uint2 stage[(ROWS || OWN) ? 1 : kWaves][2][(ROWS || OWN) ? 1 : kSB];
  // per wave: the pieces of its two queries' linear row blocks (scaled formats)
  __shared__ __attribute__((aligned(16))) uint32_t lin_lds[F::SCALED ? kWaves : 1][2 * kLinWords];
  __shared__ int s_maxt[kWaves];
  __shared__ int s_minlo[kWaves];

  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63, g = lane >> 4;
  auto swz = [](int kk) { return key_swz<NCH>(kk); };
  const int group = blockIdx.x / a.nsplit, split = blockIdx.x % a.nsplit;
  const int e0 = group * kGroupQ + wave * 2;
  // live launch entries (ROWS: a recovery pass may hold fewer than nq)
  const int nq = ROWS ? a.gate.live(a.nq) : a.nq;
  const int ea = e0 < nq ? e0 : -1;
  const int eb = e0 + 1 < nq ? e0 + 1 : -1;
  const int qa = ea < 0 ? -1 : (a.qlist ? a.qlist[ea] : a.q_offset + ea);
  const int qb = eb < 0 ? -1 : (a.qlist ? a.qlist[eb] : a.q_offset + eb);

  // Key ranges of the pair (an absent or empty query gets lo > hi).
  const QRange ra = qa >= 0 ? query_range(a.qpos, a.qfirst, a.q_start, a.L, qa) : QRange{1, 0};
  const QRange rb = qb >= 0 ? query_range(a.qpos, a.qfirst, a.q_start, a.L, qb) : QRange{1, 0};
  if (lane == 0) {
    int m = -1, lo = 0x7fffffff;
    if (ra.lo <= ra.hi) { m = ra.hi; lo = ra.lo; }
    if (rb.lo <= rb.hi) { m = max(m, rb.hi); lo = min(lo, rb.lo); }
    s_maxt[wave] = m;
    s_minlo[wave] = lo;
  }
  __syncthreads();
  int maxt = s_maxt[0], minlo = s_minlo[0];
#pragma unroll
  for (int w = 1; w < kWaves; ++w) {
    maxt = max(maxt, s_maxt[w]);
    minlo = min(minlo, s_minlo[w]);
  }
  // This split's keys that some query of the group sees, from a tile
  // boundary: [kb, ke).
  const int kb = max(split * a.split_len, minlo & ~(TK - 1));
  const int ke = min(split * a.split_len + a.split_len, maxt + 1);
  if (kb >= ke) return;  // uniform over the workgroup
  const int ntiles = (ke - kb + TK - 1) / TK;

  // DMA layout: load p of wave w fills 1 KB block p * kWaves + w of a stage; its
  // lane j lands on key kk = block * KPB + j / NCH, 16-byte slot j % NCH,
  // and fetches chunk (slot ^ swz(kk)) of that key: the swizzle the B
  // fragment reads undo.  swz(kk) does not depend on p.
  const int dma_kk = wave * KPB + lane / NCH;
  const int dma_c = ((lane % NCH) ^ swz(dma_kk)) * 16;
  const int full_tiles = (a.L - kb) / TK;  // tiles that lie entirely below L
  // Full tiles (all but the last one or two) take a per-lane constant offset
  // from a scalar tile base, and the LDS destination is wave-uniform, so
  // issuing a tile costs almost no vector work.
  const int wave_u = __builtin_amdgcn_readfirstlane(wave);
  const int dma_off = dma_kk * RBYTES + dma_c;  // load p adds p * kWaves * 1 KB
  auto issue = [&](int tile, uint8_t* buf) {
    const int k0 = kb + tile * TK;
    const uint8_t* base = a.k + (int64_t)k0 * RBYTES;
    if (tile < full_tiles) {  // uniform
#pragma unroll
      for (int p = 0; p < OPS; ++p)
        __builtin_amdgcn_global_load_lds(base + (dma_off + p * kWaves * 1024),
                                         HK_LDS(buf + (p * kWaves + wave_u) * 1024), 16, 0, 0);
    } else {
#pragma unroll
      for (int p = 0; p < OPS; ++p) {
        const int kk = dma_kk + p * kWaves * KPB;
        const int off = (min(k0 + kk, a.L - 1) - k0) * RBYTES + dma_c;  // never past L
        __builtin_amdgcn_global_load_lds(base + off, HK_LDS(buf + (p * kWaves + wave_u) * 1024), 16, 0, 0);
      }
    }
    if constexpr (F::SCALED) {
      if (lane < SKW) {  // the instruction issues in every wave (lanes 0 .. SKW - 1 active)
        const int key = min(k0 + wave * SKW + lane, a.L - 1);
        lds_dma4(static_cast<const uint8_t*>(a.k_scale) + (int64_t)key * 4, buf + TILE_BYTES + wave_u * SKW * 4);
      }
    }
  };
  // Walk position it scores key tile tile_of(it): ascending, or descending
  // when the caller asks for the reversed walk (a determinism check: the
  // candidates then reach the buffer in the opposite order, and the result,
  // which depends only on the candidate multiset, must not change).
  auto tile_of = [&](int it) { return a.reverse ? ntiles - 1 - it : it; };
  issue(tile_of(0), t0);
  if (1 < ntiles) issue(tile_of(1), t1);
  if (2 < ntiles) issue(tile_of(2), t2);

  T qt;
  qt.load(a.q, a.w, a.q_scale, a.H, qa, qb, lin_lds[F::SCALED ? wave : 0]);

  // This lane's query (lanes 0..31: A, 32..63: B) and its key limit.
  const int sel = lane >> 5;
  const int qs = sel ? qb : qa;
  const int es = sel ? eb : ea;
  const QRange rs = sel ? rb : ra;
  const int first = rs.lo;                    // keys first .. lim - 1 of this split
  const int lim = qs >= 0 ? min(rs.hi + 1, ke) : 0;
  float tau = 0.0f;
  if (!ROWS) tau = qs >= 0 ? a.tau[qs] : 0.0f;
  const bool owner = (lane & 16) == 0;  // lanes 0..15 and 32..47 own distinct (query, key)
  // Keys [in_lo, in_hi) lie inside both queries' ranges (empty when a query
  // is absent); read into scalars, so the per-pass test is a uniform branch
  // (the compiler cannot see that the ranges are wave-uniform).
  const int in_lo = __builtin_amdgcn_readfirstlane(max(ra.lo, rb.lo));
  const int in_hi =
      __builtin_amdgcn_readfirstlane((qa >= 0 && qb >= 0) ? min(min(ra.hi, rb.hi) + 1, ke) : 0);

  int cntA = 0, cntB = 0;  // candidates staged (OWN: emitted) per query (wave-uniform)

  auto flush = [&](int which, int count) {
    __builtin_amdgcn_fence(__ATOMIC_ACQ_REL, "wavefront");
    __builtin_amdgcn_wave_barrier();
    const int qf = which ? qb : qa;
    int base = 0;
    if (lane == 0) base = atomicAdd(a.cnt + qf, count);
    base = __shfl(base, 0);
    uint2* dst = a.cand + (int64_t)qf * a.cap;
    for (int j = lane; j < count; j += kWave) {
      const int p = base + j;
      if (p < a.cap) dst[p] = stage[ROWS ? 0 : wave][which][j];
    }
    HK_WAIT_VM(0);  // leave only stage loads in flight, so the per-tile counts stay exact
    __builtin_amdgcn_fence(__ATOMIC_ACQ_REL, "wavefront");
    __builtin_amdgcn_wave_barrier();
  };

  constexpr int NCP = NCB > 4 ? 4 : NCB;  // column blocks per scoring pass
  // B fragments (and the scaled formats' key-scale dword) of column block j
  // of a stage
  struct BlockIn {
    Frag b[KS];
    uint32_t sv;
  };
  auto read_block = [&](const uint8_t* stage_base, int j, BlockIn& in) {
    const int kt = j * 16 + (lane & 15);
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) in.b[ks] = stage_frag<FMT, D>(stage_base + kt * RBYTES, kt, g, ks);
    in.sv = F::SCALED ? *reinterpret_cast<const uint32_t*>(stage_base + TILE_BYTES + 4 * kt) : 0u;
  };
  BlockIn bin;
  // One key split per query (and the row path): the next block's fragments
  // are read between this block's MFMA phase and its epilogue.  With several
  // splits the staged-candidate path has no registers to spare for it.
  constexpr bool PF = OWN || ROWS;
  auto compute_part = [&](int it, int part, const uint8_t* stage_base) {
    const int k0 = kb + it * TK + part * NCP * 16;
    float sc[NCP];
    // PF: each block's partner-lane exchange is issued after the next
    // block's MFMA phase, so no MFMA phase waits for a shuffle issued just
    // before it (the pass's last exchange is waited for before the compare).
    float th[NCP], tp[NCP];
    uint32_t svs[NCP];
#pragma unroll
    for (int cb = 0; cb < NCP; ++cb) {
      const int j = part * NCP + cb;
      if constexpr (!PF) read_block(stage_base, j, bin);
      int sb[KS];
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) sb[ks] = F::MX ? (int)((bin.sv >> (8 * (4 * ks + g))) & 0xFFu) : 127;
      const uint32_t sv = bin.sv;
      typename T::Acc acc;
      qt.mma_phase(bin.b, sb, acc);
      if constexpr (PF) {
        if (cb > 0) tp[cb - 1] = __shfl_xor(th[cb - 1], 16);
        // the next block's fragments load while this block's epilogue runs
        if (j + 1 < NCB) read_block(stage_base, j + 1, bin);
        __builtin_amdgcn_sched_barrier(0);
        th[cb] = qt.half_sum(acc);
        svs[cb] = sv;
      } else {
        float s = qt.epilogue(acc);
        if constexpr (FMT == kFP8) s *= __uint_as_float(sv);
        sc[cb] = s;
      }
    }
    if constexpr (PF) {
      tp[NCP - 1] = __shfl_xor(th[NCP - 1], 16);
#pragma unroll
      for (int cb = 0; cb < NCP; ++cb) {
        float s = th[cb] + tp[cb];  // the epilogue's sum: own half + partner's half
        if constexpr (FMT == kFP8) s *= __uint_as_float(svs[cb]);
        sc[cb] = s;
      }
    }
    if constexpr (ROWS) {
#pragma unroll
      for (int cb = 0; cb < NCP; ++cb) {
        const int key = k0 + cb * 16 + (lane & 15);
        if (owner && key >= first && key < lim) a.rows[(int64_t)es * a.row_stride + key] = sc[cb];
      }
    } else {
      // One uniform branch per pass: the candidate path runs only when some
      // key of the 64 passes (about one pass in two at the 1M shape).  A
      // pass inside both queries' key ranges (all but the edges) skips the
      // per-key range test: IN is a compile-time copy of that uniform fact.
      auto candidates = [&](auto in_c) {
        constexpr bool IN = decltype(in_c)::value;
        // The ballots are taken of the comparisons themselves (lanes 16..31
        // and 48..63 hold the same scores as their partners and are masked
        // out afterwards), so they stay scalar masks with no vector work.
        constexpr uint64_t kOwners = 0x0000FFFF0000FFFFull;
        auto hits = [&](int cb, int key) {
          return (IN || (key >= first && key < lim)) && sc[cb] >= tau;
        };
        uint64_t mcb[NCP];
        uint64_t any = 0;
#pragma unroll
        for (int cb = 0; cb < NCP; ++cb) {
          mcb[cb] = __builtin_amdgcn_ballot_w64(hits(cb, k0 + cb * 16 + (lane & 15))) & kOwners;
          any |= mcb[cb];
        }
        if (!any) return;
#pragma unroll
        for (int cb = 0; cb < NCP; ++cb) {
          const int key = k0 + cb * 16 + (lane & 15);
          const uint64_t m = mcb[cb];
          if (m) {
            const uint32_t mA = (uint32_t)(m & 0xFFFFull);
            const uint32_t mB = (uint32_t)((m >> 32) & 0xFFFFull);
            if (owner && hits(cb, key)) {
              const uint32_t mm = sel ? mB : mA;
              const int rank = __popc(mm & ((1u << (lane & 15)) - 1u));
              const int slot = (sel ? cntB : cntA) + rank;
              const uint2 c = make_uint2((uint32_t)key, __float_as_uint(sc[cb]));
              if constexpr (OWN) {
                if (slot < a.cap) a.cand[(int64_t)qs * a.cap + slot] = c;
              } else {
                stage[wave][sel][slot] = c;
              }
            }
            cntA += __popc(mA);
            cntB += __popc(mB);
            if constexpr (!OWN) {
              if (cntA > kSB - 16) { flush(0, cntA); cntA = 0; }
              if (cntB > kSB - 16) { flush(1, cntB); cntB = 0; }
            }
          }
        }
      };
      if (k0 >= in_lo && k0 + NCP * 16 <= in_hi) {
        candidates(std::true_type{});
      } else {
        candidates(std::false_type{});
      }
    }
  };

  auto compute = [&](int it, const uint8_t* tb) {
    if constexpr (PF) read_block(tb, 0, bin);
#pragma unroll
    for (int part = 0; part < NCB / NCP; ++part) compute_part(it, part, tb);
  };

  // Per tile: wait for this wave's loads of tile `it`, barrier (every wave's
  // loads landed; every wave finished tile it-1), refill tile it-1's stage
  // with tile it+3, score tile it (its key scales, for the scaled formats,
  // came with it).
  auto step = [&](int it, const uint8_t* cur, uint8_t* refill) {
    const int tl = tile_of(it);
    if (it + 2 < ntiles) {
      HK_WAIT_VM(2 * VMT);
    } else if (it + 1 < ntiles) {
      HK_WAIT_VM(VMT);
    } else {
      HK_WAIT_VM(0);
    }
    __builtin_amdgcn_s_barrier();
    if (it + 3 < ntiles) issue(tile_of(it + 3), refill);
    compute(tl, cur);
  };
  for (int it = 0; it < ntiles; it += 4) {
    step(it, t0, t3);
    if (it + 1 < ntiles) step(it + 1, t1, t0);
    if (it + 2 < ntiles) step(it + 2, t2, t1);
    if (it + 3 < ntiles) step(it + 3, t3, t2);
  }
  if constexpr (!ROWS && OWN) {
    // the total count, including candidates beyond cap (the check reads it)
    if (lane == 0) {
      if (qa >= 0) a.cnt[qa] = cntA;
      if (qb >= 0) a.cnt[qb] = cntB;
    }
  } else if constexpr (!ROWS) {
    if (cntA > 0) flush(0, cntA);
    if (cntB > 0) flush(1, cntB);
  }
}

template <int RB, int D, int FMT>
static hipError_t launch_rb(const ScoreArgs& a, hipStream_t s) {
  constexpr int gq = Group<FMT>::QUERIES;
  const int groups = (a.nq + gq - 1) / gq;
  dim3 grid((unsigned)(groups * a.nsplit)), block(Group<FMT>::THREADS);
  if (a.rows) {
    hipLaunchKernelGGL((score_tile_kernel<RB, D, FMT, true, false>), grid, block, 0, s, a);
  } else if (a.nsplit == 1) {
    hipLaunchKernelGGL((score_tile_kernel<RB, D, FMT, false, true>), grid, block, 0, s, a);
  } else {
    hipLaunchKernelGGL((score_tile_kernel<RB, D, FMT, false, false>), grid, block, 0, s, a);
  }
  return hipGetLastError();
}

template <int FMT>
static hipError_t launch_d128(const ScoreArgs& a, bool small, hipStream_t s) {
  return small ? launch_rb<1, 128, FMT>(a, s) : launch_rb<8, 128, FMT>(a, s);
}

hipError_t launch_score(const ScoreArgs& a, int d, int fmt, hipStream_t s) {
  if (a.nq <= 0) return hipSuccess;
  const bool small = a.H <= 8;
  if (fmt == kBF16) {
    if (d == 64) return small ? launch_rb<1, 64, kBF16>(a, s) : launch_rb<8, 64, kBF16>(a, s);
    if (d == 128) return launch_d128<kBF16>(a, small, s);
    return hipErrorInvalidValue;
  }
  if (d != 128) return hipErrorInvalidValue;
  if (fmt == kFP8) return launch_d128<kFP8>(a, small, s);
  if (fmt == kMXFP8) return launch_d128<kMXFP8>(a, small, s);
  if (fmt == kMXFP4) return launch_d128<kMXFP4>(a, small, s);
  return hipErrorInvalidValue;
}

int score_group_queries(int fmt) {
  if (fmt == kFP8) return Group<kFP8>::QUERIES;
  if (fmt == kMXFP8) return Group<kMXFP8>::QUERIES;
  if (fmt == kMXFP4) return Group<kMXFP4>::QUERIES;
  return Group<kBF16>::QUERIES;
}

}  // namespace hk
