// C ABI of the selection library: argument validation, workspace layout and
// the launch sequence of hytopk_select / hytopk_replay /
// hytopk_baseline_select (declared in include/hytopk.h).
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <map>
#include <mutex>
#include <string>
#include <vector>

#include "hytopk.h"
#include "launch.h"

constexpr size_t kNoAllocBytes = size_t(64) << 20;
static_assert(kNoAllocBytes == HYTOPK_NOALLOC_SCRATCH_BYTES, "header and library disagree");
// The workspace of hytopk_select_noalloc (see scratch_address below).
static __device__ __align__(256) uint8_t scratch[kNoAllocBytes];

namespace {

thread_local std::string g_err;

int fail(int code, const char* msg) {
  g_err = msg;
  return code;
}

int hip_fail(hipError_t e, const char* where) {
  g_err = std::string(where) + ": " + hipGetErrorString(e);
  return HYTOPK_EHIP;
}

#define HK_HIP(expr, where)                     \
  do {                                          \
    hipError_t e_ = (expr);                     \
    if (e_ != hipSuccess) return hip_fail(e_, where); \
  } while (0)

// ------------------------------------------------------------------ tracing

struct TraceRec {
  std::string name;
  hipEvent_t a, b;
};

struct Tracer {
  std::mutex mu;
  bool on = false;
  std::vector<TraceRec> pending;
  std::vector<hipEvent_t> pool;
  std::map<std::string, std::pair<int, double>> acc;
};

Tracer& tracer() {
  static Tracer t;
  return t;
}

hipEvent_t take_event(Tracer& t) {
  if (!t.pool.empty()) {
    hipEvent_t e = t.pool.back();
    t.pool.pop_back();
    return e;
  }
  hipEvent_t e = nullptr;
  if (hipEventCreate(&e) != hipSuccess) return nullptr;
  return e;
}

// Brackets one launch with events when tracing is on.
struct Span {
  const char* name;
  hipStream_t s;
  hipEvent_t a = nullptr;
  Span(const char* nm, hipStream_t st) : name(nm), s(st) {
    Tracer& t = tracer();
    std::lock_guard<std::mutex> g(t.mu);
    if (!t.on) return;
    a = take_event(t);
    if (a && hipEventRecord(a, s) != hipSuccess) {  // no timing for this span
      (void)hipGetLastError();  // handled here; keep it from the next launch check
      t.pool.push_back(a);
      a = nullptr;
    }
  }
  ~Span() {
    if (!a) return;
    Tracer& t = tracer();
    std::lock_guard<std::mutex> g(t.mu);
    hipEvent_t b = take_event(t);
    if (b && hipEventRecord(b, s) == hipSuccess) {
      t.pending.push_back(TraceRec{name, a, b});
      return;
    }
    if (b) (void)hipGetLastError();  // handled here; keep it from the next launch check
    t.pool.push_back(a);  // the span is dropped; both events go back to the pool
    if (b) t.pool.push_back(b);
  }
};

constexpr size_t kAlign = 256;
constexpr int kMaxK = 2048;
constexpr int kMaxCap = 16384;
constexpr int kMaxM = 16384;
constexpr size_t kLdsLimit = 160 * 1024 - 10 * 1024;  // gfx950 LDS minus static scratch

size_t align_up(size_t x) { return (x + kAlign - 1) / kAlign * kAlign; }

struct Params {
  int m_min, m_max, m_div, oversample, cap, max_recover, force_path, rows_chunk;
};

int check_problem(const hytopk_problem* p) {
  if (!p) return fail(HYTOPK_EINVAL, "problem is NULL");
  if (p->L <= 0 || p->n <= 0 || p->q_start < 0) return fail(HYTOPK_EINVAL, "L, n must be > 0 and q_start >= 0");
  if (!p->q_pos && p->q_start + p->n > p->L) return fail(HYTOPK_EINVAL, "q_start + n > L");
  if (p->L >= (int64_t(1) << 31)) return fail(HYTOPK_EUNSUPPORTED, "L >= 2^31");
  if (p->n >= (int64_t(1) << 31)) return fail(HYTOPK_EUNSUPPORTED, "n >= 2^31");
  if (p->q_start >= (int64_t(1) << 31)) return fail(HYTOPK_EUNSUPPORTED, "q_start >= 2^31");
  if (p->k <= 0) return fail(HYTOPK_EINVAL, "k must be > 0");
  if (p->k > kMaxK) return fail(HYTOPK_EUNSUPPORTED, "k > 2048");
  if (p->H <= 0 || p->d <= 0) return fail(HYTOPK_EINVAL, "H, d must be > 0");
  if (p->H > 64) return fail(HYTOPK_EUNSUPPORTED, "H > 64");
  if (p->dtype == HYTOPK_BF16) {
    if (p->d != 64 && p->d != 128) return fail(HYTOPK_EUNSUPPORTED, "bf16 needs d in {64, 128}");
  } else if (p->dtype == HYTOPK_FP8_E4M3 || p->dtype == HYTOPK_MXFP8_E4M3 ||
             p->dtype == HYTOPK_MXFP4_E2M1) {
    if (p->d != 128) return fail(HYTOPK_EUNSUPPORTED, "fp8 and MX formats need d = 128");
  } else {
    return fail(HYTOPK_EINVAL, "unknown dtype");
  }
  return HYTOPK_OK;
}

Params resolve(const hytopk_problem* p, const hytopk_params* prm) {
  Params r{};
  r.m_min = (prm && prm->m_min) ? prm->m_min : 4096;
  r.m_max = (prm && prm->m_max) ? prm->m_max : 8192;
  r.m_div = (prm && prm->m_div) ? prm->m_div : 128;
  r.oversample = (prm && prm->oversample) ? prm->oversample : 3;
  r.cap = (prm && prm->cap) ? prm->cap : 6 * p->k;
  r.max_recover = (prm && prm->max_recover) ? prm->max_recover : 64;
  r.force_path = prm ? prm->force_path : HYTOPK_PATH_AUTO;
  // rows buffer: max_recover rows by default (one recovery pass)
  const int64_t dflt = std::min<int64_t>(p->n, std::max(1, r.max_recover));
  r.rows_chunk = (prm && prm->rows_chunk) ? prm->rows_chunk : (int)dflt;
  return r;
}

int check_params(const hytopk_problem* p, const Params& r) {
  if (r.m_min < 1 || r.m_max < r.m_min || r.m_div < 1 || r.oversample < 1 || r.cap < 1 ||
      r.max_recover < 0 || r.rows_chunk < 1)
    return fail(HYTOPK_EINVAL, "invalid threshold parameters");
  if (r.force_path != HYTOPK_PATH_AUTO && r.force_path != HYTOPK_PATH_ROWS_ALL)
    return fail(HYTOPK_EINVAL, "unknown force_path");
  // the rows buffer (rows_chunk x L fp32) must stay far from size_t overflow
  if (std::min<int64_t>(r.rows_chunk, p->n) * p->L > (int64_t(1) << 40))
    return fail(HYTOPK_EUNSUPPORTED, "rows_chunk * L > 2^40");
  if (r.m_max > kMaxM) return fail(HYTOPK_EUNSUPPORTED, "m_max > 16384");
  if (r.cap > kMaxCap) return fail(HYTOPK_EUNSUPPORTED, "cap > 16384");
  if (hk::cand_select_lds_bytes(r.cap, p->k) > kLdsLimit)
    return fail(HYTOPK_EUNSUPPORTED, "cap and k exceed the LDS of one workgroup");
  return HYTOPK_OK;
}

int sample_count(const hytopk_problem* p, const Params& r) {
  int64_t m = std::max<int64_t>(r.m_min, p->L / r.m_div);
  return (int)std::min<int64_t>(m, r.m_max);
}

struct Layout {
  size_t tau, cnt, failed, stats, cand, rows, split, total;
  int rows_n;
};

// Scratch of the split row top-k for up to `rows` rows (0 when that many rows
// fill the GPU one workgroup per row).
size_t split_bytes(const hytopk_problem* p, int rows) {
  if (rows > hk::kRowSplitMaxRows) return 0;
  return hk::row_select_scratch_bytes(rows, hk::row_select_max_chunks(p->L), p->k);
}

Layout layout(const hytopk_problem* p, const Params& r) {
  Layout l{};
  size_t off = 0;
  const size_t n = (size_t)p->n;
  l.tau = off; off = align_up(off + n * 4);
  l.cnt = off; off = align_up(off + n * 4);
  l.failed = off; off = align_up(off + n * 4);
  l.stats = off; off = align_up(off + sizeof(hk::DevStats));
  l.cand = off; off = align_up(off + n * (size_t)r.cap * 8);
  l.rows_n = (int)std::min<int64_t>(r.rows_chunk, p->n);
  l.rows = off; off = align_up(off + (size_t)l.rows_n * (size_t)p->L * 4);
  l.split = off; off = align_up(off + split_bytes(p, l.rows_n));
  l.total = off;
  return l;
}

int check_ws(void* ws, size_t bytes, size_t need) {
  if (!ws) return fail(HYTOPK_EWORKSPACE, "workspace is NULL");
  if (reinterpret_cast<uintptr_t>(ws) % kAlign) return fail(HYTOPK_EWORKSPACE, "workspace not 256-byte aligned");
  if (bytes < need) return fail(HYTOPK_EWORKSPACE, "workspace too small");
  return HYTOPK_OK;
}

int check_inputs(const hytopk_problem* p, const void* q, const void* qs, const void* k,
                 const void* ks, const float* w) {
  if (!q || !k || !w) return fail(HYTOPK_EINVAL, "q, k and w must be non-NULL");
  if (p->dtype != HYTOPK_BF16 && (!qs || !ks))
    return fail(HYTOPK_EINVAL, "fp8 and MX formats need q_scale and k_scale");
  auto off = [](const void* x, uintptr_t a) { return reinterpret_cast<uintptr_t>(x) % a != 0; };
  if (off(q, 16) || off(k, 16)) return fail(HYTOPK_EINVAL, "q and k must be 16-byte aligned");
  if (off(w, 4) || off(qs, 4) || off(ks, 4))
    return fail(HYTOPK_EINVAL, "w, q_scale and k_scale must be 4-byte aligned");
  return HYTOPK_OK;
}

// Splits of the key range so that the score launch has enough workgroups.
void splits(int64_t nq, int64_t maxctx, int fmt, int& nsplit, int& split_len) {
  const int64_t gq = hk::score_group_queries(fmt);
  const int64_t groups = (nq + gq - 1) / gq;
  int64_t want = (512 + groups - 1) / groups;
  const int64_t most = std::max<int64_t>(1, (maxctx + 4095) / 4096);
  want = std::max<int64_t>(1, std::min(want, most));
  int64_t len = (maxctx + want - 1) / want;
  len = (len + 127) / 128 * 128;  // whole key tiles
  nsplit = (int)((maxctx + len - 1) / len);
  split_len = (int)len;
}

// Backward workspace: u rows of one chunk of queries, then the sort buffers.
constexpr int64_t kBwdChunkBytes = int64_t(1) << 33;

struct BwdLayout {
  int64_t chunk;
  size_t u, k0, v0, k1, v1, hist, qb, kb, total;
};

BwdLayout bwd_layout(const hytopk_problem* p) {
  BwdLayout l{};
  const int64_t kp = hk::bwd_padded_k(p->k);
  const int64_t row = kp * p->d * 4;  // u bytes per query
  l.chunk = std::max<int64_t>(1, std::min<int64_t>(p->n, kBwdChunkBytes / row));
  const int64_t N = l.chunk * p->k;
  size_t off = 0;
  l.u = off; off = align_up(off + (size_t)(l.chunk * kp) * p->d * 4);
  l.k0 = off; off = align_up(off + (size_t)N * 4);
  l.v0 = off; off = align_up(off + (size_t)N * 4);
  l.k1 = off; off = align_up(off + (size_t)N * 4);
  l.v1 = off; off = align_up(off + (size_t)N * 4);
  l.hist = off; off = align_up(off + hk::bwd_sort_hist_count(N) * 4);
  if (p->dtype != HYTOPK_BF16) {  // q and k as bf16 for the gradient products
    l.qb = off; off = align_up(off + (size_t)p->n * p->H * p->d * 2);
    l.kb = off; off = align_up(off + (size_t)p->L * p->d * 2);
  }
  l.total = off;
  return l;
}

hk::ScoreArgs score_args(const hytopk_problem* p, const void* q, const void* qs, const void* k,
                         const void* ks, const float* w) {
  hk::ScoreArgs a{};
  a.q = static_cast<const uint8_t*>(q);
  a.k = static_cast<const uint8_t*>(k);
  a.w = w;
  a.q_scale = qs;
  a.k_scale = ks;
  a.L = (int)p->L;
  a.q_start = (int)p->q_start;
  a.qpos = p->q_pos;
  a.qfirst = p->q_first;
  a.H = p->H;
  // Debug knob (determinism check): HYTOPK_REVERSE_KEY_WALK=1 makes the
  // scoring kernels walk key tiles from last to first; results must not change.
  const char* rev = std::getenv("HYTOPK_REVERSE_KEY_WALK");
  a.reverse = (rev && rev[0] == '1') ? 1 : 0;
  return a;
}

// Upper bound on the key range queries first..last-1 can see.
int64_t ctx_bound(const hytopk_problem* p, int64_t last) {
  return p->q_pos ? p->L : p->q_start + last;
}

// Score `nq` queries (qlist or q_offset..) into rows, then row top-k: split
// over many workgroups per row when the rows are few and `split` scratch is
// given, else one workgroup per row.
int rows_path(const hytopk_problem* p, const hk::ScoreArgs& base, const int* qlist, int q_offset,
              int nq, int64_t maxctx, float* rows, int32_t* out_idx, float* out_score,
              void* split, hipStream_t s, hk::RowGate gate = hk::RowGate{nullptr, 0, 0}) {
  hk::ScoreArgs a = base;
  a.rows = rows;
  a.row_stride = p->L;
  a.qlist = qlist;
  a.q_offset = q_offset;
  a.nq = nq;
  a.gate = gate;
  splits(nq, maxctx, p->dtype, a.nsplit, a.split_len);
  {
    Span sp("score_rows", s);
    HK_HIP(hk::launch_score(a, p->d, p->dtype, s), "score rows launch");
  }
  Span sp("row_topk", s);
  if (split && nq <= hk::kRowSplitMaxRows) {
    hk::RowSelArgs r{};
    r.rows = rows;
    r.row_stride = p->L;
    r.qlist = qlist;
    r.q_offset = q_offset;
    r.nq = nq;
    r.qpos = p->q_pos;
    r.qfirst = p->q_first;
    r.q_start = (int)p->q_start;
    r.topk = p->k;
    r.L = (int)p->L;
    hk::row_select_chunks(nq, maxctx, p->L, r.nchunk, r.chunk_len);
    r.scratch = split;
    r.out_idx = out_idx;
    r.out_score = out_score;
    r.gate = gate;
    HK_HIP(hk::launch_row_select_split(r, s), "split row top-k launch");
  } else {
    HK_HIP(hk::launch_row_topk(rows, p->L, qlist, q_offset, nq, p->q_pos, p->q_first,
                               (int)p->q_start, p->k, (int)p->L, out_idx, out_score, gate, s),
           "row top-k launch");
  }
  return HYTOPK_OK;
}

// Library-owned workspace of hytopk_select_noalloc: one copy per GPU the
// library runs on, held until the process ends.  Host code never passes the
// array's name to a kernel or a copy (on the host it is a stand-in, not a
// device address); it uses the per-device address hipGetSymbolAddress gives.
std::mutex g_scratch_mu;
std::map<int, void*> g_scratch_ptr;  // device ordinal -> device address of `scratch`

// Device address of this device's `scratch`, looked up on the first call on
// each device (with that device current).
int scratch_address(void** out) {
  int dev = 0;
  HK_HIP(hipGetDevice(&dev), "hipGetDevice");
  std::lock_guard<std::mutex> g(g_scratch_mu);
  auto it = g_scratch_ptr.find(dev);
  if (it != g_scratch_ptr.end()) {
    *out = it->second;
    return HYTOPK_OK;
  }
  void* ptr = nullptr;
  HK_HIP(hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)), "hipGetSymbolAddress(scratch)");
  if (!ptr || reinterpret_cast<uintptr_t>(ptr) % kAlign)
    return fail(HYTOPK_EHIP, "static scratch has no usable device address");
  g_scratch_ptr[dev] = ptr;
  *out = ptr;
  return HYTOPK_OK;
}

}  // namespace

extern "C" {

const char* hytopk_status_string(int status) {
  switch (status) {
    case HYTOPK_OK: return "ok";
    case HYTOPK_EINVAL: return "invalid argument";
    case HYTOPK_EUNSUPPORTED: return "unsupported problem";
    case HYTOPK_EWORKSPACE: return "bad workspace";
    case HYTOPK_EHIP: return "HIP runtime error";
    default: return "unknown status";
  }
}

const char* hytopk_last_error(void) { return g_err.c_str(); }

int hytopk_trace_enable(int on) {
  Tracer& t = tracer();
  std::lock_guard<std::mutex> g(t.mu);
  const int prev = t.on ? 1 : 0;
  t.on = on != 0;
  if (t.on) t.acc.clear();
  return prev;
}

int hytopk_trace_read(hytopk_trace_entry* out, int max) {
  Tracer& t = tracer();
  std::lock_guard<std::mutex> g(t.mu);
  for (TraceRec& r : t.pending) {
    hipError_t e = hipEventSynchronize(r.b);
    if (e != hipSuccess) return hip_fail(e, "trace event sync");
    float ms = 0.f;
    e = hipEventElapsedTime(&ms, r.a, r.b);
    if (e != hipSuccess) return hip_fail(e, "trace elapsed time");
    auto& slot = t.acc[r.name];
    slot.first += 1;
    slot.second += ms;
    t.pool.push_back(r.a);
    t.pool.push_back(r.b);
  }
  t.pending.clear();
  int i = 0;
  for (const auto& kv : t.acc) {
    if (out && i < max) {
      std::memset(out[i].name, 0, sizeof(out[i].name));
      std::strncpy(out[i].name, kv.first.c_str(), sizeof(out[i].name) - 1);
      out[i].launches = kv.second.first;
      out[i].total_ms = kv.second.second;
    }
    ++i;
  }
  return i;
}

size_t hytopk_select_workspace(const hytopk_problem* p, const hytopk_params* prm) {
  if (check_problem(p) != HYTOPK_OK) return 0;
  Params r = resolve(p, prm);
  if (check_params(p, r) != HYTOPK_OK) return 0;
  return layout(p, r).total;
}

size_t hytopk_baseline_workspace(const hytopk_problem* p) {
  if (check_problem(p) != HYTOPK_OK) return 0;
  return (size_t)p->n * (size_t)p->L * 4;
}

}  // extern "C"

namespace {

// The selection.  status == null: the recovery path is chosen on the host
// after one synchronisation (hytopk_select).  status != null: nothing
// synchronises; recovery passes for up to max_recover failures are enqueued
// with device-side row counts, and the device status words tell whether the
// failures exceeded max_recover (hytopk_select_async).
int select_impl(const hytopk_problem* p, const hytopk_params* prm, const void* q,
                const void* q_scale, const void* k, const void* k_scale, const float* w,
                int32_t* out_idx, float* out_score, void* workspace, size_t workspace_bytes,
                void* stream, hytopk_stats* stats, int32_t* status) {
  int rc = check_problem(p);
  if (rc) return rc;
  Params r = resolve(p, prm);
  if ((rc = check_params(p, r))) return rc;
  if ((rc = check_inputs(p, q, q_scale, k, k_scale, w))) return rc;
  if (!out_idx) return fail(HYTOPK_EINVAL, "out_idx is NULL");
  const Layout l = layout(p, r);
  if ((rc = check_ws(workspace, workspace_bytes, l.total))) return rc;

  hipStream_t s = static_cast<hipStream_t>(stream);
  uint8_t* ws = static_cast<uint8_t*>(workspace);
  float* tau = reinterpret_cast<float*>(ws + l.tau);
  int* cnt = reinterpret_cast<int*>(ws + l.cnt);
  int* failed = reinterpret_cast<int*>(ws + l.failed);
  hk::DevStats* dst = reinterpret_cast<hk::DevStats*>(ws + l.stats);
  uint2* cand = reinterpret_cast<uint2*>(ws + l.cand);
  float* rows = reinterpret_cast<float*>(ws + l.rows);
  void* split = split_bytes(p, l.rows_n) ? static_cast<void*>(ws + l.split) : nullptr;
  const int fmt = p->dtype;
  const int n = (int)p->n;
  const int64_t maxctx = ctx_bound(p, p->n);
  const hk::ScoreArgs base = score_args(p, q, q_scale, k, k_scale, w);

  const bool async = status != nullptr;
  hk::DevStats hs{};
  int path = 0;
  if (r.force_path != HYTOPK_PATH_ROWS_ALL || async) {
    HK_HIP(hk::launch_zero(cnt, n, dst, s), "zero launch");
  }
  if (r.force_path != HYTOPK_PATH_ROWS_ALL) {
    hk::SampleArgs sa{};
    sa.q = base.q; sa.k = base.k; sa.w = w; sa.q_scale = q_scale; sa.k_scale = k_scale;
    sa.tau = tau; sa.L = (int)p->L; sa.q_start = (int)p->q_start; sa.n = n; sa.H = p->H;
    sa.qpos = p->q_pos; sa.qfirst = p->q_first;
    sa.topk = p->k; sa.M = sample_count(p, r); sa.oversample = r.oversample;
    {
      Span sp("sample_tau", s);
      HK_HIP(hk::launch_sample_tau(sa, p->d, fmt, s), "sample/threshold launch");
    }

    hk::ScoreArgs a = base;
    a.tau = tau;
    a.cnt = cnt;
    a.cand = cand;
    a.cap = r.cap;
    a.nq = n;
    splits(n, maxctx, p->dtype, a.nsplit, a.split_len);
    {
      Span sp("score_compact", s);
      HK_HIP(hk::launch_score(a, p->d, fmt, s), "fused score launch");
    }
    {
      Span sp("check", s);
      HK_HIP(hk::launch_check(cnt, n, p->q_pos, p->q_first, (int)p->q_start, (int)p->L, p->k,
                              r.cap, dst, failed, s),
             "check launch");
    }
    if (async) {
      path = 3;
    } else {
      HK_HIP(hipMemcpyAsync(&hs, dst, sizeof(hs), hipMemcpyDeviceToHost, s), "stats copy");
      HK_HIP(hipStreamSynchronize(s), "stream sync");
      path = hs.n_failed > r.max_recover ? 1 : 0;
    }
  } else {
    path = 2;
  }

  if (path == 3) {
    // No synchronisation: the candidate select skips the failed queries by
    // itself, and each recovery pass reads the failure count on the device.
    {
      Span sp("cand_select", s);
      HK_HIP(hk::launch_cand_select(cnt, cand, n, p->q_pos, p->q_first, (int)p->q_start, p->k,
                                    r.cap, (int)p->L, out_idx, out_score, s),
             "candidate select launch");
    }
    const int most = std::min(r.max_recover, n);
    for (int f0 = 0; f0 < most; f0 += l.rows_n) {
      const int nf = std::min(l.rows_n, most - f0);
      rc = rows_path(p, base, failed + f0, 0, nf, maxctx, rows, out_idx, out_score, split, s,
                     hk::RowGate{&dst->n_failed, r.max_recover, f0});
      if (rc) return rc;
    }
  } else if (path == 0) {
    {
      Span sp("cand_select", s);
      HK_HIP(hk::launch_cand_select(cnt, cand, n, p->q_pos, p->q_first, (int)p->q_start, p->k,
                                    r.cap, (int)p->L, out_idx, out_score, s),
             "candidate select launch");
    }
    // Recovery: full score rows for the flagged queries only, then row top-k.
    for (int f0 = 0; f0 < hs.n_failed; f0 += l.rows_n) {
      const int nf = std::min(l.rows_n, hs.n_failed - f0);
      rc = rows_path(p, base, failed + f0, 0, nf, maxctx, rows, out_idx, out_score, split, s);
      if (rc) return rc;
    }
  } else {
    // Full rescore: every query through the row path, in chunks of rows_n.
    for (int c0 = 0; c0 < n; c0 += l.rows_n) {
      const int nc = std::min(l.rows_n, n - c0);
      rc = rows_path(p, base, nullptr, c0, nc, ctx_bound(p, c0 + nc), rows, out_idx, out_score,
                     split, s);
      if (rc) return rc;
    }
  }
  if (stats && stats->failed_queries && stats->failed_capacity > 0 && hs.n_failed > 0) {
    const int m = std::min(hs.n_failed, stats->failed_capacity);
    HK_HIP(hipMemcpyAsync(stats->failed_queries, failed, (size_t)m * sizeof(int32_t),
                          hipMemcpyDeviceToHost, s),
           "failed list copy");
    HK_HIP(hipStreamSynchronize(s), "stream sync");
    std::sort(stats->failed_queries, stats->failed_queries + m);
  }
  if (stats) {
    stats->n_overflow = hs.n_overflow;
    stats->n_underk = hs.n_underk;
    stats->n_failed = hs.n_failed;
    stats->full_rescore = path != 0;
    stats->cand_total = (int64_t)hs.cand_total;
    stats->cand_max = hs.cand_max;
    stats->path = path;
  }
  if (async) HK_HIP(hk::launch_async_status(dst, r.max_recover, status, s), "status launch");
  return HYTOPK_OK;
}

}  // namespace

extern "C" {

int hytopk_select(const hytopk_problem* p, const hytopk_params* prm, const void* q,
                  const void* q_scale, const void* k, const void* k_scale, const float* w,
                  int32_t* out_idx, float* out_score, void* workspace, size_t workspace_bytes,
                  void* stream, hytopk_stats* stats) {
  g_err.clear();
  return select_impl(p, prm, q, q_scale, k, k_scale, w, out_idx, out_score, workspace,
                     workspace_bytes, stream, stats, nullptr);
}

int hytopk_select_async(const hytopk_problem* p, const hytopk_params* prm, const void* q,
                        const void* q_scale, const void* k, const void* k_scale, const float* w,
                        int32_t* out_idx, float* out_score, void* workspace,
                        size_t workspace_bytes, void* stream, int32_t* status) {
  g_err.clear();
  if (!status) return fail(HYTOPK_EINVAL, "status is NULL");
  if (reinterpret_cast<uintptr_t>(status) % 4) return fail(HYTOPK_EINVAL, "status must be 4-byte aligned");
  return select_impl(p, prm, q, q_scale, k, k_scale, w, out_idx, out_score, workspace,
                     workspace_bytes, stream, nullptr, status);
}

int hytopk_select_noalloc(const hytopk_problem* p, const hytopk_params* prm, const void* q,
                          const void* q_scale, const void* k, const void* k_scale, const float* w,
                          int32_t* out_idx, float* out_score, void* stream, hytopk_stats* stats) {
  g_err.clear();
  int rc = check_problem(p);
  if (rc) return rc;
  Params r = resolve(p, prm);
  if ((rc = check_params(p, r))) return rc;
  const size_t need = layout(p, r).total;
  if (need > kNoAllocBytes) {
    char msg[160];
    std::snprintf(msg, sizeof msg,
                  "problem needs %zu bytes of workspace, more than the %zu-byte static scratch "
                  "(use hytopk_select with a workspace, or a smaller rows_chunk / cap)",
                  need, kNoAllocBytes);
    return fail(HYTOPK_EWORKSPACE, msg);
  }
  void* ws = nullptr;
  if ((rc = scratch_address(&ws))) return rc;
  return hytopk_select(p, prm, q, q_scale, k, k_scale, w, out_idx, out_score, ws, kNoAllocBytes,
                       stream, stats);
}

int hytopk_replay(const hytopk_problem* p, const void* q, const void* q_scale, const void* k,
                  const void* k_scale, const float* w, const int32_t* idx, float* out_score,
                  void* stream) {
  g_err.clear();
  int rc = check_problem(p);
  if (rc) return rc;
  if ((rc = check_inputs(p, q, q_scale, k, k_scale, w))) return rc;
  if (!idx || !out_score) return fail(HYTOPK_EINVAL, "idx and out_score must be non-NULL");
  hk::ReplayArgs a{};
  a.q = static_cast<const uint8_t*>(q);
  a.k = static_cast<const uint8_t*>(k);
  a.w = w;
  a.q_scale = q_scale;
  a.k_scale = k_scale;
  a.idx = idx;
  a.out = out_score;
  a.L = (int)p->L;
  a.n = (int)p->n;
  a.H = p->H;
  a.topk = p->k;
  hipStream_t s = static_cast<hipStream_t>(stream);
  Span sp("replay", s);
  HK_HIP(hk::launch_replay(a, p->d, p->dtype, s), "replay launch");
  return HYTOPK_OK;
}

int hytopk_baseline_select(const hytopk_problem* p, const void* q, const void* q_scale,
                           const void* k, const void* k_scale, const float* w, int32_t* out_idx,
                           float* out_score, void* workspace, size_t workspace_bytes,
                           void* stream) {
  g_err.clear();
  int rc = check_problem(p);
  if (rc) return rc;
  if ((rc = check_inputs(p, q, q_scale, k, k_scale, w))) return rc;
  if (!out_idx) return fail(HYTOPK_EINVAL, "out_idx is NULL");
  if ((rc = check_ws(workspace, workspace_bytes, hytopk_baseline_workspace(p)))) return rc;
  const hk::ScoreArgs base = score_args(p, q, q_scale, k, k_scale, w);
  return rows_path(p, base, nullptr, 0, (int)p->n, ctx_bound(p, p->n),
                   static_cast<float*>(workspace), out_idx, out_score, nullptr,
                   static_cast<hipStream_t>(stream));
}


size_t hytopk_backward_workspace(const hytopk_problem* p) {
  if (check_problem(p) != HYTOPK_OK) return 0;
  return bwd_layout(p).total;
}

int hytopk_backward(const hytopk_problem* p, const void* q, const void* q_scale, const void* k,
                    const void* k_scale, const float* w, const int32_t* idx,
                    const float* d_score, float* dq, float* dw, float* dk, void* workspace,
                    size_t workspace_bytes, void* stream) {
  g_err.clear();
  int rc = check_problem(p);
  if (rc) return rc;
  if ((rc = check_inputs(p, q, q_scale, k, k_scale, w))) return rc;
  if (!idx || !d_score) return fail(HYTOPK_EINVAL, "idx and d_score must be non-NULL");
  const BwdLayout l = bwd_layout(p);
  const bool scaled = p->dtype != HYTOPK_BF16;
  if ((dk || scaled) && (rc = check_ws(workspace, workspace_bytes, l.total))) return rc;
  hipStream_t s = static_cast<hipStream_t>(stream);
  const int K = p->k, D = p->d;
  char* ws = static_cast<char*>(workspace);
  // Scaled formats: q and k as bf16 (decoded MX values, or FP8 codes whose
  // per-token scales the query kernel applies).
  const uint16_t* qb = static_cast<const uint16_t*>(q);
  const uint16_t* kb = static_cast<const uint16_t*>(k);
  const bool tok = p->dtype == HYTOPK_FP8_E4M3;
  if (scaled) {
    Span sp("bwd_query", s);
    uint16_t* qd = reinterpret_cast<uint16_t*>(ws + l.qb);
    uint16_t* kd = reinterpret_cast<uint16_t*>(ws + l.kb);
    HK_HIP(hk::launch_bwd_dequant(q, tok ? nullptr : q_scale, p->n * p->H, D, p->dtype, qd, s),
           "backward q decode launch");
    HK_HIP(hk::launch_bwd_dequant(k, tok ? nullptr : k_scale, p->L, D, p->dtype, kd, s),
           "backward k decode launch");
    qb = qd;
    kb = kd;
  }
  float* u = dk ? reinterpret_cast<float*>(ws + l.u) : nullptr;
  if (dk) {
    Span sp("bwd_dk", s);
    HK_HIP(hk::launch_fill_zero(dk, p->L * (int64_t)D, s), "dk clear");
  }
  for (int64_t q0 = 0; q0 < p->n; q0 += l.chunk) {
    const int nq = (int)std::min<int64_t>(l.chunk, p->n - q0);
    const uint32_t *sorted_keys = nullptr, *sorted_rows = nullptr;
    if (dk) {
      hk::DkArgs b{};
      b.idx = idx + q0 * K;
      b.L = (int)p->L;
      b.N = nq * K;
      b.topk = K;
      b.k0 = reinterpret_cast<uint32_t*>(ws + l.k0);
      b.v0 = reinterpret_cast<uint32_t*>(ws + l.v0);
      b.k1 = reinterpret_cast<uint32_t*>(ws + l.k1);
      b.v1 = reinterpret_cast<uint32_t*>(ws + l.v1);
      b.hist = reinterpret_cast<uint32_t*>(ws + l.hist);
      Span sp("bwd_dk", s);
      HK_HIP(hk::launch_bwd_sort(b, &sorted_keys, &sorted_rows, s), "backward key sort launch");
    }
    hk::BwdArgs a{};
    a.q = qb;
    a.k = kb;
    a.w = w;
    a.q_scale = tok ? static_cast<const float*>(q_scale) : nullptr;
    a.k_scale = tok ? static_cast<const float*>(k_scale) : nullptr;
    a.idx = idx;
    a.dsc = d_score;
    a.dq = dq;
    a.dw = dw;
    a.u = u;
    a.L = (int)p->L;
    a.H = p->H;
    a.topk = K;
    a.q0 = (int)q0;
    a.nq = nq;
    {
      Span sp("bwd_query", s);
      HK_HIP(hk::launch_bwd_query(a, D, s), "backward query launch");
    }
    if (dk) {
      Span sp("bwd_dk", s);
      HK_HIP(hk::launch_bwd_segments(sorted_keys, sorted_rows, nq * K, (int)p->L, u, dk, q0 > 0,
                                     D, s),
             "backward dk launch");
    }
  }
  return HYTOPK_OK;
}

}  // extern "C"
