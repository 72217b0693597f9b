// Host-side exercise of the C ABI's argument validation and workspace
// arithmetic, built with AddressSanitizer and UndefinedBehaviorSanitizer on
// the host code (the device code is unchanged).  Every call here must be
// rejected (or sized) before any HIP call, so it runs without a GPU.
// Exit status 0 when every expectation holds.
#include <cstdint>
#include <cstdio>
#include <cstring>

#include "hytopk.h"

static int failures = 0;

static void expect(bool ok, const char* what) {
  if (!ok) {
    std::printf("FAIL: %s (last error: %s)\n", what, hytopk_last_error());
    ++failures;
  }
}

static hytopk_problem base() {
  hytopk_problem p;
  std::memset(&p, 0, sizeof p);
  p.L = int64_t(1) << 20;
  p.n = 8192;
  p.q_start = p.L - p.n;
  p.H = 64;
  p.d = 128;
  p.k = 2048;
  p.dtype = HYTOPK_BF16;
  return p;
}

int main() {
  void* fake = reinterpret_cast<void*>(uintptr_t(0x1000));
  const float* fw = static_cast<const float*>(fake);
  int32_t* fi = static_cast<int32_t*>(fake);
  float* ff = static_cast<float*>(fake);

  // sizes of the worked example's shard
  hytopk_problem p = base();
  expect(hytopk_baseline_workspace(&p) == (size_t(32) << 30), "32 GiB score table");
  const size_t ws = hytopk_select_workspace(&p, nullptr);
  expect(ws > 0 && ws % 256 == 0 && ws < (size_t(11) << 27), "select workspace ~1.06 GiB");
  expect(hytopk_backward_workspace(&p) >= (size_t(8) << 30), "backward workspace");

  // invalid problems: every size query returns 0, every call an error
  struct Case { const char* name; void (*mut)(hytopk_problem&); int code; };
  const Case cases[] = {
      {"n = 0", [](hytopk_problem& q) { q.n = 0; }, HYTOPK_EINVAL},
      {"L = 0", [](hytopk_problem& q) { q.L = 0; }, HYTOPK_EINVAL},
      {"q_start < 0", [](hytopk_problem& q) { q.q_start = -1; }, HYTOPK_EINVAL},
      {"q_start + n > L", [](hytopk_problem& q) { q.q_start += 1; }, HYTOPK_EINVAL},
      {"k = 0", [](hytopk_problem& q) { q.k = 0; }, HYTOPK_EINVAL},
      {"k > 2048", [](hytopk_problem& q) { q.k = 2049; }, HYTOPK_EUNSUPPORTED},
      {"H = 65", [](hytopk_problem& q) { q.H = 65; }, HYTOPK_EUNSUPPORTED},
      {"H = 0", [](hytopk_problem& q) { q.H = 0; }, HYTOPK_EINVAL},
      {"d = 96", [](hytopk_problem& q) { q.d = 96; }, HYTOPK_EUNSUPPORTED},
      {"fp8 with d = 64", [](hytopk_problem& q) { q.dtype = HYTOPK_FP8_E4M3; q.d = 64; }, HYTOPK_EUNSUPPORTED},
      {"unknown dtype", [](hytopk_problem& q) { q.dtype = 9; }, HYTOPK_EINVAL},
      {"L >= 2^31", [](hytopk_problem& q) { q.L = int64_t(1) << 31; q.q_start = q.L - q.n; }, HYTOPK_EUNSUPPORTED},
      {"n >= 2^31", [](hytopk_problem& q) { q.n = int64_t(1) << 31; q.L = (int64_t(1) << 31) - 1; q.q_start = 0;
                                             q.q_pos = reinterpret_cast<const int32_t*>(uintptr_t(0x1000)); }, HYTOPK_EUNSUPPORTED},
      {"q_start >= 2^31", [](hytopk_problem& q) { q.q_start = int64_t(1) << 31;
                                                  q.q_pos = reinterpret_cast<const int32_t*>(uintptr_t(0x1000)); }, HYTOPK_EUNSUPPORTED},
  };
  for (const Case& c : cases) {
    hytopk_problem q = base();
    c.mut(q);
    char what[160];
    std::snprintf(what, sizeof what, "%s: sizes 0", c.name);
    expect(hytopk_select_workspace(&q, nullptr) == 0 && hytopk_baseline_workspace(&q) == 0 &&
               hytopk_backward_workspace(&q) == 0, what);
    std::snprintf(what, sizeof what, "%s: select", c.name);
    expect(hytopk_select(&q, nullptr, fake, fake, fake, fake, fw, fi, ff, fake, ~size_t(0), nullptr,
                         nullptr) == c.code, what);
    std::snprintf(what, sizeof what, "%s: select_noalloc", c.name);
    expect(hytopk_select_noalloc(&q, nullptr, fake, fake, fake, fake, fw, fi, ff, nullptr, nullptr) ==
               c.code, what);
    std::snprintf(what, sizeof what, "%s: replay", c.name);
    expect(hytopk_replay(&q, fake, fake, fake, fake, fw, fi, ff, nullptr) == c.code, what);
    std::snprintf(what, sizeof what, "%s: baseline", c.name);
    expect(hytopk_baseline_select(&q, fake, fake, fake, fake, fw, fi, ff, fake, ~size_t(0), nullptr) ==
               c.code, what);
    std::snprintf(what, sizeof what, "%s: backward", c.name);
    expect(hytopk_backward(&q, fake, fake, fake, fake, fw, fi, fw, ff, ff, ff, fake, ~size_t(0), nullptr) ==
               c.code, what);
    expect(std::strlen(hytopk_last_error()) > 0, "an error message is set");
  }
  expect(hytopk_select_workspace(nullptr, nullptr) == 0, "NULL problem");
  expect(hytopk_select(nullptr, nullptr, fake, nullptr, fake, nullptr, fw, fi, ff, fake, 1, nullptr,
                       nullptr) == HYTOPK_EINVAL, "NULL problem: select");

  // invalid parameters
  struct PCase { const char* name; hytopk_params prm; };
  hytopk_params z;
  std::memset(&z, 0, sizeof z);
  PCase pcases[8];
  for (auto& c : pcases) c.prm = z;
  pcases[0].name = "cap > 16384";        pcases[0].prm.cap = 16385;
  pcases[1].name = "m_max > 16384";      pcases[1].prm.m_max = 1 << 15;
  pcases[2].name = "force_path 5";       pcases[2].prm.force_path = 5;
  pcases[3].name = "oversample < 0";     pcases[3].prm.oversample = -1;
  pcases[4].name = "m_max < m_min";      pcases[4].prm.m_min = 8000; pcases[4].prm.m_max = 4000;
  pcases[5].name = "rows_chunk < 0";     pcases[5].prm.rows_chunk = -3;
  pcases[6].name = "max_recover < 0";    pcases[6].prm.max_recover = -1;
  pcases[7].name = "m_div < 0";          pcases[7].prm.m_div = -5;
  for (const PCase& c : pcases) {
    char what[160];
    std::snprintf(what, sizeof what, "params %s", c.name);
    expect(hytopk_select_workspace(&p, &c.prm) == 0, what);
    expect(hytopk_select(&p, &c.prm, fake, nullptr, fake, nullptr, fw, fi, ff, fake, ~size_t(0), nullptr,
                         nullptr) < 0, what);
  }
  // a rows buffer whose size would approach the size_t range is refused
  {
    hytopk_problem q = base();
    q.L = (int64_t(1) << 31) - 1;
    q.n = (int64_t(1) << 31) - 1;
    q.q_start = 0;
    q.q_pos = fi;
    q.k = 8;
    hytopk_params prm = z;
    prm.rows_chunk = 0x7FFFFFFF;
    expect(hytopk_select_workspace(&q, &prm) == 0, "rows_chunk * L overflow guard");
    prm.rows_chunk = 4;
    const size_t w = hytopk_select_workspace(&q, &prm);
    expect(w > size_t(4) * size_t(q.L) * 4 && w % 256 == 0, "huge problem, small rows buffer sized");
  }

  // pointer and workspace errors, all before any launch
  expect(hytopk_select(&p, nullptr, nullptr, nullptr, fake, nullptr, fw, fi, ff, fake, ~size_t(0), nullptr,
                       nullptr) == HYTOPK_EINVAL, "NULL q");
  expect(hytopk_select(&p, nullptr, fake, nullptr, fake, nullptr, fw, nullptr, ff, fake, ~size_t(0), nullptr,
                       nullptr) == HYTOPK_EINVAL, "NULL out_idx");
  expect(hytopk_select(&p, nullptr, fake, nullptr, fake, nullptr, fw, fi, ff, nullptr, ~size_t(0), nullptr,
                       nullptr) == HYTOPK_EWORKSPACE, "NULL workspace");
  expect(hytopk_select(&p, nullptr, fake, nullptr, fake, nullptr, fw, fi, ff, fake, ws - 1, nullptr,
                       nullptr) == HYTOPK_EWORKSPACE, "workspace one byte short");
  expect(hytopk_select(&p, nullptr, fake, nullptr, fake, nullptr, fw, fi, ff,
                       reinterpret_cast<void*>(uintptr_t(0x1080)), ~size_t(0), nullptr,
                       nullptr) == HYTOPK_EWORKSPACE, "misaligned workspace");
  expect(hytopk_baseline_select(&p, fake, nullptr, fake, nullptr, fw, fi, ff, fake, (size_t(32) << 30) - 1,
                                nullptr) == HYTOPK_EWORKSPACE, "baseline table one byte short");
  hytopk_problem p8 = base();
  p8.dtype = HYTOPK_FP8_E4M3;
  expect(hytopk_replay(&p8, fake, nullptr, fake, nullptr, fw, fi, ff, nullptr) == HYTOPK_EINVAL,
         "fp8 without scales");
  expect(hytopk_backward(&p, fake, nullptr, fake, nullptr, fw, nullptr, fw, ff, ff, ff, fake, ~size_t(0),
                         nullptr) == HYTOPK_EINVAL, "backward without idx");
  expect(hytopk_backward(&p, fake, nullptr, fake, nullptr, fw, fi, fw, ff, ff, ff, fake, 16, nullptr) ==
             HYTOPK_EWORKSPACE, "backward workspace too small");
  // the allocation-free entry point refuses problems beyond its static scratch
  expect(hytopk_select_noalloc(&p, nullptr, fake, nullptr, fake, nullptr, fw, fi, ff, nullptr, nullptr) ==
             HYTOPK_EWORKSPACE, "noalloc beyond the static scratch");
  // the asynchronous select: status array required, workspace checked first
  int32_t* fst = static_cast<int32_t*>(fake);
  expect(hytopk_select_async(&p, nullptr, fake, nullptr, fake, nullptr, fw, fi, ff, fake, ~size_t(0),
                             nullptr, nullptr) == HYTOPK_EINVAL, "async without status");
  expect(hytopk_select_async(&p, nullptr, fake, nullptr, fake, nullptr, fw, fi, ff, fake, 16, nullptr,
                             fst) == HYTOPK_EWORKSPACE, "async workspace too small");
  // status strings
  for (int s = -5; s <= 0; ++s) expect(hytopk_status_string(s) != nullptr, "status string");
  // tracing toggles without a device
  expect(hytopk_trace_enable(1) == 0 && hytopk_trace_enable(0) == 1, "trace toggle");

  std::printf("%s: %d failure(s)\n", failures ? "FAILED" : "ok", failures);
  return failures ? 1 : 0;
}
