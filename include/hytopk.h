/*
 * hytopk.h -- C ABI of the exact top-k indexer selection library for AMD
 * Instinct MI355X (gfx950).
 *
 * Operation (HyScale pages):
 *   * Learned sparse attention rates all of a query's preceding tokens with
 *     an indexer and keeps the k best; done conventionally, the complete
 *     query x key table of scores lands in device memory and a separate
 *     top-k pass loads it again ("HyScale sparse-attention training --
 *     Selection without a score table", contest paragraph).
 *   * HyTopK (also called FlashTopK) returns each query's exact top-k without
 *     that table: a threshold taken from evenly spaced samples of the query's
 *     own context, a fused score-and-compare pass that writes only passing keys
 *     into a bounded candidate buffer, a check for overflow or fewer than k
 *     candidates, recovery of the flagged queries, a full rescore when more
 *     than 64 queries fail, ties at the k-th score resolved by a radix select
 *     over positions, and a radix sort of the kept k (same page, HyTopK
 *     paragraph; the paper's abstract).
 *   * Replay: the k selected indices of each query are saved, and the
 *     recomputation pass scores just those entries again (same page,
 *     selection-replay paragraph).
 *
 * Indexer: I(t,s) = sum_h w[t,h] * ReLU(q[t,h] . k[s]), for key positions
 * s = 0..t (a query sees itself and every earlier key).  Result order: score
 * descending, then position ascending; at equal scores the lower position wins.
 *
 * Conventions for every entry point
 *   * All array arguments are DEVICE pointers to row-major, contiguous data on
 *     the current HIP device, except `stats`, which is a host pointer.  q and
 *     k must be 16-byte aligned (their rows are read in 16-byte pieces), w,
 *     q_scale and k_scale 4-byte aligned; otherwise HYTOPK_EINVAL.
 *   * q is [n][H][d], k is [L][d], in one of four storage formats (dtype):
 *       HYTOPK_BF16        bf16; q_scale = k_scale = NULL;
 *       HYTOPK_FP8_E4M3    OCP FP8 E4M3 bytes with fp32 per-token
 *                          dequantisation scales q_scale[n], k_scale[L] (> 0);
 *       HYTOPK_MXFP8_E4M3  OCP MX: E4M3 bytes, every 32 consecutive elements
 *                          of a row share one E8M0 scale byte (2^(b - 127)):
 *                          q_scale is uint8 [n][H][d/32], k_scale [L][d/32];
 *       HYTOPK_MXFP4_E2M1  OCP MX: E2M1 elements packed two per byte (element
 *                          2i in the low nibble of byte i, rows of d/2 bytes),
 *                          E8M0 scales as for MXFP8.
 *     The scale pointers are `const void*` for that reason.  w is [n][H]
 *     fp32.  Query i sits at position q_start + i and q_start + n <= L unless
 *     the problem's q_pos / q_first arrays say otherwise.
 *   * Index outputs are [n][k] int32, score outputs [n][k] fp32.  When a
 *     query's context ctx = q_start + i + 1 is shorter than k, the entries
 *     beyond ctx hold index -1 and score -inf.
 *   * `stream` is a hipStream_t (NULL = the legacy default stream).  Every
 *     call is ordered on it.  hytopk_select synchronises that stream once (to
 *     read the failure count); replay and baseline are fully asynchronous.
 *   * Ownership: the caller allocates every buffer, including the workspace.
 *     The library allocates no device memory.
 *   * Errors: arguments are validated before any launch, so a negative return
 *     means nothing was launched (HYTOPK_EHIP excepted: a HIP call failed
 *     after launches may have started).  hytopk_last_error() gives text for
 *     the calling thread's most recent failure.
 *   * Supported in this version: 1 <= H <= 64 (heads beyond a multiple of 8
 *     are zero-padded; H <= 8 uses a narrow tile); d in {64, 128} for bf16,
 *     d = 128 for FP8 E4M3 and the MX formats (the backward included);
 *     1 <= k <= 2048; L, n, q_start < 2^31; cap <= 16384 and
 *     m_max <= 16384.  Other shapes return HYTOPK_EUNSUPPORTED.
 */
#ifndef HYTOPK_H_
#define HYTOPK_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  HYTOPK_OK = 0,
  HYTOPK_EINVAL = -1,        /* bad argument: null pointer, bad size, q_start + n > L */
  HYTOPK_EUNSUPPORTED = -2,  /* valid but not implemented (shape, dtype, k) */
  HYTOPK_EWORKSPACE = -3,    /* workspace missing, too small or misaligned (256 B) */
  HYTOPK_EHIP = -4           /* a HIP runtime call failed; see hytopk_last_error() */
} hytopk_status;

typedef enum {
  HYTOPK_BF16 = 0,
  HYTOPK_FP8_E4M3 = 1,    /* per-token fp32 scales */
  HYTOPK_MXFP8_E4M3 = 2,  /* OCP MX block scales, 32 elements per E8M0 scale */
  HYTOPK_MXFP4_E2M1 = 3   /* OCP MX block scales, 32 elements per E8M0 scale */
} hytopk_dtype;

/* Path overrides for testing; results are identical on every path. */
typedef enum {
  HYTOPK_PATH_AUTO = 0,     /* threshold + candidates, recovery or full rescore as the check decides */
  HYTOPK_PATH_ROWS_ALL = 1  /* skip the threshold: score every row, then row top-k (the full rescore) */
} hytopk_path;

/* Problem shape.  By default query i sits at position q_start + i and sees
 * keys 0 .. q_start + i (one causal block at the end of the key buffer).
 * The two optional device arrays generalise that: q_pos[i] gives query i's
 * position (queries in any order, e.g. a context-parallel zigzag shard) and
 * q_first[i] the first key of its context (several sequences packed back to
 * back in one key buffer); query i then sees keys q_first[i] .. q_pos[i].
 * Values are clamped to [0, L); a query whose range is empty gets only
 * padding.  The sample count M is taken from L, the keys of the call; the
 * sample positions and the threshold rank from that query's context alone.
 * Replay and backward take explicit indices and ignore both arrays. */
typedef struct {
  int64_t L;        /* number of keys */
  int64_t n;        /* number of queries (< 2^31) */
  int64_t q_start;  /* position of query 0 when q_pos is NULL (q_start + n <= L; < 2^31) */
  int32_t H;        /* indexer heads */
  int32_t d;        /* head dimension */
  int32_t k;        /* keys kept per query */
  int32_t dtype;    /* hytopk_dtype of q and k */
  const int32_t* q_pos;    /* optional [n] device: query positions; NULL = q_start + i */
  const int32_t* q_first;  /* optional [n] device: first key of each context; NULL = 0 */
} hytopk_problem;

/* Sampled-threshold parameters.  Zero selects the default shown.
 * Sample count M = min(max(m_min, L / m_div), m_max) and the threshold is the
 * ceil(oversample * k * M_q / ctx)-th best of the M_q = min(M, ctx) samples at
 * positions floor(j * ctx / M_q) (HyScale explainer, HyTopK and worked-example
 * paragraphs).  cap is the candidate-buffer capacity per query; a query with
 * more than cap or fewer than min(k, ctx) candidates is recovered; more than
 * max_recover failures trigger the full rescore. */
typedef struct {
  int32_t m_min;        /* 4096 */
  int32_t m_max;        /* 8192 */
  int32_t m_div;        /* 128 */
  int32_t oversample;   /* 3 */
  int32_t cap;          /* 6 * k */
  int32_t max_recover;  /* 64 */
  int32_t force_path;   /* HYTOPK_PATH_AUTO */
  int32_t rows_chunk;   /* rows of the score-row buffer: queries rescored per pass by recovery
                           and the full rescore; min(n, max(1, max_recover)) (L * 4 bytes each) */
} hytopk_params;

/* What one hytopk_select call did (host struct, filled when non-NULL).
 * failed_queries / failed_capacity are inputs: when failed_queries is a host
 * array, it receives the indices of up to failed_capacity queries the check
 * flagged, in ascending order (read during the call's one synchronisation). */
typedef struct {
  int32_t n_overflow;      /* queries with more than cap candidates */
  int32_t n_underk;        /* queries with fewer than min(k, ctx) candidates */
  int32_t n_failed;        /* queries flagged by the check (either reason) */
  int32_t full_rescore;    /* 1 when every query went through the row path */
  int64_t cand_total;      /* candidates over all queries (including beyond cap) */
  int32_t cand_max;        /* largest per-query candidate count */
  int32_t path;            /* 0 candidates (+recovery), 1 full rescore (check), 2 forced rows */
  int32_t* failed_queries; /* in: optional host array for the flagged query indices */
  int32_t failed_capacity; /* in: its length */
  int32_t reserved;
} hytopk_stats;

/* Workspace bytes hytopk_select needs for this problem and parameters
 * (0 on invalid input).  The workspace must be 256-byte aligned. */
size_t hytopk_select_workspace(const hytopk_problem* p, const hytopk_params* prm);

/* Workspace bytes of hytopk_baseline_select: the n x L fp32 score table. */
size_t hytopk_baseline_workspace(const hytopk_problem* p);

/* Exact top-k per query without a score table (HyTopK).
 * out_idx [n][k] int32 receives positions; out_score [n][k] fp32 their scores
 * (may be NULL).  prm may be NULL (all defaults); stats may be NULL. */
int hytopk_select(const hytopk_problem* p, const hytopk_params* prm,
                  const void* q, const void* q_scale, const void* k, const void* k_scale,
                  const float* w, int32_t* out_idx, float* out_score,
                  void* workspace, size_t workspace_bytes, void* stream, hytopk_stats* stats);

/* Bytes of the library's static scratch used by hytopk_select_noalloc. */
#define HYTOPK_NOALLOC_SCRATCH_BYTES (64u << 20)

/* hytopk_select for callers that cannot allocate device memory (tight
 * serving loops, harnesses that forbid allocation):
 * the same arguments and results without the workspace, which is taken from a
 * static device buffer of HYTOPK_NOALLOC_SCRATCH_BYTES owned by the library
 * (one per GPU it runs on, held until the process ends).  The call allocates
 * nothing.  A problem whose hytopk_select_workspace exceeds the buffer
 * returns HYTOPK_EWORKSPACE before any launch (the rows buffer, rows_chunk *
 * L * 4 bytes, and the candidate buffer, n * cap * 8 bytes, dominate; lower
 * rows_chunk or cap to fit).  Every call on a GPU shares that GPU's buffer
 * and leaves its contents behind: calls that overlap on one GPU (on different
 * streams or threads) race and must be serialised by the caller.  Like
 * hytopk_select it synchronises its stream once (to choose the recovery
 * path), so neither entry point can be recorded under stream capture
 * (hytopk_select_async can). */
int hytopk_select_noalloc(const hytopk_problem* p, const hytopk_params* prm,
                          const void* q, const void* q_scale, const void* k, const void* k_scale,
                          const float* w, int32_t* out_idx, float* out_score, void* stream,
                          hytopk_stats* stats);

/* Words of the device status array of hytopk_select_async. */
#define HYTOPK_ASYNC_STATUS_WORDS 8

/* hytopk_select without a host synchronisation, for callers that record the
 * selection in a stream capture (HIP graph) or must not block: the same
 * arguments, workspace included, and the same results, except when more than
 * max_recover queries fail the check (see status[0]).  The threshold, the
 * fused scoring, the check and the candidate select run as in hytopk_select;
 * the recovery of up to max_recover failed queries (HyScale explainer, HyTopK
 * paragraph: the few failed queries are rescored over their whole context)
 * runs as passes enqueued blind, whose kernels read the failure count on the
 * device and do nothing beyond it.  The full rescore, whose length the host
 * cannot know without synchronising, is not enqueued.
 * status: device array of HYTOPK_ASYNC_STATUS_WORDS int32 (4-byte aligned),
 * written on the stream:
 *   [0] 1 when more than max_recover queries failed: the output rows of the
 *       failed queries are then not final (recompute them, e.g. with
 *       hytopk_select); 0 when every output row is the exact top-k,
 *   [1] queries that failed the check, [2] of them with more than cap
 *       candidates, [3] with fewer than min(k, ctx),
 *   [4] the largest candidate count of a query,
 *   [5], [6] the candidate total (low, high 32 bits), [7] 0.
 * With force_path = HYTOPK_PATH_ROWS_ALL every query takes the row path as
 * in hytopk_select (no check runs; status reads 0).  Every device operation
 * of the call is a kernel launch (no memset, copy or synchronisation); keep
 * kernel tracing off while capturing. */
int hytopk_select_async(const hytopk_problem* p, const hytopk_params* prm,
                        const void* q, const void* q_scale, const void* k, const void* k_scale,
                        const float* w, int32_t* out_idx, float* out_score,
                        void* workspace, size_t workspace_bytes, void* stream, int32_t* status);

/* Selection replay: out_score[i][j] = I(q_start + i, idx[i][j]) for the saved
 * indices idx [n][k] int32 (HyScale explainer, selection-replay paragraph).
 * An index outside [0, L) is padding and gives -inf (never dereferenced);
 * indices in (q_start + i, L) are scored although they lie after the query
 * (callers pass indices that selection returned).  The scores are
 * bit-identical to those hytopk_select returns for the same entries. */
int hytopk_replay(const hytopk_problem* p, const void* q, const void* q_scale,
                  const void* k, const void* k_scale, const float* w, const int32_t* idx,
                  float* out_score, void* stream);

/* The conventional route: write the n x L fp32 score table into the
 * workspace, then a row top-k over the table.  Same outputs as
 * hytopk_select. */
int hytopk_baseline_select(const hytopk_problem* p, const void* q, const void* q_scale,
                           const void* k, const void* k_scale, const float* w,
                           int32_t* out_idx, float* out_score,
                           void* workspace, size_t workspace_bytes, void* stream);

/* Workspace bytes of hytopk_backward (0 on invalid input): the dk rows of one
 * chunk of queries plus the buffers that group them by key (and, for FP8 and
 * MX inputs, q and k as bf16: (n * H + L) * d * 2 bytes).  The chunk size
 * depends only on the problem (up to 8 GiB of rows, d * 4 bytes per entry
 * with k padded to an even number of 32-key tiles), so results do not depend
 * on the workspace a caller passes. */
size_t hytopk_backward_workspace(const hytopk_problem* p);

/* Indexer backward at the replayed entries (HyScale explainer, key-observation
 * paragraph: the indexer's loss depends only on the scores of the selected
 * entries, and the top-k choice itself carries no gradient).  With d_score [n][k] fp32
 * the upstream gradient of the replayed scores I(q_start + i, idx[i][j]),
 * c = q[i][h] . k[idx[i][j]] and ReLU'(c) = [c > 0] (0 at c == 0):
 *   dw [n][H]    fp32: dw[i][h]    = sum_j d_score[i][j] * max(c, 0)
 *   dq [n][H][d] fp32: dq[i][h][:] = w[i][h] * sum_j d_score[i][j] [c > 0] k[idx[i][j]][:]
 *   dk [L][d]    fp32: dk[s][:]    = sum over entries with idx[i][j] = s of
 *                                    sum_h d_score[i][j] w[i][h] [c > 0] q[i][h][:]
 * Every output is fully written (dk is 0 for keys no query selected); any of
 * dq, dw, dk may be NULL to skip it (dk NULL skips the workspace traffic).
 * Indices outside [0, L) are padding and contribute nothing.  dk is summed in
 * a fixed order (query ascending, then slot), so results are bitwise
 * reproducible.  Products use bf16 MFMA with every fp32 factor split into two
 * bf16 parts (16 significant bits) and fp32 accumulation.  FP8 and MX inputs
 * are differentiated with respect to their decoded values (code times scale;
 * dq and dk are gradients of those values): MX q and k are decoded to bf16
 * (exact), FP8 codes are taken as bf16 with the per-token scales applied as
 * factors; for these formats the workspace is required whether or not dk is
 * asked for. */
int hytopk_backward(const hytopk_problem* p, const void* q, const void* q_scale,
                    const void* k, const void* k_scale, const float* w, const int32_t* idx,
                    const float* d_score, float* dq, float* dw, float* dk,
                    void* workspace, size_t workspace_bytes, void* stream);

const char* hytopk_status_string(int status);
const char* hytopk_last_error(void);  /* thread-local; "" when none */

/* Debug knob (environment, read on every call): HYTOPK_REVERSE_KEY_WALK=1
 * makes the scoring kernels of hytopk_select and hytopk_baseline_select walk
 * each query group's key tiles from the last to the first.  Candidates then
 * reach the buffer in a different order; the results are bitwise identical
 * (selection depends only on the candidate multiset). */

/* Kernel tracing.  While enabled, every launch the library makes is bracketed
 * by a pair of hipEvents recorded on the caller's stream, and the elapsed time
 * is accumulated per phase name ("sample_tau", "score_compact", "check",
 * "cand_select", "score_rows", "row_topk", "replay", "bwd_query", "bwd_dk").  Process-wide; not for
 * use with concurrent calls on different streams. */
typedef struct {
  char name[32];
  int32_t launches;
  double total_ms;
} hytopk_trace_entry;

/* Enable (1) or disable (0) tracing; enabling clears the accumulators.
 * Returns the previous state. */
int hytopk_trace_enable(int on);

/* Waits for the recorded events, then copies up to `max` accumulated entries
 * (host array) and returns how many phases exist (negative on a HIP error). */
int hytopk_trace_read(hytopk_trace_entry* out, int max);

#ifdef __cplusplus
}
#endif

#endif /* HYTOPK_H_ */
