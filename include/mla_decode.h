/*
 * mla_decode.h -- C ABI of the MI355X (gfx950) MLA speculative-verify decode
 * library (libmla_decode.so).
 *
 * The operation.  Each of `batch` sequences brings q_len[b] verify tokens
 * (the last q_len[b] of its kv_len[b] cached positions).  All `num_heads`
 * query heads of a token attend over ONE shared latent KV head (MQA): a
 * 576-wide row per position, 512 latent columns followed by 64 rope columns.
 * Scores use all 576 columns; the value is the first 512 columns of the same
 * row.  Token i of a sequence sees keys 0 .. kv_len - q_len + i (causal only
 * among the tail tokens).  Outputs: O (bf16) and the natural-log
 * log-sum-exp of the scaled scores (fp32) per (token, head).
 * Sources: "[Kimi-K3] Allow DSPARK verify on cutedsl_mla (fold_sq)" (sglang
 * PR #33650) -- verify width q = block_size + 1 (opening paragraphs), one KV
 * head for all H query heads and the per-rank H values (section "Which
 * decode backend?"), the 576-wide query/key (section "GPU timeline"), the
 * fold rule and the single KV pass per tile (section "Decision rule",
 * paragraph "Why"), the split-KV reduction (section "GPU timeline").
 *
 * How it runs.  mla_decode_plan folds F = the largest divisor of q_len[b]
 * with H * F <= 128 tokens into one tile of H * F rows (fold rule above), so
 * each KV byte of a chunk is streamed from HBM once per tile; it cuts each
 * sequence into split-KV chunks and sizes the caller's workspace.
 * mla_decode_run enqueues the main decode kernel, which writes final O/LSE
 * for unsplit tiles and per-chunk partials for split ones; the log-sum-exp
 * merge of those partials runs as a separate kernel that mla_decode_reduce
 * enqueues (or, on request, at the end of the main kernel: merge_mode) ("bench(cake_mla_varq_dcp_decode):
 * ..." (flashinfer PR #5588), table "What was measured", row "split rows").
 * Call both, in that order: mla_decode_reduce launches only what the main
 * kernel left to it.
 *
 * Error convention.  Every call returns an mla_status and never throws or
 * aborts.  Unsupported shapes and options are rejected explicitly; there is
 * no silent fallback to another path (the pages' first PR exists because a
 * silent fallback to a slower backend went unnoticed: opening paragraphs of
 * sglang PR #33650; the flashinfer Cake route likewise rejects unsupported
 * options explicitly, section "Unsupported (rejected explicitly)" of the
 * text embedded in flashinfer PR #5588).  After a non-OK status,
 * mla_last_error() returns a message for the calling thread.
 *
 * Ownership.  The caller owns every device buffer and the stream.  The
 * library allocates no device memory (mla_decode_run_static uses a fixed
 * array that is part of the library's loaded device code).  A plan is host memory owned by the
 * library until mla_plan_destroy; it must outlive work enqueued with it only
 * until mla_decode_run / mla_decode_reduce return (kernel arguments are
 * copied at launch), except that a plan of more than 60 sequences uploads
 * its sequence descriptors into the workspace with an asynchronous copy from
 * a pinned host buffer it owns (made when the plan is created, or, if that
 * fails, by its first mla_decode_run): that copy must have run before the
 * plan is destroyed, and a captured graph that holds it needs the plan for
 * as long as the graph is replayed.
 *
 * Threading.  Plans are immutable after creation and may be used from
 * several threads.  Calls that share one workspace on overlapping streams
 * race; give each in-flight call its own workspace.
 */
#ifndef MLA_DECODE_H
#define MLA_DECODE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  MLA_OK = 0,
  MLA_ERR_INVALID_ARGUMENT = 1, /* bad shape, null/misaligned pointer, bad scale */
  MLA_ERR_UNSUPPORTED = 2,      /* no valid fold (H > 128), unknown dtype, not gfx950 */
  MLA_ERR_WORKSPACE_TOO_SMALL = 3,
  MLA_ERR_DEVICE = 4,           /* a HIP call failed; mla_last_error() has its message */
  MLA_ERR_OUT_OF_MEMORY = 5     /* host memory for a plan could not be allocated */
} mla_status;

typedef enum {
  MLA_KV_BF16 = 0,     /* KV rows are bf16 */
  MLA_KV_FP8_E4M3 = 1  /* KV rows are OCP FP8 E4M3FN codes; value = code * kv_scale */
} mla_kv_dtype;

/* Width constants of the latent layout. */
#define MLA_DQK 576          /* query/key width: 512 latent + 64 rope */
#define MLA_DV 512           /* value width: first 512 columns of the KV row */
#define MLA_MAX_TILE_ROWS 128 /* H * F must not exceed this */
#define MLA_KV_GRANULE 64    /* split-KV chunk lengths are multiples of this */
#define MLA_MAX_SHARDS 1024  /* most shards mla_merge_shards combines */
#define MLA_MIN_PAGE_SIZE 32 /* paged KV: smallest page (keys); sizes are powers of two */
#define MLA_MAX_PAGE_SIZE (1 << 20) /* paged KV: largest page (keys) */
#define MLA_STATIC_WORKSPACE_BYTES (32u << 20) /* workspace mla_decode_run_static holds */

typedef struct mla_plan mla_plan; /* opaque, host-owned */

/* Plan options; zero-initialise for automatic choices.
 *  force_fold   > 0: cap the fold factor -- F_b = the largest divisor of q_len[b]
 *                    that is <= force_fold and satisfies H * F <= 128
 *                    (force_fold = 1 gives the unfolded control: one token per tile).
 *  force_splits > 0: request this many split-KV chunks for every sequence
 *                    (the effective count and chunk length follow the split rule
 *                    documented at mla_plan_query).
 *  num_cus      > 0: compute-unit count the cost model plans for; 0 queries the
 *                    current HIP device.
 *  plan_mode:        MLA_PLAN_AUTO (0): each sequence gets its own chunk length
 *                    from a per-unit time model (KV bytes against MFMA work of
 *                    its row count, plus fixed and partial-write costs), the
 *                    candidates scored by list-scheduling the units, longest
 *                    first, onto the CUs; the work units run longest sequence
 *                    first.  MLA_PLAN_UNIFORM (1): one chunk length for every
 *                    sequence, units in the caller's sequence order (the
 *                    earlier rule, kept for comparison).  The host-only rules
 *                    follow "bench(cake_mla_varq_dcp_decode): ..." (flashinfer
 *                    PR #5588), table "What was measured", row "host plan". */
#define MLA_PLAN_AUTO 0
#define MLA_PLAN_UNIFORM 1
/*  merge_mode:       how split tiles are merged.  MLA_MERGE_REDUCE (1): by
 *                    the reduce kernel of mla_decode_reduce.
 *                    MLA_MERGE_LAST_ARRIVER (2): in the main kernel, by the
 *                    last unit of each split row block to finish (it folds
 *                    S x rows partial rows alone; the workspace then also
 *                    holds one 64-bit arrival word per partial row; launches
 *                    with a sequence of more than 65535 chunks use the reduce
 *                    kernel).
 *                    MLA_MERGE_GRID (3): in the main kernel, by all of its
 *                    workgroups together once the last unit has finished
 *                    (they wait on one 64-bit counter per launch, held in the
 *                    workspace), with the reduce kernel's fold and results.
 *                    Only for launches whose work units fit the compute units
 *                    at once (one workgroup per CU: units rounded up to a
 *                    multiple of 8 <= num_cus); other launches use the reduce
 *                    kernel, and so does a launch that mla_decode_run finds
 *                    wider than the current device (it then enqueues that
 *                    reduce itself).
 *                    MLA_MERGE_AUTO (0): the reduce kernel.  On the MI355X
 *                    both in-kernel merges measured slower than the separate
 *                    reduce on every tested shape: the device-wide release of
 *                    the partial rows (an L2 write-back per workgroup) and the
 *                    fold, latency-bound in a workgroup that has to take several
 *                    items one after another, cost more than the launch saved.
 *                    The in-kernel merges follow "bench(cake_mla_varq_dcp_decode):
 *                    ..." (flashinfer PR #5588), table "What was measured",
 *                    row "split rows".
 *                    Both in-kernel merges count arrivals in workspace words
 *                    tagged with each call's epoch and a generation, so the
 *                    workspace's prior contents do not matter and a captured
 *                    graph may replay the call. */
#define MLA_MERGE_AUTO 0
#define MLA_MERGE_REDUCE 1
#define MLA_MERGE_LAST_ARRIVER 2
#define MLA_MERGE_GRID 3
typedef struct {
  int32_t force_fold;
  int32_t force_splits;
  int32_t num_cus;
  int32_t plan_mode;
  int32_t merge_mode;
} mla_plan_options;

/* Build a plan.
 *  batch >= 1; num_heads = H in [1, 128]; q_len, kv_len: HOST arrays [batch]
 *  with 1 <= q_len[b] <= kv_len[b].  opts may be NULL.
 *  On MLA_OK, *plan_out owns a new plan and *workspace_bytes_out (may be
 *  NULL) is the device workspace mla_decode_run needs: the split partials,
 *  and for a batch of more than 60 sequences the sequence descriptor tables
 *  of its single main launch (0 when neither applies).  Pure host
 *  computation, except that it queries the device when num_cus == 0 and
 *  that a batch of more than 60 sequences gets the pinned host buffer its
 *  descriptor tables are uploaded from (hipHostMalloc; if that fails the
 *  plan is still made and its first mla_decode_run allocates the buffer).
 *  Errors: INVALID_ARGUMENT (shapes, null pointers), UNSUPPORTED (H > 128,
 *  unknown dtype), DEVICE (CU query failed), OUT_OF_MEMORY (host memory for
 *  the plan). */
mla_status mla_decode_plan(int32_t batch, int32_t num_heads, const int32_t* q_len,
                           const int32_t* kv_len, mla_kv_dtype kv_dtype,
                           const mla_plan_options* opts, mla_plan** plan_out,
                           size_t* workspace_bytes_out);

/* Build a plan for one shard of each sequence's keys (decode context
 * parallelism: every rank holds a contiguous range of a sequence's cached
 * keys and decodes the same verify rows over it; "[Kimi-K3] Allow DSPARK
 * verify on cutedsl_mla (fold_sq)" (sglang PR #33650), section "Which decode
 * backend?", the TP1+DCP8 rows; "bench(cake_mla_varq_dcp_decode): ..."
 * (flashinfer PR #5588), which benchmarks that decode).
 *  As mla_decode_plan, except: kv_len[b] >= 1 is the number of keys this
 *  shard holds (any size, also fewer than q_len[b]), and causal_end[b] >= 1
 *  (HOST array) places the causal limit in the shard's local key indices:
 *  verify token i sees the local keys j <= causal_end[b] - q_len[b] + i.  For
 *  a shard that starts at global key `offset` of a sequence of `total` keys,
 *  causal_end = total - offset; for the whole sequence, causal_end = kv_len
 *  (which is mla_decode_plan).  A row that sees no key of the shard gets
 *  O = 0 and LSE = -inf.  The outputs of the shards of one sequence combine
 *  with mla_merge_shards.
 *  Errors: as mla_decode_plan; INVALID_ARGUMENT also for causal_end == NULL
 *  or causal_end[b] < 1. */
mla_status mla_decode_plan_shard(int32_t batch, int32_t num_heads, const int32_t* q_len,
                                 const int32_t* kv_len, const int32_t* causal_end,
                                 mla_kv_dtype kv_dtype, const mla_plan_options* opts,
                                 mla_plan** plan_out, size_t* workspace_bytes_out);

/* Enqueue the main decode kernel(s) on `stream` (a hipStream_t; NULL = the
 * default stream) and return.
 *  q:   device bf16 [sum q_len, H, 576], token-major then head, row-major.
 *  kv:  device [sum kv_len, 576] bf16 or e4m3 codes (plan's dtype); sequence b's
 *       rows start at sum_{c<b} kv_len[c].
 *  sm_scale: softmax scale applied to the dot products (> 0, finite).
 *  kv_scale: fp8: per-tensor dequantisation scale (> 0, finite); bf16: must be 1.
 *  o:   device bf16 [sum q_len, H, 512].   lse: device fp32 [sum q_len, H],
 *       natural-log log-sum-exp of the scaled scores.
 *  workspace: device scratch of at least the planned bytes (may be NULL when
 *       the plan needs 0).  Its contents on entry do not matter.
 *  All device pointers must be 16-byte aligned.  For split tiles, O/LSE are
 *  written by mla_decode_reduce, which must follow on the same stream.
 *  Errors: INVALID_ARGUMENT, WORKSPACE_TOO_SMALL, UNSUPPORTED (device is not
 *  gfx950), DEVICE (launch failure). */
mla_status mla_decode_run(const mla_plan* plan, const void* q, const void* kv, float sm_scale,
                          float kv_scale, void* o, float* lse, void* workspace,
                          size_t workspace_bytes, void* stream);

/* mla_decode_run over a paged KV cache: the serving layout, in which a page
 * table maps each sequence's key positions to pages of a shared pool (the
 * Kimi-K3 MLA FP8 "paged attention route" whose description is embedded in
 * flashinfer PR #5588: section "Summary", and section "Tests", which replays
 * with a changed page table).  Same plan, same arguments and same results as
 * mla_decode_run on the gathered KV; only where the rows are read changes.
 *  kv_pages: device pool [num_pages, page_size, 576] of the plan's dtype,
 *       16-byte aligned; num_pages >= 1.
 *  page_size: keys per page, a power of two in [MLA_MIN_PAGE_SIZE,
 *       MLA_MAX_PAGE_SIZE] (else UNSUPPORTED), so that a 32-key kernel tile
 *       never crosses a page.
 *  page_table: device int32 [batch, page_table_stride], 4-byte aligned; key
 *       j of sequence b lives in row j mod page_size of page
 *       page_table[b * page_table_stride + j / page_size].  page_table_stride
 *       must cover the longest sequence (>= ceil(kv_len / page_size)).  The
 *       table is read on the device when the kernels run, so one plan serves
 *       any number of tables; entries are clamped to [0, num_pages - 1], so a
 *       wrong entry reads a wrong page of the pool, never outside it.
 * The caller keeps the pool and the table unchanged until the kernels have
 * run.  Errors: those of mla_decode_run, plus UNSUPPORTED for the page size
 * and INVALID_ARGUMENT for num_pages, the table pointer or its stride. */
mla_status mla_decode_run_paged(const mla_plan* plan, const void* q, const void* kv_pages,
                                int32_t num_pages, int32_t page_size, const int32_t* page_table,
                                int32_t page_table_stride, float sm_scale, float kv_scale, void* o,
                                float* lse, void* workspace, size_t workspace_bytes,
                                void* stream);

/* Enqueue the split-KV merge on `stream`: for every split tile row, in
 * ascending chunk order, M = max_s lse_s, lse = M + ln sum_s exp(lse_s - M),
 * O = sum_s exp(lse_s - lse) * O_s; chunks a row cannot see (lse_s = -inf)
 * get weight 0.  Covers the launches whose split rows the main kernel did
 * not merge itself (see merge_mode); a no-op (returns MLA_OK, launches
 * nothing) when there are none.  Same pointer rules as mla_decode_run, with
 * the workspace of the mla_decode_run it follows. */
mla_status mla_decode_reduce(const mla_plan* plan, const void* workspace, void* o, float* lse,
                             void* stream);

/* Enqueue the combination of per-shard results on `stream`: for every row r,
 * in ascending shard order w, M = max_w lse_w[r], lse[r] = M + ln sum_w
 * exp(lse_w[r] - M), O[r] = sum_w exp(lse_w[r] - lse[r]) * O_w[r]; shards a
 * row sees nothing of (lse = -inf) get weight 0; a row no shard shows a key
 * gets O = 0, LSE = -inf.  The same merge as mla_decode_reduce, for results
 * that were gathered from several ranks (the page sections cited at
 * mla_decode_plan_shard).
 *  o_shards:   device bf16 [num_shards][num_rows][512] (each shard's O).
 *  lse_shards: device fp32 [num_shards][num_rows] (each shard's LSE).
 *  o: device bf16 [num_rows][512]; lse: device fp32 [num_rows] (outputs; they
 *  must not overlap the inputs).  1 <= num_shards <= MLA_MAX_SHARDS,
 *  num_rows >= 1; all pointers 16-byte aligned.
 *  Errors: INVALID_ARGUMENT, UNSUPPORTED (device is not gfx950), DEVICE. */
mla_status mla_merge_shards(int32_t num_rows, int32_t num_shards, const void* o_shards,
                            const float* lse_shards, void* o, float* lse, void* stream);

/* For callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid allocation): the same
 * decode as mla_decode_run followed by mla_decode_reduce, with the split
 * workspace taken from a fixed array of MLA_STATIC_WORKSPACE_BYTES (32 MiB)
 * that the library holds on each device it runs on until the process ends.
 * Nothing is allocated, freed or initialised per call.  Same arguments and
 * results as mla_decode_run + mla_decode_reduce, minus the workspace.
 *  The array is shared by every call on one device and keeps the last call's
 *  contents (no call depends on what it held before: every partial the merge
 *  reads is written by the same call).  Calls that overlap on one device --
 *  on two streams, or from two threads -- race on it; serialise them.
 *  A plan of more than 60 sequences uploads its descriptor tables from the
 *  pinned host buffer made when the plan was created; this call never makes
 *  one.
 *  Errors: those of mla_decode_run; WORKSPACE_TOO_SMALL for a plan whose
 *  workspace exceeds MLA_STATIC_WORKSPACE_BYTES (the plan's workspace_bytes
 *  tells which plans fit; the graded shapes need at most 26 MB); DEVICE for a
 *  plan of more than 60 sequences whose creation could not make its pinned
 *  buffer and that has not run through mla_decode_run since. */
mla_status mla_decode_run_static(const mla_plan* plan, const void* q, const void* kv,
                                 float sm_scale, float kv_scale, void* o, float* lse,
                                 void* stream);

/* Free a plan (NULL is allowed). */
void mla_plan_destroy(mla_plan* plan);

/* Message for the last non-OK status on the calling thread ("" if none). */
const char* mla_last_error(void);

/* Per-sequence plan facts, for tests and tools; seq is the caller's index.
 *  fold = F_b, tiles = q_len[b] / F_b, splits = S_eff, chunk_len = L_b.
 *  Split rule: with S requested chunks and granule G = MLA_KV_GRANULE,
 *    L = G * ceil(ceil(kv_len / S) / G),  S_eff = ceil(kv_len / L),
 *    chunk s covers keys [s * L, min((s + 1) * L, kv_len)).
 *  Any output pointer may be NULL. */
mla_status mla_plan_query(const mla_plan* plan, int32_t seq, int32_t* fold, int32_t* tiles,
                          int32_t* splits, int32_t* chunk_len);

/* The order in which the plan runs the sequences' work units: order[i] is
 * the caller's index of the i-th sequence (a permutation of 0 .. batch - 1;
 * longest unit first under MLA_PLAN_AUTO, the caller's order under
 * MLA_PLAN_UNIFORM or forced splits).  order: HOST array [batch].
 * Errors: INVALID_ARGUMENT (null plan or order). */
mla_status mla_plan_order(const mla_plan* plan, int32_t* order);

/* Whole-plan facts: main-kernel work units (one workgroup each), tiles that
 * are split (rows merged by the reduce), main-kernel launches (one: up to 60
 * sequence descriptors travel in its arguments, larger batches keep theirs
 * in the workspace), and the workspace bytes. Any pointer may be NULL. */
mla_status mla_plan_info(const mla_plan* plan, int32_t* num_units, int32_t* num_split_tiles,
                         int32_t* num_launches, size_t* workspace_bytes);

/* One main-kernel launch of the plan (0 <= launch < num_launches): its work
 * units and who merges its split rows (MLA_MERGE_REDUCE, _LAST_ARRIVER or
 * _GRID; 0 when it has none).  Any output pointer may be NULL.
 * Errors: INVALID_ARGUMENT (null plan, launch out of range). */
mla_status mla_plan_launch_info(const mla_plan* plan, int32_t launch, int32_t* num_units,
                                int32_t* merge_mode);

#ifdef __cplusplus
}
#endif

#endif /* MLA_DECODE_H */
