/*
 * tbe.h - C ABI of the table-batched embedding (TBE) library for MI355X (gfx950).
 *
 * What the library computes (PyTorch blog "Modernizing Table Batched Embeddings
 * with FBTriton", sections 2 and 3; layout of "Table-Batched Embeddings in
 * Triton: Gather, Pool, and Run-Length Backward", section 1):
 *
 *   forward   out[b][col_t + d] = sum_{j in bag(t,b)} psw_j * W_t[idx_j][d]
 *   backward  for every unique (table, row) touched by the batch, sum the
 *             upstream gradient rows of every lookup that touched it (each
 *             scaled by its per-sample weight when there is one), then apply
 *             exactly one optimizer step (SGD or exact row-wise Adagrad) to
 *             that row, in place.
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 *  - Pointers are DEVICE pointers unless the comment says [host].  The caller
 *    allocates and owns every buffer.  The library never allocates device
 *    memory, never synchronizes the stream and never copies device data to the
 *    host; every kernel is launched on the caller's stream, in stream order.
 *  - Every call returns a tbe_status.  Argument errors are found on the host
 *    before anything is launched (TBE_ERR_ARG / TBE_ERR_UNSUPPORTED /
 *    TBE_ERR_WORKSPACE); a failed launch is TBE_ERR_HIP.  tbe_last_error()
 *    then holds a one-line description (thread-local).  No C++ exception
 *    crosses this interface and nothing aborts.
 *  - Layout: T tables ("features"), table t has E_t rows of width D_t, B bags
 *    per table.  Weights of all tables are one buffer, table after table,
 *    each row-major E_t x D_t.  offsets has T*B+1 entries, table-major: bag
 *    (t, b) owns indices[offsets[t*B+b] .. offsets[t*B+b+1]).  Indices are row
 *    ids local to their table.  The pooled output and the upstream gradient
 *    are B x sum_t D_t fp32, row-major; table t's slice starts at column
 *    sum_{t'<t} D_t'.
 *  - Limits: 1 <= T; 0 <= B; 4 <= D_t <= 1024 with D_t % 4 == 0;
 *    sum_t E_t < 2^31 - 1 (linearized row ids are 32-bit); number of lookups
 *    <= TBE_MAX_LOOKUPS = 2^31 - 4096; T*B < 2^31.
 *  - Concurrency: calls on different streams may be made from several host
 *    threads.  The calls that use the library's second stream
 *    (tbe_forward_hoisted, and a backward with bwd_streams = 2 or its automatic
 *    choice) hold one process-wide lock from their fork to their join, that is
 *    while they enqueue their launches (never while the GPU runs them), so
 *    such calls from different threads are enqueued one after another; their
 *    second-stream work then runs in that order.
 *  - Invalid input with bounds checking off: an index outside [0, E_t)
 *    contributes nothing to the forward and nothing to the backward, and no
 *    memory outside the weights is touched; the pages leave this case to an
 *    optional repair step (tbe_bounds_check).  Offsets must be non-decreasing
 *    with offsets[0] = 0 and offsets[T*B] = num_indices; otherwise results are
 *    undefined (but every access stays inside the caller's buffers).
 */
#ifndef TBE_H_
#define TBE_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* A hipStream_t passed as an opaque pointer; NULL is the default stream. */
typedef void* tbe_stream_t;

typedef enum { TBE_F32 = 0, TBE_F16 = 1, TBE_BF16 = 2 } tbe_dtype;   /* weight storage */
typedef enum { TBE_I32 = 0, TBE_I64 = 1 } tbe_itype;                 /* indices / offsets */
typedef enum {
  TBE_OK = 0,
  TBE_ERR_ARG = 1,          /* null pointer, negative size, inconsistent geometry */
  TBE_ERR_UNSUPPORTED = 2,  /* D or dtype outside the supported range */
  TBE_ERR_WORKSPACE = 3,    /* workspace null, misaligned or smaller than required */
  TBE_ERR_HIP = 4           /* a HIP launch failed */
} tbe_status;

#define TBE_MAX_D 1024
#define TBE_MAX_LOOKUPS 2147479552LL /* 2^31 - 4096 */
#define TBE_NUM_BUCKETS 9   /* short-run buckets next_pow2(D) = 4, 8, ..., 1024 */
#define TBE_META_FIELDS 4   /* per table: row base, weight base, column base, D */

/*
 * Table geometry, filled by tbe_tables_derive.  Only `meta` must be set by
 * the caller afterwards: a device copy of the int64 array that
 * tbe_tables_derive wrote to meta_host (TBE_META_FIELDS * (T + 1) entries).
 */
typedef struct {
  int32_t T;                 /* tables */
  int32_t B;                 /* bags per table */
  int32_t w_dtype;           /* tbe_dtype of every table */
  int32_t max_D;             /* max_t D_t */
  int32_t out_width;         /* sum_t D_t: row length of out and grad_out */
  int32_t all_D_mult8;       /* 1 when every D_t % 8 == 0 (wider vector loads) */
  int32_t hist_table;        /* table eligible for the histogram forward, or -1 */
  int32_t hist_E;            /* rows of that table */
  int32_t hist_D;            /* width of that table */
  int32_t hist_col;          /* its first output column */
  int32_t row_bits;          /* bits of the largest local row id, max_t E_t - 1 (at least 1) */
  int64_t hist_w_base;       /* its first element in the weight buffer */
  int64_t total_rows;        /* sum_t E_t: linearized row ids are [0, total_rows) */
  int64_t total_elems;       /* sum_t E_t * D_t: elements of the weight buffer */
  int64_t bucket_rows[TBE_NUM_BUCKETS]; /* rows of the tables in each short-run bucket */
  const int64_t* meta;       /* device: [T+1][4] = {row base, weight base, column base, D};
                                entry T = {total_rows, total_elems, out_width, 0} */
} tbe_tables;

/*
 * Knobs (blog section 5 keeps each tuning choice as a config value rather
 * than a code path).  tbe_config_default
 * gives the pages' defaults; a NULL config pointer means the defaults.
 */
typedef struct {
  int32_t long_threshold;  /* a run with >= this many lookups is long (default 256) */
  int32_t chunk;           /* lookups per long-run chunk (default 256) */
  int32_t hist_enable;     /* 1: the eligible small table takes the histogram paths - counts x table
                              on MFMA forward, counts^T x grad_out on MFMA backward (default 1) */
  int32_t fwd_unroll;      /* forward row loads in flight per lane group: 2, 4 or 8 (default 4; the
                              fused id check takes 4 or 8) */
  int32_t bwd_unroll;      /* long-run chunk gradient rows in flight per lane group: 2, 4 or 8 (default 8) */
  int32_t sort_blocks;     /* workgroups of each radix pass (default 0 = automatic) */
  int32_t bag_windows;     /* long-run chunks are processed grouped by (table, bag window of their
                              first lookup), B / bag_windows bags per window, so that chunks that
                              read the same gradient rows run together (<= 1: off, the default;
                              measured no faster on gfx950, where these reads come from HBM) */
  int32_t fused_long;      /* 1: long runs in one launch - each chunk writes its partial, a device-scope
                              fence, then a per-run countdown; the last chunk applies the optimizer
                              (blog section 4, problem 5).  0: chunk kernel + apply kernel (default) */
  int32_t pretransposed;   /* backward and tbe_transpose: 1 = the workspace already holds this batch's
                              transpose, written by tbe_forward_hoisted; the backward skips its own,
                              tbe_transpose only describes it (default 0) */
  int32_t bags_per_wave;   /* forward: consecutive bags one wave pools, their offsets read in one
                              load ("bags per program", blog section 2), 1..64; 0 (default): the
                              smallest power of two from 8 that keeps the launch within 65536
                              workgroups */
  int32_t bwd_streams;     /* backward: 2 = long runs (chunks, apply, dense rows) on the library's
                              second stream, concurrent with the short runs; 1 = one stream;
                              0 (default): 2 when the tables' widths fall in two or more short-run
                              buckets; otherwise, when the dense rows are picked before the sort
                              or the histogram table is in use, those rows' kernels on the second
                              stream (one workgroup per CU) beside the short runs, whose grid
                              leaves room for them */
  int32_t tiny_runs;       /* backward: a wave step whose short runs all have at most this many
                              lookups serves twice as many runs with half the lanes each (rows of
                              64 .. 256 columns); default 8, 0: off */
  int32_t dense_min;       /* backward: per table (16 <= D <= 128, D % 16 == 0, not the
                              histogram table), its rows of at least this many lookups (the 128
                              with the most when more qualify; among equal counts the smaller row
                              ids) are updated from per-bag counts (with per-sample weights: per-bag
                              sums of the weights) x grad_out on MFMA instead of through the
                              sorted runs (default 1024;
                              values below long_threshold act as long_threshold; 0: off; off
                              with fused_long) */
  int32_t dense_presort;   /* backward with dense_min: 1 = the dense rows are picked before the
                              sort, from the lookups at 64 positions in every S (S the smallest
                              power of two >= 64 that leaves at most 2^20 of them; every lookup
                              up to 2^20 lookups) with dense_min scaled by 64 / S, so that rows
                              near the cut may fall either way, and their lookups stay out of
                              the sort; -1 = they are the long runs of >= dense_min lookups after
                              the sort; 0 (default): 1 from 2^26 lookups on, else -1 */
  int32_t sort_by_table;   /* backward transpose: 1 = each table's lookups are sorted on their own,
                              on the bits of the local row id (the batch keeps a table's lookups
                              together, so the order is the same as sorting the linearized ids);
                              -1 = one sort of the linearized ids; 0 (default): by table when the
                              largest table needs fewer bits than the linearized ids, there are at
                              least 2 tables and at most half as many tables as sort blocks */
} tbe_config;

/* Device-side view of the transpose, for inspection by tests (tbe_transpose). */
typedef struct {
  const uint32_t* sorted_keys;     /* [counters[13]] linearized row id, ascending (lookups of ids
                                      outside their table are left out) */
  const uint32_t* sorted_payload;  /* [counters[13]] bag id t*B+b, or lookup position when weighted */
  const uint32_t* run_key;         /* [N] key of run r (first num_runs used) */
  const uint32_t* run_start;       /* [N+1] first sorted position of run r; run_start[num_runs] =
                                      counters[13] */
  const int32_t* counters;         /* [16]: 0 runs, 1 long runs, 2 chunks, 3..11 short runs per
                                      bucket (next_pow2(D) = 4 .. 1024), 12 keys the sort covers
                                      when a table is left out, 13 keys sorted, 14 used by the
                                      backward's dense rows (0 here) */
  const uint32_t* long_list;       /* [cap][4] {key, start, len, first chunk} per long run */
  const uint32_t* long_table;      /* [cap] table of each long run */
  const uint32_t* chunk_list;      /* [cap][2] {long-run slot, chunk number} per chunk */
  const uint32_t* short_list[TBE_NUM_BUCKETS]; /* [cap][4] {key, start, len, table}, or NULL */
  int64_t long_capacity, chunk_capacity;
  int64_t short_capacity[TBE_NUM_BUCKETS];
  int32_t payload_is_position;     /* 1 for weighted calls */
  int32_t radix_passes;
  const int32_t* dense_rows;       /* [T][128] per table its dense rows (local row ids, ascending),
                                      the first dense_count[t] used, when they are picked before the
                                      sort (dense_min > 0, unweighted, and dense_presort = 1, or 0
                                      from 2^26 lookups on); their lookups are in no run.  NULL
                                      otherwise (no dense rows, or rows picked from the long runs
                                      by the backward, which stay in long_list) */
  const int32_t* dense_count;      /* [T], or NULL with dense_rows */
  int32_t sorted_by_table;         /* 1: each table's lookups were sorted on their own, on the bits
                                      of the local row id (tbe_config.sort_by_table); the result is
                                      the same order */
  int32_t reserved;
} tbe_runs_view;

/* Static description of a status code. */
const char* tbe_status_string(tbe_status s);

/* Last error message of the calling thread ("" when none). */
const char* tbe_last_error(void);

/* Fills *cfg with the defaults listed in tbe_config. */
void tbe_config_default(tbe_config* cfg);

/* Number of int64 entries tbe_tables_derive writes to meta_host: 4 * (T + 1). */
int64_t tbe_meta_entries(int32_t T);

/*
 * Host only.  Derives the geometry of T tables of E_host[t] rows and
 * D_host[t] columns, B bags each, weights of dtype w_dtype.  Writes the
 * per-table bases to meta_host [host, tbe_meta_entries(T) int64] and the
 * summary to *out (out->meta is set to NULL: the caller uploads meta_host and
 * stores the device pointer there).  pooling_hint_host [host, T, nullable] is
 * the expected lookups per bag of each table; the histogram forward is
 * offered for the first table with E <= 64, 64 <= D <= 128, D % 16 == 0,
 * fp16 weights and a hint >= 64 (blog section 2, small-table path).
 */
tbe_status tbe_tables_derive(int32_t T, int32_t B, int32_t w_dtype, const int64_t* E_host,
                             const int32_t* D_host, const int32_t* pooling_hint_host,
                             int64_t* meta_host, tbe_tables* out);

/*
 * Bounds check and repair (blog section 2, "Bounds checking"; tutorial
 * Pitfalls: an id outside its table silently reads another table's row).
 * Repairs in place: offsets become their running maximum after clamping to
 * [0, num_indices], with offsets[0] = 0 and offsets[T*B] = num_indices; then
 * every index outside [0, E_t) of the table that owns its position becomes 0.
 * error_counts [device, 2 x int64] is overwritten with {indices repaired,
 * offsets entries changed}.  workspace: tbe_bounds_check_workspace_bytes().
 */
size_t tbe_bounds_check_workspace_bytes(const tbe_tables* tables);
tbe_status tbe_bounds_check(const tbe_tables* tables, void* indices, int32_t index_type,
                            void* offsets, int32_t offset_type, int64_t num_indices,
                            int64_t* error_counts, void* workspace, size_t workspace_bytes,
                            tbe_stream_t stream);

/*
 * Forward (blog section 2).  weights: the table buffer (w_dtype); indices
 * [num_indices] and offsets [T*B+1] of index_type / offset_type;
 * per_sample_weights [num_indices] fp32 or NULL; out [B][out_width] fp32,
 * fully overwritten (an empty bag gives zeros).  fp16 / bf16 tables
 * accumulate in fp32, fp32 tables in fp64.  When the config enables it, the
 * call has no per-sample weights, and tables->hist_table >= 0, that table's
 * bags are pooled by the histogram + MFMA kernel (counts of each bag's first
 * 256 ids times the table; remaining ids gathered).
 */
tbe_status tbe_forward(const tbe_tables* tables, const void* weights, const void* indices,
                       int32_t index_type, const void* offsets, int32_t offset_type,
                       int64_t num_indices, const float* per_sample_weights, float* out,
                       const tbe_config* config, tbe_stream_t stream);

/*
 * Forward with the bounds check fused into the gather (blog section 2,
 * "Bounds checking": with the fused option the eligible kernel validates and
 * repairs ids while it looks them up; offsets keep their own small repair
 * step).  Same results as tbe_bounds_check followed by tbe_forward: offsets
 * and indices repaired in place by the same rules, error_counts [device, 2 x
 * int64] overwritten with {indices repaired, offsets changed}, out as in
 * tbe_forward.  When the histogram path is used, its kernel repairs that
 * table's ids the same way while it counts them.  workspace:
 * tbe_bounds_check_workspace_bytes().
 */
tbe_status tbe_forward_repair(const tbe_tables* tables, const void* weights, void* indices,
                              int32_t index_type, void* offsets, int32_t offset_type,
                              int64_t num_indices, const float* per_sample_weights, float* out,
                              int64_t* error_counts, void* workspace, size_t workspace_bytes,
                              const tbe_config* config, tbe_stream_t stream);

/*
 * tbe_forward_repair without a workspace argument, for callers that cannot
 * allocate device memory (code under HIP graph capture, tight serving loops,
 * harnesses that forbid hipMalloc).  Same arguments and results as
 * tbe_forward_repair minus workspace / workspace_bytes: the offsets repair's
 * block partials live in a static device array of the library,
 * TBE_NOALLOC_SCRATCH_BYTES (16 KiB) on each GPU, held until the process
 * ends; a call that would need more returns TBE_ERR_WORKSPACE.  Nothing is
 * allocated: no hipMalloc, hipFree or allocating library routine.  Every call
 * on one GPU shares that GPU's array, so calls that overlap on one GPU (on
 * different streams, or from different threads) race on it and must be
 * ordered by the caller; calls on different GPUs do not share anything.
 */
#define TBE_NOALLOC_SCRATCH_BYTES 16384
tbe_status tbe_forward_repair_noalloc(const tbe_tables* tables, const void* weights, void* indices,
                                      int32_t index_type, void* offsets, int32_t offset_type,
                                      int64_t num_indices, const float* per_sample_weights,
                                      float* out, int64_t* error_counts, const tbe_config* config,
                                      tbe_stream_t stream);

/*
 * Forward with the backward's transpose hoisted into it (blog section 2,
 * forward-state reuse and preprocessing; the tutorial's section on forward
 * slower, total faster).  Computes out exactly as tbe_forward
 * (error_counts == NULL) or tbe_forward_repair (error_counts != NULL, with
 * bounds_workspace as there), and, on a second stream owned by the library,
 * the backward's linearize / sort / run-length encoding / routing of the same
 * batch into bwd_workspace (tbe_backward_workspace_bytes for the same tables,
 * num_indices, per-sample-weights presence and config).  The second stream
 * forks from `stream` after the offsets are final and joins it again before
 * the call returns: work enqueued later on `stream` sees the output and the
 * transpose.  A following tbe_backward_* with config->pretransposed = 1 and the
 * same tables, indices, offsets, per-sample-weights presence, config and
 * bwd_workspace skips its own transpose; with the histogram table, the forward
 * also keeps each bag's lookup counts there and that backward reuses them
 * instead of counting the table's ids again.  With repair, an out-of-range id
 * counts in the transpose as row 0 of its table, the value the repair writes,
 * whichever of the two reads the id first.  Calls that overlap on one device
 * share the second stream and run their transposes in call order.
 */
tbe_status tbe_forward_hoisted(const tbe_tables* tables, const void* weights, void* indices,
                               int32_t index_type, void* offsets, int32_t offset_type,
                               int64_t num_indices, const float* per_sample_weights, float* out,
                               int64_t* error_counts, void* bounds_workspace,
                               size_t bounds_workspace_bytes, void* bwd_workspace,
                               size_t bwd_workspace_bytes, const tbe_config* config,
                               tbe_stream_t stream);

/*
 * Bytes of workspace the backward (and tbe_transpose) needs for num_indices
 * lookups; weighted = 1 when per-sample weights will be passed.  The size
 * follows from the lookup count and the table geometry alone (blog section 4:
 * the run counts stay on the device), so no device count is read back.
 */
size_t tbe_backward_workspace_bytes(const tbe_tables* tables, int64_t num_indices,
                                    int32_t weighted, const tbe_config* config);

/*
 * Backward with SGD (blog section 3): w <- w - lr * g for every touched row,
 * in place, rounded to the storage dtype (nearest even).  grad_out
 * [B][out_width] fp32.  per_sample_weights as in the forward (NULL =
 * unweighted).  workspace: at least tbe_backward_workspace_bytes, 256-byte
 * aligned; its contents are undefined after the call.  When hist_enable is
 * set, there are no per-sample weights and tables->hist_table >= 0, that
 * table's rows take their gradient from per-bag lookup counts times grad_out
 * on MFMA (blog section 2, forward-state reuse) and its lookups stay out of the
 * sort; the other tables go through the sorted runs.  With dense_min > 0, each
 * eligible table's rows of at least dense_min lookups (up to 128 a table; see
 * dense_presort for how they are counted) take the same counts x grad_out route
 * on bf16 MFMA with an exact three-part split of the gradient (with per-sample
 * weights, per-bag sums of the weights, also split in three parts, in place of
 * the counts); the step is the same up to the order of the fp32 sums.
 */
tbe_status tbe_backward_sgd(const tbe_tables* tables, void* weights, const void* indices,
                            int32_t index_type, const void* offsets, int32_t offset_type,
                            int64_t num_indices, const float* per_sample_weights,
                            const float* grad_out, float lr, void* workspace,
                            size_t workspace_bytes, const tbe_config* config, tbe_stream_t stream);

/*
 * Backward with exact row-wise Adagrad ("Table-Batched Embeddings in Triton",
 * section 5): per touched row, m <- m + sum_d g_d^2 / D_t, then
 * w <- w - lr * g / (sqrt(m) + eps) with the new m.  momentum [total_rows]
 * fp32, in place; untouched rows keep weights and momentum.
 */
tbe_status tbe_backward_rowwise_adagrad(const tbe_tables* tables, void* weights, float* momentum,
                                        const void* indices, int32_t index_type,
                                        const void* offsets, int32_t offset_type,
                                        int64_t num_indices, const float* per_sample_weights,
                                        const float* grad_out, float lr, float eps,
                                        void* workspace, size_t workspace_bytes,
                                        const tbe_config* config, tbe_stream_t stream);

/*
 * The backward's transpose and routing alone (blog section 3,
 * transpose_embedding_input, and section 4, run classification): linearize,
 * stable radix sort, run-length encoding, long/short routing with D buckets
 * and chunk plan.  Fills *view [host] with device pointers into workspace;
 * nothing is read back.  weighted selects the payload (see tbe_runs_view).
 * Every table's lookups take part and no dense rows are picked (dense_rows
 * then lists none).  With config->pretransposed = 1 nothing is launched: the
 * view describes the transpose that tbe_forward_hoisted left in `workspace`
 * for the same tables, num_indices, weighted flag and config (the histogram
 * table's lookups, the dense rows picked before the sort, and, with repair,
 * an out-of-range id counted as row 0 of its table, as that call leaves them).
 */
tbe_status tbe_transpose(const tbe_tables* tables, const void* indices, int32_t index_type,
                         const void* offsets, int32_t offset_type, int64_t num_indices,
                         int32_t weighted, void* workspace, size_t workspace_bytes,
                         const tbe_config* config, tbe_runs_view* view, tbe_stream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* TBE_H_ */
