/*
 * entwine.h -- C ABI of a tile-overlapped GEMM-ReduceScatter for AMD Instinct
 * MI355X (gfx950), taken at one GPU's share of the work.
 *
 * Method: "Entwine: Coordinating Tiled Computation and Fine-Grained
 * Communication across GPUs" (paperpeel.com/paper/2609.11562).
 *
 * The operation (Sec. 2.1, GEMM-ReduceScatter Execution; Sec. 3.1): P ranks
 * each hold a slice of the reduction dimension; rank r computes the partial
 * product C_r = X_r * W_r (M x N) and the ReduceScatter hands rank d the row
 * partition [d*M/P, (d+1)*M/P) of sum_r C_r.  This library runs rank
 * `rank`'s side on one GPU: a bf16 MFMA GEMM produces C_rank tile by tile in a
 * selectable order (Sec. 3.1, "Interleaved production", Equation (1)) and
 * publishes one ready flag per output tile after the tile's stores (Sec. 4.2);
 * a concurrent persistent reduction kernel whose grid is capped by the
 * communication budget (Sec. 3.2) waits on each tile's flags and reduces the
 * local contribution with the P-1 peer contributions in rank order (Sec. 4.2,
 * ReduceTile).  The peers' contributions are caller-provided device buffers:
 * on one GPU they stand in for the data that peers would publish.
 *
 * Conventions for every entry point:
 *   - Return value: an entwine_status.  Errors never abort the process and
 *     never throw.  When an error is detected before launch nothing is
 *     enqueued; entwine_last_error_message() gives a thread-local detail.
 *   - Calls that take a stream are asynchronous: they enqueue device work on
 *     `stream` (a hipStream_t passed as void*, NULL = the null stream) and
 *     return.  Device-side failures (the reduction watchdog) are reported by
 *     entwine_device_status().
 *   - The caller owns every buffer it passes; buffers must stay valid until
 *     the work enqueued on `stream` has completed.  The library owns its
 *     workspace (per device, grown on demand, reused across calls, released
 *     by entwine_release()).
 *   - Calls are serialized on the library's workspace: each call's kernels
 *     start after the previous call's kernels on the same device finished.
 *     Host threads may call concurrently; a mutex guards the workspace.
 *   - Graph capture: a call may be captured into a HIP graph once the same
 *     call (same shape and schedule) has run outside the capture, so that its
 *     workspace and schedule exist (else ENTWINE_ERR_INVALID_ARGUMENT).  The
 *     graph holds workspace addresses: after a capture, workspace buffers
 *     that a later, larger call outgrows stay allocated until
 *     entwine_release(), which the caller makes only after destroying the
 *     graphs.  Replays of one graph, and eager calls between them, are
 *     serialized like calls.
 *   - Element types: bf16 is IEEE binary32 truncated to its upper 16 bits
 *     (stored as uint16), rounding is to nearest even.
 */
#ifndef ENTWINE_H
#define ENTWINE_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum entwine_status {
  ENTWINE_OK = 0,
  ENTWINE_ERR_INVALID_ARGUMENT = 1, /* shape, rank, pointer, alignment, alias or enum out of range */
  ENTWINE_ERR_UNSUPPORTED = 2,      /* well-formed but not built: P > 8, K_local % 64 != 0, sizes
                                       beyond 32-bit element indexing, unsupported tile shape */
  ENTWINE_ERR_OUT_OF_MEMORY = 3,    /* workspace growth failed */
  ENTWINE_ERR_HIP = 4,              /* a HIP runtime call failed (detail in the message) */
  ENTWINE_ERR_TIMEOUT = 5           /* a reduction workgroup gave up waiting on a tile flag */
} entwine_status;

/* Production orders of the GEMM's output blocks (Sec. 2.2 "Insight 1",
 * Sec. 3.1 "Interleaved production" and Equation (1), Sec. 5.3.1).
 * Blocks inside a partition are always numbered N-major (column index
 * fastest); the orders differ in how the P partitions are visited. */
enum {
  ENTWINE_ORDER_AUTO = -1,           /* from the tuning table, else INTERLEAVED */
  ENTWINE_ORDER_ROW_MAJOR = 0,       /* partitions 0..P-1, one contiguous run each */
  ENTWINE_ORDER_PARTITION_MAJOR = 1, /* contiguous runs starting after `rank`, the local run last */
  ENTWINE_ORDER_INTERLEAVED = 2,     /* logical block p -> partition p mod P, block p / P */
  ENTWINE_ORDER_COL_MAJOR = 3        /* M-major raster over the global block grid */
};

/* comm_budget: the reduction kernel's grid size x (Sec. 3.2 "Communication
 * budget"), capped at the number Q of tiles in the rank's partition and
 * required to stay below the device's CU count (Sec. 4.3).
 * ENTWINE_BUDGET_SEQUENTIAL runs the GEMM to completion and then the
 * reduction over all tiles, with no overlap (the non-overlapped baseline). */
#define ENTWINE_BUDGET_AUTO (-1)
#define ENTWINE_BUDGET_SEQUENTIAL 0

enum { ENTWINE_BF16 = 0, ENTWINE_F32 = 1 };

/* How the readiness of a peer's contribution is modelled on one GPU.
 * PRESEEDED: the peer buffers hold finished contributions; only the local
 * tile flag is awaited.  SYMMETRIC: peer r's contribution to tile t counts as
 * ready once this GPU's GEMM has finished the block at the logical position
 * where rank r would produce tile t, i.e. all ranks are assumed to progress
 * alike (Sec. 3.1: every rank runs the same traversal). */
enum { ENTWINE_PEERS_PRESEEDED = 0, ENTWINE_PEERS_SYMMETRIC = 1 };

/* Layout of W (the K_local x N operand). */
enum {
  ENTWINE_W_KN = 0, /* [K_local][N] row-major: N contiguous (the default; entwine_gemm_rs) */
  ENTWINE_W_NK = 1  /* [N][K_local] row-major: K contiguous (a linear layer's weight, W^T) */
};

enum { ENTWINE_STAGES_ALL = 0, ENTWINE_STAGES_GEMM = 1, ENTWINE_STAGES_REDUCE = 2 };

/* How an overlapped call (comm_budget >= 1) runs producer and consumer:
 *  STREAMS  two concurrent kernels (Sec. 4.3): the GEMM on the caller's
 *           stream, and x persistent reduction workgroups that poll the tiles'
 *           flags on an internal stream forked from and joined back to it.
 *  FUSED    one kernel on the caller's stream.  Its workgroups take GEMM
 *           blocks (in the same production order, with the same per-tile
 *           flags) until every block is taken; then workgroup w < x takes
 *           reduction tasks w, w + x, ... in production order.  No fork or
 *           join.
 *  ASSISTED the FUSED kernel on the caller's stream plus x reduction
 *           workgroups on the internal stream, forked from the caller's
 *           stream but never joined back: they reduce tiles as the GEMM
 *           releases them, each task going to whoever claims it first, and
 *           the fused kernel ends only once every task is done.  The caller's
 *           stream thus waits on nothing of the internal stream.  Eager calls
 *           only: inside a graph capture the fused kernel runs alone (a
 *           captured branch needs a join).  Not with push_outgoing, not from
 *           the no-alloc entry point.
 *  AUTO     the tuning table's choice for the shape, else STREAMS.
 * All give bit-identical output.  The sequential schedule (comm_budget 0)
 * and single stages ignore this field. */
enum {
  ENTWINE_SCHEDULE_AUTO = 0,
  ENTWINE_SCHEDULE_STREAMS = 1,
  ENTWINE_SCHEDULE_FUSED = 2,
  ENTWINE_SCHEDULE_ASSISTED = 3
};

/* GEMM main-loop pipeline (entwine_config.gemm_variant).  Every pipeline
 * multiplies the K steps in the same order, so all give bit-identical output.
 *  BASE (5)  8 waves in a 2 x 4 (or 4 x 2) arrangement, K stages of 64, two
 *            LDS stages; the only pipeline of 128 x 384 blocks.
 *  1, 2      256 x 256: 4 waves, K stages of 32, 4 or 3 LDS stages.
 *  3         128 x 128, 128 x 256, 256 x 128 and 256 x 256: the other wave
 *            count (4 or 8).
 *  4         256 x 256: 8 waves in two groups that alternate between loading
 *            and MFMAs (ping-pong), K stages of 64, two LDS stages.  It uses
 *            235 registers per lane, so a two-stream reduction cannot share its
 *            CUs (ENTWINE_ERR_UNSUPPORTED when requested explicitly).
 *  AUTO (0)  the tuning table's pipeline when its entry names the block shape
 *            in use, else BASE; BASE also replaces a pipeline the two-stream
 *            reduction cannot share CUs with.  With W [K_local][N] AUTO is
 *            always BASE.
 * Pipelines 1-4 are built for W [N][K_local] only; with W [K_local][N] (the
 * default layout) BASE is the only one.  A pipeline that is not built for the
 * block shape and layout in use is refused with ENTWINE_ERR_UNSUPPORTED. */
enum { ENTWINE_GEMM_AUTO = 0, ENTWINE_GEMM_PINGPONG = 4, ENTWINE_GEMM_BASE = 5 };

/* Release granularity (Sec. 5.3.2): tiles released together. */
#define ENTWINE_RELEASE_TILE 1       /* each tile on its own flag (the method) */
#define ENTWINE_RELEASE_PARTITION 0  /* a tile waits for the last tile of its partition */
#define ENTWINE_RELEASE_OUTPUT (-1)  /* a tile waits for the last block of the whole GEMM */

/*
 * entwine_gemm_rs -- rank `rank`'s share of C = sum_r X_r * W_r followed by
 * ReduceScatter (Sec. 2.1, 3.1), with tile-level overlap.
 *
 *   X              device, bf16 [M][K_local] row-major: this rank's slice of
 *                  the activations.  16-byte aligned.
 *   W              device, bf16 [K_local][N] row-major (N contiguous): this
 *                  rank's slice of the weight, element (k, n) at W[k*N + n].
 *                  16-byte aligned.  (entwine_gemm_rs_ex also takes [N][K_local]:
 *                  entwine_config.w_layout.)
 *   peer_partials  HOST array of P device pointers.  peer_partials[r] (r !=
 *                  rank) is bf16 [M/P][N] row-major: peer r's contribution to
 *                  partition `rank`.  peer_partials[rank] is ignored (may be
 *                  NULL).  May be NULL when P == 1.  16-byte aligned.
 *   out            device, bf16 [M/P][N] row-major: rows [rank*M/P,
 *                  (rank+1)*M/P) of sum_r C_r.  Fully overwritten, never read;
 *                  must not overlap any input.  16-byte aligned.
 *   M, N, K_local  M % P == 0, N % 8 == 0, K_local % 64 == 0, all > 0;
 *                  M*K_local, N*K_local and M*N below 2^31 (W [K_local][N]:
 *                  N*K_local below 2^30); K_local <= 2^21 and N <= 2^22 (the
 *                  kernels' 32-bit buffer offsets).  Beyond any of these:
 *                  ENTWINE_ERR_UNSUPPORTED.
 *   P, rank        1 <= P <= 8, 0 <= rank < P.
 *   tile_order     ENTWINE_ORDER_* (AUTO = tuning table, else INTERLEAVED).
 *   comm_budget    x >= 1 overlapped (clamped to Q), 0 sequential, -1 AUTO.
 *                  x must be below the device's CU count.
 *   stream         hipStream_t (as void*) the work is ordered on.
 * Defaults: 128x128 reduction tiles, GEMM blocks from the tuning table or a
 * shape heuristic, 256 reducer threads, PRESEEDED peers, per-tile release.
 * Numerics: fp32 accumulation; the local own-partition partial is kept in
 * fp32, the reduction adds peers in ascending rank order in fp32 and rounds
 * once to bf16.  For a fixed GEMM block shape the output bits do not depend
 * on tile_order, comm_budget, reducer threads or peer readiness mode.
 */
int entwine_gemm_rs(const void* X, const void* W, const void* const* peer_partials, void* out,
                    int64_t M, int64_t N, int64_t K_local, int P, int rank,
                    int tile_order, int comm_budget, void* stream);

/* Extended configuration.  Zero-initialise with entwine_config_init(). */
typedef struct entwine_config {
  int32_t struct_size;     /* sizeof(entwine_config) */
  int32_t block_m;         /* GEMM block rows BM: 0 = auto, else 128 or 256 */
  int32_t block_n;         /* GEMM block cols BN: 0 = auto, else 128 or 256, or 384 with
                              block_m 128 (one round of blocks for short partitions) */
  int32_t tile_m;          /* reduction tile rows TM: 0 = 128, else 64 or 128; BM % TM == 0 */
  int32_t tile_n;          /* reduction tile cols TN: 0 = 128, else 64 or 128; BN % TN == 0 */
  int32_t reducer_threads; /* b: 128, 256 or 512 (Sec. 4.3); 0 = the tuning table's entry,
                              else 256, and 512 under static CU partitioning (reducer_cus) */
  int32_t w_layout;        /* ENTWINE_W_KN (default) or ENTWINE_W_NK.  W [K][N] is built for
                              the base pipeline of every block shape; same output bits as
                              W [N][K] */
  int32_t peer_dtype;      /* ENTWINE_BF16 or ENTWINE_F32: peers and outgoing contributions */
  int32_t out_dtype;       /* ENTWINE_BF16 or ENTWINE_F32 */
  int32_t peer_ready;      /* ENTWINE_PEERS_PRESEEDED or ENTWINE_PEERS_SYMMETRIC */
  int32_t release_group;   /* ENTWINE_RELEASE_* or g > 1 tiles per release group */
  int32_t task_slabs;      /* overlapped schedule: row slabs per reduction task, dividing
                              tile_m (0 = 1: one task per tile, Sec. 3.1) */
  uint32_t poll_timeout_ms;/* reduction watchdog; 0 = 2000 ms */
  int32_t withhold_tile;   /* failure injection for tests: 0 = off; t+1 makes tile t's local
                              wait watch a flag that no GEMM of the call sets, so that tile's
                              reduction workgroup times out (ENTWINE_ERR_TIMEOUT) */
  int32_t gemm_variant;    /* ENTWINE_GEMM_* pipeline (0 = AUTO) */
  int32_t publish_all;     /* 0: agent-scope release only for tiles a kernel on this device
                              reads (the rank's partition), progress flags for the rest;
                              1: release every tile (the cost of publishing to peers) */
  int32_t linear_dispatch; /* 0: XCD-aware dispatch within each window of co-resident blocks
                              (entwine_plan_dispatch); 1: workgroup b computes logical block b */
  int32_t stages;          /* measurement: ENTWINE_STAGES_ALL (0), or one kernel alone:
                              ENTWINE_STAGES_GEMM (the GEMM without flags) or
                              ENTWINE_STAGES_REDUCE (the reduction of whatever the workspace
                              holds, with every flag treated as ready; the budget picks the
                              schedule as usual).  A single stage leaves `out` (GEMM) or the
                              partials (reduction) as they were: for timing only. */
  int32_t schedule;        /* ENTWINE_SCHEDULE_*; FUSED is built for the variant-0 pipelines
                              of every block shape and variants 3 and 4 of 256x256 */
  int32_t reducer_cus;     /* static CU partitioning (Sec. 5.3.3).  0: shared pool (both
                              kernels may use every CU).  n in [1, CUs): the reduction's n
                              workgroups run on n CUs of their own and the GEMM's CUs - n
                              persistent workgroups on the others, one workgroup per CU.
                              The split is made by LDS reservations (each workgroup reserves
                              more than half a CU's LDS, and a GEMM and a reduction
                              workgroup more than all of it), not by CU masks; it is exact
                              per XCD when n is a multiple of 8.  Overlapped calls only, and
                              the two-stream schedule only: comm_budget must equal n (AUTO
                              picks n and the two-stream schedule, and reducer_threads 0
                              picks 512, as a reserved CU holds nothing else); FUSED ->
                              ENTWINE_ERR_UNSUPPORTED; n >= CUs or comm_budget != n ->
                              ENTWINE_ERR_INVALID_ARGUMENT.  The sequential schedule ignores
                              it.  Output is bit-identical to the shared pool's. */
  int32_t push_outgoing;   /* 0: pull only (the method); 1: the reduction workgroups also push
                              every peer-bound tile, once its flag is set, from the outgoing
                              partials into a staging buffer (entwine_staging), in production
                              order with the reductions: the sender's side of a push-based
                              transfer, on one GPU.  Overlapped schedules only (comm_budget 0:
                              ENTWINE_ERR_UNSUPPORTED); releases every tile like publish_all */
  int32_t poll_backoff;    /* a waiting reduction workgroup polls its flags with pauses that
                              start at 128 clock cycles and double up to poll_backoff x 128
                              (0 = the default, 16; 1 = a fixed 128-cycle pause; at most 4096).
                              Longer pauses load the memory system less while the GEMM runs
                              and notice a released tile later */
} entwine_config;

void entwine_config_init(entwine_config* cfg);

/* As entwine_gemm_rs with an explicit configuration (cfg may be NULL). */
int entwine_gemm_rs_ex(const void* X, const void* W, const void* const* peer_partials, void* out,
                       int64_t M, int64_t N, int64_t K_local, int P, int rank,
                       int tile_order, int comm_budget, void* stream,
                       const entwine_config* cfg);

/*
 * entwine_gemm_rs_noalloc -- entwine_gemm_rs_ex for callers that cannot
 * allocate device memory: code under HIP graph capture, tight serving loops,
 * harnesses that forbid hipMalloc.  The call allocates nothing (no hipMalloc,
 * hipFree or allocating library routine); its control words, tile flags,
 * schedule tables, fp32 own partial, outgoing partials and (push_outgoing)
 * staging copies live in a fixed 256 MiB device array of the library, one copy
 * per GPU, held from the first call on that GPU until the process ends.
 *
 *   Arguments, layouts, numerics and results are those of entwine_gemm_rs_ex;
 *   the output is bit-identical to entwine_gemm_rs_ex's with the same
 *   arguments.  Schedules: the sequential one (comm_budget 0) and the fused
 *   one (comm_budget >= 1; AUTO resolves to it), both on `stream` alone.
 *   Errors, besides entwine_gemm_rs_ex's (nothing is enqueued on any of them):
 *     ENTWINE_ERR_OUT_OF_MEMORY  the call's buffers exceed the 256 MiB array
 *                                (own partial (M/P)*N*4 + outgoing M*N*2 or *4
 *                                + staging with push + tables), or its P*Q + 1
 *                                tile flags exceed 131072;
 *     ENTWINE_ERR_UNSUPPORTED    schedule STREAMS, reducer_cus > 0, a
 *                                measurement stage, or entwine_timing /
 *                                entwine_trace switched on;
 *     ENTWINE_ERR_INVALID_ARGUMENT  `stream` is being captured and the call
 *                                is the first on the GPU (it initialises the
 *                                array) or needs new schedule tables (below).
 *   Sharing: every call on a GPU uses that GPU's one array, which keeps the
 *   last call's contents.  Calls on one stream are ordered; calls that
 *   overlap on one GPU (other streams, other host threads' streams) race on
 *   the array and give undefined results.  A call whose shape or schedule
 *   differs from the previous no-alloc call's on the GPU copies the new
 *   schedule tables into the array and synchronizes `stream`, so it is
 *   refused under graph capture; a repeat of the previous call's shape and
 *   schedule can be captured.
 *   A timeout of its reduction is reported by entwine_device_status(stream).
 */
int entwine_gemm_rs_noalloc(const void* X, const void* W, const void* const* peer_partials,
                            void* out, int64_t M, int64_t N, int64_t K_local, int P, int rank,
                            int tile_order, int comm_budget, void* stream,
                            const entwine_config* cfg);

/*
 * entwine_gemm_rs_rmsnorm -- the layer chain of Sec. 5.2.2 (Layer-Level
 * Performance): the GEMM-ReduceScatter above, then a residual addition and an
 * RMSNorm over the rank's rows, in one call with the same schedules.
 *
 *   residual  device, out dtype [M/P][N]: the residual stream's rows of
 *             partition `rank`.  May be h_out itself (in-place update);
 *             otherwise it must not overlap h_out.
 *   gamma     device, out dtype [N]: the norm weight.
 *   eps       finite, >= 0 (added to the mean of squares).
 *   h_out     device, out dtype [M/P][N]: h = RS + residual.  The residual is
 *             added in fp32 after the peers, before the single rounding to the
 *             output type, so h is what the reduction alone would give with one
 *             more contribution.
 *   y_out     device, out dtype [M/P][N]: y[i][j] = gamma[j] * h[i][j] /
 *             sqrt(mean_j(h[i][j]^2) + eps), from the rounded h, in fp32,
 *             rounded once.  Must not overlap any other operand.
 * All other arguments and all errors are those of entwine_gemm_rs_ex; a NULL,
 * misaligned or overlapping chain operand, or a bad eps, is
 * ENTWINE_ERR_INVALID_ARGUMENT.  16-byte alignment throughout.
 */
int entwine_gemm_rs_rmsnorm(const void* X, const void* W, const void* const* peer_partials,
                            const void* residual, const void* gamma, float eps, void* h_out,
                            void* y_out, int64_t M, int64_t N, int64_t K_local, int P, int rank,
                            int tile_order, int comm_budget, void* stream,
                            const entwine_config* cfg);

/* ------------------------------------------------------------------------
 * Schedule queries (host only, no GPU needed).  They return the tables that
 * the kernels receive, for inspection and testing.
 * ---------------------------------------------------------------------- */

/* Block and tile counts for a shape (Sec. 3.1: Q = tiles in one partition).
 * Any output pointer may be NULL. */
int entwine_plan_shape(int64_t M, int64_t N, int P, int block_m, int block_n, int tile_m,
                       int tile_n, int64_t* num_blocks, int64_t* blocks_per_partition,
                       int64_t* tiles_per_partition);

/* The production order (Equation (1) for INTERLEAVED): for logical position
 * p in [0, num_blocks), blocks[4p..4p+3] = (partition d, block row br within
 * the partition, block col bc, number of the block's first tile within
 * partition d).  `capacity` = number of int32 elements available. */
int entwine_plan_blocks(int64_t M, int64_t N, int P, int rank, int tile_order, int block_m,
                        int block_n, int tile_m, int tile_n, int32_t* blocks, int64_t capacity);

/* The GEMM's dispatch permutation: workgroup b computes logical position
 * dispatch[b].  Workgroups run on XCD b % 8 in order, so inside each window of
 * `window` consecutive positions (the blocks resident at once: CUs times
 * blocks per CU; 0 = identity) the positions are dealt so that each XCD gets a
 * compact rectangle of the block grid.  The production order across windows
 * is unchanged.  `capacity` = number of int32 elements available (>= blocks). */
int entwine_plan_dispatch(int64_t M, int64_t N, int P, int rank, int tile_order, int block_m,
                          int block_n, int tile_m, int tile_n, int64_t window, int32_t* dispatch,
                          int64_t capacity);

/* Tile t of a partition (numbered in N-major producer order, Sec. 3.1
 * "Matching task order") sits at tile row tiles[2t], tile col tiles[2t+1]. */
int entwine_plan_tiles(int64_t M, int64_t N, int P, int block_m, int block_n, int tile_m,
                       int tile_n, int32_t* tiles, int64_t capacity);

/* waits[t*(P+1) + r], r < P: index into the flag array F[P][Q] (flattened
 * d*Q + t') of the flag that stands for source rank r's contribution to tile
 * t of partition `rank`, or -1 when that contribution needs no wait
 * (PRESEEDED peers).  The local slot r = rank is always the tile's own flag.
 * waits[t*(P+1) + P]: the flag that releases t's release group (Sec. 5.3.2),
 * or -1 with per-tile release. */
int entwine_plan_waits(int64_t M, int64_t N, int P, int rank, int tile_order, int block_m,
                       int block_n, int tile_m, int tile_n, int peer_ready, int release_group,
                       int32_t* waits, int64_t capacity);

/* The fused schedule's task order (Sec. 3.1 "Matching task order"): task
 * k = tile * task_slabs + slab of partition `rank`, sorted by the dispatch
 * index of the last GEMM block it waits for (its own tile's block, and under
 * SYMMETRIC peers or release groups the blocks standing for the other flags
 * of its wait slots), ties by task number.  Dispatch as entwine_plan_dispatch
 * with `window`.  `capacity` = int32 elements available (>= Q * task_slabs). */
int entwine_plan_task_order(int64_t M, int64_t N, int P, int rank, int tile_order, int block_m,
                            int block_n, int tile_m, int tile_n, int peer_ready,
                            int release_group, int64_t window, int task_slabs,
                            int32_t* task_order, int64_t capacity);

/* Consumer j's task sequence j, j+x, j+2x, ... < Q (Sec. 3.1 "Matching task
 * order") with x = min(comm_budget, Q).  Writes at most `capacity` entries
 * and stores the sequence length in *count. */
int entwine_plan_tasks(int64_t Q, int comm_budget, int consumer, int32_t* tasks,
                       int64_t capacity, int64_t* count);

/* ------------------------------------------------------------------------
 * Status, diagnostics and lifetime.
 * ---------------------------------------------------------------------- */

/* Synchronizes `stream`, then returns and clears the sticky device error of
 * the current device (ENTWINE_ERR_TIMEOUT if a reduction workgroup's
 * watchdog fired since the last query, else ENTWINE_OK).  While the error is
 * set, reduction workgroups stop waiting for flags, so the output of the
 * failed call and of any later call is undefined until this query has
 * returned the error; the query also clears the flags and the epoch. */
int entwine_device_status(void* stream);

const char* entwine_status_string(int status);
const char* entwine_last_error_message(void);

/* Device pointers of the current device's workspace (for tests): the fp32
 * own-partition partial [M/P][N] and the outgoing contributions [M][N]
 * (peer dtype) written by the last call.  Any pointer may be NULL. */
int entwine_workspace(const void** own_partial, const void** outgoing, int64_t* bytes);

/* The current device's tile flags (for tests of the publication protocol):
 * the device pointer of the u32 flag array -- flag of tile t of partition d
 * at d * Q + t, Q the tiles per partition of the last call's tiling, plus one
 * slot no GEMM ever writes -- its allocated length in words, and the epoch the
 * next overlapped call will stamp into the flags it publishes (each such
 * call advances it by one, skipping 0; the sequential schedule publishes no
 * flags and leaves it).  Synchronizes like entwine_workspace.  Any pointer
 * may be NULL; ENTWINE_ERR_INVALID_ARGUMENT before any call on the device. */
int entwine_flags(const void** flags, int64_t* words, uint32_t* epoch);

/* Allocated sizes in bytes of the current device's own-partial, outgoing and
 * staging buffers (for tests that overwrite the workspace between calls, e.g.
 * with a NaN pattern, to show that no call reads data a previous call left:
 * writes must stay within these sizes).  Synchronizes like entwine_workspace.
 * Any pointer may be NULL; ENTWINE_ERR_INVALID_ARGUMENT before any call on the
 * device. */
int entwine_workspace_sizes(int64_t* own_bytes, int64_t* outgoing_bytes, int64_t* staging_bytes);

/* Device pointer of the current device's staging buffer (for tests and
 * measurements): peer dtype [M][N], whose rows of partition d != rank hold
 * the copies pushed by the last call with push_outgoing = 1 (the rank's own
 * rows are unused).  NULL before any pushing call. */
int entwine_staging(const void** staging, int64_t* bytes);

/* Per-kernel timing with HIP events recorded on the stream each kernel is
 * launched on.  entwine_timing(1) starts recording every call; reading
 * synchronizes the recorded events and returns the summed kernel durations
 * (ms) and the number of calls since the last read.  Under the FUSED
 * schedule both durations are the fused kernel's. */
int entwine_timing(int enable);
int entwine_timing_read(double* gemm_ms, double* reduce_ms, int64_t* calls);

/* Device-side trace of the communication tail (Sec. 3.2 and 5.3: the time the
 * reduction runs past the GEMM).  entwine_trace(1) makes every following
 * call record wall-clock stamps (s_memrealtime, 100 MHz on MI355X) in
 * library-owned device memory: every GEMM block its start and its end (its
 * stores and flags issued), every reduction workgroup the start of its task
 * loop (waits included) and its end (its stores issued), each in slots of its
 * own, written with plain stores.  A small kernel the call launches first
 * zeroes the slots.  entwine_trace(0) stops recording.  A call captured into a
 * graph while tracing is on records on every replay; its slots must exist,
 * i.e. the same call once outside the capture first (else
 * ENTWINE_ERR_INVALID_ARGUMENT).
 *
 * entwine_trace_read synchronizes the device and reduces the last traced
 * call's slots to µs from its first GEMM block's start: the last GEMM block's
 * end, the reduction's first start and last end, and the tail = reduction end
 * - GEMM end (0 for the reduction figures when the call ran no reduction).
 * Any pointer may be NULL.  ENTWINE_ERR_INVALID_ARGUMENT if no call on the
 * current device was traced or the last one ran no GEMM. */
int entwine_trace(int enable);
int entwine_trace_read(double* gemm_us, double* reduce_start_us, double* reduce_end_us,
                       double* tail_us);

/* Load an offline tuning table (text; one entry per line:
 * "M N K_local P tile_order comm_budget block_m block_n reducer_threads
 * [task_slabs [schedule [gemm_variant]]]", '#' starts a comment line; the
 * entry's gemm_variant is 0 for the base pipeline or 1 to 4).  Entries are
 * consulted by the AUTO settings (tile_order -1, comm_budget -1, zero config
 * fields). */
int entwine_load_tuning(const char* path);

/* Frees the current device's workspace (including buffers retired after a
 * graph capture); the next call re-creates it.  Graphs that captured calls
 * must be destroyed first. */
int entwine_release(void);

/* Number of compute units of the current device (0 when no device). */
int entwine_device_cus(void);

#ifdef __cplusplus
}
#endif

#endif /* ENTWINE_H */
