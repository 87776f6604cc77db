// kernels.h -- argument blocks and launchers of the two device kernels.
//
// gemm_publish: the producer (Sec. 4.2, Producer): one workgroup per logical
//   block position, bf16 MFMA main loop, stores, then one ready flag per
//   covered reduction tile, stored once every wave's stores of the block are
//   acknowledged (see the publication step in gemm_block.h).
// tile_reduce: the consumer (Sec. 4.2, Consumer / ReduceTile): x persistent
//   workgroups walking tasks j, j+x, ...; wait for the tile's flags, then read
//   the released data with device-coherent loads and sum local + peers (rank
//   order) in fp32, one store per output element.
#pragma once

#include <hip/hip_runtime.h>

#include <cstdint>

namespace entwine {

constexpr int kMaxRanks = 8;

struct GemmArgs {
  const uint16_t* X;        // bf16 [M][K]
  const uint16_t* W;        // bf16 [N][K], or [K][N] when w_kn is set
  float* own;               // fp32 [R][N]: partial of partition `rank`
  void* outgoing;           // peer dtype [M][N]: partials for other partitions
  uint32_t* flags;          // [P][Q] tile flags
  const int32_t* blocks;    // [NB][4]: d, br, bc, first tile
  int32_t M, N, K, R;       // R = M / P
  int32_t rank, Q;
  int32_t Rt, Ct;           // tile rows / cols per partition
  int32_t tm, tn;           // reduction tile
  int32_t outgoing_f32;     // outgoing partials in fp32 (else bf16)
  int32_t variant;          // GEMM pipeline variant (0 = default for the shape)
  int32_t w_kn;             // 1: W is [K][N] (N contiguous); 0: [N][K]
  int32_t publish;          // 0: no flags; 1: release local tiles, mark the rest; 2: release all
  int32_t flag_all;         // 1: every block stores its flags (else only the local ones)
  uint32_t* ctl;            // device control words (see check_out)
  uint64_t* trace;          // measurement stamps [2][NB] (see trace_at), nullptr: off
  int32_t trace_nb;         // NB: blocks of the call
  int32_t nb;               // NB, for the persistent (ticket) GEMM
  // Workgroups of the call that check out on ctl[kCallDone] (the ticket GEMM
  // and the reduction it runs beside): the last one advances the epoch.
  int32_t checkout_total;
};

struct ReduceArgs {
  const float* own;                 // fp32 [R][N]
  const void* peers[kMaxRanks];     // peer dtype [R][N]; [rank] unused
  void* out;                        // out dtype [R][N]
  const uint32_t* flags;            // [P][Q]
  const int32_t* waits;             // [Q][wait_slots] flag index or -1
  const int32_t* tiles;             // [Q][2] tile row, tile col
  int32_t* error;                   // sticky device error word
  int32_t R, N, P, rank, Q;
  int32_t wait_slots;               // P source ranks + 1 release-group slot
  int32_t tm, tn;
  int32_t slabs;                    // row slabs per tile (task = tile x slab)
  int32_t ntasks;                   // tasks in the call (Q * slabs without a task list)
  // Task list: entry j is the global task id (d * Q + t) * slabs + slab of
  // partition d's tile t.  d == rank: reduce the slab into `out`; d != rank:
  // push the outgoing slab into `staging` (a send task).  nullptr: task j is
  // slab j % slabs of own tile j / slabs.
  const int32_t* task_list;
  // Layer chain (residual addition before the RMSNorm): out dtype [R][N]
  // added after the peers, before the rounding; nullptr for the plain
  // operation.  May be `out` itself (each element is read, then written, by
  // the same thread).
  const void* residual;
  const void* outgoing;             // peer dtype [M][N]: the GEMM's outgoing partials
  void* staging;                    // peer dtype [M][N]: pushed copies (rows of partition d)
  uint32_t* ctl;                    // device control words (see check_out)
  uint64_t timeout_ticks;           // watchdog, in wall-clock ticks
  int32_t withhold_tile;            // -1, or a tile whose local wait watches `never_flag`
  int32_t never_flag;               // a flag slot that no GEMM of this call writes
  int32_t nowait;                   // 1: every flag counts as ready, no epoch check-out
  // 1: the peers' contributions (and the residual) were complete before the
  // call, so a task may load them before its wait; 0: they are loaded after
  // the wait, as a real peer's data would be (symmetric readiness).
  int32_t prefetch;
  uint64_t* trace;                  // measurement stamps [2][grid] (see trace_at), nullptr: off
  // Trace slots: workgroup w stores its start at trace[trace_slot0 + w] and
  // its end at trace[trace_g + trace_slot0 + w]; trace_g 0: the grid size.
  int32_t trace_slot0, trace_g;
  int32_t checkout_total;           // as GemmArgs::checkout_total
  // The assisted schedule (see kAssistCall): the call's sequence number
  // (0: not assisted) and one claim word per task (the sequence number of
  // the call in which the task was last claimed).
  uint32_t assist_seq;
  uint32_t* claims;
  // A waiting workgroup's pause between two polls starts at 128 clock cycles
  // and doubles up to nap_max x 128 cycles.
  int32_t nap_max;
};

// Epochs.  A flag is ready when it equals the call's epoch, which every
// kernel reads from ctl[kEpoch] at run time (so a captured graph replays
// correctly).  The epoch advances (skipping 0, the value of flags never
// written) only once every workgroup of the call that may store or read a
// flag has finished: in the two-stream schedule the GEMM's and the
// reduction's workgroups check out on one shared count (check_out), in the
// fused schedule the fused kernel's workgroups on its own.  So every flag a
// call stores holds that call's epoch, and a later call, whose epoch differs,
// can never take one of them for its own.
//
// The fused kernel (GEMM blocks and reduction tasks taken from tickets) keeps
// its tickets and its own check-out count in further control words; its
// last workgroup clears them and advances the epoch.  Every counter that many
// workgroups update has a 128-byte line of its own: atomics to one line are
// serialized, and with the eight block tickets in one line a multi-round
// 768-block GEMM ran 30 % slower.
//
// The assisted schedule: the fused kernel on the caller's stream and, on the
// internal stream with no event between them, reduction workgroups that help
// with the tasks while the GEMM runs.  kAssistCall holds (sequence number,
// epoch) of the call whose fused kernel is running, (sequence number, 0)
// once it has finished: the helpers of call s work only while it reads
// (s, e), so a helper that starts late or outlives its call does nothing.
// A task goes to whoever first moves its claim word to the call's sequence
// number (compare-and-swap), which succeeds only from an older call's
// number: a helper that outlives its call can never take a task from a later
// one, even while that task's flag still holds the earlier call's epoch.
// kTasksDone counts the completed tasks, and the fused kernel's last
// workgroup waits for all of them before it finishes the call.
// No wait ever depends on a helper being scheduled: a helper claims a task
// only once the task's flags are set, so a claimed task always completes.
enum {
  kLine = 32,  // control words per 128-byte line
  kEpoch = 0,
  kCallDone = 1 * kLine,     // joint check-out count of the two-stream schedule
  kFusedDone = 2 * kLine,
  kBlockTicket = 3 * kLine,  // ticket of XCD y at kBlockTicket + y * kLine
  kGemmDone = 11 * kLine,    // check-out count of the persistent (ticket) GEMM
  kAssistCall = 12 * kLine,  // two words: sequence number, epoch (0: finished)
  kTasksDone = 13 * kLine,   // tasks completed in the assisted call
  kCtlWords = 14 * kLine
};

__device__ __forceinline__ uint32_t next_epoch(uint32_t e) { return e + 1 == 0 ? 1 : e + 1; }

// Measurement trace of one call: wall-clock stamps (s_memrealtime), each
// workgroup writing its own slots with plain stores, so tracing adds no
// contended atomics to the kernels it measures.  GEMM: block b (dispatch
// index) of nb stores its start at trace[b] and its end (stores and flags
// issued) at trace[nb + b].  Reduction: workgroup w of a grid of g stores the
// start of its task loop at trace[w] and its end (stores issued) at
// trace[g + w].  The host zeroes the slots before the call and reduces them
// (first start, last end) after it; the paper's communication tail is the
// last reduction end minus the last GEMM block end.
__device__ __forceinline__ void trace_at(uint64_t* t, int64_t slot) {
  if (t) t[slot] = (uint64_t)wall_clock64();
}

// Counts one workgroup out of `total` (the two-stream schedule's GEMM and
// reduction workgroups together); the last one resets the count and advances
// the epoch.  Called by thread 0 after the workgroup's last flag store or
// flag read.
__device__ __forceinline__ void check_out(uint32_t* ctl, uint32_t epoch, uint32_t total) {
  const uint32_t n = __hip_atomic_fetch_add(ctl + kCallDone, 1u, __ATOMIC_RELAXED,
                                            __HIP_MEMORY_SCOPE_AGENT);
  if (n + 1 != total) return;
  __hip_atomic_store(ctl + kCallDone, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  __hip_atomic_store(ctl + kEpoch, next_epoch(epoch), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// The fused schedule: one kernel on the caller's stream.  Its workgroups take
// GEMM blocks from per-XCD lists (block b of the dispatch order belongs to
// XCD b % 8) until all are taken; then workgroup w < `workers` takes tasks w,
// w + workers, ... of r.task_list.
struct FusedArgs {
  GemmArgs g;
  ReduceArgs r;               // r.task_list: the tasks in production order
  int32_t nb;                 // GEMM blocks
  int32_t workers;            // workgroups that may reduce (the comm budget)
};

// The assisted schedule's helpers: `grid` workgroups of `threads` take tasks
// j, j + grid, ... of a.task_list once their flags are set (a.assist_seq,
// a.claims as for the fused kernel of the same call).
hipError_t launch_assist_reduce(const ReduceArgs& a, int peer_f32, int out_f32, int threads,
                                int grid, hipStream_t stream);
int assist_registers(int threads, int peer_f32, int out_f32);
// Registers per lane of a fused kernel instance (0 if not built).
int fused_registers(int bm, int bn, int variant, int peer_f32, int out_f32, bool wkn);

// GEMM block shapes built: (bm, bn) in {128, 256}^2.
hipError_t launch_gemm_publish(const GemmArgs& a, int bm, int bn, int num_blocks,
                               hipStream_t stream);
// The same GEMM as `grid` persistent workgroups that take blocks from the
// per-XCD tickets until all a.nb are taken (the two-stream schedule): a CU
// that also hosts a reduction workgroup then takes fewer blocks.  The last
// workgroup to finish resets the tickets.  Each workgroup reserves at least
// lds_min bytes of LDS (static CU partitioning: more than half of a CU's LDS
// keeps it alone on its CU).
hipError_t launch_gemm_tickets(const GemmArgs& a, int bm, int bn, int grid, hipStream_t stream,
                               int lds_min = 0);

// peer / out dtype: 0 = bf16, 1 = fp32.  threads in {128, 256, 512}.  flat:
// reduce the whole partition without flags (after the GEMM has finished).
// lds_bytes: LDS each workgroup reserves without using it (static CU
// partitioning keeps a reduction workgroup off the GEMM's CUs this way).
hipError_t launch_tile_reduce(const ReduceArgs& a, int peer_f32, int out_f32, int threads,
                              bool flat, int grid, hipStream_t stream, int lds_bytes = 0);

// Queries of the GEMM instance for a block shape, pipeline variant and W
// layout (wkn: W [K][N]).  Registers per lane (VGPRs + AGPRs) of the kernel a
// launch would use, for the co-residency check (0 if unknown or not built).
int gemm_registers(int bm, int bn, int variant, bool wkn, bool tickets = false);
// GEMM workgroups of a block shape resident per CU at once (0 if unknown).
int gemm_blocks_per_cu(int bm, int bn, int variant, bool wkn);
// LDS bytes a GEMM workgroup's pipeline uses (0 if not built).
int gemm_lds_bytes(int bm, int bn, int variant, bool wkn);
// Waves per GEMM workgroup (64 lanes each).
int gemm_waves(int bm, int bn, int variant, bool wkn);
// Whether the instance is built.
bool gemm_built(int bm, int bn, int variant, bool wkn);
int reduce_registers(int threads, int peer_f32, int out_f32);

// Zeroes `words` trace slots on `stream` (a kernel, so that a captured graph
// zeroes them on every replay).
hipError_t launch_trace_reset(uint64_t* trace, int64_t words, hipStream_t stream);

// RMSNorm of each of `rows` rows of h (out dtype [rows][N], N % 8 == 0):
// y = gamma * h / sqrt(mean(h^2) + eps), one 256-thread workgroup per row.
hipError_t launch_rmsnorm(const void* h, const void* gamma, void* y, int rows, int N, float eps,
                          int out_f32, hipStream_t stream);

// Fused kernel instances (the layout of W from a.g.w_kn): with W [N][K] the
// variant-0 pipelines of every block shape and variants 3 and 4 of
// 256 x 256; with W [K][N] the variant-0 pipelines of every shape, bf16 or
// fp32 I/O.  Returns hipErrorInvalidValue for others.
hipError_t launch_gemm_rs_fused(const FusedArgs& a, int bm, int bn, int variant, int peer_f32,
                                int out_f32, int grid, hipStream_t stream);
// Fused workgroups resident per CU (0 if the instance is not built).
int fused_blocks_per_cu(int bm, int bn, int variant, int peer_f32, int out_f32, bool wkn);

}  // namespace entwine
