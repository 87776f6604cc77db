// entwine_api.cpp -- the C ABI: validation, workspace, plans, launch.
//
// Method: "Entwine: Coordinating Tiled Computation and Fine-Grained
// Communication across GPUs" (paperpeel.com/paper/2609.11562).
//  * Sec. 4.1: partial outputs and flags live in buffers allocated once and
//    reused across invocations; flags are reset before each invocation; the
//    GEMM and the reduction kernel are launched on independent streams after a
//    common start event.
//  * Sec. 3.2 / 4.3: the reduction kernel's grid is the communication budget x,
//    capped by the partition's tile count and kept below the CU count.
//
// MI355X choices.  Flags hold the call's epoch instead of being cleared: a
// flag is ready when it equals the current epoch, which is equivalent to
// "reset, then set" without a clearing pass per call.  Cross-stream waits cost
// several µs each on this GPU, so only the two-stream schedule's reducer runs
// on an internal stream (default priority), forked from and joined back to
// the caller's stream with HIP events; the GEMM, the fused kernel, the
// sequential reduction (budget 0) and the layer chain's RMSNorm run on the
// caller's stream (the RMSNorm follows the reduction on its stream).
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cinttypes>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <map>
#include <memory>
#include <mutex>
#include <string>
#include <tuple>
#include <vector>

#include "api_internal.h"
#include "entwine.h"
#include "kernels.h"
#include "plan.h"

using namespace entwine;

namespace {

thread_local std::string g_last_error;

int fail(int status, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  g_last_error = buf;
  return status;
}

#define HIP_TRY(expr)                                                                    \
  do {                                                                                   \
    hipError_t e_ = (expr);                                                              \
    if (e_ != hipSuccess)                                                                \
      return fail(ENTWINE_ERR_HIP, "%s failed: %s", #expr, hipGetErrorString(e_));      \
  } while (0)

struct DevicePlan {
  Plan plan;
  int32_t* d_blocks = nullptr;
  int32_t* d_tiles = nullptr;
  int32_t* d_waits = nullptr;
  // Task lists in production order, by (task_slabs, push): the fused
  // schedule's, and the two-stream reducer's when it also pushes.
  std::map<std::pair<int, int>, int32_t*> d_task_list;
};

using PlanKey = std::tuple<int64_t, int64_t, int, int, int, int, int, int, int, int, int, int64_t>;

struct TimingPair {
  hipEvent_t g0, g1, r0, r1;
};

struct Workspace {
  int device = -1;
  int cus = 0;
  int lds_per_cu = 0;     // LDS bytes of one CU
  int lds_per_block = 0;  // the most one workgroup may reserve
  int wall_khz = 100000;
  hipStream_t s_red = nullptr;  // the overlapped schedule's reducer
  // ev_gemm / ev_red: the last eager call's GEMM and last reduction kernel.
  hipEvent_t ev_fork = nullptr, ev_gemm = nullptr, ev_red = nullptr;
  // Separate events for calls made while the caller's stream is being
  // captured into a graph, so that eager calls never wait on a captured record.
  hipEvent_t cap_fork = nullptr, cap_red = nullptr;
  bool have_prev = false;
  // The last eager call was assisted: its helpers (ev_red) never touch what a
  // later call uses, so later calls wait for its fused kernel (ev_gemm) only.
  bool prev_assisted = false;
  // The assisted schedule's sequence number (the last call's) and task claim
  // words (one per task, see kAssistCall in kernels.h).
  uint32_t assist_seq = 0;
  uint32_t* claims = nullptr;
  size_t claims_bytes = 0;
  float* own = nullptr;
  size_t own_bytes = 0;
  void* outgoing = nullptr;
  size_t outgoing_bytes = 0;
  void* staging = nullptr;  // pushed copies of the outgoing partials
  size_t staging_bytes = 0;
  uint32_t* flags = nullptr;
  size_t flag_count = 0;
  int32_t* error = nullptr;
  uint32_t* ctl = nullptr;  // kCtlWords device words: epoch and check-out counters
  std::map<PlanKey, std::unique_ptr<DevicePlan>> plans;
  std::vector<TimingPair> timing_live;
  std::vector<TimingPair> timing_free;
  // Trace slots of the last traced call: [2][trace_nb] GEMM block stamps, then
  // [2][trace_g] reduction workgroup stamps (see trace_at in kernels.h).
  uint64_t* trace = nullptr;
  size_t trace_bytes = 0;
  int64_t trace_nb = 0, trace_g = 0;
  bool trace_valid = false;
  // Once a call has been captured into a graph, the graph holds this
  // workspace's addresses: a buffer outgrown after that is retired (kept
  // allocated until entwine_release) instead of freed.
  bool captured = false;
  std::vector<void*> retired;
};

struct TuneEntry {
  int order, budget, bm, bn, threads, slabs, schedule, variant;
};

static_assert(kCtlWords * 4 <= kScratchError, "the control words fit before the error word");

std::mutex g_mu;
std::map<int, std::unique_ptr<Workspace>> g_ws;
std::map<std::tuple<int64_t, int64_t, int64_t, int>, TuneEntry> g_tuning;
bool g_timing = false;
bool g_trace = false;

void free_plan(DevicePlan* p) {
  if (p->d_blocks) (void)hipFree(p->d_blocks);
  if (p->d_tiles) (void)hipFree(p->d_tiles);
  if (p->d_waits) (void)hipFree(p->d_waits);
  p->d_blocks = p->d_tiles = p->d_waits = nullptr;
  for (auto& kv : p->d_task_list) (void)hipFree(kv.second);
  p->d_task_list.clear();
}

void destroy_workspace(Workspace* w) {
  int prev = -1;
  (void)hipGetDevice(&prev);
  (void)hipSetDevice(w->device);
  if (w->s_red) (void)hipStreamSynchronize(w->s_red);
  if (w->have_prev) {  // work on a caller's stream
    (void)hipEventSynchronize(w->ev_gemm);
    (void)hipEventSynchronize(w->ev_red);
  }
  for (auto& kv : w->plans) free_plan(kv.second.get());
  w->plans.clear();
  for (auto* v : {&w->timing_live, &w->timing_free})
    for (auto& t : *v) {
      (void)hipEventDestroy(t.g0);
      (void)hipEventDestroy(t.g1);
      (void)hipEventDestroy(t.r0);
      (void)hipEventDestroy(t.r1);
    }
  if (w->own) (void)hipFree(w->own);
  if (w->outgoing) (void)hipFree(w->outgoing);
  if (w->staging) (void)hipFree(w->staging);
  if (w->flags) (void)hipFree(w->flags);
  if (w->claims) (void)hipFree(w->claims);
  if (w->error) (void)hipFree(w->error);
  if (w->ctl) (void)hipFree(w->ctl);
  if (w->trace) (void)hipFree(w->trace);
  for (void* p : w->retired) (void)hipFree(p);
  w->retired.clear();
  for (hipEvent_t e : {w->cap_fork, w->cap_red})
    if (e) (void)hipEventDestroy(e);
  if (w->ev_fork) (void)hipEventDestroy(w->ev_fork);
  if (w->ev_gemm) (void)hipEventDestroy(w->ev_gemm);
  if (w->ev_red) (void)hipEventDestroy(w->ev_red);
  if (w->s_red) (void)hipStreamDestroy(w->s_red);

  if (prev >= 0) (void)hipSetDevice(prev);
}

int get_workspace(Workspace** out) {
  int dev = 0;
  HIP_TRY(hipGetDevice(&dev));
  auto it = g_ws.find(dev);
  if (it != g_ws.end()) {
    *out = it->second.get();
    return ENTWINE_OK;
  }
  auto w = std::make_unique<Workspace>();
  w->device = dev;
  HIP_TRY(hipDeviceGetAttribute(&w->cus, hipDeviceAttributeMultiprocessorCount, dev));
  HIP_TRY(hipDeviceGetAttribute(&w->lds_per_cu, hipDeviceAttributeMaxSharedMemoryPerMultiprocessor,
                                dev));
  HIP_TRY(hipDeviceGetAttribute(&w->lds_per_block, hipDeviceAttributeMaxSharedMemoryPerBlock, dev));
  int khz = 0;
  if (hipDeviceGetAttribute(&khz, hipDeviceAttributeWallClockRate, dev) == hipSuccess && khz > 0)
    w->wall_khz = khz;
  HIP_TRY(hipStreamCreateWithFlags(&w->s_red, hipStreamNonBlocking));
  HIP_TRY(hipEventCreateWithFlags(&w->ev_fork, hipEventDisableTiming));
  HIP_TRY(hipEventCreateWithFlags(&w->ev_gemm, hipEventDisableTiming));
  HIP_TRY(hipEventCreateWithFlags(&w->ev_red, hipEventDisableTiming));
  HIP_TRY(hipEventCreateWithFlags(&w->cap_fork, hipEventDisableTiming));
  HIP_TRY(hipEventCreateWithFlags(&w->cap_red, hipEventDisableTiming));
  HIP_TRY(hipMalloc(&w->error, sizeof(int32_t)));
  HIP_TRY(hipMemset(w->error, 0, sizeof(int32_t)));
  // The first call's epoch is 1: freshly allocated flags hold 0.
  const uint32_t ctl_init[kCtlWords] = {1};  // epoch 1; counters and tickets 0
  HIP_TRY(hipMalloc(&w->ctl, sizeof ctl_init));
  HIP_TRY(hipMemcpy(w->ctl, ctl_init, sizeof ctl_init, hipMemcpyHostToDevice));
  *out = w.get();
  g_ws[dev] = std::move(w);
  return ENTWINE_OK;
}

// Grow a device buffer; growth waits for all of this workspace's work.
int ensure(Workspace* w, void** buf, size_t* have, size_t need, bool zero) {
  if (*have >= need && *buf) return ENTWINE_OK;
  HIP_TRY(hipStreamSynchronize(w->s_red));
  // The previous eager call's kernels, which ran on a caller's stream too.
  if (w->have_prev) {
    HIP_TRY(hipEventSynchronize(w->ev_gemm));
    HIP_TRY(hipEventSynchronize(w->ev_red));
  }
  if (*buf) {
    if (w->captured)
      w->retired.push_back(*buf);  // a captured graph may still use it
    else
      HIP_TRY(hipFree(*buf));
    *buf = nullptr;
    *have = 0;
  }
  hipError_t e = hipMalloc(buf, need);
  if (e != hipSuccess) {
    *buf = nullptr;
    return fail(ENTWINE_ERR_OUT_OF_MEMORY, "workspace allocation of %zu bytes failed: %s",
                need, hipGetErrorString(e));
  }
  if (zero) HIP_TRY(hipMemset(*buf, 0, need));
  *have = need;
  return ENTWINE_OK;
}

int get_plan(Workspace* w, const Geometry& g, int rank, int order, int peer_ready,
             int release_group, int64_t window, DevicePlan** out) {
  PlanKey key{g.M, g.N, g.P, g.bm, g.bn, g.tm, g.tn, rank, order, peer_ready, release_group,
              window};
  auto it = w->plans.find(key);
  if (it != w->plans.end()) {
    *out = it->second.get();
    return ENTWINE_OK;
  }
  auto dp = std::make_unique<DevicePlan>();
  int rc = build_plan(g, rank, order, peer_ready, release_group, &dp->plan);
  if (rc != ENTWINE_OK) return fail(rc, "schedule construction failed");
  assign_dispatch(&dp->plan, window);
  const Plan& p = dp->plan;
  auto upload = [&](const std::vector<int32_t>& v, int32_t** d) -> int {
    HIP_TRY(hipMalloc(d, v.size() * sizeof(int32_t)));
    HIP_TRY(hipMemcpy(*d, v.data(), v.size() * sizeof(int32_t), hipMemcpyHostToDevice));
    return ENTWINE_OK;
  };
  if ((rc = upload(p.launch, &dp->d_blocks)) != ENTWINE_OK ||
      (rc = upload(p.tiles, &dp->d_tiles)) != ENTWINE_OK ||
      (rc = upload(p.waits, &dp->d_waits)) != ENTWINE_OK) {
    free_plan(dp.get());
    return rc;
  }
  *out = dp.get();
  w->plans[key] = std::move(dp);
  return ENTWINE_OK;
}

int take_timing_pair(Workspace* w, TimingPair* tp) {
  if (!w->timing_free.empty()) {
    *tp = w->timing_free.back();
    w->timing_free.pop_back();
    return ENTWINE_OK;
  }
  HIP_TRY(hipEventCreate(&tp->g0));
  HIP_TRY(hipEventCreate(&tp->g1));
  HIP_TRY(hipEventCreate(&tp->r0));
  HIP_TRY(hipEventCreate(&tp->r1));
  return ENTWINE_OK;
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

bool overlaps(const void* a, size_t na, const void* b, size_t nb) {
  const uintptr_t x = reinterpret_cast<uintptr_t>(a), y = reinterpret_cast<uintptr_t>(b);
  return x < y + nb && y < x + na;
}

int check_shape(int64_t M, int64_t N, int64_t K, int P, int rank) {
  if (M <= 0 || N <= 0 || K <= 0)
    return fail(ENTWINE_ERR_INVALID_ARGUMENT, "M, N, K_local must be positive (got %" PRId64
                ", %" PRId64 ", %" PRId64 ")", M, N, K);
  if (P < 1) return fail(ENTWINE_ERR_INVALID_ARGUMENT, "P must be >= 1 (got %d)", P);
  if (P > kMaxRanks) return fail(ENTWINE_ERR_UNSUPPORTED, "P = %d > %d is not built", P, kMaxRanks);
  if (rank < 0 || rank >= P)
    return fail(ENTWINE_ERR_INVALID_ARGUMENT, "rank %d outside [0, %d)", rank, P);
  if (M % P != 0)
    return fail(ENTWINE_ERR_INVALID_ARGUMENT, "M = %" PRId64 " is not divisible by P = %d", M, P);
  if (N % 8 != 0)
    return fail(ENTWINE_ERR_INVALID_ARGUMENT, "N = %" PRId64 " must be a multiple of 8", N);
  if (K % 64 != 0)
    return fail(ENTWINE_ERR_UNSUPPORTED, "K_local = %" PRId64 " must be a multiple of 64", K);
  const int64_t lim = (int64_t)1 << 31;
  if (M * K >= lim || N * K >= lim || M * N >= lim)
    return fail(ENTWINE_ERR_UNSUPPORTED, "operands beyond 2^31 elements are not built");
  // The kernels address a block's operand rows, an output strip and a
  // reduction task's rows through buffer descriptors with 32-bit byte offsets:
  // 384 rows of K_local bf16 values and 128 rows of N fp32 values must stay
  // below 2^31 bytes.
  if (K > ((int64_t)1 << 21) || N > ((int64_t)1 << 22))
    return fail(ENTWINE_ERR_UNSUPPORTED, "K_local above 2^21 or N above 2^22 is not built");
  return ENTWINE_OK;
}

struct Resolved {
  int bm, bn, tm, tn, threads, order, budget, peer_f32, out_f32, peer_ready, release_group,
      slabs, withhold_tile, variant, variant_auto, publish_all, stages, linear_dispatch, schedule,
      reducer_cus, push, wkn, poll_backoff;
  uint32_t timeout_ms;
};

int resolve(const entwine_config* cfg, int64_t M, int64_t N, int64_t K, int P, int tile_order,
            int comm_budget, Resolved* r) {
  entwine_config c;
  entwine_config_init(&c);
  if (cfg) {
    if (cfg->struct_size < (int32_t)offsetof(entwine_config, schedule))
      return fail(ENTWINE_ERR_INVALID_ARGUMENT, "entwine_config.struct_size too small");
    std::memcpy(&c, cfg, std::min<size_t>(sizeof c, (size_t)cfg->struct_size));
  }
  if (tile_order < ENTWINE_ORDER_AUTO || tile_order > ENTWINE_ORDER_COL_MAJOR)
    return fail(ENTWINE_ERR_INVALID_ARGUMENT, "tile_order %d out of range", tile_order);
  if (comm_budget < ENTWINE_BUDGET_AUTO)
    return fail(ENTWINE_ERR_INVALID_ARGUMENT, "comm_budget %d out of range", comm_budget);
  if (c.w_layout != ENTWINE_W_KN && c.w_layout != ENTWINE_W_NK)
    return fail(ENTWINE_ERR_INVALID_ARGUMENT, "w_layout %d out of range", c.w_layout);
  r->wkn = c.w_layout == ENTWINE_W_KN;
  if (r->wkn && N * K * 2 >= ((int64_t)1 << 31))
    return fail(ENTWINE_ERR_UNSUPPORTED, "W [K_local][N] of 2^31 bytes or more is not built");
  if ((c.peer_dtype != ENTWINE_BF16 && c.peer_dtype != ENTWINE_F32) ||
      (c.out_dtype != ENTWINE_BF16 && c.out_dtype != ENTWINE_F32))
    return fail(ENTWINE_ERR_INVALID_ARGUMENT, "peer_dtype/out_dtype must be BF16 or F32");
  if (c.peer_ready != ENTWINE_PEERS_PRESEEDED && c.peer_ready != ENTWINE_PEERS_SYMMETRIC)
    return fail(ENTWINE_ERR_INVALID_ARGUMENT, "peer_ready %d out of range", c.peer_ready);
  if (c.release_group < ENTWINE_RELEASE_OUTPUT)
    return fail(ENTWINE_ERR_INVALID_ARGUMENT, "release_group %d out of range", c.release_group);
  if (c.reducer_threads != 0 && c.reducer_threads != 128 && c.reducer_threads != 256 &&
      c.reducer_threads != 512)
    return fail(ENTWINE_ERR_INVALID_ARGUMENT, "reducer_threads must be 128, 256 or 512");

  const TuneEntry* te = nullptr;
  auto it = g_tuning.find(std::make_tuple(M, N, K, P));
  if (it != g_tuning.end()) te = &it->second;
  const int64_t R = M / P;
  r->bm = c.block_m ? c.block_m : (te ? te->bm : (R % 256 == 0 ? 256 : 128));
  r->bn = c.block_n ? c.block_n : (te ? te->bn : (N % 256 == 0 ? 256 : 128));
  r->tm = c.tile_m ? c.tile_m : 128;
  r->tn = c.tile_n ? c.tile_n : 128;
  // A reserved CU holds one reduction workgroup and nothing else, so the
  // static split takes the largest one (more loads in flight per CU).
  r->threads = c.reducer_threads ? c.reducer_threads
               : c.reducer_cus > 0 ? 512
                                   : (te ? te->threads : 256);
  r->order = tile_order != ENTWINE_ORDER_AUTO ? tile_order
                                              : (te ? te->order : ENTWINE_ORDER_INTERLEAVED);
  // With reducer_cus set, AUTO means one reduction workgroup per reserved CU
  // on two streams (static CU partitioning).
  r->budget = comm_budget != ENTWINE_BUDGET_AUTO ? comm_budget
              : c.reducer_cus > 0                ? c.reducer_cus
                                                 : (te ? te->budget : 32);
  r->peer_f32 = c.peer_dtype == ENTWINE_F32;
  r->out_f32 = c.out_dtype == ENTWINE_F32;
  r->peer_ready = c.peer_ready;
  r->release_group = c.release_group;
  r->slabs = c.task_slabs ? c.task_slabs : (te ? te->slabs : 1);
  r->schedule = c.schedule != ENTWINE_SCHEDULE_AUTO ? c.schedule
                : c.reducer_cus > 0 ? ENTWINE_SCHEDULE_STREAMS
                                    : (te && te->schedule ? te->schedule : ENTWINE_SCHEDULE_STREAMS);
  r->publish_all = c.publish_all;
  r->stages = c.stages;
  r->linear_dispatch = c.linear_dispatch;
  r->timeout_ms = c.poll_timeout_ms ? c.poll_timeout_ms : 2000;
  r->withhold_tile = c.withhold_tile - 1;
  // GEMM pipeline: explicit, or the tuning table's when the entry's block
  // shape is the one in use, else the base pipeline (internally 0).
  r->variant_auto = c.gemm_variant == ENTWINE_GEMM_AUTO;
  if (r->variant_auto)
    r->variant = te && te->bm == r->bm && te->bn == r->bn ? te->variant : 0;
  else
    r->variant = c.gemm_variant == ENTWINE_GEMM_BASE ? 0 : c.gemm_variant;
  // W [K][N] has the base pipeline only.
  if (r->wkn && r->variant_auto) r->variant = 0;
  if (r->slabs < 0 || (r->slabs > 0 && r->tm % r->slabs != 0))
    return fail(ENTWINE_ERR_INVALID_ARGUMENT, "task_slabs must divide tile_m");
  if (c.publish_all != 0 && c.publish_all != 1)
    return fail(ENTWINE_ERR_INVALID_ARGUMENT, "publish_all must be 0 or 1");
  if (c.linear_dispatch != 0 && c.linear_dispatch != 1)
    return fail(ENTWINE_ERR_INVALID_ARGUMENT, "linear_dispatch must be 0 or 1");
  if (c.stages < ENTWINE_STAGES_ALL || c.stages > ENTWINE_STAGES_REDUCE)
    return fail(ENTWINE_ERR_INVALID_ARGUMENT, "stages %d out of range", c.stages);
  if (r->schedule < ENTWINE_SCHEDULE_STREAMS || r->schedule > ENTWINE_SCHEDULE_ASSISTED)
    return fail(ENTWINE_ERR_INVALID_ARGUMENT, "schedule %d out of range", r->schedule);
  r->reducer_cus = c.reducer_cus;
  r->push = c.push_outgoing;
  if (c.poll_backoff < 0 || c.poll_backoff > 4096)
    return fail(ENTWINE_ERR_INVALID_ARGUMENT, "poll_backoff %d outside [0, 4096]", c.poll_backoff);
  r->poll_backoff = c.poll_backoff ? c.poll_backoff : 16;
  if (c.push_outgoing != 0 && c.push_outgoing != 1)
    return fail(ENTWINE_ERR_INVALID_ARGUMENT, "push_outgoing must be 0 or 1");
  if (c.reducer_cus < 0)
    return fail(ENTWINE_ERR_INVALID_ARGUMENT, "reducer_cus %d is negative", c.reducer_cus);
  return ENTWINE_OK;
}

// The layer chain after the ReduceScatter (Sec. 5.2.2): `out` receives
// h = RS + residual, and y = RMSNorm(h) with weight gamma.
struct Chain {
  const void* residual = nullptr;
  const void* gamma = nullptr;
  void* y = nullptr;
  float eps = 0.0f;
};

// Validation shared by every entry point that runs the operation: shapes,
// configuration, pointers (presence, alignment, no aliasing of the outputs).
// Nothing is enqueued.
int prepare(const void* X, const void* W, const void* const* peers, void* out, int64_t M,
            int64_t N, int64_t K, int P, int rank, int tile_order, int comm_budget,
            const entwine_config* cfg, const Chain* chain, Resolved* rs_out, Geometry* g_out) {
  int rc = check_shape(M, N, K, P, rank);
  if (rc) return rc;
  Resolved rs;
  if ((rc = resolve(cfg, M, N, K, P, tile_order, comm_budget, &rs))) return rc;
  Geometry g;
  if ((rc = make_geometry(M, N, P, rs.bm, rs.bn, rs.tm, rs.tn, &g)))
    return fail(rc, "unsupported tile geometry (block %dx%d, tile %dx%d)", rs.bm, rs.bn, rs.tm,
                rs.tn);
  if (!gemm_built(rs.bm, rs.bn, rs.variant, rs.wkn != 0))
    return fail(ENTWINE_ERR_UNSUPPORTED, "the GEMM is not built for %dx%d blocks, pipeline %d, "
                "W %s", rs.bm, rs.bn, rs.variant, rs.wkn ? "[K][N]" : "[N][K]");

  // Pointers: presence, alignment, no aliasing of the output.
  if (!X || !W || !out) return fail(ENTWINE_ERR_INVALID_ARGUMENT, "X, W and out must be non-NULL");
  if (!aligned16(X) || !aligned16(W) || !aligned16(out))
    return fail(ENTWINE_ERR_INVALID_ARGUMENT, "X, W and out must be 16-byte aligned");
  if (P > 1 && !peers) return fail(ENTWINE_ERR_INVALID_ARGUMENT, "peer_partials is NULL");
  const size_t peer_sz = rs.peer_f32 ? 4 : 2, out_sz = rs.out_f32 ? 4 : 2;
  const size_t out_bytes = (size_t)g.R * N * out_sz;
  if (overlaps(out, out_bytes, X, (size_t)M * K * 2) || overlaps(out, out_bytes, W, (size_t)N * K * 2))
    return fail(ENTWINE_ERR_INVALID_ARGUMENT, "out overlaps X or W");
  for (int r = 0; r < P; ++r) {
    if (r == rank) continue;
    if (!peers[r]) return fail(ENTWINE_ERR_INVALID_ARGUMENT, "peer_partials[%d] is NULL", r);
    if (!aligned16(peers[r]))
      return fail(ENTWINE_ERR_INVALID_ARGUMENT, "peer_partials[%d] is not 16-byte aligned", r);
    if (overlaps(out, out_bytes, peers[r], (size_t)g.R * N * peer_sz))
      return fail(ENTWINE_ERR_INVALID_ARGUMENT, "out overlaps peer_partials[%d]", r);
  }
  if (chain) {
    if (!chain->residual || !chain->gamma || !chain->y)
      return fail(ENTWINE_ERR_INVALID_ARGUMENT, "residual, gamma and y_out must be non-NULL");
    if (!aligned16(chain->residual) || !aligned16(chain->gamma) || !aligned16(chain->y))
      return fail(ENTWINE_ERR_INVALID_ARGUMENT, "residual, gamma and y_out must be 16-byte aligned");
    if (!(chain->eps >= 0.0f) || chain->eps > 3.0e38f)
      return fail(ENTWINE_ERR_INVALID_ARGUMENT, "eps must be finite and >= 0");
    const size_t g_bytes = (size_t)N * out_sz;
    const void* y = chain->y;
    if (overlaps(y, out_bytes, X, (size_t)M * K * 2) || overlaps(y, out_bytes, W, (size_t)N * K * 2) ||
        overlaps(y, out_bytes, out, out_bytes) || overlaps(y, out_bytes, chain->residual, out_bytes) ||
        overlaps(y, out_bytes, chain->gamma, g_bytes))
      return fail(ENTWINE_ERR_INVALID_ARGUMENT, "y_out overlaps another operand");
    for (int r = 0; r < P; ++r)
      if (r != rank && overlaps(y, out_bytes, peers[r], (size_t)g.R * N * peer_sz))
        return fail(ENTWINE_ERR_INVALID_ARGUMENT, "y_out overlaps peer_partials[%d]", r);
    if (chain->residual != out && overlaps(chain->residual, out_bytes, out, out_bytes))
      return fail(ENTWINE_ERR_INVALID_ARGUMENT, "residual must be h_out itself or not overlap it");
    if (overlaps(chain->gamma, g_bytes, out, out_bytes))
      return fail(ENTWINE_ERR_INVALID_ARGUMENT, "gamma overlaps h_out");
  }

  *rs_out = rs;
  *g_out = g;
  return ENTWINE_OK;
}

// The device buffers a call runs on: the library workspace's, or the
// caller-free scratch of entwine_gemm_rs_noalloc.
struct Buffers {
  float* own = nullptr;
  void* outgoing = nullptr;
  void* staging = nullptr;
  uint32_t* flags = nullptr;
  int32_t* error = nullptr;
  uint32_t* ctl = nullptr;
  const int32_t* blocks = nullptr;
  const int32_t* tiles = nullptr;
  const int32_t* waits = nullptr;
  const int32_t* task_list = nullptr;
  int wait_slots = 0;
};

// Kernel arguments common to every schedule (the schedule-specific fields --
// publication, grids, task counts -- are set by the caller).
void fill_args(const Resolved& rs, const Geometry& g, const void* X, const void* W,
               const void* const* peers, void* out, int64_t M, int64_t N, int64_t K, int P,
               int rank, const Chain* chain, const Buffers& b, uint64_t timeout_ticks,
               GemmArgs* ga_out, ReduceArgs* ra_out) {
  GemmArgs ga{};
  ga.X = static_cast<const uint16_t*>(X);
  ga.W = static_cast<const uint16_t*>(W);
  ga.own = b.own;
  ga.outgoing = b.outgoing;
  ga.flags = b.flags;
  ga.blocks = b.blocks;
  ga.M = (int32_t)M;
  ga.N = (int32_t)N;
  ga.K = (int32_t)K;
  ga.R = (int32_t)g.R;
  ga.rank = rank;
  ga.Q = (int32_t)g.Q;
  ga.Rt = (int32_t)g.Rt;
  ga.Ct = (int32_t)g.Ct;
  ga.tm = g.tm;
  ga.tn = g.tn;
  ga.outgoing_f32 = rs.peer_f32;
  ga.variant = rs.variant;
  ga.w_kn = rs.wkn;
  ga.ctl = b.ctl;
  ga.nb = (int32_t)g.NB;

  ReduceArgs ra{};
  ra.own = b.own;
  for (int r = 0; r < P; ++r) ra.peers[r] = r == rank ? nullptr : peers[r];
  ra.out = out;
  ra.flags = b.flags;
  ra.waits = b.waits;
  ra.tiles = b.tiles;
  ra.error = b.error;
  ra.R = (int32_t)g.R;
  ra.N = (int32_t)N;
  ra.P = P;
  ra.rank = rank;
  ra.Q = (int32_t)g.Q;
  ra.wait_slots = b.wait_slots;
  ra.tm = g.tm;
  ra.tn = g.tn;
  ra.ctl = b.ctl;
  ra.timeout_ticks = timeout_ticks;
  ra.withhold_tile = rs.withhold_tile;
  ra.never_flag = (int32_t)(g.P * g.Q);
  ra.outgoing = b.outgoing;
  ra.staging = rs.push ? b.staging : nullptr;
  ra.residual = chain ? chain->residual : nullptr;
  ra.task_list = b.task_list;
  ra.nap_max = rs.poll_backoff;
  // Preseeded peers (and the residual) exist before the call: a task may load
  // them before its wait.  Under symmetric readiness they count as produced
  // with the tiles, so they are read only after the wait.
  ra.prefetch = rs.peer_ready == ENTWINE_PEERS_PRESEEDED;
  *ga_out = ga;
  *ra_out = ra;
}

// Flags a call's GEMM publishes: tiles a kernel on this device reads are
// released (publish 1: the rank's own tiles; 2: every tile, when peer-bound
// tiles are pushed or published too); flags of peer-bound tiles are stored
// when some wait reads them (send tasks, symmetric peers, release groups).
void set_publication(const Resolved& rs, GemmArgs* ga) {
  ga->publish = rs.publish_all || rs.push ? 2 : 1;
  ga->flag_all = rs.publish_all || rs.push || rs.peer_ready == ENTWINE_PEERS_SYMMETRIC ||
                 rs.release_group != ENTWINE_RELEASE_TILE;
}

// The sequential schedule's reduction grid: up to 8 workgroups per CU over
// the partition's 8-element chunks, two chunks per thread.
int flat_grid(const Geometry& g, int64_t N, int threads, int cus) {
  const int64_t chunks = g.R * N / 8;
  const int64_t per_wg = (int64_t)threads * 2;
  return (int)std::max<int64_t>(1, std::min<int64_t>((chunks + per_wg - 1) / per_wg,
                                                      (int64_t)8 * cus));
}

int run(const void* X, const void* W, const void* const* peers, void* out, int64_t M, int64_t N,
        int64_t K, int P, int rank, int tile_order, int comm_budget, void* stream_,
        const entwine_config* cfg, const Chain* chain = nullptr) {
  Resolved rs;
  Geometry g;
  int rc = prepare(X, W, peers, out, M, N, K, P, rank, tile_order, comm_budget, cfg, chain, &rs,
                   &g);
  if (rc) return rc;
  hipStream_t stream = static_cast<hipStream_t>(stream_);
  hipStreamCaptureStatus cap = hipStreamCaptureStatusNone;
  HIP_TRY(hipStreamIsCapturing(stream, &cap));
  const bool capturing = cap != hipStreamCaptureStatusNone;

  std::lock_guard<std::mutex> lock(g_mu);
  if (capturing) {
    int dev = 0;
    HIP_TRY(hipGetDevice(&dev));
    if (g_ws.find(dev) == g_ws.end())
      return fail(ENTWINE_ERR_INVALID_ARGUMENT,
                  "no workspace on this device: make the same call once outside the capture");
    if (g_timing)
      return fail(ENTWINE_ERR_INVALID_ARGUMENT, "entwine_timing cannot record inside a capture");
  }
  Workspace* w = nullptr;
  if ((rc = get_workspace(&w))) return rc;
  if (capturing) w->captured = true;
  if (rs.budget >= w->cus)
    return fail(ENTWINE_ERR_INVALID_ARGUMENT,
                "comm_budget %d must stay below the device's %d compute units", rs.budget, w->cus);

  const bool sequential = (rs.budget == ENTWINE_BUDGET_SEQUENTIAL);
  const bool fused = !sequential && rs.stages == ENTWINE_STAGES_ALL &&
                     (rs.schedule == ENTWINE_SCHEDULE_FUSED ||
                      rs.schedule == ENTWINE_SCHEDULE_ASSISTED);
  // The assisted schedule's helpers run eagerly only: inside a capture the
  // fused kernel does every task.
  const bool assisted = fused && rs.schedule == ENTWINE_SCHEDULE_ASSISTED && !capturing;
  if (rs.push && sequential)
    return fail(ENTWINE_ERR_UNSUPPORTED, "push_outgoing applies to the overlapped schedules "
                "(comm_budget >= 1)");
  if (rs.push && fused && rs.schedule == ENTWINE_SCHEDULE_ASSISTED)
    return fail(ENTWINE_ERR_UNSUPPORTED, "push_outgoing is built for the two-stream and fused "
                "schedules, not the assisted one");
  // A list of tasks in production order: always for the fused kernel, and for
  // the two-stream reducer when it also pushes.
  const bool listed = !sequential && (fused || rs.push);
  const int slabs_eff = rs.slabs ? rs.slabs : 1;
  int fused_per_cu = 0;
  if (fused) {
    fused_per_cu = fused_blocks_per_cu(g.bm, g.bn, rs.variant, rs.peer_f32, rs.out_f32, rs.wkn);
    if (fused_per_cu <= 0)
      return fail(ENTWINE_ERR_UNSUPPORTED, "the fused schedule is not built for %dx%d blocks, "
                  "GEMM variant %d", g.bm, g.bn, rs.variant);
  }
  if (assisted) {
    // The helpers help only beside the fused kernel's workgroups: one helper
    // workgroup must fit on a CU that holds a fused one.
    const int hr = assist_registers(rs.threads, rs.peer_f32, rs.out_f32);
    const int fr = fused_registers(g.bm, g.bn, rs.variant, rs.peer_f32, rs.out_f32, rs.wkn);
    if (hr <= 0 || fr <= 0) return fail(ENTWINE_ERR_HIP, "kernel register counts unavailable");
    auto up8 = [](int v) { return (v + 7) / 8 * 8; };
    const int fw = (gemm_waves(g.bm, g.bn, rs.variant, rs.wkn) + 3) / 4;
    const int hw = (rs.threads / 64 + 3) / 4;
    if (fw * up8(fr) + hw * up8(hr) > 512)
      return fail(ENTWINE_ERR_UNSUPPORTED,
                  "a %d-thread helper workgroup (%d registers per lane) cannot share a CU with "
                  "a %dx%d fused workgroup (%d registers per lane)",
                  rs.threads, hr, g.bm, g.bn, fr);
  }
  // Static CU partitioning (Sec. 5.3.3): the reduction's x workgroups on x
  // CUs of their own, the GEMM's persistent workgroups on the other CUs.
  // CU-masked streams would say this directly, but partial masks failed or
  // crashed inside the HIP runtime on MI355X; LDS reservations say it instead.
  // Every workgroup of either kernel reserves more than half of a CU's LDS,
  // and a GEMM and a reduction workgroup together more than all of it, so no
  // CU ever holds two of them: the CUs - x GEMM workgroups and the x reduction
  // workgroups take CUs - x and x distinct CUs (exactly x per XCD group when
  // x is a multiple of the 8 XCDs).  Nothing waits on a workgroup that is not
  // resident: the GEMM's workgroups never wait for the reduction, and a
  // workgroup left undispatched runs once one ahead of it ends.
  const bool static_cus = rs.reducer_cus > 0 && !sequential && rs.stages == ENTWINE_STAGES_ALL;
  int lds_gemm = 0, lds_red = 0;
  if (static_cus) {
    if (rs.reducer_cus >= w->cus)
      return fail(ENTWINE_ERR_INVALID_ARGUMENT, "reducer_cus %d must stay below the device's "
                  "%d compute units", rs.reducer_cus, w->cus);
    if (fused)
      return fail(ENTWINE_ERR_UNSUPPORTED, "static CU partitioning (reducer_cus > 0) is built "
                  "for the two-stream schedule; the fused kernel's workgroups do both tasks");
    if (rs.budget != rs.reducer_cus)
      return fail(ENTWINE_ERR_INVALID_ARGUMENT, "comm_budget %d must equal reducer_cus %d: one "
                  "reduction workgroup per reserved CU", rs.budget, rs.reducer_cus);
    const int half = w->lds_per_cu / 2 + 1024;
    lds_gemm = std::max(gemm_lds_bytes(g.bm, g.bn, rs.variant, rs.wkn), half);
    lds_red = std::max(half, w->lds_per_cu - lds_gemm + 1024);
    if (w->lds_per_cu <= 0 || lds_gemm > w->lds_per_block || lds_red > w->lds_per_block)
      return fail(ENTWINE_ERR_UNSUPPORTED, "static CU partitioning needs LDS reservations of "
                  "%d and %d bytes; a workgroup may reserve %d of the CU's %d", lds_gemm,
                  lds_red, w->lds_per_block, w->lds_per_cu);
  }
  if (!sequential && !fused && !static_cus && rs.stages == ENTWINE_STAGES_ALL) {
    // The reduction workgroups wait for GEMM blocks, so a CU holding one
    // must still fit a GEMM block: otherwise reduction workgroups spread
    // over the device could starve the GEMM until the watchdog fires.
    const int red_waves_per_simd = (rs.threads / 64 + 3) / 4;
    const int rr = reduce_registers(rs.threads, rs.peer_f32, rs.out_f32);
    auto up8 = [](int v) { return (v + 7) / 8 * 8; };
    auto fits = [&](int variant, int* gr) {
      *gr = gemm_registers(g.bm, g.bn, variant, rs.wkn, /*tickets=*/true);
      const int gemm_waves_per_simd = (gemm_waves(g.bm, g.bn, variant, rs.wkn) + 3) / 4;
      return gemm_waves_per_simd * up8(*gr) + red_waves_per_simd * up8(rr) <= 512;
    };
    int gr = 0;
    bool ok = fits(rs.variant, &gr);
    // An automatically chosen pipeline that leaves no room for the reducer
    // gives way to the base pipeline (same accumulation order, same result).
    if (!ok && rs.variant_auto && rs.variant != 0) {
      rs.variant = 0;
      ok = fits(0, &gr);
    }
    if (gr <= 0 || rr <= 0)
      return fail(ENTWINE_ERR_HIP, "kernel register counts unavailable");
    if (!ok)
      return fail(ENTWINE_ERR_UNSUPPORTED,
                  "a %d-thread reduction workgroup (%d registers per lane) cannot share a CU "
                  "with a %dx%d GEMM block (%d registers per lane)",
                  rs.threads, rr, g.bm, g.bn, gr);
  }

  // Blocks resident at once: the window inside which dispatch is XCD-aware.
  int64_t window = 0;
  if (!rs.linear_dispatch) {
    const int per_cu = gemm_blocks_per_cu(g.bm, g.bn, rs.variant, rs.wkn);
    window = (int64_t)std::max(per_cu, 1) * w->cus;
  }

  const size_t peer_sz = rs.peer_f32 ? 4 : 2;
  const size_t own_need = (size_t)g.R * N * 4, og_need = (size_t)M * N * peer_sz;
  // One slot past the P x Q flags is never written by any GEMM (failure injection).
  const size_t flag_need = ((size_t)g.P * g.Q + 1) * 4;
  if (capturing) {
    // Allocation, upload and synchronization are not allowed while capturing.
    PlanKey key{g.M, g.N, g.P, g.bm, g.bn, g.tm, g.tn, rank, rs.order, rs.peer_ready,
                rs.release_group, window};
    auto pit = w->plans.find(key);
    if (w->own_bytes < own_need || w->outgoing_bytes < og_need || w->flag_count * 4 < flag_need ||
        (rs.push && w->staging_bytes < og_need) || pit == w->plans.end() ||
        (listed && !pit->second->d_task_list.count({slabs_eff, rs.push})))
      return fail(ENTWINE_ERR_INVALID_ARGUMENT,
                  "the workspace and schedule for this shape must exist before a graph capture: "
                  "make the same call once outside the capture");
  }
  if ((rc = ensure(w, (void**)&w->own, &w->own_bytes, own_need, false))) return rc;
  if ((rc = ensure(w, &w->outgoing, &w->outgoing_bytes, og_need, false))) return rc;
  if (rs.push && (rc = ensure(w, &w->staging, &w->staging_bytes, og_need, false))) return rc;
  size_t flag_bytes = w->flag_count * 4;
  if ((rc = ensure(w, (void**)&w->flags, &flag_bytes, flag_need, true))) return rc;
  w->flag_count = flag_bytes / 4;
  if (assisted &&
      (rc = ensure(w, (void**)&w->claims, &w->claims_bytes, (size_t)g.Q * slabs_eff * 4, true)))
    return rc;
  // Tracing: the call's slots are sized once its grids are known (arm_trace).
  uint64_t* trace = nullptr;
  auto arm_trace = [&](int64_t nb, int64_t grid_red, hipStream_t s) -> int {
    if (!g_trace) return ENTWINE_OK;
    const size_t need = (size_t)2 * (nb + grid_red) * sizeof(uint64_t);
    if (w->trace_bytes < need) {
      if (capturing)
        return fail(ENTWINE_ERR_INVALID_ARGUMENT, "tracing is on: make the same call once "
                    "outside the capture first");
      if (w->trace) {
        if (w->captured) {
          w->retired.push_back(w->trace);  // a captured graph may still use it
        } else {
          // Kernels of earlier calls may still write their stamps: the
          // internal stream's (an assisted call's helpers are never joined)
          // and the previous eager call's.
          if (hipStreamSynchronize(w->s_red) != hipSuccess ||
              (w->have_prev && (hipEventSynchronize(w->ev_gemm) != hipSuccess ||
                                hipEventSynchronize(w->ev_red) != hipSuccess)))
            return fail(ENTWINE_ERR_HIP, "trace slots: synchronization failed");
          (void)hipFree(w->trace);
        }
      }
      w->trace = nullptr;
      w->trace_bytes = 0;
      if (hipMalloc((void**)&w->trace, need) != hipSuccess) {
        w->trace = nullptr;
        return fail(ENTWINE_ERR_OUT_OF_MEMORY, "trace slots: allocation failed");
      }
      w->trace_bytes = need;
    }
    trace = w->trace;
    w->trace_nb = nb;
    w->trace_g = grid_red;
    w->trace_valid = true;
    // Zeroed by a kernel, so that a captured call zeroes them on every replay.
    const hipError_t e = launch_trace_reset(trace, (int64_t)(need / sizeof(uint64_t)), s);
    if (e != hipSuccess) return fail(ENTWINE_ERR_HIP, "trace reset: %s", hipGetErrorString(e));
    return ENTWINE_OK;
  };

  DevicePlan* dp = nullptr;
  if ((rc = get_plan(w, g, rank, rs.order, rs.peer_ready, rs.release_group, window, &dp)))
    return rc;

  int32_t* d_task_list = nullptr;
  if (listed) {
    auto it = dp->d_task_list.find({slabs_eff, rs.push});
    if (it == dp->d_task_list.end()) {
      const std::vector<int32_t> order = task_list(dp->plan, slabs_eff, rs.push != 0);
      HIP_TRY(hipMalloc(&d_task_list, order.size() * sizeof(int32_t)));
      dp->d_task_list[{slabs_eff, rs.push}] = d_task_list;
      HIP_TRY(hipMemcpy(d_task_list, order.data(), order.size() * sizeof(int32_t),
                        hipMemcpyHostToDevice));
    } else {
      d_task_list = it->second;
    }
  }

  TimingPair tp{};
  if (g_timing && (rc = take_timing_pair(w, &tp))) return rc;

  Buffers bufs;
  bufs.own = w->own;
  bufs.outgoing = w->outgoing;
  bufs.staging = w->staging;
  bufs.flags = w->flags;
  bufs.error = w->error;
  bufs.ctl = w->ctl;
  bufs.blocks = dp->d_blocks;
  bufs.tiles = dp->d_tiles;
  bufs.waits = dp->d_waits;
  bufs.task_list = d_task_list;
  bufs.wait_slots = dp->plan.wait_slots;
  GemmArgs ga;
  ReduceArgs ra;
  fill_args(rs, g, X, W, peers, out, M, N, K, P, rank, chain, bufs,
            (uint64_t)rs.timeout_ms * (uint64_t)w->wall_khz, &ga, &ra);

  if (fused) {
    // One kernel on the caller's stream, after this workspace's previous
    // eager call (which may have run on other streams).
    set_publication(rs, &ga);
    ra.slabs = slabs_eff;
    ra.ntasks = (int32_t)(g.Q * ra.slabs * (rs.push ? g.P : 1));
    FusedArgs fa{};
    fa.g = ga;
    fa.r = ra;
    fa.nb = (int32_t)g.NB;
    fa.workers = (int32_t)std::min<int64_t>(rs.budget, ra.ntasks);
    // Resident workgroups, but no more than there is work for.
    const int64_t grid =
        std::min<int64_t>((int64_t)fused_per_cu * w->cus, g.NB + (int64_t)fa.workers);
    if (w->have_prev && !capturing) {
      HIP_TRY(hipStreamWaitEvent(stream, w->ev_gemm, 0));
      if (!w->prev_assisted) HIP_TRY(hipStreamWaitEvent(stream, w->ev_red, 0));
    }
    // The assisted schedule's helpers: x workgroups on the internal stream.
    const int hgrid = assisted ? (int)std::min<int64_t>(rs.budget, ra.ntasks) : 0;
    if ((rc = arm_trace(g.NB, grid + hgrid, stream))) return rc;
    if (trace) {
      fa.g.trace = trace;
      fa.g.trace_nb = (int32_t)g.NB;
      fa.r.trace = trace + 2 * g.NB;
      fa.r.trace_g = (int32_t)(grid + hgrid);
    }
    if (assisted) {
      // A fresh sequence number (never 0), and the fork: the helpers start
      // after the caller's earlier work, which wrote the inputs.  No join:
      // the fused kernel ends only once every task is done.
      if (++w->assist_seq == 0x80000000u) {
        // Claim words and the liveness word compare sequence numbers within
        // half the 32-bit range: before leaving it, wait until no kernel of
        // an earlier call runs, clear both and start again from 1.
        HIP_TRY(hipStreamSynchronize(stream));
        HIP_TRY(hipStreamSynchronize(w->s_red));
        HIP_TRY(hipMemset(w->claims, 0, w->claims_bytes));
        HIP_TRY(hipMemset(w->ctl + kAssistCall, 0, 2 * sizeof(uint32_t)));
        w->assist_seq = 1;
      }
      fa.r.assist_seq = w->assist_seq;
      fa.r.claims = w->claims;
      HIP_TRY(hipEventRecord(w->ev_fork, stream));
      HIP_TRY(hipStreamWaitEvent(w->s_red, w->ev_fork, 0));
    }
    if (g_timing) {
      HIP_TRY(hipEventRecord(tp.g0, stream));
      HIP_TRY(hipEventRecord(tp.r0, stream));
    }
    hipError_t e = launch_gemm_rs_fused(fa, g.bm, g.bn, rs.variant, rs.peer_f32, rs.out_f32,
                                        (int)grid, stream);
    if (e != hipSuccess)
      return fail(ENTWINE_ERR_HIP, "fused launch failed: %s", hipGetErrorString(e));
    if (assisted) {
      ReduceArgs ha = fa.r;
      ha.trace_slot0 = (int32_t)grid;
      if ((e = launch_assist_reduce(ha, rs.peer_f32, rs.out_f32, rs.threads, hgrid, w->s_red)) !=
          hipSuccess)
        return fail(ENTWINE_ERR_HIP, "helper launch failed: %s", hipGetErrorString(e));
      HIP_TRY(hipEventRecord(w->ev_red, w->s_red));
    }
    if (chain && (e = launch_rmsnorm(out, chain->gamma, chain->y, (int)g.R, (int)N, chain->eps,
                                     rs.out_f32, stream)) != hipSuccess)
      return fail(ENTWINE_ERR_HIP, "RMSNorm launch failed: %s", hipGetErrorString(e));
    if (g_timing) {
      HIP_TRY(hipEventRecord(tp.g1, stream));
      HIP_TRY(hipEventRecord(tp.r1, stream));
      w->timing_live.push_back(tp);
    }
    if (!capturing) {
      HIP_TRY(hipEventRecord(w->ev_gemm, stream));
      if (!assisted) HIP_TRY(hipEventRecord(w->ev_red, stream));
      w->have_prev = true;
      w->prev_assisted = assisted;
    }
    return ENTWINE_OK;
  }

  // Sequential schedule (budget 0): the GEMM publishes nothing and the
  // reduction streams the whole partition after the GEMM kernel has ended.
  // Overlapped schedule: the GEMM releases its tiles and x persistent
  // reduction workgroups consume them as they become ready.
  int grid;
  if (sequential) {
    ga.publish = 0;
    ra.slabs = 1;
    ra.ntasks = 0;
    grid = flat_grid(g, N, rs.threads, w->cus);
  } else {
    set_publication(rs, &ga);
    ra.slabs = slabs_eff;
    ra.ntasks = (int32_t)(g.Q * ra.slabs * (rs.push ? g.P : 1));
    grid = (int)std::min<int64_t>(rs.budget, ra.ntasks);  // x, capped by the task count
  }

  // Measurement stages: one kernel alone, outside the flag protocol.
  const bool run_gemm = rs.stages != ENTWINE_STAGES_REDUCE;
  const bool run_red = rs.stages != ENTWINE_STAGES_GEMM;
  if (rs.stages != ENTWINE_STAGES_ALL) {
    ga.publish = 0;
    ra.nowait = 1;
  }

  // Everything but the overlapped schedule's reducer runs on the caller's
  // stream: the GEMM, the sequential reduction, a single stage.  The reducer
  // runs on an internal stream forked from the caller's stream just before
  // the GEMM, and the caller's stream joins it after the GEMM; cross-stream
  // waits cost several µs each, so no other stream is forked.  The work
  // starts after this workspace's previous eager call.  Inside a capture the
  // graph's own edges order the work and the capture events are used instead.
  const bool forked = !sequential && rs.stages == ENTWINE_STAGES_ALL;
  hipStream_t s_red = forked ? w->s_red : stream;
  hipEvent_t ev_fork = capturing ? w->cap_fork : w->ev_fork;
  hipEvent_t ev_red = capturing ? w->cap_red : w->ev_red;
  if (w->have_prev && !capturing) {
    HIP_TRY(hipStreamWaitEvent(stream, w->ev_gemm, 0));
    if (!w->prev_assisted) HIP_TRY(hipStreamWaitEvent(stream, w->ev_red, 0));
  }
  if ((rc = arm_trace(run_gemm ? g.NB : 0, run_red ? grid : 0, stream))) return rc;
  if (trace) {
    ga.trace = run_gemm ? trace : nullptr;
    ga.trace_nb = (int32_t)g.NB;
    ra.trace = run_red ? trace + 2 * (run_gemm ? g.NB : 0) : nullptr;
  }
  if (forked) {
    HIP_TRY(hipEventRecord(ev_fork, stream));
    HIP_TRY(hipStreamWaitEvent(s_red, ev_fork, 0));
  }

  if (g_timing) HIP_TRY(hipEventRecord(tp.g0, stream));
  if (run_gemm) {
    // Beside the two-stream reduction the GEMM's workgroups take blocks from
    // tickets: a CU that also runs a reduction workgroup is slower and takes
    // fewer blocks.  With a fixed deal, a budget of 16 to 64 workgroups
    // delayed the whole large_mlp GEMM by 10-25 % (the CUs that hosted busy
    // reducers finished their blocks last).
    hipError_t e;
    if (forked) {
      // Static partitioning: one workgroup on each CU not reserved for the
      // reduction.
      const int per_cu = static_cus ? 1 : std::max(gemm_blocks_per_cu(g.bm, g.bn, rs.variant, rs.wkn), 1);
      const int gemm_cus = static_cus ? w->cus - rs.reducer_cus : w->cus;
      const int64_t gemm_grid = std::min<int64_t>((int64_t)per_cu * gemm_cus, g.NB);
      // Both kernels' workgroups check out on one count; the last advances
      // the epoch, once no workgroup of the call can still store a flag.
      ga.checkout_total = ra.checkout_total = (int32_t)(gemm_grid + grid);
      e = launch_gemm_tickets(ga, g.bm, g.bn, (int)gemm_grid, stream, lds_gemm);
    } else {
      e = launch_gemm_publish(ga, g.bm, g.bn, (int)g.NB, stream);
    }
    if (e != hipSuccess)
      return fail(ENTWINE_ERR_HIP, "GEMM launch failed: %s", hipGetErrorString(e));
  }
  if (g_timing) HIP_TRY(hipEventRecord(tp.g1, stream));
  if (!capturing) HIP_TRY(hipEventRecord(w->ev_gemm, stream));
  if (g_timing) HIP_TRY(hipEventRecord(tp.r0, s_red));
  if (run_red) {
    hipError_t e =
        launch_tile_reduce(ra, rs.peer_f32, rs.out_f32, rs.threads, sequential, grid, s_red,
                           lds_red);
    if (e != hipSuccess)
      return fail(ENTWINE_ERR_HIP, "reduction launch failed: %s", hipGetErrorString(e));
    // The chain's normalization needs whole rows: after the reduction.
    if (chain && (e = launch_rmsnorm(out, chain->gamma, chain->y, (int)g.R, (int)N, chain->eps,
                                     rs.out_f32, s_red)) != hipSuccess)
      return fail(ENTWINE_ERR_HIP, "RMSNorm launch failed: %s", hipGetErrorString(e));
  }
  if (g_timing) HIP_TRY(hipEventRecord(tp.r1, s_red));
  if (forked || !capturing) HIP_TRY(hipEventRecord(ev_red, s_red));
  if (!capturing) {
    w->have_prev = true;
    w->prev_assisted = false;
  }
  // Join: the caller's stream continues after the reducer too.
  if (forked) HIP_TRY(hipStreamWaitEvent(stream, ev_red, 0));
  if (g_timing) w->timing_live.push_back(tp);
  return ENTWINE_OK;
}

// Host-side state of the no-alloc path on one device: the schedule tables
// its scratch holds (their key), and their host copy, the source of the last
// upload.
struct NoAllocTables {
  bool valid = false;
  std::tuple<PlanKey, int, int> key;
  std::vector<int32_t> host;
  size_t bytes = 0;
};
std::map<int, NoAllocTables> g_noalloc;

size_t up256(size_t v) { return (v + 255) & ~size_t(255); }

}  // namespace

namespace entwine {

int report(int status, const char* message) { return fail(status, "%s", message); }

int run_noalloc(void* scratch, size_t scratch_bytes, const void* X, const void* W,
                const void* const* peers, void* out, int64_t M, int64_t N, int64_t K, int P,
                int rank, int tile_order, int comm_budget, hipStream_t stream,
                const entwine_config* cfg) {
  Resolved rs;
  Geometry g;
  int rc = prepare(X, W, peers, out, M, N, K, P, rank, tile_order, comm_budget, cfg, nullptr,
                   &rs, &g);
  if (rc) return rc;
  int dev = 0, cus = 0, khz = 0;
  HIP_TRY(hipGetDevice(&dev));
  HIP_TRY(hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev));
  if (hipDeviceGetAttribute(&khz, hipDeviceAttributeWallClockRate, dev) != hipSuccess || khz <= 0)
    khz = 100000;
  if (rs.budget >= cus)
    return fail(ENTWINE_ERR_INVALID_ARGUMENT,
                "comm_budget %d must stay below the device's %d compute units", rs.budget, cus);
  const bool sequential = rs.budget == ENTWINE_BUDGET_SEQUENTIAL;
  // Only schedules that run on the caller's stream alone: a second stream and
  // its events would be allocations.
  if (cfg && cfg->struct_size >= (int32_t)(offsetof(entwine_config, schedule) + sizeof(int32_t)) &&
      (cfg->schedule == ENTWINE_SCHEDULE_STREAMS || cfg->schedule == ENTWINE_SCHEDULE_ASSISTED) &&
      !sequential)
    return fail(ENTWINE_ERR_UNSUPPORTED, "the no-alloc entry point runs the sequential and the "
                "fused schedules only (the two-stream and assisted schedules need a stream and "
                "events)");
  if (rs.reducer_cus > 0 && !sequential)
    return fail(ENTWINE_ERR_UNSUPPORTED, "static CU partitioning (reducer_cus) runs on two "
                "streams: not available without allocation");
  if (rs.stages != ENTWINE_STAGES_ALL)
    return fail(ENTWINE_ERR_UNSUPPORTED, "measurement stages are not available without allocation");
  if (rs.push && sequential)
    return fail(ENTWINE_ERR_UNSUPPORTED, "push_outgoing applies to the overlapped schedules "
                "(comm_budget >= 1)");
  std::lock_guard<std::mutex> lock(g_mu);
  if (g_timing || g_trace)
    return fail(ENTWINE_ERR_UNSUPPORTED, "entwine_timing and entwine_trace record into allocated "
                "memory: turn them off for the no-alloc entry point");

  int fused_per_cu = 0;
  if (!sequential) {
    fused_per_cu = fused_blocks_per_cu(g.bm, g.bn, rs.variant, rs.peer_f32, rs.out_f32, rs.wkn);
    if (fused_per_cu <= 0 && rs.variant_auto && rs.variant != 0) {
      rs.variant = 0;  // same accumulation order, same result
      fused_per_cu = fused_blocks_per_cu(g.bm, g.bn, 0, rs.peer_f32, rs.out_f32, rs.wkn);
    }
    if (fused_per_cu <= 0)
      return fail(ENTWINE_ERR_UNSUPPORTED, "the fused schedule is not built for %dx%d blocks, "
                  "GEMM variant %d", g.bm, g.bn, rs.variant);
  }
  const int slabs = rs.slabs ? rs.slabs : 1;
  int64_t window = 0;
  if (!rs.linear_dispatch)
    window = (int64_t)std::max(gemm_blocks_per_cu(g.bm, g.bn, rs.variant, rs.wkn), 1) * cus;

  // Schedule tables (host-built, cached by key; uploaded into the scratch
  // when the key changes).
  const size_t flag_words = (size_t)g.P * (size_t)g.Q + 1;
  if (flag_words > kScratchFlagWords)
    return fail(ENTWINE_ERR_OUT_OF_MEMORY, "%zu tile flags exceed the no-alloc scratch's %zu",
                flag_words, kScratchFlagWords);
  NoAllocTables& nt = g_noalloc[dev];
  const auto key = std::make_tuple(PlanKey{g.M, g.N, g.P, g.bm, g.bn, g.tm, g.tn, rank, rs.order,
                                           rs.peer_ready, rs.release_group, window},
                                   sequential ? 0 : slabs, sequential ? 0 : rs.push + 1);
  size_t n_blocks = 0, n_tiles = 0, n_waits = 0, n_tasks = 0;
  int wait_slots = 0;
  std::vector<int32_t> host;
  if (!(nt.valid && nt.key == key)) {
    Plan plan;
    if ((rc = build_plan(g, rank, rs.order, rs.peer_ready, rs.release_group, &plan)))
      return fail(rc, "schedule construction failed");
    assign_dispatch(&plan, window);
    std::vector<int32_t> tasks;
    if (!sequential) tasks = task_list(plan, slabs, rs.push != 0);
    host.reserve(plan.launch.size() + plan.tiles.size() + plan.waits.size() + tasks.size() + 1);
    host.push_back(plan.wait_slots);  // header: the table sizes follow from the key
    host.insert(host.end(), plan.launch.begin(), plan.launch.end());
    host.insert(host.end(), plan.tiles.begin(), plan.tiles.end());
    host.insert(host.end(), plan.waits.begin(), plan.waits.end());
    host.insert(host.end(), tasks.begin(), tasks.end());
  }
  const std::vector<int32_t>& tab = host.empty() ? nt.host : host;
  wait_slots = tab[0];
  n_blocks = (size_t)g.NB * 4;
  n_tiles = (size_t)g.Q * 2;
  n_waits = (size_t)g.Q * wait_slots;
  n_tasks = tab.size() - 1 - n_blocks - n_tiles - n_waits;

  // Scratch layout: the fixed part, then tables, own partial, outgoing
  // partials and (push) staging, each 256-byte aligned.
  const size_t peer_sz = rs.peer_f32 ? 4 : 2;
  const size_t off_tab = kScratchFixed;
  const size_t off_own = up256(off_tab + tab.size() * 4);
  const size_t off_og = up256(off_own + (size_t)g.R * N * 4);
  const size_t off_st = up256(off_og + (size_t)M * N * peer_sz);
  const size_t need = rs.push ? up256(off_st + (size_t)M * N * peer_sz) : off_st;
  if (need > scratch_bytes)
    return fail(ENTWINE_ERR_OUT_OF_MEMORY, "the call needs %zu bytes of scratch; the no-alloc "
                "entry point's maximum is %zu", need, scratch_bytes);

  char* base = static_cast<char*>(scratch);
  if (!host.empty()) {
    // The upload is a copy from host memory followed by a synchronization,
    // neither of which a graph capture may hold.
    hipStreamCaptureStatus cap = hipStreamCaptureStatusNone;
    HIP_TRY(hipStreamIsCapturing(stream, &cap));
    if (cap != hipStreamCaptureStatusNone)
      return fail(ENTWINE_ERR_INVALID_ARGUMENT, "the schedule tables of this shape and "
                  "configuration are not in the no-alloc scratch: make the same call once "
                  "outside the graph capture");
    // The previous call's kernels may still read the old tables: the copy is
    // ordered after them on `stream`, and waited for, so that the host source
    // stays valid until the device has it.
    HIP_TRY(hipMemcpyAsync(base + off_tab, host.data(), host.size() * 4, hipMemcpyHostToDevice,
                           stream));
    HIP_TRY(hipStreamSynchronize(stream));
    nt.host.swap(host);
    nt.key = key;
    nt.valid = true;
  }
  const int32_t* d_tab = reinterpret_cast<const int32_t*>(base + off_tab) + 1;
  Buffers b;
  b.ctl = reinterpret_cast<uint32_t*>(base + kScratchCtl);
  b.error = reinterpret_cast<int32_t*>(base + kScratchError);
  b.flags = reinterpret_cast<uint32_t*>(base + kScratchFlags);
  b.blocks = d_tab;
  b.tiles = d_tab + n_blocks;
  b.waits = d_tab + n_blocks + n_tiles;
  b.task_list = n_tasks ? d_tab + n_blocks + n_tiles + n_waits : nullptr;
  b.wait_slots = wait_slots;
  b.own = reinterpret_cast<float*>(base + off_own);
  b.outgoing = base + off_og;
  b.staging = rs.push ? base + off_st : nullptr;
  GemmArgs ga;
  ReduceArgs ra;
  fill_args(rs, g, X, W, peers, out, M, N, K, P, rank, nullptr, b,
            (uint64_t)rs.timeout_ms * (uint64_t)khz, &ga, &ra);
  hipError_t e;
  if (sequential) {
    ga.publish = 0;
    ra.slabs = 1;
    ra.ntasks = 0;
    if ((e = launch_gemm_publish(ga, g.bm, g.bn, (int)g.NB, stream)) != hipSuccess)
      return fail(ENTWINE_ERR_HIP, "GEMM launch failed: %s", hipGetErrorString(e));
    if ((e = launch_tile_reduce(ra, rs.peer_f32, rs.out_f32, rs.threads, true,
                                flat_grid(g, N, rs.threads, cus), stream)) != hipSuccess)
      return fail(ENTWINE_ERR_HIP, "reduction launch failed: %s", hipGetErrorString(e));
    return ENTWINE_OK;
  }
  set_publication(rs, &ga);
  ra.slabs = slabs;
  ra.ntasks = (int32_t)(g.Q * slabs * (rs.push ? g.P : 1));
  FusedArgs fa{};
  fa.g = ga;
  fa.r = ra;
  fa.nb = (int32_t)g.NB;
  fa.workers = (int32_t)std::min<int64_t>(rs.budget, ra.ntasks);
  const int64_t grid = std::min<int64_t>((int64_t)fused_per_cu * cus, g.NB + (int64_t)fa.workers);
  if ((e = launch_gemm_rs_fused(fa, g.bm, g.bn, rs.variant, rs.peer_f32, rs.out_f32, (int)grid,
                                stream)) != hipSuccess)
    return fail(ENTWINE_ERR_HIP, "fused launch failed: %s", hipGetErrorString(e));
  return ENTWINE_OK;
}

}  // namespace entwine

extern "C" {

void entwine_config_init(entwine_config* cfg) {
  if (!cfg) return;
  std::memset(cfg, 0, sizeof *cfg);
  cfg->struct_size = (int32_t)sizeof *cfg;
  cfg->w_layout = ENTWINE_W_KN;
  cfg->peer_dtype = ENTWINE_BF16;
  cfg->out_dtype = ENTWINE_BF16;
  cfg->peer_ready = ENTWINE_PEERS_PRESEEDED;
  cfg->release_group = ENTWINE_RELEASE_TILE;
}

int entwine_gemm_rs(const void* X, const void* W, const void* const* peer_partials, void* out,
                    int64_t M, int64_t N, int64_t K_local, int P, int rank, int tile_order,
                    int comm_budget, void* stream) {
  return run(X, W, peer_partials, out, M, N, K_local, P, rank, tile_order, comm_budget, stream,
             nullptr);
}

int entwine_gemm_rs_ex(const void* X, const void* W, const void* const* peer_partials, void* out,
                       int64_t M, int64_t N, int64_t K_local, int P, int rank, int tile_order,
                       int comm_budget, void* stream, const entwine_config* cfg) {
  return run(X, W, peer_partials, out, M, N, K_local, P, rank, tile_order, comm_budget, stream,
             cfg);
}

int entwine_gemm_rs_rmsnorm(const void* X, const void* W, const void* const* peer_partials,
                            const void* residual, const void* gamma, float eps, void* h_out,
                            void* y_out, int64_t M, int64_t N, int64_t K_local, int P, int rank,
                            int tile_order, int comm_budget, void* stream,
                            const entwine_config* cfg) {
  Chain c;
  c.residual = residual;
  c.gamma = gamma;
  c.y = y_out;
  c.eps = eps;
  return run(X, W, peer_partials, h_out, M, N, K_local, P, rank, tile_order, comm_budget, stream,
             cfg, &c);
}

int entwine_plan_shape(int64_t M, int64_t N, int P, int block_m, int block_n, int tile_m,
                       int tile_n, int64_t* num_blocks, int64_t* blocks_per_partition,
                       int64_t* tiles_per_partition) {
  Geometry g;
  int rc = make_geometry(M, N, P, block_m, block_n, tile_m, tile_n, &g);
  if (rc) return fail(rc, "invalid geometry");
  if (num_blocks) *num_blocks = g.NB;
  if (blocks_per_partition) *blocks_per_partition = g.Bd;
  if (tiles_per_partition) *tiles_per_partition = g.Q;
  return ENTWINE_OK;
}

static int plan_for(int64_t M, int64_t N, int P, int rank, int order, int bm, int bn, int tm,
                    int tn, int peer_ready, int release_group, Plan* p) {
  Geometry g;
  int rc = make_geometry(M, N, P, bm, bn, tm, tn, &g);
  if (rc) return fail(rc, "invalid geometry");
  if (order == ENTWINE_ORDER_AUTO) order = ENTWINE_ORDER_INTERLEAVED;
  rc = build_plan(g, rank, order, peer_ready, release_group, p);
  if (rc) return fail(rc, "invalid schedule arguments");
  return ENTWINE_OK;
}

int entwine_plan_blocks(int64_t M, int64_t N, int P, int rank, int tile_order, int block_m,
                        int block_n, int tile_m, int tile_n, int32_t* blocks, int64_t capacity) {
  Plan p;
  int rc = plan_for(M, N, P, rank, tile_order, block_m, block_n, tile_m, tile_n,
                    ENTWINE_PEERS_PRESEEDED, ENTWINE_RELEASE_TILE, &p);
  if (rc) return rc;
  if (!blocks || capacity < (int64_t)p.blocks.size())
    return fail(ENTWINE_ERR_INVALID_ARGUMENT, "blocks needs %zu entries", p.blocks.size());
  std::copy(p.blocks.begin(), p.blocks.end(), blocks);
  return ENTWINE_OK;
}

int entwine_plan_dispatch(int64_t M, int64_t N, int P, int rank, int tile_order, int block_m,
                          int block_n, int tile_m, int tile_n, int64_t window, int32_t* dispatch,
                          int64_t capacity) {
  Plan p;
  int rc = plan_for(M, N, P, rank, tile_order, block_m, block_n, tile_m, tile_n,
                    ENTWINE_PEERS_PRESEEDED, ENTWINE_RELEASE_TILE, &p);
  if (rc) return rc;
  if (window < 0) return fail(ENTWINE_ERR_INVALID_ARGUMENT, "window must be >= 0");
  assign_dispatch(&p, window);
  if (!dispatch || capacity < (int64_t)p.dispatch.size())
    return fail(ENTWINE_ERR_INVALID_ARGUMENT, "dispatch needs %zu entries", p.dispatch.size());
  std::copy(p.dispatch.begin(), p.dispatch.end(), dispatch);
  return ENTWINE_OK;
}

int entwine_plan_tiles(int64_t M, int64_t N, int P, int block_m, int block_n, int tile_m,
                       int tile_n, int32_t* tiles, int64_t capacity) {
  Plan p;
  int rc = plan_for(M, N, P, 0, ENTWINE_ORDER_INTERLEAVED, block_m, block_n, tile_m, tile_n,
                    ENTWINE_PEERS_PRESEEDED, ENTWINE_RELEASE_TILE, &p);
  if (rc) return rc;
  if (!tiles || capacity < (int64_t)p.tiles.size())
    return fail(ENTWINE_ERR_INVALID_ARGUMENT, "tiles needs %zu entries", p.tiles.size());
  std::copy(p.tiles.begin(), p.tiles.end(), tiles);
  return ENTWINE_OK;
}

int entwine_plan_waits(int64_t M, int64_t N, int P, int rank, int tile_order, int block_m,
                       int block_n, int tile_m, int tile_n, int peer_ready, int release_group,
                       int32_t* waits, int64_t capacity) {
  Plan p;
  int rc = plan_for(M, N, P, rank, tile_order, block_m, block_n, tile_m, tile_n, peer_ready,
                    release_group, &p);
  if (rc) return rc;
  if (!waits || capacity < (int64_t)p.waits.size())
    return fail(ENTWINE_ERR_INVALID_ARGUMENT, "waits needs %zu entries", p.waits.size());
  std::copy(p.waits.begin(), p.waits.end(), waits);
  return ENTWINE_OK;
}

int entwine_plan_task_order(int64_t M, int64_t N, int P, int rank, int tile_order, int block_m,
                            int block_n, int tile_m, int tile_n, int peer_ready,
                            int release_group, int64_t window, int task_slabs,
                            int32_t* task_order, int64_t capacity) {
  Plan p;
  int rc = plan_for(M, N, P, rank, tile_order, block_m, block_n, tile_m, tile_n, peer_ready,
                    release_group, &p);
  if (rc) return rc;
  if (window < 0) return fail(ENTWINE_ERR_INVALID_ARGUMENT, "window must be >= 0");
  if (task_slabs < 1 || tile_m % task_slabs != 0)
    return fail(ENTWINE_ERR_INVALID_ARGUMENT, "task_slabs must divide tile_m");
  assign_dispatch(&p, window);
  const std::vector<int32_t> order = task_list(p, task_slabs, false);
  if (!task_order || capacity < (int64_t)order.size())
    return fail(ENTWINE_ERR_INVALID_ARGUMENT, "task_order needs %zu entries", order.size());
  // Global ids (rank * Q + t) * slabs + s -> the partition's own numbering.
  for (size_t k = 0; k < order.size(); ++k)
    task_order[k] = order[k] - (int32_t)(rank * p.g.Q * task_slabs);
  return ENTWINE_OK;
}

int entwine_plan_tasks(int64_t Q, int comm_budget, int consumer, int32_t* tasks, int64_t capacity,
                       int64_t* count) {
  if (Q < 0 || comm_budget < 1 || consumer < 0)
    return fail(ENTWINE_ERR_INVALID_ARGUMENT, "need Q >= 0, comm_budget >= 1, consumer >= 0");
  const int64_t x = std::min<int64_t>(comm_budget, Q);
  int64_t n = 0;
  if (consumer < x)
    for (int64_t t = consumer; t < Q; t += x) {
      if (tasks && n < capacity) tasks[n] = (int32_t)t;
      ++n;
    }
  if (count) *count = n;
  if (n > capacity) return fail(ENTWINE_ERR_INVALID_ARGUMENT, "tasks needs %" PRId64 " entries", n);
  return ENTWINE_OK;
}

int entwine_device_status(void* stream) {
  std::lock_guard<std::mutex> lock(g_mu);
  int dev = 0;
  HIP_TRY(hipGetDevice(&dev));
  HIP_TRY(hipStreamSynchronize(static_cast<hipStream_t>(stream)));
  int status = ENTWINE_OK;
  const uint32_t ctl_init[kCtlWords] = {1};  // epoch 1; counters and tickets 0
  auto it = g_ws.find(dev);
  if (it != g_ws.end()) {
    Workspace* w = it->second.get();
    HIP_TRY(hipStreamSynchronize(w->s_red));
    if (w->have_prev) {
      HIP_TRY(hipEventSynchronize(w->ev_gemm));
      HIP_TRY(hipEventSynchronize(w->ev_red));
    }
    int32_t err = 0;
    HIP_TRY(hipMemcpy(&err, w->error, sizeof err, hipMemcpyDeviceToHost));
    if (err != 0) {
      // An aborted reduction advanced the epoch while GEMM blocks may still
      // have been publishing; with every stream idle, start the flags afresh.
      HIP_TRY(hipMemset(w->error, 0, sizeof(int32_t)));
      if (w->flags) HIP_TRY(hipMemset(w->flags, 0, w->flag_count * sizeof(uint32_t)));
      if (w->claims) HIP_TRY(hipMemset(w->claims, 0, w->claims_bytes));
      HIP_TRY(hipMemcpy(w->ctl, ctl_init, sizeof ctl_init, hipMemcpyHostToDevice));
      status = err;
    }
  }
  // The no-alloc entry point's scratch (its calls ran on `stream`).
  if (char* sc = static_cast<char*>(noalloc_scratch(dev))) {
    int32_t err = 0;
    HIP_TRY(hipMemcpy(&err, sc + kScratchError, sizeof err, hipMemcpyDeviceToHost));
    if (err != 0) {
      HIP_TRY(hipMemset(sc + kScratchError, 0, sizeof(int32_t)));
      HIP_TRY(hipMemset(sc + kScratchFlags, 0, kScratchFlagWords * sizeof(uint32_t)));
      HIP_TRY(hipMemcpy(sc + kScratchCtl, ctl_init, sizeof ctl_init, hipMemcpyHostToDevice));
      status = err;
    }
  }
  if (status != ENTWINE_OK)
    return fail(status, "a reduction workgroup timed out waiting for a tile flag");
  return ENTWINE_OK;
}

const char* entwine_status_string(int status) {
  switch (status) {
    case ENTWINE_OK: return "ENTWINE_OK";
    case ENTWINE_ERR_INVALID_ARGUMENT: return "ENTWINE_ERR_INVALID_ARGUMENT";
    case ENTWINE_ERR_UNSUPPORTED: return "ENTWINE_ERR_UNSUPPORTED";
    case ENTWINE_ERR_OUT_OF_MEMORY: return "ENTWINE_ERR_OUT_OF_MEMORY";
    case ENTWINE_ERR_HIP: return "ENTWINE_ERR_HIP";
    case ENTWINE_ERR_TIMEOUT: return "ENTWINE_ERR_TIMEOUT";
    default: return "ENTWINE_ERR_UNKNOWN";
  }
}

const char* entwine_last_error_message(void) { return g_last_error.c_str(); }

int entwine_workspace(const void** own_partial, const void** outgoing, int64_t* bytes) {
  std::lock_guard<std::mutex> lock(g_mu);
  int dev = 0;
  HIP_TRY(hipGetDevice(&dev));
  auto it = g_ws.find(dev);
  if (it == g_ws.end()) return fail(ENTWINE_ERR_INVALID_ARGUMENT, "no workspace on this device yet");
  Workspace* w = it->second.get();
  HIP_TRY(hipStreamSynchronize(w->s_red));
  if (w->have_prev) {
    HIP_TRY(hipEventSynchronize(w->ev_gemm));
    HIP_TRY(hipEventSynchronize(w->ev_red));
  }
  if (own_partial) *own_partial = w->own;
  if (outgoing) *outgoing = w->outgoing;
  if (bytes)
    *bytes = (int64_t)(w->own_bytes + w->outgoing_bytes + w->staging_bytes + w->flag_count * 4);
  return ENTWINE_OK;
}

int entwine_flags(const void** flags, int64_t* words, uint32_t* epoch) {
  std::lock_guard<std::mutex> lock(g_mu);
  int dev = 0;
  HIP_TRY(hipGetDevice(&dev));
  auto it = g_ws.find(dev);
  if (it == g_ws.end()) return fail(ENTWINE_ERR_INVALID_ARGUMENT, "no workspace on this device yet");
  Workspace* w = it->second.get();
  HIP_TRY(hipStreamSynchronize(w->s_red));
  if (w->have_prev) {
    HIP_TRY(hipEventSynchronize(w->ev_gemm));
    HIP_TRY(hipEventSynchronize(w->ev_red));
  }
  if (flags) *flags = w->flags;
  if (words) *words = (int64_t)w->flag_count;
  if (epoch) HIP_TRY(hipMemcpy(epoch, w->ctl + kEpoch, sizeof *epoch, hipMemcpyDeviceToHost));
  return ENTWINE_OK;
}

int entwine_workspace_sizes(int64_t* own_bytes, int64_t* outgoing_bytes, int64_t* staging_bytes) {
  std::lock_guard<std::mutex> lock(g_mu);
  int dev = 0;
  HIP_TRY(hipGetDevice(&dev));
  auto it = g_ws.find(dev);
  if (it == g_ws.end()) return fail(ENTWINE_ERR_INVALID_ARGUMENT, "no workspace on this device yet");
  Workspace* w = it->second.get();
  HIP_TRY(hipStreamSynchronize(w->s_red));
  if (w->have_prev) {
    HIP_TRY(hipEventSynchronize(w->ev_gemm));
    HIP_TRY(hipEventSynchronize(w->ev_red));
  }
  if (own_bytes) *own_bytes = (int64_t)w->own_bytes;
  if (outgoing_bytes) *outgoing_bytes = (int64_t)w->outgoing_bytes;
  if (staging_bytes) *staging_bytes = (int64_t)w->staging_bytes;
  return ENTWINE_OK;
}

int entwine_staging(const void** staging, int64_t* bytes) {
  std::lock_guard<std::mutex> lock(g_mu);
  int dev = 0;
  HIP_TRY(hipGetDevice(&dev));
  auto it = g_ws.find(dev);
  if (it == g_ws.end()) return fail(ENTWINE_ERR_INVALID_ARGUMENT, "no workspace on this device yet");
  Workspace* w = it->second.get();
  HIP_TRY(hipStreamSynchronize(w->s_red));
  if (w->have_prev) {
    HIP_TRY(hipEventSynchronize(w->ev_gemm));
    HIP_TRY(hipEventSynchronize(w->ev_red));
  }
  if (staging) *staging = w->staging;
  if (bytes) *bytes = (int64_t)w->staging_bytes;
  return ENTWINE_OK;
}

int entwine_timing(int enable) {
  std::lock_guard<std::mutex> lock(g_mu);
  g_timing = enable != 0;
  return ENTWINE_OK;
}

int entwine_timing_read(double* gemm_ms, double* reduce_ms, int64_t* calls) {
  std::lock_guard<std::mutex> lock(g_mu);
  double gs = 0, rsum = 0;
  int64_t n = 0;
  for (auto& kv : g_ws) {
    Workspace* w = kv.second.get();
    for (auto& t : w->timing_live) {
      HIP_TRY(hipEventSynchronize(t.g1));
      HIP_TRY(hipEventSynchronize(t.r1));
      float a = 0, b = 0;
      HIP_TRY(hipEventElapsedTime(&a, t.g0, t.g1));
      HIP_TRY(hipEventElapsedTime(&b, t.r0, t.r1));
      gs += a;
      rsum += b;
      ++n;
      w->timing_free.push_back(t);
    }
    w->timing_live.clear();
  }
  if (gemm_ms) *gemm_ms = gs;
  if (reduce_ms) *reduce_ms = rsum;
  if (calls) *calls = n;
  return ENTWINE_OK;
}

int entwine_trace(int enable) {
  std::lock_guard<std::mutex> lock(g_mu);
  g_trace = enable != 0;
  return ENTWINE_OK;
}

int entwine_trace_read(double* gemm_us, double* reduce_start_us, double* reduce_end_us,
                       double* tail_us) {
  std::lock_guard<std::mutex> lock(g_mu);
  int dev = 0;
  HIP_TRY(hipGetDevice(&dev));
  auto it = g_ws.find(dev);
  if (it == g_ws.end() || !it->second->trace || !it->second->trace_valid)
    return fail(ENTWINE_ERR_INVALID_ARGUMENT, "no traced call on this device");
  Workspace* w = it->second.get();
  HIP_TRY(hipDeviceSynchronize());
  const int64_t nb = w->trace_nb, gr = w->trace_g;
  std::vector<uint64_t> t((size_t)2 * (nb + gr));
  HIP_TRY(hipMemcpy(t.data(), w->trace, t.size() * sizeof(uint64_t), hipMemcpyDeviceToHost));
  // First start and last end of each part; unwritten slots hold 0.
  auto span = [&](int64_t base, int64_t n, uint64_t* first, uint64_t* last) {
    *first = UINT64_MAX;
    *last = 0;
    for (int64_t i = 0; i < n; ++i) {
      if (t[base + i]) *first = std::min(*first, t[base + i]);
      *last = std::max(*last, t[base + n + i]);
    }
    return *first != UINT64_MAX && *last != 0;
  };
  uint64_t g0, g1, r0, r1;
  if (!span(0, nb, &g0, &g1))
    return fail(ENTWINE_ERR_INVALID_ARGUMENT, "the last traced call ran no GEMM");
  const bool red = span(2 * nb, gr, &r0, &r1);
  const double us_per_tick = 1000.0 / (double)w->wall_khz;
  auto at = [&](uint64_t v) { return ((double)v - (double)g0) * us_per_tick; };
  if (gemm_us) *gemm_us = at(g1);
  if (reduce_start_us) *reduce_start_us = red ? at(r0) : 0.0;
  if (reduce_end_us) *reduce_end_us = red ? at(r1) : 0.0;
  if (tail_us) *tail_us = red ? at(r1) - at(g1) : 0.0;
  return ENTWINE_OK;
}

int entwine_load_tuning(const char* path) {
  if (!path) return fail(ENTWINE_ERR_INVALID_ARGUMENT, "path is NULL");
  FILE* f = std::fopen(path, "r");
  if (!f) return fail(ENTWINE_ERR_INVALID_ARGUMENT, "cannot open %s", path);
  std::map<std::tuple<int64_t, int64_t, int64_t, int>, TuneEntry> table;
  char line[512];
  int lineno = 0;
  while (std::fgets(line, sizeof line, f)) {
    ++lineno;
    if (line[0] == '#' || line[0] == '\n') continue;
    long long M, N, K;
    int P, order, budget, bm, bn, threads, slabs = 1, schedule = ENTWINE_SCHEDULE_AUTO, variant = 0;
    const int n = std::sscanf(line, "%lld %lld %lld %d %d %d %d %d %d %d %d %d", &M, &N, &K, &P,
                              &order, &budget, &bm, &bn, &threads, &slabs, &schedule, &variant);
    if (n < 9 || schedule < ENTWINE_SCHEDULE_AUTO || schedule > ENTWINE_SCHEDULE_ASSISTED ||
        variant < 0 || variant > 4) {
      std::fclose(f);
      return fail(ENTWINE_ERR_INVALID_ARGUMENT,
                  "%s:%d: expected 9 to 12 integers (schedule 0 to 3; GEMM variant 0 to 4)",
                  path, lineno);
    }
    table[std::make_tuple((int64_t)M, (int64_t)N, (int64_t)K, P)] =
        TuneEntry{order, budget, bm, bn, threads, slabs, schedule, variant};
  }
  std::fclose(f);
  std::lock_guard<std::mutex> lock(g_mu);
  g_tuning = std::move(table);
  return ENTWINE_OK;
}

int entwine_release(void) {
  std::lock_guard<std::mutex> lock(g_mu);
  int dev = 0;
  HIP_TRY(hipGetDevice(&dev));
  auto it = g_ws.find(dev);
  if (it == g_ws.end()) return ENTWINE_OK;
  destroy_workspace(it->second.get());
  g_ws.erase(it);
  return ENTWINE_OK;
}

int entwine_device_cus(void) {
  int dev = 0, cus = 0;
  if (hipGetDevice(&dev) != hipSuccess) return 0;
  if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
    return 0;
  return cus;
}

}  // extern "C"
