// gemm_rs_fused.hip -- the fused schedule: one kernel whose workgroups first
// compute GEMM blocks and then reduce tiles, with the same per-tile flags.
//
// Method: "Entwine: Coordinating Tiled Computation and Fine-Grained
// Communication across GPUs" (paperpeel.com/paper/2609.11562).
//  * Sec. 3.1: blocks are produced in the host-chosen order and reduction
//    tasks are taken in production order ("matching task order").
//  * Sec. 3.2: at most x workgroups (the communication budget) reduce.
//  * Sec. 4.2: producers release each tile with a flag after the block's
//    stores; a consumer observes every flag of a task before reading it (with
//    device-coherent loads in place of an acquire; see tile_reduce.hip).
//
// Why a single kernel on MI355X.  The paper runs producer and consumer as two
// kernels on two streams.  On this GPU a step that forks to a second stream
// and joins back costs 12-20 us more in graph replay than the same work on one
// stream, about as much as the whole reduction of a 4096 x 4096 output.  Here
// one kernel on the caller's stream does both, so nothing forks or joins.
//
// Forward progress.  GEMM blocks come from device-wide tickets, not from
// blockIdx: a workgroup takes blocks until every block has been taken and
// only then waits for its reduction tasks (workgroup w < x takes tasks w,
// w + x, ...).  A task waits only for flags of blocks that running workgroups
// have already taken, and a workgroup computing a block never waits, so every
// wait ends whatever the dispatch order.  (Withheld flags end through the
// watchdog.)
//
// XCD locality.  The host's dispatch order deals each window of concurrent
// blocks to the 8 XCDs as compact rectangles (block b to XCD b % 8).  Each
// XCD keeps its own ticket, so a workgroup reads its XCD from the hardware
// register and takes that XCD's next block; when its list is exhausted it
// takes blocks from the other lists.
//
// Reduction phase.  A task's time is set by memory latency rather than by
// its bytes, so tasks are small (row slabs of a tile, one chunk per thread)
// and a worker takes four at a time: the inputs that existed before the call
// (preseeded peers, the residual) are loaded before the wait, wave 0 polls
// the four tasks' flags at once, and the four own-partial loads are in flight
// together.  Operands go through buffer descriptors based at each slab, which
// keeps four tasks within the GEMM's register budget.
//
// Check-out.  Every workgroup counts itself out; the last one clears the
// tickets and advances the epoch, so the next call (or graph replay) starts
// from zeroed tickets with a fresh epoch.
//
// The assisted schedule runs this kernel beside helper workgroups on another
// stream (tile_reduce.hip, assist_reduce_kernel).  Then a worker reduces only
// the tasks it claims (a claim word per task, moved to the call's sequence
// number), every claimer counts its finished tasks, and the last workgroup
// waits for the count to reach the task count before it finishes the call.
#include "gemm_block.h"
#include "reduce_task.h"

namespace entwine {
namespace {

__device__ void fused_check_out(const ReduceArgs& r, uint32_t epoch) {
  uint32_t* const ctl = r.ctl;
  const uint32_t n = __hip_atomic_fetch_add(ctl + kFusedDone, 1u, __ATOMIC_RELAXED,
                                            __HIP_MEMORY_SCOPE_AGENT);
  if (n + 1 != gridDim.x) return;
  // Every other workgroup has taken its last ticket before checking out.
  auto clear = [&](int i) {
    __hip_atomic_store(ctl + i, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  };
  if (r.assist_seq) {
    // The assisted schedule: every task of the call was claimed (this
    // kernel's workers claimed all that were left), and a helper claims a
    // task only once its flags are set, so the count reaches the task count
    // within one task's time.  Then the call is over for the helpers too.
    const uint64_t start = wall_clock64();
    while (__hip_atomic_load(ctl + kTasksDone, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) !=
           (uint32_t)r.ntasks) {
      if (__hip_atomic_load(r.error, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) != 0) break;
      if (wall_clock64() - start > r.timeout_ticks) {
        __hip_atomic_store(r.error, (int32_t)5 /* ENTWINE_ERR_TIMEOUT */, __ATOMIC_RELAXED,
                           __HIP_MEMORY_SCOPE_AGENT);
        break;
      }
      __builtin_amdgcn_s_sleep(2);
    }
    clear(kTasksDone);
    __hip_atomic_store(reinterpret_cast<uint64_t*>(ctl + kAssistCall), assist_pack(r.assist_seq, 0),
                       __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
  for (int y = 0; y < 8; ++y) clear(kBlockTicket + y * kLine);
  clear(kFusedDone);
  __hip_atomic_store(ctl + kEpoch, next_epoch(epoch), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// A reduction task begun but not completed: its slab and its U chunks per
// thread (with the inputs loaded so far).
template <int U, bool PEER_F32, bool OUT_F32>
struct Pending {
  static constexpr int kChunks = U;
  Slab s;
  RelChunks<U, PEER_F32, OUT_F32> c;
};

template <int BM, int BN, int BK, int NS, int WGM, int WGN, bool PP, bool WKN, bool PEER_F32,
          bool OUT_F32>
__global__ __launch_bounds__(64 * WGM * WGN, 1) void gemm_rs_fused_kernel(FusedArgs f) {
  constexpr int kThreads = 64 * WGM * WGN;
  // Tasks taken together after the GEMM phase, and the chunks (8 elements)
  // per thread of each whose loads are issued at once.  A task of 32 x 128
  // elements (a 128 x 128 tile in four slabs) is one chunk per thread of a
  // 512-thread workgroup.  Four tasks with bf16 data need about 240
  // registers per lane.  The 4-wave 128 x 128 instance takes two, so that two
  // of its workgroups still fit on a CU, and so does an fp32 output; fp32
  // peers take twice the registers per chunk, and one task.
  constexpr int kB = PEER_F32 ? 1 : (kThreads >= 512 && !OUT_F32 ? 4 : 2), kU = 1;
  extern __shared__ __attribute__((aligned(1024))) char smem[];
  // Thread 0's broadcast word.  Slots alternate: the next write to a slot
  // comes after a barrier that every wave passes only once it has read it.
  __shared__ int s_word[2];
  const int tid = threadIdx.x;
  uint32_t* const ctl = f.g.ctl;
  const ReduceArgs& r = f.r;
  const uint32_t epoch = peek(ctl + kEpoch);
  // The assisted schedule: the call is live for its helpers from here on.
  if (r.assist_seq && blockIdx.x == 0 && tid == 0)
    __hip_atomic_store(reinterpret_cast<uint64_t*>(ctl + kAssistCall),
                       assist_pack(r.assist_seq, epoch), __ATOMIC_RELAXED,
                       __HIP_MEMORY_SCOPE_AGENT);
  int parity = 0;
  // Thread 0's v, for every thread, as a wave-uniform (scalar) value.
  auto share = [&](int v) {
    if (tid == 0) s_word[parity] = v;
    __syncthreads();
    const int out = __builtin_amdgcn_readfirstlane(s_word[parity]);
    parity ^= 1;
    return out;
  };

  // Start of a reduction task: the slab's chunk placement and, when
  // r.prefetch is set, the loads of the inputs that were complete before the
  // call (the peers, the residual) for this thread's first kU chunks.  A
  // send task loads only after its wait.  `lt` is the thread index.
  auto begin = [&](int task, auto& p, int lt) {
    const TaskRef k = task_ref(r, task);
    if (k.d != r.rank) return;  // a send task loads after its wait
    p.s = slab_of(r, k.t, k.slab);
    place_rel<std::remove_reference_t<decltype(p)>::kChunks, kThreads>(p.s, lt, p.c);
    if (r.prefetch) load_inputs_rel(r, slab_io<PEER_F32, OUT_F32>(r, p.s.e0), p.c);
  };

  // One batch: tasks t0, t0 + x, ..., t0 + (kB - 1) x of the
  // production-ordered list (x = the workers).  The peers' loads are issued
  // first (with preseeded peers), wave 0 then waits for all the tasks' flags
  // at once (16 lanes per task), and all their own-partial loads are in
  // flight before any is summed, so each memory round trip serves kB tasks.
  // False when the watchdog or the sticky error ended the wait.
  static_assert(kB * 16 <= 64, "16 wait lanes per task");
  const int x = f.workers;
  auto batch = [&](int t0) -> bool {
    // The thread index, laundered so that the batch recomputes its offsets
    // rather than keeping the GEMM's in registers (fewer registers in all).
    int lt = tid;
    asm volatile("" : "+v"(lt));
    // The batch's tasks this workgroup reduces: all of them, or in the
    // assisted schedule those it claims (helpers have the others).
    int mine = (1 << kB) - 1;
    if (r.assist_seq) {
      int m = 0;
      if (tid == 0)
        for (int b = 0; b < kB; ++b)
          if (t0 + b * x < r.ntasks && claim_task(r.claims, t0 + b * x, r.assist_seq)) m |= 1 << b;
      mine = share(m);
      if (mine == 0) return true;
    }
    Pending<kU, PEER_F32, OUT_F32> p[kB];
#pragma unroll
    for (int b = 0; b < kB; ++b)
      if (t0 + b * x < r.ntasks && ((mine >> b) & 1)) begin(t0 + b * x, p[b], lt);
    int ok = 1;
    if (lt < 64) {
      const int tw = t0 + (lt >> 4) * x;
      const uint32_t* fl = nullptr;
      if (tw < r.ntasks && ((mine >> (lt >> 4)) & 1)) {
        const TaskRef k = task_ref(r, tw);
        fl = wait_flag(r, k.d, k.t, lt & 15);
      }
      ok = wait_flags(r, epoch, fl, lt);
    }
    // The flag waits are ordered before every wave's reads of the tiles.
    if (!share(ok)) return false;
    Raw8<true> own[kB][kU];
#pragma unroll
    for (int b = 0; b < kB; ++b) {
      const int t = t0 + b * x;
      if (t < r.ntasks && ((mine >> b) & 1) && task_ref(r, t).d == r.rank) {
        const SlabIO io = slab_io<PEER_F32, OUT_F32>(r, p[b].s.e0);
        if (!r.prefetch) load_inputs_rel(r, io, p[b].c);
        load_own_rel(io, p[b].c, own[b]);
      }
    }
#pragma unroll
    for (int b = 0; b < kB; ++b) {
      const int t = t0 + b * x;
      if (t >= r.ntasks) break;
      if (!((mine >> b) & 1)) continue;
      const TaskRef k = task_ref(r, t);
      if (k.d == r.rank) {
        sum_store_rel(r, slab_io<PEER_F32, OUT_F32>(r, p[b].s.e0), p[b].c, own[b]);
        reduce_slab<kThreads, kU, PEER_F32, OUT_F32>(r, p[b].s, lt, kU * kThreads);
      } else {
        push_slab<kThreads, PEER_F32>(r, k.d, k.t, k.slab, lt);
      }
    }
    if (r.assist_seq && tid == 0)
      __hip_atomic_fetch_add(ctl + kTasksDone, (uint32_t)__builtin_popcount(mine), __ATOMIC_RELAXED,
                             __HIP_MEMORY_SCOPE_AGENT);
    return true;
  };

  // GEMM blocks until every list is exhausted (tickets of this XCD first).
  // The thread index is laundered: the block's lane offsets are recomputed
  // per block rather than held in registers into the reduction phase.
  const int xcd = xcd_id();
  while (true) {
    int pick = 0;
    if (tid < 64) pick = next_block(ctl, f.nb, xcd, tid);
    const int b = share(pick);
    if (b < 0) break;
    int ltid = tid;
    asm volatile("" : "+v"(ltid));
    gemm_block<BM, BN, BK, NS, WGM, WGN, PP, WKN>(f.g, reinterpret_cast<const int4*>(f.g.blocks)[b],
                                                  b, smem, ltid);
  }

  // Every block has been taken: workgroup w < x (the budget) owns tasks w,
  // w + x, ... of the production-ordered list (Sec. 3.1), kB at a time.  A
  // task waits only for blocks that running workgroups have taken.  A static
  // deal needs no per-task atomic: one ticket counter shared by all workers
  // serialized them.  (Reducing released tasks between GEMM blocks instead
  // was measured: each batch holds its CU at memory latency, and the GEMM
  // ended later by more than the whole reduction takes on its own.)
  int task = (int)blockIdx.x < x ? (int)blockIdx.x : r.ntasks;
  const bool worker = task < r.ntasks;  // uniform
  const int trace_g = r.trace_g ? r.trace_g : (int)gridDim.x;
  if (r.trace && worker && tid == 0) trace_at(r.trace, r.trace_slot0 + blockIdx.x);
  while (task < r.ntasks) {
    if (!batch(task)) break;  // the watchdog or the sticky error ended the wait
    task += kB * x;
  }
  if (r.trace && worker) {  // uniform: every wave's stores issued
    __syncthreads();
    if (tid == 0) trace_at(r.trace, (int64_t)trace_g + r.trace_slot0 + blockIdx.x);
  }
  if (tid == 0) fused_check_out(r, epoch);
}

template <int BM, int BN, int BK, int NS, int WGM, int WGN, bool PP, bool WKN, bool PF, bool OF>
struct Inst {
  using S = Shape<BM, BN, BK, NS, WGM, WGN, WKN>;
  static const void* fn() {
    return (const void*)gemm_rs_fused_kernel<BM, BN, BK, NS, WGM, WGN, PP, WKN, PF, OF>;
  }
  static hipError_t launch(const FusedArgs& a, int grid, hipStream_t s) {
    static bool attr_set = false;
    if (!attr_set) {
      hipError_t e = hipFuncSetAttribute(fn(), hipFuncAttributeMaxDynamicSharedMemorySize, S::kLds);
      if (e != hipSuccess) return e;
      attr_set = true;
    }
    gemm_rs_fused_kernel<BM, BN, BK, NS, WGM, WGN, PP, WKN, PF, OF>
        <<<grid, S::kThreads, S::kLds, s>>>(a);
    return hipGetLastError();
  }
  static int per_cu() {
    int n = 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, fn(), S::kThreads, S::kLds) != hipSuccess)
      return 0;
    return n;
  }
};

// f.template run<Inst<...>>() for the instance of a shape, variant, W layout
// and the peer / output dtypes; f.none() if it is not built.
template <bool PF, bool OF, class F>
auto with_shape(int bm, int bn, int variant, bool wkn, F&& f) {
  if (wkn) {
    if constexpr (PF == OF) {
      if (variant != 0) return f.none();
      if (bm == 128 && bn == 128) return f.template run<Inst<128, 128, 64, 2, 2, 2, false, true, PF, OF>>();
      if (bm == 128 && bn == 256) return f.template run<Inst<128, 256, 64, 2, 2, 4, false, true, PF, OF>>();
      if (bm == 256 && bn == 128) return f.template run<Inst<256, 128, 64, 2, 4, 2, false, true, PF, OF>>();
      if (bm == 256 && bn == 256) return f.template run<Inst<256, 256, 64, 2, 2, 4, false, true, PF, OF>>();
      if (bm == 128 && bn == 384) return f.template run<Inst<128, 384, 64, 2, 2, 4, false, true, PF, OF>>();
    }
    return f.none();
  }
  if (bm == 128 && bn == 128 && variant == 0) return f.template run<Inst<128, 128, 64, 2, 2, 2, false, false, PF, OF>>();
  if (bm == 128 && bn == 256 && variant == 0) return f.template run<Inst<128, 256, 64, 2, 2, 4, false, false, PF, OF>>();
  if (bm == 128 && bn == 384 && variant == 0) return f.template run<Inst<128, 384, 64, 2, 2, 4, false, false, PF, OF>>();
  if (bm == 256 && bn == 128 && variant == 0) return f.template run<Inst<256, 128, 64, 2, 4, 2, false, false, PF, OF>>();
  if (bm == 256 && bn == 256 && variant == 0) return f.template run<Inst<256, 256, 64, 2, 2, 4, false, false, PF, OF>>();
  if (bm == 256 && bn == 256 && variant == 3) return f.template run<Inst<256, 256, 64, 2, 2, 2, false, false, PF, OF>>();
  if (bm == 256 && bn == 256 && variant == 4) return f.template run<Inst<256, 256, 64, 2, 2, 4, true, false, PF, OF>>();
  return f.none();
}

template <class F>
auto with_fused(int bm, int bn, int variant, int peer_f32, int out_f32, bool wkn, F&& f) {
  if (!peer_f32 && !out_f32) return with_shape<false, false>(bm, bn, variant, wkn, f);
  if (!peer_f32 && out_f32) return with_shape<false, true>(bm, bn, variant, wkn, f);
  if (peer_f32 && !out_f32) return with_shape<true, false>(bm, bn, variant, wkn, f);
  return with_shape<true, true>(bm, bn, variant, wkn, f);
}

struct FusedLaunch {
  const FusedArgs& a;
  int grid;
  hipStream_t s;
  template <class I>
  hipError_t run() { return I::launch(a, grid, s); }
  hipError_t none() { return hipErrorInvalidValue; }
};
struct FusedOccupancy {
  template <class I>
  int run() { return I::per_cu(); }
  int none() { return 0; }
};
struct FusedRegisters {
  template <class I>
  int run() {
    hipFuncAttributes at{};
    return hipFuncGetAttributes(&at, I::fn()) == hipSuccess ? at.numRegs : 0;
  }
  int none() { return 0; }
};

}  // namespace

hipError_t launch_gemm_rs_fused(const FusedArgs& a, int bm, int bn, int variant, int peer_f32,
                                int out_f32, int grid, hipStream_t stream) {
  return with_fused(bm, bn, variant, peer_f32, out_f32, a.g.w_kn != 0,
                    FusedLaunch{a, grid, stream});
}

int fused_blocks_per_cu(int bm, int bn, int variant, int peer_f32, int out_f32, bool wkn) {
  return with_fused(bm, bn, variant, peer_f32, out_f32, wkn, FusedOccupancy{});
}

int fused_registers(int bm, int bn, int variant, int peer_f32, int out_f32, bool wkn) {
  return with_fused(bm, bn, variant, peer_f32, out_f32, wkn, FusedRegisters{});
}

}  // namespace entwine
