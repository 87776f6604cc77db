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
// only then works on its reduction tasks (workgroup w < x takes tasks w,
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
// Check-out.  Every workgroup counts itself out; the last one clears the
// tickets and advances the epoch, so the next call (or graph replay) starts
// from zeroed tickets with a fresh epoch.
#include "gemm_block.h"
#include "reduce_task.h"

namespace entwine {
namespace {

// XCC_ID hardware register (id 20), bits [3:0]: the XCD this wave runs on.
__device__ __forceinline__ int xcd_id() {
  return __builtin_amdgcn_s_getreg((3 << 11) | (0 << 6) | 20) & 7;
}

__device__ __forceinline__ uint32_t take(uint32_t* w) {
  return __hip_atomic_fetch_add(w, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ uint32_t peek(const uint32_t* w) {
  return __hip_atomic_load(w, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Thread 0: the dispatch index of the next GEMM block for a workgroup on XCD
// x, or -1 once every list is exhausted.  List y holds blocks y, y + 8, ...;
// tickets only grow, so a list seen exhausted stays exhausted.
__device__ int next_block(uint32_t* ctl, int nb, int x) {
  for (int k = 0; k < 8; ++k) {
    const int y = (x + k) & 7;
    const uint32_t len = nb > y ? (uint32_t)((nb - y + 7) >> 3) : 0u;
    uint32_t* const c = ctl + kBlockTicket + y * kLine;
    // The own list is taken from directly; other lists are looked at first,
    // so that exhausted lists cost a load rather than an atomic.
    if (k > 0 && peek(c) >= len) continue;
    const uint32_t i = take(c);
    if (i < len) return y + 8 * (int)i;
  }
  return -1;
}

__device__ void fused_check_out(uint32_t* ctl, uint32_t epoch) {
  const uint32_t n = __hip_atomic_fetch_add(ctl + kFusedDone, 1u, __ATOMIC_RELAXED,
                                            __HIP_MEMORY_SCOPE_AGENT);
  if (n + 1 != gridDim.x) return;
  // Every other workgroup has taken its last ticket before checking out.
  auto clear = [&](int i) {
    __hip_atomic_store(ctl + i, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  };
  for (int y = 0; y < 8; ++y) clear(kBlockTicket + y * kLine);
  clear(kFusedDone);
  __hip_atomic_store(ctl + kEpoch, next_epoch(epoch), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

template <int BM, int BN, int BK, int NS, int WGM, int WGN, bool PP, bool PEER_F32, bool OUT_F32>
__global__ __launch_bounds__(64 * WGM * WGN, 1) void gemm_rs_fused_kernel(FusedArgs f) {
  constexpr int kThreads = 64 * WGM * WGN;
  extern __shared__ __attribute__((aligned(1024))) char smem[];
  // Broadcast slots alternate so that thread 0 never overwrites a value a
  // slower wave has yet to read.
  __shared__ int s_pick[2];
  __shared__ int s_abort[2];
  const int tid = threadIdx.x;
  uint32_t* const ctl = f.g.ctl;
  const uint32_t epoch = peek(ctl + kEpoch);
  int parity = 0;

  // GEMM blocks, until every list is exhausted.
  const int x = xcd_id();
  while (true) {
    if (tid == 0) s_pick[parity] = next_block(ctl, f.nb, x);
    __syncthreads();
    // Wave-uniform (scalar) values from here on: the block's descriptors and
    // output addresses stay in scalar registers, with no waterfall loops.
    const int b = __builtin_amdgcn_readfirstlane(s_pick[parity]);
    parity ^= 1;
    if (b < 0) break;
    gemm_block<BM, BN, BK, NS, WGM, WGN, PP>(f.g, reinterpret_cast<const int4*>(f.g.blocks)[b],
                                             smem);
  }

  // Reduction tasks: workgroup w < x (the budget) takes tasks w, w + x, ...
  // of the production-ordered list (Sec. 3.1), once it has left the GEMM
  // loop, i.e. once every block has been taken.  A static deal needs no
  // per-task atomic: one ticket counter shared by all workers serialized them.
  if ((int)blockIdx.x < f.workers) {
    for (int task = blockIdx.x; task < f.r.ntasks; task += f.workers, parity ^= 1) {
      const TaskRef k = task_ref(f.r, task);
      if (tid < 64) {
        const bool ok = wait_tile(f.r, epoch, k.d, k.t, tid);
        if (tid == 0) s_abort[parity] = ok ? 0 : 1;
      }
      // The flag wait is ordered before every wave's reads of the tile.
      __syncthreads();
      if (s_abort[parity]) break;  // uniform
      if (k.d == f.r.rank)
        reduce_slab<kThreads, PEER_F32, OUT_F32>(f.r, k.t, k.slab, tid);
      else
        push_slab<kThreads, PEER_F32>(f.r, k.d, k.t, k.slab, tid);
    }
  }
  if (tid == 0) fused_check_out(ctl, epoch);
}

template <int BM, int BN, int BK, int NS, int WGM, int WGN, bool PP, bool PF, bool OF>
struct Inst {
  using S = Shape<BM, BN, BK, NS, WGM, WGN>;
  static const void* fn() { return (const void*)gemm_rs_fused_kernel<BM, BN, BK, NS, WGM, WGN, PP, PF, OF>; }
  static hipError_t launch(const FusedArgs& a, int grid, hipStream_t s) {
    static bool attr_set = false;
    if (!attr_set) {
      hipError_t e = hipFuncSetAttribute(fn(), hipFuncAttributeMaxDynamicSharedMemorySize, S::kLds);
      if (e != hipSuccess) return e;
      attr_set = true;
    }
    gemm_rs_fused_kernel<BM, BN, BK, NS, WGM, WGN, PP, PF, OF><<<grid, S::kThreads, S::kLds, s>>>(a);
    return hipGetLastError();
  }
  static int per_cu() {
    int n = 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, fn(), S::kThreads, S::kLds) != hipSuccess)
      return 0;
    return n;
  }
};

// f.template run<Inst<...>>() for the instance of a shape, variant and the
// peer / output dtypes; f.none() if it is not built.
template <bool PF, bool OF, class F>
auto with_shape(int bm, int bn, int variant, F&& f) {
  if (bm == 128 && bn == 128 && variant == 0) return f.template run<Inst<128, 128, 64, 2, 2, 2, false, PF, OF>>();
  if (bm == 128 && bn == 256 && variant == 0) return f.template run<Inst<128, 256, 64, 2, 2, 4, false, PF, OF>>();
  if (bm == 128 && bn == 384 && variant == 0) return f.template run<Inst<128, 384, 64, 2, 2, 4, false, PF, OF>>();
  if (bm == 256 && bn == 128 && variant == 0) return f.template run<Inst<256, 128, 64, 2, 4, 2, false, PF, OF>>();
  if (bm == 256 && bn == 256 && variant == 0) return f.template run<Inst<256, 256, 64, 2, 2, 4, false, PF, OF>>();
  if (bm == 256 && bn == 256 && variant == 3) return f.template run<Inst<256, 256, 64, 2, 2, 2, false, PF, OF>>();
  if (bm == 256 && bn == 256 && variant == 4) return f.template run<Inst<256, 256, 64, 2, 2, 4, true, PF, OF>>();
  return f.none();
}

template <class F>
auto with_fused(int bm, int bn, int variant, int peer_f32, int out_f32, F&& f) {
  if (!peer_f32 && !out_f32) return with_shape<false, false>(bm, bn, variant, f);
  if (!peer_f32 && out_f32) return with_shape<false, true>(bm, bn, variant, f);
  if (peer_f32 && !out_f32) return with_shape<true, false>(bm, bn, variant, f);
  return with_shape<true, true>(bm, bn, variant, f);
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

}  // namespace

hipError_t launch_gemm_rs_fused(const FusedArgs& a, int bm, int bn, int variant, int peer_f32,
                                int out_f32, int grid, hipStream_t stream) {
  return with_fused(bm, bn, variant, peer_f32, out_f32, FusedLaunch{a, grid, stream});
}

int fused_blocks_per_cu(int bm, int bn, int variant, int peer_f32, int out_f32) {
  return with_fused(bm, bn, variant, peer_f32, out_f32, FusedOccupancy{});
}

}  // namespace entwine
