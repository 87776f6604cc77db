// gemm_publish.hip -- the producer: a bf16 MFMA GEMM whose workgroups follow a
// host-chosen production order and publish one ready flag per output tile.
//
// Method: "Entwine: Coordinating Tiled Computation and Fine-Grained
// Communication across GPUs" (paperpeel.com/paper/2609.11562).
//  * Sec. 2.1: rank r computes its full-size partial product C_r = X_r W_r;
//    rows of its own partition stay local, all other rows are contributions
//    to peers.
//  * Sec. 3.1 / Equation (1): the workgroup at logical position p computes the
//    block that the order table names for p (a custom block swizzle).
//  * Sec. 4.2: after all of a block's output stores, the block publishes the
//    flags of every reduction tile it covers (stores, a CTA barrier, then
//    thread 0's release store of the flags).
//
// MI355X (gfx950) design.
//  * 512 threads = 8 waves of 64 (two per SIMD, so one wave's waits are
//    covered by the other's MFMAs) in a 2 x 4 (or 4 x 2) arrangement; a wave
//    owns a (BM/WGM) x (BN/WGN) sub-block computed with
//    v_mfma_f32_16x16x32_bf16 into fp32 accumulators (the 32 x 32 x 16 form
//    builds with -DENTWINE_MFMA_EDGE=32: the same nominal rate, but the chip
//    clocks lower under it).  A 4-wave (2 x 2)
//    instance remains as variant 3, and variant 4 of 256 x 256 runs the
//    ping-pong schedule of gemm_block.h (the dispatcher places waves i and
//    i + 4 of a workgroup on the same SIMD).  128 x 384 blocks (64 x 96 per
//    wave) serve partitions of at most 128 rows: a third of the blocks of
//    128 x 128, each with 1.5 times the MFMA work per byte loaded.  The MFMA's
//    first operand is the W fragment and the second the X fragment, so each
//    lane holds runs of 4 consecutive output columns.
//  * K advances in stages of 64 (128 bytes per row).  X is K-contiguous, so
//    each stage's X slab is BM x 128 B; W's is BN x 128 B when W is held
//    [N][K], and 64 rows of BN columns when it is held [K][N] (the default),
//    transposed on its way into the MFMA by transposing LDS reads.  Slabs
//    move from global memory straight into LDS with buffer_load_dwordx4 ...
//    lds: one wave instruction fills 1 KiB = 8 rows.  The buffer descriptors
//    bound the block's rows, so rows past the partition's (or N's) end read as
//    zeros without any clamping.  Two LDS stages: the loads of stage k+1 are
//    in flight while stage k is multiplied.
//  * LDS rows are XOR-swizzled in 16-byte chunks (chunk c of row r is stored
//    at c ^ swz(r), a function chosen per MFMA form by the bank-conflict
//    counter), so the rows one fragment read touches spread over all banks.
//    The swizzle is realised through each lane's global source address,
//    since the LDS destination of lane l is fixed at 16*l.
//  * Each 32-deep K step runs in four quarters (X half times W half of the
//    wave's tiles); a quarter's fragments are read from LDS while the
//    previous quarter's MFMAs run.  The workgroup barrier that hands over the
//    next stage sits before the last quarter of the stage, whose MFMAs cover
//    the barrier and the next stage's first fragment reads.
//  * Epilogue: accumulators leave through LDS in 32-row strips so that the
//    global stores write whole cache lines.
//  * Publication: tiles read on this device are written with device-coherent
//    (SC1) stores; every wave waits until its stores are acknowledged
//    (s_waitcnt vmcnt(0)), the workgroup synchronizes, then thread 0 stores
//    the call's epoch into the flag of every tile the block covers.  This
//    orders the data before the flag without an agent-scope release fence,
//    which would write back the XCD's whole L2.
//  * Two launch forms.  gemm_publish_kernel: one workgroup per block, block
//    b of the dispatch order on workgroup b (sequential schedule, single
//    stages).  gemm_ticket_kernel: persistent workgroups taking blocks from
//    per-XCD tickets (beside the two-stream reduction, whose workgroups slow
//    the CUs they share).
#include "gemm_block.h"

namespace entwine {
namespace {

template <int BM, int BN, int BK, int NS, int WGM, int WGN, bool PP, bool WKN>
__global__ __launch_bounds__(64 * WGM * WGN, 1) void gemm_publish_kernel(GemmArgs a) {
  extern __shared__ __attribute__((aligned(1024))) char smem[];
  gemm_block<BM, BN, BK, NS, WGM, WGN, PP, WKN>(
      a, reinterpret_cast<const int4*>(a.blocks)[blockIdx.x], (int)blockIdx.x, smem);
}

// Persistent form: each workgroup takes blocks from its XCD's ticket (then
// from the others) until every block is taken.  Used beside the two-stream
// schedule's reduction workgroups: a CU shared with one runs its blocks more
// slowly and simply takes fewer of them, where a fixed block-to-workgroup
// deal would make the whole GEMM wait for the slowest such CU.
template <int BM, int BN, int BK, int NS, int WGM, int WGN, bool PP, bool WKN>
__global__ __launch_bounds__(64 * WGM * WGN, 1) void gemm_ticket_kernel(GemmArgs a) {
  extern __shared__ __attribute__((aligned(1024))) char smem[];
  // Thread 0's pick; slots alternate, and the next write to a slot comes
  // after a barrier that every wave passes once it has read it.
  __shared__ int s_pick[2];
  const int tid = threadIdx.x;
  const int xcd = xcd_id();
  // The call's epoch: it cannot change before this workgroup has checked out.
  const uint32_t epoch = tid == 0 ? peek(a.ctl + kEpoch) : 0u;
  int parity = 0;
  while (true) {
    int pick = 0;
    if (tid < 64) pick = next_block(a.ctl, a.nb, xcd, tid);
    if (tid == 0) s_pick[parity] = pick;
    __syncthreads();
    const int b = __builtin_amdgcn_readfirstlane(s_pick[parity]);
    parity ^= 1;
    if (b < 0) break;
    // Laundered thread index: the block's lane offsets are recomputed per
    // block instead of living in registers across blocks, which keeps this
    // kernel at the stand-alone GEMM's register count, and so beside a
    // reduction workgroup on a CU.
    int ltid = tid;
    asm volatile("" : "+v"(ltid));
    gemm_block<BM, BN, BK, NS, WGM, WGN, PP, WKN>(a, reinterpret_cast<const int4*>(a.blocks)[b], b,
                                             smem, ltid);
  }
  // Check-out.  The last GEMM workgroup (every other one has taken its last
  // ticket) resets the tickets for the next call.  Then the workgroup, whose
  // flag stores are all issued, checks out of the call together with the
  // reduction's workgroups: the last of either advances the epoch.
  if (tid == 0) {
    const uint32_t n = __hip_atomic_fetch_add(a.ctl + kGemmDone, 1u, __ATOMIC_RELAXED,
                                              __HIP_MEMORY_SCOPE_AGENT);
    if (n + 1 == gridDim.x) {
      for (int y = 0; y < 8; ++y)
        __hip_atomic_store(a.ctl + kBlockTicket + y * kLine, 0u, __ATOMIC_RELAXED,
                           __HIP_MEMORY_SCOPE_AGENT);
      __hip_atomic_store(a.ctl + kGemmDone, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
    if (a.checkout_total > 0) check_out(a.ctl, epoch, (uint32_t)a.checkout_total);
  }
}

template <int BM, int BN, int BK, int NS, int WGM, int WGN, bool PP, bool WKN>
hipError_t launch_shape(const GemmArgs& a, int num_blocks, hipStream_t s) {
  using S = Shape<BM, BN, BK, NS, WGM, WGN, WKN>;
  static bool attr_set = false;
  if (!attr_set) {
    hipError_t e = hipFuncSetAttribute((const void*)gemm_publish_kernel<BM, BN, BK, NS, WGM, WGN, PP, WKN>,
                                       hipFuncAttributeMaxDynamicSharedMemorySize, S::kLds);
    if (e != hipSuccess) return e;
    attr_set = true;
  }
  gemm_publish_kernel<BM, BN, BK, NS, WGM, WGN, PP, WKN><<<num_blocks, S::kThreads, S::kLds, s>>>(a);
  return hipGetLastError();
}

// lds_min: LDS bytes each workgroup reserves at least (the pipeline uses the
// first S::kLds of them); a reservation above half of a CU's LDS keeps every
// workgroup alone on its CU.
template <int BM, int BN, int BK, int NS, int WGM, int WGN, bool PP, bool WKN>
hipError_t launch_tickets(const GemmArgs& a, int grid, int lds_min, hipStream_t s) {
  using S = Shape<BM, BN, BK, NS, WGM, WGN, WKN>;
  const int lds = lds_min > S::kLds ? lds_min : S::kLds;
  static int attr_bytes = 0;
  if (lds > attr_bytes) {
    hipError_t e = hipFuncSetAttribute((const void*)gemm_ticket_kernel<BM, BN, BK, NS, WGM, WGN, PP, WKN>,
                                       hipFuncAttributeMaxDynamicSharedMemorySize, lds);
    if (e != hipSuccess) return e;
    attr_bytes = lds;
  }
  gemm_ticket_kernel<BM, BN, BK, NS, WGM, WGN, PP, WKN><<<grid, S::kThreads, lds, s>>>(a);
  return hipGetLastError();
}

template <int BM, int BN, int BK, int NS, int WGM, int WGN, bool PP, bool WKN>
int occupancy_of() {
  using S = Shape<BM, BN, BK, NS, WGM, WGN, WKN>;
  int n = 0;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(
          &n, (const void*)gemm_publish_kernel<BM, BN, BK, NS, WGM, WGN, PP, WKN>, S::kThreads,
          S::kLds) != hipSuccess)
    return 0;
  return n;
}

template <int BM, int BN, int BK, int NS, int WGM, int WGN, bool PP, bool WKN>
int regs_of() {
  hipFuncAttributes at{};
  if (hipFuncGetAttributes(&at, (const void*)gemm_publish_kernel<BM, BN, BK, NS, WGM, WGN, PP, WKN>) !=
      hipSuccess)
    return 0;
  return at.numRegs;
}

template <int BM, int BN, int BK, int NS, int WGM, int WGN, bool PP, bool WKN>
int ticket_regs_of() {
  hipFuncAttributes at{};
  if (hipFuncGetAttributes(&at, (const void*)gemm_ticket_kernel<BM, BN, BK, NS, WGM, WGN, PP, WKN>) !=
      hipSuccess)
    return 0;
  return at.numRegs;
}

// The kernel instance for a block shape, variant and W layout, handed to `f`
// as a template functor call f.template run<BM, BN, BK, NS, WGM, WGN, PP, WKN>()
// (PP: the ping-pong main loop; WKN: W held [K][N]).  W [K][N] is built for
// the base pipeline of every block shape.
template <class F>
auto with_instance(int bm, int bn, int variant, bool wkn,
                   F&& f) -> decltype(f.template run<128, 128, 64, 2, 2, 2, false, false>()) {
  if (wkn) {
    if (variant != 0) return f.template run<0, 0, 0, 0, 0, 0, false, false>();
    if (bm == 128 && bn == 128) return f.template run<128, 128, 64, 2, 2, 2, false, true>();
    if (bm == 128 && bn == 256) return f.template run<128, 256, 64, 2, 2, 4, false, true>();
    if (bm == 256 && bn == 128) return f.template run<256, 128, 64, 2, 4, 2, false, true>();
    if (bm == 256 && bn == 256) return f.template run<256, 256, 64, 2, 2, 4, false, true>();
    if (bm == 128 && bn == 384) return f.template run<128, 384, 64, 2, 2, 4, false, true>();
    return f.template run<0, 0, 0, 0, 0, 0, false, false>();
  }
  if (bm == 128 && bn == 128) {
    if (variant == 3) return f.template run<128, 128, 64, 2, 2, 4, false, false>();
    return f.template run<128, 128, 64, 2, 2, 2, false, false>();
  }
  if (bm == 128 && bn == 256) {
    if (variant == 3) return f.template run<128, 256, 64, 2, 2, 2, false, false>();
    return f.template run<128, 256, 64, 2, 2, 4, false, false>();
  }
  if (bm == 128 && bn == 384) return f.template run<128, 384, 64, 2, 2, 4, false, false>();
  if (bm == 256 && bn == 128) {
    if (variant == 3) return f.template run<256, 128, 64, 2, 2, 2, false, false>();
    return f.template run<256, 128, 64, 2, 4, 2, false, false>();
  }
  if (bm == 256 && bn == 256) {
    if (variant == 1) return f.template run<256, 256, 32, 4, 2, 2, false, false>();
    if (variant == 2) return f.template run<256, 256, 32, 3, 2, 2, false, false>();
    if (variant == 3) return f.template run<256, 256, 64, 2, 2, 2, false, false>();
    if (variant == 4) return f.template run<256, 256, 64, 2, 2, 4, true, false>();
    return f.template run<256, 256, 64, 2, 2, 4, false, false>();
  }
  return f.template run<0, 0, 0, 0, 0, 0, false, false>();
}

struct Launch {
  const GemmArgs& a;
  int num_blocks;
  hipStream_t s;
  template <int BM, int BN, int BK, int NS, int WGM, int WGN, bool PP, bool WKN>
  hipError_t run() {
    if constexpr (BM == 0) return hipErrorInvalidValue;
    else return launch_shape<BM, BN, BK, NS, WGM, WGN, PP, WKN>(a, num_blocks, s);
  }
};
struct LaunchTickets {
  const GemmArgs& a;
  int grid;
  int lds_min;
  hipStream_t s;
  template <int BM, int BN, int BK, int NS, int WGM, int WGN, bool PP, bool WKN>
  hipError_t run() {
    if constexpr (BM == 0) return hipErrorInvalidValue;
    else return launch_tickets<BM, BN, BK, NS, WGM, WGN, PP, WKN>(a, grid, lds_min, s);
  }
};
struct LdsBytes {
  template <int BM, int BN, int BK, int NS, int WGM, int WGN, bool PP, bool WKN>
  int run() {
    if constexpr (BM == 0) return 0;
    else return Shape<BM, BN, BK, NS, WGM, WGN, WKN>::kLds;
  }
};
struct Occupancy {
  template <int BM, int BN, int BK, int NS, int WGM, int WGN, bool PP, bool WKN>
  int run() {
    if constexpr (BM == 0) return 0;
    else return occupancy_of<BM, BN, BK, NS, WGM, WGN, PP, WKN>();
  }
};
struct Registers {
  bool tickets;
  template <int BM, int BN, int BK, int NS, int WGM, int WGN, bool PP, bool WKN>
  int run() {
    if constexpr (BM == 0) return 0;
    else if (tickets) return ticket_regs_of<BM, BN, BK, NS, WGM, WGN, PP, WKN>();
    else return regs_of<BM, BN, BK, NS, WGM, WGN, PP, WKN>();
  }
};

}  // namespace

int gemm_registers(int bm, int bn, int variant, bool wkn, bool tickets) {
  return with_instance(bm, bn, variant, wkn, Registers{tickets});
}

int gemm_blocks_per_cu(int bm, int bn, int variant, bool wkn) {
  return with_instance(bm, bn, variant, wkn, Occupancy{});
}

struct Waves {
  template <int BM, int BN, int BK, int NS, int WGM, int WGN, bool PP, bool WKN>
  int run() { return WGM * WGN; }
};

int gemm_waves(int bm, int bn, int variant, bool wkn) {
  return with_instance(bm, bn, variant, wkn, Waves{});
}

bool gemm_built(int bm, int bn, int variant, bool wkn) {
  return with_instance(bm, bn, variant, wkn, LdsBytes{}) > 0;
}

hipError_t launch_gemm_publish(const GemmArgs& a, int bm, int bn, int num_blocks,
                               hipStream_t stream) {
  return with_instance(bm, bn, a.variant, a.w_kn != 0, Launch{a, num_blocks, stream});
}

int gemm_lds_bytes(int bm, int bn, int variant, bool wkn) {
  return with_instance(bm, bn, variant, wkn, LdsBytes{});
}

hipError_t launch_gemm_tickets(const GemmArgs& a, int bm, int bn, int grid, hipStream_t stream,
                               int lds_min) {
  return with_instance(bm, bn, a.variant, a.w_kn != 0, LaunchTickets{a, grid, lds_min, stream});
}

}  // namespace entwine
