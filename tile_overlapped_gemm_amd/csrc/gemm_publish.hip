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
//    flags of every reduction tile it covers with release semantics.
//
// MI355X (gfx950) design.
//  * 512 threads = 8 waves of 64 (two per SIMD, so one wave's waits are
//    covered by the other's MFMAs) in a 2 x 4 (or 4 x 2) arrangement; a wave
//    owns a (BM/WGM) x (BN/WGN) sub-block computed with
//    v_mfma_f32_32x32x16_bf16 into fp32 accumulators.  A 4-wave (2 x 2)
//    instance remains as variant 3, and variant 4 of 256 x 256 runs the
//    ping-pong schedule of gemm_block.h (the dispatcher places waves i and
//    i + 4 of a workgroup on the same SIMD).  128 x 384 blocks (64 x 96 per
//    wave) serve partitions of at most 128 rows: a third of the blocks of
//    128 x 128, each with 1.5 times the MFMA work per byte loaded.  The MFMA's
//    first operand is the W fragment and the second the X fragment, so each
//    lane holds runs of 4 consecutive output columns.
//  * K advances in stages of 64 (128 bytes per row).  X and W are both
//    K-contiguous, so each stage is a BM x 128 B and a BN x 128 B slab.  Slabs
//    move from global memory straight into LDS with buffer_load_dwordx4 ...
//    lds: one wave instruction fills 1 KiB = 8 rows.  The buffer descriptors
//    bound the block's rows, so rows past the partition's (or N's) end read as
//    zeros without any clamping.  Two LDS stages: the loads of stage k+1 are
//    in flight while stage k is multiplied.
//  * LDS rows are XOR-swizzled in 16-byte chunks (chunk c of row r is stored
//    at c ^ swz(r)), so the 32 rows one fragment read touches spread over all
//    banks.  The swizzle is realised through each lane's global source
//    address, since the LDS destination of lane l is fixed at 16*l.
//  * Fragments are double-buffered in registers across the four 16-deep K
//    steps of a stage and across the stage boundary: the workgroup barrier
//    that hands over the next stage sits before the last K step's MFMAs, which
//    cover the barrier and the next stage's first fragment reads.
//  * Epilogue: accumulators leave through LDS in 32-row strips so that the
//    global stores write whole cache lines.
//  * Publication: tiles read on this device are written with device-coherent
//    (SC1) stores; the workgroup synchronizes after its stores, then thread 0
//    stores the call's epoch into the flag of every tile the block covers.
#include "gemm_block.h"

namespace entwine {
namespace {

template <int BM, int BN, int BK, int NS, int WGM, int WGN, bool PP>
__global__ __launch_bounds__(64 * WGM * WGN, 1) void gemm_publish_kernel(GemmArgs a) {
  extern __shared__ __attribute__((aligned(1024))) char smem[];
  gemm_block<BM, BN, BK, NS, WGM, WGN, PP>(
      a, reinterpret_cast<const int4*>(a.blocks)[blockIdx.x], (int)blockIdx.x, smem);
}

template <int BM, int BN, int BK, int NS, int WGM, int WGN, bool PP>
hipError_t launch_shape(const GemmArgs& a, int num_blocks, hipStream_t s) {
  using S = Shape<BM, BN, BK, NS, WGM, WGN>;
  static bool attr_set = false;
  if (!attr_set) {
    hipError_t e = hipFuncSetAttribute((const void*)gemm_publish_kernel<BM, BN, BK, NS, WGM, WGN, PP>,
                                       hipFuncAttributeMaxDynamicSharedMemorySize, S::kLds);
    if (e != hipSuccess) return e;
    attr_set = true;
  }
  gemm_publish_kernel<BM, BN, BK, NS, WGM, WGN, PP><<<num_blocks, S::kThreads, S::kLds, s>>>(a);
  return hipGetLastError();
}

template <int BM, int BN, int BK, int NS, int WGM, int WGN, bool PP>
int occupancy_of() {
  using S = Shape<BM, BN, BK, NS, WGM, WGN>;
  int n = 0;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(
          &n, (const void*)gemm_publish_kernel<BM, BN, BK, NS, WGM, WGN, PP>, S::kThreads,
          S::kLds) != hipSuccess)
    return 0;
  return n;
}

template <int BM, int BN, int BK, int NS, int WGM, int WGN, bool PP>
int regs_of() {
  hipFuncAttributes at{};
  if (hipFuncGetAttributes(&at, (const void*)gemm_publish_kernel<BM, BN, BK, NS, WGM, WGN, PP>) !=
      hipSuccess)
    return 0;
  return at.numRegs;
}

// The kernel instance for a block shape and variant, handed to `f` as a
// template functor call f.template run<BM, BN, BK, NS, WGM, WGN, PP>() (PP: the
// ping-pong main loop).
template <class F>
auto with_instance(int bm, int bn, int variant, F&& f) -> decltype(f.template run<128, 128, 64, 2, 2, 2, false>()) {
  if (bm == 128 && bn == 128) {
    if (variant == 3) return f.template run<128, 128, 64, 2, 2, 4, false>();
    return f.template run<128, 128, 64, 2, 2, 2, false>();
  }
  if (bm == 128 && bn == 256) {
    if (variant == 3) return f.template run<128, 256, 64, 2, 2, 2, false>();
    return f.template run<128, 256, 64, 2, 2, 4, false>();
  }
  if (bm == 128 && bn == 384) return f.template run<128, 384, 64, 2, 2, 4, false>();
  if (bm == 256 && bn == 128) {
    if (variant == 3) return f.template run<256, 128, 64, 2, 2, 2, false>();
    return f.template run<256, 128, 64, 2, 4, 2, false>();
  }
  if (bm == 256 && bn == 256) {
    if (variant == 1) return f.template run<256, 256, 32, 4, 2, 2, false>();
    if (variant == 2) return f.template run<256, 256, 32, 3, 2, 2, false>();
    if (variant == 3) return f.template run<256, 256, 64, 2, 2, 2, false>();
    if (variant == 4) return f.template run<256, 256, 64, 2, 2, 4, true>();
    return f.template run<256, 256, 64, 2, 2, 4, false>();
  }
  return f.template run<0, 0, 0, 0, 0, 0, false>();
}

struct Launch {
  const GemmArgs& a;
  int num_blocks;
  hipStream_t s;
  template <int BM, int BN, int BK, int NS, int WGM, int WGN, bool PP>
  hipError_t run() {
    if constexpr (BM == 0) return hipErrorInvalidValue;
    else return launch_shape<BM, BN, BK, NS, WGM, WGN, PP>(a, num_blocks, s);
  }
};
struct Occupancy {
  template <int BM, int BN, int BK, int NS, int WGM, int WGN, bool PP>
  int run() {
    if constexpr (BM == 0) return 0;
    else return occupancy_of<BM, BN, BK, NS, WGM, WGN, PP>();
  }
};
struct Registers {
  template <int BM, int BN, int BK, int NS, int WGM, int WGN, bool PP>
  int run() {
    if constexpr (BM == 0) return 0;
    else return regs_of<BM, BN, BK, NS, WGM, WGN, PP>();
  }
};

}  // namespace

int gemm_registers(int bm, int bn, int variant) { return with_instance(bm, bn, variant, Registers{}); }

int gemm_blocks_per_cu(int bm, int bn, int variant) {
  return with_instance(bm, bn, variant, Occupancy{});
}

struct Waves {
  template <int BM, int BN, int BK, int NS, int WGM, int WGN, bool PP>
  int run() { return WGM * WGN; }
};

int gemm_waves(int bm, int bn, int variant) { return with_instance(bm, bn, variant, Waves{}); }

hipError_t launch_gemm_publish(const GemmArgs& a, int bm, int bn, int num_blocks,
                               hipStream_t stream) {
  return with_instance(bm, bn, a.variant, Launch{a, num_blocks, stream});
}

}  // namespace entwine
