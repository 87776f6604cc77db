// gemm_block.h -- device code of one GEMM block with per-tile release,
// shared by the stand-alone GEMM kernel and the fused GEMM + reduction
// kernel.
//
// Method: "Entwine: Coordinating Tiled Computation and Fine-Grained
// Communication across GPUs" (paperpeel.com/paper/2609.11562), Sec. 2.1,
// Sec. 3.1 and Sec. 4.2; the MI355X design is described in gemm_publish.hip.
#pragma once

#include <type_traits>

#include "kernels.h"

namespace entwine {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) void* lds_ptr_t;

constexpr int kRsrcWord3 = 0x00020000;  // raw buffer, 32-bit data format

// MFMA tile edge: 16 (v_mfma_f32_16x16x32_bf16, the default) or 32
// (v_mfma_f32_32x32x16_bf16, built with -DENTWINE_MFMA_EDGE=32 for
// comparison).  Both have the same peak rate per cycle; the 16 x 16 form runs
// the GEMM about 5 % faster here, at a higher clock under the same power.
#ifndef ENTWINE_MFMA_EDGE
#define ENTWINE_MFMA_EDGE 16
#endif

// Block BM x BN, K stage BK (32 or 64), NS LDS stages, WGM x WGN waves; W
// held [N][K] (K contiguous) or, with WKN, [K][N] (N contiguous).
template <int BM, int BN, int BK, int NS, int WGM = 2, int WGN = 2, bool WKN = false>
struct Shape {
  static constexpr int kWaves = WGM * WGN;
  static constexpr int kThreads = 64 * kWaves;
  static constexpr int kWavesN = WGN;
  static constexpr bool kWKN = WKN;
  static constexpr int kRow = BK * 2;                 // bytes per X slab row (and W's, [N][K])
  static constexpr int kRowB = WKN ? BN * 2 : kRow;   // bytes per W slab row in LDS
  static constexpr int kRowsPerLoad = 1024 / kRow;    // rows per 1 KiB wave load
  static constexpr int kLanesPerRow = kRow / 16;
  // MFMA tiles: 16 x 16 and 32 deep, or 32 x 32 and 16 deep.
  static constexpr int kMF = ENTWINE_MFMA_EDGE;
  static constexpr int kMK = kMF == 16 ? 32 : 16;     // MFMA depth
  static constexpr int kKS = BK / kMK;                // MFMA K steps per stage
  static constexpr int kWM = BM / WGM, kWN = BN / WGN;  // wave sub-block
  static constexpr int kMT = kWM / kMF, kNT = kWN / kMF;
  static_assert(kMT * kMF == kWM && kNT * kMF == kWN, "wave sub-block of whole MFMA tiles");
  static constexpr int kA = BM * kRow, kB = BN * BK * 2;  // stage slabs
  static constexpr int kStage = kA + kB;
  static constexpr int kLds = NS * kStage;
  static constexpr int kLoadsA = BM / (kWaves * kRowsPerLoad);  // per wave per stage
  static constexpr int kLoadsB = kB / (kWaves * 1024);
  static_assert(kLoadsA * kWaves * kRowsPerLoad == BM && kLoadsB * kWaves * 1024 == kB,
                "slab rows must split evenly over the waves");
  static_assert(!WKN || (kRowB % 256 == 0 && BK == 64),
                "[K][N] W slabs: rows of whole 16-chunk swizzle groups");
  // W [K][N] rows that a 1 KiB wave load does not cover whole (384 wide):
  // each load group of the lane has a source offset of its own.
  static constexpr bool kPerLoadB = WKN && (1024 % kRowB != 0);
  static_assert(kWaves % 2 == 0, "load groups keep the row parity of the swizzle");
  static constexpr int kLoads = kLoadsA + kLoadsB;
  static_assert(kMF != 16 || (kMT % 2 == 0 && kNT % 2 == 0), "quarter steps: tiles split in halves");
  // W [K][N] with 16 x 16 tiles and a wave sub-block 64 wide: the LDS offsets
  // of the lane's W fragments differ from fragment 0's by an XOR (see Lanes).
  static constexpr bool kKnXor = WKN && kMF == 16 && kWN == 64;
  static_assert(kLoads * (NS - 2 > 0 ? NS - 2 : 0) < 64, "vmcnt range");
};

// XOR swizzle of the 16-byte chunks of an X (or W [N][K]) slab row r: the
// physical chunk of logical chunk c is c ^ swz(r).  A fragment read names the
// same logical chunk in 16 (16 x 16 tiles) or 32 (32 x 32) consecutive rows;
// each form has its own swizzle, chosen by the LDS bank-conflict counter
// (SQ_LDS_BANK_CONFLICT): 0 conflict cycles per read with the forms below,
// about 4 with the other form's swizzle.
template <int BK, int MF>
__device__ __forceinline__ int swz(int r) {
  if constexpr (MF == 16)
    return BK == 64 ? (r & 7) : ((r >> 1) & 3);
  else if constexpr (BK == 64)
    return (r & 7) ^ ((r >> 3) & 1);
  else
    return ((r >> 1) ^ (r >> 3)) & 3;
}

// XOR swizzle of the 16-byte chunks of W [K][N] slab row k: (k & 3) << 2
// spreads the four rows one 16-lane group of a transposing read names over
// the banks, and bit 3 of k moves the next group's rows (8 further) to other
// banks again, so that 32 lanes of a read are served without conflict.
__device__ __forceinline__ int kn_swz(int k) { return ((k & 3) << 2) ^ (((k >> 3) & 1) << 1); }

// Wait until at most VM of this wave's vector-memory operations are pending
// and all of its LDS reads returned, then synchronize the workgroup.  No
// global-memory fence: the stage hand-over only needs LDS.
template <int VM>
__device__ __forceinline__ void stage_barrier() {
  asm volatile("s_waitcnt vmcnt(%0) lgkmcnt(0)\n\ts_barrier" ::"n"(VM) : "memory");
}

// Device-coherent global stores (buffer cache policy SC1) through a
// wave-uniform buffer descriptor; `off` is the lane's byte offset.
typedef unsigned u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned u32x2 __attribute__((ext_vector_type(2)));
constexpr int kCoherent = 16;  // SC1

__device__ __forceinline__ __amdgpu_buffer_rsrc_t rsrc_of(const void* base, int bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, bytes, kRsrcWord3);
}

__device__ __forceinline__ bf16x8 lds_frag(const char* p) {
  return *reinterpret_cast<const bf16x8*>(p);
}

// Per-lane operand offsets of one block.  Loads: the lane's byte offset in
// the X and W slabs of a K stage and the step between its load groups, and
// the bytes W advances per K stage.  Fragments: LDS offsets of the lane's X
// fragment per K step and of its W fragment (per K step with W [N][K]; per
// 32-column fragment with W [K][N], whose K steps are fixed offsets).
template <class S>
struct Lanes {
  int voff_a, step_a;
  int voff_b, step_b, stage_b;
  int voff_bj[S::kPerLoadB ? S::kLoadsB : 1];  // per load group (kPerLoadB)
  int a_off[S::kKS];
  int b_off[S::kKnXor ? 1 : (S::kWKN ? S::kNT : S::kKS)];
};

// LDS offset of the lane's W [K][N] fragment j (first read, K step 0).  With
// kKnXor, fragment j covers 16-byte chunks 2j and 2j + 1 more than fragment
// 0 within the wave's 64 columns, and the row swizzle touches other chunk
// bits, so its offset is fragment 0's XOR 32*j.  Fragment 0's offset is
// laundered where it is used, so that the compiler computes the XORs there
// rather than holding one register per fragment through the main loop.
template <class S>
__device__ __forceinline__ int kn_b_off(const Lanes<S>& ln, int j) {
  if constexpr (S::kKnXor) {
    int o = ln.b_off[0];
    asm volatile("" : "+v"(o));
    return o ^ (32 * j);
  } else {
    return ln.b_off[j];
  }
}

// One stage's global->LDS copies for this wave: X's slab (PART 1), W's
// (PART 2) or both (3), load group wave + kWaves*j, 1 KiB each; voffset is the
// lane's swizzled source, soffset the group and the stage.
// One 16-byte-per-lane buffer load into LDS (lane l's bytes land at
// lds + 16 l).  With W [K][N] the loads are issued through inline assembly:
// the compiler then does not track them, which it otherwise does by waiting
// for every outstanding vector memory operation before each transposing LDS
// read (it cannot tell that the read and the loads touch different buffers),
// stalling every K stage on its own prefetch.  The loads have no result
// registers; the pipeline's stage barriers wait for them explicitly
// (s_waitcnt vmcnt), as for the compiler-issued form.
template <bool ASM>
__device__ __forceinline__ void load_lds16(__amdgpu_buffer_rsrc_t r, char* lds, int voff,
                                           int soff) {
#if defined(__HIP_DEVICE_COMPILE__)
  if constexpr (ASM) {
    const uint32_t m0 = (uint32_t)(uintptr_t)(lds_ptr_t)lds;
    asm volatile("s_mov_b32 m0, %0\n\tbuffer_load_dwordx4 %1, %2, %3 offen lds"
                 :
                 : "s"(m0), "v"(voff), "s"(r), "s"(soff)
                 : "memory", "m0");
  } else {
    __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_ptr_t)lds, 16, voff, soff, 0, 0);
  }
#endif
}

template <class S>
struct Copy {
  template <int PART = 3>
  __device__ static __forceinline__ void stage(__amdgpu_buffer_rsrc_t ra,
                                               __amdgpu_buffer_rsrc_t rb, char* lds,
                                               const Lanes<S>& ln, int st, int wave) {
  if constexpr ((PART & 1) != 0) {
#pragma unroll
    for (int j = 0; j < S::kLoadsA; ++j)
      load_lds16<S::kWKN>(ra, lds + (wave + S::kWaves * j) * 1024, ln.voff_a,
                          j * ln.step_a + st * S::kRow);
  }
  if constexpr ((PART & 2) != 0) {
#pragma unroll
    for (int j = 0; j < S::kLoadsB; ++j) {
      if constexpr (S::kPerLoadB)
        load_lds16<true>(rb, lds + S::kA + (wave + S::kWaves * j) * 1024, ln.voff_bj[j],
                         st * ln.stage_b);
      else
        load_lds16<S::kWKN>(rb, lds + S::kA + (wave + S::kWaves * j) * 1024, ln.voff_b,
                            j * ln.step_b + st * ln.stage_b);
    }
  }
  }
};

template <class S>
struct Frags {
  bf16x8 b[S::kNT];  // W fragments (MFMA rows = output columns)
  bf16x8 a[S::kMT];  // X fragments (MFMA cols = output rows)
};

typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) i16x4* lds_i16x4_ptr;

// K step ks of a stage: the lane's W fragments (8 consecutive k of one output
// column) and X fragments (8 consecutive k of one output row).  With W [K][N]
// each W fragment is two transposing LDS reads: lanes 4e..4e+3 of each
// 16-lane group name row k0 + e (16 columns), and lane i receives column i of
// the four rows, i.e. k0..k0+3 of its own column.
template <class S>
__device__ __forceinline__ void read_frags(Frags<S>& f, const char* stage, const Lanes<S>& ln,
                                           int ks) {
  if constexpr (S::kWKN) {
#pragma unroll
    for (int j = 0; j < S::kNT; ++j) {
      const char* p = stage + S::kA + kn_b_off<S>(ln, j) + ks * S::kMK * S::kRowB;
      const i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4_ptr)p);
      const i16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4_ptr)(p + 4 * S::kRowB));
      f.b[j] = __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
    }
  } else {
#pragma unroll
    for (int j = 0; j < S::kNT; ++j)
      f.b[j] = lds_frag(stage + S::kA + ln.b_off[ks] + j * S::kMF * S::kRow);
  }
#pragma unroll
  for (int i = 0; i < S::kMT; ++i)
    f.a[i] = lds_frag(stage + ln.a_off[ks] + i * S::kMF * S::kRow);
}

// One MFMA tile's accumulators: 4 per lane (16 x 16) or 16 (32 x 32).
template <class S>
struct Acc {
  typedef typename std::conditional<S::kMF == 16, f32x4, f32x16>::type Tile;
  Tile c[S::kMT][S::kNT];
};

template <class S>
__device__ __forceinline__ void mfma_step(Acc<S>& acc, const Frags<S>& f) {
#pragma unroll
  for (int i = 0; i < S::kMT; ++i)
#pragma unroll
    for (int j = 0; j < S::kNT; ++j) {
      if constexpr (S::kMF == 16)
        acc.c[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(f.b[j], f.a[i], acc.c[i][j], 0, 0, 0);
      else
        acc.c[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(f.b[j], f.a[i], acc.c[i][j], 0, 0, 0);
    }
}

// Workgroup barrier that the compiler may not schedule any instruction across
// (MFMAs included), after this wave's LDS reads and all but VM of its vector
// memory operations have completed.
template <int VM>
__device__ __forceinline__ void phase_barrier() {
  __builtin_amdgcn_sched_barrier(0);
  stage_barrier<VM>();
  __builtin_amdgcn_sched_barrier(0);
}

// The same barrier without waiting for vector memory operations.
__device__ __forceinline__ void phase_barrier_lds() {
  __builtin_amdgcn_sched_barrier(0);
  asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
  __builtin_amdgcn_sched_barrier(0);
}

// phase_barrier<PER * n> for a wave-uniform n in [0, 2].
template <int PER>
__device__ __forceinline__ void phase_barrier_n(int n) {
  if (n >= 2)
    phase_barrier<2 * PER>();
  else if (n == 1)
    phase_barrier<PER>();
  else
    phase_barrier<0>();
}

// Ping-pong main loop for 8 waves.  The waves form two groups of four (waves
// 0-3 and 4-7, one of each on every SIMD) that run the same sequence of
// phases half a stage apart: in a memory phase a wave issues its share of a
// future stage's global->LDS copies and reads all of the current stage's
// fragments into registers; in the compute phase that follows it runs the
// stage's MFMAs back to back on those registers, at raised issue priority.
// While one group computes, the other loads, so every SIMD alternates between
// the MFMAs of its two waves, and one workgroup barrier ends every phase.
//
// Stage i lives in LDS buffer i % NS and is read in phases 2i (group 0) and
// 2i + 1 (group 1).  Its copies are issued in phase 2(i - L), L = NS - 1, by
// both groups (group 1 at the start of a compute phase), into the buffer that
// stage i - NS left at barrier 2(i - L); every wave has waited for its own
// copies of stage j before barrier 2j.
template <class S>
__device__ __forceinline__ void pingpong_loop(Acc<S>& acc, __amdgpu_buffer_rsrc_t ra,
                                              __amdgpu_buffer_rsrc_t rb, char* smem,
                                              const Lanes<S>& ln, int nk, int wave) {
  constexpr int NS = S::kLds / S::kStage, L = NS - 1;
  static_assert(S::kWaves == 8 && NS >= 2 && NS <= 4, "ping-pong: 8 waves, 2 to 4 stages");
  constexpr int PER = S::kLoads;
  static_assert(PER * (L - 1) < 64, "vmcnt range");
  auto issue = [&](int st) {
    Copy<S>::template stage<3>(ra, rb, smem + (st % NS) * S::kStage, ln, st, wave);
  };
  const bool g1 = wave >= 4;  // wave-uniform
  // Prologue: stages 0 .. L-1, then stage 0 landed for every wave.
#pragma unroll
  for (int st = 0; st < L; ++st)
    if (st < nk) issue(st);
  phase_barrier_n<PER>(min(L - 1, nk - 1));
  if (g1) {
    // Group 1's phase 0: the copies of stage L, and no compute.
    if (L < nk) issue(L);
    phase_barrier_lds();
  }
  Frags<S> fr[S::kKS];
  for (int i = 0; i < nk; ++i) {
    const char* cur = smem + (i % NS) * S::kStage;
    // Memory phase of stage i.
    if (!g1 && i + L < nk) issue(i + L);
#pragma unroll
    for (int ks = 0; ks < S::kKS; ++ks) read_frags<S>(fr[ks], cur, ln, ks);
    if (g1)
      phase_barrier_n<PER>(min(L - 1, nk - 2 - i));  // barrier 2(i+1): stage i+1 landed
    else
      phase_barrier_lds();
    // Compute phase of stage i.
    __builtin_amdgcn_s_setprio(1);
    if (g1 && i + 1 + L < nk) issue(i + 1 + L);
#pragma unroll
    for (int ks = 0; ks < S::kKS; ++ks) mfma_step<S>(acc, fr[ks]);
    __builtin_amdgcn_s_setprio(0);
    if (!g1)
      phase_barrier_n<PER>(min(L - 1, nk - 2 - i));  // barrier 2(i+1): stage i+1 landed
    else if (i + 1 < nk)
      phase_barrier_lds();
  }
}

// Half of a K step's X fragments (MFMA row tiles h*kMT/2 ..) or of its W
// fragments (column tiles h*kNT/2 ..), for the quarter-step pipeline.
template <class S>
struct HalfA {
  bf16x8 a[S::kMT / 2];
};
template <class S>
struct HalfB {
  bf16x8 b[S::kNT / 2];
};

template <class S>
__device__ __forceinline__ void read_half_a(HalfA<S>& f, const char* stage, const Lanes<S>& ln,
                                            int ks, int h) {
#pragma unroll
  for (int i = 0; i < S::kMT / 2; ++i)
    f.a[i] = lds_frag(stage + ln.a_off[ks] + (h * S::kMT / 2 + i) * S::kMF * S::kRow);
}

template <class S>
__device__ __forceinline__ void read_half_b(HalfB<S>& f, const char* stage, const Lanes<S>& ln,
                                            int ks, int h) {
#pragma unroll
  for (int j = 0; j < S::kNT / 2; ++j) {
    const int jj = h * S::kNT / 2 + j;
    if constexpr (S::kWKN) {
      const char* p = stage + S::kA + kn_b_off<S>(ln, jj) + ks * S::kMK * S::kRowB;
      const i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4_ptr)p);
      const i16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4_ptr)(p + 4 * S::kRowB));
      f.b[j] = __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
    } else {
      f.b[j] = lds_frag(stage + S::kA + ln.b_off[ks] + jj * S::kMF * S::kRow);
    }
  }
}

// The MFMAs of one quarter of a K step: X half HA times W half HB.
template <class S, int HA, int HB>
__device__ __forceinline__ void mfma_quarter(Acc<S>& acc, const HalfA<S>& fa, const HalfB<S>& fb) {
  static_assert(S::kMF == 16, "quarter steps are built for 16 x 16 tiles");
#pragma unroll
  for (int i = 0; i < S::kMT / 2; ++i)
#pragma unroll
    for (int j = 0; j < S::kNT / 2; ++j) {
      auto& c = acc.c[HA * S::kMT / 2 + i][HB * S::kNT / 2 + j];
      c = __builtin_amdgcn_mfma_f32_16x16x32_bf16(fb.b[j], fa.a[i], c, 0, 0, 0);
    }
}

// The base main loop.  Prologue: stages 0 .. NS-2 in flight, wait for stage
// 0, then stage NS-1.  Stage kt + NS is loaded in two halves: X's slab right
// after the barrier that frees its buffer, W's after the next stage's first
// MFMAs, so that the eight waves' loads do not all reach the address units
// and LDS at once (1.5-2 % on the 4-round shapes).
//
// 16 x 16 tiles: each K step runs in four quarters (X half 0 or 1 times W
// half 0 or 1), and the fragments of a quarter are read while the previous
// quarter's MFMAs run: W half 1 during quarter 0, X half 1 during quarter 1,
// the next step's X and W halves 0 after quarter 2 (after the stage barrier
// at a stage's last step), so four half sets (as many registers as one K
// step's fragments) are live and each read batch stays within the LDS
// counter's reach.  Every output tile still accumulates its K steps in order.
// 32 x 32 tiles: whole K steps of fragments, double-buffered.
template <class S>
__device__ __forceinline__ void base_loop(Acc<S>& acc, __amdgpu_buffer_rsrc_t ra,
                                          __amdgpu_buffer_rsrc_t rb, char* smem,
                                          const Lanes<S>& ln, int nk, int wave) {
  constexpr int NS = S::kLds / S::kStage;
#pragma unroll
  for (int s = 0; s < NS - 1; ++s)
    if (s < nk) Copy<S>::template stage<3>(ra, rb, smem + s * S::kStage, ln, s, wave);
  if (nk >= NS - 1)
    stage_barrier<S::kLoads * (NS - 2)>();
  else
    stage_barrier<0>();
  if (NS - 1 < nk) Copy<S>::template stage<3>(ra, rb, smem + (NS - 1) * S::kStage, ln, NS - 1, wave);

  // The barrier that ends stage kt: stage kt+1 landed (stages up to kt+NS-1
  // were issued) and every wave done reading stage kt's buffer, which then
  // takes X's slab of stage kt+NS.
  int pending_w = -1;  // stage whose W slab is still to be issued
  auto hand_over = [&](int kt) {
    if (kt + NS - 1 < nk)
      stage_barrier<S::kLoads * (NS - 2)>();
    else
      stage_barrier<0>();
    if (kt + NS < nk) {
      Copy<S>::template stage<1>(ra, rb, smem + (kt % NS) * S::kStage, ln, kt + NS, wave);
      pending_w = kt + NS;
    }
  };
  // W's slab of stage pending_w, whose buffer (not the current one) the
  // previous barrier freed.
  auto issue_w = [&]() {
    if (pending_w >= 0) {
      Copy<S>::template stage<2>(ra, rb, smem + (pending_w % NS) * S::kStage, ln, pending_w, wave);
      pending_w = -1;
    }
  };

  if constexpr (S::kMF == 16) {
    HalfA<S> alo, ahi;
    HalfB<S> blo, bhi;
    read_half_b<S>(blo, smem, ln, 0, 0);
    read_half_a<S>(alo, smem, ln, 0, 0);
    for (int kt = 0; kt < nk; ++kt) {
      const char* cur = smem + (kt % NS) * S::kStage;
#pragma unroll
      for (int ks = 0; ks < S::kKS; ++ks) {
        // The scheduling barriers keep each read batch between the quarters
        // named above: hoisted further, the reads would need registers of
        // their own and a wait for all of them before the first MFMA.
        read_half_b<S>(bhi, cur, ln, ks, 1);
        __builtin_amdgcn_sched_barrier(0);
        mfma_quarter<S, 0, 0>(acc, alo, blo);
        __builtin_amdgcn_sched_barrier(0);
        if (ks == 0) issue_w();
        read_half_a<S>(ahi, cur, ln, ks, 1);
        __builtin_amdgcn_sched_barrier(0);
        mfma_quarter<S, 0, 1>(acc, alo, bhi);
        mfma_quarter<S, 1, 0>(acc, ahi, blo);
        __builtin_amdgcn_sched_barrier(0);
        if (ks + 1 < S::kKS) {
          read_half_b<S>(blo, cur, ln, ks + 1, 0);
          read_half_a<S>(alo, cur, ln, ks + 1, 0);
        } else if (kt + 1 < nk) {
          hand_over(kt);
          const char* nxt = smem + ((kt + 1) % NS) * S::kStage;
          read_half_b<S>(blo, nxt, ln, 0, 0);
          read_half_a<S>(alo, nxt, ln, 0, 0);
        }
        __builtin_amdgcn_sched_barrier(0);
        mfma_quarter<S, 1, 1>(acc, ahi, bhi);
        __builtin_amdgcn_sched_barrier(0);
      }
    }
  } else {
    static_assert(S::kKS % 2 == 0, "fragment double buffer needs an even K-step count");
    Frags<S> f0, f1;
    read_frags<S>(f0, smem, ln, 0);
    for (int kt = 0; kt < nk; ++kt) {
      const char* cur = smem + (kt % NS) * S::kStage;
#pragma unroll
      for (int ks = 0; ks + 1 < S::kKS; ks += 2) {
        read_frags<S>(f1, cur, ln, ks + 1);
        mfma_step<S>(acc, f0);
        if (ks == 0) issue_w();
        if (ks + 2 < S::kKS) {
          read_frags<S>(f0, cur, ln, ks + 2);
          mfma_step<S>(acc, f1);
        }
      }
      if (kt + 1 < nk) {
        hand_over(kt);
        read_frags<S>(f0, smem + ((kt + 1) % NS) * S::kStage, ln, 0);
      }
      mfma_step<S>(acc, f1);
    }
  }
}

// Block tickets (the fused kernel and the persistent GEMM): block b of the
// XCD-aware dispatch order belongs to XCD b % 8, whose ticket hands out its
// blocks in order.
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

// Wave 0 (lane = 0..63): the dispatch index of the next GEMM block for a
// workgroup on XCD x, or -1 once every list is exhausted (uniform).  List y
// holds blocks y, y + 8, ...; tickets only grow, so a list seen exhausted
// stays exhausted.  The own list is taken from directly; once it is empty,
// lanes 0-7 look at all eight tickets at once, so finding that every list is
// empty costs one load latency, not eight.
__device__ int next_block(uint32_t* ctl, int nb, int x, int lane) {
  auto len = [nb](int y) { return nb > y ? (uint32_t)((nb - y + 7) >> 3) : 0u; };
  int got = -1;
  if (lane == 0) {
    const uint32_t i = take(ctl + kBlockTicket + x * kLine);
    if (i < len(x)) got = x + 8 * (int)i;
  }
  got = __builtin_amdgcn_readfirstlane(got);
  while (got < 0) {
    const bool open = lane < 8 && lane != x && peek(ctl + kBlockTicket + lane * kLine) < len(lane);
    const uint64_t m = __ballot(open);
    if (m == 0) return -1;
    // The first open list after x, cyclically.
    const uint32_t rot = (uint32_t)(((m >> (x + 1)) | (m << (7 - x))) & 0xffu);
    const int y = (x + 1 + __builtin_ctz(rot)) & 7;
    if (lane == 0) {
      const uint32_t i = take(ctl + kBlockTicket + y * kLine);
      if (i < len(y)) got = y + 8 * (int)i;
    }
    got = __builtin_amdgcn_readfirstlane(got);
  }
  return got;
}

// One BM x BN block of C_r = X_r W_r: main loop, epilogue stores and the
// block's flags.  `blk` = (partition d, block row, block column, first tile);
// `bidx` is its dispatch index; `smem` is the workgroup's S::kLds bytes of LDS;
// `tid` is threadIdx.x (a persistent caller passes it laundered, so that the
// lane's offsets are recomputed per block rather than held across blocks).  Every thread of the
// workgroup calls it; it contains workgroup barriers.
template <int BM, int BN, int BK, int NS, int WGM, int WGN, bool PP = false, bool WKN = false>
__device__ __forceinline__ void gemm_block(const GemmArgs& a, const int4 blk, int bidx,
                                           char* smem, int tid = threadIdx.x) {
  using S = Shape<BM, BN, BK, NS, WGM, WGN, WKN>;

  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave / WGN, wn = wave % WGN;
  if (a.trace && tid == 0) trace_at(a.trace, bidx);

  const int d = blk.x, br = blk.y, bc = blk.z, t_first = blk.w;
  const int row0 = br * BM;  // within the partition
  const int col0 = bc * BN;
  const int K = a.K;
  const int kbytes = K * 2;

  // Buffer descriptors bound the block's rows: X rows of partition d from
  // row0 and, with W [N][K], W rows (output columns) from col0; out-of-range
  // rows read 0.  With W [K][N] the descriptor starts at column col0 and runs
  // to W's end: columns past N read the next row's values (or 0 past the
  // end), which only reach output columns that are never stored.
  const int rows_a = min(BM, a.R - row0);
  const __amdgpu_buffer_rsrc_t ra = __builtin_amdgcn_make_buffer_rsrc(
      (void*)(a.X + ((int64_t)d * a.R + row0) * K), (short)0, rows_a * kbytes, kRsrcWord3);
  const __amdgpu_buffer_rsrc_t rb =
      WKN ? __builtin_amdgcn_make_buffer_rsrc((void*)(a.W + col0), (short)0,
                                              (int)(((int64_t)K * a.N - col0) * 2), kRsrcWord3)
          : __builtin_amdgcn_make_buffer_rsrc((void*)(a.W + (int64_t)col0 * K), (short)0,
                                              min(BN, a.N - col0) * kbytes, kRsrcWord3);

  Lanes<S> ln;
  // X (and W [N][K]): row wave*RPL + lane/LPR of each group of kWaves*RPL
  // rows, logical chunk (lane % LPR) ^ swz(row).
  const int lrow = wave * S::kRowsPerLoad + lane / S::kLanesPerRow;
  const int lchunk = (lane % S::kLanesPerRow) ^ swz<BK, S::kMF>(lrow);
  ln.voff_a = lrow * kbytes + lchunk * 16;
  ln.step_a = S::kWaves * S::kRowsPerLoad * kbytes;
  if constexpr (S::kPerLoadB) {
    // W [K][N], rows not a divisor of 1 KiB: the lane's 16 bytes of load
    // group wave + kWaves*j land at slab byte q = 1024*(wave + kWaves*j) +
    // 16*lane, i.e. row q / kRowB, physical chunk (q % kRowB) / 16, which
    // holds the logical chunk XOR kn_swz(row).
    constexpr int CPR = BN / 8;
    const int nbytes = a.N * 2;
#pragma unroll
    for (int j = 0; j < S::kLoadsB; ++j) {
      const int q = (wave + S::kWaves * j) * 64 + lane;  // 16-byte chunk of the slab
      const int krow = q / CPR, pc = q % CPR;
      ln.voff_bj[j] = krow * nbytes + ((pc ^ kn_swz(krow)) << 4);
    }
    ln.voff_b = 0;
    ln.step_b = 0;
    ln.stage_b = BK * nbytes;
  } else if constexpr (WKN) {
    // W [K][N]: slab row k holds BN columns (CPR 16-byte chunks); the lane
    // fills physical chunk lane % CPR of row wave*RPL + lane / CPR with the
    // logical chunk XOR kn_swz(k) (the same in every load group, which are
    // a multiple of 16 rows apart).
    constexpr int CPR = BN / 8, RPL = 64 / CPR;
    const int krow = wave * RPL + lane / CPR;
    const int nbytes = a.N * 2;
    static_assert(S::kWaves * RPL % 16 == 0, "load groups keep kn_swz");
    ln.voff_b = krow * nbytes + (((lane % CPR) ^ kn_swz(krow)) << 4);
    ln.step_b = S::kWaves * RPL * nbytes;
    ln.stage_b = BK * nbytes;
  } else {
    ln.voff_b = ln.voff_a;
    ln.step_b = ln.step_a;
    ln.stage_b = S::kRow;
  }

  // LDS fragment offsets.  X (and W [N][K]): MFMA lane l reads row
  // l % kMF of a kMF-row group at logical chunk (kMK/8)*ks + l / kMF, i.e. the
  // 8 consecutive k that the lane's group takes in K step ks.  W [K][N]: lane
  // l of 16-lane group g names row k0 + e (e = (l & 15) >> 2; 4 more for the
  // second read; kMK*ks more per K step) at columns c0 + 4*(l & 3) of the
  // fragment, with k0 = 8*g and c0 = 0 for 16 x 16 tiles, k0 = 8*(g >> 1)
  // and c0 = 16*(g & 1) for 32 x 32; the row's XOR is kn_swz(k0 + e), the
  // same for both reads and every K step (k0 is a multiple of 8).
  const int frow = lane % S::kMF;
  const int kgrp = lane / S::kMF;
#pragma unroll
  for (int ks = 0; ks < S::kKS; ++ks) {
    const int c = ((S::kMK / 8 * ks + kgrp) ^ swz<BK, S::kMF>(frow)) << 4;
    ln.a_off[ks] = (wm * S::kWM + frow) * S::kRow + c;
    if constexpr (!WKN) ln.b_off[ks] = (wn * S::kWN + frow) * S::kRow + c;
  }
  if constexpr (WKN) {
    const int g = lane >> 4, e = (lane & 15) >> 2, q = lane & 3;
    const int k0 = S::kMF == 16 ? 8 * g : 8 * (g >> 1);
    const int c0 = S::kMF == 16 ? 0 : 16 * (g & 1);
#pragma unroll
    for (int j = 0; j < (S::kKnXor ? 1 : S::kNT); ++j) {
      const int n = wn * S::kWN + S::kMF * j + c0 + 4 * q;
      ln.b_off[j] = (k0 + e) * S::kRowB + (((n >> 3) ^ kn_swz(k0 + e)) << 4) + (q & 1) * 8;
    }
  }

  Acc<S> acc;
#pragma unroll
  for (int i = 0; i < S::kMT; ++i)
#pragma unroll
    for (int j = 0; j < S::kNT; ++j)
#pragma unroll
      for (int v = 0; v < (S::kMF == 16 ? 4 : 16); ++v) acc.c[i][j][v] = 0.0f;

  // The epilogue's publication arguments, loaded now into scalar registers:
  // a scalar load still in flight when the main loop starts would make the
  // compiler wait for every outstanding LDS read (lgkmcnt 0) at the top of
  // each K stage, since scalar loads may return in any order.
  int publish = __builtin_amdgcn_readfirstlane(a.publish);
  int flag_all = __builtin_amdgcn_readfirstlane(a.flag_all);
  asm volatile("" : "+s"(publish), "+s"(flag_all));

  const int nk = K / BK;
  if constexpr (PP)
    pingpong_loop<S>(acc, ra, rb, smem, ln, nk, wave);
  else
    base_loop<S>(acc, ra, rb, smem, ln, nk, wave);

  // Epilogue.  With the W fragment as the MFMA's row operand, accumulator
  // element v of lane l holds output row l % 16 of its 16 x 16 tile and column
  // 4*(l/16) + v (32 x 32: row l % 32, columns 8*(v/4) + 4*(l/32) + v%4).
  // Each 32-row strip of the wave's
  // sub-block is staged through the wave's own LDS area (rows padded by 16
  // bytes so the transposed writes spread over the banks) and read back
  // row-contiguous, so every global store instruction covers whole 128-byte
  // lines: 16-byte fp32 stores for the local partition, 16-byte bf16 (8
  // columns; 8-byte where a wave's 96 columns do not split so) or 16-byte
  // fp32 stores for the outgoing contributions.
  //
  // Tiles that are released to a consumer are written with device-coherent
  // stores (cache policy SC1, the encoding of a relaxed agent-scope atomic
  // store): the data is written through this XCD's L2, so once a store is
  // acknowledged a reader on any XCD sees it and the release needs no
  // write-back of the whole L2.  Outgoing bf16 contributions that no kernel
  // of the call reads are stored non-temporally (streaming): they do not
  // linger as dirty L2 lines for the kernel's end or the reduction's reads
  // to write back (about 1 % on every workload).
  constexpr int kPitch = S::kWN * 4 + 16;
  constexpr int kLanesPerRow = S::kWN / 4;
  // Rows one store instruction covers; with a 96-column sub-block 48 of the
  // 64 lanes store (two rows) and the rest idle.
  constexpr int kRowsPerStore = 64 / kLanesPerRow;
  static_assert(32 % kRowsPerStore == 0, "a strip splits into whole store rounds");
  static_assert(S::kWaves * 32 * kPitch <= S::kLds, "epilogue staging exceeds LDS");
  __syncthreads();  // every wave is done with the pipeline buffers
  char* wbuf = smem + wave * 32 * kPitch;
  const bool local = (d == a.rank);
  const int rsub = lane / kLanesPerRow;
  const int csub = (lane % kLanesPerRow) * 4;
  const int col = col0 + wn * S::kWN + csub;
  const bool col_ok = col < a.N && lane < kRowsPerStore * kLanesPerRow;
  // The 8-column form for bf16 rows, where whole rows split over the lanes
  // (N is a multiple of 8, so a lane's 8 columns are all in or all out).
  constexpr int kLanes16 = S::kWN / 8;
  constexpr int kRows16 = 64 / kLanes16;
  constexpr bool kWide16 = 64 % kLanes16 == 0 && 32 % kRows16 == 0;
  const int rsub16 = lane / kLanes16;
  const int csub16 = (lane % kLanes16) * 8;
  const int col16 = col0 + wn * S::kWN + csub16;
  const bool col16_ok = col16 < a.N;
  const bool coherent = local ? publish != 0 : publish == 2;
  const int strip_bytes = 32 * a.N * (local || a.outgoing_f32 ? 4 : 2);
  static_assert(S::kWM % 32 == 0, "the wave sub-block splits into 32-row strips");
#pragma unroll
  for (int i = 0; i < S::kWM / 32; ++i) {
    if constexpr (S::kMF == 16) {
#pragma unroll
      for (int h = 0; h < 2; ++h)
#pragma unroll
        for (int j = 0; j < S::kNT; ++j)
          *reinterpret_cast<f32x4*>(wbuf + (16 * h + frow) * kPitch + (16 * j + 4 * kgrp) * 4) =
              acc.c[2 * i + h][j];
    } else {
#pragma unroll
      for (int j = 0; j < S::kNT; ++j)
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          f32x4 v;
          v[0] = acc.c[i][j][4 * g + 0];
          v[1] = acc.c[i][j][4 * g + 1];
          v[2] = acc.c[i][j][4 * g + 2];
          v[3] = acc.c[i][j][4 * g + 3];
          *reinterpret_cast<f32x4*>(wbuf + frow * kPitch + (32 * j + 8 * g + 4 * kgrp) * 4) = v;
        }
    }
    __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0): the strip is in LDS
    __builtin_amdgcn_wave_barrier();
    // The strip's first row (wave-uniform) in the partition, and the output
    // it lands in: the fp32 local partial or the outgoing contributions.
    const int srow = row0 + wm * S::kWM + 32 * i;
    float* const own_strip = a.own + (int64_t)srow * a.N;
    const int64_t og_row = (int64_t)d * a.R + srow;
    float* const og32_strip = static_cast<float*>(a.outgoing) + og_row * a.N;
    __bf16* const og16_strip = static_cast<__bf16*>(a.outgoing) + og_row * a.N;
    bool stored = false;
    if constexpr (kWide16) {
      if (!local && !a.outgoing_f32) {
        // bf16 contributions: 8 columns (one 16-byte store) per lane, half
        // the store instructions of the 4-column form below.
#pragma unroll
        for (int q = 0; q < 32 / kRows16; ++q) {
          const int r = q * kRows16 + rsub16;
          const char* src = wbuf + r * kPitch + csub16 * 4;
          const f32x4 v0 = *reinterpret_cast<const f32x4*>(src);
          const f32x4 v1 = *reinterpret_cast<const f32x4*>(src + 16);
          if (srow + r >= a.R || !col16_ok) continue;
          const int e = r * a.N + col16;
          bf16x8 h;
#pragma unroll
          for (int k = 0; k < 4; ++k) {
            h[k] = static_cast<__bf16>(v0[k]);
            h[4 + k] = static_cast<__bf16>(v1[k]);
          }
          if (coherent)
            __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, h),
                                                   rsrc_of(og16_strip, strip_bytes), e * 2, 0,
                                                   kCoherent);
          else
            __builtin_nontemporal_store(__builtin_bit_cast(u32x4, h),
                                        reinterpret_cast<u32x4*>(og16_strip + e));
        }
        stored = true;
      }
    }
    if (!stored) {
#pragma unroll
    for (int q = 0; q < 32 / kRowsPerStore; ++q) {
      const int r = q * kRowsPerStore + rsub;
      const f32x4 v = *reinterpret_cast<const f32x4*>(wbuf + r * kPitch + csub * 4);
      if (srow + r >= a.R || !col_ok) continue;
      const int e = r * a.N + col;  // element offset inside the strip
      if (local || a.outgoing_f32) {
        float* const base = local ? own_strip : og32_strip;
        if (coherent)
          __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, v),
                                                 rsrc_of(base, strip_bytes), e * 4, 0, kCoherent);
        else
          *reinterpret_cast<f32x4*>(base + e) = v;
      } else {
        bf16x4 h;
        h[0] = static_cast<__bf16>(v[0]);
        h[1] = static_cast<__bf16>(v[1]);
        h[2] = static_cast<__bf16>(v[2]);
        h[3] = static_cast<__bf16>(v[3]);
        if (coherent)
          __builtin_amdgcn_raw_buffer_store_b64(__builtin_bit_cast(u32x2, h),
                                                rsrc_of(og16_strip, strip_bytes), e * 2, 0,
                                                kCoherent);
        else
          __builtin_nontemporal_store(__builtin_bit_cast(u32x2, h),
                                      reinterpret_cast<u32x2*>(og16_strip + e));
      }
    }
    }
    __builtin_amdgcn_s_waitcnt(0xC07F);  // strip read back before the next overwrites it
    __builtin_amdgcn_wave_barrier();
  }

  // Publish (Sec. 4.2): all stores of the block, then the tiles' flags.
  //  1. Every wave waits until each of its own stores has been acknowledged
  //     (vmcnt 0).  The released tiles were stored device-coherent (SC1), so
  //     an acknowledged store is visible to a device-coherent load from any
  //     XCD.  The wait is explicit: the workgroup barrier's own fence has
  //     workgroup scope and does not wait for outstanding stores.
  //  2. The workgroup barrier: no wave passes it before every wave's stores
  //     are acknowledged.
  //  3. Thread 0 stores the covered tiles' flags (agent scope).
  // The release is therefore a wait for acknowledgements, not a write-back of
  // the XCD's whole L2 (which an agent-scope release fence would issue).
  // Flags of tiles bound for peers only mark progress; they are stored when
  // some wait reads them (flag_all).
  if (publish != 0 && (local || flag_all)) {
    __builtin_amdgcn_sched_barrier(0);
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();
    if (tid == 0) {
      const int sub_m = BM / a.tm, sub_n = BN / a.tn;
      const int vm = min(sub_m, a.Rt - br * sub_m);
      const int vn = min(sub_n, a.Ct - bc * sub_n);
      const uint32_t epoch = peek(a.ctl + kEpoch);
      uint32_t* f = a.flags + (int64_t)d * a.Q + t_first;
      for (int t = 0; t < vm * vn; ++t)
        __hip_atomic_store(f + t, epoch, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
  }
  if (a.trace) {  // uniform: every wave's stores issued
    __syncthreads();
    if (tid == 0) trace_at(a.trace, (int64_t)a.trace_nb + bidx);
  }
}

}  // namespace
}  // namespace entwine
