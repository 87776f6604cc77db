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
//  * 256 threads = 4 waves of 64 in a 2 x 2 arrangement; a wave owns a
//    (BM/2) x (BN/2) sub-block computed with v_mfma_f32_32x32x16_bf16 into
//    fp32 accumulators.
//  * K advances in stages of 64 (128 bytes per row).  Each stage of X rows and
//    W rows (W is [N][K], K contiguous, so both operands are K-major) moves
//    from global memory straight into LDS with global_load_lds_dwordx4: one
//    wave instruction fills 1 KiB = 8 rows of 128 bytes.  Two stages are
//    double-buffered so the next stage's loads overlap the current MFMAs.
//  * LDS rows are XOR-swizzled in 16-byte chunks (chunk c of row r is stored
//    at c ^ swz(r)), so the 32 rows that one MFMA operand read touches spread
//    over all banks.  The swizzle is realised by choosing each lane's global
//    source address, since the LDS destination of lane l is fixed at 16*l.
//  * Rows past the partition's end (or N's end) are clamped on load and
//    masked on store, so edge blocks never read out of bounds.
//  * Publication: every wave issues an agent-scope release fence after its
//    own stores (the gfx950 workgroup barrier does not wait for other waves'
//    stores), the workgroup synchronizes, then one lane per covered tile
//    release-stores the call's epoch into the tile's flag.
#include "kernels.h"

namespace entwine {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

constexpr int kBK = 64;          // K per stage
constexpr int kRowBytes = 128;   // kBK bf16
constexpr int kThreads = 256;

typedef __attribute__((address_space(3))) void* lds_ptr_t;

__device__ __forceinline__ int swz(int r) { return (r & 7) ^ ((r >> 3) & 1); }

template <int BM, int BN>
struct Tile {
  static constexpr int kWM = BM / 2, kWN = BN / 2;  // wave sub-block
  static constexpr int kMT = kWM / 32, kNT = kWN / 32;
  static constexpr int kStageA = BM * kRowBytes, kStageB = BN * kRowBytes;
  static constexpr int kStage = kStageA + kStageB;
  static constexpr int kLds = 2 * kStage;
  static constexpr int kOctA = BM / 8 / 4, kOctB = BN / 8 / 4;  // octets per wave
};

// Issue the global->LDS copies of one K stage.  Octet o (8 rows) of a
// tile is loaded by wave (o % 4); lane l fills physical chunk (l & 7) of row
// 8o + (l >> 3), i.e. logical chunk (l & 7) ^ swz(row).
template <int BM, int BN>
__device__ __forceinline__ void load_stage(const uint16_t* __restrict__ X,
                                           const uint16_t* __restrict__ W, char* lds_stage,
                                           int K, int k0, int wave, int lane,
                                           const int* __restrict__ a_row,
                                           const int* __restrict__ b_row) {
  using T = Tile<BM, BN>;
  const int r_in = lane >> 3;
  const int pc = lane & 7;
#pragma unroll
  for (int j = 0; j < T::kOctA; ++j) {
    const int o = wave + 4 * j;
    const int r = 8 * o + r_in;
    const uint16_t* src = X + (int64_t)a_row[j] * K + k0 + 8 * (pc ^ swz(r));
    __builtin_amdgcn_global_load_lds(src, (lds_ptr_t)(lds_stage + o * 1024), 16, 0, 0);
  }
#pragma unroll
  for (int j = 0; j < T::kOctB; ++j) {
    const int o = wave + 4 * j;
    const int r = 8 * o + r_in;
    const uint16_t* src = W + (int64_t)b_row[j] * K + k0 + 8 * (pc ^ swz(r));
    __builtin_amdgcn_global_load_lds(src, (lds_ptr_t)(lds_stage + T::kStageA + o * 1024), 16,
                                     0, 0);
  }
}

__device__ __forceinline__ bf16x8 read_frag(const char* lds_tile, int row, int chunk) {
  return *reinterpret_cast<const bf16x8*>(lds_tile + row * kRowBytes +
                                          ((chunk ^ swz(row)) << 4));
}

template <int BM, int BN>
__global__ __launch_bounds__(kThreads) void gemm_publish_kernel(GemmArgs a) {
  using T = Tile<BM, BN>;
  extern __shared__ __attribute__((aligned(1024))) char smem[];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave >> 1, wn = wave & 1;

  const int4 blk = reinterpret_cast<const int4*>(a.blocks)[blockIdx.x];
  const int d = blk.x, br = blk.y, bc = blk.z, t_first = blk.w;
  const int row_base = br * BM;  // within the partition
  const int col_base = bc * BN;

  // Source rows of this lane's load octets, clamped to the partition / N.
  int a_row[T::kOctA], b_row[T::kOctB];
#pragma unroll
  for (int j = 0; j < T::kOctA; ++j) {
    const int r = 8 * (wave + 4 * j) + (lane >> 3);
    a_row[j] = d * a.R + min(row_base + r, a.R - 1);
  }
#pragma unroll
  for (int j = 0; j < T::kOctB; ++j) {
    const int r = 8 * (wave + 4 * j) + (lane >> 3);
    b_row[j] = min(col_base + r, a.N - 1);
  }

  f32x16 acc[T::kMT][T::kNT];
#pragma unroll
  for (int i = 0; i < T::kMT; ++i)
#pragma unroll
    for (int j = 0; j < T::kNT; ++j)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[i][j][v] = 0.0f;

  const int nk = a.K / kBK;
  load_stage<BM, BN>(a.X, a.W, smem, a.K, 0, wave, lane, a_row, b_row);
  __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0): this wave's stage-0 copies landed
  __syncthreads();

  const int a_row0 = wm * T::kWM + (lane & 31);
  const int b_row0 = wn * T::kWN + (lane & 31);
  const int khalf = lane >> 5;

  for (int kt = 0; kt < nk; ++kt) {
    char* cur = smem + (kt & 1) * T::kStage;
    if (kt + 1 < nk)
      load_stage<BM, BN>(a.X, a.W, smem + ((kt + 1) & 1) * T::kStage, a.K, (kt + 1) * kBK,
                         wave, lane, a_row, b_row);
    const char* As = cur;
    const char* Bs = cur + T::kStageA;
#pragma unroll
    for (int ks = 0; ks < kBK / 16; ++ks) {
      const int chunk = 2 * ks + khalf;
      bf16x8 af[T::kMT], bfr[T::kNT];
#pragma unroll
      for (int i = 0; i < T::kMT; ++i) af[i] = read_frag(As, a_row0 + 32 * i, chunk);
#pragma unroll
      for (int j = 0; j < T::kNT; ++j) bfr[j] = read_frag(Bs, b_row0 + 32 * j, chunk);
#pragma unroll
      for (int i = 0; i < T::kMT; ++i)
#pragma unroll
        for (int j = 0; j < T::kNT; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[i], bfr[j], acc[i][j], 0, 0, 0);
    }
    __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0): next stage's copies landed
    __syncthreads();                      // and every wave is done with `cur`
  }

  // Epilogue.  Accumulator element v of lane l holds row
  // 8*(v/4) + 4*(l/32) + (v%4) and column l%32 of its 32x32 MFMA tile.
  const int col_l = lane & 31;
  const int row_l = 4 * (lane >> 5);
  const bool local = (d == a.rank);
#pragma unroll
  for (int i = 0; i < T::kMT; ++i) {
#pragma unroll
    for (int j = 0; j < T::kNT; ++j) {
      const int col = col_base + wn * T::kWN + 32 * j + col_l;
      if (col >= a.N) continue;
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const int prow = row_base + wm * T::kWM + 32 * i + 8 * (v >> 2) + row_l + (v & 3);
        if (prow >= a.R) continue;
        const float x = acc[i][j][v];
        if (local) {
          a.own[(int64_t)prow * a.N + col] = x;
        } else {
          const int64_t e = (int64_t)(d * a.R + prow) * a.N + col;
          if (a.outgoing_f32)
            static_cast<float*>(a.outgoing)[e] = x;
          else
            static_cast<__bf16*>(a.outgoing)[e] = static_cast<__bf16>(x);
        }
      }
    }
  }

  // Publish (Sec. 4.2): all stores of the block, then the tiles' flags.
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "agent");
  __syncthreads();
  const int sub_m = BM / a.tm, sub_n = BN / a.tn;
  const int vm = min(sub_m, a.Rt - br * sub_m);
  const int vn = min(sub_n, a.Ct - bc * sub_n);
  if (tid < vm * vn)
    __hip_atomic_store(a.flags + (int64_t)d * a.Q + t_first + tid, a.epoch, __ATOMIC_RELEASE,
                       __HIP_MEMORY_SCOPE_AGENT);
}

template <int BM, int BN>
hipError_t launch_shape(const GemmArgs& a, int num_blocks, hipStream_t s) {
  using T = Tile<BM, BN>;
  static bool attr_set = false;
  if (!attr_set) {
    hipError_t e = hipFuncSetAttribute((const void*)gemm_publish_kernel<BM, BN>,
                                       hipFuncAttributeMaxDynamicSharedMemorySize, T::kLds);
    if (e != hipSuccess) return e;
    attr_set = true;
  }
  gemm_publish_kernel<BM, BN><<<num_blocks, kThreads, T::kLds, s>>>(a);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_gemm_publish(const GemmArgs& a, int bm, int bn, int num_blocks,
                               hipStream_t stream) {
  if (bm == 128 && bn == 128) return launch_shape<128, 128>(a, num_blocks, stream);
  if (bm == 128 && bn == 256) return launch_shape<128, 256>(a, num_blocks, stream);
  if (bm == 256 && bn == 128) return launch_shape<256, 128>(a, num_blocks, stream);
  if (bm == 256 && bn == 256) return launch_shape<256, 256>(a, num_blocks, stream);
  return hipErrorInvalidValue;
}

}  // namespace entwine
