// rmsnorm.hip -- the layer chain's normalization after the ReduceScatter.
//
// Method: "Entwine: Coordinating Tiled Computation and Fine-Grained
// Communication across GPUs" (paperpeel.com/paper/2609.11562), Sec. 5.2.2
// (Layer-Level Performance): the ReduceScatter's output, with the residual
// added, goes through an RMSNorm.  The residual addition is part of the
// reduction's store (reduce_task.h); this kernel normalizes the rows:
//   y[i][j] = gamma[j] * h[i][j] / sqrt(mean_j(h[i][j]^2) + eps).
//
// MI355X design.  HBM-bound: one 256-thread workgroup per row.  The first
// pass reads the row (16-byte loads, 8 elements per thread step) and sums
// squares in fp32; wave sums use cross-lane shuffles and the four wave sums
// meet in LDS.  The second pass reads the row again -- an L2 hit, rows are at
// most tens of KiB -- with the weight, and writes y with 16-byte stores.
// Bytes per element: h read once from HBM, y written once.
#include "kernels.h"

namespace entwine {
namespace {

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef unsigned u32x4 __attribute__((ext_vector_type(4)));

struct Row8 {
  float v[8];
};

template <bool F32>
__device__ __forceinline__ Row8 load8(const void* base, int64_t e) {
  Row8 r;
  if constexpr (F32) {
    const f32x4 a = *reinterpret_cast<const f32x4*>(static_cast<const float*>(base) + e);
    const f32x4 b = *reinterpret_cast<const f32x4*>(static_cast<const float*>(base) + e + 4);
    for (int i = 0; i < 4; ++i) {
      r.v[i] = a[i];
      r.v[4 + i] = b[i];
    }
  } else {
    const u32x4 w = *reinterpret_cast<const u32x4*>(static_cast<const uint16_t*>(base) + e);
    for (int i = 0; i < 4; ++i) {
      r.v[2 * i] = __uint_as_float(w[i] << 16);  // bf16 -> fp32 is exact
      r.v[2 * i + 1] = __uint_as_float(w[i] & 0xffff0000u);
    }
  }
  return r;
}

template <bool F32>
__device__ __forceinline__ void store8(void* base, int64_t e, const Row8& r) {
  if constexpr (F32) {
    f32x4 a, b;
    for (int i = 0; i < 4; ++i) {
      a[i] = r.v[i];
      b[i] = r.v[4 + i];
    }
    *reinterpret_cast<f32x4*>(static_cast<float*>(base) + e) = a;
    *reinterpret_cast<f32x4*>(static_cast<float*>(base) + e + 4) = b;
  } else {
    u32x4 w;
    for (int i = 0; i < 4; ++i) {
      const __bf16 lo = static_cast<__bf16>(r.v[2 * i]);  // round to nearest even
      const __bf16 hi = static_cast<__bf16>(r.v[2 * i + 1]);
      w[i] = (uint32_t)__builtin_bit_cast(uint16_t, lo) |
             ((uint32_t)__builtin_bit_cast(uint16_t, hi) << 16);
    }
    *reinterpret_cast<u32x4*>(static_cast<uint16_t*>(base) + e) = w;
  }
}

constexpr int kThreads = 256;

template <bool F32>
__global__ __launch_bounds__(kThreads) void rmsnorm_rows_kernel(const void* h, const void* gamma,
                                                                void* y, int N, float eps) {
  __shared__ float s_part[kThreads / 64];
  const int tid = threadIdx.x;
  const int64_t row = (int64_t)blockIdx.x * N;
  const int chunks = N >> 3;
  float ss = 0.0f;
  for (int c = tid; c < chunks; c += kThreads) {
    const Row8 v = load8<F32>(h, row + 8 * c);
    for (int i = 0; i < 8; ++i) ss += v.v[i] * v.v[i];
  }
  for (int off = 32; off > 0; off >>= 1) ss += __shfl_xor(ss, off, 64);
  if ((tid & 63) == 0) s_part[tid >> 6] = ss;
  __syncthreads();
  float total = 0.0f;
  for (int w = 0; w < kThreads / 64; ++w) total += s_part[w];
  const float scale = 1.0f / __builtin_sqrtf(total / (float)N + eps);
  for (int c = tid; c < chunks; c += kThreads) {
    const Row8 v = load8<F32>(h, row + 8 * c);
    const Row8 g = load8<F32>(gamma, 8 * c);
    Row8 o;
    for (int i = 0; i < 8; ++i) o.v[i] = g.v[i] * (v.v[i] * scale);
    store8<F32>(y, row + 8 * c, o);
  }
}

}  // namespace

hipError_t launch_rmsnorm(const void* h, const void* gamma, void* y, int rows, int N, float eps,
                          int out_f32, hipStream_t stream) {
  if (rows <= 0) return hipSuccess;
  if (out_f32)
    rmsnorm_rows_kernel<true><<<rows, kThreads, 0, stream>>>(h, gamma, y, N, eps);
  else
    rmsnorm_rows_kernel<false><<<rows, kThreads, 0, stream>>>(h, gamma, y, N, eps);
  return hipGetLastError();
}

}  // namespace entwine
