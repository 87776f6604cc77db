// tile_reduce.hip -- the consumer: a persistent tile-reduction kernel.
//
// Method: "Entwine: Coordinating Tiled Computation and Fine-Grained
// Communication across GPUs" (paperpeel.com/paper/2609.11562).
//  * Sec. 3.1 "Matching task order": consumer workgroup j takes tasks j, j+x,
//    j+2x, ... in production order and waits for each tile before reducing it.
//  * Sec. 3.2 "Communication budget": x = the grid size, fixed for the call.
//  * Sec. 4.2: before a tile is read, its flags (the local one and the
//    peers') are observed with acquire semantics and the workgroup then
//    synchronizes; each thread reduces a disjoint part of the tile, starting
//    from the local contribution and adding the peers in rank order; each
//    output element has exactly one writer.
//
// MI355X mapping.  Wave 0 polls the tile's P flags in parallel, one lane per
// source rank, with relaxed agent-scope loads, then issues one agent-scope
// acquire fence (which invalidates this XCD's non-coherent L2 lines, so the
// producer's data written back from another XCD is seen) and a workgroup
// barrier releases the other waves.  The element loop moves 8 elements per
// thread step: two 16-byte fp32 loads of the local partial, one 16-byte load
// per bf16 peer (all issued before any add), fp32 adds in rank order, one
// round-to-nearest-even conversion and one 16-byte store.
#include "kernels.h"

namespace entwine {
namespace {

struct F8 {
  float v[8];
};

__device__ __forceinline__ F8 load8_f32(const float* p) {
  const float4 a = *reinterpret_cast<const float4*>(p);
  const float4 b = *reinterpret_cast<const float4*>(p + 4);
  F8 r;
  r.v[0] = a.x; r.v[1] = a.y; r.v[2] = a.z; r.v[3] = a.w;
  r.v[4] = b.x; r.v[5] = b.y; r.v[6] = b.z; r.v[7] = b.w;
  return r;
}

// Raw 16-byte (bf16) or 32-byte (fp32) chunk of 8 elements.
template <bool F32>
struct Raw8;
template <>
struct Raw8<false> {
  uint4 w;
};
template <>
struct Raw8<true> {
  float4 a, b;
};

template <bool F32>
__device__ __forceinline__ Raw8<F32> load_raw8(const void* base, int64_t e);
template <>
__device__ __forceinline__ Raw8<false> load_raw8<false>(const void* base, int64_t e) {
  return Raw8<false>{*reinterpret_cast<const uint4*>(static_cast<const uint16_t*>(base) + e)};
}
template <>
__device__ __forceinline__ Raw8<true> load_raw8<true>(const void* base, int64_t e) {
  const float* p = static_cast<const float*>(base) + e;
  return Raw8<true>{*reinterpret_cast<const float4*>(p), *reinterpret_cast<const float4*>(p + 4)};
}

// bf16 -> fp32 is exact: the bf16 bits are the upper half of the binary32.
__device__ __forceinline__ float lo_bf16(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float hi_bf16(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

__device__ __forceinline__ void add8(F8& acc, const Raw8<false>& r) {
  const uint32_t w[4] = {r.w.x, r.w.y, r.w.z, r.w.w};
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    acc.v[2 * i] += lo_bf16(w[i]);
    acc.v[2 * i + 1] += hi_bf16(w[i]);
  }
}
__device__ __forceinline__ void add8(F8& acc, const Raw8<true>& r) {
  acc.v[0] += r.a.x; acc.v[1] += r.a.y; acc.v[2] += r.a.z; acc.v[3] += r.a.w;
  acc.v[4] += r.b.x; acc.v[5] += r.b.y; acc.v[6] += r.b.z; acc.v[7] += r.b.w;
}

// fp32 -> bf16, round to nearest even (the hardware conversion on gfx950).
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  const __bf16 l = static_cast<__bf16>(lo);
  const __bf16 h = static_cast<__bf16>(hi);
  return (uint32_t)__builtin_bit_cast(uint16_t, l) | ((uint32_t)__builtin_bit_cast(uint16_t, h) << 16);
}

template <bool F32>
__device__ __forceinline__ void store8(void* base, int64_t e, const F8& acc);
template <>
__device__ __forceinline__ void store8<false>(void* base, int64_t e, const F8& acc) {
  uint4 o;
  o.x = pack_bf16x2(acc.v[0], acc.v[1]);
  o.y = pack_bf16x2(acc.v[2], acc.v[3]);
  o.z = pack_bf16x2(acc.v[4], acc.v[5]);
  o.w = pack_bf16x2(acc.v[6], acc.v[7]);
  *reinterpret_cast<uint4*>(static_cast<uint16_t*>(base) + e) = o;
}
template <>
__device__ __forceinline__ void store8<true>(void* base, int64_t e, const F8& acc) {
  float* p = static_cast<float*>(base) + e;
  *reinterpret_cast<float4*>(p) = make_float4(acc.v[0], acc.v[1], acc.v[2], acc.v[3]);
  *reinterpret_cast<float4*>(p + 4) = make_float4(acc.v[4], acc.v[5], acc.v[6], acc.v[7]);
}

// Wave 0 waits until every flag that tile t depends on equals `epoch`.
// Lane r (< P) watches source rank r's flag.  Returns false if the watchdog
// expired (uniform across the wave).
__device__ bool wait_tile(const ReduceArgs& a, int t, int lane) {
  int32_t idx = -1;
  if (lane < a.P) idx = a.waits[t * a.P + lane];
  if (t == a.withhold_tile && lane == a.rank) idx = a.never_flag;
  const uint32_t* f = idx >= 0 ? a.flags + idx : nullptr;
  const uint64_t start = wall_clock64();
  while (true) {
    bool ready = true;
    if (f) ready = __hip_atomic_load(f, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) == a.epoch;
    if (__all(ready)) break;
    if (wall_clock64() - start > a.timeout_ticks) {
      if (lane == 0)
        __hip_atomic_store(a.error, (int32_t)5 /* ENTWINE_ERR_TIMEOUT */, __ATOMIC_RELAXED,
                           __HIP_MEMORY_SCOPE_AGENT);
      return false;
    }
    __builtin_amdgcn_s_sleep(2);
  }
  // One acquire per task: later reads of the tile see the producers' stores.
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
  return true;
}

template <int THREADS, bool PEER_F32, bool OUT_F32>
__global__ __launch_bounds__(THREADS) void tile_reduce_kernel(ReduceArgs a) {
  __shared__ int s_abort;
  const int tid = threadIdx.x;
  const int chunks_per_row = a.tn >> 3;
  const int slab_rows = a.tm / a.slabs;
  for (int task = blockIdx.x; task < a.ntasks; task += gridDim.x) {
    const int t = task / a.slabs;
    const int slab = task - t * a.slabs;
    if (tid < 64) {
      const bool ok = wait_tile(a, t, tid);
      if (tid == 0) s_abort = ok ? 0 : 1;
    }
    __syncthreads();
    if (s_abort) return;  // uniform: every thread read the same value

    const int row0 = a.tiles[2 * t] * a.tm + slab * slab_rows;
    const int col0 = a.tiles[2 * t + 1] * a.tn;
    const int rows = min(slab_rows, a.R - row0);
    const int n_chunks = rows > 0 ? rows * chunks_per_row : 0;
    for (int c = tid; c < n_chunks; c += THREADS) {
      const int r = c / chunks_per_row;
      const int col = col0 + ((c - r * chunks_per_row) << 3);
      if (col >= a.N) continue;
      const int64_t e = (int64_t)(row0 + r) * a.N + col;
      // Issue every load before the first add.
      F8 acc = load8_f32(a.own + e);
      Raw8<PEER_F32> pv[kMaxRanks];
#pragma unroll
      for (int q = 0; q < kMaxRanks; ++q)
        if (q < a.P && q != a.rank) pv[q] = load_raw8<PEER_F32>(a.peers[q], e);
#pragma unroll
      for (int q = 0; q < kMaxRanks; ++q)
        if (q < a.P && q != a.rank) add8(acc, pv[q]);
      store8<OUT_F32>(a.out, e, acc);
    }
    // s_abort is rewritten by the next task's wait; keep it stable until
    // every wave has read it.
    __syncthreads();
  }
}

template <int THREADS>
hipError_t launch_threads(const ReduceArgs& a, int peer_f32, int out_f32, int grid,
                          hipStream_t s) {
  if (!peer_f32 && !out_f32)
    tile_reduce_kernel<THREADS, false, false><<<grid, THREADS, 0, s>>>(a);
  else if (!peer_f32 && out_f32)
    tile_reduce_kernel<THREADS, false, true><<<grid, THREADS, 0, s>>>(a);
  else if (peer_f32 && !out_f32)
    tile_reduce_kernel<THREADS, true, false><<<grid, THREADS, 0, s>>>(a);
  else
    tile_reduce_kernel<THREADS, true, true><<<grid, THREADS, 0, s>>>(a);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_tile_reduce(const ReduceArgs& a, int peer_f32, int out_f32, int threads,
                              int grid, hipStream_t stream) {
  switch (threads) {
    case 128: return launch_threads<128>(a, peer_f32, out_f32, grid, stream);
    case 256: return launch_threads<256>(a, peer_f32, out_f32, grid, stream);
    case 512: return launch_threads<512>(a, peer_f32, out_f32, grid, stream);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace entwine
