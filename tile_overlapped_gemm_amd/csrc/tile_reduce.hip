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
// MI355X mapping.
//  * A task is one row slab of a reduction tile (slabs = 1: the whole tile),
//    numbered tile-major, so the tiles' slabs spread over consecutive
//    workgroups.
//  * Wave 0 polls the task's flags in parallel, one lane per flag, with
//    relaxed agent-scope loads and an s_sleep back-off, then issues one
//    agent-scope acquire fence (it invalidates this XCD's L2 so that data
//    written back by a producer on another XCD is read from memory); the
//    other waves wait at the workgroup barrier meanwhile.
//  * The element loop moves 8 elements per thread step: two 16-byte fp32 loads
//    of the local partial and one 16-byte load per bf16 peer.  Two steps are
//    loaded before any add so that 2 * (P + 1) loads per thread are in flight.
//    fp32 adds run in rank order; one round-to-nearest-even conversion and one
//    16-byte store per step.
//  * Without waits (the sequential schedule, after the GEMM kernel has
//    finished) the kernel streams the partition as one flat array with a
//    grid-stride loop.
#include "kernels.h"

namespace entwine {
namespace {

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef unsigned u32x4 __attribute__((ext_vector_type(4)));

struct F8 {
  float v[8];
};

// Raw chunk of 8 elements: 16 bytes of bf16 or 32 bytes of fp32.
template <bool F32>
struct Raw8;
template <>
struct Raw8<false> {
  u32x4 w;
};
template <>
struct Raw8<true> {
  f32x4 a, b;
};

template <bool F32>
__device__ __forceinline__ Raw8<F32> load_raw8(const void* base, int64_t e);
// Every input element is read exactly once: nontemporal (streaming) loads
// keep the partials from displacing the concurrent GEMM's operands in the
// caches.
template <>
__device__ __forceinline__ Raw8<false> load_raw8<false>(const void* base, int64_t e) {
  return Raw8<false>{__builtin_nontemporal_load(
      reinterpret_cast<const u32x4*>(static_cast<const uint16_t*>(base) + e))};
}
template <>
__device__ __forceinline__ Raw8<true> load_raw8<true>(const void* base, int64_t e) {
  const float* p = static_cast<const float*>(base) + e;
  return Raw8<true>{__builtin_nontemporal_load(reinterpret_cast<const f32x4*>(p)),
                    __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(p + 4))};
}

// bf16 -> fp32 is exact: the bf16 bits are the upper half of the binary32.
__device__ __forceinline__ float lo_bf16(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float hi_bf16(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

__device__ __forceinline__ F8 widen(const Raw8<true>& r) {
  F8 f;
  f.v[0] = r.a[0]; f.v[1] = r.a[1]; f.v[2] = r.a[2]; f.v[3] = r.a[3];
  f.v[4] = r.b[0]; f.v[5] = r.b[1]; f.v[6] = r.b[2]; f.v[7] = r.b[3];
  return f;
}

__device__ __forceinline__ void add8(F8& acc, const Raw8<false>& r) {
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    acc.v[2 * i] += lo_bf16(r.w[i]);
    acc.v[2 * i + 1] += hi_bf16(r.w[i]);
  }
}
__device__ __forceinline__ void add8(F8& acc, const Raw8<true>& r) {
  acc.v[0] += r.a[0]; acc.v[1] += r.a[1]; acc.v[2] += r.a[2]; acc.v[3] += r.a[3];
  acc.v[4] += r.b[0]; acc.v[5] += r.b[1]; acc.v[6] += r.b[2]; acc.v[7] += r.b[3];
}

// fp32 -> bf16, round to nearest even (the hardware conversion on gfx950).
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  const __bf16 l = static_cast<__bf16>(lo);
  const __bf16 h = static_cast<__bf16>(hi);
  return (uint32_t)__builtin_bit_cast(uint16_t, l) |
         ((uint32_t)__builtin_bit_cast(uint16_t, h) << 16);
}

template <bool F32>
__device__ __forceinline__ void store8(void* base, int64_t e, const F8& acc);
template <>
__device__ __forceinline__ void store8<false>(void* base, int64_t e, const F8& acc) {
  u32x4 o;
  o[0] = pack_bf16x2(acc.v[0], acc.v[1]);
  o[1] = pack_bf16x2(acc.v[2], acc.v[3]);
  o[2] = pack_bf16x2(acc.v[4], acc.v[5]);
  o[3] = pack_bf16x2(acc.v[6], acc.v[7]);
  *reinterpret_cast<u32x4*>(static_cast<uint16_t*>(base) + e) = o;
}
template <>
__device__ __forceinline__ void store8<true>(void* base, int64_t e, const F8& acc) {
  float* p = static_cast<float*>(base) + e;
  f32x4 lo, hi;
  lo[0] = acc.v[0]; lo[1] = acc.v[1]; lo[2] = acc.v[2]; lo[3] = acc.v[3];
  hi[0] = acc.v[4]; hi[1] = acc.v[5]; hi[2] = acc.v[6]; hi[3] = acc.v[7];
  *reinterpret_cast<f32x4*>(p) = lo;
  *reinterpret_cast<f32x4*>(p + 4) = hi;
}

// Reduce U chunks at element offsets e[0..U): all loads first, then the
// fixed-order fp32 sums, then the stores.  ok[u] masks chunks past the end.
template <int U, bool PEER_F32, bool OUT_F32>
__device__ __forceinline__ void reduce_chunks(const ReduceArgs& a, const int64_t (&e)[U],
                                              const bool (&ok)[U]) {
  Raw8<true> own[U];
  Raw8<PEER_F32> pv[U][kMaxRanks];
#pragma unroll
  for (int u = 0; u < U; ++u) {
    if (!ok[u]) continue;
    own[u] = load_raw8<true>(a.own, e[u]);
#pragma unroll
    for (int q = 0; q < kMaxRanks; ++q)
      if (q < a.P && q != a.rank) pv[u][q] = load_raw8<PEER_F32>(a.peers[q], e[u]);
  }
#pragma unroll
  for (int u = 0; u < U; ++u) {
    if (!ok[u]) continue;
    F8 acc = widen(own[u]);
#pragma unroll
    for (int q = 0; q < kMaxRanks; ++q)
      if (q < a.P && q != a.rank) add8(acc, pv[u][q]);
    store8<OUT_F32>(a.out, e[u], acc);
  }
}

// Wave 0 waits until every flag that task tile t depends on equals `epoch`.
// Lane k (< P + 1) watches wait slot k.  Returns false if the watchdog
// expired (uniform across the wave).
__device__ bool wait_tile(const ReduceArgs& a, uint32_t epoch, int t, int lane) {
  int32_t idx = -1;
  if (lane < a.wait_slots) idx = a.waits[t * a.wait_slots + lane];
  if (t == a.withhold_tile && lane == a.rank) idx = a.never_flag;
  const uint32_t* f = idx >= 0 ? a.flags + idx : nullptr;
  const uint64_t start = wall_clock64();
  while (true) {
    bool ready = true;
    if (f) ready = __hip_atomic_load(f, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) == epoch;
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

constexpr int kUnroll = 2;

template <int THREADS, bool PEER_F32, bool OUT_F32>
__global__ __launch_bounds__(THREADS) void tile_reduce_kernel(ReduceArgs a) {
  __shared__ int s_abort[2];
  const int tid = threadIdx.x;
  const uint32_t epoch = a.ctl[kEpoch];
  const int chunks_per_row = a.tn >> 3;
  const int slab_rows = a.tm / a.slabs;
  int parity = 0;
  for (int task = blockIdx.x; task < a.ntasks; task += gridDim.x, parity ^= 1) {
    const int t = task / a.slabs;
    const int slab = task - t * a.slabs;
    if (tid < 64) {
      const bool ok = a.nowait || wait_tile(a, epoch, t, tid);
      if (tid == 0) s_abort[parity] = ok ? 0 : 1;
    }
    // The flag wait is ordered before every wave's reads of the tile.  The
    // abort word alternates between two slots, so wave 0 can write the next
    // task's word while a slower wave still reads this one.
    __syncthreads();
    if (s_abort[parity]) break;  // uniform: every thread read the same value

    const int row0 = a.tiles[2 * t] * a.tm + slab * slab_rows;
    const int col0 = a.tiles[2 * t + 1] * a.tn;
    const int rows = min(slab_rows, a.R - row0);
    const int cols = min(a.tn, a.N - col0);
    const int n_chunks = rows > 0 ? rows * chunks_per_row : 0;
    for (int c0 = tid; c0 < n_chunks; c0 += kUnroll * THREADS) {
      int64_t e[kUnroll];
      bool ok[kUnroll];
#pragma unroll
      for (int u = 0; u < kUnroll; ++u) {
        const int c = c0 + u * THREADS;
        const int r = c / chunks_per_row;
        const int col = (c - r * chunks_per_row) << 3;
        ok[u] = c < n_chunks && col < cols;
        e[u] = (int64_t)(row0 + r) * a.N + col0 + col;
      }
      reduce_chunks<kUnroll, PEER_F32, OUT_F32>(a, e, ok);
    }
  }
  // Every workgroup, finished or timed out, checks out.
  if (tid == 0 && !a.nowait) check_out(a.ctl, epoch);
}

// The sequential schedule's reduction: no flags; the partition is one flat
// array of R * N / 8 chunks walked with a grid-stride loop.
template <int THREADS, bool PEER_F32, bool OUT_F32>
__global__ __launch_bounds__(THREADS) void flat_reduce_kernel(ReduceArgs a) {
  const int64_t n_chunks = (int64_t)a.R * a.N / 8;
  const int64_t stride = (int64_t)gridDim.x * THREADS * kUnroll;
  for (int64_t c0 = (int64_t)blockIdx.x * THREADS * kUnroll + threadIdx.x; c0 < n_chunks;
       c0 += stride) {
    int64_t e[kUnroll];
    bool ok[kUnroll];
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
      const int64_t c = c0 + u * THREADS;
      ok[u] = c < n_chunks;
      e[u] = c * 8;
    }
    reduce_chunks<kUnroll, PEER_F32, OUT_F32>(a, e, ok);
  }
}

template <int THREADS, bool PEER_F32, bool OUT_F32>
void launch_typed(const ReduceArgs& a, bool flat, int grid, hipStream_t s) {
  if (flat)
    flat_reduce_kernel<THREADS, PEER_F32, OUT_F32><<<grid, THREADS, 0, s>>>(a);
  else
    tile_reduce_kernel<THREADS, PEER_F32, OUT_F32><<<grid, THREADS, 0, s>>>(a);
}

template <int THREADS>
hipError_t launch_threads(const ReduceArgs& a, int peer_f32, int out_f32, bool flat, int grid,
                          hipStream_t s) {
  if (!peer_f32 && !out_f32)
    launch_typed<THREADS, false, false>(a, flat, grid, s);
  else if (!peer_f32 && out_f32)
    launch_typed<THREADS, false, true>(a, flat, grid, s);
  else if (peer_f32 && !out_f32)
    launch_typed<THREADS, true, false>(a, flat, grid, s);
  else
    launch_typed<THREADS, true, true>(a, flat, grid, s);
  return hipGetLastError();
}

template <int THREADS, bool PEER_F32, bool OUT_F32>
int regs_typed() {
  hipFuncAttributes at{};
  if (hipFuncGetAttributes(&at, (const void*)tile_reduce_kernel<THREADS, PEER_F32, OUT_F32>) !=
      hipSuccess)
    return 0;
  return at.numRegs;
}

template <int THREADS>
int regs_threads(int peer_f32, int out_f32) {
  if (!peer_f32 && !out_f32) return regs_typed<THREADS, false, false>();
  if (!peer_f32 && out_f32) return regs_typed<THREADS, false, true>();
  if (peer_f32 && !out_f32) return regs_typed<THREADS, true, false>();
  return regs_typed<THREADS, true, true>();
}

}  // namespace

int reduce_registers(int threads, int peer_f32, int out_f32) {
  switch (threads) {
    case 128: return regs_threads<128>(peer_f32, out_f32);
    case 256: return regs_threads<256>(peer_f32, out_f32);
    case 512: return regs_threads<512>(peer_f32, out_f32);
    default: return 0;
  }
}

hipError_t launch_tile_reduce(const ReduceArgs& a, int peer_f32, int out_f32, int threads,
                              bool flat, int grid, hipStream_t stream) {
  switch (threads) {
    case 128: return launch_threads<128>(a, peer_f32, out_f32, flat, grid, stream);
    case 256: return launch_threads<256>(a, peer_f32, out_f32, flat, grid, stream);
    case 512: return launch_threads<512>(a, peer_f32, out_f32, flat, grid, stream);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace entwine
