// reduce_task.h -- device code of one reduction task (wait for its flags,
// then local + peers in rank order), shared by the persistent reduction
// kernel and the fused GEMM + reduction kernel.
//
// Method: "Entwine: Coordinating Tiled Computation and Fine-Grained
// Communication across GPUs" (paperpeel.com/paper/2609.11562), Sec. 4.2
// (Consumer); the MI355X design is described in tile_reduce.hip.
#pragma once

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

// Data that another workgroup of this device stored during the call and
// released through a tile flag (the own partial, and the outgoing partials of
// a send task) is read with device-coherent loads (cache policy SC1): no stale
// L1 or L2 line can satisfy them, so the flag wait needs no acquire, which on
// this GPU invalidates the XCD's whole L2 -- under a GEMM that is still
// reading its operands from it.  The descriptor's base is the task's first
// element (wave-uniform); offsets stay within the task's rows.
constexpr int kSC1 = 16;
__device__ __forceinline__ __amdgpu_buffer_rsrc_t coherent_rsrc(const void* base) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, 0x7fffffff,
                                           0x00020000);
}
__device__ __forceinline__ u32x4 load_coherent16(__amdgpu_buffer_rsrc_t r, int byte_off) {
  return __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(r, byte_off, 0, kSC1));
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

// U chunks of one thread: their element offsets, which of them lie inside
// the slab, and the inputs that were ready before the call (the peers'
// contributions and the residual), loaded before the own partial.
template <int U, bool PEER_F32, bool OUT_F32>
struct Chunks {
  int64_t e[U];
  bool ok[U];
  Raw8<PEER_F32> pv[U][kMaxRanks];
  Raw8<OUT_F32> res[U];
};

// Issue the loads of the peers and the residual (all U chunks, nothing waits).
template <int U, bool PEER_F32, bool OUT_F32>
__device__ __forceinline__ void load_inputs(const ReduceArgs& a, Chunks<U, PEER_F32, OUT_F32>& c) {
  const bool with_res = a.residual != nullptr;  // uniform
#pragma unroll
  for (int u = 0; u < U; ++u) {
    if (!c.ok[u]) continue;
#pragma unroll
    for (int q = 0; q < kMaxRanks; ++q)
      if (q < a.P && q != a.rank) c.pv[u][q] = load_raw8<PEER_F32>(a.peers[q], c.e[u]);
    if (with_res) c.res[u] = load_raw8<OUT_F32>(a.residual, c.e[u]);
  }
}

// The own partial of U chunks.  COH: device-coherent loads relative to
// element e0 (wave-uniform).
template <int U, bool PEER_F32, bool OUT_F32, bool COH>
__device__ __forceinline__ void load_own(const ReduceArgs& a, const Chunks<U, PEER_F32, OUT_F32>& c,
                                         int64_t e0, Raw8<true> (&own)[U]) {
  const __amdgpu_buffer_rsrc_t own_r = coherent_rsrc(a.own + e0);
#pragma unroll
  for (int u = 0; u < U; ++u) {
    if (!c.ok[u]) continue;
    if constexpr (COH) {
      const int off = (int)((c.e[u] - e0) * 4);
      own[u].a = __builtin_bit_cast(f32x4, load_coherent16(own_r, off));
      own[u].b = __builtin_bit_cast(f32x4, load_coherent16(own_r, off + 16));
    } else {
      own[u] = load_raw8<true>(a.own, c.e[u]);
    }
  }
}

// The fixed-order fp32 sums (own, peers ascending, then the residual if
// any), one rounding, the stores.
template <int U, bool PEER_F32, bool OUT_F32>
__device__ __forceinline__ void sum_store(const ReduceArgs& a, const Chunks<U, PEER_F32, OUT_F32>& c,
                                          const Raw8<true> (&own)[U]) {
  const bool with_res = a.residual != nullptr;  // uniform
#pragma unroll
  for (int u = 0; u < U; ++u) {
    if (!c.ok[u]) continue;
    F8 acc = widen(own[u]);
#pragma unroll
    for (int q = 0; q < kMaxRanks; ++q)
      if (q < a.P && q != a.rank) add8(acc, c.pv[u][q]);
    if (with_res) add8(acc, c.res[u]);
    store8<OUT_F32>(a.out, c.e[u], acc);
  }
}

template <int U, bool PEER_F32, bool OUT_F32, bool COH>
__device__ __forceinline__ void finish(const ReduceArgs& a, Chunks<U, PEER_F32, OUT_F32>& c,
                                       int64_t e0) {
  Raw8<true> own[U];
  load_own<U, PEER_F32, OUT_F32, COH>(a, c, e0, own);
  sum_store(a, c, own);
}

// Wave 0 waits until every flag that tile t of partition d depends on equals
// `epoch`.  For the own partition lane k (< P + 1) watches wait slot k; a
// send task (d != rank) waits for the tile's own flag only.  Returns false (uniform across the
// wave) if the watchdog expired, or if the sticky error word is set: once one
// workgroup has timed out, the others stop waiting too, so a failed call ends
// within one timeout whatever its task count.
__device__ __forceinline__ const uint32_t* wait_flag(const ReduceArgs& a, int d, int t, int lane) {
  int32_t idx = -1;
  if (d != a.rank) {
    idx = lane == 0 ? d * a.Q + t : -1;  // a send task: the tile's own flag
  } else {
    if (lane < a.wait_slots) idx = a.waits[t * a.wait_slots + lane];
    if (t == a.withhold_tile && lane == a.rank) idx = a.never_flag;
  }
  return idx >= 0 ? a.flags + idx : nullptr;
}

// Wave 0 waits until the flag each lane watches (f; nullptr: none) equals
// `epoch`.  The flag and the sticky error word are loaded together, so one
// poll costs one memory round trip.  The pause between polls doubles from
// 128 cycles up to a.nap_max x 128: workgroups that wait long (a tile the
// GEMM produces late) then poll rarely, which keeps their device-coherent
// loads out of the way of the GEMM sharing the memory system.
__device__ bool wait_flags(const ReduceArgs& a, uint32_t epoch, const uint32_t* f, int lane) {
  const uint64_t start = wall_clock64();
  int nap = 1;
  while (true) {
    const uint32_t v = f ? __hip_atomic_load(f, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) : epoch;
    const int32_t err = __hip_atomic_load(a.error, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    if (__all(v == epoch)) break;
    if (__builtin_amdgcn_readfirstlane(err) != 0) return false;
    if (wall_clock64() - start > a.timeout_ticks) {
      if (lane == 0)
        __hip_atomic_store(a.error, (int32_t)5 /* ENTWINE_ERR_TIMEOUT */, __ATOMIC_RELAXED,
                           __HIP_MEMORY_SCOPE_AGENT);
      return false;
    }
    for (int i = 0; i < nap; ++i) __builtin_amdgcn_s_sleep(2);
    nap = min(2 * nap, a.nap_max);
  }
  // No acquire: the tile's data is read with device-coherent loads, issued
  // after this wait (program order, then the workgroup barrier that follows).
  return true;
}

__device__ __forceinline__ bool wait_tile(const ReduceArgs& a, uint32_t epoch, int d, int t,
                                          int lane) {
  return wait_flags(a, epoch, wait_flag(a, d, t, lane), lane);
}

constexpr int kUnroll = 2;

// Row slab `slab` of own tile t: 8-element chunks numbered row-major, chunk c
// at row c / cpr, columns 8 (c % cpr) onward; masked past the partition's
// last row and past N.
struct Slab {
  int64_t e0;    // element offset of the slab's first element
  int cpr;       // chunks per tile row
  int cols;      // valid columns of the tile
  int n_chunks;  // chunks in the slab's valid rows
  int N;
};
__device__ __forceinline__ Slab slab_of(const ReduceArgs& a, int t, int slab) {
  const int slab_rows = a.tm / a.slabs;
  const int row0 = a.tiles[2 * t] * a.tm + slab * slab_rows;
  const int col0 = a.tiles[2 * t + 1] * a.tn;
  const int rows = min(slab_rows, a.R - row0);
  Slab s;
  s.e0 = (int64_t)row0 * a.N + col0;
  s.cpr = a.tn >> 3;
  s.cols = min(a.tn, a.N - col0);
  s.n_chunks = rows > 0 ? rows * s.cpr : 0;
  s.N = a.N;
  return s;
}

// Chunks c0, c0 + STEP, ..., c0 + (U - 1) STEP of slab s.
template <int U, int STEP, bool PEER_F32, bool OUT_F32>
__device__ __forceinline__ void place(const Slab& s, int c0, Chunks<U, PEER_F32, OUT_F32>& c) {
#pragma unroll
  for (int u = 0; u < U; ++u) {
    const int k = c0 + u * STEP;
    const int r = k / s.cpr;
    const int col = (k - r * s.cpr) << 3;
    c.ok[u] = k < s.n_chunks && col < s.cols;
    c.e[u] = s.e0 + (int64_t)r * s.N + col;
  }
}

// Reduce row slab `slab` of task tile t: thread tid of THREADS takes chunks
// tid, tid + THREADS, ... of the slab, U at a time.
template <int THREADS, int U, bool PEER_F32, bool OUT_F32>
__device__ __forceinline__ void reduce_slab(const ReduceArgs& a, const Slab& s, int tid,
                                            int first = 0) {
  for (int c0 = tid + first; c0 < s.n_chunks; c0 += U * THREADS) {
    Chunks<U, PEER_F32, OUT_F32> c;
    place<U, THREADS>(s, c0, c);
    load_inputs(a, c);
    finish<U, PEER_F32, OUT_F32, true>(a, c, s.e0);
  }
}

// Slab-relative form (the fused kernel's tasks).  Every operand of a slab is
// reached through a wave-uniform buffer descriptor based at the slab's first
// element, so a chunk needs one 32-bit element offset rather than a 64-bit
// address per operand, and the peers are numbered compactly (ranks ascending,
// the own rank skipped), so no register holds the unused slot.  Same loads,
// same order of the sums, same rounding as above.
constexpr int kNT = 2;  // buffer cache policy NT: streaming

struct SlabIO {
  __amdgpu_buffer_rsrc_t peer[kMaxRanks - 1];  // j -> rank j + (j >= rank)
  __amdgpu_buffer_rsrc_t own, res, out;
};

__device__ __forceinline__ __amdgpu_buffer_rsrc_t rel_rsrc(const void* base) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, 0x7fffffff,
                                           0x00020000);
}

template <bool PEER_F32, bool OUT_F32>
__device__ __forceinline__ SlabIO slab_io(const ReduceArgs& a, int64_t e0) {
  constexpr int ps = PEER_F32 ? 4 : 2, os = OUT_F32 ? 4 : 2;
  SlabIO io;
#pragma unroll
  for (int j = 0; j < kMaxRanks - 1; ++j) {
    const int q = j + (j >= a.rank ? 1 : 0);
    io.peer[j] = rel_rsrc(j < a.P - 1 ? static_cast<const char*>(a.peers[q]) + e0 * ps : nullptr);
  }
  io.own = rel_rsrc(a.own + e0);
  io.res = rel_rsrc(a.residual ? static_cast<const char*>(a.residual) + e0 * os : nullptr);
  io.out = rel_rsrc(static_cast<char*>(a.out) + e0 * os);
  return io;
}

template <bool F32, int AUX>
__device__ __forceinline__ Raw8<F32> load_rel(__amdgpu_buffer_rsrc_t r, int off) {
  if constexpr (F32) {
    return Raw8<true>{
        __builtin_bit_cast(f32x4, __builtin_amdgcn_raw_buffer_load_b128(r, off * 4, 0, AUX)),
        __builtin_bit_cast(f32x4, __builtin_amdgcn_raw_buffer_load_b128(r, off * 4 + 16, 0, AUX))};
  } else {
    return Raw8<false>{
        __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(r, off * 2, 0, AUX))};
  }
}

template <int U, bool PEER_F32, bool OUT_F32>
struct RelChunks {
  int off[U];  // element offset from the slab's first element
  bool ok[U];
  Raw8<PEER_F32> pv[U][kMaxRanks - 1];
  Raw8<OUT_F32> res[U];
};

// Chunks c0, c0 + STEP, ..., c0 + (U - 1) STEP of slab s.
template <int U, int STEP, bool PEER_F32, bool OUT_F32>
__device__ __forceinline__ void place_rel(const Slab& s, int c0,
                                          RelChunks<U, PEER_F32, OUT_F32>& c) {
#pragma unroll
  for (int u = 0; u < U; ++u) {
    const int k = c0 + u * STEP;
    const int r = k / s.cpr;
    const int col = (k - r * s.cpr) << 3;
    c.ok[u] = k < s.n_chunks && col < s.cols;
    c.off[u] = r * s.N + col;
  }
}

// The peers' and the residual's loads (complete before the call).
template <int U, bool PEER_F32, bool OUT_F32>
__device__ __forceinline__ void load_inputs_rel(const ReduceArgs& a, const SlabIO& io,
                                                RelChunks<U, PEER_F32, OUT_F32>& c) {
  const bool with_res = a.residual != nullptr;  // uniform
#pragma unroll
  for (int u = 0; u < U; ++u) {
    if (!c.ok[u]) continue;
#pragma unroll
    for (int j = 0; j < kMaxRanks - 1; ++j)
      if (j < a.P - 1) c.pv[u][j] = load_rel<PEER_F32, kNT>(io.peer[j], c.off[u]);
    if (with_res) c.res[u] = load_rel<OUT_F32, kNT>(io.res, c.off[u]);
  }
}

// The own partial, device-coherent.
template <int U, bool PEER_F32, bool OUT_F32>
__device__ __forceinline__ void load_own_rel(const SlabIO& io,
                                             const RelChunks<U, PEER_F32, OUT_F32>& c,
                                             Raw8<true> (&own)[U]) {
#pragma unroll
  for (int u = 0; u < U; ++u)
    if (c.ok[u]) own[u] = load_rel<true, kSC1>(io.own, c.off[u]);
}

// own + peers (ranks ascending) + residual in fp32, one rounding, the store
// (cache policy OUT_AUX: kSC1 makes an acknowledged store visible device-wide).
template <int U, bool PEER_F32, bool OUT_F32, int OUT_AUX = 0>
__device__ __forceinline__ void sum_store_rel(const ReduceArgs& a, const SlabIO& io,
                                              const RelChunks<U, PEER_F32, OUT_F32>& c,
                                              const Raw8<true> (&own)[U]) {
  const bool with_res = a.residual != nullptr;  // uniform
#pragma unroll
  for (int u = 0; u < U; ++u) {
    if (!c.ok[u]) continue;
    F8 acc = widen(own[u]);
#pragma unroll
    for (int j = 0; j < kMaxRanks - 1; ++j)
      if (j < a.P - 1) add8(acc, c.pv[u][j]);
    if (with_res) add8(acc, c.res[u]);
    if constexpr (OUT_F32) {
      f32x4 lo, hi;
      lo[0] = acc.v[0]; lo[1] = acc.v[1]; lo[2] = acc.v[2]; lo[3] = acc.v[3];
      hi[0] = acc.v[4]; hi[1] = acc.v[5]; hi[2] = acc.v[6]; hi[3] = acc.v[7];
      __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, lo), io.out, c.off[u] * 4, 0,
                                             OUT_AUX);
      __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, hi), io.out,
                                             c.off[u] * 4 + 16, 0, OUT_AUX);
    } else {
      u32x4 o;
      o[0] = pack_bf16x2(acc.v[0], acc.v[1]);
      o[1] = pack_bf16x2(acc.v[2], acc.v[3]);
      o[2] = pack_bf16x2(acc.v[4], acc.v[5]);
      o[3] = pack_bf16x2(acc.v[6], acc.v[7]);
      __builtin_amdgcn_raw_buffer_store_b128(o, io.out, c.off[u] * 2, 0, OUT_AUX);
    }
  }
}

// The assisted schedule (kernels.h, kAssistCall).  The (sequence number,
// epoch) word of the call whose fused kernel runs.
__device__ __forceinline__ uint64_t assist_word(const uint32_t* ctl) {
  return __hip_atomic_load(reinterpret_cast<const uint64_t*>(ctl + kAssistCall), __ATOMIC_RELAXED,
                           __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ uint64_t assist_pack(uint32_t seq, uint32_t epoch) {
  return (uint64_t)seq | ((uint64_t)epoch << 32);
}

// Sequence numbers of assisted calls compare within half the 32-bit range
// (the host clears the claim words before a call's number would leave it).
__device__ __forceinline__ bool seq_newer(uint32_t a, uint32_t b) { return (int32_t)(a - b) > 0; }

// Claims task j for the assisted call `seq`: true if this caller moved the
// task's claim word from an older call's number to seq; false if the word
// already holds seq (someone of this call has the task) or a later call's
// number (this call is over).
__device__ __forceinline__ bool claim_task(uint32_t* claims, int j, uint32_t seq) {
  uint32_t old = __hip_atomic_load(claims + j, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  while (seq_newer(seq, old)) {
    if (__hip_atomic_compare_exchange_strong(claims + j, &old, seq, __ATOMIC_RELAXED,
                                             __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT))
      return true;
  }
  return false;
}

// Global task id -> (partition, tile, slab).
struct TaskRef {
  int d, t, slab;
};
__device__ __forceinline__ TaskRef task_ref(const ReduceArgs& a, int j) {
  const int g = a.task_list ? a.task_list[j] : a.rank * a.Q * a.slabs + j;
  const int dt = g / a.slabs;
  const int d = dt / a.Q;
  return TaskRef{d, dt - d * a.Q, g - dt * a.slabs};
}

// Push row slab `slab` of partition d's tile t from the outgoing partials to
// the staging buffer (the stand-in for the transfer to peer d): 16-byte
// chunks, thread tid of THREADS takes chunks tid, tid + THREADS, ...
template <int THREADS, bool PEER_F32>
__device__ __forceinline__ void push_slab(const ReduceArgs& a, int d, int t, int slab, int tid) {
  constexpr int kPerChunk = PEER_F32 ? 4 : 8;  // elements per 16 bytes
  const int chunks_per_row = a.tn / kPerChunk;
  const int slab_rows = a.tm / a.slabs;
  const int row0 = a.tiles[2 * t] * a.tm + slab * slab_rows;
  const int col0 = a.tiles[2 * t + 1] * a.tn;
  const int rows = min(slab_rows, a.R - row0);
  const int cols = min(a.tn, a.N - col0);
  const int n_chunks = rows > 0 ? rows * chunks_per_row : 0;
  constexpr int kSize = PEER_F32 ? 4 : 2;
  const int64_t base = (((int64_t)d * a.R + row0) * a.N + col0) * kSize;
  const __amdgpu_buffer_rsrc_t src = coherent_rsrc(static_cast<const char*>(a.outgoing) + base);
  char* const dst = static_cast<char*>(a.staging) + base;
  for (int c = tid; c < n_chunks; c += THREADS) {
    const int r = c / chunks_per_row;
    const int col = (c - r * chunks_per_row) * kPerChunk;
    if (col >= cols) continue;
    const int off = (r * a.N + col) * kSize;  // within the slab's rows
    __builtin_nontemporal_store(load_coherent16(src, off), reinterpret_cast<u32x4*>(dst + off));
  }
}

}  // namespace
}  // namespace entwine
