// tile_reduce.hip -- the consumer: a persistent tile-reduction kernel.
//
// Method: "Entwine: Coordinating Tiled Computation and Fine-Grained
// Communication across GPUs" (paperpeel.com/paper/2609.11562).
//  * Sec. 3.1 "Matching task order": consumer workgroup j takes tasks j, j+x,
//    j+2x, ... in production order and waits for each tile before reducing it.
//  * Sec. 3.2 "Communication budget": x = the grid size, fixed for the call.
//  * Sec. 4.2: before a tile is read, thread 0 acquires its flags (the local
//    one and the peers') and the workgroup then synchronizes; each thread
//    reduces a disjoint part of the tile, starting from the local
//    contribution and adding the peers in rank order; each output element
//    has exactly one writer.  Here the acquire is replaced by
//    device-coherent loads of the released data (below).
//
// MI355X mapping.
//  * A task is one row slab of a reduction tile (slabs = 1: the whole tile),
//    numbered tile-major, so the tiles' slabs spread over consecutive
//    workgroups.
//  * Wave 0 polls the task's flags in parallel, one lane per flag, with
//    relaxed agent-scope loads and an s_sleep back-off; the other waves wait
//    at the workgroup barrier meanwhile.  The polls are relaxed; in place of
//    an acquire fence (which on this GPU invalidates the XCD's whole L2, where
//    a GEMM sharing the XCD still reads its operands), the released data is
//    read with device-coherent (SC1) loads.  Every producer wave's SC1 stores
//    were acknowledged before the workgroup barrier that precedes the flag
//    store (gemm_block.h), and these loads are issued only after the wait
//    (the loop's exit depends on the flag value, then the barrier) and
//    cannot hit a stale cache line, so they return the stored data.
//  * The element loop moves 8 elements per thread step: two 16-byte fp32 loads
//    of the local partial and one 16-byte load per bf16 peer.  Two steps are
//    loaded before any add so that 2 * (P + 1) loads per thread are in flight.
//    fp32 adds run in rank order; one round-to-nearest-even conversion and one
//    16-byte store per step.
//  * Without waits (the sequential schedule, after the GEMM kernel has
//    finished) the kernel streams the partition as one flat array with a
//    grid-stride loop.
#include "reduce_task.h"

namespace entwine {
namespace {

template <int THREADS, bool PEER_F32, bool OUT_F32>
__global__ __launch_bounds__(THREADS) void tile_reduce_kernel(ReduceArgs a) {
  __shared__ int s_abort[2];
  const int tid = threadIdx.x;
  const uint32_t epoch = __hip_atomic_load(a.ctl + kEpoch, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  int parity = 0;
  if (a.trace && tid == 0) trace_at(a.trace, blockIdx.x);
  for (int task = blockIdx.x; task < a.ntasks; task += gridDim.x, parity ^= 1) {
    const TaskRef k = task_ref(a, task);
    if (tid < 64) {
      const bool ok = a.nowait || wait_tile(a, epoch, k.d, k.t, tid);
      if (tid == 0) s_abort[parity] = ok ? 0 : 1;
    }
    // The flag wait is ordered before every wave's reads of the tile.  The
    // abort word alternates between two slots, so wave 0 can write the next
    // task's word while a slower wave still reads this one.
    __syncthreads();
    if (s_abort[parity]) break;  // uniform: every thread read the same value

    if (k.d == a.rank)
      reduce_slab<THREADS, kUnroll, PEER_F32, OUT_F32>(a, slab_of(a, k.t, k.slab), tid);
    else
      push_slab<THREADS, PEER_F32>(a, k.d, k.t, k.slab, tid);
  }
  if (a.trace) {  // uniform: every wave's stores issued
    __syncthreads();
    if (tid == 0) trace_at(a.trace, (int64_t)gridDim.x + blockIdx.x);
  }
  // Every workgroup, finished or timed out, checks out.
  if (tid == 0 && !a.nowait) check_out(a.ctl, epoch, (uint32_t)a.checkout_total);
}

// Wave 0 of an assisted helper, for task j whose flags lane `lane` watches
// (f; nullptr: none): 1 if the task is or becomes claimed by someone else of
// this call, 2 once its flags are set and this workgroup has claimed it, 0 to
// leave (the call is over -- its liveness word has changed or a later call
// holds the task --, the sticky error is set, or the watchdog expired; a
// helper never raises the error itself: the fused kernel does what is left).
// A helper that outlives its call cannot take a task of a later one: the
// claim moves a word only from an older call's number (claim_task), so flags
// that still hold this call's epoch do not matter.  Uniform across the wave.
__device__ uint32_t assist_take(const ReduceArgs& a, uint32_t epoch, uint64_t live, int j,
                                const uint32_t* f, int lane) {
  // 1: claimed in this call; 0: a later call has claimed it; 2: free.
  auto state = [&]() -> uint32_t {
    const uint32_t c = __builtin_amdgcn_readfirstlane(
        __hip_atomic_load(a.claims + j, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT));
    return c == a.assist_seq ? 1u : seq_newer(c, a.assist_seq) ? 0u : 2u;
  };
  uint32_t st = state();
  if (st != 2) return st;
  const uint64_t start = wall_clock64();
  int nap = 1;
  while (true) {
    const uint32_t v = f ? __hip_atomic_load(f, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) : epoch;
    if (__all(v == epoch)) break;
    if (__builtin_amdgcn_readfirstlane(
            __hip_atomic_load(a.error, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT)) != 0)
      return 0;
    if (assist_word(a.ctl) != live || wall_clock64() - start > a.timeout_ticks) return 0;
    if ((st = state()) != 2) return st;
    for (int i = 0; i < nap; ++i) __builtin_amdgcn_s_sleep(2);
    nap = min(2 * nap, a.nap_max);
  }
  uint32_t won = 0;
  if (lane == 0) won = claim_task(a.claims, j, a.assist_seq) ? 2u : 1u;
  return __builtin_amdgcn_readfirstlane(won);
}

// The assisted schedule's helpers (kernels.h, kAssistCall).  They run on the
// internal stream with no event after the fused kernel of their call, so they
// may start before it, beside it or after it has finished.  A helper first
// waits (bounded) until the call's (sequence number, epoch) word shows the
// fused kernel running, and leaves at once if the call is over or a later
// call runs.  Then it walks tasks j, j + grid, ... of the production-ordered
// list: it skips claimed tasks, waits for a task's flags while the call
// lasts, claims it, reduces it (the fused kernel's slab code, with
// device-coherent output stores), and once every wave's stores are
// acknowledged counts it done; the fused kernel's last workgroup waits for
// that count, so the call's output is complete when the fused kernel ends.
template <int THREADS, bool PEER_F32, bool OUT_F32>
__global__ __launch_bounds__(THREADS) void assist_reduce_kernel(ReduceArgs a) {
  constexpr int kU = 2;  // chunks per thread per pass
  __shared__ uint32_t s_word[2];
  const int tid = threadIdx.x;
  int parity = 0;
  // Thread 0's v, for every thread, as a wave-uniform value.
  auto share = [&](uint32_t v) {
    if (tid == 0) s_word[parity] = v;
    __syncthreads();
    const uint32_t out = __builtin_amdgcn_readfirstlane(s_word[parity]);
    parity ^= 1;
    return out;
  };
  uint32_t epoch = 0;
  if (tid == 0) {
    const uint64_t start = wall_clock64();
    int nap = 1;
    while (true) {
      const uint64_t w = assist_word(a.ctl);
      const uint32_t seq = (uint32_t)w;
      if (seq == a.assist_seq) {
        epoch = (uint32_t)(w >> 32);  // 0: the call is over
        break;
      }
      if ((int32_t)(seq - a.assist_seq) > 0 || wall_clock64() - start > a.timeout_ticks) break;
      for (int i = 0; i < nap; ++i) __builtin_amdgcn_s_sleep(2);
      nap = min(2 * nap, a.nap_max);
    }
  }
  epoch = share(epoch);
  if (epoch == 0) return;  // uniform
  const uint64_t live = assist_pack(a.assist_seq, epoch);
  const int trace_g = a.trace_g ? a.trace_g : (int)gridDim.x;
  if (a.trace && tid == 0) trace_at(a.trace, a.trace_slot0 + blockIdx.x);
  for (int j = blockIdx.x; j < a.ntasks; j += gridDim.x) {
    const TaskRef k = task_ref(a, j);
    if (k.d != a.rank) continue;  // send tasks are not built here (the host refuses them)
    uint32_t go = 0;
    if (tid < 64) go = assist_take(a, epoch, live, j, wait_flag(a, k.d, k.t, tid), tid);
    // The flag wait and the claim are ordered before every wave's reads.
    go = share(go);
    if (go == 0) break;  // uniform
    if (go == 1) continue;
    const Slab sl = slab_of(a, k.t, k.slab);
    const SlabIO io = slab_io<PEER_F32, OUT_F32>(a, sl.e0);
    for (int c0 = tid; c0 < sl.n_chunks; c0 += kU * THREADS) {
      RelChunks<kU, PEER_F32, OUT_F32> c;
      place_rel<kU, THREADS>(sl, c0, c);
      load_inputs_rel(a, io, c);
      Raw8<true> own[kU];
      load_own_rel(io, c, own);
      sum_store_rel<kU, PEER_F32, OUT_F32, kSC1>(a, io, c, own);
    }
    // Every wave's stores acknowledged (device-coherent: visible to any XCD),
    // then the count.
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();
    if (tid == 0)
      __hip_atomic_fetch_add(a.ctl + kTasksDone, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
  if (a.trace) {  // uniform: every wave's stores issued
    __syncthreads();
    if (tid == 0) trace_at(a.trace, (int64_t)trace_g + a.trace_slot0 + blockIdx.x);
  }
}

// The sequential schedule's reduction: no flags; the partition is one flat
// array of R * N / 8 chunks walked with a grid-stride loop.
template <int THREADS, bool PEER_F32, bool OUT_F32>
__global__ __launch_bounds__(THREADS) void flat_reduce_kernel(ReduceArgs a) {
  if (a.trace && threadIdx.x == 0) trace_at(a.trace, blockIdx.x);
  const int64_t n_chunks = (int64_t)a.R * a.N / 8;
  const int64_t stride = (int64_t)gridDim.x * THREADS * kUnroll;
  for (int64_t c0 = (int64_t)blockIdx.x * THREADS * kUnroll + threadIdx.x; c0 < n_chunks;
       c0 += stride) {
    Chunks<kUnroll, PEER_F32, OUT_F32> c;
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
      const int64_t k = c0 + u * THREADS;
      c.ok[u] = k < n_chunks;
      c.e[u] = k * 8;
    }
    load_inputs(a, c);
    finish<kUnroll, PEER_F32, OUT_F32, false>(a, c, 0);
  }
  if (a.trace) {  // uniform: every wave's stores issued
    __syncthreads();
    if (threadIdx.x == 0) trace_at(a.trace, (int64_t)gridDim.x + blockIdx.x);
  }
}

// lds: dynamic LDS each tile-reduction workgroup reserves and never touches
// (0 unless the reduction is confined to CUs of its own).
template <int THREADS, bool PEER_F32, bool OUT_F32>
hipError_t launch_typed(const ReduceArgs& a, bool flat, int grid, int lds, hipStream_t s) {
  if (flat) {
    flat_reduce_kernel<THREADS, PEER_F32, OUT_F32><<<grid, THREADS, 0, s>>>(a);
    return hipGetLastError();
  }
  static int attr_bytes = 0;
  if (lds > attr_bytes) {
    hipError_t e = hipFuncSetAttribute((const void*)tile_reduce_kernel<THREADS, PEER_F32, OUT_F32>,
                                       hipFuncAttributeMaxDynamicSharedMemorySize, lds);
    if (e != hipSuccess) return e;
    attr_bytes = lds;
  }
  tile_reduce_kernel<THREADS, PEER_F32, OUT_F32><<<grid, THREADS, lds, s>>>(a);
  return hipGetLastError();
}

template <int THREADS>
hipError_t launch_threads(const ReduceArgs& a, int peer_f32, int out_f32, bool flat, int grid,
                          int lds, hipStream_t s) {
  if (!peer_f32 && !out_f32) return launch_typed<THREADS, false, false>(a, flat, grid, lds, s);
  if (!peer_f32 && out_f32) return launch_typed<THREADS, false, true>(a, flat, grid, lds, s);
  if (peer_f32 && !out_f32) return launch_typed<THREADS, true, false>(a, flat, grid, lds, s);
  return launch_typed<THREADS, true, true>(a, flat, grid, lds, s);
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

template <int THREADS, bool PEER_F32, bool OUT_F32>
int assist_regs_typed() {
  hipFuncAttributes at{};
  if (hipFuncGetAttributes(&at, (const void*)assist_reduce_kernel<THREADS, PEER_F32, OUT_F32>) !=
      hipSuccess)
    return 0;
  return at.numRegs;
}

template <int THREADS>
hipError_t assist_launch_threads(const ReduceArgs& a, int peer_f32, int out_f32, int grid,
                                 hipStream_t s) {
  if (!peer_f32 && !out_f32)
    assist_reduce_kernel<THREADS, false, false><<<grid, THREADS, 0, s>>>(a);
  else if (!peer_f32 && out_f32)
    assist_reduce_kernel<THREADS, false, true><<<grid, THREADS, 0, s>>>(a);
  else if (peer_f32 && !out_f32)
    assist_reduce_kernel<THREADS, true, false><<<grid, THREADS, 0, s>>>(a);
  else
    assist_reduce_kernel<THREADS, true, true><<<grid, THREADS, 0, s>>>(a);
  return hipGetLastError();
}

template <int THREADS>
int assist_regs_threads(int peer_f32, int out_f32) {
  if (!peer_f32 && !out_f32) return assist_regs_typed<THREADS, false, false>();
  if (!peer_f32 && out_f32) return assist_regs_typed<THREADS, false, true>();
  if (peer_f32 && !out_f32) return assist_regs_typed<THREADS, true, false>();
  return assist_regs_typed<THREADS, true, true>();
}

}  // namespace

hipError_t launch_assist_reduce(const ReduceArgs& a, int peer_f32, int out_f32, int threads,
                                int grid, hipStream_t stream) {
  switch (threads) {
    case 128: return assist_launch_threads<128>(a, peer_f32, out_f32, grid, stream);
    case 256: return assist_launch_threads<256>(a, peer_f32, out_f32, grid, stream);
    case 512: return assist_launch_threads<512>(a, peer_f32, out_f32, grid, stream);
    default: return hipErrorInvalidValue;
  }
}

int assist_registers(int threads, int peer_f32, int out_f32) {
  switch (threads) {
    case 128: return assist_regs_threads<128>(peer_f32, out_f32);
    case 256: return assist_regs_threads<256>(peer_f32, out_f32);
    case 512: return assist_regs_threads<512>(peer_f32, out_f32);
    default: return 0;
  }
}

int reduce_registers(int threads, int peer_f32, int out_f32) {
  switch (threads) {
    case 128: return regs_threads<128>(peer_f32, out_f32);
    case 256: return regs_threads<256>(peer_f32, out_f32);
    case 512: return regs_threads<512>(peer_f32, out_f32);
    default: return 0;
  }
}

// The trace slots' reset before a traced call: a kernel rather than a
// memset, so that a captured graph resets them on every replay.
__global__ void trace_reset_kernel(uint64_t* t, int64_t words) {
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < words;
       i += (int64_t)gridDim.x * blockDim.x)
    t[i] = 0;
}

hipError_t launch_trace_reset(uint64_t* trace, int64_t words, hipStream_t stream) {
  int64_t blocks = (words + 255) / 256;
  if (blocks > 256) blocks = 256;
  if (blocks < 1) blocks = 1;
  trace_reset_kernel<<<(int)blocks, 256, 0, stream>>>(trace, words);
  return hipGetLastError();
}

hipError_t launch_tile_reduce(const ReduceArgs& a, int peer_f32, int out_f32, int threads,
                              bool flat, int grid, hipStream_t stream, int lds_bytes) {
  switch (threads) {
    case 128: return launch_threads<128>(a, peer_f32, out_f32, flat, grid, lds_bytes, stream);
    case 256: return launch_threads<256>(a, peer_f32, out_f32, flat, grid, lds_bytes, stream);
    case 512: return launch_threads<512>(a, peer_f32, out_f32, flat, grid, lds_bytes, stream);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace entwine
