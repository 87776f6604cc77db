// api_internal.h -- host entry points shared between the library's source
// files (not part of the C ABI).
#pragma once

#include <hip/hip_runtime.h>

#include <cstddef>
#include <cstdint>

#include "entwine.h"

namespace entwine {

// Layout of the fixed part of the no-alloc scratch (byte offsets from its
// start): control words, the sticky error word, and a flag region of fixed
// size that nothing else ever overlaps, so that no flag word can hold stale
// data of another buffer.
constexpr size_t kScratchCtl = 0;
constexpr size_t kScratchError = 2048;
constexpr size_t kScratchFlags = 4096;
constexpr size_t kScratchFlagWords = size_t(1) << 17;
constexpr size_t kScratchFixed = kScratchFlags + kScratchFlagWords * 4;

// Runs entwine_gemm_rs_ex's operation on `scratch` (scratch_bytes of device
// memory on the current device, set up by the caller: control words
// initialised, flag region zero) instead of the library workspace, without
// allocating device memory: the sequential schedule or the fused one, on
// `stream` only.
int run_noalloc(void* scratch, size_t scratch_bytes, const void* X, const void* W,
                const void* const* peer_partials, void* out, int64_t M, int64_t N,
                int64_t K_local, int P, int rank, int tile_order, int comm_budget,
                hipStream_t stream, const entwine_config* cfg);

// The no-alloc scratch of `device`, or nullptr if no call has set it up.
void* noalloc_scratch(int device);

// Records `message` as the calling thread's entwine_last_error_message and
// returns `status`.
int report(int status, const char* message);

}  // namespace entwine
