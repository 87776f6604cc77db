// noalloc.hip -- entwine_gemm_rs_noalloc: the operation of entwine_gemm_rs_ex
// for callers that cannot allocate device memory (code under HIP graph
// capture, tight serving loops, harnesses that forbid hipMalloc).
//
// Its buffers -- control words, tile flags, the schedule tables, the fp32
// own-partition partial, the outgoing partials and (with push_outgoing) the
// staging copies -- live in one file-scope device array, `scratch`, of
// kScratchBytes.  Every GPU the library runs on holds its own copy of the
// array until the process ends.  In host code the array's name is only a
// host-side stand-in, so the device address of each GPU's copy is taken once,
// with that GPU current, by hipGetSymbolAddress, and only that address is
// ever handed to kernels or copies.
#include <hip/hip_runtime.h>

#include <mutex>

#include "api_internal.h"
#include "kernels.h"

namespace entwine {
namespace {

// 256 MiB: holds the partials of a 16384 x 5120 output (fp32 own partition of
// 4096 rows and bf16 outgoing rows, 240 MiB) with its tables and flags.
constexpr size_t kScratchBytes = size_t(256) << 20;

static __device__ __align__(256) unsigned char scratch[kScratchBytes];

constexpr int kMaxDevices = 64;
void* g_ptr[kMaxDevices];  // device address of each GPU's copy (nullptr: not set up)
std::mutex g_setup_mu;

// The control words' initial state: epoch 1 (flags never written hold 0),
// every counter and ticket 0, no sticky error.  Run once per device, on the
// stream of that device's first call, before its kernels.
__global__ void init_scratch_kernel(uint32_t* ctl, int32_t* error) {
  for (int i = threadIdx.x; i < kCtlWords; i += blockDim.x) ctl[i] = i == kEpoch ? 1u : 0u;
  if (threadIdx.x == 0) *error = 0;
}

// Device address of the current device's scratch; the first call on a
// device takes it and initialises the control words on `stream`.
int setup(hipStream_t stream, char** out) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return report(ENTWINE_ERR_HIP, "hipGetDevice failed");
  if (dev < 0 || dev >= kMaxDevices)
    return report(ENTWINE_ERR_UNSUPPORTED, "device index beyond the no-alloc scratch table");
  std::lock_guard<std::mutex> lock(g_setup_mu);
  if (!g_ptr[dev]) {
    // The initialisation is a kernel on `stream`: captured into a graph, it
    // would reset the epoch at every replay, and flags of the previous replay
    // would read as ready.  The first call on a device must not be captured.
    hipStreamCaptureStatus cap = hipStreamCaptureStatusNone;
    if (hipStreamIsCapturing(stream, &cap) != hipSuccess)
      return report(ENTWINE_ERR_HIP, "hipStreamIsCapturing failed");
    if (cap != hipStreamCaptureStatusNone)
      return report(ENTWINE_ERR_INVALID_ARGUMENT, "the first no-alloc call on a device sets up "
                    "its scratch: make it outside a graph capture");
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p)
      return report(ENTWINE_ERR_HIP, "hipGetSymbolAddress of the no-alloc scratch failed");
    char* c = static_cast<char*>(p);
    init_scratch_kernel<<<1, 256, 0, stream>>>(reinterpret_cast<uint32_t*>(c + kScratchCtl),
                                               reinterpret_cast<int32_t*>(c + kScratchError));
    if (hipGetLastError() != hipSuccess)
      return report(ENTWINE_ERR_HIP, "the no-alloc scratch's initialisation failed to launch");
    g_ptr[dev] = p;
  }
  *out = static_cast<char*>(g_ptr[dev]);
  return ENTWINE_OK;
}

}  // namespace

void* noalloc_scratch(int device) {
  if (device < 0 || device >= kMaxDevices) return nullptr;
  std::lock_guard<std::mutex> lock(g_setup_mu);
  return g_ptr[device];
}

}  // namespace entwine

extern "C" int entwine_gemm_rs_noalloc(const void* X, const void* W,
                                       const void* const* peer_partials, void* out, int64_t M,
                                       int64_t N, int64_t K_local, int P, int rank,
                                       int tile_order, int comm_budget, void* stream,
                                       const entwine_config* cfg) {
  char* base = nullptr;
  const int rc = entwine::setup(static_cast<hipStream_t>(stream), &base);
  if (rc != ENTWINE_OK) return rc;
  return entwine::run_noalloc(base, entwine::kScratchBytes, X, W, peer_partials, out, M, N,
                              K_local, P, rank, tile_order, comm_budget,
                              static_cast<hipStream_t>(stream), cfg);
}
