// lowrank_linear_forward_noalloc: lowrank_linear_forward with its device
// scratch in a file-scope array of this library instead of a caller-provided
// workspace, for callers that cannot allocate (code under graph capture,
// serving loops, harnesses that forbid allocation).
//
// The array lives in the code object: each GPU the library runs on holds its
// own copy, zero-filled when the module loads, until the process ends.  Host
// code never uses the array's name as an address (in host code that name is a
// stand-in, not device memory); it takes each device's address once with
// hipGetSymbolAddress, the device current, and passes that address to the
// kernels exactly where a workspace pointer would go.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <mutex>

#include "lowrank.h"
#include "lr_kernels.h"

namespace {

constexpr size_t kScratchBytes = (size_t)LR_NOALLOC_SCRATCH_BYTES;
constexpr int kMaxDevices = 64;

__device__ __align__(256) uint8_t scratch[kScratchBytes];

// The decode path's control words (counters, flags, error words) must start
// at zero; they return to zero at the end of every call.
constexpr size_t kCtlBytes = lr::kCtlAreaBytes;
static_assert(kCtlBytes % 16 == 0 && kCtlBytes <= kScratchBytes, "control area");

__global__ void __launch_bounds__(256) clear_words(uint4* p, size_t n) {
  for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < n;
       i += (size_t)gridDim.x * blockDim.x)
    p[i] = make_uint4(0u, 0u, 0u, 0u);
}

std::mutex g_mu;
void* g_ptr[kMaxDevices] = {nullptr};

// Set-up, once per device with that device current: take this device's
// address of `scratch` and clear its control area with a kernel on the
// caller's stream (no memset node, so a first call under capture also works).
// Returns nullptr when either step fails; the next call then tries again.
void* scratch_ptr(hipStream_t stream) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return nullptr;
  std::lock_guard<std::mutex> lock(g_mu);
  if (!g_ptr[dev]) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return nullptr;
    hipLaunchKernelGGL(clear_words, dim3(32), dim3(256), 0, stream, static_cast<uint4*>(p),
                       kCtlBytes / 16);
    if (hipGetLastError() != hipSuccess) return nullptr;
    g_ptr[dev] = p;
  }
  return g_ptr[dev];
}

}  // namespace

extern "C" lr_status lowrank_linear_forward_noalloc(lr_dtype dt, int64_t T, int64_t d_in,
                                                    int64_t r, int64_t d_out, const void* x,
                                                    int64_t ldx, const void* Ut, int64_t ldu,
                                                    const void* Vt, int64_t ldv, void* y,
                                                    int64_t ldy, float* t_io, int64_t ldt,
                                                    unsigned flags, hipStream_t stream) {
  const size_t need = lowrank_workspace_bytes(0, dt, T, d_in, r, d_out, 0);
  if (need > kScratchBytes) return LR_ERR_CAPACITY;
  void* ws = scratch_ptr(stream);
  if (!ws) return LR_ERR_HIP;
  return lowrank_linear_forward(dt, T, d_in, r, d_out, x, ldx, Ut, ldu, Vt, ldv, y, ldy, t_io,
                                ldt, flags, ws, kScratchBytes, stream);
}
