// dg_noalloc.hip -- the library-owned split-K workspace behind dg_gemm_fp8_nt_noalloc:
// one statically sized array per GPU, for callers that cannot allocate device memory
// (code under graph capture, tight serving loops).
//
// The array is a device global, so every GPU the library runs on holds its own copy
// at its own address until the process ends.  Host code never passes the array's name
// to a kernel (on the host that name is only a stand-in, not a device address): the
// address comes from hipGetSymbolAddress, looked up once per device with that device
// current, and is cached per device.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <mutex>

#include "dg_internal.h"

namespace dg {
namespace {

// Largest split-K workspace any instance asks for: the arrival records plus two 128x128
// fp32 partial tiles for each of kStreamGrid workgroups (32 MiB + 16 KiB), rounded up.
constexpr size_t kScratchBytes = ((size_t)32 << 20) + ((size_t)64 << 10);

// Zero at load (static storage) and left zero by every call that uses it.
static __device__ __align__(256) uint8_t scratch[kScratchBytes];

constexpr int kMaxDevices = 64;
void* g_scratch_ptr[kMaxDevices];
bool g_scratch_ready[kMaxDevices];
std::mutex g_scratch_mu;

__global__ void __launch_bounds__(256) zero_words(uint4* p, size_t n) {
  for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < n;
       i += (size_t)gridDim.x * blockDim.x)
    p[i] = make_uint4(0u, 0u, 0u, 0u);
}

}  // namespace

size_t scratch_capacity() { return kScratchBytes; }

// The current device's scratch address.  On the first call for a device: look the
// address up and, unless `stream` is being captured into a graph, zero the array with a
// kernel on `stream` (no memset node, no allocation).  Returns hipSuccess or the error.
hipError_t scratch_for_current_device(void** out, hipStream_t stream) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lk(g_scratch_mu);
  if (!g_scratch_ready[dev]) {
    void* ptr = nullptr;
    e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    if (!ptr) return hipErrorInvalidSymbol;
    hipStreamCaptureStatus cs = hipStreamCaptureStatusNone;
    e = hipStreamIsCapturing(stream, &cs);
    if (e != hipSuccess) return e;
    if (cs == hipStreamCaptureStatusNone) {
      hipLaunchKernelGGL(zero_words, dim3(512), dim3(256), 0, stream, (uint4*)ptr,
                         kScratchBytes / sizeof(uint4));
      e = hipGetLastError();
      if (e != hipSuccess) return e;
    }
    g_scratch_ptr[dev] = ptr;
    g_scratch_ready[dev] = true;
  }
  *out = g_scratch_ptr[dev];
  return hipSuccess;
}

}  // namespace dg
