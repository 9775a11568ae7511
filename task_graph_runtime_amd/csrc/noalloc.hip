// The static scratch area of the no-allocation decode step
// (mpk_decode_step_noalloc in include/mpk.h), for callers that cannot
// allocate device memory.  A file-scope device array holds the step's
// per-call mutable state -- event counters and sub-counters, scheduler and
// JIT rings with their state words, attention split arrivals, and the fp32
// activations -- so the step makes no hipMalloc.  Each device the library
// runs on holds its own copy of the array (kScratchBytes) until the process
// ends; host code reaches it only through the address hipGetSymbolAddress
// returns for the current device, looked up once per device.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <mutex>

namespace mpk {

constexpr size_t kScratchBytes = size_t(64) << 20;

static __device__ __align__(256) char scratch[kScratchBytes];

namespace {

constexpr int kMaxDevices = 64;
void* g_scratch_ptr[kMaxDevices];   // device address of `scratch`, per device
std::mutex g_scratch_mu;

// Zero [p, p + 16 n16) (a fill kernel, not a memset: a caller may capture
// the step into a graph).
__global__ void __launch_bounds__(256) scratch_zero_kernel(uint4* p, size_t n16) {
  for (size_t i = (size_t)blockIdx.x * 256 + threadIdx.x; i < n16; i += (size_t)gridDim.x * 256)
    p[i] = make_uint4(0u, 0u, 0u, 0u);
}

}  // namespace

size_t scratch_capacity() { return kScratchBytes; }

// The device address of `scratch` on `device`, which must be the current
// device; looked up on the first call for that device.
hipError_t scratch_address(int device, void** out) {
  if (device < 0 || device >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[device]) {
    void* p = nullptr;
    const hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    g_scratch_ptr[device] = p;
  }
  *out = g_scratch_ptr[device];
  return hipSuccess;
}

// Zero `bytes` (a multiple of 16) of scratch starting at device address p.
hipError_t scratch_zero(void* p, size_t bytes, hipStream_t stream) {
  const size_t n16 = bytes / 16;
  if (n16 == 0) return hipSuccess;
  const int blocks = (int)std::min<size_t>(1024, (n16 + 255) / 256);
  hipLaunchKernelGGL(scratch_zero_kernel, dim3(blocks), dim3(256), 0, stream, reinterpret_cast<uint4*>(p), n16);
  return hipGetLastError();
}

}  // namespace mpk
