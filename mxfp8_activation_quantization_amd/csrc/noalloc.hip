// fp8_gemm_nt_noalloc: fp8_gemm_nt for callers that cannot allocate device
// memory (code under HIP graph capture, tight serving loops, harnesses that
// forbid hipMalloc).  Its scratch -- the split-K arrival counters and fp32
// partial tiles of the few-token kernels, and BF16 activations quantized to
// MXFP8 before the tile kernels -- lives in one fixed device array of this file
// instead of a caller-supplied workspace.  The kernels are fp8_gemm_nt's, so the
// results are its results, bit for bit.
#include <hip/hip_runtime.h>

#include <mutex>

#include "../../include/mxfp8.h"
#include "launch.hpp"

#define MX_API extern "C" __attribute__((visibility("default")))

namespace {

// 16 MiB per GPU, held from the library's load until the process ends.
constexpr int64_t kScratchBytes = int64_t(16) << 20;
// The leading part the split-K kernels keep their arrival counters in (zero between calls).
constexpr int64_t kCounterRegion = 65536;

static __device__ __align__(256) uint8_t scratch[kScratchBytes];

constexpr int kMaxDevices = 256;
std::mutex g_mu;
void* g_ptr[kMaxDevices];       // device address of `scratch` on each device (null until looked up)
bool g_cleared[kMaxDevices];    // the counter region's zero fill has been enqueued on this device

__global__ void clear_words(uint32_t* p, int64_t n) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) p[i] = 0u;
}

// The device address of the current device's copy of `scratch`.  On the first call on a device it is
// looked up (each device holds its own copy at its own address) and a zero fill of the counter region is
// enqueued on `stream` ahead of the caller's kernels.  Null when the lookup or the launch fails.
void* scratch_on_current(hipStream_t stream) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return nullptr;
  std::lock_guard<std::mutex> lock(g_mu);
  if (!g_ptr[dev]) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return nullptr;
    g_ptr[dev] = p;
  }
  if (!g_cleared[dev]) {
    const int64_t words = kCounterRegion / 4;
    hipLaunchKernelGGL(clear_words, dim3((unsigned)((words + 255) / 256)), dim3(256), 0, stream,
                       static_cast<uint32_t*>(g_ptr[dev]), words);
    if (hipGetLastError() != hipSuccess) return nullptr;
    g_cleared[dev] = true;
  }
  return g_ptr[dev];
}

}  // namespace

MX_API int fp8_gemm_nt_noalloc(int a_kind, const void* a, int64_t ld_a, const int32_t* a_sf, int64_t ld_asf,
                               int64_t M, int64_t N, int64_t K, const void* b, const int32_t* b_sf, void* d,
                               int64_t ld_d, void* stream) {
  static_assert(kScratchBytes == MXFP8_NOALLOC_SCRATCH_BYTES, "the size the header states");
  return mx::gemm_entry(mx::SPLITK_LOCAL, a_kind, a, ld_a, a_sf, ld_asf, M, N, K, b, b_sf, d, ld_d, nullptr, 0,
                        stream, scratch_on_current, kScratchBytes);
}
