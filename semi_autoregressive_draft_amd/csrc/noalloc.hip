// dspark_markov_propose_noalloc: the Markov proposal with the library's own
// scratch in place of a caller workspace, for callers that cannot allocate
// device memory.  The scratch is a static device array, one copy per device;
// host code never passes the array's name to a kernel (on the host it is only
// a stand-in for the symbol): it uses the address hipGetSymbolAddress returns
// for the current device, taken once per device on its first call.
#include <mutex>

#include "common.h"
#include "dspark.h"
#include "internal.h"

namespace {

constexpr size_t kScratchBytes = static_cast<size_t>(64) << 20;   // 64 MiB per device
constexpr int kMaxDevices = 64;

static __device__ __align__(256) unsigned char scratch[kScratchBytes];

__global__ __launch_bounds__(256) void zero_scratch(dspark::u32x4* __restrict__ p, size_t n16) {
  const size_t stride = static_cast<size_t>(gridDim.x) * 256;
  for (size_t i = static_cast<size_t>(blockIdx.x) * 256 + threadIdx.x; i < n16; i += stride)
    p[i] = dspark::u32x4{0u, 0u, 0u, 0u};
}

struct Slot {
  std::mutex mu;
  void* ptr = nullptr;   // this device's copy of `scratch`
};
Slot g_slots[kMaxDevices];

// The current device's scratch address; on the first call on a device, its
// address is looked up and a fill kernel on `s` zeroes the whole array (the
// chain's wait tree at its start must read zero when a call begins; every
// call leaves it zero again).
hipError_t acquire_scratch(hipStream_t s, void** out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  Slot& sl = g_slots[dev];
  std::lock_guard<std::mutex> lock(sl.mu);
  if (!sl.ptr) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    if (p == nullptr) return hipErrorInvalidSymbol;
    hipLaunchKernelGGL(zero_scratch, dim3(1024), dim3(256), 0, s, static_cast<dspark::u32x4*>(p),
                       kScratchBytes / 16);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
    sl.ptr = p;
  }
  *out = sl.ptr;
  return hipSuccess;
}

const dspark::ScratchProvider kProvider{kScratchBytes, acquire_scratch};

}  // namespace

extern "C" dspark_status_t dspark_markov_propose_noalloc(
    const float* U, int64_t B, int64_t gamma, int64_t V, const int32_t* anchor, const void* A,
    const void* Bm, dspark_dtype_t wdt, int64_t r, float temperature, const uint64_t* seeds,
    uint64_t offset, int32_t topk, int32_t* tokens, float* tok_logit, float* lse,
    int32_t* topk_idx, float* topk_prob, float* logits_out, int32_t* status, hipStream_t stream) {
  return propose_impl("dspark_markov_propose_noalloc", dspark::kHeadLinear, nullptr, 0, nullptr, U, B, gamma, V,
                      anchor, A, Bm, wdt, r, temperature, seeds, offset, topk, tokens, tok_logit, lse, topk_idx,
                      topk_prob, logits_out, nullptr, 0, &kProvider, status, stream);
}
