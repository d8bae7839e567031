// Sequential-head variants: the r-vector m_j that the up-projection receives
// at position j.  "DSpark 论文精读：置信度调度推测解码、半自回归生成与大模型推理加速",
// §2.3 heads table: VanillaMarkov b_j = W_up SiLU(W_down[x_{j-1}]);
// GatedMarkovHead g_j = sigma(W_g [h_j; W_down[x_{j-1}]]),
// b_j = W_up (g_j * W_down[x_{j-1}]).  With A = W_down and Bm = W_up^T the
// per-position step kernels stay as they are: before each position this
// kernel writes m_j (rounded to the tables' dtype, as a module computing in
// that dtype hands it on) for every request, and the step and top-k kernels
// read their A operand from those rows instead of A[x_{j-1}].
//
// One workgroup of 256 threads per request.  SiLU: elementwise over r.
// Gated: the concatenation [h_j; A[x_{j-1}]] (H + r floats) sits in LDS and
// each wave computes r / 4 of the gate's dot products with rows of W_g
// [r, H + r] (lanes over the row, a fixed-order wave reduction), then
// m_k = sigma(z_k) * a_k.
#include "common.h"
#include "internal.h"
#include "markov_dev.h"

namespace dspark {

constexpr int kHeadThreads = 256;

__device__ __forceinline__ uint16_t bf16_round(float f) {
  const uint32_t u = __float_as_uint(f);
  return static_cast<uint16_t>((u + 0x7FFFu + ((u >> 16) & 1u)) >> 16);
}
template <typename T> __device__ __forceinline__ T store_as(float v);
template <> __device__ __forceinline__ float store_as<float>(float v) { return v; }
template <> __device__ __forceinline__ uint16_t store_as<uint16_t>(float v) { return bf16_round(v); }

template <typename WT>
__global__ __launch_bounds__(kHeadThreads) void markov_head_prep(StepArgs a, int head, const WT* __restrict__ h,
                                                                  int H, const WT* __restrict__ Wg, WT* __restrict__ M) {
  extern __shared__ float xs[];                        // gated: [H + r]
  const int b = blockIdx.x, tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const WT* arow = static_cast<const WT*>(a.A) + static_cast<size_t>(prev_token(a, b, a.j)) * a.r;
  WT* out = M + (static_cast<size_t>(b) * a.gamma + a.j) * a.r;
  if (head == kHeadSilu) {
    for (int k = tid; k < a.r; k += kHeadThreads) {
      const float x = to_f32(arow[k]);
      out[k] = store_as<WT>(x / (1.0f + expf(-x)));
    }
    return;
  }
  const WT* hrow = h + (static_cast<size_t>(b) * a.gamma + a.j) * H;
  for (int i = tid; i < H; i += kHeadThreads) xs[i] = to_f32(hrow[i]);
  for (int k = tid; k < a.r; k += kHeadThreads) xs[H + k] = to_f32(arow[k]);
  __syncthreads();
  const int D = H + a.r;
  for (int k = w; k < a.r; k += kHeadThreads / kWave) {
    const WT* wrow = Wg + static_cast<size_t>(k) * D;
    float z = 0.f;
    for (int i = lane; i < D; i += kWave) z = fmaf(to_f32(wrow[i]), xs[i], z);
    z = wave_sum(z);
    if (lane == 0) out[k] = store_as<WT>(xs[H + k] / (1.0f + expf(-z)));
  }
}

hipError_t launch_head_prep(const StepArgs& a, bool bf16, int head, const void* h, int H, const void* Wg, void* M,
                            hipStream_t s) {
  const size_t lds = head == kHeadGated ? static_cast<size_t>(H + a.r) * 4 : 0;
  if (lds > 64 * 1024) {
    const void* fn = bf16 ? reinterpret_cast<const void*>(&markov_head_prep<uint16_t>)
                          : reinterpret_cast<const void*>(&markov_head_prep<float>);
    const hipError_t e = hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize, static_cast<int>(lds));
    if (e != hipSuccess) return e;
  }
  if (bf16)
    hipLaunchKernelGGL(markov_head_prep<uint16_t>, dim3(a.B), dim3(kHeadThreads), lds, s, a, head,
                       static_cast<const uint16_t*>(h), H, static_cast<const uint16_t*>(Wg), static_cast<uint16_t*>(M));
  else
    hipLaunchKernelGGL(markov_head_prep<float>, dim3(a.B), dim3(kHeadThreads), lds, s, a, head,
                       static_cast<const float*>(h), H, static_cast<const float*>(Wg), static_cast<float*>(M));
  return hipGetLastError();
}

}  // namespace dspark
