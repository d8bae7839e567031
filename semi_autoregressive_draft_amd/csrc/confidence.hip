// Confidence head and prefix survival.
// "Qwen3.8-Flash-Next DSpark 训练实验", Confidence head: s_i = w_c^T [h_i; m_i] + b_c,
// a^_i = sigmoid(s_i) with m_i = W_1[t_{i-1}]; "DeepSpec 训练全流程详解", §4.3
// predict_confidence_step (hidden states only, the w_m == null case);
// "DSpark 论文精读", §3.1: a_{r,j} = prod_{i<=j} c_{r,i}.
//
// One workgroup per request: each of the gamma dot products (H + r terms) is
// reduced by a fixed tree, and thread 0 runs the sigmoid and the running
// product in position order.  The work is a few KB per request, so the
// kernel is bound by launch latency, not by HBM.
#include "common.h"
#include "internal.h"

namespace dspark {

template <typename T>
__global__ __launch_bounds__(256) void confidence_survival_kernel(
    const T* __restrict__ h, int gamma, int H, const T* __restrict__ w_c, float b_c,
    const T* __restrict__ w_m, const T* __restrict__ A, int r, const int32_t* __restrict__ anchor,
    const int32_t* __restrict__ tokens, float* __restrict__ conf, float* __restrict__ surv) {
  __shared__ float part[kMaxGamma][4];
  const int b = blockIdx.x, tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  for (int j = 0; j < gamma; ++j) {
    const T* hr = h + (static_cast<size_t>(b) * gamma + j) * H;
    float s = 0.f;
    for (int k = tid; k < H; k += 256) s = fmaf(to_f32(hr[k]), to_f32(w_c[k]), s);
    if (w_m) {
      const int prev = j == 0 ? anchor[b] : tokens[b * gamma + j - 1];
      const T* ar = A + static_cast<size_t>(prev) * r;
      for (int k = tid; k < r; k += 256) s = fmaf(to_f32(ar[k]), to_f32(w_m[k]), s);
    }
    s = wave_sum(s);
    if (lane == 0) part[j][w] = s;
  }
  __syncthreads();
  if (tid == 0) {
    float run = 1.f;
    for (int j = 0; j < gamma; ++j) {
      const float s = ((part[j][0] + part[j][1]) + (part[j][2] + part[j][3])) + b_c;
      const float c = 1.0f / (1.0f + __expf(-s));
      run *= c;
      conf[b * gamma + j] = c;
      surv[b * gamma + j] = run;
    }
  }
}

hipError_t launch_confidence(const void* h, bool bf16, int B, int gamma, int H,
                             const void* w_c, float b_c, const void* w_m, const void* A, int r,
                             const int32_t* anchor, const int32_t* tokens, float* conf,
                             float* surv, hipStream_t s) {
  if (bf16)
    hipLaunchKernelGGL(confidence_survival_kernel<uint16_t>, dim3(B), dim3(256), 0, s,
                       static_cast<const uint16_t*>(h), gamma, H, static_cast<const uint16_t*>(w_c),
                       b_c, static_cast<const uint16_t*>(w_m), static_cast<const uint16_t*>(A), r,
                       anchor, tokens, conf, surv);
  else
    hipLaunchKernelGGL(confidence_survival_kernel<float>, dim3(B), dim3(256), 0, s,
                       static_cast<const float*>(h), gamma, H, static_cast<const float*>(w_c), b_c,
                       static_cast<const float*>(w_m), static_cast<const float*>(A), r, anchor,
                       tokens, conf, surv);
  return hipGetLastError();
}

}  // namespace dspark
