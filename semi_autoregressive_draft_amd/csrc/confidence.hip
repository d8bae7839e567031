// Confidence head and prefix survival.
// "Qwen3.8-Flash-Next DSpark 训练实验", Confidence head: s_i = w_c^T [h_i; m_i] + b_c,
// a^_i = sigmoid(s_i) with m_i = W_1[t_{i-1}]; "DeepSpec 训练全流程详解", §4.3
// predict_confidence_step (hidden states only, the w_m == null case);
// "DSpark 论文精读", §3.1: a_{r,j} = prod_{i<=j} c_{r,i}.
//
// One workgroup per request with one wave per slot j: each wave reduces its
// dot product (H terms, plus r for the Markov term) from 16-byte loads by a
// fixed tree, then thread 0 runs the sigmoid and the running product in
// position order.  The work is a few KB per request, so the kernel is bound by
// latency, not by HBM; the gamma dot products run concurrently.
#include "common.h"
#include "internal.h"

namespace dspark {

template <typename T>
__device__ __forceinline__ float dot_row(const T* x, const T* y, int n, int lane, bool vec) {
  float s = 0.f;
  int done = 0;
  if (vec) {  // 16-byte loads: 8 bf16 or 4 float per lane and step
    constexpr int E = 16 / sizeof(T);
    const int nv = n / E;
    for (int i = lane; i < nv; i += kWave) {
      const u32x4 a = reinterpret_cast<const u32x4*>(x)[i];
      const u32x4 b = reinterpret_cast<const u32x4*>(y)[i];
      if constexpr (sizeof(T) == 2) {
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          s = fmaf(__uint_as_float(a[q] << 16), __uint_as_float(b[q] << 16), s);
          s = fmaf(__uint_as_float(a[q] & 0xFFFF0000u), __uint_as_float(b[q] & 0xFFFF0000u), s);
        }
      } else {
#pragma unroll
        for (int q = 0; q < 4; ++q) s = fmaf(__uint_as_float(a[q]), __uint_as_float(b[q]), s);
      }
    }
    done = nv * E;
  }
  for (int k = done + lane; k < n; k += kWave) s = fmaf(to_f32(x[k]), to_f32(y[k]), s);
  return s;
}

template <typename T>
__global__ __launch_bounds__(kWave* kMaxGamma) void confidence_survival_kernel(
    const T* __restrict__ h, int gamma, int H, const T* __restrict__ w_c, float b_c,
    const T* __restrict__ w_m, const T* __restrict__ A, int r, const int32_t* __restrict__ anchor,
    const int32_t* __restrict__ tokens, float* __restrict__ conf, float* __restrict__ surv,
    int vec_h, int vec_r) {
  __shared__ float part[kMaxGamma];
  const int b = blockIdx.x, lane = threadIdx.x & 63, j = threadIdx.x >> 6;
  float s = dot_row(h + (static_cast<size_t>(b) * gamma + j) * H, w_c, H, lane, vec_h);
  if (w_m) {
    // a -1 token (a chain that timed out) contributes no Markov term
    const int prev = j == 0 ? anchor[b] : tokens[b * gamma + j - 1];
    if (prev >= 0) s += dot_row(A + static_cast<size_t>(prev) * r, w_m, r, lane, vec_r);
  }
  s = wave_sum(s);
  if (lane == 0) part[j] = s;
  __syncthreads();
  if (threadIdx.x == 0) {
    float run = 1.f;
    for (int jj = 0; jj < gamma; ++jj) {
      const float c = 1.0f / (1.0f + __expf(-(part[jj] + b_c)));
      run *= c;
      conf[b * gamma + jj] = c;
      surv[b * gamma + jj] = run;
    }
  }
}

static bool al16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

hipError_t launch_confidence(const void* h, bool bf16, int B, int gamma, int H,
                             const void* w_c, float b_c, const void* w_m, const void* A, int r,
                             const int32_t* anchor, const int32_t* tokens, float* conf,
                             float* surv, hipStream_t s) {
  const int es = bf16 ? 2 : 4;
  const int vec_h = al16(h) && al16(w_c) && (H * es) % 16 == 0;
  const int vec_r = w_m && al16(A) && al16(w_m) && (r * es) % 16 == 0;
  const dim3 block(kWave * gamma);
  if (bf16)
    hipLaunchKernelGGL(confidence_survival_kernel<uint16_t>, dim3(B), block, 0, s,
                       static_cast<const uint16_t*>(h), gamma, H, static_cast<const uint16_t*>(w_c),
                       b_c, static_cast<const uint16_t*>(w_m), static_cast<const uint16_t*>(A), r,
                       anchor, tokens, conf, surv, vec_h, vec_r);
  else
    hipLaunchKernelGGL(confidence_survival_kernel<float>, dim3(B), block, 0, s,
                       static_cast<const float*>(h), gamma, H, static_cast<const float*>(w_c), b_c,
                       static_cast<const float*>(w_m), static_cast<const float*>(A), r, anchor,
                       tokens, conf, surv, vec_h, vec_r);
  return hipGetLastError();
}

}  // namespace dspark
