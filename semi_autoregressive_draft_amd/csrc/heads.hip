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
// SiLU: one workgroup of 256 threads per request, elementwise over r.
// Gated, bf16 with H % 8 == 0: the gate pre-activations are a small GEMM,
// Z [B, r] = X [B, H + r] W_g^T with X = [h_j; A[x_{j-1}]], on MFMA: one wave
// per 16 requests x 16 outputs, K in chunks of 32 (X rows as the A operand,
// W_g rows as the B operand, both contiguous in k), then
// m = sigma(z) * a.  Otherwise one workgroup per request with X in LDS and a
// wave per output row of W_g.
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

// gated head on MFMA (bf16, H % 8 == 0): grid (ceil(r / 16), ceil(B / 16)),
// one wave each.  Lane (g, n) loads 8 consecutive k of request row n (from h
// for k < H, else from A[x_{j-1}]) and of gate row n; D[4g + i][n] is request
// 4g + i, output n.
__global__ __launch_bounds__(kWave) void markov_head_gate_bf16(StepArgs a, const uint16_t* __restrict__ h, int H,
                                                               const uint16_t* __restrict__ Wg,
                                                               uint16_t* __restrict__ M) {
  const int lane = threadIdx.x, g = lane >> 4, n = lane & 15;
  const int o0 = blockIdx.x * 16, b0 = blockIdx.y * 16;
  const int D = H + a.r;
  const int bx = min(b0 + n, a.B - 1);                 // this lane's request row (A operand)
  const int ox = min(o0 + n, a.r - 1);                 // this lane's gate row (B operand)
  const uint16_t* A = static_cast<const uint16_t*>(a.A);
  const uint16_t* hrow = h + (static_cast<size_t>(bx) * a.gamma + a.j) * H;
  const uint16_t* arow = A + static_cast<size_t>(prev_token(a, bx, a.j)) * a.r;
  const uint16_t* wrow = Wg + static_cast<size_t>(ox) * D;
  f32x4 acc = {0.f, 0.f, 0.f, 0.f};
  const int nk = (D + 31) / 32;
#pragma unroll 8
  for (int c = 0; c < nk; ++c) {
    const int k = 32 * c + 8 * g;                       // a multiple of 8: never straddles h and A (H % 8 == 0)
    u32x4 xa = {0u, 0u, 0u, 0u}, wb = {0u, 0u, 0u, 0u};
    if (k < D) {
      xa = k < H ? *reinterpret_cast<const u32x4*>(hrow + k) : *reinterpret_cast<const u32x4*>(arow + (k - H));
      wb = *reinterpret_cast<const u32x4*>(wrow + k);
    }
    acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(xa), as_bf16x8(wb), acc, 0, 0, 0);
  }
  const int o = o0 + n;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int b = b0 + 4 * g + i;
    if (b < a.B && o < a.r) {
      const float av = bf16_to_f32(A[static_cast<size_t>(prev_token(a, b, a.j)) * a.r + o]);
      M[(static_cast<size_t>(b) * a.gamma + a.j) * a.r + o] = bf16_round(av / (1.0f + expf(-acc[i])));
    }
  }
}

hipError_t launch_head_prep(const StepArgs& a, bool bf16, int head, const void* h, int H, const void* Wg, void* M,
                            hipStream_t s) {
  if (head == kHeadGated && bf16 && H % 8 == 0 && (reinterpret_cast<uintptr_t>(h) & 15) == 0 &&
      (reinterpret_cast<uintptr_t>(Wg) & 15) == 0 && (reinterpret_cast<uintptr_t>(a.A) & 15) == 0 &&
      a.r % 8 == 0) {
    const dim3 grid((a.r + 15) / 16, (a.B + 15) / 16);
    hipLaunchKernelGGL(markov_head_gate_bf16, grid, dim3(kWave), 0, s, a, static_cast<const uint16_t*>(h), H,
                       static_cast<const uint16_t*>(Wg), static_cast<uint16_t*>(M));
    return hipGetLastError();
  }
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
