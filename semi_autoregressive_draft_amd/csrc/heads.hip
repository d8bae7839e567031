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
//
// RNN head (same table, row RNNHead, and the RNN head passage of "Baseline
// 架构"): state s_j of rank r, zero before the block; input
// z_j = [s_{j-1}; A[x_{j-1}]; h_j]; s_j = (1 - g) * s_{j-1} + g * c with
// g = sigma(W_gate z_j), c = tanh(W_cand z_j); m_j = SiLU(W_out [s_j; A[x_{j-1}]; h_j]).
// W = [W_gate; W_cand; W_out] is [3r, 2r + H]; the state table S [B, gamma, r]
// (tables' dtype, one row per position) follows the m_j table in the
// workspace.  bf16 with H % 8 == 0: two MFMA launches per position, the state
// (gate and candidate rows share each input fragment) and then the output,
// laid out as the gated head's with K split over four waves.  Otherwise one workgroup per request with z in LDS.
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

template <typename WT>
__global__ __launch_bounds__(kHeadThreads) void markov_head_rnn(StepArgs a, const WT* __restrict__ h, int H,
                                                                const WT* __restrict__ W, WT* __restrict__ M,
                                                                WT* __restrict__ S) {
  extern __shared__ float xs[];                        // [2r + H] input, then [r] new state
  const int b = blockIdx.x, tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int r = a.r, D = 2 * r + H;
  const size_t row = static_cast<size_t>(b) * a.gamma + a.j;
  const WT* arow = static_cast<const WT*>(a.A) + static_cast<size_t>(prev_token(a, b, a.j)) * r;
  const WT* hrow = h + row * H;
  const WT* sprev = S + (a.j > 0 ? row - 1 : row) * r;
  float* sn = xs + D;
  for (int k = tid; k < r; k += kHeadThreads) {
    xs[k] = a.j > 0 ? to_f32(sprev[k]) : 0.f;
    xs[r + k] = to_f32(arow[k]);
  }
  for (int i = tid; i < H; i += kHeadThreads) xs[2 * r + i] = to_f32(hrow[i]);
  __syncthreads();
  for (int k = w; k < r; k += kHeadThreads / kWave) {
    const WT* wg = W + static_cast<size_t>(k) * D;
    const WT* wc = W + static_cast<size_t>(r + k) * D;
    float zg = 0.f, zc = 0.f;
    for (int i = lane; i < D; i += kWave) {
      zg = fmaf(to_f32(wg[i]), xs[i], zg);
      zc = fmaf(to_f32(wc[i]), xs[i], zc);
    }
    zg = wave_sum(zg);
    zc = wave_sum(zc);
    if (lane == 0) {
      const float g = 1.0f / (1.0f + expf(-zg));
      const WT sv = store_as<WT>((1.0f - g) * xs[k] + g * tanhf(zc));
      S[row * r + k] = sv;
      sn[k] = to_f32(sv);
    }
  }
  __syncthreads();
  for (int k = tid; k < r; k += kHeadThreads) xs[k] = sn[k];
  __syncthreads();
  for (int k = w; k < r; k += kHeadThreads / kWave) {
    const WT* wo = W + static_cast<size_t>(2 * r + k) * D;
    float z = 0.f;
    for (int i = lane; i < D; i += kWave) z = fmaf(to_f32(wo[i]), xs[i], z);
    z = wave_sum(z);
    if (lane == 0) M[row * r + k] = store_as<WT>(z / (1.0f + expf(-z)));
  }
}

// 8 consecutive inputs k..k+7 of z = [state; A[x_{j-1}]; h_j] (k a multiple of
// 8; r % 8 == 0 and H % 8 == 0, so a fragment never straddles two parts)
__device__ __forceinline__ u32x4 rnn_input8(const uint16_t* srow, bool has_s, const uint16_t* arow,
                                            const uint16_t* hrow, int r, int k) {
  if (k < r) return has_s ? *reinterpret_cast<const u32x4*>(srow + k) : u32x4{0u, 0u, 0u, 0u};
  if (k < 2 * r) return *reinterpret_cast<const u32x4*>(arow + (k - r));
  return *reinterpret_cast<const u32x4*>(hrow + (k - 2 * r));
}

// grid (ceil(r / 16), ceil(B / 16)), kRnnWaves waves each, wave w taking the
// 32-deep K chunks c = w mod kRnnWaves; wave 0 adds the others' partial sums
// from LDS and finishes.  OUT = false: gate and candidate rows -> S[b, j];
// OUT = true: output rows over [S[b, j]; ...] -> M[b, j]
constexpr int kRnnWaves = 4;
template <bool OUT>
__global__ __launch_bounds__(kRnnWaves * kWave) void markov_head_rnn_bf16(StepArgs a, const uint16_t* __restrict__ h, int H,
                                                              const uint16_t* __restrict__ W,
                                                              uint16_t* __restrict__ M, uint16_t* __restrict__ S) {
  __shared__ f32x4 red[2][kRnnWaves - 1][kWave];
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6, g = lane >> 4, n = lane & 15;
  const int o0 = blockIdx.x * 16, b0 = blockIdx.y * 16;
  const int r = a.r, D = 2 * r + H;
  const int bx = min(b0 + n, a.B - 1);                 // this lane's request row (A operand)
  const int ox = min(o0 + n, r - 1);                   // this lane's weight row within a block (B operand)
  const uint16_t* A = static_cast<const uint16_t*>(a.A);
  const size_t rowx = static_cast<size_t>(bx) * a.gamma + a.j;
  const bool has_s = OUT || a.j > 0;
  const uint16_t* srow = S + (OUT || a.j == 0 ? rowx : rowx - 1) * r;
  const uint16_t* arow = A + static_cast<size_t>(prev_token(a, bx, a.j)) * r;
  const uint16_t* hrow = h + rowx * H;
  const uint16_t* w0 = W + static_cast<size_t>((OUT ? 2 * r : 0) + ox) * D;
  const uint16_t* w1 = W + static_cast<size_t>(r + ox) * D;
  f32x4 acc0 = {0.f, 0.f, 0.f, 0.f}, acc1 = {0.f, 0.f, 0.f, 0.f};
  const int nk = (D + 31) / 32;
#pragma unroll 4
  for (int c = wv; c < nk; c += kRnnWaves) {
    const int k = 32 * c + 8 * g;
    u32x4 xa = {0u, 0u, 0u, 0u}, wa = {0u, 0u, 0u, 0u}, wb = {0u, 0u, 0u, 0u};
    if (k < D) {
      xa = rnn_input8(srow, has_s, arow, hrow, r, k);
      wa = *reinterpret_cast<const u32x4*>(w0 + k);
      if (!OUT) wb = *reinterpret_cast<const u32x4*>(w1 + k);
    }
    acc0 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(xa), as_bf16x8(wa), acc0, 0, 0, 0);
    if (!OUT) acc1 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(xa), as_bf16x8(wb), acc1, 0, 0, 0);
  }
  if (wv > 0) {
    red[0][wv - 1][lane] = acc0;
    if (!OUT) red[1][wv - 1][lane] = acc1;
  }
  __syncthreads();
  if (wv > 0) return;
#pragma unroll
  for (int q = 0; q < kRnnWaves - 1; ++q) {
    acc0 += red[0][q][lane];
    if (!OUT) acc1 += red[1][q][lane];
  }
  const int o = o0 + n;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int b = b0 + 4 * g + i;
    if (b < a.B && o < r) {
      const size_t row = static_cast<size_t>(b) * a.gamma + a.j;
      if (OUT) {
        M[row * r + o] = bf16_round(acc0[i] / (1.0f + expf(-acc0[i])));
      } else {
        const float gt = 1.0f / (1.0f + expf(-acc0[i]));
        const float sp = a.j > 0 ? bf16_to_f32(S[(row - 1) * r + o]) : 0.f;
        S[row * r + o] = bf16_round((1.0f - gt) * sp + gt * tanhf(acc1[i]));
      }
    }
  }
}

hipError_t launch_head_rnn(const StepArgs& a, bool bf16, const void* h, int H, const void* W, void* M,
                           hipStream_t s) {
  const size_t es = bf16 ? 2 : 4;
  void* S = static_cast<char*>(M) + static_cast<size_t>(a.B) * a.gamma * a.r * es;
  if (bf16 && H % 8 == 0 && a.r % 8 == 0 && (reinterpret_cast<uintptr_t>(h) & 15) == 0 &&
      (reinterpret_cast<uintptr_t>(W) & 15) == 0 && (reinterpret_cast<uintptr_t>(a.A) & 15) == 0 &&
      (reinterpret_cast<uintptr_t>(S) & 15) == 0) {
    const dim3 grid((a.r + 15) / 16, (a.B + 15) / 16);
    const uint16_t* hb = static_cast<const uint16_t*>(h);
    const uint16_t* Wb = static_cast<const uint16_t*>(W);
    uint16_t* Mb = static_cast<uint16_t*>(M);
    uint16_t* Sb = static_cast<uint16_t*>(S);
    hipLaunchKernelGGL(markov_head_rnn_bf16<false>, grid, dim3(kRnnWaves * kWave), 0, s, a, hb, H, Wb, Mb, Sb);
    hipLaunchKernelGGL(markov_head_rnn_bf16<true>, grid, dim3(kRnnWaves * kWave), 0, s, a, hb, H, Wb, Mb, Sb);
    return hipGetLastError();
  }
  const size_t lds = static_cast<size_t>(3 * a.r + H) * 4;
  const void* fn = bf16 ? reinterpret_cast<const void*>(&markov_head_rnn<uint16_t>)
                        : reinterpret_cast<const void*>(&markov_head_rnn<float>);
  if (lds > 64 * 1024) {
    const hipError_t e = hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize, static_cast<int>(lds));
    if (e != hipSuccess) return e;
  }
  if (bf16)
    hipLaunchKernelGGL(markov_head_rnn<uint16_t>, dim3(a.B), dim3(kHeadThreads), lds, s, a,
                       static_cast<const uint16_t*>(h), H, static_cast<const uint16_t*>(W), static_cast<uint16_t*>(M),
                       static_cast<uint16_t*>(S));
  else
    hipLaunchKernelGGL(markov_head_rnn<float>, dim3(a.B), dim3(kHeadThreads), lds, s, a,
                       static_cast<const float*>(h), H, static_cast<const float*>(W), static_cast<float*>(M),
                       static_cast<float*>(S));
  return hipGetLastError();
}

hipError_t launch_head_prep(const StepArgs& a, bool bf16, int head, const void* h, int H, const void* Wg, void* M,
                            hipStream_t s) {
  if (head == kHeadRnn) return launch_head_rnn(a, bf16, h, H, Wg, M, s);
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
