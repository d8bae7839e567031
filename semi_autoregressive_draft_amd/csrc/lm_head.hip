// LM-head contraction U[m, v] = sum_k h[m, k] * W_lm[v, k], float32 out.
// "DSpark 论文精读", §2.2: U_1..U_gamma = W_lm [h_1..h_gamma]; "DeepSpec 训练全流程详解",
// §4.3 compute_logits(block_hidden).  Both operands are K-contiguous ("NT"),
// which is exactly the per-lane layout of the MFMA operands.
#include "common.h"
#include "internal.h"

namespace dspark {

// ---------------------------------------------------------------------------
// Skinny path, M <= 16 (one or a few requests): HBM-bound on W_lm.  The whole
// h (M rows, padded stride to spread LDS banks) sits in LDS; each wave streams
// 16 vocabulary rows of W_lm at a time straight from HBM into the A operand of
// v_mfma_f32_16x16x32_bf16 (row n = lane%16, 8 consecutive k per lane), with h
// as the B operand (zero for columns >= M).  The output tile D[v][m] leaves each
// lane 4 consecutive vocabulary entries of one row m: one 16-byte store.
constexpr int kSkinnyWaves = 4;
constexpr int kSkinnyTilesPerWave = 1;
constexpr int kSkinnyUnroll = 8;

__global__ __launch_bounds__(kWave* kSkinnyWaves) void lm_head_skinny_bf16(
    const uint16_t* __restrict__ h, const uint16_t* __restrict__ W, float* __restrict__ U,
    int M, int H, int V) {
  extern __shared__ uint16_t hs[];  // [M][H + 8]
  const int ld = H + 8;
  for (int e = threadIdx.x; e < M * (H / 8); e += blockDim.x) {
    const int m = e / (H / 8), kk = (e % (H / 8)) * 8;
    *reinterpret_cast<u32x4*>(hs + m * ld + kk) =
        *reinterpret_cast<const u32x4*>(h + static_cast<size_t>(m) * H + kk);
  }
  __syncthreads();

  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int g = lane >> 4, n = lane & 15;
  const bool hcol = n < M;
  const uint16_t* hrow = hs + n * ld;
  const int nk = H / 32;           // full 32-wide k chunks
  const bool ktail = (H % 32) != 0;

  for (int t = 0; t < kSkinnyTilesPerWave; ++t) {
    const int v0 = ((blockIdx.x * kSkinnyWaves + w) * kSkinnyTilesPerWave + t) * 16;
    if (v0 >= V) break;
    const int vr = v0 + n;
    const bool vok = vr < V;
    const uint16_t* wrow = W + static_cast<size_t>(vok ? vr : 0) * H + 8 * g;
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
    int kc = 0;
    for (; kc + kSkinnyUnroll <= nk; kc += kSkinnyUnroll) {
      u32x4 wa[kSkinnyUnroll];
#pragma unroll
      for (int u = 0; u < kSkinnyUnroll; ++u)
        wa[u] = vok ? *reinterpret_cast<const u32x4*>(wrow + (kc + u) * 32) : u32x4{0u, 0u, 0u, 0u};
#pragma unroll
      for (int u = 0; u < kSkinnyUnroll; ++u) {
        const u32x4 hb = hcol ? *reinterpret_cast<const u32x4*>(hrow + (kc + u) * 32 + 8 * g)
                              : u32x4{0u, 0u, 0u, 0u};
        acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(wa[u]), as_bf16x8(hb), acc, 0, 0, 0);
      }
    }
    for (; kc < nk + (ktail ? 1 : 0); ++kc) {
      const int k = kc * 32 + 8 * g;
      const bool kok = k < H;
      const u32x4 wa = (vok && kok) ? *reinterpret_cast<const u32x4*>(wrow + kc * 32) : u32x4{0u, 0u, 0u, 0u};
      const u32x4 hb = (hcol && kok) ? *reinterpret_cast<const u32x4*>(hrow + k) : u32x4{0u, 0u, 0u, 0u};
      acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(wa), as_bf16x8(hb), acc, 0, 0, 0);
    }
    // D[4g + i][n] = U[m = n][v0 + 4g + i]
    const int vo = v0 + 4 * g;
    if (hcol && vo < V)
      *reinterpret_cast<f32x4*>(U + static_cast<size_t>(n) * V + vo) = acc;
  }
}

// ---------------------------------------------------------------------------
// Tiled path, M > 16: 128 (vocabulary) x 128 (rows of h) tiles, K steps of 64,
// 4 waves in a 2 x 2 layout with 64 x 64 each (4 x 4 MFMA 16x16x32 tiles).
// Operands are staged through LDS (rows padded by 16 bytes against bank
// conflicts), double-buffered with a register prefetch of the next K step.
// The A operand is W (vocabulary rows), the B operand h, so each lane stores
// 4 consecutive vocabulary entries.
constexpr int kTV = 128, kTM = 128, kTK = 64, kLd = kTK + 8;

__global__ __launch_bounds__(256) void lm_head_tiled_bf16(
    const uint16_t* __restrict__ h, const uint16_t* __restrict__ W, float* __restrict__ U,
    int M, int H, int V) {
  __shared__ uint16_t Ws[2][kTV * kLd];
  __shared__ uint16_t Hs[2][kTM * kLd];
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int g = lane >> 4, n = lane & 15;
  const int wv = w & 1, wm = w >> 1;
  const int v0 = blockIdx.x * kTV, m0 = blockIdx.y * kTM;
  const int nkt = (H + kTK - 1) / kTK;

  // global -> register staging: 4 chunks of 16 bytes per operand per thread
  u32x4 rw[4], rh[4];
  auto gload = [&](int kt) {
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int id = tid + 256 * q;
      const int row = id >> 3, kk = kt * kTK + (id & 7) * 8;
      const bool kok = kk < H;
      const int vr = v0 + row, mr = m0 + row;
      rw[q] = (kok && vr < V) ? *reinterpret_cast<const u32x4*>(W + static_cast<size_t>(vr) * H + kk)
                              : u32x4{0u, 0u, 0u, 0u};
      rh[q] = (kok && mr < M) ? *reinterpret_cast<const u32x4*>(h + static_cast<size_t>(mr) * H + kk)
                              : u32x4{0u, 0u, 0u, 0u};
    }
  };
  auto sstore = [&](int buf) {
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int id = tid + 256 * q;
      const int row = id >> 3, kk = (id & 7) * 8;
      *reinterpret_cast<u32x4*>(&Ws[buf][row * kLd + kk]) = rw[q];
      *reinterpret_cast<u32x4*>(&Hs[buf][row * kLd + kk]) = rh[q];
    }
  };

  f32x4 acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int jn = 0; jn < 4; ++jn) acc[i][jn] = f32x4{0.f, 0.f, 0.f, 0.f};

  gload(0);
  sstore(0);
  __syncthreads();
  for (int kt = 0; kt < nkt; ++kt) {
    const int buf = kt & 1;
    if (kt + 1 < nkt) gload(kt + 1);
#pragma unroll
    for (int ks = 0; ks < kTK / 32; ++ks) {
      u32x4 a[4], bb[4];
#pragma unroll
      for (int i = 0; i < 4; ++i)
        a[i] = *reinterpret_cast<const u32x4*>(&Ws[buf][(wv * 64 + i * 16 + n) * kLd + ks * 32 + 8 * g]);
#pragma unroll
      for (int jn = 0; jn < 4; ++jn)
        bb[jn] = *reinterpret_cast<const u32x4*>(&Hs[buf][(wm * 64 + jn * 16 + n) * kLd + ks * 32 + 8 * g]);
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int jn = 0; jn < 4; ++jn)
          acc[i][jn] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(a[i]), as_bf16x8(bb[jn]),
                                                               acc[i][jn], 0, 0, 0);
    }
    if (kt + 1 < nkt) sstore(buf ^ 1);
    __syncthreads();
  }
  // D[4g + ii][n]: vocabulary v0 + wv*64 + i*16 + 4g + ii, row m0 + wm*64 + jn*16 + n
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int vo = v0 + wv * 64 + i * 16 + 4 * g;
    if (vo >= V) continue;
#pragma unroll
    for (int jn = 0; jn < 4; ++jn) {
      const int m = m0 + wm * 64 + jn * 16 + n;
      if (m < M) *reinterpret_cast<f32x4*>(U + static_cast<size_t>(m) * V + vo) = acc[i][jn];
    }
  }
}

// ---------------------------------------------------------------------------
// float32 path (small reference shapes): 64 x 64 LDS tiles, 4 x 4 per thread.
__global__ __launch_bounds__(256) void lm_head_f32(const float* __restrict__ h,
                                                   const float* __restrict__ W,
                                                   float* __restrict__ U, int M, int H, int V) {
  __shared__ float hs[16][64 + 1];
  __shared__ float ws[16][64 + 1];
  const int tx = threadIdx.x & 15, ty = threadIdx.x >> 4;
  const int v0 = blockIdx.x * 64, m0 = blockIdx.y * 64;
  float acc[4][4] = {};
  for (int k0 = 0; k0 < H; k0 += 16) {
    for (int e = threadIdx.x; e < 16 * 64; e += 256) {
      const int r = e >> 4, kk = e & 15;
      const int k = k0 + kk;
      hs[kk][r] = (m0 + r < M && k < H) ? h[static_cast<size_t>(m0 + r) * H + k] : 0.f;
      ws[kk][r] = (v0 + r < V && k < H) ? W[static_cast<size_t>(v0 + r) * H + k] : 0.f;
    }
    __syncthreads();
    for (int kk = 0; kk < 16; ++kk)
      for (int i = 0; i < 4; ++i)
        for (int jv = 0; jv < 4; ++jv) acc[i][jv] = fmaf(hs[kk][ty * 4 + i], ws[kk][tx * 4 + jv], acc[i][jv]);
    __syncthreads();
  }
  for (int i = 0; i < 4; ++i) {
    const int m = m0 + ty * 4 + i;
    if (m >= M) continue;
    for (int jv = 0; jv < 4; ++jv) {
      const int v = v0 + tx * 4 + jv;
      if (v < V) U[static_cast<size_t>(m) * V + v] = acc[i][jv];
    }
  }
}

size_t lm_head_skinny_lds(int64_t M, int64_t H) { return static_cast<size_t>(M) * (H + 8) * 2; }

hipError_t launch_lm_head(const void* h, const void* w, bool bf16, int64_t M, int64_t H,
                          int64_t V, float* U, hipStream_t s) {
  if (!bf16) {
    const dim3 grid((V + 63) / 64, (M + 63) / 64);
    hipLaunchKernelGGL(lm_head_f32, grid, dim3(256), 0, s, static_cast<const float*>(h),
                       static_cast<const float*>(w), U, (int)M, (int)H, (int)V);
  } else if (M <= 16 && lm_head_skinny_lds(M, H) <= kSkinnyMaxLds) {
    const int64_t tiles = (V + 15) / 16;
    const int64_t per_block = kSkinnyWaves * kSkinnyTilesPerWave;
    const dim3 grid((tiles + per_block - 1) / per_block);
    hipLaunchKernelGGL(lm_head_skinny_bf16, grid, dim3(kWave * kSkinnyWaves),
                       lm_head_skinny_lds(M, H), s, static_cast<const uint16_t*>(h),
                       static_cast<const uint16_t*>(w), U, (int)M, (int)H, (int)V);
  } else {
    const dim3 grid((V + kTV - 1) / kTV, (M + kTM - 1) / kTM);
    hipLaunchKernelGGL(lm_head_tiled_bf16, grid, dim3(256), 0, s, static_cast<const uint16_t*>(h),
                       static_cast<const uint16_t*>(w), U, (int)M, (int)H, (int)V);
  }
  return hipGetLastError();
}

}  // namespace dspark
