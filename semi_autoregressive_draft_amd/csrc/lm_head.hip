// LM-head contraction U[m, v] = sum_k h[m, k] * W_lm[v, k], float32 out (the
// few-row path lives in lm_head_skinny.hip).
// "DSpark 论文精读", §2.2: U_1..U_gamma = W_lm [h_1..h_gamma]; "DeepSpec 训练全流程详解",
// §4.3 compute_logits(block_hidden).  Both operands are K-contiguous ("NT"),
// which is exactly the per-lane layout of the MFMA operands.
#include "common.h"
#include "internal.h"

namespace dspark {

// ---------------------------------------------------------------------------
// Tiled path (larger M): the bound moves from HBM to MFMA (2MHV flops over
// 2VH bytes of W_lm).  Workgroup tile 256 (vocabulary) x 256 (rows of h), K in
// stages of 32, 4 waves in a 2 x 2 layout, each wave 128 x 128 as a 4 x 4 grid
// of v_mfma_f32_32x32x16_bf16 tiles (8 LDS operand reads feed 16 MFMAs of 32
// cycles).
//
// Operands move global -> LDS by DMA (global_load_lds_dwordx4: each wave
// instruction fills 1 KB of LDS in lane order) into a ring of 4 stages, so
// loads run 3 stages ahead of the MFMAs without staging registers.  A stage
// holds 256 rows x 64 bytes of W_lm and of h; LDS lines of 256 bytes hold four
// rows, and 16-byte chunk slots are XOR-swizzled by the line index, so that the
// DMA writes stay contiguous and the MFMA operand reads (16 consecutive rows
// per 16 lanes) touch every bank once.
//
// Tile order is XCD-aware: workgroup L runs on XCD L % 8, and the k-th
// workgroup of an XCD takes vocabulary tile 8 (k / MT) + L % 8 and row tile
// k % MT, so the MT row tiles that share one W_lm tile run back to back on the
// same XCD and reuse it from that XCD's L2 (W_lm is read from HBM about once).
constexpr int kGV = 256, kGM = 256, kGK = 32, kGStages = 4;
constexpr int kGStageBytes = (kGV + kGM) * kGK * 2;                 // 32 KB
constexpr size_t kGemmLds = static_cast<size_t>(kGStages) * kGStageBytes;

// LDS byte offset of (row, 16-byte chunk c < 4) inside one 256-row operand
// block: 256-byte lines of 4 rows, slots XOR-swizzled by the line index so that
// 16 consecutive rows at one chunk fall in 16 distinct 16-byte bank groups
// (64 banks of 4 bytes)
__device__ __forceinline__ int swz(int row, int c) {
  const int line = row >> 2;
  return line * 256 + ((((row & 3) << 2) | c) ^ (line & 3)) * 16;
}

template <int N>
__device__ __forceinline__ void wait_vmcnt() { asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory"); }

__global__ __launch_bounds__(256, 1) void lm_head_gemm_bf16(
    const uint16_t* __restrict__ h, const uint16_t* __restrict__ W, float* __restrict__ U,
    int M, int H, int V, int VT, int MT) {
  extern __shared__ __attribute__((aligned(1024))) unsigned char gsm[];
  const int L = blockIdx.x, kx = L >> 3;
  const int vt = (kx / MT) * 8 + (L & 7), mt = kx % MT;
  if (vt >= VT) return;                                 // whole workgroup
  const int v0 = vt * kGV, m0 = mt * kGM;
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int wv = w & 1, wm = w >> 1;
  const int l32 = lane & 31, hi = lane >> 5;
  const int nst = (H + kGK - 1) / kGK;

  // DMA issue for stage st: wave w fills 1 KB blocks w*4 .. w*4+3 of the W
  // operand block (instructions 0..3) and of the h block (4..7); lane i of an
  // instruction writes byte 16 i of its 1 KB, i.e. line 4 blk + i / 16 and slot
  // i % 16, and loads the (row, chunk) that the swizzle places there.
  auto issue = [&](int st) {
    unsigned char* base = gsm + (st % kGStages) * kGStageBytes;
#pragma unroll
    for (int q = 0; q < 8; ++q) {
      const bool isW = q < 4;
      const int line = (w * 4 + (q & 3)) * 4 + (lane >> 4);        // 0..63
      const int slot = (lane & 15) ^ (line & 3);
      const int row = 4 * line + (slot >> 2), c = slot & 3;
      const int k = st * kGK + 8 * c;
      const int gr = (isW ? v0 : m0) + row;
      const bool ok = st < nst && k < H && gr < (isW ? V : M);
      const uint16_t* src = ok ? (isW ? W : h) + static_cast<size_t>(gr) * H + k
                               : (isW ? W : h);                       // any valid address
      unsigned char* dst = base + (isW ? 0 : kGV * kGK * 2) + (w * 4 + (q & 3)) * 1024;
      __builtin_amdgcn_global_load_lds(src, reinterpret_cast<void*>(dst), 16, 0, 0);
      if (!ok) {}  // zero-fill below
    }
  };
  // rows past V / M and chunks past H must read as zero: the DMA above loads a
  // valid but unrelated address there, so such lanes patch their slot to zero
  // after the data has landed (only ragged edge tiles take this path)
  const bool edge = (v0 + kGV > V) || (m0 + kGM > M) || (H % kGK != 0);
  auto zero_fill = [&](int st) {
    unsigned char* base = gsm + (st % kGStages) * kGStageBytes;
#pragma unroll
    for (int q = 0; q < 8; ++q) {
      const bool isW = q < 4;
      const int line = (w * 4 + (q & 3)) * 4 + (lane >> 4);
      const int slot = (lane & 15) ^ (line & 3);
      const int row = 4 * line + (slot >> 2), c = slot & 3;
      const int k = st * kGK + 8 * c;
      const int gr = (isW ? v0 : m0) + row;
      if (!(k < H && gr < (isW ? V : M)))
        *reinterpret_cast<u32x4*>(base + (isW ? 0 : kGV * kGK * 2) + (w * 4 + (q & 3)) * 1024 + lane * 16) =
            u32x4{0u, 0u, 0u, 0u};
    }
  };

  f32x16 acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int jn = 0; jn < 4; ++jn)
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[i][jn][e] = 0.f;

  issue(0);
  issue(1);
  issue(2);
  for (int st = 0; st < nst; ++st) {
    // this wave's DMA for stage st has landed once at most the later stages'
    // 8 instructions each are outstanding
    if (st + 2 < nst) wait_vmcnt<16>();
    else if (st + 1 < nst) wait_vmcnt<8>();
    else wait_vmcnt<0>();
    if (edge) {
      zero_fill(st);
      asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
    }
    // every wave's part of stage st landed (each waited for its own DMA above);
    // stage st-1 fully consumed (its LDS reads fed MFMAs issued before this
    // point).  A bare barrier: a fenced one would also drain the DMA of the
    // stages still in flight.
    asm volatile("s_barrier" ::: "memory");
    if (st + 3 < nst) issue(st + 3);
    const unsigned char* wbase = gsm + (st % kGStages) * kGStageBytes;
    const unsigned char* hbase = wbase + kGV * kGK * 2;
#pragma unroll
    for (int ks = 0; ks < kGK / 16; ++ks) {
      u32x4 a[4], b[4];
#pragma unroll
      for (int i = 0; i < 4; ++i)
        a[i] = *reinterpret_cast<const u32x4*>(wbase + swz(wv * 128 + i * 32 + l32, 2 * ks + hi));
#pragma unroll
      for (int jn = 0; jn < 4; ++jn)
        b[jn] = *reinterpret_cast<const u32x4*>(hbase + swz(wm * 128 + jn * 32 + l32, 2 * ks + hi));
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int jn = 0; jn < 4; ++jn)
          acc[i][jn] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(a[i]), as_bf16x8(b[jn]),
                                                               acc[i][jn], 0, 0, 0);
    }
  }
  // D[row][col] of a 32x32 tile: lane holds rows 8 (e/4) + 4 hi + (e%4), column l32.
  // Rows are vocabulary entries, columns are rows of h: each group of 4
  // accumulators is one 16-byte store of 4 consecutive vocabulary entries.
#pragma unroll
  for (int i = 0; i < 4; ++i) {
#pragma unroll
    for (int jn = 0; jn < 4; ++jn) {
      const int m = m0 + wm * 128 + jn * 32 + l32;
      if (m >= M) continue;
#pragma unroll
      for (int e4 = 0; e4 < 4; ++e4) {
        const int v = v0 + wv * 128 + i * 32 + 8 * e4 + 4 * hi;
        if (v < V)
          *reinterpret_cast<f32x4*>(U + static_cast<size_t>(m) * V + v) =
              f32x4{acc[i][jn][4 * e4], acc[i][jn][4 * e4 + 1], acc[i][jn][4 * e4 + 2], acc[i][jn][4 * e4 + 3]};
      }
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

hipError_t launch_lm_head(const void* h, const void* w, bool bf16, int64_t M, int64_t H,
                          int64_t V, float* U, hipStream_t s) {
  if (!bf16) {
    const dim3 grid((V + 63) / 64, (M + 63) / 64);
    hipLaunchKernelGGL(lm_head_f32, grid, dim3(256), 0, s, static_cast<const float*>(h),
                       static_cast<const float*>(w), U, (int)M, (int)H, (int)V);
  } else if (lm_head_skinny_fits(M, H)) {
    return launch_lm_head_skinny(static_cast<const uint16_t*>(h), static_cast<const uint16_t*>(w), M, H, V, U, s);
  } else {
    const int VT = static_cast<int>((V + kGV - 1) / kGV), MT = static_cast<int>((M + kGM - 1) / kGM);
    const int grid = 8 * ((VT + 7) / 8) * MT;
    // opt in to more than 64 KB of dynamic LDS (a host-side attribute call)
    const hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(lm_head_gemm_bf16),
                                             hipFuncAttributeMaxDynamicSharedMemorySize,
                                             static_cast<int>(kGemmLds));
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(lm_head_gemm_bf16, dim3(grid), dim3(256), kGemmLds, s,
                       static_cast<const uint16_t*>(h), static_cast<const uint16_t*>(w), U, (int)M,
                       (int)H, (int)V, VT, MT);
  }
  return hipGetLastError();
}

}  // namespace dspark
