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
// stages of 64, 8 waves in a 2 (vocabulary) x 4 (rows) layout, each wave
// 128 x 64 as a 4 x 2 grid of v_mfma_f32_32x32x16_bf16 tiles.  128
// accumulators per wave leave room for two waves per SIMD, so one wave's waits
// hide under the other's MFMAs.
//
// Operands move global -> LDS by DMA (global_load_lds_dwordx4: each wave
// instruction fills 1 KB of LDS in lane order) into a ring of 2 stages of
// 64 KB.  A stage holds 256 rows x 128 bytes (one whole cache line per row) of
// W_lm and of h; LDS lines of 256 bytes hold two rows, and 16-byte chunk slots
// are XOR-swizzled by the line index mod 8, so that the DMA writes stay
// contiguous and the MFMA operand reads (16 consecutive rows per 16 lanes)
// touch every bank once.  The DMA of stage st + 2 is issued right after the
// barrier that ends stage st.
//
// Fragment reads are software-pipelined over two register sets: the reads of
// 16-deep step ks + 1 are in flight while the MFMAs of step ks run.  They are
// issued as inline-asm ds_read_b128 with explicit lgkmcnt waits, because the
// compiler counts the in-flight LDS DMA against lgkmcnt as well and would
// otherwise drain every outstanding read before each MFMA group.
//
// MFMA operands are (h rows, W_lm rows), so a lane holds one vocabulary column
// of the 32 x 32 tile and each dword store of 64 lanes writes two whole
// 128-byte rows of U.
//
// Tile order is XCD-aware: workgroup L runs on XCD L % 8, and the k-th
// workgroup of an XCD takes vocabulary tile 8 (k / MT) + L % 8 and row tile
// k % MT, so the MT row tiles that share one W_lm tile run back to back on the
// same XCD and reuse it from that XCD's L2 (W_lm is read from HBM about once).
constexpr int kGV = 256, kGM = 256, kGK = 64, kGThreads = 512;
constexpr int kGOpBytes = kGV * kGK * 2;                             // 32 KB
constexpr int kGStageBytes = 2 * kGOpBytes;                          // 64 KB
constexpr size_t kGemmLds = 2 * static_cast<size_t>(kGStageBytes);

// LDS byte offset of (row, 16-byte chunk c < 8) inside one 256-row operand
// block: 256-byte lines of 2 rows, slots XOR-swizzled by the line index so that
// 16 consecutive rows at one chunk fall in 16 distinct 16-byte bank groups
// (64 banks of 4 bytes).  Row + 32 adds exactly 4096 bytes.
__device__ __forceinline__ int swz(int row, int c) {
  const int line = row >> 1;
  return line * 256 + ((((row & 1) << 3) | c) ^ (line & 7)) * 16;
}

template <int N>
__device__ __forceinline__ void wait_vmcnt() { asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory"); }

__global__ __launch_bounds__(kGThreads, 1) void lm_head_gemm_bf16(
    const uint16_t* __restrict__ h, const uint16_t* __restrict__ W, float* __restrict__ U,
    int M, int H, int V, int VT, int MT) {
  extern __shared__ __attribute__((aligned(1024))) unsigned char gsm[];
  const int L = blockIdx.x, kx = L >> 3;
  const int vt = (kx / MT) * 8 + (L & 7), mt = kx % MT;
  if (vt >= VT) return;                                 // whole workgroup
  const int v0 = vt * kGV, m0 = mt * kGM;
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int wv = w & 1, wm = w >> 1;                    // 2 x 4 waves
  const int l32 = lane & 31, hi = lane >> 5;
  const int nst = (H + kGK - 1) / kGK;
  const int nfull = H / kGK;                            // stages with no K tail
  // output base, forced into registers before the main loop: a scalar load
  // left pending across the loop would also make its LDS waits full drains
  float* Ub = U + static_cast<size_t>(m0) * V + v0;
  asm volatile("" : "+s"(Ub));

  // DMA: wave w fills 1 KB blocks 4w .. 4w + 3 of the W_lm block (instructions
  // q = 0..3) and of the h block (q = 4..7).  Lane i of an instruction writes
  // byte 16 i of its block, i.e. line 4 blk + i / 16, slot i % 16, and loads the
  // (row, chunk) the swizzle places there.  Rows past V or M read the last
  // valid row (their outputs are never stored); H % 8 == 0, so every chunk is
  // whole, and chunks past H are clamped into the row and zeroed once landed.
  const uint16_t* rowp[8];
  int c8[8];
#pragma unroll
  for (int q = 0; q < 8; ++q) {
    const bool isW = q < 4;
    const int blk = w * 4 + (q & 3);
    const int line = blk * 4 + (lane >> 4);
    const int slot = (lane & 15) ^ (line & 7);
    const int row = line * 2 + (slot >> 3);
    const int gr = min((isW ? v0 : m0) + row, (isW ? V : M) - 1);
    rowp[q] = (isW ? W : h) + static_cast<size_t>(gr) * H;
    c8[q] = 8 * (slot & 7);
  }
  auto issue = [&](int st) {
    unsigned char* base = gsm + (st & 1) * kGStageBytes;
    const bool full = st < nfull;
#pragma unroll
    for (int q = 0; q < 8; ++q) {
      const int off = full ? st * kGK + c8[q] : min(st * kGK + c8[q], H - 8);
      unsigned char* dst = base + (q < 4 ? 0 : kGOpBytes) + (w * 4 + (q & 3)) * 1024;
      __builtin_amdgcn_global_load_lds(rowp[q] + off, reinterpret_cast<void*>(dst), 16, 0, 0);
    }
  };
  auto zero_tail = [&](int st) {
    if (st < nfull) return;
    unsigned char* base = gsm + (st & 1) * kGStageBytes;
#pragma unroll
    for (int q = 0; q < 8; ++q)
      if (st * kGK + c8[q] >= H)
        *reinterpret_cast<u32x4*>(base + (q < 4 ? 0 : kGOpBytes) + (w * 4 + (q & 3)) * 1024 + lane * 16) =
            u32x4{0u, 0u, 0u, 0u};
  };

  f32x16 acc[4][2];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int jn = 0; jn < 2; ++jn)
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[i][jn][e] = 0.f;

  // fragment registers, two sets: fa = 4 W_lm row groups, fb = 2 h row groups
  u32x4 fa[2][4], fb[2][2];
  const uint32_t lds0 = static_cast<uint32_t>(reinterpret_cast<uintptr_t>(gsm));
  uint32_t aw[4], ah[4];                                // per 16-deep step ks
#pragma unroll
  for (int ks = 0; ks < 4; ++ks) {
    aw[ks] = lds0 + swz(wv * 128 + l32, 2 * ks + hi);
    ah[ks] = lds0 + kGOpBytes + swz(wm * 64 + l32, 2 * ks + hi);
  }
  auto load_frag = [&](int set, uint32_t so, int ks) {
    const uint32_t pw = aw[ks] + so, ph = ah[ks] + so;
    asm volatile("ds_read_b128 %0, %1" : "=v"(fa[set][0]) : "v"(pw));
    asm volatile("ds_read_b128 %0, %1 offset:4096" : "=v"(fa[set][1]) : "v"(pw));
    asm volatile("ds_read_b128 %0, %1 offset:8192" : "=v"(fa[set][2]) : "v"(pw));
    asm volatile("ds_read_b128 %0, %1 offset:12288" : "=v"(fa[set][3]) : "v"(pw));
    asm volatile("ds_read_b128 %0, %1" : "=v"(fb[set][0]) : "v"(ph));
    asm volatile("ds_read_b128 %0, %1 offset:4096" : "=v"(fb[set][1]) : "v"(ph));
  };
  // at most N of this wave's LDS reads outstanding; the set's registers pass
  // through the wait so that its MFMAs cannot be scheduled above it
#define DSPARK_GEMM_WAIT_SET(set, n)                                                               \
  asm volatile("s_waitcnt lgkmcnt(%6)"                                                             \
               : "+v"(fa[set][0]), "+v"(fa[set][1]), "+v"(fa[set][2]), "+v"(fa[set][3]), "+v"(fb[set][0]), \
                 "+v"(fb[set][1])                                                                  \
               : "n"(n))
  auto mma = [&](int set) {
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int jn = 0; jn < 2; ++jn)
        acc[i][jn] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(fb[set][jn]), as_bf16x8(fa[set][i]),
                                                             acc[i][jn], 0, 0, 0);
  };

  issue(0);
  wait_vmcnt<0>();
  zero_tail(0);
  asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
  if (nst > 1) issue(1);
  load_frag(0, 0, 0);
  for (int st = 0; st < nst; ++st) {
    const uint32_t so = (st & 1) * kGStageBytes;
    load_frag(1, so, 1);
    DSPARK_GEMM_WAIT_SET(0, 6);
    mma(0);
    __builtin_amdgcn_sched_barrier(0);
    load_frag(0, so, 2);
    DSPARK_GEMM_WAIT_SET(1, 6);
    mma(1);
    __builtin_amdgcn_sched_barrier(0);
    load_frag(1, so, 3);
    DSPARK_GEMM_WAIT_SET(0, 6);
    mma(0);
    __builtin_amdgcn_sched_barrier(0);
    DSPARK_GEMM_WAIT_SET(1, 0);
    if (st + 1 < nst) {
      // this wave's DMA for st + 1 has landed and its reads of stage st are
      // done; past the barrier every wave's are, so stage st's slot is free
      wait_vmcnt<0>();
      zero_tail(st + 1);
      asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
      if (st + 2 < nst) issue(st + 2);
      load_frag(0, so ^ kGStageBytes, 0);
    }
    __builtin_amdgcn_sched_barrier(0);
    mma(1);
    __builtin_amdgcn_sched_barrier(0);
  }
#undef DSPARK_GEMM_WAIT_SET
  // D[m][v] of a 32 x 32 tile: lane column v = l32, rows 8 (e / 4) + 4 hi + e % 4
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int vr = wv * 128 + i * 32 + l32;
    if (v0 + vr >= V) continue;
#pragma unroll
    for (int jn = 0; jn < 2; ++jn)
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        const int mr = wm * 64 + jn * 32 + 8 * (e >> 2) + 4 * hi + (e & 3);
        if (m0 + mr < M) Ub[static_cast<size_t>(mr) * V + vr] = acc[i][jn][e];
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
    hipLaunchKernelGGL(lm_head_gemm_bf16, dim3(grid), dim3(kGThreads), kGemmLds, s,
                       static_cast<const uint16_t*>(h), static_cast<const uint16_t*>(w), U, (int)M,
                       (int)H, (int)V, VT, MT);
  }
  return hipGetLastError();
}

}  // namespace dspark
