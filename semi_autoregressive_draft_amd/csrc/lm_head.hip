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
// 2VH bytes of W_lm).  Workgroup tile 320 (vocabulary) x 256 (rows of h), K in
// stages of 64, 8 waves in a 2 (vocabulary) x 4 (rows) layout, each wave
// 160 x 64 as a 5 x 2 grid of v_mfma_f32_32x32x16_bf16 tiles.  160
// accumulators per wave leave room for two waves per SIMD, so one wave's waits
// hide under the other's MFMAs.  (A 320-wide tile moves 10% fewer operand
// bytes per output than a square 256 one, and 475 x 7 tiles at V = 151936,
// M = 1792 fill 13 whole rounds of the 256 CUs.)
//
// Operands move global -> LDS by DMA (buffer_load_dwordx4 ... lds: each wave
// instruction fills 1 KB of LDS in lane order) into a ring of 2 stages of
// 72 KB.  A stage holds 320 rows of W_lm and 256 rows of h, 128 bytes (one
// whole cache line) per row; LDS lines of 256 bytes hold two rows, and 16-byte
// chunk slots are XOR-swizzled by the line index mod 8, so that the DMA writes
// stay contiguous and the MFMA operand reads (16 consecutive rows per 16
// lanes) touch every bank once.  The DMA goes through buffer resources over
// the tile's valid rows: a lane's offset is one of two per-lane values (even
// and odd blocks) plus a uniform block and stage offset, and rows past V or M
// read 0 (their outputs are never stored).
//
// A wave cannot issue past a DMA instruction until the memory pipeline takes
// it, and a stage's 72 KB drain at the L2's pace (~1 KB per 20-35 cycles per
// CU).  So waves 0-3 issue every DMA instruction of their SIMD (their own
// blocks and those of wave w + 4), while waves 4-7 run their MFMAs from the
// barrier on; the W_lm rows of stage st + 2 go out right after the barrier
// that ends stage st, its h rows two MFMA groups into stage st + 1.  (With
// every wave issuing its own 9 instructions after the barrier, the second
// wave of each SIMD reached the barrier ~1,500 cycles after the first, and a
// stage took ~4,400 cycles for 2,560 cycles of MFMA work per SIMD; split this
// way it takes ~3,250.)
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
// Tile order is XCD-aware: the tiles, row tile fastest, are cut into 8
// contiguous runs whose lengths differ by at most one; workgroup L runs on XCD
// L % 8 and takes tile L / 8 of run L % 8.  The MT row tiles that share one
// W_lm tile thus run back to back on one XCD and reuse it from that XCD's L2
// (W_lm is read from HBM about once), and no XCD has a round more than another.
constexpr int kGNI = 5;                                                // 32-column MFMA tiles per wave
constexpr int kGV = 64 * kGNI, kGM = 256, kGK = 64, kGThreads = 512;
constexpr int kGWBytes = kGV * kGK * 2;                                // 40 KB
constexpr int kGHBytes = kGM * kGK * 2;                                // 32 KB
constexpr int kGStageBytes = kGWBytes + kGHBytes;                      // 72 KB
constexpr size_t kGemmLds = 2 * static_cast<size_t>(kGStageBytes);
constexpr int kGDma = kGNI + 4;                                        // DMA instructions per wave and stage

// LDS byte offset of (row, 16-byte chunk c < 8) inside one operand block:
// 256-byte lines of 2 rows, slots XOR-swizzled by the line index so that 16
// consecutive rows at one chunk fall in 16 distinct 16-byte bank groups (64
// banks of 4 bytes).  Row + 32 adds exactly 4096 bytes.
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
  const int L = blockIdx.x, x = L & 7;
  const int T = VT * MT;
  const int s0 = static_cast<int>((static_cast<long long>(x) * T) >> 3);
  const int s1 = static_cast<int>((static_cast<long long>(x + 1) * T) >> 3);
  const int tile = s0 + (L >> 3);
  if (tile >= s1) return;                               // whole workgroup
  const int vt = tile / MT, mt = tile - vt * MT;
  const int v0 = vt * kGV, m0 = mt * kGM;
  const int tid = threadIdx.x, lane = tid & 63, w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wv = w & 1, wm = w >> 1;                    // 2 x 4 waves
  const int l32 = lane & 31, hi = lane >> 5;
  const int nst = (H + kGK - 1) / kGK;
  const int nfull = H / kGK;                            // stages with no K tail
  // output base, forced into registers before the main loop: a scalar load
  // left pending across the loop would also make its LDS waits full drains
  float* Ub = U + static_cast<size_t>(m0) * V + v0;
  asm volatile("" : "+s"(Ub));
  // the tile's first rows of W_lm and h: the DMA offsets below are relative
  // to them (at most 320 rows, so 32 bits hold them)
  const uint16_t* const Wt = W + static_cast<size_t>(v0) * H;
  const uint16_t* const ht = h + static_cast<size_t>(m0) * H;
  const __amdgpu_buffer_rsrc_t rw = buf_rsrc(Wt, static_cast<size_t>(min(kGV, V - v0)) * H * 2);
  const __amdgpu_buffer_rsrc_t rh = buf_rsrc(ht, static_cast<size_t>(min(kGM, M - m0)) * H * 2);

  // DMA: block b (1 KB) of the W_lm or h part of a stage holds rows
  // 8b .. 8b + 7.  Lane i of its instruction writes byte 16 i of the block,
  // i.e. line 4b + i / 16, slot i % 16, and loads the (row, chunk) the swizzle
  // places there: row 8b + 2 (i / 16) + slot' / 8 and chunk slot' % 8 with
  // slot' = (i % 16) ^ (line % 8), where line % 8 depends on b only through
  // b % 2.  H % 8 == 0, so every chunk is whole; in a stage with a K tail,
  // chunks past H are clamped into the row and zeroed once landed.
  uint32_t vo[2];                                       // byte offset in an even / odd block
  int c8[2];                                            // its first column in the stage
#pragma unroll
  for (int p = 0; p < 2; ++p) {
    const int line = 4 * p + (lane >> 4);
    const int slot = (lane & 15) ^ (line & 7);
    c8[p] = 8 * (slot & 7);
    vo[p] = static_cast<uint32_t>(((2 * (lane >> 4) + (slot >> 3)) * H + c8[p]) * 2);
  }
  // the lane's byte offset of stage st in a block of parity p
  auto stage_ofs = [&](int st, int p) __attribute__((always_inline)) {
    const int k = st < nfull ? st * kGK : min(st * kGK + c8[p], H - 8) - c8[p];
    return vo[p] + static_cast<uint32_t>(k * 2);
  };
  auto dma = [&](unsigned char* base, bool isW, int blk, uint32_t ofs) __attribute__((always_inline)) {
    __builtin_amdgcn_raw_ptr_buffer_load_lds(
        isW ? rw : rh, (__attribute__((address_space(3))) void*)(base + (isW ? 0 : kGWBytes) + blk * 1024), 16,
        ofs + static_cast<uint32_t>(16 * blk * H), 0, 0, 0);
  };
  // waves 0-3 only: the blocks of wave w and of wave w + 4 (same parity)
  auto issue_w = [&](int st) __attribute__((always_inline)) {
    if (w >= 4) return;
    unsigned char* base = gsm + (st & 1) * kGStageBytes;
    const uint32_t o0 = stage_ofs(st, 0), o1 = stage_ofs(st, 1);
    const uint32_t oe = (w & 1) ? o1 : o0, od = (w & 1) ? o0 : o1;   // block w kGNI + q: parity (w + q) % 2
#pragma unroll
    for (int q = 0; q < kGNI; ++q) dma(base, true, w * kGNI + q, q & 1 ? od : oe);
#pragma unroll
    for (int q = 0; q < kGNI; ++q) dma(base, true, (w + 4) * kGNI + q, q & 1 ? od : oe);
  };
  auto issue_h = [&](int st) __attribute__((always_inline)) {
    if (w >= 4) return;
    unsigned char* base = gsm + (st & 1) * kGStageBytes;
    const uint32_t o0 = stage_ofs(st, 0), o1 = stage_ofs(st, 1);  // block 4 w + q: parity q % 2
#pragma unroll
    for (int q = 0; q < 4; ++q) dma(base, false, w * 4 + q, q & 1 ? o1 : o0);
#pragma unroll
    for (int q = 0; q < 4; ++q) dma(base, false, (w + 4) * 4 + q, q & 1 ? o1 : o0);
  };
  auto zero_tail = [&](int st) __attribute__((always_inline)) {
    if (st < nfull || w >= 4) return;
    unsigned char* base = gsm + (st & 1) * kGStageBytes;
    const u32x4 z = {0u, 0u, 0u, 0u};
#pragma unroll
    for (int q = 0; q < kGNI; ++q) {
      const int b0 = w * kGNI + q, b1 = b0 + 4 * kGNI;    // same parity
      if (st * kGK + c8[b0 & 1] >= H) {
        *reinterpret_cast<u32x4*>(base + b0 * 1024 + lane * 16) = z;
        *reinterpret_cast<u32x4*>(base + b1 * 1024 + lane * 16) = z;
      }
    }
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int b0 = w * 4 + q, b1 = b0 + 16;
      if (st * kGK + c8[b0 & 1] >= H) {
        *reinterpret_cast<u32x4*>(base + kGWBytes + b0 * 1024 + lane * 16) = z;
        *reinterpret_cast<u32x4*>(base + kGWBytes + b1 * 1024 + lane * 16) = z;
      }
    }
  };

  f32x16 acc[kGNI][2];
#pragma unroll
  for (int i = 0; i < kGNI; ++i)
#pragma unroll
    for (int jn = 0; jn < 2; ++jn)
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[i][jn][e] = 0.f;

  // fragment registers, two sets: fa = 5 W_lm row groups, fb = 2 h row groups
  u32x4 fa[2][kGNI], fb[2][2];
  const uint32_t lds0 = static_cast<uint32_t>(reinterpret_cast<uintptr_t>(gsm));
  // per 16-deep step ks; the h rows sit a wave-uniform distance from the W_lm
  // rows (both first rows are multiples of 16, so the swizzle is the same)
  uint32_t aw[4];
#pragma unroll
  for (int ks = 0; ks < 4; ++ks) aw[ks] = lds0 + swz(wv * 32 * kGNI + l32, 2 * ks + hi);
  const uint32_t dh = __builtin_amdgcn_readfirstlane(kGWBytes + swz(wm * 64, 0) - swz(wv * 32 * kGNI, 0));
  auto load_frag = [&](int set, uint32_t so, int ks) __attribute__((always_inline)) {
    const uint32_t pw = aw[ks] + so, ph = pw + dh;
    asm volatile("ds_read_b128 %0, %1" : "=v"(fa[set][0]) : "v"(pw));
    asm volatile("ds_read_b128 %0, %1 offset:4096" : "=v"(fa[set][1]) : "v"(pw));
    asm volatile("ds_read_b128 %0, %1 offset:8192" : "=v"(fa[set][2]) : "v"(pw));
    asm volatile("ds_read_b128 %0, %1 offset:12288" : "=v"(fa[set][3]) : "v"(pw));
    asm volatile("ds_read_b128 %0, %1 offset:16384" : "=v"(fa[set][4]) : "v"(pw));
    asm volatile("ds_read_b128 %0, %1" : "=v"(fb[set][0]) : "v"(ph));
    asm volatile("ds_read_b128 %0, %1 offset:4096" : "=v"(fb[set][1]) : "v"(ph));
  };
  // at most N of this wave's LDS reads outstanding; the set's registers pass
  // through the wait so that its MFMAs cannot be scheduled above it
#define DSPARK_GEMM_WAIT_SET(set, n)                                                               \
  asm volatile("s_waitcnt lgkmcnt(%7)"                                                             \
               : "+v"(fa[set][0]), "+v"(fa[set][1]), "+v"(fa[set][2]), "+v"(fa[set][3]), "+v"(fa[set][4]), \
                 "+v"(fb[set][0]), "+v"(fb[set][1])                                                \
               : "n"(n))
  auto mma = [&](int set) __attribute__((always_inline)) {
#pragma unroll
    for (int i = 0; i < kGNI; ++i)
#pragma unroll
      for (int jn = 0; jn < 2; ++jn)
        acc[i][jn] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(fb[set][jn]), as_bf16x8(fa[set][i]),
                                                             acc[i][jn], 0, 0, 0);
  };

  issue_w(0);
  issue_h(0);
  wait_vmcnt<0>();
  zero_tail(0);
  asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
  if (nst > 1) {
    issue_w(1);
    issue_h(1);
  }
  load_frag(0, 0, 0);
  for (int st = 0; st < nst; ++st) {
    const uint32_t so = (st & 1) * kGStageBytes;
    load_frag(1, so, 1);
    DSPARK_GEMM_WAIT_SET(0, kGNI + 2);
    mma(0);
    __builtin_amdgcn_sched_barrier(0);
    load_frag(0, so, 2);
    DSPARK_GEMM_WAIT_SET(1, kGNI + 2);
    mma(1);
    __builtin_amdgcn_sched_barrier(0);
    // the h rows of stage st + 1 (its W_lm rows went out after the last barrier)
    if (st >= 1 && st + 1 < nst) issue_h(st + 1);
    load_frag(1, so, 3);
    DSPARK_GEMM_WAIT_SET(0, kGNI + 2);
    mma(0);
    __builtin_amdgcn_sched_barrier(0);
    DSPARK_GEMM_WAIT_SET(1, 0);
    if (st + 1 < nst) {
      // this wave's DMA for st + 1 has landed and its reads of stage st are
      // done; past the barrier every wave's are, so stage st's slot is free
      wait_vmcnt<0>();
      zero_tail(st + 1);
      asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
      if (st + 2 < nst) issue_w(st + 2);
      load_frag(0, so ^ kGStageBytes, 0);
    }
    __builtin_amdgcn_sched_barrier(0);
    mma(1);
    __builtin_amdgcn_sched_barrier(0);
  }
#undef DSPARK_GEMM_WAIT_SET
  // D[m][v] of a 32 x 32 tile: lane column v = l32, rows 8 (e / 4) + 4 hi + e % 4.
  // The stores carry the non-temporal hint: U is far larger than the caches and
  // is read back row by row much later, so its lines are not kept where the
  // row tiles share their W_lm tiles in L2 or where the Markov step keeps Bm
  // (measured at B = 256: GEMM 1258 -> 1235 us, Markov stage 524 -> 512 us).
#pragma unroll
  for (int i = 0; i < kGNI; ++i) {
    const int vr = wv * 32 * kGNI + i * 32 + l32;
    if (v0 + vr >= V) continue;
#pragma unroll
    for (int jn = 0; jn < 2; ++jn)
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        const int mr = wm * 64 + jn * 32 + 8 * (e >> 2) + 4 * hi + (e & 3);
        if (m0 + mr < M) __builtin_nontemporal_store(acc[i][jn][e], &Ub[static_cast<size_t>(mr) * V + vr]);
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
    const int grid = 8 * ((VT * MT + 7) / 8);
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
