// LM-head contraction for few rows (M <= 16): U[m, v] = sum_k h[m, k] W_lm[v, k].
// "DSpark 论文精读", §2.2: U_1..U_gamma = W_lm [h_1..h_gamma]; "DeepSpec 训练全流程详解",
// §4.3 compute_logits(block_hidden).
//
// HBM-bound on W_lm (2VH bytes against 2MHV flops).  The whole h (M rows,
// stride H + 8 to spread LDS banks) sits in LDS and feeds the B operand of
// v_mfma_f32_16x16x32_bf16 (column m = lane%16, zero for m >= M); each wave
// streams 16 vocabulary rows of W_lm into the A operand (row n = lane%16, 8
// consecutive k per lane group g = lane/16).
//
// Load pattern: every 16-byte load instruction covers whole 128-byte lines,
// 8 rows x 128 bytes (a wave reading 16 rows x 64 bytes per instruction
// requests each line twice and streams measurably slower).  For a chunk of 64
// k, load 0 reads rows 0-7 and load 1 rows 8-15, with the 8 16-byte pieces of
// a row's line spread as follows (lane (g, n), row r = n mod 8):
//   load 0: n < 8 -> piece g, n >= 8 -> piece 4 + g      (rows 0..7)
//   load 1: n < 8 -> piece 4 + g, n >= 8 -> piece g      (rows 8..15)
// Then the operand of k 0..31 (pieces 0..3) is load 0 in lanes n < 8 and load
// 1 in lanes n >= 8, and the operand of k 32..63 (pieces 4..7) the opposite
// select, which holds row n ^ 8 in lane n: that product goes to a second
// accumulator whose rows are permuted by 8, i.e. whose lane groups g and g ^ 2
// are exchanged; one lane swap per tile (lane ^ 32) realigns it.  The output
// tile D[v][m] leaves each lane 4 consecutive vocabulary entries of one row m:
// one 16-byte store.
//
// W_lm is read once per call, with non-temporal loads: they keep its 0.78 GB
// from displacing what the next kernels read from the last-level cache (the
// Markov tables and U), and the stream itself measured faster (140.6 -> 128.7
// us at V = 151936, H = 2560; the Markov chain after it 66.5 -> 61.1 us).
//
// h reaches LDS by DMA (global_load_lds) issued before the first W loads, and
// each wave waits only for those older operations (an explicit vmcnt and a
// bare s_barrier), so the W stream starts without waiting for h.
//
// With a confidence head (conf != NULL, the hidden-only head of
// "Qwen3.8-Flash-Next DSpark 训练实验", Confidence head, and "DSpark 论文精读",
// §3.1 prefix survival), workgroup 0 also computes c = sigmoid(w_c . h_m + b_c)
// for its M = B gamma rows of h, already in its LDS, and the running product
// per request, while its first W_lm batches are in flight: the whole S5 step
// costs no launch of its own.
#include "common.h"
#include "internal.h"

namespace dspark {

constexpr int kSkinnyWaves = 4;
constexpr int kSkinnyUnroll = 4;     // chunks of 64 k per batch (8 KB per wave)

// s_waitcnt vmcnt(N) as the compiler's own instruction (which its wait-count
// pass takes into account, unlike inline asm): simm16 holds vmcnt in bits
// 3:0 and 15:14, expcnt in 6:4 and lgkmcnt in 11:8 (the last two left at max)
template <int N>
__device__ __forceinline__ void wait_vmcnt_le() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
}

// The confidence head of the M rows in LDS (row m = b gamma + j), by the
// kSkinnyWaves waves of one workgroup: wave w reduces rows w, w + kSkinnyWaves,
// ... over 16-byte pieces of h (LDS) and w_c, then thread 0 runs the sigmoid
// and the running product in position order.
struct SkinnyConf {
  const uint16_t* w_c;
  float b_c;
  int gamma;
  float* conf;
  float* surv;
};

__device__ void skinny_confidence(const uint16_t* hs, int ld, int M, int H, const SkinnyConf& c, int w, int lane,
                                  float* part) {
  for (int m = w; m < M; m += kSkinnyWaves) {
    float acc = 0.f;
    for (int i = lane; i < H / 8; i += kWave) {
      const u32x4 x = *reinterpret_cast<const u32x4*>(hs + m * ld + 8 * i);
      const u32x4 y = *reinterpret_cast<const u32x4*>(c.w_c + 8 * i);
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        acc = fmaf(__uint_as_float(x[q] << 16), __uint_as_float(y[q] << 16), acc);
        acc = fmaf(__uint_as_float(x[q] & 0xFFFF0000u), __uint_as_float(y[q] & 0xFFFF0000u), acc);
      }
    }
    acc = wave_sum(acc);
    if (lane == 0) part[m] = acc;
  }
  __syncthreads();
  if (w == 0 && lane == 0) {
    for (int b = 0; b * c.gamma < M; ++b) {
      float run = 1.f;
      for (int j = 0; j < c.gamma; ++j) {
        const int m = b * c.gamma + j;
        const float cj = 1.0f / (1.0f + __expf(-(part[m] + c.b_c)));
        run *= cj;
        c.conf[m] = cj;
        c.surv[m] = run;
      }
    }
  }
}

// PIPE (H >= 512, at least one pair of batches): the pipelined form below;
// otherwise one chunk of 64 k at a time.
template <bool PIPE>
__global__ __launch_bounds__(kWave* kSkinnyWaves) void lm_head_skinny_bf16(
    const uint16_t* __restrict__ h, const uint16_t* __restrict__ W, float* __restrict__ U,
    int M, int H, int V, SkinnyConf cf) {
  __shared__ float cpart[16];
  extern __shared__ uint16_t hs[];  // [M][H + 8]
  const int ld = H + 8;
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int g = lane >> 4, n = lane & 15;
  const bool lo = n < 8;
  const bool hcol = n < M;
  // B-operand column m = n: lanes past the last row read row M - 1, so that
  // every LDS read is unconditional; they only feed output columns m >= M,
  // which are never stored
  const uint16_t* hrow = hs + min(n, M - 1) * ld;
  const int v0 = (blockIdx.x * kSkinnyWaves + w) * 16;

  // h rows into LDS by DMA: instruction i moves bytes [1024 q, 1024 q + 1024)
  // of row m (i = m * nq + q), lane l its 16 bytes l; the waves share them
  const int nq = (H * 2 + 1023) / 1024;
  for (int i = w; i < M * nq; i += kSkinnyWaves) {
    const int m = i / nq, q = i - m * nq;
    const int k = q * 512 + lane * 8;
    if (k < H)
      __builtin_amdgcn_global_load_lds(h + static_cast<size_t>(m) * H + k,
                                       reinterpret_cast<void*>(hs + m * ld + q * 512), 16, 0, 0);
  }

  const int r0 = v0 + (n & 7), r1 = v0 + 8 + (n & 7);
  const bool ok0 = r0 < V, ok1 = r1 < V;
  const uint16_t* w0 = W + static_cast<size_t>(ok0 ? r0 : 0) * H + (lo ? g : 4 + g) * 8;
  const uint16_t* w1 = W + static_cast<size_t>(ok1 ? r1 : 0) * H + (lo ? 4 + g : g) * 8;
  f32x4 acc = {0.f, 0.f, 0.f, 0.f};
  f32x4 acc8 = {0.f, 0.f, 0.f, 0.f};   // rows permuted by 8 (lane groups g <-> g ^ 2)

  auto chunk = [&](const u32x4& a0, const u32x4& a1, int k0) {
    u32x4 m0, m1;
#pragma unroll
    for (int d = 0; d < 4; ++d) {
      m0[d] = lo ? a0[d] : a1[d];
      m1[d] = lo ? a1[d] : a0[d];
    }
    const u32x4 hb0 = *reinterpret_cast<const u32x4*>(hrow + k0 + 8 * g);
    const u32x4 hb1 = *reinterpret_cast<const u32x4*>(hrow + k0 + 32 + 8 * g);
    acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(m0), as_bf16x8(hb0), acc, 0, 0, 0);
    acc8 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(m1), as_bf16x8(hb1), acc8, 0, 0, 0);
  };

  // Pairs of batches of kSkinnyUnroll chunks, software-pipelined over two
  // register sets: the loads of one batch are in flight while the other is
  // computed.  Both batches of the first pair are issued before the wait for
  // h, so that 16 KB per wave is in flight while h lands; the last pair is
  // peeled, so no load reaches past the rows' end.  Every load is
  // unconditional (the compiler's wait counts stay exact): rows past V read
  // row 0, whose outputs are never stored.  Chunks past the last pair take the
  // plain loop below.
  const int npairs = (H / 64) / (2 * kSkinnyUnroll);
  u32x4 x0[kSkinnyUnroll], x1[kSkinnyUnroll], y0[kSkinnyUnroll], y1[kSkinnyUnroll];
  auto issue = [&](u32x4 (&b0)[kSkinnyUnroll], u32x4 (&b1)[kSkinnyUnroll], int bt) {
#pragma unroll
    for (int u = 0; u < kSkinnyUnroll; ++u) {
      b0[u] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(w0 + (bt * kSkinnyUnroll + u) * 64));
      b1[u] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(w1 + (bt * kSkinnyUnroll + u) * 64));
    }
  };
  auto compute = [&](const u32x4 (&b0)[kSkinnyUnroll], const u32x4 (&b1)[kSkinnyUnroll], int bt) {
#pragma unroll
    for (int u = 0; u < kSkinnyUnroll; ++u) chunk(b0[u], b1[u], (bt * kSkinnyUnroll + u) * 64);
  };
  if constexpr (PIPE) {
    issue(x0, x1, 0);
    __builtin_amdgcn_sched_barrier(0);
    issue(y0, y1, 1);
    __builtin_amdgcn_sched_barrier(0);
    wait_vmcnt_le<4 * kSkinnyUnroll>();           // this wave's h DMA (older) has landed
  } else {
    wait_vmcnt_le<0>();
  }
  asm volatile("s_barrier" ::: "memory");          // every wave's h DMA has landed
  if (cf.conf && blockIdx.x == 0) skinny_confidence(hs, ld, M, H, cf, w, lane, cpart);   // uniform per workgroup
  // (waves past V run to the end on row 0 and store nothing: an early exit
  // would let the compiler sink the first batches below it)
  if constexpr (PIPE) {                            // npairs >= 1: the batches above are used
    // the scheduling barriers keep each batch's loads ahead of the other
    // batch's arithmetic (the LDS reads of h are free to move, and would
    // otherwise take the loads with them)
    for (int p = 0; p + 1 < npairs; ++p) {
      compute(x0, x1, 2 * p);
      __builtin_amdgcn_sched_barrier(0);
      issue(x0, x1, 2 * p + 2);
      __builtin_amdgcn_sched_barrier(0);
      compute(y0, y1, 2 * p + 1);
      __builtin_amdgcn_sched_barrier(0);
      issue(y0, y1, 2 * p + 3);
      __builtin_amdgcn_sched_barrier(0);
    }
    compute(x0, x1, 2 * npairs - 2);
    compute(y0, y1, 2 * npairs - 1);
  }
  for (int kc = PIPE ? 2 * npairs * kSkinnyUnroll : 0; kc < H / 64; ++kc) {
    const u32x4 a0 = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(w0 + kc * 64));
    const u32x4 a1 = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(w1 + kc * 64));
    chunk(a0, a1, kc * 64);
  }
  // k beyond the last full chunk of 64 (H % 64, a multiple of 8): 32-wide
  // chunks in the plain layout, lane (g, n) = row n, k = 8g
  const int vr = v0 + n;
  const bool vok = vr < V;
  for (int k0 = (H / 64) * 64; k0 < H; k0 += 32) {
    const int k = k0 + 8 * g;
    const bool kok = k < H;
    const u32x4 wa = (vok && kok) ? *reinterpret_cast<const u32x4*>(W + static_cast<size_t>(vr) * H + k)
                                  : u32x4{0u, 0u, 0u, 0u};
    const u32x4 hb = kok ? *reinterpret_cast<const u32x4*>(hrow + k) : u32x4{0u, 0u, 0u, 0u};
    acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(wa), as_bf16x8(hb), acc, 0, 0, 0);
  }
#pragma unroll
  for (int i = 0; i < 4; ++i) acc[i] += __shfl_xor(acc8[i], 32);
  // D[4g + i][n] = U[m = n][v0 + 4g + i]
  const int vo = v0 + 4 * g;
  if (hcol && vo < V) *reinterpret_cast<f32x4*>(U + static_cast<size_t>(n) * V + vo) = acc;
}

size_t lm_head_skinny_lds(int64_t M, int64_t H) { return static_cast<size_t>(M) * (H + 8) * 2; }

bool lm_head_skinny_fits(int64_t M, int64_t H) { return M <= 16 && lm_head_skinny_lds(M, H) <= kSkinnyMaxLds; }

hipError_t launch_lm_head_skinny(const uint16_t* h, const uint16_t* w, int64_t M, int64_t H, int64_t V,
                                 float* U, hipStream_t s, const uint16_t* w_c, float b_c, int gamma, float* conf,
                                 float* surv) {
  const SkinnyConf cf{w_c, b_c, gamma, conf, surv};
  const int64_t tiles = (V + 15) / 16;
  const dim3 grid(static_cast<unsigned>((tiles + kSkinnyWaves - 1) / kSkinnyWaves));
  if (H >= 128 * kSkinnyUnroll)
    hipLaunchKernelGGL(lm_head_skinny_bf16<true>, grid, dim3(kWave * kSkinnyWaves), lm_head_skinny_lds(M, H), s, h,
                       w, U, static_cast<int>(M), static_cast<int>(H), static_cast<int>(V), cf);
  else
    hipLaunchKernelGGL(lm_head_skinny_bf16<false>, grid, dim3(kWave * kSkinnyWaves), lm_head_skinny_lds(M, H), s,
                       h, w, U, static_cast<int>(M), static_cast<int>(H), static_cast<int>(V), cf);
  return hipGetLastError();
}

}  // namespace dspark
