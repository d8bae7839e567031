// Sequential Vanilla-Markov stage of the DSpark draft proposal.
//
// Per position j (the sequential dependency), for every request b:
//   U~_j[v] = U[b, j, v] + sum_k A[x_{j-1}, k] * Bm[k, v]      (x_{-1} = anchor)
//   x_j     = argmax_v U~_j[v]                 (temperature 0)
//           = argmax_v U~_j[v] / T + G[b,j,v]  (Gumbel-max sampling)
//   lse_j   = log sum_v exp U~_j[v]
// "Qwen3.8-Flash-Next DSpark 训练实验", Baseline 架构/Markov 顺序修正
// (m_i = W_1[t_{i-1}], b_i = W_2 m_i, l_i = l_i^0 + b_i); "DSpark 论文精读", §2.2
// (U~_j = U_j + b(x_{j-1}), x_j ~ softmax(U~_j)).
//
// One position is two launches: a step kernel that streams Bm and U_j once
// for all requests and leaves one partial (max, sum-exp, best score/index) per
// (request, vocabulary tile), and a merge kernel with one workgroup per
// request that combines the partials in a fixed order and writes x_j (plus the
// top-k candidate set when asked).  The merge of position j is what position
// j+1's step kernel reads as its previous token.
#include "common.h"
#include "internal.h"

namespace dspark {

// ---------------------------------------------------------------------------
// bf16 step kernel: the bias m . Bm runs on MFMA (v_mfma_f32_16x16x32_bf16).
//
// A wave owns a tile of 16*RG requests x 128 vocabulary columns.  Lane
// (g = lane/16, n = lane%16) loads, for 8 consecutive rows k of Bm, the 8
// consecutive columns v0+8n .. v0+8n+7 (16-byte loads, 256 contiguous bytes per
// 16 lanes), and transposes that 8x8 bf16 block in registers (v_perm) into the
// eight B operands "column v0+8n+c, rows k..k+7".  The A operand is row n of
// the gathered A[x_{j-1}] block.  After the r-loop, lane (g, n) holds requests
// 4g..4g+3 of each 16-request group for the 8 consecutive columns v0+8n+c, so
// its U row reads are 32 contiguous bytes.  KS waves of a workgroup split r
// and add their accumulators through LDS in a fixed order.
constexpr int kMarkovTile = 128;   // vocabulary columns per bf16 step tile
constexpr int kMarkovTileF32 = 256;
constexpr int kSeg = 32;           // vocabulary columns per top-k segment

template <int RG, int KS>
__global__ __launch_bounds__(kWave* KS) void markov_step_bf16(StepArgs a) {
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int g = lane >> 4, n = lane & 15;
  const int tile = blockIdx.x;
  const int vcol = tile * kMarkovTile + 8 * n;
  const bool vok = vcol < a.V;
  const int req0 = blockIdx.y * (16 * RG);

  const uint16_t* A = static_cast<const uint16_t*>(a.A);
  const uint16_t* Bm = static_cast<const uint16_t*>(a.Bm);

  const uint16_t* arow[RG];
  bool bok[RG];
#pragma unroll
  for (int rg = 0; rg < RG; ++rg) {
    const int b = req0 + 16 * rg + n;
    bok[rg] = b < a.B;
    const int prev = !bok[rg] ? 0 : (a.j == 0 ? a.anchor[b] : a.tokens[b * a.gamma + a.j - 1]);
    arow[rg] = A + static_cast<size_t>(prev) * a.r;
  }

  f32x4 acc[RG][8];
#pragma unroll
  for (int rg = 0; rg < RG; ++rg)
#pragma unroll
    for (int c = 0; c < 8; ++c) acc[rg][c] = f32x4{0.f, 0.f, 0.f, 0.f};

  const int kper = a.r / KS;
  const int kbeg = w * kper;
  const uint16_t* bcol = Bm + vcol;
  const size_t V = static_cast<size_t>(a.V);
  for (int kc = kbeg; kc < kbeg + kper; kc += 32) {
    const int k = kc + 8 * g;
    u32x4 rows[8];
#pragma unroll
    for (int i = 0; i < 8; ++i)
      rows[i] = vok ? *reinterpret_cast<const u32x4*>(bcol + static_cast<size_t>(k + i) * V)
                    : u32x4{0u, 0u, 0u, 0u};
    u32x4 bop[8];
#pragma unroll
    for (int c = 0; c < 8; ++c) {
      const uint32_t sel = (c & 1) ? 0x07060302u : 0x05040100u;
#pragma unroll
      for (int p = 0; p < 4; ++p)
        bop[c][p] = __builtin_amdgcn_perm(rows[2 * p + 1][c >> 1], rows[2 * p][c >> 1], sel);
    }
#pragma unroll
    for (int rg = 0; rg < RG; ++rg) {
      const u32x4 av = bok[rg] ? *reinterpret_cast<const u32x4*>(arow[rg] + k)
                               : u32x4{0u, 0u, 0u, 0u};
#pragma unroll
      for (int c = 0; c < 8; ++c)
        acc[rg][c] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(av), as_bf16x8(bop[c]),
                                                             acc[rg][c], 0, 0, 0);
    }
  }

  if constexpr (KS > 1) {
    __shared__ f32x4 red[KS - 1][RG][8][kWave];
    if (w > 0) {
#pragma unroll
      for (int rg = 0; rg < RG; ++rg)
#pragma unroll
        for (int c = 0; c < 8; ++c) red[w - 1][rg][c][lane] = acc[rg][c];
    }
    __syncthreads();
    if (w != 0) return;
#pragma unroll
    for (int s = 0; s < KS - 1; ++s)
#pragma unroll
      for (int rg = 0; rg < RG; ++rg)
#pragma unroll
        for (int c = 0; c < 8; ++c) acc[rg][c] += red[s][rg][c][lane];
  }

  // ---- epilogue (wave 0): add U_j, sample noise, local stats, partials ----
  const int P = a.P;
#pragma unroll
  for (int rg = 0; rg < RG; ++rg) {
#pragma unroll
    for (int ii = 0; ii < 4; ++ii) {
      const int b = req0 + 16 * rg + 4 * g + ii;
      const bool live = (b < a.B) && vok;
      float x[8];
      if (live) {
        const float* urow = a.U + (static_cast<size_t>(b) * a.gamma + a.j) * V + vcol;
        const f32x4 u0 = *reinterpret_cast<const f32x4*>(urow);
        const f32x4 u1 = *reinterpret_cast<const f32x4*>(urow + 4);
#pragma unroll
        for (int c = 0; c < 4; ++c) {
          x[c] = acc[rg][c][ii] + u0[c];
          x[c + 4] = acc[rg][c + 4][ii] + u1[c];
        }
        if (a.logits_out) {
          float* orow = a.logits_out + (static_cast<size_t>(b) * a.gamma + a.j) * V + vcol;
          *reinterpret_cast<f32x4*>(orow) = f32x4{x[0], x[1], x[2], x[3]};
          *reinterpret_cast<f32x4*>(orow + 4) = f32x4{x[4], x[5], x[6], x[7]};
        }
      } else {
#pragma unroll
        for (int c = 0; c < 8; ++c) x[c] = kNegInf;
      }
      float m8 = x[0];
#pragma unroll
      for (int c = 1; c < 8; ++c) m8 = fmaxf(m8, x[c]);
      float s8 = 0.f;
      if (live) {
#pragma unroll
        for (int c = 0; c < 8; ++c) s8 += __expf(x[c] - m8);
      }
      LseState ls{m8, s8};

      float score[8];
      if (a.sample && live) {
        const uint64_t sd = a.seeds[b];
        const uint32_t k0 = static_cast<uint32_t>(sd), k1 = static_cast<uint32_t>(sd >> 32);
        const Philox4 r0 = philox4x32_10(vcol >> 2, a.j, a.off_lo, a.off_hi, k0, k1);
        const Philox4 r1 = philox4x32_10((vcol >> 2) + 1, a.j, a.off_lo, a.off_hi, k0, k1);
        const uint32_t wd[8] = {r0.x, r0.y, r0.z, r0.w, r1.x, r1.y, r1.z, r1.w};
#pragma unroll
        for (int c = 0; c < 8; ++c) score[c] = x[c] * a.inv_temp + gumbel_from_word(wd[c]);
      } else {
#pragma unroll
        for (int c = 0; c < 8; ++c) score[c] = x[c];
      }
      ArgState as{score[0], live ? vcol : 0x7fffffff, x[0]};
#pragma unroll
      for (int c = 1; c < 8; ++c)
        if (score[c] > as.score) as = ArgState{score[c], vcol + c, x[c]};

      if (a.segmax) {  // max over 32 consecutive columns = 4 neighbouring lanes
        float sm = fmaxf(m8, __shfl_xor(m8, 1));
        sm = fmaxf(sm, __shfl_xor(sm, 2));
        if ((n & 3) == 0 && live) a.segmax[static_cast<size_t>(b) * a.S + vcol / kSeg] = sm;
      }
#pragma unroll
      for (int o = 1; o < 16; o <<= 1) {
        ls = lse_merge(ls, shfl_xor(ls, o));
        as = arg_merge(as, shfl_xor(as, o));
      }
      if (n == 0 && b < a.B) {
        const size_t q = static_cast<size_t>(b) * P + tile;
        a.p_m[q] = ls.m;
        a.p_s[q] = ls.s;
        a.p_score[q] = as.score;
        a.p_idx[q] = as.idx;
        a.p_x[q] = as.x;
      }
    }
  }
}

// ---------------------------------------------------------------------------
// float32 step kernel (any rank, any V): one thread per (request, column),
// the bias as a plain dot product over the gathered A row held in LDS.
__global__ __launch_bounds__(256) void markov_step_f32(StepArgs a) {
  __shared__ float arow[kMaxRank];
  __shared__ LseState red_l[4];
  __shared__ ArgState red_a[4];
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int tile = blockIdx.x, b = blockIdx.y;
  const float* A = static_cast<const float*>(a.A);
  const float* Bm = static_cast<const float*>(a.Bm);
  const int prev = a.j == 0 ? a.anchor[b] : a.tokens[b * a.gamma + a.j - 1];
  for (int k = tid; k < a.r; k += 256) arow[k] = A[static_cast<size_t>(prev) * a.r + k];
  __syncthreads();

  const int v = tile * kMarkovTileF32 + tid;
  const bool live = v < a.V;
  const size_t V = static_cast<size_t>(a.V);
  float x = kNegInf, score = kNegInf;
  if (live) {
    float bias = 0.f;
    for (int k = 0; k < a.r; ++k) bias = fmaf(arow[k], Bm[static_cast<size_t>(k) * V + v], bias);
    const size_t row = static_cast<size_t>(b) * a.gamma + a.j;
    x = a.U[row * V + v] + bias;
    if (a.logits_out) a.logits_out[row * V + v] = x;
    score = x;
    if (a.sample) {
      const uint64_t sd = a.seeds[b];
      const Philox4 r = philox4x32_10(v >> 2, a.j, a.off_lo, a.off_hi, static_cast<uint32_t>(sd),
                                      static_cast<uint32_t>(sd >> 32));
      const uint32_t wd = (v & 3) == 0 ? r.x : (v & 3) == 1 ? r.y : (v & 3) == 2 ? r.z : r.w;
      score = x * a.inv_temp + gumbel_from_word(wd);
    }
  }
  if (a.segmax) {
    float sm = x;
#pragma unroll
    for (int o = 1; o < kSeg; o <<= 1) sm = fmaxf(sm, __shfl_xor(sm, o));
    if ((lane & (kSeg - 1)) == 0 && live) a.segmax[static_cast<size_t>(b) * a.S + v / kSeg] = sm;
  }
  LseState ls{x, live ? 1.0f : 0.0f};
  ArgState as{score, live ? v : 0x7fffffff, x};
#pragma unroll
  for (int o = 1; o < kWave; o <<= 1) {
    ls = lse_merge(ls, shfl_xor(ls, o));
    as = arg_merge(as, shfl_xor(as, o));
  }
  if (lane == 0) { red_l[w] = ls; red_a[w] = as; }
  __syncthreads();
  if (tid == 0) {
    for (int i = 1; i < 4; ++i) { ls = lse_merge(red_l[0], red_l[i]); as = arg_merge(red_a[0], red_a[i]); red_l[0] = ls; red_a[0] = as; }
    const size_t q = static_cast<size_t>(b) * a.P + tile;
    a.p_m[q] = red_l[0].m;
    a.p_s[q] = red_l[0].s;
    a.p_score[q] = red_a[0].score;
    a.p_idx[q] = red_a[0].idx;
    a.p_x[q] = red_a[0].x;
  }
}

// ---------------------------------------------------------------------------
// Merge kernel: one workgroup of 256 threads per request.
//
// Greedy/sampled token and lse: thread t folds partials t, t+256, ... in
// order; the 256 thread states are folded by a fixed xor tree and then wave 0..3
// in order.
//
// Top-k (k <= 32), exact: the step kernel left the maximum of every segment of
// 32 columns.  (1) theta0 = k-th largest of the 256 per-thread maxima of those
// segment maxima: k distinct segments have a maximum >= theta0, so every
// element of the top k lies in a segment whose maximum is >= theta0.  (2) The
// candidate segments are recomputed element by element (U + A[x_{j-1}] . Bm
// in float32).  (3) theta1 = k-th largest candidate-segment maximum bounds the
// k-th largest element from below; the elements >= theta1 are ranked by
// (value descending, index ascending) and the first k kept.  If a list
// overflows its LDS capacity (massive ties), a slow exact path selects the k
// elements one by one over the whole row.
constexpr int kMergeThreads = 256;
constexpr int kCandSegCap = 128;
constexpr int kSurvCap = 256;

template <typename WT>
__device__ float recompute_logit(const StepArgs& a, const float* arow_s, int b, int v) {
  const WT* Bm = static_cast<const WT*>(a.Bm);
  const size_t V = static_cast<size_t>(a.V);
  float bias = 0.f;
  for (int k = 0; k < a.r; ++k) bias = fmaf(arow_s[k], to_f32(Bm[static_cast<size_t>(k) * V + v]), bias);
  return a.U[(static_cast<size_t>(b) * a.gamma + a.j) * V + v] + bias;
}

__device__ __forceinline__ bool ranks_before(float xa, int ia, float xb, int ib) {
  return xa > xb || (xa == xb && ia < ib);
}

template <typename WT>
__global__ __launch_bounds__(kMergeThreads) void markov_merge(StepArgs a) {
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int b = blockIdx.x;
  __shared__ LseState red_l[4];
  __shared__ ArgState red_a[4];

  LseState ls{kNegInf, 0.f};
  ArgState as{kNegInf, 0x7fffffff, 0.f};
  const size_t base = static_cast<size_t>(b) * a.P;
  for (int p = tid; p < a.Pn; p += kMergeThreads) {
    ls = lse_merge(ls, LseState{a.p_m[base + p], a.p_s[base + p]});
    as = arg_merge(as, ArgState{a.p_score[base + p], a.p_idx[base + p], a.p_x[base + p]});
  }
#pragma unroll
  for (int o = 1; o < kWave; o <<= 1) {
    ls = lse_merge(ls, shfl_xor(ls, o));
    as = arg_merge(as, shfl_xor(as, o));
  }
  if (lane == 0) { red_l[w] = ls; red_a[w] = as; }
  __syncthreads();
  if (tid == 0) {
    LseState l = red_l[0];
    ArgState s = red_a[0];
    for (int i = 1; i < 4; ++i) { l = lse_merge(l, red_l[i]); s = arg_merge(s, red_a[i]); }
    const int row = b * a.gamma + a.j;
    a.tokens[row] = s.idx;
    if (a.tok_logit) a.tok_logit[row] = s.x;
    if (a.lse) a.lse[row] = l.m + logf(l.s);
  }
  if (a.topk == 0) return;

  // ------------------------------ top-k ------------------------------------
  __shared__ float arow_s[kMaxRank];
  __shared__ float tmax[kMergeThreads];
  __shared__ int cseg[kCandSegCap];
  __shared__ float cval[kCandSegCap * kSeg];
  __shared__ float csegmax[kCandSegCap];
  __shared__ float sval[kSurvCap];
  __shared__ int sidx[kSurvCap];
  __shared__ int counter[2];
  __shared__ float theta[2];
  __shared__ float selv[kMaxTopk];
  __shared__ int seli[kMaxTopk];

  const int k = a.topk;
  const int prev = a.j == 0 ? a.anchor[b] : a.tokens[b * a.gamma + a.j - 1];
  const WT* A = static_cast<const WT*>(a.A);
  for (int i = tid; i < a.r; i += kMergeThreads) arow_s[i] = to_f32(A[static_cast<size_t>(prev) * a.r + i]);
  const float* sm = a.segmax + static_cast<size_t>(b) * a.S;
  float mt = kNegInf;
  for (int s = tid; s < a.S; s += kMergeThreads) mt = fmaxf(mt, sm[s]);
  tmax[tid] = mt;
  if (tid < 2) counter[tid] = 0;
  __syncthreads();
  {  // (1) theta0: the thread maximum of rank k-1
    int rank = 0;
    for (int u = 0; u < kMergeThreads; ++u) {
      const float o = tmax[u];
      rank += (o > mt) || (o == mt && u < tid);
    }
    if (rank == k - 1) theta[0] = mt;
  }
  __syncthreads();
  const float th0 = theta[0];
  for (int s = tid; s < a.S; s += kMergeThreads) {
    if (sm[s] >= th0) {
      const int slot = atomicAdd(&counter[0], 1);
      if (slot < kCandSegCap) cseg[slot] = s;
    }
  }
  __syncthreads();
  const int ncs = counter[0];
  bool overflow = ncs > kCandSegCap;
  if (!overflow) {
    // (2) recompute the candidate segments
    for (int e = tid; e < ncs * kSeg; e += kMergeThreads) {
      const int v = cseg[e / kSeg] * kSeg + (e % kSeg);
      cval[e] = v < a.V ? recompute_logit<WT>(a, arow_s, b, v) : kNegInf;
    }
    __syncthreads();
    for (int c = tid; c < ncs; c += kMergeThreads) {
      float m = kNegInf;
      for (int i = 0; i < kSeg; ++i) m = fmaxf(m, cval[c * kSeg + i]);
      csegmax[c] = m;
    }
    __syncthreads();
    // (3) theta1: k-th largest candidate-segment maximum (fewer than k
    // candidate segments only happens when every segment is a candidate)
    if (tid < ncs) {
      const float m = csegmax[tid];
      int rank = 0;
      for (int u = 0; u < ncs; ++u) rank += (csegmax[u] > m) || (csegmax[u] == m && u < tid);
      if (rank == k - 1) theta[1] = m;
    }
    if (tid == 0 && ncs < k) theta[1] = kNegInf;
    __syncthreads();
    const float th1 = theta[1];
    for (int e = tid; e < ncs * kSeg; e += kMergeThreads) {
      const float x = cval[e];
      if (x >= th1 && x != kNegInf) {
        const int slot = atomicAdd(&counter[1], 1);
        if (slot < kSurvCap) { sval[slot] = x; sidx[slot] = cseg[e / kSeg] * kSeg + (e % kSeg); }
      }
    }
    __syncthreads();
    const int ns = counter[1];
    overflow = ns > kSurvCap;
    if (!overflow) {
      for (int s = tid; s < ns; s += kMergeThreads) {
        int rank = 0;
        for (int u = 0; u < ns; ++u) rank += ranks_before(sval[u], sidx[u], sval[s], sidx[s]);
        if (rank < k) { selv[rank] = sval[s]; seli[rank] = sidx[s]; }
      }
    }
  }
  if (overflow) {
    // slow exact path: k rounds of "best element strictly after the last one
    // in (value desc, index asc) order" over the whole row
    __shared__ float rv[4];
    __shared__ int ri[4];
    float lastv = __builtin_huge_valf();
    int lasti = -1;
    for (int t = 0; t < k; ++t) {
      float bv = kNegInf;
      int bi = 0x7fffffff;
      for (int v = tid; v < a.V; v += kMergeThreads) {
        const float x = recompute_logit<WT>(a, arow_s, b, v);
        if (ranks_before(lastv, lasti, x, v) && ranks_before(x, v, bv, bi)) { bv = x; bi = v; }
      }
#pragma unroll
      for (int o = 1; o < kWave; o <<= 1) {
        const float ov = __shfl_xor(bv, o);
        const int oi = __shfl_xor(bi, o);
        if (ranks_before(ov, oi, bv, bi)) { bv = ov; bi = oi; }
      }
      if (lane == 0) { rv[w] = bv; ri[w] = bi; }
      __syncthreads();
      if (tid == 0) {
        for (int i = 1; i < 4; ++i)
          if (ranks_before(rv[i], ri[i], rv[0], ri[0])) { rv[0] = rv[i]; ri[0] = ri[i]; }
        selv[t] = rv[0];
        seli[t] = ri[0];
      }
      __syncthreads();
      lastv = selv[t];
      lasti = seli[t];
    }
  }
  __syncthreads();
  if (tid == 0) {
    const size_t o = (static_cast<size_t>(b) * a.gamma + a.j) * k;
    float ssum = 0.f;
    for (int t = 0; t < k; ++t) ssum += __expf(selv[t] - selv[0]);
    const float inv = 1.0f / ssum;
    for (int t = 0; t < k; ++t) {
      a.topk_idx[o + t] = seli[t];
      a.topk_prob[o + t] = __expf(selv[t] - selv[0]) * inv;
    }
  }
}

// ---------------------------------------------------------------------------
// host-side launchers

size_t markov_partials(int64_t V) { return static_cast<size_t>((V + kMarkovTile - 1) / kMarkovTile); }
size_t markov_segments(int64_t V) { return static_cast<size_t>((V + kSeg - 1) / kSeg); }

template <int RG, int KS>
static void launch_bf16(const StepArgs& a, hipStream_t s) {
  const dim3 grid((a.V + kMarkovTile - 1) / kMarkovTile, (a.B + 16 * RG - 1) / (16 * RG));
  hipLaunchKernelGGL((markov_step_bf16<RG, KS>), grid, dim3(kWave * KS), 0, s, a);
}

hipError_t launch_markov_position(StepArgs a, bool bf16, hipStream_t s) {
  if (bf16) {
    a.Pn = static_cast<int>((a.V + kMarkovTile - 1) / kMarkovTile);
    // request blocking and r-split: small batches split r over 4 waves so a
    // step has enough waves in flight; large batches reuse each transposed Bm
    // block for 4 request groups.
    if (a.B <= 16) {
      if (a.r % 128 == 0) launch_bf16<1, 4>(a, s);
      else if (a.r % 64 == 0) launch_bf16<1, 2>(a, s);
      else launch_bf16<1, 1>(a, s);
    } else if (a.B <= 32) {
      if (a.r % 64 == 0) launch_bf16<2, 2>(a, s);
      else launch_bf16<2, 1>(a, s);
    } else {
      launch_bf16<4, 1>(a, s);
    }
  } else {
    a.Pn = static_cast<int>((a.V + kMarkovTileF32 - 1) / kMarkovTileF32);
    const dim3 grid(a.Pn, a.B);
    hipLaunchKernelGGL(markov_step_f32, grid, dim3(256), 0, s, a);
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  if (bf16) hipLaunchKernelGGL(markov_merge<uint16_t>, dim3(a.B), dim3(kMergeThreads), 0, s, a);
  else hipLaunchKernelGGL(markov_merge<float>, dim3(a.B), dim3(kMergeThreads), 0, s, a);
  return hipGetLastError();
}

}  // namespace dspark
