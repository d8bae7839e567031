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
// Two launches per position: the step kernel streams Bm and U_j once for all
// requests and leaves one partial (max, sum-exp, best score/index) per
// (request, vocabulary tile); a merge kernel with one workgroup per request
// folds them in a fixed order into x_j, U~_j[x_j] and lse_j.  The top-k
// candidates are selected after the chain, off the sequential path.  (Small
// batches run the whole chain in one kernel instead: markov_resident.hip.)
#include <map>
#include <mutex>
#include <type_traits>
#include <utility>

#include "common.h"
#include "internal.h"
#include "markov_dev.h"

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
constexpr int kSeg = 8;            // vocabulary columns per top-k segment

// ---------------------------------------------------------------------------
// Fold of one request's per-tile partials of position j by a 256-thread
// workgroup: thread t takes tiles t, t+256, ... (loads issued kFoldBatch at a
// time), then a fixed xor tree and waves 0..3 in order; writes U~_j[x_j] and
// lse_j.  x_j is the fold's own argmax (per-position chain) or, after the
// resident chain, the chain's final key (the same element: both rank by
// score, then lowest index), which the fold then clears; -1 marks a resident
// chain whose grid-wide wait ran out of time in this call.
constexpr int kMergeThreads = 256;
constexpr int kFoldBatch = 4;

// The fold's results for (request, position): written by thread 0 at the
// fold's end, or, when the caller passes `out`, handed back to thread 0 for a
// later store (a store left outstanding here would hold up the caller's
// next waits on older loads).
struct FoldOut {
  int token;
  float tok_logit, lse;
};

__device__ __forceinline__ void store_fold(const StepArgs& a, int row, bool from_key, const FoldOut& f) {
  a.tokens[row] = f.token;
  if (from_key) a.best[row] = 0ull;
  if (a.tok_logit) a.tok_logit[row] = f.tok_logit;
  if (a.lse) a.lse[row] = f.lse;
}

__device__ void fold_request(const StepArgs& a, int b, int j, bool from_key, FoldOut* out = nullptr) {
  __shared__ LseState red_l[kMergeThreads / kWave];
  __shared__ ArgState red_a[kMergeThreads / kWave];
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  LseState ls{kNegInf, 0.f};
  ArgState as{kNegInf, 0x7fffffff, 0.f};
  const size_t base = (static_cast<size_t>(b) * a.gamma + j) * a.P;
  const int row = b * a.gamma + j;
  // the chain's final key and the time-out word, loaded beside the partials
  // (vector loads: a scalar load here would be waited for before the
  // partials' loads are issued)
  // (only the key's low word, the index part, is loaded: a 64-bit load whose
  // high register the compiler reuses would be waited for before the
  // partials' loads go out)
  unsigned key_lo = 0u;
  unsigned mark = 0u;
  if (from_key) {
    key_lo = __hip_atomic_load(reinterpret_cast<const unsigned*>(a.best + row), __ATOMIC_RELAXED,
                               __HIP_MEMORY_SCOPE_AGENT);
    mark = __hip_atomic_load(a.sync, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
  for (int p0 = 0; p0 < a.Pn; p0 += kFoldBatch * kMergeThreads) {
    LseState l[kFoldBatch];
    ArgState g[kFoldBatch];
#pragma unroll
    for (int u = 0; u < kFoldBatch; ++u) {
      const int p = p0 + u * kMergeThreads + tid;
      if (p < a.Pn) {
        l[u] = LseState{a.p_m[base + p], a.p_s[base + p]};
        g[u] = ArgState{a.p_score[base + p], a.p_idx[base + p], a.p_x[base + p]};
      } else {
        l[u] = LseState{kNegInf, 0.f};
        g[u] = ArgState{kNegInf, 0x7fffffff, 0.f};
      }
    }
#pragma unroll
    for (int u = 0; u < kFoldBatch; ++u) { ls = lse_merge(ls, l[u]); as = arg_merge(as, g[u]); }
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
    for (int i = 1; i < kMergeThreads / kWave; ++i) { l = lse_merge(l, red_l[i]); s = arg_merge(s, red_a[i]); }
    FoldOut f;
    if (from_key) f.token = mark == a.epoch ? -1 : best_index(key_lo);
    else f.token = (s.idx >= 0 && s.idx < a.V) ? s.idx : -1;   // -1: no orderable value (NaN row)
    f.tok_logit = s.x;
    f.lse = l.m + logf(l.s);
    // every fold of a call reads the same time-out word, so one of them reports it
    if (a.status && b == 0 && j == a.gamma - 1)
      *a.status = (from_key && mark == a.epoch) ? kStatusTimeout : kStatusOk;
    if (out) *out = f;
    else store_fold(a, row, from_key, f);
  }
}

// ---------------------------------------------------------------------------
// Step epilogue for one wave: lane (g, n) holds requests req0 + 16 rg + 4 g + ii
// (ii < 4) for the 8 consecutive columns vcol..vcol+7 of this tile.  Per
// request: add U_j (optionally dump U~), take the 16-lane group maximum M, sum
// exp(U~ - M) (one exponential per element), draw the Gumbel noise when
// sampling, reduce (best score, index, U~ there), and write one partial per
// request plus the 8-column segment maxima for top-k.  A scheduling barrier
// between requests keeps one request's working set live at a time.
// U_j for the lane's requests and columns, loaded before the r-loop so that its
// latency hides under the Bm stream: up[rg][ii][half] = U[b, j, vcol + 4 half ..]
template <int RG>
__device__ __forceinline__ void prefetch_u(const StepArgs& a, int req0, int vcol, bool vok, int g,
                                           f32x4 (&up)[RG][4][2]) {
  const size_t V = static_cast<size_t>(a.V);
#pragma unroll
  for (int rg = 0; rg < RG; ++rg)
#pragma unroll
    for (int ii = 0; ii < 4; ++ii) {
      const int b = req0 + 16 * rg + 4 * g + ii;
      if ((b < a.B) && vok) {
        const float* urow = a.U + (static_cast<size_t>(b) * a.gamma + a.j) * V + vcol;
        up[rg][ii][0] = *reinterpret_cast<const f32x4*>(urow);
        up[rg][ii][1] = *reinterpret_cast<const f32x4*>(urow + 4);
      } else {
        up[rg][ii][0] = up[rg][ii][1] = f32x4{0.f, 0.f, 0.f, 0.f};
      }
    }
}

template <int RG, bool SAMPLE>
__device__ __forceinline__ void epilogue_store(const StepArgs& a, const f32x4 (&acc)[RG][8],
                                               const f32x4 (&up)[RG][4][2],
                                               int req0, int tile, int vcol, bool vok, int g, int n) {
  const size_t V = static_cast<size_t>(a.V);
#pragma unroll
  for (int q = 0; q < 4 * RG; ++q) {
    const int b = req0 + 16 * (q >> 2) + 4 * g + (q & 3);
    const bool live = (b < a.B) && vok;
    float x[8];
#pragma unroll
    for (int c = 0; c < 8; ++c) x[c] = acc[q >> 2][c][q & 3];
    const size_t row = static_cast<size_t>(b) * a.gamma + a.j;
    if (live) {
      const f32x4 u0 = up[q >> 2][q & 3][0], u1 = up[q >> 2][q & 3][1];
#pragma unroll
      for (int c = 0; c < 4; ++c) { x[c] += u0[c]; x[c + 4] += u1[c]; }
      if (a.logits_out) {
        float* orow = a.logits_out + row * V + vcol;
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
    if (a.segmax && live) a.segmax[row * a.S + vcol / kSeg] = m8;   // one top-k segment
    float M = m8;
    M = row16_max(M);
    float ssum = 0.f;
    if (live) {
#pragma unroll
      for (int c = 0; c < 8; ++c) ssum += __expf(x[c] - M);
    }
    ssum = row16_sum(ssum);

    float score[8];
    if constexpr (SAMPLE) {
      if (live) {
        const uint64_t sd = a.seeds[b];
        const uint32_t k0 = static_cast<uint32_t>(sd), k1 = static_cast<uint32_t>(sd >> 32);
        const Philox4 r0 = philox4x32_10(vcol >> 2, a.j, a.off_lo, a.off_hi, k0, k1);
        const Philox4 r1 = philox4x32_10((vcol >> 2) + 1, a.j, a.off_lo, a.off_hi, k0, k1);
        const uint32_t wd[8] = {r0.x, r0.y, r0.z, r0.w, r1.x, r1.y, r1.z, r1.w};
#pragma unroll
        for (int c = 0; c < 8; ++c) score[c] = x[c] * a.inv_temp + gumbel_from_word(wd[c]);
      } else {
#pragma unroll
        for (int c = 0; c < 8; ++c) score[c] = kNegInf;
      }
    } else {
#pragma unroll
      for (int c = 0; c < 8; ++c) score[c] = x[c];
    }
    ArgState as{score[0], live ? vcol : 0x7fffffff, x[0]};
#pragma unroll
    for (int c = 1; c < 8; ++c)
      if (score[c] > as.score) as = ArgState{score[c], vcol + c, x[c]};
    as = row16_arg(as);
    if (n == 0 && b < a.B) {
      const size_t pq = row * a.P + tile;
      a.p_m[pq] = M;
      a.p_s[pq] = ssum;
      a.p_score[pq] = as.score;
      a.p_idx[pq] = as.idx;
      a.p_x[pq] = as.x;
    }
    __builtin_amdgcn_sched_barrier(0);
  }
}

template <int RG, int KS, bool SAMPLE>
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
    arow[rg] = bok[rg] ? a_operand_row<uint16_t>(a, b, a.j) : A;
  }

  f32x4 acc[RG][8];
#pragma unroll
  for (int rg = 0; rg < RG; ++rg)
#pragma unroll
    for (int c = 0; c < 8; ++c) acc[rg][c] = f32x4{0.f, 0.f, 0.f, 0.f};
  f32x4 up[RG][4][2];
  if (w == 0) prefetch_u<RG>(a, req0, vcol, vok, g, up);

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
    if (w == 0) {
#pragma unroll
      for (int s = 0; s < KS - 1; ++s)
#pragma unroll
        for (int rg = 0; rg < RG; ++rg)
#pragma unroll
          for (int c = 0; c < 8; ++c) acc[rg][c] += red[s][rg][c][lane];
    }
  }

  if (w == 0) epilogue_store<RG, SAMPLE>(a, acc, up, req0, tile, vcol, vok, g, n);
}

// ---------------------------------------------------------------------------
// Wide bf16 step kernel (B > 16, r <= 256).  A workgroup owns a contiguous
// range of 64-column tiles for up to 8 waves x 16 requests.
//  - Each wave keeps its requests' A[x_{j-1}] rows (the MFMA A operands, one
//    per 32-row chunk) in registers for the whole range.
//  - A tile's Bm (r x 64) sits in LDS in MFMA B-operand form (the 4-column
//    byte permute of load_chunk: operand c of lane (g, n) is column 4n + c,
//    rows 8g .. 8g+7 of a 32-row chunk), double-buffered: the waves fetch
//    later tiles' rows into registers while the current tile is computed,
//    and one barrier per tile separates the buffers.
//  - U_j of the next tile is fetched a tile ahead as well.  Every load is
//    unconditional (addresses clamped into the arrays, values masked), the
//    loop is unrolled by two so that no loaded register is copied while in
//    flight, and the barrier waits for LDS writes only, so the loads stay in
//    flight across it.
//  - Each lane keeps, per request, lane-local online states over its columns
//    of all tiles: (max, sum-exp) with one rescale per tile, and the best
//    score with its column (columns arrive in increasing order, so a strict
//    comparison keeps the lowest index) and U~ there.  The 16-lane reductions
//    (DPP) run once per request per workgroup; the argmax travels as a 64-bit
//    order key (best_key).  One partial per (request, workgroup range).
constexpr int kWideCols = 64;

// LDS of the wide kernel: two B-operand buffers of nch chunks, then (when
// sampling) the seeds of up to 8 x 16 requests
// (each buffer has one spare chunk slot: waves with no chunk of their own store
// there, so the store needs no branch)
__host__ __device__ constexpr size_t wide_ops_bytes(int nch) { return static_cast<size_t>(nch + 1) * 2 * 4 * kWave * 16; }
constexpr size_t kWideSeedBytes = 8 * 16 * 8;

// 16-lane maximum of 64-bit keys
__device__ __forceinline__ unsigned long long row16_max_u64(unsigned long long k) {
  auto step = [&](auto ctrl) {
    constexpr int C = decltype(ctrl)::value;
    const unsigned lo = static_cast<unsigned>(dpp_i<C>(static_cast<int>(static_cast<uint32_t>(k))));
    const unsigned hi = static_cast<unsigned>(dpp_i<C>(static_cast<int>(static_cast<uint32_t>(k >> 32))));
    const unsigned long long o = (static_cast<unsigned long long>(hi) << 32) | lo;
    k = o > k ? o : k;
  };
  step(std::integral_constant<int, kDppXor1>{});
  step(std::integral_constant<int, kDppXor2>{});
  step(std::integral_constant<int, kDppHalfMirror>{});
  step(std::integral_constant<int, kDppMirror>{});
  return k;
}

// this wave's LDS writes are complete, then a plain s_barrier: unlike
// __syncthreads it leaves outstanding global loads in flight
__device__ __forceinline__ void lds_barrier() {
  __builtin_amdgcn_s_waitcnt(0xC07F);   // lgkmcnt(0); vmcnt and expcnt at their maxima
  asm volatile("s_barrier" ::: "memory");
}

// The wide kernel addresses every array through buffer resources (buf_rsrc,
// whose sizes the launcher keeps below 2 GiB) with a per-lane 32-bit offset
// that stays fixed across tiles plus the tile's offset in a scalar register,
// so a tile's loads and stores cost no vector address arithmetic.
constexpr uint32_t kDropOffset = 0x80000000u;   // past every resource: the access is dropped
// Stores of more than 8 bytes take their whole offset in the vector register
// and a constant 0 as scalar offset: the compiler then keeps a VALU write of
// the store's data registers one wait state behind the store.  With the tile
// offset in a scalar register it inserted none, and on gfx950 the register
// overwritten right after a 16-byte store reached memory with its new value
// in some lanes (block logits of one column in four read -inf).

// STATS = false: teacher-forced block logits only (every row's previous token
// given; each tile's U~ is stored to logits_out and nothing else is kept).
// DUMP = false: the chain with no U~ dump requested (no dump store is issued;
// a store to a resource of no records still costs its issue).
// BMT: position 0 of a chain whose top-k reads BmT: the step also stores it.
template <int NCH, int CPW, bool SAMPLE, bool STATS = true, bool DUMP = true, bool BMT = false>
__global__ __launch_bounds__(512) void markov_step_wide(StepArgs a, int tpw) {
  extern __shared__ __align__(16) unsigned char wide_lds[];
  u32x4* const ops = reinterpret_cast<u32x4*>(wide_lds);   // [2][NCH + 1][4][64] B operands
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6, nw = blockDim.x >> 6;
  const int g = lane >> 4, n = lane & 15;
  const int req0 = (blockIdx.y * nw + w) * 16;
  const int tb = blockIdx.x * tpw;                                   // first tile
  const int nt = min(tpw, (a.V + kWideCols - 1) / kWideCols - tb);
  if (nt <= 0) return;                     // padding of the grid (whole workgroup)
  const int last = nt - 1;
  const uint32_t V = static_cast<uint32_t>(a.V);
  const size_t rows = static_cast<size_t>(a.B) * a.gamma;

  // Requests past the batch (a ragged last group) are computed as request
  // B - 1: the same A row and U row, hence the same values, and their stores
  // repeat that request's; only the final partials skip them.
  const __amdgpu_buffer_rsrc_t u_rsrc = buf_rsrc(a.U, rows * V * 4);
  const __amdgpu_buffer_rsrc_t bm_rsrc = buf_rsrc(a.Bm, static_cast<size_t>(a.r) * V * 2);
  const __amdgpu_buffer_rsrc_t out_rsrc =
      a.logits_out ? buf_rsrc(a.logits_out, rows * V * 4) : buf_rsrc(a.U, 0);
  const __amdgpu_buffer_rsrc_t seg_rsrc =
      a.segmax ? buf_rsrc(a.segmax, rows * a.S * 4) : buf_rsrc(a.U, 0);
  uint32_t uoff[4], soff[4];     // request 4g + ii: U / U~ row and segment-maxima row at tile 0
#pragma unroll
  for (int ii = 0; ii < 4; ++ii) {
    const uint32_t row = static_cast<uint32_t>(min(req0 + 4 * g + ii, a.B - 1)) * a.gamma + a.j;
    uoff[ii] = (row * V + tb * kWideCols + 4 * n) * 4;
    soff[ii] = (row * a.S + tb * (kWideCols / kSeg) + (n >> 1)) * 4;
  }
  // BMT: the step also stores the transposed Bm (BmT [V, r]) for the top-k
  // recompute: the B-operand pieces it builds anyway are 16-byte pieces of
  // BmT rows (column 4n + c, rows 32q + 8g ..).  Request group y stores the
  // chunks q with q % ny == y, so the stores spread evenly.
  constexpr bool bmt_w = STATS && BMT;
  const __amdgpu_buffer_rsrc_t bmt_rsrc =
      bmt_w ? buf_rsrc(a.BmT, static_cast<size_t>(a.r) * V * 2) : buf_rsrc(a.U, 0);
  // Bm rows of this wave's chunks (chunks w, w + nw, ...; NCH <= CPW * nw)
  uint32_t boff[CPW][8];
#pragma unroll
  for (int s = 0; s < CPW; ++s) {
    const int q = min(w + s * nw, NCH - 1);
#pragma unroll
    for (int i = 0; i < 8; ++i) boff[s][i] = ((32 * q + 8 * g + i) * V + tb * kWideCols + 4 * n) * 2;
  }
  // look-aheads past the range reload the last tile (an L2 hit)
  auto load_u = [&](int t, f32x4 (&u)[4]) __attribute__((always_inline)) {
    const int tof = min(t, last) * kWideCols * 4;
#pragma unroll
    for (int ii = 0; ii < 4; ++ii)
      u[ii] = __builtin_bit_cast(f32x4, __builtin_amdgcn_raw_buffer_load_b128(u_rsrc, static_cast<int>(uoff[ii]), tof,
                                                                              kBufferNonTemporal));
  };
  auto load_bm = [&](int t, u32x2 (&raw)[CPW][8]) __attribute__((always_inline)) {
    const int tof = min(t, last) * kWideCols * 2;
#pragma unroll
    for (int s = 0; s < CPW; ++s)
#pragma unroll
      for (int i = 0; i < 8; ++i)
        raw[s][i] = __builtin_bit_cast(u32x2, __builtin_amdgcn_raw_buffer_load_b64(bm_rsrc, static_cast<int>(boff[s][i]),
                                                                                 tof, 0));
  };
  auto store_bm = [&](int buf, u32x2 (&raw)[CPW][8], int tt) __attribute__((always_inline)) {
    u32x4* const o = ops + buf * (NCH + 1) * 4 * kWave;
#pragma unroll
    for (int s = 0; s < CPW; ++s) {
      const int q = min(w + s * nw, NCH);              // NCH: the spare slot
      // pin the byte permutes here: as plain register arithmetic they could be
      // hoisted over the preceding barrier to right after the rows' loads,
      // which would then be waited for a whole tile early
#pragma unroll
      for (int i = 0; i < 8; ++i) asm volatile("" : "+v"(raw[s][i]));
      u32x4 op[4];
      transpose_rows4(raw[s], op);
#pragma unroll
      for (int c = 0; c < 4; ++c) o[(q * 4 + c) * kWave + lane] = op[c];
      if constexpr (bmt_w) {
        // tile tt's own rows only (a look-ahead past the range reloads the
        // last tile), one request group per chunk; columns past V fall
        // outside the resource and are dropped
        const bool mine = tt <= last && q < NCH && q % static_cast<int>(gridDim.y) == static_cast<int>(blockIdx.y);
        const uint32_t base = ((static_cast<uint32_t>(tb + tt) * kWideCols + 4 * n) * a.r + 32 * q + 8 * g) * 2;
#pragma unroll
        for (int c = 0; c < 4; ++c)
          __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, op[c]), bmt_rsrc,
                                                 static_cast<int>(mine ? base + c * a.r * 2 : kDropOffset), 0, 0);
      }
    }
  };

  // A operands: lane (g, n) holds request req0 + n, rows 32q + 8g .. of chunk q
  u32x4 av[NCH];
  {
    const int b = min(req0 + n, a.B - 1);
    const uint16_t* arow = a_operand_row<uint16_t>(a, b, a.j) + 8 * g;
#pragma unroll
    for (int q = 0; q < NCH; ++q) av[q] = *reinterpret_cast<const u32x4*>(arow + 32 * q);
  }

  // sampling seeds of the workgroup's requests, staged in LDS before the first
  // barrier (a global load inside the tile loop would wait for every
  // look-ahead load issued before it)
  uint64_t* const seeds_s = reinterpret_cast<uint64_t*>(wide_lds + wide_ops_bytes(NCH));
  if constexpr (SAMPLE) {
    if (lane < 16) seeds_s[w * 16 + lane] = a.seeds[min(req0 + lane, a.B - 1)];
  }

  // Lane-local states per request 4g + ii over the lane's columns: the
  // running maximum ml of U~ and the sum sl of exp(U~ - ml) (rescaled when ml
  // moves); the best score bs with its column bc and U~ there (greedy: the
  // best score is ml itself and its U~ too).
  float ml[4], sl[4], bs[4], bx[4];
  int bc[4];
#pragma unroll
  for (int ii = 0; ii < 4; ++ii) { ml[ii] = kNegInf; sl[ii] = 0.f; bs[ii] = kNegInf; bx[ii] = 0.f; bc[ii] = 0x7fffffff; }

  // The bias of one tile: NCH x 4 MFMAs from B-operand buffer `buf`.
  auto mma = [&](int buf, f32x4 (&acc)[4]) __attribute__((always_inline)) {
    const u32x4* const o = ops + buf * (NCH + 1) * 4 * kWave;
#pragma unroll
    for (int c = 0; c < 4; ++c) acc[c] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int q = 0; q < NCH; ++q)
#pragma unroll
      for (int c = 0; c < 4; ++c)
        acc[c] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(av[q]), as_bf16x8(o[(q * 4 + c) * kWave + lane]),
                                                         acc[c], 0, 0, 0);
  };
  // The epilogue of tile t from its bias `acc` and U_j values `u`; branch-free
  // (the whole tile pair is one basic block for the scheduler).  Each request's
  // U_j registers are reloaded with tile tn right after their last use, so
  // that the wave's U_j loads enter the memory pipeline spread over the
  // epilogue rather than in one burst.
  // MASK: the range's last tiles, where columns may lie past V (the last tile
  // of the vocabulary) or past the range (the padding tile t == nt of an odd
  // range): those carry -inf and store nothing.  Every other tile is whole.
  auto epi = [&](auto mask_tag, int t, const f32x4 (&acc)[4], f32x4 (&u)[4], int tn) __attribute__((always_inline)) {
    constexpr bool MASK = decltype(mask_tag)::value;
    const int col = (tb + t) * kWideCols + 4 * n;
    const bool cok = !MASK || (t < nt && col < a.V);
    const int tofx = t * kWideCols * 4, tofs = t * (kWideCols / kSeg) * 4;
    float xs[4][4];
    float seg[4];
#pragma unroll
    for (int ii = 0; ii < 4; ++ii) {
      float* const x = xs[ii];
#pragma unroll
      for (int c = 0; c < 4; ++c) x[c] = acc[c][ii] + u[ii][c];
      u[ii] = __builtin_bit_cast(f32x4, __builtin_amdgcn_raw_buffer_load_b128(u_rsrc, static_cast<int>(uoff[ii]),
                                                                              min(tn, last) * kWideCols * 4,
                                                                              kBufferNonTemporal));
      if constexpr (MASK) {
#pragma unroll
        for (int c = 0; c < 4; ++c) x[c] = cok ? x[c] : kNegInf;
      }
      if constexpr (!STATS) {
        __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, f32x4{x[0], x[1], x[2], x[3]}), out_rsrc,
                                               static_cast<int>(cok ? uoff[ii] + tofx : kDropOffset), 0,
                                               kBufferNonTemporal);
        continue;
      }
      const float m4 = fmaxf(fmaxf(x[0], x[1]), fmaxf(x[2], x[3]));
      // lanes 2s and 2s + 1 both end with the maximum of 8-column segment s
      seg[ii] = fmaxf(m4, dpp_f<kDppXor1>(m4));
      if (ii & 1) {
        // one store for requests ii - 1 and ii: the even lane of each pair
        // stores the first's segment maximum, the odd lane the second's
        const bool odd = (n & 1) != 0;
        __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(odd ? seg[ii] : seg[ii - 1]), seg_rsrc,
                                              static_cast<int>(cok ? (odd ? soff[ii] : soff[ii - 1]) : kDropOffset),
                                              tofs, 0);
      }
      if constexpr (SAMPLE) {
        const uint64_t sd = seeds_s[w * 16 + 4 * g + ii];
        const Philox4 r = philox4x32_10(col >> 2, a.j, a.off_lo, a.off_hi, static_cast<uint32_t>(sd),
                                        static_cast<uint32_t>(sd >> 32));
        const uint32_t wd[4] = {r.x, r.y, r.z, r.w};
#pragma unroll
        for (int c = 0; c < 4; ++c) {
          const float sc = x[c] * a.inv_temp + gumbel_from_word(wd[c]);
          const bool up = sc > bs[ii];
          bs[ii] = up ? sc : bs[ii];
          bc[ii] = up ? col + c : bc[ii];
          bx[ii] = up ? x[c] : bx[ii];
        }
      } else {
        // greedy: the score is U~ itself, so the best so far is the running
        // maximum; it moves only where this tile's maximum exceeds it
        // (strictly: the lowest column keeps a tie), to the first column
        // holding that maximum
        const bool up = m4 > ml[ii];
        int c4 = 3;                                     // selects, not branches
        c4 = x[2] == m4 ? 2 : c4;
        c4 = x[1] == m4 ? 1 : c4;
        c4 = x[0] == m4 ? 0 : c4;
        bc[ii] = up ? col + c4 : bc[ii];
      }
      // sum of exp in base 2: one fused multiply-add and one exp2 per element
      const float mn = fmaxf(ml[ii], m4);
      const float mref = mn == kNegInf ? 0.f : mn;     // no column yet: keep s = 0
      const float nm2 = -mref * kLog2e;
      const float e0 = __builtin_amdgcn_exp2f(fmaf(x[0], kLog2e, nm2)), e1 = __builtin_amdgcn_exp2f(fmaf(x[1], kLog2e, nm2));
      const float e2 = __builtin_amdgcn_exp2f(fmaf(x[2], kLog2e, nm2)), e3 = __builtin_amdgcn_exp2f(fmaf(x[3], kLog2e, nm2));
      sl[ii] = fmaf(sl[ii], __builtin_amdgcn_exp2f(fmaf(ml[ii], kLog2e, nm2)), (e0 + e1) + (e2 + e3));
      ml[ii] = mn;
    }
    if constexpr (STATS && DUMP) {
      // the U~ dump
#pragma unroll
      for (int ii = 0; ii < 4; ++ii)
        __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, f32x4{xs[ii][0], xs[ii][1], xs[ii][2], xs[ii][3]}),
                                               out_rsrc, static_cast<int>(cok ? uoff[ii] + tofx : kDropOffset), 0,
                                               kBufferNonTemporal);
    }
  };
  using Whole = std::integral_constant<bool, false>;
  using Masked = std::integral_constant<bool, true>;

  // Tile t's bias comes from buffer t & 1.  Each wave issues the MFMAs of
  // tile t + 1 before the epilogue of tile t, so the matrix unit works on
  // the next tile while the vector unit runs this one's softmax statistics
  // (the MFMAs' results are read one step later).  U registers u0 / u1 hold
  // tiles t / t + 1 and are refilled two tiles ahead inside the epilogue; the
  // bias of a tile past the range is computed but never used.  With one chunk
  // per wave the Bm rows have two register sets (ra: even tiles, rb: odd ones),
  // fetched two tiles before their LDS store; with two chunks one set, a tile
  // before.  Each half-pair opens with the LDS store of the next tile's
  // operands (into the buffer whose last reads came before the barrier) and
  // the loads of a later tile's Bm rows, so that a wave's loads leave in two
  // groups per tile, not one burst after the epilogue (measured: ~1.5% off
  // the step at B = 256, none at B = 64).
  // The loop runs whole tiles; the last pair (the range's last tile, which
  // may be partial, and the padding tile of an odd range) runs masked.
  f32x4 u0[4], u1[4];
  f32x4 acc0[4], acc1[4];
  u32x2 ra[CPW][8];
  int t = 0;
  if constexpr (CPW == 1) {
    u32x2 rb[CPW][8];
    auto pair = [&](auto mask_tag) __attribute__((always_inline)) {
      store_bm(0, ra, t + 2);                           // tile t + 2
      load_bm(t + 4, ra);
      mma(1, acc1);                                     // tile t + 1
      epi(mask_tag, t, acc0, u0, t + 2);
      lds_barrier();
      store_bm(1, rb, t + 3);                           // tile t + 3
      load_bm(t + 5, rb);
      mma(0, acc0);                                     // tile t + 2
      epi(mask_tag, t + 1, acc1, u1, t + 3);
      lds_barrier();
    };
    load_bm(0, ra);
    load_u(0, u0);
    load_bm(1, rb);
    load_u(1, u1);
    store_bm(0, ra, 0);                                 // tile 0
    load_bm(2, ra);
    lds_barrier();
    mma(0, acc0);
    store_bm(1, rb, 1);                                 // tile 1
    load_bm(3, rb);
    lds_barrier();
    for (; t + 2 < nt; t += 2) pair(Whole{});
    pair(Masked{});
  } else {
    auto pair = [&](auto mask_tag) __attribute__((always_inline)) {
      store_bm(0, ra, t + 2);                           // tile t + 2
      load_bm(t + 3, ra);
      mma(1, acc1);                                     // tile t + 1
      epi(mask_tag, t, acc0, u0, t + 2);
      lds_barrier();
      store_bm(1, ra, t + 3);                           // tile t + 3
      load_bm(t + 4, ra);
      mma(0, acc0);                                     // tile t + 2
      epi(mask_tag, t + 1, acc1, u1, t + 3);
      lds_barrier();
    };
    load_bm(0, ra);
    load_u(0, u0);
    store_bm(0, ra, 0);                                 // tile 0
    load_bm(1, ra);
    load_u(1, u1);
    lds_barrier();
    mma(0, acc0);
    store_bm(1, ra, 1);                                 // tile 1
    load_bm(2, ra);
    lds_barrier();
    for (; t + 2 < nt; t += 2) pair(Whole{});
    pair(Masked{});
  }

  // one partial per request: 16-lane reductions of the lane states
  if constexpr (!STATS) return;
#pragma unroll
  for (int ii = 0; ii < 4; ++ii) {
    const int b = req0 + 4 * g + ii;
    if constexpr (!SAMPLE) { bs[ii] = ml[ii]; bx[ii] = ml[ii]; }
    const float M = row16_max(ml[ii]);
    const float ssum = row16_sum(ml[ii] == kNegInf ? 0.f : sl[ii] * __expf(ml[ii] - M));
    const unsigned long long key = row16_max_u64(bs[ii] == kNegInf ? 0ull : best_key(bs[ii], bc[ii]));
    const float xw = row16_max((bs[ii] != kNegInf && best_key(bs[ii], bc[ii]) == key) ? bx[ii] : kNegInf);
    if (n == 0 && b < a.B) {
      const size_t pq = (static_cast<size_t>(b) * a.gamma + a.j) * a.P + blockIdx.x;
      a.p_m[pq] = M;
      a.p_s[pq] = ssum;
      a.p_score[pq] = best_value(key);
      a.p_idx[pq] = best_index(key);
      a.p_x[pq] = xw;
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
  const float* Bm = static_cast<const float*>(a.Bm);
  const float* ar = a_operand_row<float>(a, b, a.j);
  for (int k = tid; k < a.r; k += 256) arow[k] = ar[k];
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
    if ((lane & (kSeg - 1)) == 0 && live) a.segmax[(static_cast<size_t>(b) * a.gamma + a.j) * a.S + v / kSeg] = sm;
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
    const size_t q = (static_cast<size_t>(b) * a.gamma + a.j) * a.P + tile;
    a.p_m[q] = red_l[0].m;
    a.p_s[q] = red_l[0].s;
    a.p_score[q] = red_a[0].score;
    a.p_idx[q] = red_a[0].idx;
    a.p_x[q] = red_a[0].x;
  }
}

// ---------------------------------------------------------------------------
// The per-position merge, and the fold of every (request, position) after the
// resident chain.  After the resident chain the finish kernels (markov_fold,
// markov_topk_lists) leave the wait tree zeroed for the next call: their
// workgroups clear, in slices, exactly the words this call's chain used (all
// of their readers have finished): the counter and release flag of each
// group of kFanIn workgroups, the top counter, and the keys of the call's
// positions, groups and requests.  Word 0, the time-out mark, holds a call
// number and is never cleared.
__device__ __forceinline__ void clear_wait_tree(const StepArgs& a) {
  const int L = blockIdx.x * a.gamma + blockIdx.y, n = a.B * a.gamma;
  const int ng = (a.nlist + kFanIn - 1) / kFanIn;
  const int total = 2 * ng + 1 + a.gamma * ng * a.B;
  unsigned long long* keys = reinterpret_cast<unsigned long long*>(a.sync + kSyncKeys);
  for (int i = L * blockDim.x + threadIdx.x; i < total; i += n * blockDim.x) {
    if (i < ng) {
      a.sync[kSyncGroupCnt + 64 * i] = 0u;
    } else if (i < 2 * ng) {
      a.sync[kSyncRelease + 64 * (i - ng)] = 0u;
    } else if (i == 2 * ng) {
      a.sync[kSyncTopCnt] = 0u;
    } else {
      const int q = i - 2 * ng - 1, b = q % a.B, r = q / a.B, grp = r % ng, j = r / ng;
      keys[(j * kFanIn + grp) * kResidentMaxB + b] = 0ull;
    }
  }
}

__global__ __launch_bounds__(kMergeThreads) void markov_merge(StepArgs a) {
  fold_request(a, blockIdx.x, a.j, false);
}

__global__ __launch_bounds__(kMergeThreads) void markov_fold(StepArgs a) {
  fold_request(a, blockIdx.x, blockIdx.y, true);
  clear_wait_tree(a);
}

// ---------------------------------------------------------------------------
// Top-k kernel of the per-position chain (off the sequential path): one
// workgroup per (request, position), launched once after the chain.  Exact for
// k <= 32.
//
// Bounds used (each holds because k distinct tiles or segments reach them):
//  theta00 = k-th largest of the 256 per-thread maxima of the tile maxima
//            (the per-tile U~ maximum from the step kernel); every segment whose
//            maximum is >= theta00 lies in a tile whose maximum is >= theta00,
//            and at least k segments do;
//  theta   = exact k-th largest segment maximum, found among those segments;
//            the k-th largest element is >= theta, so the top k lie in the
//            segments (8 columns each) whose maximum is >= theta: k plus ties.
// Those segments are recomputed column by column (U + A[x_{j-1}] . Bm in
// float32, 16 threads per segment over slices of r, 8 columns per 16-byte
// load) and their elements ranked by (value descending, index ascending).  If
// a candidate list overflows its LDS capacity (massive ties), a slow exact
// path selects the k elements one by one over the whole row.
constexpr int kTopkThreads = 256;
constexpr int kTileCap = 128;
constexpr int kCand1Cap = 512;
constexpr int kCand2Cap = 64;
constexpr int kSliceThreads = 16;   // threads sharing one segment's r-loop

template <typename WT>
__device__ float recompute_logit(const StepArgs& a, const float* arow_s, const float* urow, int v) {
  const WT* Bm = static_cast<const WT*>(a.Bm);
  const size_t V = static_cast<size_t>(a.V);
  float bias = 0.f;
  for (int k = 0; k < a.r; ++k) bias = fmaf(arow_s[k], to_f32(Bm[static_cast<size_t>(k) * V + v]), bias);
  return urow[v] + bias;
}

// 8 consecutive columns v0..v0+7 of Bm row k (columns >= V read as 0), kept
// packed until use: one 16-byte load for bf16 (V % 8 == 0 there)
template <typename WT> struct SegRows;
template <> struct SegRows<uint16_t> {
  static constexpr int kBatch = 16;
  typedef u32x4 Raw;
  static __device__ __forceinline__ Raw load(const uint16_t* Bm, int k, int v0, int V) {
    return *reinterpret_cast<const u32x4*>(Bm + static_cast<size_t>(k) * V + v0);
  }
  static __device__ __forceinline__ void unpack(const Raw& w, float* c) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      c[2 * i] = __uint_as_float(w[i] << 16);
      c[2 * i + 1] = __uint_as_float(w[i] & 0xFFFF0000u);
    }
  }
};
template <> struct SegRows<float> {
  static constexpr int kBatch = 8;
  struct Raw { float c[8]; };
  static __device__ __forceinline__ Raw load(const float* Bm, int k, int v0, int V) {
    Raw r;
    const float* row = Bm + static_cast<size_t>(k) * V;
#pragma unroll
    for (int i = 0; i < 8; ++i) r.c[i] = (v0 + i < V) ? row[v0 + i] : 0.f;
    return r;
  }
  static __device__ __forceinline__ void unpack(const Raw& w, float* c) {
#pragma unroll
    for (int i = 0; i < 8; ++i) c[i] = w.c[i];
  }
};

// Order-preserving map of floats to unsigned keys (and back).
__device__ __forceinline__ unsigned float_key(float x) {
  const unsigned u = __float_as_uint(x);
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}
__device__ __forceinline__ float key_float(unsigned o) {
  return __uint_as_float((o & 0x80000000u) ? (o & 0x7fffffffu) : ~o);
}

// The k-th largest of the n values of `vals` (16-byte aligned in LDS), NaNs
// left out; -inf when fewer than k values are not NaN.  It is the smallest
// value m with fewer than k values strictly above it, so each thread counts,
// for its own values, the values above them (one compare each, four per
// 16-byte LDS read at the same address in every lane), and the values that
// qualify meet in an LDS minimum over order-preserving keys.  kmin (~0u) and
// kcnt (0) are set before the barrier that precedes the call.  Every thread
// calls it and gets the result.
__device__ float kth_largest(const float* vals, int n, int k, unsigned* kmin, int* kcnt) {
  constexpr int kBatch = 8;                   // 16-byte reads in flight
  const f32x4* v4 = reinterpret_cast<const f32x4*>(vals);
  const int n4 = n >> 2;
  for (int i0 = 0; i0 < n; i0 += kTopkThreads) {
    const int i = i0 + static_cast<int>(threadIdx.x);
    const float m = i < n ? vals[i] : __builtin_nanf("");
    const bool live = m == m;
    const unsigned long long bal = __ballot(live);
    if ((threadIdx.x & (kWave - 1)) == 0 && bal) atomicAdd(kcnt, __popcll(bal));
    if (!live) continue;
    int gt = 0, u = 0;
    for (; u + kBatch <= n4; u += kBatch) {
      f32x4 q[kBatch];
#pragma unroll
      for (int t = 0; t < kBatch; ++t) q[t] = v4[u + t];
#pragma unroll
      for (int t = 0; t < kBatch; ++t)
#pragma unroll
        for (int c = 0; c < 4; ++c) gt += q[t][c] > m;
    }
    for (u *= 4; u < n; ++u) gt += vals[u] > m;
    if (gt < k) atomicMin(kmin, float_key(m));
  }
  __syncthreads();
  return *kcnt < k ? kNegInf : key_float(*kmin);
}

// The second launch bound is an occupancy target (waves per SIMD): 7 for the
// BmT form, whose 70 registers let 7 workgroups per CU hold a 256 x 7 grid at
// once, and 4 for the others (their register counts).  Without it the
// compiler kept the argument block in over 100 scalar registers and spilled a
// third of them into vector lanes inside the loops (20% slower at B = 256,
// V = 151936).
template <typename WT, bool BMT = false>
__global__ __launch_bounds__(kTopkThreads, BMT ? 7 : 4) void markov_topk(StepArgs a, int tile_cols) {
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int b = blockIdx.x, j = blockIdx.y;
  const int k = a.topk;
  const size_t row = static_cast<size_t>(b) * a.gamma + j;
  __shared__ float arow_s[kMaxRank];
  __shared__ __align__(16) float tmax[kTopkThreads];
  __shared__ int tiles[kTileCap];
  __shared__ int c1s[kCand1Cap];
  __shared__ __align__(16) float c1v[kCand1Cap];
  __shared__ int c2s[kCand2Cap];
  __shared__ __align__(16) float ev[kCand2Cap * kSeg];
  __shared__ int counter[3];
  __shared__ unsigned kmin[2];             // k-th largest searches: minimum key, values counted
  __shared__ int kcnt[2];
  __shared__ float selv[kMaxTopk];
  __shared__ int seli[kMaxTopk];

  const WT* ar = a_operand_row<WT>(a, b, j);
  for (int i = tid; i < a.r; i += kTopkThreads) arow_s[i] = to_f32(ar[i]);
  if (tid < kMaxTopk) {            // a row without k orderable values (NaN) reports -1 ids
    selv[tid] = kNegInf;
    seli[tid] = -1;
  }
  const float* pm = a.p_m + row * a.P;
  const float* sm = a.segmax + row * a.S;
  const float* urow = a.U + row * static_cast<size_t>(a.V);
  // per-thread maximum of the tile maxima; the first kKeep of this thread's
  // tiles stay in registers for the filter below
  constexpr int kKeep = 8;
  float keep[kKeep];
  float mt = kNegInf;
#pragma unroll
  for (int u = 0; u < kKeep; ++u) {
    const int p = u * kTopkThreads + tid;
    keep[u] = p < a.Pn ? pm[p] : kNegInf;
  }
#pragma unroll
  for (int u = 0; u < kKeep; ++u) mt = fmaxf(mt, keep[u]);
  for (int p = kKeep * kTopkThreads + tid; p < a.Pn; p += kTopkThreads) mt = fmaxf(mt, pm[p]);
  tmax[tid] = mt;
  if (tid < 3) counter[tid] = 0;
  if (tid < 2) { kmin[tid] = ~0u; kcnt[tid] = 0; }
  __syncthreads();
  // threads past the partial count hold -inf (no tile): rank among the others
  const float th00 = kth_largest(tmax, min(kTopkThreads, a.Pn), k, &kmin[0], &kcnt[0]);
  // tiles that can hold a segment >= theta00
#pragma unroll
  for (int u = 0; u < kKeep; ++u) {
    if (keep[u] >= th00 && keep[u] != kNegInf) {
      const int slot = atomicAdd(&counter[0], 1);
      if (slot < kTileCap) tiles[slot] = u * kTopkThreads + tid;
    }
  }
  for (int p = kKeep * kTopkThreads + tid; p < a.Pn; p += kTopkThreads) {
    if (pm[p] >= th00) {
      const int slot = atomicAdd(&counter[0], 1);
      if (slot < kTileCap) tiles[slot] = p;
    }
  }
  __syncthreads();
  const int nt = counter[0];
  const int spt = tile_cols / kSeg;      // segments per tile
  bool overflow = nt > kTileCap;
  if (!overflow) {
    for (int e0 = 0; e0 < nt * spt; e0 += kFoldBatch * kTopkThreads) {
      float v[kFoldBatch];
      int sg[kFoldBatch];
#pragma unroll
      for (int u = 0; u < kFoldBatch; ++u) {
        const int e = e0 + u * kTopkThreads + tid;
        sg[u] = e < nt * spt ? tiles[e / spt] * spt + e % spt : a.S;
        v[u] = sg[u] < a.S ? sm[sg[u]] : kNegInf;
      }
#pragma unroll
      for (int u = 0; u < kFoldBatch; ++u) {
        if (sg[u] < a.S && v[u] >= th00) {
          const int slot = atomicAdd(&counter[1], 1);
          if (slot < kCand1Cap) { c1s[slot] = sg[u]; c1v[slot] = v[u]; }
        }
      }
    }
    __syncthreads();
    const int n1 = counter[1];
    overflow = n1 > kCand1Cap;
    if (!overflow) {
      const float th = kth_largest(c1v, n1, k, &kmin[1], &kcnt[1]);
      for (int i = tid; i < n1; i += kTopkThreads) {
        if (c1v[i] >= th) {
          const int slot = atomicAdd(&counter[2], 1);
          if (slot < kCand2Cap) c2s[slot] = c1s[i];
        }
      }
      __syncthreads();
      const int n2 = counter[2];
      overflow = n2 > kCand2Cap;
      if (!overflow) {
        const WT* Bm = static_cast<const WT*>(a.Bm);
        const int q = tid % kSliceThreads;
        for (int c0 = 0; c0 < n2; c0 += kTopkThreads / kSliceThreads) {
          const int c = c0 + tid / kSliceThreads;
          const bool on = c < n2;          // uniform across each 16-lane slice group
          const int v0 = on ? c2s[c] * kSeg : 0;
          float acc[kSeg];
#pragma unroll
          for (int i = 0; i < kSeg; ++i) acc[i] = 0.f;
          if (BMT && on) {
            // bf16 only: column v0 + i is row v0 + i of BmT (r contiguous
            // values); the thread takes 8-wide k-chunks q, q + 16, ... of all
            // 8 columns (whole 16-byte pieces of rows, instead of 16 useful
            // bytes of each of r Bm rows)
            const uint16_t* BmT = static_cast<const uint16_t*>(a.BmT);
            for (int k0 = 8 * q; k0 < a.r; k0 += 8 * kSliceThreads) {
              u32x4 raw[kSeg];
#pragma unroll
              for (int i = 0; i < kSeg; ++i)
                raw[i] = *reinterpret_cast<const u32x4*>(BmT + static_cast<size_t>(v0 + i) * a.r + k0);
              float am[8];
#pragma unroll
              for (int t = 0; t < 8; ++t) am[t] = arow_s[k0 + t];
#pragma unroll
              for (int i = 0; i < kSeg; ++i) {
                float col[8];
                SegRows<uint16_t>::unpack(raw[i], col);
#pragma unroll
                for (int t = 0; t < 8; ++t) acc[i] = fmaf(am[t], col[t], acc[i]);
              }
            }
          } else if (on) {
            // rows q, q+16, ... of Bm, issued RB at a time in packed form
            constexpr int RB = SegRows<WT>::kBatch;
            for (int k0 = q; k0 < a.r; k0 += RB * kSliceThreads) {
              typename SegRows<WT>::Raw raw[RB];
#pragma unroll
              for (int u = 0; u < RB; ++u) {
                const int kk = k0 + u * kSliceThreads;
                raw[u] = SegRows<WT>::load(Bm, kk < a.r ? kk : 0, v0, a.V);
              }
#pragma unroll
              for (int u = 0; u < RB; ++u) {
                const int kk = k0 + u * kSliceThreads;
                const float am = kk < a.r ? arow_s[kk] : 0.f;
                float col[kSeg];
                SegRows<WT>::unpack(raw[u], col);
#pragma unroll
                for (int i = 0; i < kSeg; ++i) acc[i] = fmaf(am, col[i], acc[i]);
              }
            }
          }
#pragma unroll
          for (int i = 0; i < kSeg; ++i) {
#pragma unroll
            for (int o = 1; o < kSliceThreads; o <<= 1) acc[i] += __shfl_xor(acc[i], o);
          }
          if (on && q == 0) {
#pragma unroll
            for (int i = 0; i < kSeg; ++i)
              ev[c * kSeg + i] = (v0 + i < a.V) ? urow[v0 + i] + acc[i] : kNegInf;
          }
        }
        __syncthreads();
        const int ne = n2 * kSeg;
        for (int e = tid; e < ne; e += kTopkThreads) {
          const float x = ev[e];
          const int ix = c2s[e / kSeg] * kSeg + e % kSeg;
          int rank = 0;
          for (int c = 0; c < n2; ++c) {       // 8 columns of one candidate segment per step
            const int v0 = c2s[c] * kSeg;
            const f32x4 lo = *reinterpret_cast<const f32x4*>(&ev[c * kSeg]);
            const f32x4 hi = *reinterpret_cast<const f32x4*>(&ev[c * kSeg + 4]);
#pragma unroll
            for (int i = 0; i < 4; ++i)
              rank += ranks_before(lo[i], v0 + i, x, ix) + ranks_before(hi[i], v0 + 4 + i, x, ix);
          }
          if (rank < k) { selv[rank] = x; seli[rank] = ix; }
        }
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
      for (int v = tid; v < a.V; v += kTopkThreads) {
        const float x = recompute_logit<WT>(a, arow_s, urow, v);
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
  if (w == 0) {  // softmax over the k candidates at T = 1, summed in rank order
    const size_t o = row * k;
    const float e = lane < k ? __expf(selv[lane] - selv[0]) : 0.f;
    float ssum = 0.f;
    for (int t = 0; t < k; ++t) ssum += __shfl(e, t);
    if (lane < k) {
      a.topk_idx[o + lane] = seli[lane];
      a.topk_prob[o + lane] = e / ssum;
    }
  }
}

// ---------------------------------------------------------------------------
// Top-k after the resident chain: one workgroup per (request, position) folds
// the per-workgroup partials (fold_request), then merges the per-workgroup
// candidate lists (each the k largest order keys of one workgroup's columns,
// sorted descending; best_key orders by value descending, then index
// ascending, and 0 pads short lists).  Exact: let list L's head rank r_L among
// the live heads.  Entry p of list L is preceded by the p entries before it in
// L and by the r_L heads larger than L's head, so it can be among the k
// largest only if p + r_L < k.  That leaves at most k(k+1)/2 candidates, each
// ranked by counting the larger ones (live keys are distinct; padding, equal
// to 0, ranks after every live key and never reaches the first k, since
// k <= V).
constexpr int kMaxMergeCand = kMaxTopk * (kMaxTopk + 1) / 2;

// Number of keys[0..n) greater than x, for keys in LDS (16-byte aligned) read
// by every thread alike: two keys per 16-byte load, 32 keys per batch in
// flight (the count is bound by LDS latency, not by the compares).
__device__ __forceinline__ int count_greater(const unsigned long long* keys, int n, unsigned long long x) {
  typedef unsigned long long u64x2 __attribute__((ext_vector_type(2)));
  const u64x2* k2 = reinterpret_cast<const u64x2*>(keys);
  int c = 0, f = 0;
  for (; f + 32 <= n; f += 32) {
    u64x2 v[16];
#pragma unroll
    for (int q = 0; q < 16; ++q) v[q] = k2[f / 2 + q];
#pragma unroll
    for (int q = 0; q < 16; ++q) c += (v[q].x > x) + (v[q].y > x);
  }
  for (; f < n; ++f) c += keys[f] > x;
  return c;
}

__global__ __launch_bounds__(kTopkThreads) void markov_topk_lists(StepArgs a) {
  const int tid = threadIdx.x, w = tid >> 6, lane = tid & 63;
  const int b = blockIdx.x, j = blockIdx.y;
  const int k = a.topk, L = a.nlist;
  const size_t row = static_cast<size_t>(b) * a.gamma + j;
  __shared__ __align__(16) unsigned long long hk[kMaxLists];
  __shared__ int act[kMaxTopk];
  __shared__ int nlive;
  __shared__ __align__(16) unsigned long long mk[kMaxMergeCand];
  __shared__ unsigned long long sel[kMaxTopk];
  __shared__ unsigned long long thr_s[kTopkThreads / kWave];
  __shared__ int nsurv;

  const unsigned long long* ck = a.cand_key + row * L * k;
  // the head's load lands with the fold's (stored after it, so that the fold's
  // loads are not held back by a wait for it)
  const unsigned long long head = tid < L ? ck[static_cast<size_t>(tid) * k] : 0ull;
  if (tid == 0) {
    nlive = 0;
    nsurv = 0;
  }
  FoldOut fo{};
  fold_request(a, b, j, true, &fo);                   // thread 0 stores fo at the end
  // from here on only LDS is shared between threads
  hk[tid] = head;
  lds_barrier();
  // The heads of rank < k, exactly, without counting 256 x 256: the k-th
  // largest head of each wave's 64 is at most the k-th largest of all, so
  // their maximum t bounds every head of rank < k from below.  Heads >= t
  // survive (into mk, free until the gather), and a survivor's rank among
  // the survivors is its rank among all heads, since every larger head is
  // a survivor too.  (A wave with fewer than k live heads gives t_w = 0.)
  {
    const int rw = count_greater(hk + w * kWave, kWave, head);
    unsigned long long tw = rw == k - 1 ? head : 0ull;
#pragma unroll
    for (int o = 1; o < kWave; o <<= 1) {
      const unsigned long long ot = __shfl_xor(tw, o);
      tw = ot > tw ? ot : tw;
    }
    if (lane == 0) thr_s[w] = tw;
  }
  lds_barrier();
  unsigned long long t = thr_s[0];
#pragma unroll
  for (int i = 1; i < kTopkThreads / kWave; ++i) t = thr_s[i] > t ? thr_s[i] : t;
  if (head != 0ull && head >= t) mk[atomicAdd(&nsurv, 1)] = head;
  lds_barrier();
  if (head != 0ull && head >= t) {
    const int rank = count_greater(mk, nsurv, head);
    if (rank < k) {
      act[rank] = tid;
      atomicAdd(&nlive, 1);
    }
  }
  lds_barrier();
  // candidates of the list of head rank r: entries p < k - r, stored from
  // offset r k - r (r - 1) / 2
  const int na = nlive;
  const int nc = na * k - na * (na - 1) / 2;
  for (int e = tid; e < nc; e += kTopkThreads) {
    int r = 0;
    while ((r + 1) * k - (r + 1) * r / 2 <= e) ++r;
    const int p = e - (r * k - r * (r - 1) / 2);
    mk[e] = ck[static_cast<size_t>(act[r]) * k + p];
  }
  lds_barrier();
  for (int e = tid; e < nc; e += kTopkThreads) {
    const unsigned long long key = mk[e];
    const int rank = count_greater(mk, nc, key);
    if (rank < k && key != 0ull) sel[rank] = key;
  }
  lds_barrier();
  if (w == 0) {  // softmax over the k candidates at T = 1, summed in rank order
    const size_t o = row * k;
    const float v = lane < k ? best_value(sel[lane]) : 0.f;
    const float e = lane < k ? __expf(v - __shfl(v, 0)) : 0.f;
    float ssum = 0.f;
    for (int t = 0; t < k; ++t) ssum += __shfl(e, t);
    if (lane < k) {
      a.topk_idx[o + lane] = best_index(sel[lane]);
      a.topk_prob[o + lane] = e / ssum;
    }
  }
  if (tid == 0) store_fold(a, static_cast<int>(row), true, fo);
  // last: the compiler puts a wait for every outstanding store ahead of a
  // loop that stores and does not load; here it waits for nothing that the
  // kernel's end would not wait for anyway
  clear_wait_tree(a);
}

// ---------------------------------------------------------------------------
// host-side launchers

// partial stride: enough for the narrowest tiles (64 columns, resident chain)
size_t markov_partials(int64_t V) { return static_cast<size_t>((V + 63) / 64); }
size_t markov_segments(int64_t V) { return static_cast<size_t>((V + kSeg - 1) / kSeg); }

template <int RG, int KS>
static void launch_bf16(const StepArgs& a, hipStream_t s) {
  const dim3 grid((a.V + kMarkovTile - 1) / kMarkovTile, (a.B + 16 * RG - 1) / (16 * RG));
  if (a.sample) hipLaunchKernelGGL((markov_step_bf16<RG, KS, true>), grid, dim3(kWave * KS), 0, s, a);
  else hipLaunchKernelGGL((markov_step_bf16<RG, KS, false>), grid, dim3(kWave * KS), 0, s, a);
}

// wide kernel plan: one request group of 16 per wave (up to 8 waves), each
// wave loading at most 2 of a tile's 32-row Bm chunks, and as many
// workgroups as the device holds at once, each over a contiguous tile range.
// The grid's x extent is padded to a multiple of 8 (the padding returns at
// once): workgroups are dealt to the 8 XCDs by linear index, so the ny
// workgroups of one tile range then share an XCD and its L2.
struct WidePlan {
  const void* fn;
  void (*launch)(const StepArgs&, int, dim3, int, hipStream_t);
  // the same kernel without the U~ dump stores (a chain with no dump): the
  // same registers and LDS, so the plan (from fn's occupancy) holds for it
  void (*launch_nodump)(const StepArgs&, int, dim3, int, hipStream_t);
  // no dump, and the step stores BmT as well (position 0 of a top-k chain)
  void (*launch_nodump_bmt)(const StepArgs&, int, dim3, int, hipStream_t);
  int nw, ny, tpw, nx, gx;
  size_t lds;
};

template <int NCH, int CPW, bool SAMPLE, bool STATS, bool DUMP = true, bool BMT = false>
static void launch_wide_kernel(const StepArgs& a, int tpw, dim3 grid, int nw, hipStream_t s) {
  hipLaunchKernelGGL((markov_step_wide<NCH, CPW, SAMPLE, STATS, DUMP, BMT>), grid, dim3(kWave * nw),
                     wide_ops_bytes(NCH) + (SAMPLE ? kWideSeedBytes : 0), s, a, tpw);
}

// stats = false: the block-logits variant (never sampled)
template <int NCH, int CPW>
static void pick_wide(bool sample, bool stats, WidePlan* p) {
  if (!stats) {
    p->fn = reinterpret_cast<const void*>(&markov_step_wide<NCH, CPW, false, false>);
    p->launch = &launch_wide_kernel<NCH, CPW, false, false>;
    p->launch_nodump = p->launch;
    p->launch_nodump_bmt = nullptr;
    p->lds = wide_ops_bytes(NCH);
    return;
  }
  p->fn = sample ? reinterpret_cast<const void*>(&markov_step_wide<NCH, CPW, true, true>)
                 : reinterpret_cast<const void*>(&markov_step_wide<NCH, CPW, false, true>);
  p->launch = sample ? &launch_wide_kernel<NCH, CPW, true, true> : &launch_wide_kernel<NCH, CPW, false, true>;
  p->launch_nodump = sample ? &launch_wide_kernel<NCH, CPW, true, true, false>
                            : &launch_wide_kernel<NCH, CPW, false, true, false>;
  p->launch_nodump_bmt = sample ? &launch_wide_kernel<NCH, CPW, true, true, false, true>
                                : &launch_wide_kernel<NCH, CPW, false, true, false, true>;
  p->lds = wide_ops_bytes(NCH) + (sample ? kWideSeedBytes : 0);
}

// workgroups of fn (with nw waves) resident per compute unit, cached
static int wide_occupancy(const void* fn, int nw, size_t lds) {
  static std::mutex mu;
  static std::map<std::pair<const void*, int>, int> cache;
  std::lock_guard<std::mutex> lock(mu);
  const auto key = std::make_pair(fn, nw);
  auto it = cache.find(key);
  if (it != cache.end()) return it->second;
  int nb = 0;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&nb, fn, kWave * nw, lds) != hipSuccess || nb < 1) nb = 1;
  cache[key] = nb;
  return nb;
}

// false: the shape takes another kernel (fp32 tables, a rank other than 32,
// 64, 128 or 256, or, for the chain, B <= 16)
static bool wide_plan(bool bf16, bool sample, int B, int gamma, int r, int V, WidePlan* p, bool stats = true) {
  const int nch = r / 32;
  if (!bf16 || (stats && B <= 16) || r % 32 || (nch != 1 && nch != 2 && nch != 4 && nch != 8)) return false;
  // the kernel's buffer offsets are 32-bit and its dropped accesses use 2^31:
  // every array it addresses must stay below 2 GiB
  if (static_cast<size_t>(B) * gamma * V * 4 >= (static_cast<size_t>(1) << 31)) return false;
  const int groups = (B + 15) / 16;
  // at least nch / 2 waves, so that a wave loads at most 2 chunks (waves
  // past the last request only load and store operands)
  p->nw = min(8, max(groups, nch / 2));
  p->ny = (groups + p->nw - 1) / p->nw;
  const bool two = nch > p->nw;                        // chunks per wave: 1 or 2
  switch (nch * 2 + (two ? 1 : 0)) {
    case 2: pick_wide<1, 1>(sample, stats, p); break;
    case 4: pick_wide<2, 1>(sample, stats, p); break;
    case 8: pick_wide<4, 1>(sample, stats, p); break;
    case 9: pick_wide<4, 2>(sample, stats, p); break;
    case 16: pick_wide<8, 1>(sample, stats, p); break;
    default: pick_wide<8, 2>(sample, stats, p); break;
  }
  const int ntiles = (V + kWideCols - 1) / kWideCols;
  const int slots = max(1, wide_occupancy(p->fn, p->nw, p->lds) * max(1, device_info().cus));
  const int nx = max(1, slots / p->ny);
  p->tpw = (ntiles + nx - 1) / nx;
  p->nx = (ntiles + p->tpw - 1) / p->tpw;
  p->gx = (p->nx + 7) / 8 * 8;
  return true;
}

static int partial_count(const StepArgs& a) { return (a.V + a.tile_cols - 1) / a.tile_cols; }

int markov_tile_cols(bool bf16, bool sample, int B, int gamma, int r, int V) {
  if (!bf16) return kMarkovTileF32;
  WidePlan p{};
  return wide_plan(bf16, sample, B, gamma, r, V, &p) ? p.tpw * kWideCols : kMarkovTile;
}

bool markov_bmt_in_step(bool sample, int B, int gamma, int r, int V) {
  WidePlan p{};
  return static_cast<size_t>(r) * V * 2 < (static_cast<size_t>(1) << 31) && wide_plan(true, sample, B, gamma, r, V, &p);
}

hipError_t launch_markov_position(StepArgs a, bool bf16, hipStream_t s) {
  a.Pn = partial_count(a);
  if (bf16) {
    WidePlan p{};
    if (wide_plan(bf16, a.sample, a.B, a.gamma, a.r, a.V, &p)) {
      if (p.tpw * kWideCols != a.tile_cols) return hipErrorInvalidValue;   // plan changed since tile_cols was set
      if (a.bmt_step && a.logits_out) return hipErrorInvalidValue;      // the BmT variant has no dump
      (a.logits_out ? p.launch : a.bmt_step && a.j == 0 ? p.launch_nodump_bmt : p.launch_nodump)(
          a, p.tpw, dim3(p.gx, p.ny), p.nw, s);
    } else if (a.r % 128 == 0) {
      // small batches split r over waves so that a step has enough waves in flight
      launch_bf16<1, 4>(a, s);
    } else if (a.r % 64 == 0) {
      launch_bf16<1, 2>(a, s);
    } else {
      launch_bf16<1, 1>(a, s);
    }
  } else {
    const dim3 grid(a.Pn, a.B);
    hipLaunchKernelGGL(markov_step_f32, grid, dim3(256), 0, s, a);
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(markov_merge, dim3(a.B), dim3(kMergeThreads), 0, s, a);
  return hipGetLastError();
}

// Bm [r, V] -> BmT [V, r] (bf16) through a 32 (rows of Bm) x 64 (columns)
// LDS tile: 16-byte loads along a Bm row, 16-byte stores along a BmT row.
// V % 8 == 0 and r % 32 == 0, so every 8-element piece is whole.
constexpr int kTrR = 32, kTrC = 64;
__global__ __launch_bounds__(256) void transpose_bm_bf16(const uint16_t* __restrict__ Bm,
                                                        uint16_t* __restrict__ BmT, int r, int V) {
  __shared__ uint16_t tile[kTrR][kTrC + 8];
  const int c0 = blockIdx.x * kTrC, k0 = blockIdx.y * kTrR, t = threadIdx.x;
  {
    const int kr = t >> 3, cc = (t & 7) * 8;             // Bm row k0 + kr, columns c0 + cc ..
    if (c0 + cc < V) {
      const u32x4 v = *reinterpret_cast<const u32x4*>(Bm + static_cast<size_t>(k0 + kr) * V + c0 + cc);
      *reinterpret_cast<u32x4*>(&tile[kr][cc]) = v;
    }
  }
  __syncthreads();
  {
    const int c = t >> 2, kk = (t & 3) * 8;              // BmT row c0 + c, k0 + kk ..
    if (c0 + c < V) {
      uint32_t w[4];
#pragma unroll
      for (int i = 0; i < 4; ++i)
        w[i] = static_cast<uint32_t>(tile[kk + 2 * i][c]) | (static_cast<uint32_t>(tile[kk + 2 * i + 1][c]) << 16);
      *reinterpret_cast<u32x4*>(BmT + static_cast<size_t>(c0 + c) * r + k0 + kk) = u32x4{w[0], w[1], w[2], w[3]};
    }
  }
}

size_t markov_bmt_bytes(int64_t r, int64_t V) { return (static_cast<size_t>(r) * V * 2 + 255) / 256 * 256; }

// The recompute reads, per (request, position) and per candidate segment of 8
// columns, 16 bytes from each of r Bm rows (whole 128-byte lines); with BmT it
// reads 8 rows of r values, after a copy that reads and writes r V values.
bool markov_bmt_pays(int64_t B, int64_t gamma, int64_t V, int64_t r, int32_t topk) {
  const double rows = static_cast<double>(B) * gamma, segs = topk;
  const double strided = rows * segs * r * 128.0;
  const double copied = 2.0 * r * V * 2.0 + rows * segs * 8.0 * r * 2.0;
  return copied < strided;
}

hipError_t launch_markov_finish(StepArgs a, bool bf16, hipStream_t s) {
  a.Pn = partial_count(a);
  const dim3 grid(a.B, a.gamma);
  if (a.resident) {                        // resident chain: fold, then merge its candidate lists
    a.Pn = a.nlist;                        // one partial per workgroup
    if (a.topk == 0) hipLaunchKernelGGL(markov_fold, grid, dim3(kMergeThreads), 0, s, a);
    else hipLaunchKernelGGL(markov_topk_lists, grid, dim3(kTopkThreads), 0, s, a);
    return hipGetLastError();
  }
  if (a.topk == 0) return hipSuccess;
  if (bf16 && a.BmT) {
    if (!a.bmt_step) {                     // else position 0's step kernel stored it
      const dim3 tg((a.V + kTrC - 1) / kTrC, a.r / kTrR);
      hipLaunchKernelGGL(transpose_bm_bf16, tg, dim3(256), 0, s, static_cast<const uint16_t*>(a.Bm),
                         static_cast<uint16_t*>(const_cast<void*>(a.BmT)), a.r, a.V);
    }
    hipLaunchKernelGGL((markov_topk<uint16_t, true>), grid, dim3(kTopkThreads), 0, s, a, a.tile_cols);
  } else if (bf16)
    hipLaunchKernelGGL(markov_topk<uint16_t>, grid, dim3(kTopkThreads), 0, s, a, a.tile_cols);
  else
    hipLaunchKernelGGL(markov_topk<float>, grid, dim3(kTopkThreads), 0, s, a, a.tile_cols);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Teacher-forced block logits ("DSpark 论文精读", §2.3 apply_block_logits;
// "DeepSpec 训练全流程详解", §3.3 prev_token_ids = [anchor, t_1, ...]):
// U~[m, v] = U[m, v] + sum_k A[prev[m], k] Bm[k, v] for every row m at once.
// bf16 tables with r in {32, 64, 128, 256} take the wide step kernel in its
// store-only form (rows as requests, the previous token of row m given);
// other shapes take this kernel: one thread per (row, column), the A row in
// LDS, a plain dot product over r (Bm is re-read per row: a fallback for
// fp32 tables and uncommon ranks).
template <typename WT>
__global__ __launch_bounds__(256) void block_logits_generic(const float* __restrict__ U, const int32_t* __restrict__ prev,
                                                            const WT* __restrict__ A, const WT* __restrict__ Bm, int V,
                                                            int r, float* __restrict__ out) {
  __shared__ float arow[kMaxRank];
  const int m = blockIdx.y, tid = threadIdx.x;
  const int pv = min(max(prev[m], 0), V - 1);         // the gathered row stays inside A
  for (int k = tid; k < r; k += 256) arow[k] = to_f32(A[static_cast<size_t>(pv) * r + k]);
  __syncthreads();
  const int v = blockIdx.x * 256 + tid;
  if (v >= V) return;
  float bias = 0.f;
  for (int k = 0; k < r; ++k) bias = fmaf(arow[k], to_f32(Bm[static_cast<size_t>(k) * V + v]), bias);
  out[static_cast<size_t>(m) * V + v] = U[static_cast<size_t>(m) * V + v] + bias;
}

// vec: bf16 tables, V % 8 == 0 and 16-byte aligned operands (the MFMA kernel)
hipError_t launch_block_logits(const float* U, const int32_t* prev, const void* A, const void* Bm, bool vec,
                               int M, int V, int r, float* out, hipStream_t s, bool bf16) {
  StepArgs a{};
  a.U = U;
  a.anchor = prev;
  a.A = A;
  a.Bm = Bm;
  a.B = M;
  a.gamma = 1;
  a.j = 0;
  a.V = V;
  a.r = r;
  a.logits_out = out;
  // the wide kernel addresses U and the output with 32-bit offsets: rows go
  // in chunks of at most 2 GiB of logits each (multiples of 16 rows)
  const int chunk = static_cast<int>(((static_cast<size_t>(1) << 31) - 1) / (static_cast<size_t>(V) * 4)) / 16 * 16;
  WidePlan p{};
  if (vec && chunk > 0 && wide_plan(true, false, min(M, chunk), 1, r, V, &p, false)) {
    for (int m0 = 0; m0 < M; m0 += chunk) {
      StepArgs c = a;
      c.B = min(chunk, M - m0);
      c.U = U + static_cast<size_t>(m0) * V;
      c.anchor = prev + m0;
      c.logits_out = out + static_cast<size_t>(m0) * V;
      if (m0 > 0 && !wide_plan(true, false, c.B, 1, r, V, &p, false)) return hipErrorInvalidValue;
      p.launch(c, p.tpw, dim3(p.gx, p.ny), p.nw, s);
      const hipError_t e = hipGetLastError();
      if (e != hipSuccess) return e;
    }
  } else {
    const dim3 grid((V + 255) / 256, M);
    if (bf16)
      hipLaunchKernelGGL(block_logits_generic<uint16_t>, grid, dim3(256), 0, s, U, prev,
                         static_cast<const uint16_t*>(A), static_cast<const uint16_t*>(Bm), V, r, out);
    else
      hipLaunchKernelGGL(block_logits_generic<float>, grid, dim3(256), 0, s, U, prev, static_cast<const float*>(A),
                         static_cast<const float*>(Bm), V, r, out);
  }
  return hipGetLastError();
}

}  // namespace dspark
