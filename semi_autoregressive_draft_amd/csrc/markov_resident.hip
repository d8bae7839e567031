// Resident Markov chain for small batches (bf16; B = 1 with r = 64, 128 or 256,
// or 1 < B <= 16 with r = 256).
//
// Same computation as the per-position step kernels (markov.hip):
//   U~_j[v] = U[b, j, v] + sum_k A[x_{j-1}, k] * Bm[k, v],  x_j = argmax (or
//   Gumbel-max) of U~_j, with one (max, sum-exp, best) partial per
//   (request, position, workgroup) for the fold after the chain.
// "Qwen3.8-Flash-Next DSpark 训练实验", Baseline 架构/Markov 顺序修正;
// "DSpark 论文精读", §2.2.
//
// At small B each position is bound by streaming all of Bm (r x V bf16) from
// HBM, gamma times.  Bm fits on chip instead: one persistent workgroup per
// compute unit loads its share of Bm once, already transposed into MFMA B
// operands, keeps it in registers (8 groups of 64 columns per workgroup) and in
// LDS (the rest), and runs all gamma positions.  Between positions the
// workgroups meet at a grid-wide wait: each one raises the argmax keys of its
// requests (atomic max), then adds one arrival to a counter and waits until all
// workgroups have arrived; the next position's previous token is the final key.
// The wait is a two-level tree so that no address sees more than 16
// workgroups: each workgroup raises its group's key and counter (groups of 16
// workgroups); the last arriver of a group, known from the counter's old
// value, raises the request's final key and the top counter; the last group to
// arrive there writes one release flag per group, and each workgroup polls its
// group's flag.  Every step uses atomics or loads at device scope and waits
// for their return before the next, so a key is final when its counter says
// so.  The grid is one workgroup per compute unit, and the launcher checks
// with the occupancy query that a compute unit holds one: on a device running
// nothing else every workgroup is resident at once, and work on other streams
// can only delay a workgroup's start (its own workgroups finish without
// waiting for this kernel).  Each wait is bounded in time, so every wave
// terminates whatever happens; a wait that runs out writes the call's number
// into word 0 of the wait tree, and the fold then returns -1 tokens.  (A
// cooperative launch would give the same residency guarantee but costs about
// 11 us of dispatch gap on each side of the kernel.)
//
// The wait tree and the keys are zero when a call starts: the workspace is
// zero-filled before its first use and the finish kernels clear both again.
//
// The epilogue leaves U~_j in LDS (over the U_j rows it read, two buffers
// alternating by position).  While wave 0 walks the wait tree, with top-k
// the list waves select this workgroup's k best U~_j per request into a
// sorted list of 64-bit order keys (best_key: value descending, index
// ascending; 0 pads lists of workgroups with fewer than k live columns; the
// finish kernel merges the lists exactly), and the helper waves fetch
// U_{j+1}, copy U~_j to the dump and store the workgroup's partial and the
// previous position's lists.  The waves that lead the next position (wave 0
// and the list waves) issue no plain stores, so no wait for store
// completion falls on them.
//
// Group layout: group G covers columns 64G .. 64G+63 and belongs to workgroup
// G mod nwg.  For each 32-row chunk q of r, lane (g = lane/16, n = lane%16)
// holds four B operands (c = 0..3): rows 32q+8g .. 32q+8g+7 of column
// 64G+4n+c, built from eight 8-byte row loads by byte permutes.  With the A
// operand "request n, rows 32q+8g..+7 of A[x_{j-1}]", accumulator c of lane
// (g, n) holds requests 4g..4g+3 for column 64G+4n+c.
#include "common.h"
#include "internal.h"
#include "markov_dev.h"

namespace dspark {

// barrier for LDS traffic only: waits for this wave's LDS operations, not its
// global loads and stores (__syncthreads waits for both)
__device__ __forceinline__ void res_lds_barrier() {
  __builtin_amdgcn_s_waitcnt(0xC07F);
  asm volatile("s_barrier" ::: "memory");
}

constexpr int kResThreads = 512;
constexpr int kResWaves = kResThreads / kWave;
constexpr int kResCols = 64;                  // vocabulary columns per group
constexpr int kResMaxB = kResidentMaxB;
constexpr size_t kResLdsMax = 144 * 1024;     // dynamic LDS: LDS groups + U_j rows (static: ~15 KB)

struct ResidentArgs {
  int nwg;             // workgroups (one per compute unit)
  int G;               // groups: ceil(V / 64)
  int T;               // groups per workgroup: ceil(G / nwg)
  int nreg;            // groups per workgroup held in registers (kResWaves * RGW)
  int nlds;            // groups per workgroup held in LDS
  unsigned* sync;      // wait tree, kSyncWords words (zero at launch)
  unsigned long long wait_ticks;   // bound of one grid-wide wait, wall-clock ticks
};

// Wait-tree layout: internal.h (kSync*), shared with the finish kernels that clear it.

__device__ __forceinline__ unsigned atomic_add_dev(unsigned* p, unsigned v) {
  return __hip_atomic_fetch_add(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ unsigned long long atomic_max_dev(unsigned long long* p, unsigned long long v) {
  return __hip_atomic_fetch_max(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
template <typename T>
__device__ __forceinline__ T load_dev(const T* p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
// keep the value live so that the wave waits for the atomic's return here
__device__ __forceinline__ void returned(unsigned long long v) { asm volatile("" ::"v"(v) : "memory"); }

// Position j's keys (lanes b < B of wave 0 hold request b's workgroup key)
// into the tree; returns after the final keys a.best[., j] are known to this
// workgroup (j + 1 < gamma) or after its part is done (last position).
__device__ void chain_tree(const StepArgs& a, const ResidentArgs& ra, int wg, int j,
                           unsigned long long key, int lane, bool wait) {
  unsigned* sy = ra.sync;
  unsigned long long* gkeys = reinterpret_cast<unsigned long long*>(sy + kSyncKeys);
  const int grp = wg / kFanIn, ng = (ra.nwg + kFanIn - 1) / kFanIn;
  const unsigned gsize = static_cast<unsigned>(min(kFanIn, ra.nwg - kFanIn * grp));
  unsigned long long* gk = gkeys + (j * kFanIn + grp) * kResMaxB;
  unsigned long long r0 = 0;
  if (lane < a.B) r0 = atomic_max_dev(gk + lane, key);
  returned(r0);
  int last = 0;
  if (lane == 0) last = atomic_add_dev(sy + kSyncGroupCnt + 64 * grp, 1u) == gsize * (j + 1) - 1;
  last = __shfl(last, 0);
  if (last) {                                            // group complete: push its key
    unsigned long long r1 = 0;
    if (lane < a.B) r1 = atomic_max_dev(a.best + lane * a.gamma + j, load_dev(gk + lane));
    returned(r1);
    int top = 0;
    if (lane == 0) top = atomic_add_dev(sy + kSyncTopCnt, 1u) == static_cast<unsigned>(ng) * (j + 1) - 1;
    top = __shfl(top, 0);
    if (top && lane < ng) {                              // all groups in: release them
      // the lane's flag address, formed here: hoisted out of the position
      // loop it would be spilled and reloaded on this path
      unsigned off = 64u * static_cast<unsigned>(lane);
      asm volatile("" : "+v"(off));
      __hip_atomic_store(sy + kSyncRelease + off, static_cast<unsigned>(j + 1), __ATOMIC_RELAXED,
                         __HIP_MEMORY_SCOPE_AGENT);
    }
  }
  if (!wait) return;
  if (lane == 0) {
    const unsigned long long t0 = wall_clock64();
    while (load_dev(sy + kSyncRelease + 64 * grp) < static_cast<unsigned>(j + 1)) {
      if (wall_clock64() - t0 > ra.wait_ticks) {
        __hip_atomic_store(sy + kSyncTimeout, a.epoch, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        break;
      }
      __builtin_amdgcn_s_sleep(1);
    }
  }
}

// Epilogue of one group for the lane's requests 4g + ii (ii < QN): add U_j
// (from LDS, replaced there by U~_j), optional U~ dump, the 16-lane max /
// sum-exp / argmax of the group, folded into the wave's running states (the
// same in all 16 lanes of a row).
template <int QN, bool SAMPLE>
__device__ __forceinline__ void resident_epilogue(const StepArgs& a, const f32x4 (&acc)[4], float* urows,
                                                  int gid, int g, int n, LseState (&run)[QN],
                                                  ArgState (&best)[QN]) {
  const size_t V = static_cast<size_t>(a.V);
  const int col = gid * kResCols + 4 * n;
  const bool cok = col < a.V;
#pragma unroll
  for (int ii = 0; ii < QN; ++ii) {
    const int b = 4 * g + ii;
    const bool live = b < a.B && cok;
    const size_t row = static_cast<size_t>(b) * a.gamma + a.j;
    float x[4];
    if (live) {
      f32x4* up = reinterpret_cast<f32x4*>(urows + b * kResCols + 4 * n);
      const f32x4 u = *up;
#pragma unroll
      for (int c = 0; c < 4; ++c) x[c] = acc[c][ii] + u[c];
      const f32x4 xv{x[0], x[1], x[2], x[3]};
      *up = xv;
    } else {
#pragma unroll
      for (int c = 0; c < 4; ++c) x[c] = kNegInf;
    }
    float M = fmaxf(fmaxf(x[0], x[1]), fmaxf(x[2], x[3]));
    M = row16_max(M);
    float ssum = 0.f;
    if (live) {
#pragma unroll
      for (int c = 0; c < 4; ++c) ssum += __expf(x[c] - M);
    }
    ssum = row16_sum(ssum);

    float score[4];
    if constexpr (SAMPLE) {
      if (live) {
        const uint64_t sd = a.seeds[b];
        const Philox4 r = philox4x32_10(col >> 2, a.j, a.off_lo, a.off_hi, static_cast<uint32_t>(sd),
                                        static_cast<uint32_t>(sd >> 32));
        const uint32_t wd[4] = {r.x, r.y, r.z, r.w};
#pragma unroll
        for (int c = 0; c < 4; ++c) score[c] = x[c] * a.inv_temp + gumbel_from_word(wd[c]);
      } else {
#pragma unroll
        for (int c = 0; c < 4; ++c) score[c] = kNegInf;
      }
    } else {
#pragma unroll
      for (int c = 0; c < 4; ++c) score[c] = x[c];
    }
    ArgState as{score[0], live ? col : 0x7fffffff, x[0]};
#pragma unroll
    for (int c = 1; c < 4; ++c)
      if (score[c] > as.score) as = ArgState{score[c], col + c, x[c]};
    as = row16_arg(as);
    run[ii] = lse_merge(run[ii], LseState{M, ssum});
    best[ii] = arg_merge(best[ii], as);
    __builtin_amdgcn_sched_barrier(0);
  }
}

// This workgroup's k best U~_j of request b as sorted order keys, by one wave.
// Lane l owns the workgroup's columns l, l + 64, ... (in group order); dead
// columns (past V, or groups this workgroup does not have) take no part.
//
// theta, the k-th largest of the 64 lane maxima (with multiplicity), bounds
// the k-th largest element from below (k lanes each hold an element >= theta),
// so the k best lie among the elements >= theta.  Their keys are compacted
// into LDS (ballot prefix) and each is ranked by counting the larger keys
// (keys of live columns are distinct).  If more than kLocCap elements reach
// theta (many equal values), a serial selection takes over: k rounds of
// "largest key below the last one taken".
constexpr int kLocCap = 128;

__device__ __forceinline__ float wave_max_dpp(float v) {
  v = row16_max(v);
  const float r0 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 0));
  const float r1 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 16));
  const float r2 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 32));
  const float r3 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 48));
  return fmaxf(fmaxf(r0, r1), fmaxf(r2, r3));
}

__device__ void local_topk(const StepArgs& a, const ResidentArgs& ra, const float* xs, int b, int wg, int lane,
                           float* lmx, unsigned long long* ck, unsigned long long* out) {
  const int ncol = ra.T * kResCols, k = a.topk;
  // U~ of the lane's i-th column (kNegInf and column -1 when dead)
  auto get = [&](int i, float& v, int& col) {
    const int gid = wg + ra.nwg * i;
    col = gid * kResCols + lane;
    const bool live = i < ra.T && gid < ra.G && col < a.V;
    v = live ? xs[(i * a.B + b) * kResCols + lane] : kNegInf;
    if (!live) col = -1;
  };
  float lm = kNegInf;
  int i = 0;
  for (; i + 4 <= ra.T; i += 4) {
    float v[4];
    int c[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) get(i + u, v[u], c[u]);
#pragma unroll
    for (int u = 0; u < 4; ++u) lm = fmaxf(lm, v[u]);
  }
  for (; i < ra.T; ++i) {
    float v;
    int c;
    get(i, v, c);
    lm = fmaxf(lm, v);
  }
  lmx[lane] = lm;
  __builtin_amdgcn_wave_barrier();
  int cnt = 0;
#pragma unroll 16
  for (int l = 0; l < kWave; ++l) cnt += lmx[l] >= lm;
  const float theta = wave_max_dpp(cnt >= k ? lm : kNegInf);

  int m = 0;
  for (int t = 0; t < ra.T; ++t) {
    float v;
    int col;
    get(t, v, col);
    const bool take = col >= 0 && v >= theta;
    const unsigned long long bal = __ballot(take);
    const int pos = m + __popcll(bal & ((1ull << lane) - 1ull));
    if (take && pos < kLocCap) ck[pos] = best_key(v, col);
    m += __popcll(bal);
  }
  __builtin_amdgcn_wave_barrier();
  if (m <= kLocCap) {
    for (int e = lane; e < m; e += kWave) {
      const unsigned long long key = ck[e];
      int rank = 0, f = 0;
      for (; f + 8 <= m; f += 8) {
#pragma unroll
        for (int u = 0; u < 8; ++u) rank += ck[f + u] > key;
      }
      for (; f < m; ++f) rank += ck[f] > key;
      if (rank < k) out[rank] = key;
    }
    for (int t = m + lane; t < k; t += kWave) out[t] = 0ull;
    return;
  }
  // serial selection over keys: the lane's largest key below the last taken
  auto scan = [&](unsigned long long last) {
    unsigned long long bk = 0;
    for (int t = 0; t < ra.T; ++t) {
      float v;
      int col;
      get(t, v, col);
      const unsigned long long key = col >= 0 ? best_key(v, col) : 0ull;
      if (key < last && key > bk) bk = key;
    }
    return bk;
  };
  unsigned long long mine = scan(~0ull);
  for (int t = 0; t < k; ++t) {
    unsigned long long wk = mine;
#pragma unroll
    for (int o = 1; o < kWave; o <<= 1) {
      const unsigned long long ok = __shfl_xor(wk, o);
      wk = ok > wk ? ok : wk;
    }
    if (lane == 0) out[t] = wk;
    if (mine == wk && wk != 0ull) mine = scan(wk);
  }
}

// Candidate list (k keys in LDS, written by this wave) of request b at
// position j to its workspace slot: one store per lane < k.
__device__ __forceinline__ void flush_list(const StepArgs& a, const ResidentArgs& ra, const unsigned long long* src,
                                           int b, int j, int wg, int lane) {
  __builtin_amdgcn_wave_barrier();
  asm volatile("" : "+v"(lane));        // per-lane address math stays here, not hoisted and spilled
  if (lane < a.topk) a.cand_key[((static_cast<size_t>(b) * a.gamma + j) * ra.nwg + wg) * a.topk + lane] = src[lane];
}

// Candidate lists stay in LDS for one position when all of a position's
// lists fit (B k keys): a wave stores position j's lists while the wait of
// position j + 1 runs, so no barrier of the chain waits for those stores.
constexpr int kListKeys = (kResWaves - 1) * kMaxTopk;

template <int KCH, int QN, bool SAMPLE>
__global__ __launch_bounds__(kResThreads) void markov_resident(StepArgs a, ResidentArgs ra) {
  constexpr int RGW = 8 / KCH;   // register groups per wave (128 VGPRs of operands)
  extern __shared__ __align__(16) unsigned char res_lds[];
  __shared__ ArgState wbest[kResWaves][kResMaxB];
  __shared__ LseState wlse[kResWaves][kResMaxB];
  __shared__ int prev_s[kResMaxB];
  __shared__ float ltk_max[kResWaves - 1][kWave];        // local top-k scratch of waves 1..7
  __shared__ unsigned long long ltk_key[kResWaves - 1][kLocCap];
  __shared__ unsigned long long lst_s[2][kListKeys];    // candidate lists: [position parity][b * k ..]

  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int g = lane >> 4, n = lane & 15;
  const int wg = blockIdx.x;
  const size_t V = static_cast<size_t>(a.V);
  const uint16_t* A = static_cast<const uint16_t*>(a.A);
  const uint16_t* Bm = static_cast<const uint16_t*>(a.Bm);
  u32x4* lds_ops = reinterpret_cast<u32x4*>(res_lds);                       // [nlds][KCH][4][64]
  float* lds_u0 = reinterpret_cast<float*>(res_lds + static_cast<size_t>(ra.nlds) * KCH * 4 * kWave * 16);
  const int ubuf = ra.T * a.B * kResCols;            // floats per buffer; [2][T][B][64]
  auto gid_of = [&](int t) { return wg + ra.nwg * t; };
  auto has = [&](int t) { return t < ra.T && gid_of(t) < ra.G; };

  // U_j rows of this workgroup's groups, [t][b][64] floats, into buffer j % 2,
  // through registers: wave wv of nwv moves 16-byte pieces p = 64 (wv + nwv i)
  // + lane (row p / 16, bytes 16 (p % 16)), four loads in flight before their
  // LDS writes.  (An LDS DMA here would make the compiler wait for every
  // global access of the wave, stores included, before its next LDS read.)
  const int nrows = ra.T * a.B;
  auto fetch_u = [&](int j, int wv, int nwv) {
    float* lds_u = lds_u0 + (j & 1) * ubuf;
    const int np = nrows * (kResCols / 4);
    int ln = lane;                      // opaque: keeps the per-lane address math in here
    asm volatile("" : "+v"(ln));
    for (int p0 = kWave * wv; p0 < np; p0 += 4 * kWave * nwv) {
      f32x4 v[4];
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const int p = p0 + u * kWave * nwv + ln;
        const int rr = p >> 4, t = rr / a.B, b = rr - t * a.B;
        const int col = gid_of(t) * kResCols + 4 * (p & 15);
        v[u] = f32x4{0.f, 0.f, 0.f, 0.f};      // dead groups and columns past V: never read
        if (p < np && has(t) && col < a.V)
          v[u] = *reinterpret_cast<const f32x4*>(a.U + (static_cast<size_t>(b) * a.gamma + j) * V + col);
      }
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const int p = p0 + u * kWave * nwv + ln;
        if (p < np) *reinterpret_cast<f32x4*>(lds_u + 4 * p) = v[u];
      }
    }
  };
  // U~_j (in buffer j % 2 after the epilogue) to the dump, the same pieces
  auto dump_u = [&](int j, int wv, int nwv) {
    const float* lds_u = lds_u0 + (j & 1) * ubuf;
    const int np = nrows * (kResCols / 4);
    int ln = lane;
    asm volatile("" : "+v"(ln));
    for (int p = kWave * wv + ln; p < np; p += kWave * nwv) {
      const int rr = p >> 4, t = rr / a.B, b = rr - t * a.B;
      const int col = gid_of(t) * kResCols + 4 * (p & 15);
      if (has(t) && col < a.V)
        *reinterpret_cast<f32x4*>(a.logits_out + (static_cast<size_t>(b) * a.gamma + j) * V + col) =
            *reinterpret_cast<const f32x4*>(lds_u + 4 * p);
    }
  };
  fetch_u(0, w, kResWaves);

  // Bm share: register groups t = w*RGW + s, LDS group t = nreg + w
  u32x4 dreg[RGW][KCH][4];
#pragma unroll
  for (int s = 0; s < RGW; ++s) {
    const int t = w * RGW + s;
    const bool on = has(t);
    const int col = gid_of(t) * kResCols + 4 * n;
#pragma unroll
    for (int q = 0; q < KCH; ++q) load_chunk<KCH>(Bm, V, col, on && col < a.V, q, g, dreg[s][q]);
  }
  if (w < ra.nlds && has(ra.nreg + w)) {
    const int col = gid_of(ra.nreg + w) * kResCols + 4 * n;
#pragma unroll
    for (int q = 0; q < KCH; ++q) {
      u32x4 op[4];
      load_chunk<KCH>(Bm, V, col, col < a.V, q, g, op);
#pragma unroll
      for (int c = 0; c < 4; ++c) lds_ops[((w * KCH + q) * 4 + c) * kWave + lane] = op[c];
    }
  }
  if (w == 0 && lane < a.B) prev_s[lane] = a.anchor[lane];   // x_{-1}
  __syncthreads();   // LDS operands, U_0 and the anchors written

  for (int j = 0; j < a.gamma; ++j) {
    a.j = j;
    float* lds_u = lds_u0 + (j & 1) * ubuf;
    int prev = n < a.B ? prev_s[n] : 0;              // LDS only: no global load ahead of the gather
    prev = min(max(prev, 0), a.V - 1);              // guard of the gathered row
    // lanes of requests n >= B gather row 0: their products are never read
    u32x4 av[KCH];
#pragma unroll
    for (int q = 0; q < KCH; ++q)
      av[q] = *reinterpret_cast<const u32x4*>(A + static_cast<size_t>(prev) * a.r + 32 * q + 8 * g);
    ArgState best[QN];
    LseState run[QN];
#pragma unroll
    for (int ii = 0; ii < QN; ++ii) {
      best[ii] = ArgState{kNegInf, 0x7fffffff, 0.f};
      run[ii] = LseState{kNegInf, 0.f};
    }

    // products of the register groups and the LDS group; with one register
    // group per wave both accumulators are formed before either epilogue, so
    // the A operands are dead during the epilogues
    auto mfma_reg = [&](int s, f32x4 (&acc)[4]) {
#pragma unroll
      for (int c = 0; c < 4; ++c) acc[c] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int q = 0; q < KCH; ++q)
#pragma unroll
        for (int c = 0; c < 4; ++c)
          acc[c] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(av[q]), as_bf16x8(dreg[s][q][c]), acc[c], 0, 0, 0);
    };
    auto mfma_lds = [&](f32x4 (&acc)[4]) {
#pragma unroll
      for (int c = 0; c < 4; ++c) acc[c] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int q = 0; q < KCH; ++q)
#pragma unroll
        for (int c = 0; c < 4; ++c)
          acc[c] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
              as_bf16x8(av[q]), as_bf16x8(lds_ops[((w * KCH + q) * 4 + c) * kWave + lane]), acc[c], 0, 0, 0);
    };
    const int tl = ra.nreg + w;
    const bool lds_on = w < ra.nlds && has(tl);
    if constexpr (RGW == 1) {
      const int t = w;
      f32x4 acc0[4], acc1[4];
      if (has(t)) mfma_reg(0, acc0);
      if (lds_on) mfma_lds(acc1);
      if (has(t)) resident_epilogue<QN, SAMPLE>(a, acc0, lds_u + t * a.B * kResCols, gid_of(t), g, n, run, best);
      if (lds_on) resident_epilogue<QN, SAMPLE>(a, acc1, lds_u + tl * a.B * kResCols, gid_of(tl), g, n, run, best);
    } else {
#pragma unroll
      for (int s = 0; s < RGW; ++s) {
        const int t = w * RGW + s;
        if (!has(t)) continue;                        // uniform per wave
        f32x4 acc[4];
        mfma_reg(s, acc);
        resident_epilogue<QN, SAMPLE>(a, acc, lds_u + t * a.B * kResCols, gid_of(t), g, n, run, best);
      }
      if (lds_on) {
        f32x4 acc[4];
        mfma_lds(acc);
        resident_epilogue<QN, SAMPLE>(a, acc, lds_u + tl * a.B * kResCols, gid_of(tl), g, n, run, best);
      }
    }
    if (n == 0) {
#pragma unroll
      for (int ii = 0; ii < QN; ++ii)
        if (4 * g + ii < a.B) {
          wbest[w][4 * g + ii] = best[ii];
          wlse[w][4 * g + ii] = run[ii];
        }
    }
    res_lds_barrier();                                // wave bests and U~_j in LDS
    // Beside wave 0's wait: list waves 1..nl build this position's candidate
    // lists (LDS only); helper waves (the rest of 1..7) fetch U_{j+1), copy
    // U~_j from LDS to the dump, write this workgroup's partial and store
    // position j - 1's lists.  Every plain store of the position is a helper
    // wave's: the compiler makes a wave wait for its outstanding stores
    // before it reuses their data registers, which keeps those waits off the
    // waves that lead the next position.  With lists on every wave (B >= 7)
    // the list waves are also the helpers and store their lists at once.
    const int nl = a.topk > 0 ? min(a.B, kResWaves - 1) : 0;
    const int nh = nl < kResWaves - 1 ? kResWaves - 1 - nl : kResWaves - 1;   // helper waves
    const int hw = nl < kResWaves - 1 ? w - 1 - nl : w - 1;                  // this wave's helper index
    const bool defer = nl > 0 && nl < kResWaves - 1 && a.B * a.topk <= kListKeys;
    if (w > 0 && hw >= 0) {
      if (j + 1 < a.gamma) fetch_u(j + 1, hw, nh);
      if (a.logits_out) dump_u(j, hw, nh);
      if (hw == nh - 1 && lane < a.B) {
        int ln = lane;
        asm volatile("" : "+v"(ln));
        ArgState s = wbest[0][ln];
        LseState l = wlse[0][ln];
        for (int v = 1; v < kResWaves; ++v) {
          s = arg_merge(s, wbest[v][ln]);
          l = lse_merge(l, wlse[v][ln]);
        }
        const size_t pq = (static_cast<size_t>(ln) * a.gamma + j) * a.P + wg;
        a.p_m[pq] = l.m;
        a.p_s[pq] = l.s;
        a.p_score[pq] = s.score;
        a.p_idx[pq] = s.idx;
        a.p_x[pq] = s.x;
      }
      if (defer && j > 0)
        for (int b = hw; b < a.B; b += nh) flush_list(a, ra, &lst_s[(j - 1) & 1][b * a.topk], b, j - 1, wg, lane);
    }
    if (w > 0 && w <= nl) {                          // local candidate lists
      for (int b = w - 1; b < a.B; b += nl) {
        unsigned long long* dst = defer ? &lst_s[j & 1][b * a.topk] : &lst_s[0][(w - 1) * kMaxTopk];
        local_topk(a, ra, lds_u, b, wg, lane, ltk_max[w - 1], ltk_key[w - 1], dst);
        if (!defer) flush_list(a, ra, dst, b, j, wg, lane);
      }
    }
    if (w == 0) {
      unsigned long long key = 0;
      if (lane < a.B) {                               // this workgroup's partial, waves in order
        ArgState s = wbest[0][lane];
        LseState l = wlse[0][lane];
        for (int v = 1; v < kResWaves; ++v) {
          s = arg_merge(s, wbest[v][lane]);
          l = lse_merge(l, wlse[v][lane]);
        }
        key = best_key(s.score, s.idx);
      }
      const bool more = j + 1 < a.gamma;
      chain_tree(a, ra, wg, j, key, lane, more);
      if (more && lane < a.B) prev_s[lane] = best_index(load_dev(a.best + lane * a.gamma + j));
    }
    // LDS only: U_{j+1} and prev_s written; the workgroup's stores (partials,
    // lists, U~ dump) stay in flight
    res_lds_barrier();
  }
  {                                                  // the last position's deferred lists
    const int nl = a.topk > 0 ? min(a.B, kResWaves - 1) : 0;
    if (nl > 0 && nl < kResWaves - 1 && a.B * a.topk <= kListKeys && w > nl) {
      const int nh = kResWaves - 1 - nl, hw = w - 1 - nl;
      for (int b = hw; b < a.B; b += nh) flush_list(a, ra, &lst_s[(a.gamma - 1) & 1][b * a.topk], b, a.gamma - 1, wg, lane);
    }
  }
}

// ---------------------------------------------------------------------------
// host side

namespace {

template <int KCH, int QN, bool SAMPLE>
hipError_t launch_res(StepArgs a, ResidentArgs ra, size_t lds, hipStream_t s) {
  const void* fn = reinterpret_cast<const void*>(&markov_resident<KCH, QN, SAMPLE>);
  hipError_t e = hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize, static_cast<int>(lds));
  if (e != hipSuccess) return e;
  // every workgroup must fit at once: at most one per compute unit is asked for
  int per_cu = 0;
  e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, fn, kResThreads, lds);
  if (e != hipSuccess) return e;
  if (per_cu < 1) return hipErrorLaunchOutOfResources;
  void* args[] = {&a, &ra};
  return hipLaunchKernel(fn, dim3(ra.nwg), dim3(kResThreads), args, lds, s);
}

template <int KCH>
hipError_t launch_b1(const StepArgs& a, const ResidentArgs& ra, size_t lds, hipStream_t s) {
  return a.sample ? launch_res<KCH, 1, true>(a, ra, lds, s) : launch_res<KCH, 1, false>(a, ra, lds, s);
}
}  // namespace

// Plan of the resident chain for these sizes; false when it does not apply
// (the caller then runs the per-position kernels).  `max_wg` > 0 caps the
// number of workgroups (more groups per workgroup, as on a smaller device).
bool markov_resident_plan(int B, int V, int r, int max_wg, int* nwg_out, size_t* lds_out) {
  // the register budget of one wave (operands, accumulators, epilogue) holds
  // without spills for these shapes
  if (B < 1 || B > kResMaxB) return false;
  static_assert(kMaxLists >= 256, "one candidate list per workgroup");
  if (B == 1 ? (r != 64 && r != 128 && r != 256) : r != 256) return false;
  const DeviceInfo d = device_info();
  if (d.cus <= 0 || d.clock_khz <= 0) return false;
  const int KCH = r / 32, nreg = kResWaves * (8 / KCH);
  const int G = (V + kResCols - 1) / kResCols;
  int nwg = d.cus < kMaxLists ? d.cus : kMaxLists;
  if (max_wg > 0 && max_wg < nwg) nwg = max_wg;
  if (nwg > G) nwg = G;
  const int T = (G + nwg - 1) / nwg;
  const int nlds = T > nreg ? T - nreg : 0;
  if (nlds > kResWaves) return false;
  const size_t lds = static_cast<size_t>(nlds) * KCH * 4 * kWave * 16 + 2 * static_cast<size_t>(T) * B * kResCols * 4;
  if (lds > kResLdsMax) return false;
  *nwg_out = nwg;
  *lds_out = lds;
  return true;
}

hipError_t launch_markov_resident(StepArgs a, unsigned* sync, int nwg, size_t lds, hipStream_t s) {
  const DeviceInfo d = device_info();
  ResidentArgs ra{};
  ra.nwg = nwg;
  ra.G = (a.V + kResCols - 1) / kResCols;
  ra.T = (ra.G + nwg - 1) / nwg;
  const int KCH = a.r / 32;
  ra.nreg = kResWaves * (8 / KCH);
  ra.nlds = ra.T > ra.nreg ? ra.T - ra.nreg : 0;
  ra.sync = sync;
  ra.wait_ticks = static_cast<unsigned long long>(d.clock_khz) * 100;   // 100 ms
  a.j = 0;
  if (a.B > 1) return a.sample ? launch_res<8, 4, true>(a, ra, lds, s) : launch_res<8, 4, false>(a, ra, lds, s);
  switch (KCH) {
    case 2: return launch_b1<2>(a, ra, lds, s);
    case 4: return launch_b1<4>(a, ra, lds, s);
    default: return launch_b1<8>(a, ra, lds, s);
  }
}

}  // namespace dspark
