// Distribution overlap and probabilistic acceptance length.
// "Qwen3.8-Flash-Next DSpark 训练实验", 评估口径/离线指标:
//   a_i = sum_v min(p_i(v), q_i(v)) = 1 - ||p_i - q_i||_1 / 2,
//   tau_prob = 1 + sum_{i=0}^{6} prod_{j<=i} a_j per valid block; invalid slots
//   get a_i = 0; accept_rate@i is averaged over valid slots; in the candidate
//   evaluation q is the softmax over the candidates (zero elsewhere) and p stays
//   the full-vocabulary teacher softmax.
// "DSpark 论文精读", §3.1 and the clamp to [0, 1] in its loss code.
//
// Many rows: one workgroup per (block, slot) row.  Pass 1 streams both logit
// rows once and keeps per-thread online (max, sum-exp) states; a fixed-order
// tree gives the two log-normalisers L_p, L_q.  Pass 2 adds
// exp(min(t - L_p, d - L_q)) (one exponential per element, as exp is
// monotone) and walks the row backwards so that its first reads hit what pass
// 1 touched last.  Few rows (below kSplitRowsMax): each row is split into
// chunks over several workgroups (statistics, then sums, then a fixed-order
// finish that also computes tau when one workgroup can).
#include <cstdlib>

#include "common.h"
#include "internal.h"

namespace dspark {

constexpr int kOvThreads = 512;
constexpr int kSplitThreads = 256;
constexpr int kTauThreads = 256;
constexpr int kSplitChunk = 2048;      // elements per workgroup on the split path
constexpr int kSplitRowsMax = 1024;    // at and above this many rows, one workgroup per row
constexpr int kFusedFinishRows = 64;   // up to this many rows, one workgroup finishes rows and tau
// candidate mode from this many rows: one workgroup per row rather than the
// split path, which reads each row through several workgroups and then
// launches a finish (448 rows x 151936: 48.3 against 54.9 us per call)
constexpr int kCandRowsPath = 384;

// wait words and 64-bit exchange slots of the launches whose workgroups wait
// for each other (their layout is described where they are used)
constexpr int kFusedPer = 4;                    // float4 per thread and array
constexpr int kOvTimeout = 0;                   // word 0: call number of a timed-out wait
constexpr int kOvRowsDone = 32;
constexpr int kOvCnt1 = 64;                     // + 32 * row: chunk states published
constexpr int kOvCnt2 = kOvCnt1 + 32 * kFusedFinishRows;   // + 32 * row: chunk sums published
static_assert(kOvCnt2 + 32 * kFusedFinishRows <= kOvSyncWords, "overlap wait words");

__device__ __forceinline__ unsigned long long pack2(float x, float y) {
  return (static_cast<unsigned long long>(__float_as_uint(y)) << 32) | __float_as_uint(x);
}
__device__ __forceinline__ float lo_f(unsigned long long v) { return __uint_as_float(static_cast<uint32_t>(v)); }
__device__ __forceinline__ float hi_f(unsigned long long v) { return __uint_as_float(static_cast<uint32_t>(v >> 32)); }
__device__ __forceinline__ unsigned long long xchg_dev(unsigned long long* p, unsigned long long v) {
  return __hip_atomic_exchange(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ unsigned add_dev(unsigned* p, unsigned v) {
  return __hip_atomic_fetch_add(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
template <typename T>
__device__ __forceinline__ T ld_dev(const T* p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
// keep the value live so that the wave waits for the atomic's return here
__device__ __forceinline__ void wait_for(unsigned long long v) { asm volatile("" ::"v"(v) : "memory"); }
// a wait of this call ran out (only the launches that wait take a call number)
__device__ __forceinline__ bool call_timed_out(const OverlapArgs& a) {
  return a.epoch != 0u && a.sync && ld_dev(a.sync + kOvTimeout) == a.epoch;
}

__device__ __forceinline__ float sum_exp_min4(f32x4 t, f32x4 d, float Lt, float Ld) {
  return (__expf(fminf(t[0] - Lt, d[0] - Ld)) + __expf(fminf(t[1] - Lt, d[1] - Ld))) +
         (__expf(fminf(t[2] - Lt, d[2] - Ld)) + __expf(fminf(t[3] - Lt, d[3] - Ld)));
}

// sum over the same elements of exp(min(t - Lt, d - Ld)), the elements taken
// in the order `first, first - stride, ...` down to e0 (walk_down) or up from
// first to e1
static_assert(kStreamUnroll == 4, "range_min_sum folds four partial sums");
template <bool WALK_DOWN>
__device__ float range_min_sum(const f32x4* tp, const f32x4* dp, int first, int e0, int e1, int stride, float Lt,
                               float Ld) {
  float s[kStreamUnroll];
#pragma unroll
  for (int u = 0; u < kStreamUnroll; ++u) s[u] = 0.f;
  const int step = WALK_DOWN ? -stride : stride;
  int e = first;
  auto more = [&](int x) { return WALK_DOWN ? x >= e0 : x < e1; };
  for (; more(e + (kStreamUnroll - 1) * step); e += kStreamUnroll * step) {
    f32x4 t[kStreamUnroll], d[kStreamUnroll];
#pragma unroll
    for (int u = 0; u < kStreamUnroll; ++u) {
      t[u] = tp[e + u * step];
      d[u] = dp[e + u * step];
    }
#pragma unroll
    for (int u = 0; u < kStreamUnroll; ++u) s[u] += sum_exp_min4(t[u], d[u], Lt, Ld);
  }
  for (; more(e); e += step) s[0] += sum_exp_min4(tp[e], dp[e], Lt, Ld);
  return (s[0] + s[1]) + (s[2] + s[3]);
}

template <int NW>
__device__ LseState block_lse_state(LseState st, LseState* red) {
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
#pragma unroll
  for (int o = 1; o < kWave; o <<= 1) st = lse_merge(st, shfl_xor(st, o));
  if (lane == 0) red[w] = st;
  __syncthreads();
  LseState r = red[0];
  for (int i = 1; i < NW; ++i) r = lse_merge(r, red[i]);
  __syncthreads();
  return r;
}

template <int NW>
__device__ float block_sum(float v, float* red) {
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  v = wave_sum(v);
  if (lane == 0) red[w] = v;
  __syncthreads();
  float r = 0.f;
  for (int i = 0; i < NW; ++i) r += red[i];
  __syncthreads();
  return r;
}

// candidate-set overlap of one row: this thread's share (candidates first,
// first + stride, ...) of the sum over the k candidates of min(p, q'); an id
// outside [0, V) (no candidate) adds nothing and reads nothing
__device__ float candidate_overlap(const OverlapArgs& a, int row, float Lt, int first, int stride) {
  float s = 0.f;
  for (int c = first; c < a.k; c += stride) {
    const size_t ci = static_cast<size_t>(row) * a.k + c;
    const int id = a.cand_idx[ci];
    if (id < 0 || id >= a.V) continue;
    const float p = __expf(a.teacher[static_cast<size_t>(row) * a.V + id] - Lt);
    s += fminf(p, a.cand_prob[ci]);
  }
  return s;
}

// ---- one workgroup per row (many rows) ------------------------------------
// TR threads per row: 512, or 128 when there are enough rows for every CU to
// hold several of them at once (one round of workgroups instead of ~1.75
// rounds of 512-thread ones at 1,792 rows: ~3% off the pass)
template <int TR>
__global__ __launch_bounds__(TR) void overlap_rows(OverlapArgs a) {
  constexpr int NW = TR / kWave;
  __shared__ LseState red_l[NW];
  __shared__ float red_f[NW];
  const int row = blockIdx.x, tid = threadIdx.x;
  if (a.valid && !a.valid[row]) {
    if (tid == 0) a.alpha[row] = 0.f;
    return;
  }
  const size_t V = static_cast<size_t>(a.V);
  const f32x4* tp = reinterpret_cast<const f32x4*>(a.teacher + row * V);
  const int n4 = a.V / 4;
  float total;
  if (a.draft) {
    const f32x4* dp = reinterpret_cast<const f32x4*>(a.draft + row * V);
    const LseState lt = range_lse<false>(tp, tid, n4, TR);
    const LseState ld = range_lse<false>(dp, tid, n4, TR);
    const LseState rt = block_lse_state<NW>(lt, red_l);
    const LseState rd = block_lse_state<NW>(ld, red_l);
    const float Lt = rt.m + logf(rt.s), Ld = rd.m + logf(rd.s);
    // second pass walks down, to reuse what the first touched last
    const int last = (n4 - 1 - tid) >= 0 ? tid + ((n4 - 1 - tid) / TR) * TR : -1;
    const float s = range_min_sum<true>(tp, dp, last, 0, n4, TR, Lt, Ld);
    total = block_sum<NW>(s, red_f);
    if (tid == 0) {
      if (a.lse_draft) a.lse_draft[row] = Ld;
      if (a.ov_sum) a.ov_sum[row] = total;
    }
  } else {
    const LseState lt = range_lse<true>(tp, tid, n4, TR);   // the row is read once
    const LseState rt = block_lse_state<NW>(lt, red_l);
    total = block_sum<NW>(candidate_overlap(a, row, rt.m + logf(rt.s), tid, TR), red_f);
  }
  if (tid == 0) a.alpha[row] = fminf(fmaxf(total, 0.f), 1.f);
}

// ---- many rows, each read once (dense mode) --------------------------------
// A resident grid of kResK x S workgroups: slot s = workgroup / kResK takes
// rows s, s + S, s + 2S, ..., and workgroup c = workgroup % kResK of the slot
// holds chunk c of each of those rows (its teacher and draft values) in
// registers across both passes, so every logit is read from memory once.
// Per row: the chunk's online states are published as four 64-bit words, each
// tagged with this call's number (a word is its own release flag); wave 0
// polls the row's kResK x 4 words, folds them in chunk order into the
// normalisers (every chunk of the row folds the same words in the same order,
// so all hold the same L_p, L_q), and the data waves add
// exp(min(t - L_p, d - L_q)) over their registers; the chunk's sum goes to the
// workspace and a fold kernel adds the kResK sums in chunk order into alpha.
// Wave 0 does no data loads, so its waits never drain the data waves'
// look-ahead: while wave 0 waits for the row's partners, waves 1..7 already
// stream the slot's next row into their second register set.  The wait is
// bounded in time; a wait that runs out marks the call in the time-out word,
// and from then on no workgroup of the call waits (alpha and tau become NaN,
// the status word DSPARK_ETIMEOUT).
constexpr int kResK = 16;                                  // chunks (workgroups) per row (4 kResK <= 64 words polled)
constexpr int kResThreads = 512;
constexpr int kResData = kResThreads - kWave;              // threads of waves 1..7
constexpr int kResMaxSlotRows = 16384;                     // validity flags of a slot's rows in LDS

template <int P>
struct ResSet { f32x4 t[P], d[P]; };

// wave-wide max and sum with the in-row steps on DPP and two cross-row
// shuffles; every lane ends with the same value
__device__ __forceinline__ float wave_max_dpp(float v) {
  v = row16_max(v);
  v = fmaxf(v, __shfl_xor(v, 16));
  return fmaxf(v, __shfl_xor(v, 32));
}
__device__ __forceinline__ float wave_sum_dpp(float v) {
  v = row16_sum(v);
  v += __shfl_xor(v, 16);
  return v + __shfl_xor(v, 32);
}
// (max, sum exp(x - max)) of the wave from each lane's (m, s): the maximum
// first, then each lane's sum rescaled once
__device__ __forceinline__ LseState wave_lse(float m, float s) {
  const float M = wave_max_dpp(m);
  return LseState{M, wave_sum_dpp(m == kNegInf ? 0.f : s * __expf(m - M))};
}

template <int P>
__global__ __launch_bounds__(kResThreads, 1) void overlap_rows_resident(OverlapArgs a, int S) {
  __shared__ unsigned char va_s[kResMaxSlotRows];
  __shared__ LseState red_t[2][kResThreads / kWave], red_d[2][kResThreads / kWave];
  __shared__ float red_f[2][kResThreads / kWave];
  __shared__ float L_s[2][2];
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int slot = blockIdx.x / kResK, c = blockIdx.x % kResK;
  if (slot >= S) return;                                   // padding (whole workgroup)
  const int rows = a.N * a.gamma;
  const int n4 = a.V / 4;
  const int e0 = min(c * a.chunk4, n4), e1 = min(e0 + a.chunk4, n4);
  const int dt = tid - kWave;                              // data thread index (waves 1..7)
  const size_t V = static_cast<size_t>(a.V);
  unsigned* sy = a.sync;
  // validity of this slot's rows, staged before the loop (a global load in
  // the loop would wait for the look-ahead loads issued before it)
  for (int i = tid; i * S + slot < rows; i += kResThreads) va_s[i] = a.valid ? a.valid[i * S + slot] : 1;
  __syncthreads();

  // the chunk's elements through buffer resources over exactly the chunk:
  // lanes past its end read 0 without touching memory (and are masked out
  // of every sum by `in`)
  const int voff = dt * 16;
  auto in = [&](int i) __attribute__((always_inline)) { return dt + i * kResData < e1 - e0; };
  // Every wave issues the same loads at every step, whether or not the row
  // exists, is valid or is this wave's (wave 0 holds no data): the resource
  // of a load that is not wanted has no records, so it reads 0 without
  // touching memory.  With loads behind a branch the compiler cannot count
  // the loads still in flight, and it waited for all of them (the
  // look-ahead included) before using a set.
  auto load = [&](ResSet<P>& X, int it) __attribute__((always_inline)) {
    const int r = slot + it * S;
    // uniform over the wave (readfirstlane), so that the resources live in
    // scalar registers: with a per-lane resource the compiler loops over lanes
    const bool on = __builtin_amdgcn_readfirstlane(w > 0 && r < rows && va_s[min(it, kResMaxSlotRows - 1)]) != 0;
    const size_t base = on ? r * V + static_cast<size_t>(e0) * 4 : 0;
    const size_t bytes = on ? static_cast<size_t>(e1 - e0) * 16 : 0;
    const __amdgpu_buffer_rsrc_t tr = buf_rsrc(a.teacher + base, bytes);
    const __amdgpu_buffer_rsrc_t dr = buf_rsrc(a.draft + base, bytes);
#pragma unroll
    for (int i = 0; i < P; ++i) {
      X.t[i] = __builtin_bit_cast(f32x4, __builtin_amdgcn_raw_buffer_load_b128(tr, voff, i * kResData * 16,
                                                                              kBufferNonTemporal));
      X.d[i] = __builtin_bit_cast(f32x4, __builtin_amdgcn_raw_buffer_load_b128(dr, voff, i * kResData * 16,
                                                                              kBufferNonTemporal));
    }
  };
  // Step it, one barrier at its end.  Data waves: the overlap sum of row
  // it - 1 (its normalisers came from wave 0 in step it - 1), then set
  // (it - 1) % 4, free again, starts streaming row it + 3, then the chunk
  // states of row it + 1 (set (it + 1) % 4, streamed since step it - 2).
  // Wave 0 meanwhile: the chunk sum of row it - 2 to the workspace, the
  // chunk states of row it (its waves' states from step it - 1) published,
  // the row's kResK x 4 words polled and folded into its normalisers.  So
  // the exchange of a row runs beside a whole step of data work.  Shared
  // words are double-buffered by row parity.
  float mth[4] = {kNegInf, kNegInf, kNegInf, kNegInf}, mdh[4] = {kNegInf, kNegInf, kNegInf, kNegInf};
  auto valid_row = [&](int it) __attribute__((always_inline)) {
    return it >= 0 && slot + it * S < rows && va_s[it] != 0;
  };
  // chunk states of row it from set X (history slot h), by the data waves
  auto states = [&](ResSet<P>& X, int it, int h) __attribute__((always_inline)) {
    if (w == 0 || !valid_row(it)) return;
    float mt = kNegInf, md = kNegInf;
#pragma unroll
    for (int i = 0; i < P; ++i) {
      const float xt = fmaxf(fmaxf(X.t[i][0], X.t[i][1]), fmaxf(X.t[i][2], X.t[i][3]));
      const float xd = fmaxf(fmaxf(X.d[i][0], X.d[i][1]), fmaxf(X.d[i][2], X.d[i][3]));
      mt = in(i) ? fmaxf(mt, xt) : mt;
      md = in(i) ? fmaxf(md, xd) : md;
    }
    // the set now keeps exp(x - m) of this thread's maximum m (base 2, one
    // fused multiply-add and one exponential per element); the overlap sum
    // rescales it instead of taking a second exponential
    const float nt = -(mt == kNegInf ? 0.f : mt) * kLog2e, nd = -(md == kNegInf ? 0.f : md) * kLog2e;
    float st = 0.f, sd = 0.f;
#pragma unroll
    for (int i = 0; i < P; ++i) {
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        X.t[i][k] = __builtin_amdgcn_exp2f(fmaf(X.t[i][k], kLog2e, nt));
        X.d[i][k] = __builtin_amdgcn_exp2f(fmaf(X.d[i][k], kLog2e, nd));
      }
      const float et = (X.t[i][0] + X.t[i][1]) + (X.t[i][2] + X.t[i][3]);
      const float ed = (X.d[i][0] + X.d[i][1]) + (X.d[i][2] + X.d[i][3]);
      st += in(i) ? et : 0.f;
      sd += in(i) ? ed : 0.f;
    }
    mth[h] = mt;
    mdh[h] = md;
    const LseState lt = wave_lse(mt, st), ld = wave_lse(md, sd);
    if (lane == 0) { red_t[it & 1][w] = lt; red_d[it & 1][w] = ld; }
  };
  // overlap sum of row it from set Z (history slot h), by the data waves:
  // min(p, q) = min(e_t exp(m_t - L_p), e_d exp(m_d - L_q)) with the kept
  // e = exp(x - m) of this thread's maxima m
  auto overlap_sum = [&](ResSet<P>& Z, int it, int h) __attribute__((always_inline)) {
    if (w == 0 || !valid_row(it)) return;
    const float mpt = mth[h], mpd = mdh[h];
    const float at = mpt == kNegInf ? 0.f : __expf(mpt - L_s[it & 1][0]);
    const float ad = mpd == kNegInf ? 0.f : __expf(mpd - L_s[it & 1][1]);
    float sm = 0.f;
#pragma unroll
    for (int i = 0; i < P; ++i) {
      const float e = (fminf(Z.t[i][0] * at, Z.d[i][0] * ad) + fminf(Z.t[i][1] * at, Z.d[i][1] * ad)) +
                      (fminf(Z.t[i][2] * at, Z.d[i][2] * ad) + fminf(Z.t[i][3] * at, Z.d[i][3] * ad));
      sm += in(i) ? e : 0.f;
    }
    sm = wave_sum_dpp(sm);
    if (lane == 0) red_f[it & 1][w] = sm;
  };
  // wave 0's part of step it
  auto exchange = [&](int it) __attribute__((always_inline)) {
    if (w != 0) return;
    if (tid == 0 && valid_row(it - 2)) {                   // the chunk sum of row it - 2
      const float* rf = red_f[(it - 2) & 1];
      float tot = rf[1];
      for (int i = 2; i < kResThreads / kWave; ++i) tot += rf[i];
      a.ws_split[static_cast<size_t>(slot + (it - 2) * S) * kResK + c] = tot;
    }
    if (!valid_row(it)) return;
    const int r = slot + it * S;
    const unsigned long long tag = static_cast<unsigned long long>(a.epoch) << 32;
    unsigned long long* words = a.ws_fused + static_cast<size_t>(r) * kResK * 4;
    {
      // the data waves' states: lane i of each 8-lane group takes wave i
      // (wave 0's entry is empty), then a fixed butterfly over the group
      const int wi = lane & 7;
      const LseState rt = wi ? red_t[it & 1][wi] : LseState{kNegInf, 0.f};
      const LseState rd = wi ? red_d[it & 1][wi] : LseState{kNegInf, 0.f};
      float mt = rt.m, md = rd.m;
#pragma unroll
      for (int o = 1; o < 8; o <<= 1) { mt = fmaxf(mt, __shfl_xor(mt, o)); md = fmaxf(md, __shfl_xor(md, o)); }
      float st = rt.m == kNegInf ? 0.f : rt.s * __expf(rt.m - mt);
      float sd = rd.m == kNegInf ? 0.f : rd.s * __expf(rd.m - md);
#pragma unroll
      for (int o = 1; o < 8; o <<= 1) { st += __shfl_xor(st, o); sd += __shfl_xor(sd, o); }
      if (lane < 4) {   // a plain atomic store: nothing waits for it here
        const float v = lane == 0 ? mt : lane == 1 ? st : lane == 2 ? md : sd;
        __hip_atomic_store(words + 4 * c + lane, tag | __float_as_uint(v), __ATOMIC_RELAXED,
                           __HIP_MEMORY_SCOPE_AGENT);
      }
    }
    // the row's kResK x 4 words, one per lane; waits end at a time-out of
    // any workgroup of this call
    unsigned long long v = 0ull;
    if (ld_dev(sy + kOvTimeout) != a.epoch) {
      const unsigned long long t0 = wall_clock64();
      while (true) {
        v = lane < 4 * kResK ? ld_dev(words + lane) : tag;
        if (__builtin_amdgcn_ballot_w64((v >> 32) != a.epoch) == 0ull) break;
        if (wall_clock64() - t0 > a.wait_ticks || ld_dev(sy + kOvTimeout) == a.epoch) {
          if (lane == 0) __hip_atomic_store(sy + kOvTimeout, a.epoch, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
          break;
        }
        __builtin_amdgcn_s_sleep(1);
      }
    }
    // fold: lane k < kResK takes chunk k's states; the maxima, then the
    // rescaled sums, over a fixed butterfly (every lane ends with the same
    // values, in every workgroup of the row)
    const float f = __uint_as_float(static_cast<uint32_t>(v));
    const int k4 = 4 * (lane & (kResK - 1));
    const float tm = __shfl(f, k4), ts = __shfl(f, k4 + 1), dm = __shfl(f, k4 + 2), ds = __shfl(f, k4 + 3);
    const float Mt = row16_max(tm), Md = row16_max(dm);
    const float Lt = Mt + logf(row16_sum(tm == kNegInf ? 0.f : ts * __expf(tm - Mt)));
    const float Ld = Md + logf(row16_sum(dm == kNegInf ? 0.f : ds * __expf(dm - Md)));
    if (lane == 0) {
      L_s[it & 1][0] = Lt;
      L_s[it & 1][1] = Ld;
      if (c == 0 && a.lse_draft) a.lse_draft[r] = Ld;
    }
  };
  // set i % 4 holds row i; the four set indices of each step are constants
  auto step = [&](ResSet<P>& Sm, ResSet<P>& St, int it, int hm, int hs) __attribute__((always_inline)) {
    exchange(it);
    overlap_sum(Sm, it - 1, hm);
    load(Sm, it + 3);                                       // every wave (see load)
    states(St, it + 1, hs);
    asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
  };

  ResSet<P> A, B, C, D;
  load(A, 0);
  // keep the rows' loads in row order (the steps count on it)
  __builtin_amdgcn_sched_barrier(0);
  load(B, 1);
  __builtin_amdgcn_sched_barrier(0);
  load(C, 2);
  states(A, 0, 0);
  asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
  // the last row, n - 1, is published at step n - 1, summed at step n and
  // stored at step n + 1; the step count is rounded up to whole rotations so
  // that every step (and its loads) runs unconditionally and the compiler
  // can count the loads in flight
  const int n = (rows - slot + S - 1) / S;
  for (int it = 0; it < n + 2; it += 4) {
    step(D, B, it, 3, 1);
    step(A, C, it + 1, 0, 2);
    step(B, D, it + 2, 1, 3);
    step(C, A, it + 3, 2, 0);
  }
}

// alpha (and the overlap sums) of every row from its kResK chunk sums, in
// chunk order; NaN for every row when a wait of the call ran out
__global__ __launch_bounds__(256) void overlap_rows_resident_fold(OverlapArgs a) {
  const int r = blockIdx.x * 256 + threadIdx.x;
  if (r >= a.N * a.gamma) return;
  const bool timed_out = ld_dev(a.sync + kOvTimeout) == a.epoch;
  const bool vr = !a.valid || a.valid[r];
  float s = 0.f;
  if (vr) {
#pragma unroll
    for (int k = 0; k < kResK; ++k) s += a.ws_split[static_cast<size_t>(r) * kResK + k];
    if (a.ov_sum) a.ov_sum[r] = s;
  }
  a.alpha[r] = timed_out ? __builtin_nanf("") : (vr ? fminf(fmaxf(s, 0.f), 1.f) : 0.f);
}

// ---- several workgroups per row (few rows) ---------------------------------
// pass 1: per (row, chunk) online states of teacher and draft
__global__ __launch_bounds__(kSplitThreads) void overlap_split_stats(OverlapArgs a) {
  constexpr int NW = kSplitThreads / kWave;
  __shared__ LseState red_l[NW];
  const int c = blockIdx.x, row = blockIdx.y, tid = threadIdx.x;
  if (a.valid && !a.valid[row]) return;
  const size_t V = static_cast<size_t>(a.V);
  const int e0 = c * a.chunk4, e1 = min(e0 + a.chunk4, a.V / 4);
  const f32x4* tp = reinterpret_cast<const f32x4*>(a.teacher + row * V);
  // candidate mode reads the teacher once; the dense pass 2 reads both again
  LseState lt, ld{kNegInf, 0.f};
  if (a.draft) {
    const f32x4* dp = reinterpret_cast<const f32x4*>(a.draft + row * V);
    lt = range_lse<false>(tp, e0 + tid, e1, kSplitThreads);
    ld = range_lse<false>(dp, e0 + tid, e1, kSplitThreads);
  } else {
    lt = range_lse<true>(tp, e0 + tid, e1, kSplitThreads);
  }
  const LseState rt = block_lse_state<NW>(lt, red_l);
  const LseState rd = block_lse_state<NW>(ld, red_l);
  if (tid == 0) {
    float* st = a.ws_split + (static_cast<size_t>(row) * a.nchunk + c) * 5;
    st[0] = rt.m; st[1] = rt.s; st[2] = rd.m; st[3] = rd.s;
  }
}

// log-normalisers of one row from its chunk states, merged by one wave: lane
// c folds chunks c, c+64, ... in order, then a fixed xor tree (all lanes
// return the same values)
__device__ void row_normalisers(const OverlapArgs& a, int row, float& Lt, float& Ld) {
  const int lane = threadIdx.x & 63;
  LseState lt{kNegInf, 0.f}, ld{kNegInf, 0.f};
  const float* st = a.ws_split + static_cast<size_t>(row) * a.nchunk * 5;
  for (int c = lane; c < a.nchunk; c += kWave) {
    lt = lse_merge(lt, LseState{st[c * 5 + 0], st[c * 5 + 1]});
    ld = lse_merge(ld, LseState{st[c * 5 + 2], st[c * 5 + 3]});
  }
#pragma unroll
  for (int o = 1; o < kWave; o <<= 1) {
    lt = lse_merge(lt, shfl_xor(lt, o));
    ld = lse_merge(ld, shfl_xor(ld, o));
  }
  Lt = lt.m + logf(lt.s);
  Ld = ld.m + logf(ld.s);
}

// pass 2 (dense): per (row, chunk) sum of exp(min(t - L_p, d - L_q))
__global__ __launch_bounds__(kSplitThreads) void overlap_split_sum(OverlapArgs a) {
  constexpr int NW = kSplitThreads / kWave;
  __shared__ float L[2];
  __shared__ float red_f[NW];
  const int c = blockIdx.x, row = blockIdx.y, tid = threadIdx.x;
  if (a.valid && !a.valid[row]) return;
  if (tid < kWave) {
    float lt, ld;
    row_normalisers(a, row, lt, ld);
    if (tid == 0) { L[0] = lt; L[1] = ld; }
  }
  __syncthreads();
  const float Lt = L[0], Ld = L[1];
  const size_t V = static_cast<size_t>(a.V);
  const int e0 = c * a.chunk4, e1 = min(e0 + a.chunk4, a.V / 4);
  const f32x4* tp = reinterpret_cast<const f32x4*>(a.teacher + row * V);
  const f32x4* dp = reinterpret_cast<const f32x4*>(a.draft + row * V);
  const float s = range_min_sum<false>(tp, dp, e0 + tid, e0, e1, kSplitThreads, Lt, Ld);
  const float tot = block_sum<NW>(s, red_f);
  if (tid == 0) a.ws_split[(static_cast<size_t>(row) * a.nchunk + c) * 5 + 4] = tot;
}

// pass 3: one wave per row folds the chunk sums (dense) or gathers the
// candidates (candidate mode)
__global__ __launch_bounds__(kWave) void overlap_split_finish(OverlapArgs a) {
  const int row = blockIdx.x, lane = threadIdx.x;
  if (a.valid && !a.valid[row]) {
    if (lane == 0) a.alpha[row] = 0.f;
    return;
  }
  float s = 0.f;
  if (a.draft) {
    const float* st = a.ws_split + static_cast<size_t>(row) * a.nchunk * 5;
    for (int c = lane; c < a.nchunk; c += kWave) s += st[c * 5 + 4];
    if (a.lse_draft) {
      float lt, ld;
      row_normalisers(a, row, lt, ld);
      if (lane == 0) a.lse_draft[row] = ld;
    }
  } else {
    float lt, ld;
    row_normalisers(a, row, lt, ld);
    s = candidate_overlap(a, row, lt, lane, kWave);
  }
  s = wave_sum(s);
  if (lane == 0) {
    a.alpha[row] = fminf(fmaxf(s, 0.f), 1.f);
    if (a.draft && a.ov_sum) a.ov_sum[row] = s;
  }
}

// tau per block and per-workgroup partial sums for the aggregates (a full
// workgroup of kTauThreads threads calls it for its range of blocks).  DEV:
// alpha was written by other workgroups of the same launch, so it is read at
// device scope.
template <bool DEV = false>
__device__ void tau_range(const OverlapArgs& a, int blk) {
  __shared__ double red[kTauThreads / kWave][2 * kMaxGamma + 2];
  __shared__ double tot[2 * kMaxGamma + 2];
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int n = blk * kTauThreads + tid;
  const int G = a.gamma;
  double acc[kMaxGamma], cnt[kMaxGamma];
  double tsum = 0.0, tcnt = 0.0;
#pragma unroll
  for (int i = 0; i < kMaxGamma; ++i) { acc[i] = 0.0; cnt[i] = 0.0; }
  if (n < a.N) {
    float run = 1.f, tau = 1.f;
    bool has = false;
#pragma unroll
    for (int i = 0; i < kMaxGamma; ++i) {
      if (i < G) {
        const float al = DEV ? __hip_atomic_load(a.alpha + n * G + i, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT)
                             : a.alpha[n * G + i];
        const bool v = a.valid ? a.valid[n * G + i] != 0 : true;
        has |= v;
        run *= al;
        tau += run;
        if (v) { acc[i] = al; cnt[i] = 1.0; }
      }
    }
    a.tau[n] = has ? tau : 0.f;
    if (has) { tsum = tau; tcnt = 1.0; }
  }
#pragma unroll
  for (int i = 0; i < kMaxGamma; ++i) {
    if (i < G) {
      const double s1 = wave_sum(acc[i]), s2 = wave_sum(cnt[i]);
      if (lane == 0) { red[w][i] = s1; red[w][G + i] = s2; }
    }
  }
  {
    const double s1 = wave_sum(tsum), s2 = wave_sum(tcnt);
    if (lane == 0) { red[w][2 * G] = s1; red[w][2 * G + 1] = s2; }
  }
  __syncthreads();
  const int F = 2 * G + 2;
  if (tid < F) {
    double s = 0.0;
    for (int i = 0; i < kTauThreads / kWave; ++i) s += red[i][tid];
    if (a.nblk > 1) a.ws_acc[static_cast<size_t>(blk) * F + tid] = s;
    else tot[tid] = s;
  }
  if (a.nblk == 1) {  // one workgroup holds every block: finish here
    __syncthreads();
    if (tid < G && a.accept_rate_at) a.accept_rate_at[tid] = tot[G + tid] > 0.0 ? tot[tid] / tot[G + tid] : 0.0;
    if (tid == 0 && a.tau_mean) *a.tau_mean = tot[2 * G + 1] > 0.0 ? tot[2 * G] / tot[2 * G + 1] : 0.0;
    if (tid == 0 && a.status) *a.status = call_timed_out(a) ? kStatusTimeout : kStatusOk;
  }
}

__global__ __launch_bounds__(kTauThreads) void tau_blocks(OverlapArgs a) { tau_range<false>(a, blockIdx.x); }

// few rows: one workgroup finishes every row (a wave per row) and then tau
__global__ __launch_bounds__(kTauThreads) void overlap_split_finish_tau(OverlapArgs a) {
  const int w = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int rows = a.N * a.gamma;
  for (int row = w; row < rows; row += kTauThreads / kWave) {
    float s = 0.f;
    const bool vr = !a.valid || a.valid[row];
    if (vr) {
      if (a.draft) {
        const float* st = a.ws_split + static_cast<size_t>(row) * a.nchunk * 5;
        for (int c = lane; c < a.nchunk; c += kWave) s += st[c * 5 + 4];
        if (a.lse_draft) {
          float lt, ld;
          row_normalisers(a, row, lt, ld);
          if (lane == 0) a.lse_draft[row] = ld;
        }
      } else {
        float lt, ld;
        row_normalisers(a, row, lt, ld);
        s = candidate_overlap(a, row, lt, lane, kWave);
      }
      s = wave_sum(s);
    }
    if (lane == 0) {
      a.alpha[row] = fminf(fmaxf(s, 0.f), 1.f);
      if (vr && a.draft && a.ov_sum) a.ov_sum[row] = s;
    }
  }
  __syncthreads();   // alpha of every row written by this workgroup
  tau_range<false>(a, 0);
}

// ---- one launch for few rows ----------------------------------------------
// Grid (chunk, row) with the chunk's teacher (and draft) values held in
// registers across both passes.  Each chunk publishes its online states with
// device-scope atomics (both exchanges in flight together) and counts itself
// in at its row; the row's last arriver (known from the counter's old value)
// folds the states in chunk order into the normalisers.
//   Dense mode: the last arriver publishes them tagged with this call's
//   number (the tag releases the row); every chunk of the row then adds its
//   sum of exp(min(t - L_p, d - L_q)) and counts itself in again; the row's
//   last one counts the row in at the call, and the call's last row folds
//   every row's sums in chunk order into alpha and computes tau.
//   Candidate mode: the last arriver gathers the candidates and writes alpha;
//   no chunk waits, and the last row to finish computes tau.
// The last workgroup also clears the counters for the next call.  Dense mode
// needs every chunk resident at once (the launcher checks the occupancy); the
// wait is bounded in time, and a wait that runs out marks the call, which then
// reports NaN for tau.

// By one workgroup: tau of every block, accept_rate@i and the mean tau from
// the alphas al_s and the validity flags va_s of all rows (<= 64 rows).
__device__ void fused_tau(const OverlapArgs& a, const float* al_s, const unsigned char* va_s, bool timed_out) {
  const int tid = threadIdx.x, G = a.gamma;
  const float nan = __builtin_nanf("");
  if (tid < a.N) {
    float run = 1.f, tau_n = 1.f;
    bool has = false;
    for (int i = 0; i < G; ++i) {
      has |= va_s[tid * G + i] != 0;
      run *= al_s[tid * G + i];
      tau_n += run;
    }
    a.tau[tid] = timed_out ? nan : (has ? tau_n : 0.f);
  }
  if (tid < G) {   // accept_rate@i over valid slots, blocks in order
    double s1 = 0.0, s2 = 0.0;
    for (int n = 0; n < a.N; ++n)
      if (va_s[n * G + tid]) { s1 += al_s[n * G + tid]; s2 += 1.0; }
    if (a.accept_rate_at) a.accept_rate_at[tid] = s2 > 0.0 ? s1 / s2 : 0.0;
  }
  if (tid == 0 && a.tau_mean) {   // mean tau over blocks with a valid slot, in order
    double s1 = 0.0, s2 = 0.0;
    for (int n = 0; n < a.N; ++n) {
      float run = 1.f, tn = 1.f;
      bool hv = false;
      for (int i = 0; i < G; ++i) {
        hv |= va_s[n * G + i] != 0;
        run *= al_s[n * G + i];
        tn += run;
      }
      if (hv) { s1 += tn; s2 += 1.0; }
    }
    *a.tau_mean = timed_out ? static_cast<double>(nan) : (s2 > 0.0 ? s1 / s2 : 0.0);
  }
  if (tid == 0 && a.status) *a.status = timed_out ? kStatusTimeout : kStatusOk;
}

// By wave 0: the teacher and draft log-normalisers of `row` from its chunk
// states, in chunk order (lanes take chunks lane and lane + 64, then a
// butterfly, so every lane ends with the same values).
__device__ __forceinline__ void fold_row_states(const OverlapArgs& a, int row, int lane, float& Lt, float& Ld) {
  LseState t{kNegInf, 0.f}, d{kNegInf, 0.f};
  const unsigned long long* rs = a.ws_fused + static_cast<size_t>(row) * a.nchunk * 3;
  unsigned long long st[2] = {0ull, 0ull}, sd[2] = {0ull, 0ull};   // all loads issued first
#pragma unroll
  for (int u = 0; u < 2; ++u) {
    const int k = lane + u * kWave;
    if (k < a.nchunk) { st[u] = ld_dev(rs + 3 * k); sd[u] = ld_dev(rs + 3 * k + 1); }
  }
#pragma unroll
  for (int u = 0; u < 2; ++u) {
    if (lane + u * kWave < a.nchunk) {
      t = lse_merge(t, LseState{lo_f(st[u]), hi_f(st[u])});
      d = lse_merge(d, LseState{lo_f(sd[u]), hi_f(sd[u])});
    }
  }
#pragma unroll
  for (int o = 1; o < kWave; o <<= 1) {
    t = lse_merge(t, shfl_xor(t, o));
    d = lse_merge(d, shfl_xor(d, o));
  }
  Lt = t.m + logf(t.s);
  Ld = d.m + logf(d.s);
}

template <bool DENSE>
__global__ __launch_bounds__(kSplitThreads) void overlap_fused(OverlapArgs a) {
  constexpr int NW = kSplitThreads / kWave;
  __shared__ LseState red_l[NW];
  __shared__ float red_f[NW];
  __shared__ int flag_s;
  __shared__ float L_s[2];
  __shared__ float al_s[kFusedFinishRows];
  __shared__ unsigned char va_s[kFusedFinishRows];
  const int c = blockIdx.x, row = blockIdx.y, tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int rows = a.N * a.gamma;
  const bool valid = !a.valid || a.valid[row];
  const size_t V = static_cast<size_t>(a.V);
  const int e0 = c * a.chunk4, e1 = min(e0 + a.chunk4, a.V / 4);
  const f32x4* tp = reinterpret_cast<const f32x4*>(a.teacher + row * V);
  const f32x4* dp = reinterpret_cast<const f32x4*>(DENSE ? a.draft + row * V : a.teacher + row * V);
  unsigned* sy = a.sync;
  unsigned long long* slot = a.ws_fused + (static_cast<size_t>(row) * a.nchunk + c) * 3;

  f32x4 tv[kFusedPer], dv[kFusedPer];
  LseState lt{kNegInf, 0.f}, ld{kNegInf, 0.f};
#pragma unroll
  for (int i = 0; i < kFusedPer; ++i) {
    const int e = e0 + tid + i * kSplitThreads;
    const bool on = valid && e < e1;
    tv[i] = on ? tp[e] : f32x4{kNegInf, kNegInf, kNegInf, kNegInf};
    dv[i] = (DENSE && on) ? dp[e] : f32x4{kNegInf, kNegInf, kNegInf, kNegInf};
  }
#pragma unroll
  for (int i = 0; i < kFusedPer; ++i) {
    if (valid && e0 + tid + i * kSplitThreads < e1) {
      online_add4(lt, tv[i]);
      if (DENSE) online_add4(ld, dv[i]);
    }
  }
  const LseState rt = block_lse_state<NW>(lt, red_l);
  const LseState rd = block_lse_state<NW>(ld, red_l);

  // 1. publish the chunk states and count the chunk in at its row
  if (tid == 0) {
    const unsigned long long o0 = xchg_dev(slot, pack2(rt.m, rt.s));
    const unsigned long long o1 = xchg_dev(slot + 1, pack2(rd.m, rd.s));
    wait_for(o0);
    wait_for(o1);
    flag_s = add_dev(sy + kOvCnt1 + 32 * row, 1u) == static_cast<unsigned>(a.nchunk) - 1u;
  }
  __syncthreads();

  if constexpr (DENSE) {
    // 2. the row's last arriver publishes the normalisers; every chunk waits for them
    if (flag_s && w == 0) {
      float Lt, Ld;
      fold_row_states(a, row, lane, Lt, Ld);
      if (lane == 0 && valid && a.lse_draft) a.lse_draft[row] = Ld;
      // each normaliser travels with this call's number in one 64-bit word,
      // so the word is its own release flag
      if (lane < 2) {
        const unsigned long long tagged =
            (static_cast<unsigned long long>(a.epoch) << 32) | __float_as_uint(lane == 0 ? Lt : Ld);
        __hip_atomic_store(a.ws_norm + 2 * row + lane, tagged, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      }
    }
    if (tid == 0) {
      const unsigned long long t0 = wall_clock64();
      unsigned long long nt, nd;
      while (true) {
        nt = ld_dev(a.ws_norm + 2 * row);
        nd = ld_dev(a.ws_norm + 2 * row + 1);
        if (static_cast<unsigned>(nt >> 32) == a.epoch && static_cast<unsigned>(nd >> 32) == a.epoch) break;
        if (wall_clock64() - t0 > a.wait_ticks) {
          __hip_atomic_store(sy + kOvTimeout, a.epoch, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
          break;
        }
        __builtin_amdgcn_s_sleep(1);
      }
      L_s[0] = __uint_as_float(static_cast<uint32_t>(nt));
      L_s[1] = __uint_as_float(static_cast<uint32_t>(nd));
    }
    __syncthreads();
    // 3. this chunk's overlap sum; the row's last chunk counts the row in, the
    //    call's last row finishes every row
    const float Lt = L_s[0], Ld = L_s[1];
    float sm = 0.f;
#pragma unroll
    for (int i = 0; i < kFusedPer; ++i)
      if (valid && e0 + tid + i * kSplitThreads < e1) sm += sum_exp_min4(tv[i], dv[i], Lt, Ld);
    const float tot = block_sum<NW>(sm, red_f);
    if (tid == 0) {
      wait_for(xchg_dev(slot + 2, __float_as_uint(tot)));
      bool last = add_dev(sy + kOvCnt2 + 32 * row, 1u) == static_cast<unsigned>(a.nchunk) - 1u;
      if (last) last = add_dev(sy + kOvRowsDone, 1u) == static_cast<unsigned>(rows) - 1u;
      flag_s = last;
    }
    __syncthreads();
    if (!flag_s) return;
    // 4. alpha of every row from its chunk sums in chunk order
    for (int r = w; r < rows; r += NW) {
      const unsigned long long* rs = a.ws_fused + static_cast<size_t>(r) * a.nchunk * 3;
      unsigned long long sv[2] = {0ull, 0ull};                       // all loads issued first
#pragma unroll
      for (int u = 0; u < 2; ++u)
        if (lane + u * kWave < a.nchunk) sv[u] = ld_dev(rs + 3 * (lane + u * kWave) + 2);
      float s2 = __uint_as_float(static_cast<uint32_t>(sv[0])) + __uint_as_float(static_cast<uint32_t>(sv[1]));
      s2 = wave_sum(s2);
      const bool vr = !a.valid || a.valid[r];
      if (lane == 0) {
        if (vr && a.ov_sum) a.ov_sum[r] = s2;
        const float al = vr ? fminf(fmaxf(s2, 0.f), 1.f) : 0.f;
        a.alpha[r] = al;
        al_s[r] = al;
        va_s[r] = vr;
      }
    }
    __syncthreads();
  } else {
    // 2. the row's last arriver: normalisers, candidate overlap, alpha
    bool row_done = false;                       // this workgroup has written alpha[row]
    if (flag_s && w == 0) {
      float Lt, Ld;
      fold_row_states(a, row, lane, Lt, Ld);
      float sc = valid ? candidate_overlap(a, row, Lt, lane, kWave) : 0.f;
      sc = wave_sum(sc);
      if (lane == 0) {
        const float al = valid ? fminf(fmaxf(sc, 0.f), 1.f) : 0.f;
        wait_for(__hip_atomic_exchange(reinterpret_cast<unsigned*>(a.alpha) + row, __float_as_uint(al),
                                       __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT));
      }
      row_done = true;
    }
    // 3. the last row to finish computes tau
    __syncthreads();
    if (tid == 0) flag_s = 0;
    __syncthreads();
    if (row_done && tid == 0) flag_s = add_dev(sy + kOvRowsDone, 1u) == static_cast<unsigned>(rows) - 1u;
    __syncthreads();
    if (!flag_s) return;
    if (tid < rows) {
      al_s[tid] = __uint_as_float(ld_dev(reinterpret_cast<const unsigned*>(a.alpha) + tid));
      va_s[tid] = a.valid ? a.valid[tid] : 1;
    }
    __syncthreads();
  }
  fused_tau(a, al_s, va_s, ld_dev(sy + kOvTimeout) == a.epoch);
  // clear the counters used by this call (the release words and the time-out
  // word hold call numbers)
  if (tid < rows) {
    sy[kOvCnt1 + 32 * tid] = 0u;
    sy[kOvCnt2 + 32 * tid] = 0u;
  }
  if (tid == 0) sy[kOvRowsDone] = 0u;
}

__global__ __launch_bounds__(64) void tau_finish(OverlapArgs a) {
  const int G = a.gamma, F = 2 * G + 2, f = threadIdx.x;
  __shared__ double tot[2 * kMaxGamma + 2];
  if (f < F) {
    double s = 0.0;
    for (int b = 0; b < a.nblk; ++b) s += a.ws_acc[static_cast<size_t>(b) * F + f];
    tot[f] = s;
  }
  __syncthreads();
  if (f < G && a.accept_rate_at) a.accept_rate_at[f] = tot[G + f] > 0.0 ? tot[f] / tot[G + f] : 0.0;
  if (f == 0 && a.tau_mean) *a.tau_mean = tot[2 * G + 1] > 0.0 ? tot[2 * G] / tot[2 * G + 1] : 0.0;
  if (f == 0 && a.status) *a.status = call_timed_out(a) ? kStatusTimeout : kStatusOk;
}

int overlap_tau_blocks(int64_t N) { return static_cast<int>((N + kTauThreads - 1) / kTauThreads); }

int overlap_split_chunks(int64_t rows, int64_t V) {
  if (rows >= kSplitRowsMax) return 1;
  const int64_t by_size = (V + kSplitChunk - 1) / kSplitChunk;
  const int64_t by_rows = (2 * kSplitRowsMax + rows - 1) / rows;
  return static_cast<int>(by_size < by_rows ? by_size : by_rows);
}

// whether every (chunk, row) workgroup of the single-launch path fits at once
static bool fused_fits(const OverlapArgs& a, int rows) {
  const DeviceInfo d = device_info();
  if (d.cus <= 0 || d.clock_khz <= 0) return false;
  if (!a.draft) return true;                     // candidate mode: nothing waits
  int per_cu = 0;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, reinterpret_cast<const void*>(overlap_fused<true>),
                                                   kSplitThreads, 0) != hipSuccess)
    return false;
  return static_cast<long long>(per_cu) * d.cus >= static_cast<long long>(a.nchunk) * rows;
}

size_t overlap_resident_ws_bytes(int64_t rows) {
  return static_cast<size_t>(rows) * kResK * (4 * sizeof(unsigned long long) + sizeof(float));
}

// The single-read path for many rows when it applies (dense mode, the row's
// chunk fits the register sets, every workgroup resident at once; the
// environment variable DSPARK_OVERLAP_RESIDENT=0 turns it off): launches it
// with a.epoch, a.chunk4 and a.wait_ticks set and returns true.
static bool resident_rows_launch(OverlapArgs& a, int rows, hipStream_t s) {
  const char* env = std::getenv("DSPARK_OVERLAP_RESIDENT");
  if (env && env[0] == '0') return false;
  const DeviceInfo d = device_info();
  if (d.cus <= 0 || d.clock_khz <= 0) return false;
  const int n4 = a.V / 4;
  const int chunk4 = (n4 + kResK - 1) / kResK;
  const int need = (chunk4 + kResData - 1) / kResData;           // float4 per thread and array
  const void* fn = need <= 2 ? reinterpret_cast<const void*>(&overlap_rows_resident<2>)
                 : need <= 4 ? reinterpret_cast<const void*>(&overlap_rows_resident<4>)
                 : need <= 6 ? reinterpret_cast<const void*>(&overlap_rows_resident<6>) : nullptr;
  if (!fn) return false;
  int per_cu = 0;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, fn, kResThreads, 0) != hipSuccess || per_cu < 1)
    return false;
  const int S = per_cu * d.cus / kResK;
  if (S < 1 || static_cast<long long>(S) * kResMaxSlotRows < rows) return false;
  a.chunk4 = chunk4;
  a.epoch = next_epoch();
  // the wait bound: 100 ms, or DSPARK_OVERLAP_WAIT_US microseconds (a test
  // sets a bound too short to wait out, to take the time-out path)
  const char* wenv = std::getenv("DSPARK_OVERLAP_WAIT_US");
  a.wait_ticks = static_cast<unsigned long long>(d.clock_khz) *
                 (wenv ? static_cast<unsigned long long>(std::strtoull(wenv, nullptr, 10)) : 100000ull) / 1000ull;
  const dim3 grid(S * kResK);
  if (need <= 2) hipLaunchKernelGGL(overlap_rows_resident<2>, grid, dim3(kResThreads), 0, s, a, S);
  else if (need <= 4) hipLaunchKernelGGL(overlap_rows_resident<4>, grid, dim3(kResThreads), 0, s, a, S);
  else hipLaunchKernelGGL(overlap_rows_resident<6>, grid, dim3(kResThreads), 0, s, a, S);
  return true;
}

hipError_t launch_overlap_tau(OverlapArgs a, hipStream_t s) {
  a.nblk = overlap_tau_blocks(a.N);
  const int rows = a.N * a.gamma;
  if (a.nchunk > 1 && rows <= kFusedFinishRows && a.nblk == 1 && a.sync) {
    const int n4 = a.V / 4;
    a.chunk4 = (n4 + a.nchunk - 1) / a.nchunk;
    if (a.chunk4 <= kFusedPer * kSplitThreads && a.nchunk <= 2 * kWave && fused_fits(a, rows)) {
      a.epoch = next_epoch();
      a.wait_ticks = static_cast<unsigned long long>(device_info().clock_khz) * 100;   // 100 ms
      const dim3 grid(a.nchunk, rows);
      if (a.draft) hipLaunchKernelGGL(overlap_fused<true>, grid, dim3(kSplitThreads), 0, s, a);
      else hipLaunchKernelGGL(overlap_fused<false>, grid, dim3(kSplitThreads), 0, s, a);
      return hipGetLastError();
    }
  }
  if (a.nchunk <= 1 && a.draft && a.sync && a.ws_fused && a.ws_split && resident_rows_launch(a, rows, s)) {
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(overlap_rows_resident_fold, dim3((rows + 255) / 256), dim3(256), 0, s, a);
  } else if (a.nchunk <= 1 || (!a.draft && rows >= kCandRowsPath)) {
    if (rows >= 4 * device_info().cus) hipLaunchKernelGGL(overlap_rows<128>, dim3(rows), dim3(128), 0, s, a);
    else hipLaunchKernelGGL(overlap_rows<kOvThreads>, dim3(rows), dim3(kOvThreads), 0, s, a);
  } else {
    const int n4 = a.V / 4;
    a.chunk4 = (n4 + a.nchunk - 1) / a.nchunk;
    const dim3 grid(a.nchunk, rows);
    hipLaunchKernelGGL(overlap_split_stats, grid, dim3(kSplitThreads), 0, s, a);
    if (a.draft) hipLaunchKernelGGL(overlap_split_sum, grid, dim3(kSplitThreads), 0, s, a);
    if (rows <= kFusedFinishRows && a.nblk == 1) {
      hipLaunchKernelGGL(overlap_split_finish_tau, dim3(1), dim3(kTauThreads), 0, s, a);
      return hipGetLastError();
    }
    hipLaunchKernelGGL(overlap_split_finish, dim3(rows), dim3(kWave), 0, s, a);
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(tau_blocks, dim3(a.nblk), dim3(kTauThreads), 0, s, a);
  e = hipGetLastError();
  if (e != hipSuccess || a.nblk == 1) return e;
  hipLaunchKernelGGL(tau_finish, dim3(1), dim3(64), 0, s, a);
  return hipGetLastError();
}

}  // namespace dspark
