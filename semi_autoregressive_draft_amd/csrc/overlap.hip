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
#include "common.h"
#include "internal.h"

namespace dspark {

constexpr int kOvThreads = 512;
constexpr int kSplitThreads = 256;
constexpr int kTauThreads = 256;
constexpr int kSplitChunk = 2048;      // elements per workgroup on the split path
constexpr int kSplitRowsMax = 1024;    // at and above this many rows, one workgroup per row
constexpr int kFusedFinishRows = 64;   // up to this many rows, one workgroup finishes rows and tau

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
__global__ __launch_bounds__(kOvThreads) void overlap_rows(OverlapArgs a) {
  constexpr int NW = kOvThreads / kWave;
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
    const LseState lt = range_lse<false>(tp, tid, n4, kOvThreads);
    const LseState ld = range_lse<false>(dp, tid, n4, kOvThreads);
    const LseState rt = block_lse_state<NW>(lt, red_l);
    const LseState rd = block_lse_state<NW>(ld, red_l);
    const float Lt = rt.m + logf(rt.s), Ld = rd.m + logf(rd.s);
    // second pass walks down, to reuse what the first touched last
    const int last = (n4 - 1 - tid) >= 0 ? tid + ((n4 - 1 - tid) / kOvThreads) * kOvThreads : -1;
    const float s = range_min_sum<true>(tp, dp, last, 0, n4, kOvThreads, Lt, Ld);
    total = block_sum<NW>(s, red_f);
    if (tid == 0) {
      if (a.lse_draft) a.lse_draft[row] = Ld;
      if (a.ov_sum) a.ov_sum[row] = total;
    }
  } else {
    const LseState lt = range_lse<true>(tp, tid, n4, kOvThreads);   // the row is read once
    const LseState rt = block_lse_state<NW>(lt, red_l);
    total = block_sum<NW>(candidate_overlap(a, row, rt.m + logf(rt.s), tid, kOvThreads), red_f);
  }
  if (tid == 0) a.alpha[row] = fminf(fmaxf(total, 0.f), 1.f);
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
    if (tid == 0 && a.status) *a.status = kStatusOk;   // these paths never wait
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
  if (f == 0 && a.status) *a.status = kStatusOk;
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
  if (a.nchunk <= 1) {
    hipLaunchKernelGGL(overlap_rows, dim3(rows), dim3(kOvThreads), 0, s, a);
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
