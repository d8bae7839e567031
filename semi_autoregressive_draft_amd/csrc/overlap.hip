// Distribution overlap and probabilistic acceptance length.
// "Qwen3.8-Flash-Next DSpark 训练实验", 评估口径/离线指标:
//   a_i = sum_v min(p_i(v), q_i(v)) = 1 - ||p_i - q_i||_1 / 2,
//   tau_prob = 1 + sum_{i=0}^{6} prod_{j<=i} a_j per valid block; invalid slots
//   get a_i = 0; accept_rate@i is averaged over valid slots; in the candidate
//   evaluation q is the softmax over the candidates (zero elsewhere) and p stays
//   the full-vocabulary teacher softmax.
// "DSpark 论文精读", §3.1 and the clamp to [0, 1] in its loss code.
//
// One workgroup per (block, slot) row.  Pass 1 streams both logit rows once and
// keeps per-thread online (max, sum-exp) states; a fixed-order tree gives the
// two log-normalisers L_p, L_q.  Pass 2 adds exp(min(t - L_p, d - L_q)) (one
// exponential per element, as exp is monotone) and walks the row backwards so
// that its first reads hit what pass 1 touched last.
#include "common.h"
#include "internal.h"

namespace dspark {

constexpr int kOvThreads = 512;
constexpr int kOvWaves = kOvThreads / kWave;
constexpr int kTauThreads = 256;

__device__ __forceinline__ void online_add4(LseState& st, f32x4 x) {
  const float m4 = fmaxf(fmaxf(x[0], x[1]), fmaxf(x[2], x[3]));
  if (m4 > st.m) {
    st.s = (st.m == kNegInf) ? 0.f : st.s * __expf(st.m - m4);
    st.m = m4;
  }
  st.s += (__expf(x[0] - st.m) + __expf(x[1] - st.m)) + (__expf(x[2] - st.m) + __expf(x[3] - st.m));
}

__device__ float block_lse(LseState st, LseState* red) {
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
#pragma unroll
  for (int o = 1; o < kWave; o <<= 1) st = lse_merge(st, shfl_xor(st, o));
  if (lane == 0) red[w] = st;
  __syncthreads();
  LseState r = red[0];
  for (int i = 1; i < kOvWaves; ++i) r = lse_merge(r, red[i]);
  __syncthreads();
  return r.m + logf(r.s);
}

__device__ float block_sum(float v, float* red) {
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  v = wave_sum(v);
  if (lane == 0) red[w] = v;
  __syncthreads();
  float r = 0.f;
  for (int i = 0; i < kOvWaves; ++i) r += red[i];
  return r;
}

__global__ __launch_bounds__(kOvThreads) void overlap_rows(OverlapArgs a) {
  __shared__ LseState red_l[kOvWaves];
  __shared__ float red_f[kOvWaves];
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
    LseState lt{kNegInf, 0.f}, ld{kNegInf, 0.f};
    for (int e = tid; e < n4; e += kOvThreads) {
      online_add4(lt, tp[e]);
      online_add4(ld, dp[e]);
    }
    const float Lt = block_lse(lt, red_l);
    const float Ld = block_lse(ld, red_l);
    float s = 0.f;
    const int last = (n4 - 1 - tid) >= 0 ? tid + ((n4 - 1 - tid) / kOvThreads) * kOvThreads : -1;
    for (int e = last; e >= 0; e -= kOvThreads) {
      const f32x4 t = tp[e], d = dp[e];
      s += (__expf(fminf(t[0] - Lt, d[0] - Ld)) + __expf(fminf(t[1] - Lt, d[1] - Ld))) +
           (__expf(fminf(t[2] - Lt, d[2] - Ld)) + __expf(fminf(t[3] - Lt, d[3] - Ld)));
    }
    total = block_sum(s, red_f);
  } else {
    LseState lt{kNegInf, 0.f};
    for (int e = tid; e < n4; e += kOvThreads) online_add4(lt, tp[e]);
    const float Lt = block_lse(lt, red_l);
    float s = 0.f;
    if (tid < a.k) {
      const size_t c = static_cast<size_t>(row) * a.k + tid;
      const float p = __expf(a.teacher[row * V + a.cand_idx[c]] - Lt);
      s = fminf(p, a.cand_prob[c]);
    }
    total = block_sum(s, red_f);
  }
  if (tid == 0) a.alpha[row] = fminf(fmaxf(total, 0.f), 1.f);
}

// tau per block and per-workgroup partial sums for the aggregates
__global__ __launch_bounds__(kTauThreads) void tau_blocks(OverlapArgs a) {
  __shared__ double red[kTauThreads / kWave][2 * kMaxGamma + 2];
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int n = blockIdx.x * kTauThreads + tid;
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
        const float al = a.alpha[n * G + i];
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
    a.ws_acc[static_cast<size_t>(blockIdx.x) * F + tid] = s;
  }
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
}

int overlap_tau_blocks(int64_t N) { return static_cast<int>((N + kTauThreads - 1) / kTauThreads); }

hipError_t launch_overlap_tau(OverlapArgs a, hipStream_t s) {
  a.nblk = overlap_tau_blocks(a.N);
  hipLaunchKernelGGL(overlap_rows, dim3(a.N * a.gamma), dim3(kOvThreads), 0, s, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(tau_blocks, dim3(a.nblk), dim3(kTauThreads), 0, s, a);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(tau_finish, dim3(1), dim3(64), 0, s, a);
  return hipGetLastError();
}

}  // namespace dspark
