// Hardware-aware prefix scheduler: for each request r the number l_r of its
// draft tokens to verify, maximising Theta = tau(l) * SPS(B(l)) with
// B = sum_r (1 + l_r) and tau = sum_r (1 + sum_{j <= l_r} a_{r,j}).
// "DSpark 论文精读：置信度调度推测解码、半自回归生成与大模型推理加速", §3.2 (the
// objective and the scan over candidates in descending order of survival)
// and §7.2 (SPS(B) is a lookup table measured offline; the sort makes the
// step O(R gamma log(R gamma))).
//
// One workgroup of npad / E threads (E = max(2, npad / 1024) keys per
// thread, so up to 1024 threads: the compare-exchange stages are latency-bound
// and want many waves); all shared state in LDS:
//  1. 64-bit order keys: the survival value clamped to [0, 1] (NaN read as 0)
//     in the high word, the complement of the flat index r * gamma + j in the
//     low word (equal values go lower index first), zero padding up to a power
//     of two; a bitonic sort puts them in descending order.  Thread t holds
//     positions [tE, tE + E) in registers throughout: compare-exchange stages
//     whose partner is in the same thread run on registers, those whose
//     partner is in the same wave exchange through lane shuffles, and only
//     the stages with partners in other waves go through LDS (two barriers
//     each, about ten stages).
//  2. Thread t owns sorted positions [tE, tE + E).  tau at cut k (the k
//     largest values taken) is R plus a prefix sum, computed exactly in 192-bit
//     fixed point: every float in [0, 1] is an integer multiple of 2^-149
//     below 2^150, and R + 16384 such values stay below 2^43 * 2^149.  A block
//     prefix scan of the owned sums gives each cut's exact tau, which is then
//     rounded once to double, so the result does not depend on the order in
//     which the threads add.
//  3. Theta_k = tau_k * SPS(R + k) for every owned cut with R + k inside the
//     table; the block keeps the largest Theta (an order key of the double)
//     and, among equal ones, the smallest k.  Cut 0 belongs to thread 0.
//  4. l_r counts the first k* sorted candidates that belong to r (LDS
//     counters over the key buffer); stats = {Theta*, tau*, R + k*}.
#include <climits>

#include "common.h"
#include "internal.h"

namespace dspark {

constexpr int kSchedThreads = 1024;

struct Fx192 {
  unsigned long long w0, w1, w2;                 // value = (w2:w1:w0) * 2^-149
};

__device__ __forceinline__ Fx192 fx_add(const Fx192& a, const Fx192& b) {
  Fx192 r;
  r.w0 = a.w0 + b.w0;
  const unsigned long long c0 = r.w0 < a.w0 ? 1ull : 0ull;
  const unsigned long long t1 = a.w1 + b.w1;
  const unsigned long long c1 = t1 < a.w1 ? 1ull : 0ull;
  r.w1 = t1 + c0;
  const unsigned long long c2 = r.w1 < t1 ? 1ull : 0ull;
  r.w2 = a.w2 + b.w2 + c1 + c2;
  return r;
}

// a float in [0, 1] (sign clear) as an integer multiple of 2^-149
__device__ __forceinline__ Fx192 fx_of(float v) {
  const uint32_t b = __float_as_uint(v);
  const uint32_t e = b >> 23;
  const unsigned long long m = e ? ((b & 0x7FFFFFu) | 0x800000u) : (b & 0x7FFFFFu);
  const int sh = e ? static_cast<int>(e) - 1 : 0;     // 0 .. 126
  Fx192 r{0ull, 0ull, 0ull};
  if (sh < 64) {
    r.w0 = m << sh;
    r.w1 = sh ? m >> (64 - sh) : 0ull;
  } else {
    const int s = sh - 64;
    r.w1 = m << s;
    r.w2 = s ? m >> (64 - s) : 0ull;
  }
  return r;
}

__device__ __forceinline__ unsigned long long fx_limb(const Fx192& x, int i) {
  return i == 0 ? x.w0 : (i == 1 ? x.w1 : (i == 2 ? x.w2 : 0ull));
}

// round to the nearest double, ties to even
__device__ double fx_to_double(const Fx192& x) {
  int top;
  if (x.w2) top = 2;
  else if (x.w1) top = 1;
  else if (x.w0) top = 0;
  else return 0.0;
  const int p = 64 * top + 63 - __clzll(fx_limb(x, top));   // most significant set bit
  unsigned long long win;                                    // bits p-63 .. p, msb at bit 63
  bool sticky = false;                                       // any set bit below the window
  if (p < 64) {
    win = x.w0 << (63 - p);
  } else {
    const int lo = p - 63, li = lo >> 6, off = lo & 63;
    win = off ? (fx_limb(x, li) >> off) | (fx_limb(x, li + 1) << (64 - off)) : fx_limb(x, li);
    sticky = off && (fx_limb(x, li) << (64 - off)) != 0ull;
    for (int i = 0; i < li; ++i) sticky = sticky || fx_limb(x, i) != 0ull;
  }
  unsigned long long mant = win >> 11;                       // 53 bits
  const unsigned long long rem = win & 0x7FFull;
  int e = p;
  if ((rem & 0x400ull) && (sticky || (rem & 0x3FFull) || (mant & 1ull))) {
    ++mant;
    if (mant >> 53) {
      mant >>= 1;
      ++e;
    }
  }
  return ldexp(static_cast<double>(mant), e - 52 - 149);
}

// order key of a double (larger key = larger value); NaN maps to the bottom
__device__ __forceinline__ unsigned long long theta_key(double t) {
  if (!(t == t)) return 0ull;
  const unsigned long long b = static_cast<unsigned long long>(__double_as_longlong(t));
  return (b >> 63) ? ~b : (b | 0x8000000000000000ull);
}

__device__ __forceinline__ Fx192 fx_shfl_up(const Fx192& v, int d) {
  return Fx192{__shfl_up(v.w0, d), __shfl_up(v.w1, d), __shfl_up(v.w2, d)};
}

// one side of a compare-exchange: keep the larger of (x, y) when keep_max,
// else the smaller.  Keys are distinct except for equal zero padding, so one
// comparison decides.
__device__ __forceinline__ unsigned long long cx(unsigned long long x, unsigned long long y, bool keep_max) {
  return ((y > x) == keep_max) ? y : x;
}

// descending bitonic sort of npad keys, E per thread at positions tid*E + i
template <int E>
__device__ void sort_desc(unsigned long long (&x)[E], unsigned long long* lds, int npad, int tid) {
  const int lane = tid & (kWave - 1);
  for (int k = 2; k <= npad; k <<= 1) {
    for (int j = k >> 1; j >= E; j >>= 1) {
      if (j < kWave * E) {                  // partner lane tid ^ (j / E) of this wave
        const int d = j / E;
        // the direction bit k of tid * E + i is that of tid * E (i < E <= j < k)
        const bool keep_max = ((lane & d) == 0) == (((tid * E) & k) == 0);
#pragma unroll
        for (int i = 0; i < E; ++i) x[i] = cx(x[i], __shfl_xor(x[i], d), keep_max);
      } else {                              // partner in another wave: through LDS
#pragma unroll
        for (int i = 0; i < E; ++i) lds[tid * E + i] = x[i];
        __syncthreads();
#pragma unroll
        for (int i = 0; i < E; ++i) {
          const int e = tid * E + i;
          x[i] = cx(x[i], lds[e ^ j], ((e & j) == 0) == ((e & k) == 0));
        }
        __syncthreads();
      }
    }
    // partners inside the thread (j < E), compile-time register indices
#pragma unroll
    for (int j = E >> 1; j > 0; j >>= 1) {
      if (j < k) {
#pragma unroll
        for (int i = 0; i < E; ++i) {
          if ((i & j) == 0) {
            const bool desc = ((tid * E + i) & k) == 0;
            const unsigned long long a = x[i], b = x[i + j];
            const bool swap = (b > a) == desc;
            x[i] = swap ? b : a;
            x[i + j] = swap ? a : b;
          }
        }
      }
    }
  }
}

template <int E>
__global__ __launch_bounds__(kSchedThreads) void prefix_schedule_kernel(
    const float* __restrict__ surv, int R, int gamma, const double* __restrict__ sps, int kmax, int npad,
    int32_t* __restrict__ lengths, double* __restrict__ stats) {
  extern __shared__ __align__(16) unsigned long long keys[];   // [npad] exchange buffer; later the counts
  __shared__ Fx192 wave_sum[kSchedThreads / kWave];
  __shared__ unsigned long long best_key_s;
  __shared__ int best_k_s;
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int nthr = blockDim.x;               // npad / E
  const int K = R * gamma;

  // 1. keys of positions tid*E + i, then a descending bitonic sort
  unsigned long long mine[E];
#pragma unroll
  for (int i = 0; i < E; ++i) {
    const int p = tid * E + i;
    unsigned long long k = 0ull;
    if (p < K) {
      float v = surv[p];
      v = v > 0.f ? fminf(v, 1.f) : 0.f;
      k = (static_cast<unsigned long long>(__float_as_uint(v) | 0x80000000u) << 32) |
          static_cast<unsigned long long>(0xFFFFFFFFu - static_cast<uint32_t>(p));
    }
    mine[i] = k;
  }
  if (tid == 0) {
    best_key_s = 0ull;
    best_k_s = INT_MAX;
  }
  // SPS of the owned cuts (B = R + p + 1 <= R + kmax <= n_sps), fetched
  // before the sort; positions past kmax read an entry in range, unused
  double sps_own[E];
#pragma unroll
  for (int i = 0; i < E; ++i) sps_own[i] = sps[kmax > 0 ? R + min(tid * E + i, kmax - 1) : R - 1];
  const double sps_r = sps[R - 1];
  sort_desc<E>(mine, keys, npad, tid);

  // 2. owned positions and their exact sum
  const int p0 = tid * E;
  Fx192 own{0ull, 0ull, 0ull};
#pragma unroll
  for (int e = 0; e < E; ++e)
    if (p0 + e < kmax) own = fx_add(own, fx_of(__uint_as_float(static_cast<uint32_t>(mine[e] >> 32) & 0x7FFFFFFFu)));
  // block exclusive scan of the owned sums, on top of R (R * 2^149 sits at bit 21 of w2)
  Fx192 inc = own;
#pragma unroll
  for (int d = 1; d < kWave; d <<= 1) {
    const Fx192 y = fx_shfl_up(inc, d);
    if (lane >= d) inc = fx_add(inc, y);
  }
  if (lane == kWave - 1) wave_sum[w] = inc;
  Fx192 run = fx_shfl_up(inc, 1);
  if (lane == 0) run = Fx192{0ull, 0ull, 0ull};
  __syncthreads();
  run = fx_add(run, Fx192{0ull, 0ull, static_cast<unsigned long long>(R) << 21});
  for (int v = 0; v < w; ++v) run = fx_add(run, wave_sum[v]);

  // 3. Theta at each owned cut; the thread's first best
  unsigned long long tkey = 0ull;
  int tk = INT_MAX;
  double ttheta = 0.0, ttau = 0.0;
  if (tid == 0) {
    ttau = static_cast<double>(R);
    ttheta = ttau * sps_r;
    tkey = theta_key(ttheta);
    tk = 0;
  }
#pragma unroll
  for (int e = 0; e < E; ++e) {
    const int p = p0 + e;
    if (p < kmax) {
      run = fx_add(run, fx_of(__uint_as_float(static_cast<uint32_t>(mine[e] >> 32) & 0x7FFFFFFFu)));
      const double tau = fx_to_double(run);
      const double theta = tau * sps_own[e];
      const unsigned long long key = theta_key(theta);
      if (tk == INT_MAX || key > tkey) {
        tkey = key;
        tk = p + 1;
        ttheta = theta;
        ttau = tau;
      }
    }
  }
  if (tk != INT_MAX) atomicMax(&best_key_s, tkey);
  __syncthreads();
  if (tk != INT_MAX && tkey == best_key_s) atomicMin(&best_k_s, tk);
  __syncthreads();
  const int kstar = best_k_s;
  if (tk == kstar) {
    stats[0] = ttheta;
    stats[1] = ttau;
    stats[2] = static_cast<double>(R + kstar);
  }

  // 4. lengths: counters over the exchange buffer (its last use ended at a barrier)
  int* const cnt = reinterpret_cast<int*>(keys);
  for (int r = tid; r < R; r += nthr) cnt[r] = 0;
  __syncthreads();
#pragma unroll
  for (int e = 0; e < E; ++e) {
    const int p = p0 + e;
    if (p < kstar) {
      const uint32_t m = 0xFFFFFFFFu - static_cast<uint32_t>(mine[e]);
      atomicAdd(&cnt[m / static_cast<uint32_t>(gamma)], 1);
    }
  }
  __syncthreads();
  for (int r = tid; r < R; r += nthr) lengths[r] = cnt[r];
}

template <int E>
static hipError_t launch_sched(const float* survival, int R, int gamma, const double* sps, int kmax, int npad,
                               int32_t* lengths, double* stats, hipStream_t s) {
  const size_t lds = static_cast<size_t>(npad) * 8;
  if (lds > 64 * 1024) {
    const hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(&prefix_schedule_kernel<E>),
                                             hipFuncAttributeMaxDynamicSharedMemorySize, static_cast<int>(lds));
    if (e != hipSuccess) return e;
  }
  hipLaunchKernelGGL(prefix_schedule_kernel<E>, dim3(1), dim3(npad / E), lds, s, survival, R, gamma, sps, kmax,
                     npad, lengths, stats);
  return hipGetLastError();
}

// E = positions per thread: at least 2, and enough that npad / E <= 1024
hipError_t launch_prefix_schedule(const float* survival, int R, int gamma, const double* sps, int kmax,
                                  int32_t* lengths, double* stats, hipStream_t s) {
  int npad = 2;
  while (npad < R * gamma) npad <<= 1;
  if (npad <= 2 * kSchedThreads) return launch_sched<2>(survival, R, gamma, sps, kmax, npad, lengths, stats, s);
  if (npad <= 4 * kSchedThreads) return launch_sched<4>(survival, R, gamma, sps, kmax, npad, lengths, stats, s);
  if (npad <= 8 * kSchedThreads) return launch_sched<8>(survival, R, gamma, sps, kmax, npad, lengths, stats, s);
  return launch_sched<16>(survival, R, gamma, sps, kmax, npad, lengths, stats, s);
}

}  // namespace dspark
