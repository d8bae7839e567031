// Rejection-sampling verification of a drafted block.
// "DeepSpec 训练全流程详解（以 Qwen3 + DSpark 为例）", §4.4 verify_draft_tokens: with
// p_j = softmax(target row j) and q_j = softmax(draft row j), drafted token
// x_j is accepted with probability min(1, p_j(x_j) / q_j(x_j)); only the
// leading run of accepts counts; after a rejection at n the next token is
// drawn from max(p_n - q_n, 0) normalised, and when all L are accepted from
// p_L.  "DSpark 论文精读", §2.1: this keeps the emitted tokens distributed as
// the target's.
//
// Randomness (the pages name no generator): Philox4x32-10 under the request's
// seed, on counter streams apart from the draft sampler's (whose counter word
// 1 is the position j < 16): acceptance uniform u_j from word 0 of counter
// (0, 2^30 | j, offset), mapped as u = (floor(w / 2^9) + 1/2) 2^-23; Gumbel
// noise for the final draw from word v mod 4 of counter (floor(v / 4),
// 2^31 | n, offset); the kernel takes the equivalent argmax of r(v) / E_v with
// E_v = -log u_v the exponential variate behind G_v = -log E_v.  Token j is accepted iff log u_j < min(0, log p_j(x_j) -
// log q_j(x_j)) (the same event as u_j < min(1, p/q)).  The final draw is
// Gumbel-max over log r(v) + G_v with r = max(p_n - q_n, 0) after a rejection
// (or r = p_n if that residual has no mass) and r = p_L otherwise.
//
// Four launches:
//  1. verify_stats: (chunk, row) workgroups give the online (max, sum-exp) of
//     every needed target row (j <= L) and draft row (j < L);
//  2. verify_decide: one wave per request folds the chunk states in a fixed
//     order into the normalisers, takes the decisions in position order and
//     stops at the first rejection;
//  3. verify_sample: (chunk, request) workgroups, with finer chunks than pass 1
//     (the pass is heavy in Philox and logarithm arithmetic), compute the best
//     Gumbel-max order key of the residual and of p_n over their chunk of row n;
//  4. verify_finish: one wave per request folds the keys into the next token.
// All HBM traffic is in pass 1 (every needed row once) and pass 3 (one target
// row and at most one draft row per request).
#include "common.h"
#include "internal.h"
#include "markov_dev.h"

namespace dspark {

constexpr int kVerThreads = 256;
constexpr int kVerChunk = 2048;           // target elements per workgroup when rows are few
constexpr uint32_t kVerUniform = 0x40000000u;
constexpr uint32_t kVerGumbel = 0x80000000u;

struct VerifyArgs {
  const float* target;       // [B][G + 1][V]
  const float* draft;        // [B][G][V]
  const int32_t* tokens;     // [B][G]
  const int32_t* lengths;    // [B] or NULL (all G)
  const uint64_t* seeds;     // [B]
  uint32_t off_lo, off_hi;
  int B, G, V;
  int nchunk, chunk4;        // pass 1: chunks per row and float4 per chunk
  int nchunk_s, chunk4_s;    // pass 3 (one row per request: finer chunks)
  int32_t* accepted;         // [B]
  int32_t* next_token;       // [B]
  float* accept_prob;        // [B][G] or NULL
  float* ws_state;           // [rows][nchunk][2]: target rows first, then draft rows
  float* ws_req;             // [B][4]: n, L_t(n), L_d(n), proposal length
  unsigned long long* ws_key;  // [B][nchunk_s][2]: residual key, target key
};

__device__ __forceinline__ int proposal_len(const VerifyArgs& a, int b) {
  return a.lengths ? min(max(a.lengths[b], 0), a.G) : a.G;
}

// 1. chunk states of the needed rows
__global__ __launch_bounds__(kVerThreads) void verify_stats(VerifyArgs a) {
  __shared__ LseState red[kVerThreads / kWave];
  const int c = blockIdx.x, r = blockIdx.y, tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int nt = a.B * (a.G + 1);
  const bool is_t = r < nt;
  const int b = is_t ? r / (a.G + 1) : (r - nt) / a.G;
  const int j = is_t ? r % (a.G + 1) : (r - nt) % a.G;
  const int L = proposal_len(a, b);
  if (is_t ? j > L : j >= L) return;                      // row not needed (whole workgroup)
  const size_t V = static_cast<size_t>(a.V);
  const f32x4* row = reinterpret_cast<const f32x4*>(is_t ? a.target + static_cast<size_t>(r) * V
                                                         : a.draft + static_cast<size_t>(r - nt) * V);
  const int e0 = c * a.chunk4, e1 = min(e0 + a.chunk4, a.V / 4);
  LseState st = range_lse<true>(row, e0 + tid, e1, kVerThreads);
#pragma unroll
  for (int o = 1; o < kWave; o <<= 1) st = lse_merge(st, shfl_xor(st, o));
  if (lane == 0) red[w] = st;
  __syncthreads();
  if (tid == 0) {
    LseState t = red[0];
    for (int i = 1; i < kVerThreads / kWave; ++i) t = lse_merge(t, red[i]);
    float* o = a.ws_state + (static_cast<size_t>(r) * a.nchunk + c) * 2;
    o[0] = t.m;
    o[1] = t.s;
  }
}

// log-normaliser of state row r, folded by one wave (every lane returns it)
__device__ float fold_lse(const VerifyArgs& a, int r) {
  const int lane = threadIdx.x & 63;
  LseState st{kNegInf, 0.f};
  const float* s = a.ws_state + static_cast<size_t>(r) * a.nchunk * 2;
  for (int c = lane; c < a.nchunk; c += kWave) st = lse_merge(st, LseState{s[2 * c], s[2 * c + 1]});
#pragma unroll
  for (int o = 1; o < kWave; o <<= 1) st = lse_merge(st, shfl_xor(st, o));
  return st.m + logf(st.s);
}

__device__ __forceinline__ int clamp_token(int x, int V) { return min(max(x, 0), V - 1); }

// 2. decisions, one wave per request
__global__ __launch_bounds__(kWave) void verify_decide(VerifyArgs a) {
  const int b = blockIdx.x, lane = threadIdx.x;
  const int L = proposal_len(a, b);
  const int nt = a.B * (a.G + 1);
  const size_t V = static_cast<size_t>(a.V);
  const uint64_t sd = a.seeds[b];
  int n = L;
  float Lt_n = 0.f, Ld_n = 0.f;
  for (int j = 0; j < L; ++j) {
    const int rt = b * (a.G + 1) + j, rd = nt + b * a.G + j;
    const float Lt = fold_lse(a, rt), Ld = fold_lse(a, rd);
    const int x = clamp_token(a.tokens[b * a.G + j], a.V);
    const float delta = (a.target[static_cast<size_t>(rt) * V + x] - Lt) -
                        (a.draft[static_cast<size_t>(b * a.G + j) * V + x] - Ld);
    const Philox4 ph = philox4x32_10(0u, kVerUniform | static_cast<uint32_t>(j), a.off_lo, a.off_hi,
                                     static_cast<uint32_t>(sd), static_cast<uint32_t>(sd >> 32));
    const float u = (static_cast<float>(ph.x >> 9) + 0.5f) * 0x1p-23f;
    if (a.accept_prob && lane == 0) a.accept_prob[b * a.G + j] = fminf(1.f, expf(delta));
    if (!(logf(u) < fminf(0.f, delta))) {
      n = j;
      Lt_n = Lt;
      Ld_n = Ld;
      break;
    }
  }
  if (n == L) Lt_n = fold_lse(a, b * (a.G + 1) + L);
  if (lane == 0) {
    if (a.accept_prob)   // positions past the decided ones
      for (int j = n < L ? n + 1 : L; j < a.G; ++j) a.accept_prob[b * a.G + j] = 0.f;
    float* q = a.ws_req + static_cast<size_t>(b) * 4;
    q[0] = __int_as_float(n);
    q[1] = Lt_n;
    q[2] = Ld_n;
    q[3] = __int_as_float(L);
    a.accepted[b] = n;
  }
}

// 3. Gumbel-max keys over one chunk of row n: the residual's and the target's
__global__ __launch_bounds__(kVerThreads) void verify_sample(VerifyArgs a) {
  __shared__ unsigned long long red[kVerThreads / kWave][2];
  const int c = blockIdx.x, b = blockIdx.y, tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const float* q = a.ws_req + static_cast<size_t>(b) * 4;
  const int n = __float_as_int(q[0]);
  const float Lt = q[1], Ld = q[2];
  const int L = __float_as_int(q[3]);
  const bool residual = n < L;
  const size_t V = static_cast<size_t>(a.V);
  const f32x4* trow = reinterpret_cast<const f32x4*>(a.target + (static_cast<size_t>(b) * (a.G + 1) + n) * V);
  const f32x4* drow = reinterpret_cast<const f32x4*>(a.draft + (static_cast<size_t>(b) * a.G + (residual ? n : 0)) * V);
  const uint64_t sd = a.seeds[b];
  const int e0 = c * a.chunk4_s, e1 = min(e0 + a.chunk4_s, a.V / 4);
  unsigned long long kr = 0ull, kt = 0ull;
  for (int e = e0 + tid; e < e1; e += kVerThreads) {
    const f32x4 t = trow[e];
    const Philox4 ph = philox4x32_10(static_cast<uint32_t>(e), kVerGumbel | static_cast<uint32_t>(n), a.off_lo,
                                     a.off_hi, static_cast<uint32_t>(sd), static_cast<uint32_t>(sd >> 32));
    const uint32_t wd[4] = {ph.x, ph.y, ph.z, ph.w};
    f32x4 d = f32x4{0.f, 0.f, 0.f, 0.f};
    if (residual) d = drow[e];
    // argmax_v log r(v) + G_v with G = -log E, E = -log u, is argmax_v r(v) / E_v:
    // one logarithm per element instead of three (a probability that
    // underflows float32 cannot win: G stays below 16.7 for this u)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const float E = neg_log_uniform(uniform_from_word(wd[i]));
      const float inv = __builtin_amdgcn_rcpf(E);         // E is normal: at least 4e-8
      const float p = __expf(t[i] - Lt);
      const unsigned long long k2 = best_key(p * inv, 4 * e + i);
      kt = k2 > kt ? k2 : kt;
      if (residual) {
        const float r = p - __expf(d[i] - Ld);
        const unsigned long long k1 = r > 0.f ? best_key(r * inv, 4 * e + i) : 0ull;
        kr = k1 > kr ? k1 : kr;
      }
    }
  }
#pragma unroll
  for (int o = 1; o < kWave; o <<= 1) {
    const unsigned long long yr = __shfl_xor(kr, o), yt = __shfl_xor(kt, o);
    kr = yr > kr ? yr : kr;
    kt = yt > kt ? yt : kt;
  }
  if (lane == 0) {
    red[w][0] = kr;
    red[w][1] = kt;
  }
  __syncthreads();
  if (tid == 0) {
    for (int i = 1; i < kVerThreads / kWave; ++i) {
      kr = red[i][0] > kr ? red[i][0] : kr;
      kt = red[i][1] > kt ? red[i][1] : kt;
    }
    unsigned long long* o = a.ws_key + (static_cast<size_t>(b) * a.nchunk_s + c) * 2;
    o[0] = kr;
    o[1] = kt;
  }
}

// 4. next token: the residual's best key, or the target's when the residual
// has no mass or every token was accepted
__global__ __launch_bounds__(kWave) void verify_finish(VerifyArgs a) {
  const int b = blockIdx.x, lane = threadIdx.x;
  unsigned long long kr = 0ull, kt = 0ull;
  const unsigned long long* k = a.ws_key + static_cast<size_t>(b) * a.nchunk_s * 2;
  for (int c = lane; c < a.nchunk_s; c += kWave) {
    kr = k[2 * c] > kr ? k[2 * c] : kr;
    kt = k[2 * c + 1] > kt ? k[2 * c + 1] : kt;
  }
#pragma unroll
  for (int o = 1; o < kWave; o <<= 1) {
    const unsigned long long yr = __shfl_xor(kr, o), yt = __shfl_xor(kt, o);
    kr = yr > kr ? yr : kr;
    kt = yt > kt ? yt : kt;
  }
  if (lane == 0) a.next_token[b] = best_index(kr != 0ull ? kr : kt);
}

// chunks per row: at most one per kVerChunk elements, and no more than it
// takes for `target` workgroups over all rows
static int chunks_for(int64_t rows, int64_t V, int64_t target) {
  const int64_t by_size = (V + kVerChunk - 1) / kVerChunk;
  const int64_t by_rows = (target + rows - 1) / rows;
  const int64_t n = by_size < by_rows ? by_size : by_rows;
  return static_cast<int>(n < 1 ? 1 : n);
}

// pass 1 streams every needed row; pass 3 one row per request, with the
// Philox and Gumbel arithmetic per element, so it is split more finely
int verify_chunks(int64_t rows, int64_t V) { return chunks_for(rows, V, 4096); }
static int verify_chunks_sample(int64_t B, int64_t V) { return chunks_for(B, V, 8192); }

size_t verify_ws_bytes(int64_t B, int64_t G, int64_t V) {
  const int64_t rows = B * (2 * G + 1);
  const int nchunk = verify_chunks(rows, V), nchunk_s = verify_chunks_sample(B, V);
  auto al = [](size_t x) { return (x + 255) & ~static_cast<size_t>(255); };
  return al(static_cast<size_t>(rows) * nchunk * 2 * 4) + al(static_cast<size_t>(B) * 16) +
         al(static_cast<size_t>(B) * nchunk_s * 16);
}

hipError_t launch_verify(const float* target, const float* draft, const int32_t* tokens, const int32_t* lengths,
                         const uint64_t* seeds, uint64_t offset, int B, int G, int V, int32_t* accepted,
                         int32_t* next_token, float* accept_prob, void* ws, hipStream_t s) {
  VerifyArgs a{};
  a.target = target;
  a.draft = draft;
  a.tokens = tokens;
  a.lengths = lengths;
  a.seeds = seeds;
  a.off_lo = static_cast<uint32_t>(offset);
  a.off_hi = static_cast<uint32_t>(offset >> 32);
  a.B = B;
  a.G = G;
  a.V = V;
  const int64_t rows = static_cast<int64_t>(B) * (2 * G + 1);
  a.nchunk = verify_chunks(rows, V);
  a.chunk4 = (V / 4 + a.nchunk - 1) / a.nchunk;
  a.nchunk_s = verify_chunks_sample(B, V);
  a.chunk4_s = (V / 4 + a.nchunk_s - 1) / a.nchunk_s;
  a.accepted = accepted;
  a.next_token = next_token;
  a.accept_prob = accept_prob;
  auto al = [](size_t x) { return (x + 255) & ~static_cast<size_t>(255); };
  char* p = static_cast<char*>(ws);
  a.ws_state = reinterpret_cast<float*>(p);
  p += al(static_cast<size_t>(rows) * a.nchunk * 2 * 4);
  a.ws_req = reinterpret_cast<float*>(p);
  p += al(static_cast<size_t>(B) * 16);
  a.ws_key = reinterpret_cast<unsigned long long*>(p);
  hipLaunchKernelGGL(verify_stats, dim3(a.nchunk, static_cast<unsigned>(rows)), dim3(kVerThreads), 0, s, a);
  hipLaunchKernelGGL(verify_decide, dim3(B), dim3(kWave), 0, s, a);
  hipLaunchKernelGGL(verify_sample, dim3(a.nchunk_s, B), dim3(kVerThreads), 0, s, a);
  hipLaunchKernelGGL(verify_finish, dim3(B), dim3(kWave), 0, s, a);
  return hipGetLastError();
}

}  // namespace dspark
