// Device helpers shared by the DSpark hot-path kernels (gfx950, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace dspark {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr int kWave = 64;
constexpr float kNegInf = -__builtin_huge_valf();

__device__ __forceinline__ float bf16_to_f32(uint16_t b) {
  return __uint_as_float(static_cast<uint32_t>(b) << 16);
}

template <typename T> __device__ __forceinline__ float to_f32(T x);
template <> __device__ __forceinline__ float to_f32<float>(float x) { return x; }
template <> __device__ __forceinline__ float to_f32<uint16_t>(uint16_t x) { return bf16_to_f32(x); }

// Reinterpret four packed dwords (8 bf16) as an MFMA operand.
__device__ __forceinline__ bf16x8 as_bf16x8(u32x4 v) {
  return __builtin_bit_cast(bf16x8, v);
}

// -------------------------------------------------------------------------
// Philox4x32-10 (Salmon, Moraes, Dror, Shaw, SC'11): ten rounds; each round
// multiplies words 0 and 2 by the round constants, exchanges the halves of
// the products with the other words and xors in the key, which is bumped by
// the Weyl constants between rounds.
struct Philox4 { uint32_t x, y, z, w; };

__device__ __forceinline__ Philox4 philox4x32_10(uint32_t c0, uint32_t c1, uint32_t c2,
                                                 uint32_t c3, uint32_t k0, uint32_t k1) {
  constexpr uint32_t M0 = 0xD2511F53u, M1 = 0xCD9E8D57u;
  constexpr uint32_t W0 = 0x9E3779B9u, W1 = 0xBB67AE85u;
#pragma unroll
  for (int rnd = 0; rnd < 10; ++rnd) {
    // one 32 x 32 -> 64-bit product each (v_mad_u64_u32) instead of a
    // separate low and high multiply
    const uint64_t p0 = static_cast<uint64_t>(M0) * c0, p1 = static_cast<uint64_t>(M1) * c2;
    const uint32_t n0 = static_cast<uint32_t>(p1 >> 32) ^ c1 ^ k0, n2 = static_cast<uint32_t>(p0 >> 32) ^ c3 ^ k1;
    c0 = n0; c1 = static_cast<uint32_t>(p1); c2 = n2; c3 = static_cast<uint32_t>(p0);
    k0 += W0; k1 += W1;
  }
  return {c0, c1, c2, c3};
}

// Uniform from one 32-bit word: u = (w >> 9 + 1/2) 2^-23 lies in (0, 1) and is
// exact in binary32.
__device__ __forceinline__ float uniform_from_word(uint32_t w) {
  return (static_cast<float>(w >> 9) + 0.5f) * 0x1p-23f;
}

constexpr float kLn2f = 0.693147180559945309f;
constexpr float kLog2e = 1.44269504088896341f;   // 1 / ln 2

// -ln u for u on that grid, from the hardware base-2 logarithm (v_log_f32).
// Its result keeps a relative error of about one ulp even next to u = 1, where
// -ln u is tiny: over all 2^23 grid values the Gumbel noise below is within
// 1.7e-6 of its float64 value, no worse than the libm logf/log1pf pair, at two
// transcendental instructions instead of two library sequences.
__device__ __forceinline__ float neg_log_uniform(float u) { return -kLn2f * __builtin_amdgcn_logf(u); }

// Standard Gumbel noise G = -ln(-ln u) = -ln 2 log2(-log2 u) - ln ln 2.
__device__ __forceinline__ float gumbel_from_word(uint32_t w) {
  constexpr float kNegLnLn2 = 0.366512920581664327f;          // -ln(ln 2)
  const float u = uniform_from_word(w);
  return fmaf(-kLn2f, __builtin_amdgcn_logf(-__builtin_amdgcn_logf(u)), kNegLnLn2);
}

// A buffer resource over [base, base + bytes) (bytes < 2^31): loads past it
// read 0 without touching memory and stores past it are dropped.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t buf_rsrc(const void* base, size_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, static_cast<int>(bytes), 0x00020000);
}
// cache-policy operand of a buffer access: the non-temporal hint (data used
// once)
constexpr int kBufferNonTemporal = 2;

// -------------------------------------------------------------------------
// Online log-sum-exp and argmax states, merged in a fixed order.
struct LseState { float m, s; };  // value max, sum of exp(x - m)

__device__ __forceinline__ LseState lse_merge(LseState a, LseState b) {
  const float m = fmaxf(a.m, b.m);
  if (m == kNegInf) return {kNegInf, 0.0f};
  const float sa = (a.m == kNegInf) ? 0.0f : a.s * __expf(a.m - m);
  const float sb = (b.m == kNegInf) ? 0.0f : b.s * __expf(b.m - m);
  return {m, sa + sb};
}

// online (max, sum exp) update with four elements
__device__ __forceinline__ void online_add4(LseState& st, f32x4 x) {
  const float m4 = fmaxf(fmaxf(x[0], x[1]), fmaxf(x[2], x[3]));
  if (m4 > st.m) {
    st.s = (st.m == kNegInf) ? 0.f : st.s * __expf(st.m - m4);
    st.m = m4;
  }
  st.s += (__expf(x[0] - st.m) + __expf(x[1] - st.m)) + (__expf(x[2] - st.m) + __expf(x[3] - st.m));
}

// Streaming passes keep kStreamUnroll loads per thread in flight: as many
// independent online states (or partial sums), one per load slot, merged in a
// fixed order at the end.  (One state per thread serialises the loop: each
// load's value feeds the next update, and the wave waits for every load
// before issuing the next.)  NT: non-temporal loads, for rows read once.
constexpr int kStreamUnroll = 4;

template <bool NT>
__device__ __forceinline__ f32x4 ld4(const f32x4* p) {
  if constexpr (NT) return __builtin_nontemporal_load(p);
  else return *p;
}

// online (max, sum exp) of elements e0 + tid, e0 + tid + stride, ... < e1
template <bool NT>
__device__ LseState range_lse(const f32x4* p, int e0, int e1, int stride) {
  LseState st[kStreamUnroll];
#pragma unroll
  for (int u = 0; u < kStreamUnroll; ++u) st[u] = LseState{kNegInf, 0.f};
  int e = e0;
  for (; e + (kStreamUnroll - 1) * stride < e1; e += kStreamUnroll * stride) {
    f32x4 v[kStreamUnroll];
#pragma unroll
    for (int u = 0; u < kStreamUnroll; ++u) v[u] = ld4<NT>(p + e + u * stride);
#pragma unroll
    for (int u = 0; u < kStreamUnroll; ++u) online_add4(st[u], v[u]);
  }
  for (; e < e1; e += stride) online_add4(st[0], ld4<NT>(p + e));
#pragma unroll
  for (int u = 1; u < kStreamUnroll; ++u) st[0] = lse_merge(st[0], st[u]);
  return st[0];
}


struct ArgState { float score; int idx; float x; };  // best score, its index, U~ there

__device__ __forceinline__ ArgState arg_merge(ArgState a, ArgState b) {
  const bool take_b = (b.score > a.score) || (b.score == a.score && b.idx < a.idx);
  return take_b ? b : a;
}

__device__ __forceinline__ LseState shfl_xor(LseState v, int mask) {
  return {__shfl_xor(v.m, mask), __shfl_xor(v.s, mask)};
}
__device__ __forceinline__ ArgState shfl_xor(ArgState v, int mask) {
  return {__shfl_xor(v.score, mask), __shfl_xor(v.idx, mask), __shfl_xor(v.x, mask)};
}

// -------------------------------------------------------------------------
// Reductions over rows of 16 lanes through DPP lane permutes (VALU, no LDS):
// xor 1 and xor 2 within quads, then the half-row mirror (lane i <-> 7 - i)
// and the row mirror (i <-> 15 - i); in this order each step pairs lanes whose
// partial results cover disjoint lane sets, so after four steps every lane of
// a row holds the same, complete result.
constexpr int kDppXor1 = 0xB1;        // quad_perm(1, 0, 3, 2)
constexpr int kDppXor2 = 0x4E;        // quad_perm(2, 3, 0, 1)
constexpr int kDppHalfMirror = 0x141;
constexpr int kDppMirror = 0x140;

template <int CTRL>
__device__ __forceinline__ int dpp_i(int v) {
  return __builtin_amdgcn_update_dpp(0, v, CTRL, 0xF, 0xF, false);
}
template <int CTRL>
__device__ __forceinline__ float dpp_f(float v) {
  return __int_as_float(dpp_i<CTRL>(__float_as_int(v)));
}

__device__ __forceinline__ float row16_max(float v) {
  v = fmaxf(v, dpp_f<kDppXor1>(v));
  v = fmaxf(v, dpp_f<kDppXor2>(v));
  v = fmaxf(v, dpp_f<kDppHalfMirror>(v));
  return fmaxf(v, dpp_f<kDppMirror>(v));
}
__device__ __forceinline__ float row16_sum(float v) {
  v += dpp_f<kDppXor1>(v);
  v += dpp_f<kDppXor2>(v);
  v += dpp_f<kDppHalfMirror>(v);
  return v + dpp_f<kDppMirror>(v);
}
template <int CTRL>
__device__ __forceinline__ ArgState arg_step(ArgState a) {
  return arg_merge(a, ArgState{dpp_f<CTRL>(a.score), dpp_i<CTRL>(a.idx), dpp_f<CTRL>(a.x)});
}
__device__ __forceinline__ ArgState row16_arg(ArgState a) {
  a = arg_step<kDppXor1>(a);
  a = arg_step<kDppXor2>(a);
  a = arg_step<kDppHalfMirror>(a);
  return arg_step<kDppMirror>(a);
}

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o);
  return v;
}
__device__ __forceinline__ double wave_sum(double v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o);
  return v;
}
__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o));
  return v;
}

}  // namespace dspark
