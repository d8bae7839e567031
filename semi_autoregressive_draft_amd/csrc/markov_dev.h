// Device helpers shared by the Markov chain kernels: the running-argmax key
// and the previous-token lookup.
#pragma once

#include "common.h"
#include "internal.h"

namespace dspark {

// Running argmax of one (request, position) as a 64-bit key whose unsigned
// order is (score ascending, then index descending): the largest key holds
// the best score with ties on the lowest index, in whatever order the tiles
// arrive.
__device__ __forceinline__ unsigned long long best_key(float score, int idx) {
  if (score == 0.f) score = 0.f;                   // -0 ranks equal to +0
  uint32_t u = __float_as_uint(score);
  u = (u & 0x80000000u) ? ~u : (u | 0x80000000u);
  return (static_cast<unsigned long long>(u) << 32) | static_cast<uint32_t>(~static_cast<uint32_t>(idx));
}

__device__ __forceinline__ int best_index(unsigned long long key) {
  return static_cast<int>(~static_cast<uint32_t>(key));
}

// the score of a key (inverse of the order map; -0 comes back as +0)
__device__ __forceinline__ float best_value(unsigned long long key) {
  const uint32_t u = static_cast<uint32_t>(key >> 32);
  return __uint_as_float((u & 0x80000000u) ? (u & 0x7FFFFFFFu) : ~u);
}

// (value descending, index ascending): the order of the top-k candidates
// (bitwise, not short-circuit, operators: no branch per comparison)
__device__ __forceinline__ bool ranks_before(float xa, int ia, float xb, int ib) {
  return (xa > xb) | ((xa == xb) & (ia < ib));
}

typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

// Four B operands (columns c = 0..3) from eight rows of four bf16 columns:
// operand c, dword p = (row 2p+1, column c) << 16 | (row 2p, column c).
__device__ __forceinline__ void transpose_rows4(const u32x2 (&rows)[8], u32x4 (&op)[4]) {
#pragma unroll
  for (int c = 0; c < 4; ++c) {
    const uint32_t sel = (c & 1) ? 0x07060302u : 0x05040100u;
#pragma unroll
    for (int p = 0; p < 4; ++p) op[c][p] = __builtin_amdgcn_perm(rows[2 * p + 1][c >> 1], rows[2 * p][c >> 1], sel);
  }
}

// Operands of chunk q of group column base `col` (= 64G + 4n), zero past V.
template <int KCH>
__device__ __forceinline__ void load_chunk(const uint16_t* Bm, size_t V, int col, bool cok, int q, int g,
                                           u32x4 (&op)[4]) {
  u32x2 rows[8];
#pragma unroll
  for (int i = 0; i < 8; ++i)
    rows[i] = cok ? *reinterpret_cast<const u32x2*>(Bm + static_cast<size_t>(32 * q + 8 * g + i) * V + col)
                  : u32x2{0u, 0u};
  transpose_rows4(rows, op);
}

// x_{j-1} of request b on the per-position chain: the anchor for j == 0, else
// the token the merge of position j-1 wrote, clamped into [0, V) so that the
// gathered table row stays inside the table (a -1 token, from a row with no
// orderable value, and an out-of-range anchor read row 0 or V - 1 instead)
__device__ __forceinline__ int prev_token(const StepArgs& a, int b, int j) {
  const int t = j == 0 ? a.anchor[b] : a.tokens[b * a.gamma + j - 1];
  return min(max(t, 0), a.V - 1);
}

// The A-operand row of (request b, position j): row x_{j-1} of A, or, with a
// sequential-head variant, row b * gamma + j of the head vectors m_j that the
// prep kernel wrote (a.Mrow, same dtype as A).
template <typename T>
__device__ __forceinline__ const T* a_operand_row(const StepArgs& a, int b, int j) {
  if (a.Mrow) return static_cast<const T*>(a.Mrow) + (static_cast<size_t>(b) * a.gamma + j) * a.r;
  return static_cast<const T*>(a.A) + static_cast<size_t>(prev_token(a, b, j)) * a.r;
}

}  // namespace dspark
