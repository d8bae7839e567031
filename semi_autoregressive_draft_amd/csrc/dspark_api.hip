// C ABI of the DSpark draft-proposal hot path: argument checks, workspace
// carving and kernel dispatch.  Every check runs before anything is enqueued.
#include <algorithm>
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstdlib>
#include <cstdint>

#include "dspark.h"
#include "internal.h"

using namespace dspark;

namespace {

thread_local char g_err[512] = "";

dspark_status_t fail(dspark_status_t st, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof(g_err), fmt, ap);
  va_end(ap);
  return st;
}

dspark_status_t hip_status(hipError_t e, const char* what) {
  if (e == hipSuccess) return DSPARK_OK;
  return fail(DSPARK_EHIP, "%s: %s", what, hipGetErrorString(e));
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }
bool aligned4(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 3u) == 0; }

size_t align_up(size_t x) { return (x + 255) & ~static_cast<size_t>(255); }

constexpr int64_t kI32Max = 2147483647;

// per (request, position): 5 partial arrays of one entry per vocabulary tile,
// one 8-byte argmax key; one block for the resident chain's wait tree; with
// top-k, the segment maxima (per-position chain) and, when the batch is small
// enough for the resident chain, its per-workgroup candidate lists
size_t markov_cand_bytes(int64_t B, int64_t gamma, int32_t topk) {
  return align_up(static_cast<size_t>(B) * gamma * kMaxLists * topk * 8);
}

// The part that must be zero when a call starts (the resident chain's wait tree
// and its keys, sized for the largest resident batch) sits at a fixed offset,
// the start, so that calls of any shape find it where the last call cleared it.
constexpr size_t kZeroHead = kSyncWords * 4 + static_cast<size_t>(kResidentMaxB) * kMaxGamma * 8;

size_t markov_ws_bytes(int64_t B, int64_t gamma, int64_t V, int32_t topk) {
  const size_t rows = static_cast<size_t>(B) * gamma;
  size_t s = kZeroHead + 5 * align_up(rows * markov_partials(V) * 4);
  if (topk > 0) s += align_up(rows * markov_segments(V) * 4);
  if (topk > 0 && B <= kResidentMaxB) s += markov_cand_bytes(B, gamma, topk);
  return s;
}

// The resident chain where it applies (DSPARK_MARKOV_RESIDENT=0 turns it off,
// DSPARK_MARKOV_WORKGROUPS caps its workgroups), else one launch per position.
bool resident_chain(bool bf16, int B, int V, int r, int* nwg, size_t* lds) {
  const char* res_env = std::getenv("DSPARK_MARKOV_RESIDENT");
  const char* wg_env = std::getenv("DSPARK_MARKOV_WORKGROUPS");
  return bf16 && !(res_env && res_env[0] == '0') &&
         markov_resident_plan(B, V, r, wg_env ? std::atoi(wg_env) : 0, nwg, lds);
}

size_t overlap_ws_tau_bytes(int64_t N, int64_t gamma) {
  return align_up(static_cast<size_t>(overlap_tau_blocks(N)) * (2 * gamma + 2) * sizeof(double));
}

// zero head (the single-launch path's counters, fixed offset 0), tau
// partials, chunk states of the split path, and for the single-launch path
// the row normalisers and 64-bit chunk slots
void carve_overlap_ws(OverlapArgs& a, void* ws, int64_t N, int64_t gamma, int64_t V);

size_t overlap_ws_bytes(int64_t N, int64_t gamma, int64_t V) {
  const int64_t rows = N * gamma;
  const int nchunk = overlap_split_chunks(rows, V);
  size_t s = kOvSyncWords * 4 + overlap_ws_tau_bytes(N, gamma);
  if (nchunk > 1) {
    s += align_up(static_cast<size_t>(rows) * nchunk * 5 * sizeof(float));
    s += align_up(static_cast<size_t>(rows) * 16) + align_up(static_cast<size_t>(rows) * nchunk * 3 * 8);
  } else {
    s += align_up(overlap_resident_ws_bytes(rows));
  }
  return s;
}

// the overlap workspace: the zero head (wait words) first, then the per-block
// tau partials and, on the split path, the chunk states, tagged normalisers
// and single-launch slots
void carve_overlap_ws(OverlapArgs& a, void* ws, int64_t N, int64_t gamma, int64_t V) {
  char* p = static_cast<char*>(ws);
  a.sync = reinterpret_cast<unsigned*>(p);
  p += kOvSyncWords * 4;
  a.ws_acc = reinterpret_cast<double*>(p);
  p += overlap_ws_tau_bytes(N, gamma);
  a.nchunk = overlap_split_chunks(N * gamma, V);
  if (a.nchunk > 1) {
    const size_t rows = static_cast<size_t>(N * gamma);
    a.ws_split = reinterpret_cast<float*>(p);
    p += align_up(rows * a.nchunk * 5 * sizeof(float));
    a.ws_norm = reinterpret_cast<unsigned long long*>(p);
    p += align_up(rows * 16);
    a.ws_fused = reinterpret_cast<unsigned long long*>(p);
  } else {
    // the single-read path: tagged chunk-state words, then chunk sums
    const size_t rows = static_cast<size_t>(N * gamma);
    a.ws_fused = reinterpret_cast<unsigned long long*>(p);
    a.ws_split = reinterpret_cast<float*>(p + overlap_resident_ws_bytes(rows) - rows * 16 * sizeof(float));
  }
}

// compute_loss: the overlap workspace, then alpha [rows], tau [N], the draft
// log-normalisers [rows] and the overlap sums [rows]
size_t loss_ws_bytes(int64_t B, int64_t gamma, int64_t V) {
  const size_t rows = static_cast<size_t>(B * gamma);
  return align_up(overlap_ws_bytes(B, gamma, V)) + 3 * align_up(rows * 4) + align_up(static_cast<size_t>(B) * 4);
}

}  // namespace

extern "C" const char* dspark_last_error(void) { return g_err; }

extern "C" const char* dspark_version(void) { return "dspark-mi355x 0.1.0 gfx950"; }

// ---------------------------------------------------------------------------
namespace {
// the arguments of the LM head (dspark_lm_head and the fused call)
dspark_status_t check_lm_head(const char* fn, const void* h, const void* w_lm, dspark_dtype_t dt, int64_t M,
                              int64_t H, int64_t V, const float* U) {
  if (!h || !w_lm || !U) return fail(DSPARK_EINVAL, "%s: h, w_lm and U must be non-NULL", fn);
  if (M <= 0 || H <= 0 || V <= 0) return fail(DSPARK_EINVAL, "%s: M, H, V must be positive", fn);
  if (V > kI32Max || H > kI32Max || M > kI32Max || M * V > (int64_t(1) << 40))
    return fail(DSPARK_EINVAL, "%s: sizes too large (M=%lld H=%lld V=%lld)", fn, (long long)M, (long long)H,
                (long long)V);
  if (dt != DSPARK_F32 && dt != DSPARK_BF16) return fail(DSPARK_EUNSUPPORTED, "%s: unknown dtype %d", fn, (int)dt);
  if (dt == DSPARK_BF16) {
    if (H % 8 || V % 8) return fail(DSPARK_EUNSUPPORTED, "%s: bf16 needs H %% 8 == 0 and V %% 8 == 0", fn);
    if (!aligned16(h) || !aligned16(w_lm) || !aligned16(U))
      return fail(DSPARK_EUNSUPPORTED, "%s: bf16 operands must be 16-byte aligned", fn);
    if ((M + 127) / 128 > 65535) return fail(DSPARK_EINVAL, "%s: M too large", fn);
  } else if ((M + 63) / 64 > 65535) {
    return fail(DSPARK_EINVAL, "%s: M too large", fn);
  }
  return DSPARK_OK;
}
}  // namespace

extern "C" dspark_status_t dspark_lm_head(const void* h, const void* w_lm, dspark_dtype_t dt,
                                          int64_t M, int64_t H, int64_t V, float* U,
                                          hipStream_t stream) {
  const dspark_status_t st = check_lm_head("dspark_lm_head", h, w_lm, dt, M, H, V, U);
  if (st != DSPARK_OK) return st;
  return hip_status(launch_lm_head(h, w_lm, dt == DSPARK_BF16, M, H, V, U, stream), "dspark_lm_head");
}

extern "C" dspark_status_t dspark_lm_head_confidence(const void* h, const void* w_lm, dspark_dtype_t dt,
                                                     int64_t B, int64_t gamma, int64_t H, int64_t V, float* U,
                                                     const void* w_c, float b_c, float* conf, float* survival,
                                                     hipStream_t stream) {
  const char* fn = "dspark_lm_head_confidence";
  if (!w_c || !conf || !survival) return fail(DSPARK_EINVAL, "%s: w_c, conf and survival must be non-NULL", fn);
  if (B <= 0 || gamma <= 0) return fail(DSPARK_EINVAL, "%s: B and gamma must be positive", fn);
  if (B > kI32Max || B * gamma > kI32Max) return fail(DSPARK_EINVAL, "%s: sizes too large", fn);
  if (gamma > kMaxGamma) return fail(DSPARK_EUNSUPPORTED, "%s: gamma > %d", fn, kMaxGamma);
  const int64_t M = B * gamma;
  const dspark_status_t st = check_lm_head(fn, h, w_lm, dt, M, H, V, U);
  if (st != DSPARK_OK) return st;
  const bool bf16 = dt == DSPARK_BF16;
  hipError_t e;
  if (bf16 && lm_head_skinny_fits(M, H) && aligned16(w_c)) {   // one launch
    e = launch_lm_head_skinny(static_cast<const uint16_t*>(h), static_cast<const uint16_t*>(w_lm), M, H, V, U,
                              stream, static_cast<const uint16_t*>(w_c), b_c, static_cast<int>(gamma), conf,
                              survival);
  } else {                                                     // the two steps' own launches
    e = launch_lm_head(h, w_lm, bf16, M, H, V, U, stream);
    if (e == hipSuccess)
      e = launch_confidence(h, bf16, static_cast<int>(B), static_cast<int>(gamma), static_cast<int>(H), w_c, b_c,
                            nullptr, nullptr, 0, nullptr, nullptr, conf, survival, stream);
  }
  return hip_status(e, fn);
}

// ---------------------------------------------------------------------------
extern "C" dspark_status_t dspark_markov_propose_workspace(int64_t B, int64_t gamma, int64_t V,
                                                           int32_t topk, size_t* bytes) {
  if (!bytes) return fail(DSPARK_EINVAL, "dspark_markov_propose_workspace: bytes is NULL");
  if (B <= 0 || gamma <= 0 || V <= 0 || topk < 0)
    return fail(DSPARK_EINVAL, "dspark_markov_propose_workspace: B, gamma, V must be positive, topk >= 0");
  if (V > kI32Max || B > kI32Max) return fail(DSPARK_EINVAL, "dspark_markov_propose_workspace: sizes too large");
  *bytes = markov_ws_bytes(B, gamma, V, topk);
  return DSPARK_OK;
}

extern "C" dspark_status_t dspark_markov_propose_plan(int64_t B, int64_t V, int64_t r,
                                                      dspark_dtype_t wdt, int32_t* resident_workgroups) {
  if (!resident_workgroups) return fail(DSPARK_EINVAL, "dspark_markov_propose_plan: resident_workgroups is NULL");
  if (B <= 0 || V <= 0 || r <= 0 || V > kI32Max || B > kI32Max)
    return fail(DSPARK_EINVAL, "dspark_markov_propose_plan: B, V, r must be positive");
  int nwg = 0;
  size_t lds = 0;
  const bool res = resident_chain(wdt == DSPARK_BF16, static_cast<int>(B), static_cast<int>(V),
                                  static_cast<int>(r), &nwg, &lds);
  *resident_workgroups = res ? nwg : 0;
  return DSPARK_OK;
}

// head vectors of the sequential-head variants, after the chain's workspace
// (the RNN head's state table follows its m_j table)
size_t head_table_bytes(int head, int64_t B, int64_t gamma, int64_t r, bool bf16) {
  const size_t one = static_cast<size_t>(B) * gamma * r * (bf16 ? 2 : 4);
  return head == kHeadLinear ? 0 : align_up(head == kHeadRnn ? 2 * one : one);
}

dspark_status_t propose_impl(
    const char* fn, int head_kind, const void* h, int64_t H, const void* Wg,
    const float* U, int64_t B, int64_t gamma, int64_t V, const int32_t* anchor, const void* A,
    const void* Bm, dspark_dtype_t wdt, int64_t r, float temperature, const uint64_t* seeds,
    uint64_t offset, int32_t topk, int32_t* tokens, float* tok_logit, float* lse,
    int32_t* topk_idx, float* topk_prob, float* logits_out, void* ws, size_t ws_bytes,
    const ScratchProvider* scratch, int32_t* status, hipStream_t stream) {
  if (!U || !anchor || !A || !Bm || !tokens)
    return fail(DSPARK_EINVAL, "%s: U, anchor, A, Bm and tokens must be non-NULL", fn);
  if (B <= 0 || gamma <= 0 || V <= 0 || r <= 0)
    return fail(DSPARK_EINVAL, "%s: B, gamma, V, r must be positive", fn);
  if (V > kI32Max || B > kI32Max / 16 || B * gamma > kI32Max)
    return fail(DSPARK_EINVAL, "%s: sizes too large", fn);
  if (!std::isfinite(temperature) || temperature < 0.0f)
    return fail(DSPARK_EINVAL, "%s: temperature must be finite and >= 0", fn);
  if (temperature > 0.0f && !seeds) return fail(DSPARK_EINVAL, "%s: sampling (T > 0) needs seeds", fn);
  if (topk < 0) return fail(DSPARK_EINVAL, "%s: topk must be >= 0", fn);
  if (topk > 0 && (!topk_idx || !topk_prob))
    return fail(DSPARK_EINVAL, "%s: topk > 0 needs topk_idx and topk_prob", fn);
  if (topk == 0 && (topk_idx || topk_prob))
    return fail(DSPARK_EINVAL, "%s: topk_idx/topk_prob must be NULL when topk == 0", fn);
  if (topk > V) return fail(DSPARK_EINVAL, "%s: topk > V", fn);
  if (!aligned4(status)) return fail(DSPARK_EINVAL, "%s: status must be 4-byte aligned", fn);
  if (gamma > kMaxGamma) return fail(DSPARK_EUNSUPPORTED, "%s: gamma > %d", fn, kMaxGamma);
  if (topk > kMaxTopk) return fail(DSPARK_EUNSUPPORTED, "%s: topk > %d", fn, kMaxTopk);
  if (wdt != DSPARK_F32 && wdt != DSPARK_BF16) return fail(DSPARK_EUNSUPPORTED, "%s: unknown dtype %d", fn, (int)wdt);
  if (r > kMaxRank) return fail(DSPARK_EUNSUPPORTED, "%s: r > %d", fn, kMaxRank);
  const bool bf16 = wdt == DSPARK_BF16;
  if (bf16) {
    if (r % 32) return fail(DSPARK_EUNSUPPORTED, "%s: bf16 needs r %% 32 == 0", fn);
    if (V % 8) return fail(DSPARK_EUNSUPPORTED, "%s: bf16 needs V %% 8 == 0", fn);
    if (!aligned16(U) || !aligned16(A) || !aligned16(Bm) || (logits_out && !aligned16(logits_out)))
      return fail(DSPARK_EUNSUPPORTED, "%s: U, A, Bm, logits_out must be 16-byte aligned", fn);
  }
  const size_t need = markov_ws_bytes(B, gamma, V, topk) + head_table_bytes(head_kind, B, gamma, r, bf16);
  if (scratch) {            // the library's own scratch: exactly the plain workspace, no transposed Bm
    if (need > scratch->capacity)
      return fail(DSPARK_EWORKSPACE, "%s: these sizes need %zu bytes of scratch; the library's static scratch "
                  "holds %zu (use the entry point that takes a workspace)", fn, need, scratch->capacity);
    const hipError_t e = scratch->acquire(stream, &ws);
    if (e != hipSuccess) return hip_status(e, fn);
    ws_bytes = need;
  }
  if (!ws || ws_bytes < need)
    return fail(DSPARK_EWORKSPACE, "%s: workspace of %zu bytes needed, %zu given", fn, need, ws ? ws_bytes : 0);

  StepArgs a{};
  a.U = U;
  a.anchor = anchor;
  a.tokens = tokens;
  a.A = A;
  a.Bm = Bm;
  a.B = static_cast<int>(B);
  a.gamma = static_cast<int>(gamma);
  a.V = static_cast<int>(V);
  a.r = static_cast<int>(r);
  a.sample = temperature > 0.0f;
  a.inv_temp = temperature > 0.0f ? 1.0f / temperature : 1.0f;
  a.seeds = seeds;
  a.off_lo = static_cast<uint32_t>(offset);
  a.off_hi = static_cast<uint32_t>(offset >> 32);
  const size_t P = markov_partials(V);
  const size_t arr = align_up(static_cast<size_t>(B) * gamma * P * 4);
  char* const head = static_cast<char*>(ws);
  a.sync = reinterpret_cast<unsigned*>(head);
  a.best = reinterpret_cast<unsigned long long*>(head + kSyncWords * 4);
  char* base = head + kZeroHead;
  a.p_score = reinterpret_cast<float*>(base);
  a.p_idx = reinterpret_cast<int32_t*>(base + arr);
  a.p_x = reinterpret_cast<float*>(base + 2 * arr);
  a.p_m = reinterpret_cast<float*>(base + 3 * arr);
  a.p_s = reinterpret_cast<float*>(base + 4 * arr);
  a.P = static_cast<int>(P);
  a.S = static_cast<int>(markov_segments(V));
  char* tail = base + 5 * arr;
  a.logits_out = logits_out;
  a.tok_logit = tok_logit;
  a.lse = lse;
  a.topk = topk;
  a.topk_idx = topk_idx;
  a.topk_prob = topk_prob;
  a.status = status;
  int nwg = 0;
  size_t lds = 0;
  // the head variants run per position: the prep kernel writes m_j between positions
  const bool resident = head_kind == kHeadLinear && resident_chain(bf16, a.B, a.V, a.r, &nwg, &lds);
  void* mtab = head_kind == kHeadLinear ? nullptr : static_cast<char*>(ws) + markov_ws_bytes(B, gamma, V, topk);
  // a workspace that also holds the transposed Bm (see the _bmt query) turns on
  // the contiguous top-k recompute where it pays off
  const size_t bmt = markov_bmt_bytes(r, V);
  if (!resident && topk > 0 && bf16 && ws_bytes >= need + bmt && markov_bmt_pays(B, gamma, V, r, topk)) {
    a.BmT = static_cast<char*>(ws) + need;
    // the step kernel stores BmT at position 0 (its store-only variant has no dump)
    a.bmt_step = !logits_out && markov_bmt_in_step(a.sample != 0, a.B, a.gamma, a.r, a.V);
  }
  a.Mrow = mtab;
  a.tile_cols = resident ? 64 : markov_tile_cols(bf16, a.sample, a.B, a.gamma, a.r, a.V);
  a.resident = resident;
  a.nlist = nwg;
  if (topk > 0) {
    const size_t seg = align_up(static_cast<size_t>(B) * gamma * markov_segments(V) * 4);
    a.segmax = resident ? nullptr : reinterpret_cast<float*>(tail);
    if (resident) a.cand_key = reinterpret_cast<unsigned long long*>(tail + seg);
  }
  hipError_t e = hipSuccess;
  if (resident) {
    a.epoch = next_epoch();
    e = launch_markov_resident(a, a.sync, nwg, lds, stream);
  } else {
    for (int j = 0; j < gamma && e == hipSuccess; ++j) {
      a.j = j;
      if (mtab) e = launch_head_prep(a, bf16, head_kind, h, static_cast<int>(H), Wg, mtab, stream);
      if (e == hipSuccess) e = launch_markov_position(a, bf16, stream);
    }
  }
  if (e == hipSuccess) e = launch_markov_finish(a, bf16, stream);
  return hip_status(e, fn);
}

extern "C" dspark_status_t dspark_markov_propose(
    const float* U, int64_t B, int64_t gamma, int64_t V, const int32_t* anchor, const void* A,
    const void* Bm, dspark_dtype_t wdt, int64_t r, float temperature, const uint64_t* seeds,
    uint64_t offset, int32_t topk, int32_t* tokens, float* tok_logit, float* lse,
    int32_t* topk_idx, float* topk_prob, float* logits_out, void* ws, size_t ws_bytes,
    int32_t* status, hipStream_t stream) {
  return propose_impl("dspark_markov_propose", kHeadLinear, nullptr, 0, nullptr, U, B, gamma, V, anchor, A, Bm,
                      wdt, r, temperature, seeds, offset, topk, tokens, tok_logit, lse, topk_idx, topk_prob,
                      logits_out, ws, ws_bytes, nullptr, status, stream);
}

extern "C" dspark_status_t dspark_markov_propose_head_workspace(int32_t head, int64_t B, int64_t gamma, int64_t V,
                                                                int64_t r, dspark_dtype_t wdt, int32_t topk,
                                                                size_t* bytes) {
  const char* fn = "dspark_markov_propose_head_workspace";
  if (!bytes) return fail(DSPARK_EINVAL, "%s: bytes is NULL", fn);
  if (head != kHeadLinear && head != kHeadSilu && head != kHeadGated && head != kHeadRnn)
    return fail(DSPARK_EINVAL, "%s: unknown head %d", fn, head);
  if (B <= 0 || gamma <= 0 || V <= 0 || r <= 0 || topk < 0)
    return fail(DSPARK_EINVAL, "%s: B, gamma, V, r must be positive, topk >= 0", fn);
  if (V > kI32Max || B > kI32Max / 16 || r > kMaxRank) return fail(DSPARK_EINVAL, "%s: sizes too large", fn);
  *bytes = markov_ws_bytes(B, gamma, V, topk) + head_table_bytes(head, B, gamma, r, wdt == DSPARK_BF16);
  return DSPARK_OK;
}

extern "C" dspark_status_t dspark_markov_propose_workspace_bmt(int32_t head, int64_t B, int64_t gamma, int64_t V,
                                                               int64_t r, dspark_dtype_t wdt, int32_t topk,
                                                               size_t* bytes) {
  const char* fn = "dspark_markov_propose_workspace_bmt";
  const dspark_status_t st = dspark_markov_propose_head_workspace(head, B, gamma, V, r, wdt, topk, bytes);
  if (st != DSPARK_OK) return st;
  if (wdt != DSPARK_F32 && wdt != DSPARK_BF16) return fail(DSPARK_EUNSUPPORTED, "%s: unknown dtype %d", fn, (int)wdt);
  if (topk > 0 && wdt == DSPARK_BF16) *bytes += markov_bmt_bytes(r, V);
  return DSPARK_OK;
}

extern "C" dspark_status_t dspark_markov_propose_head(
    int32_t head, const void* h, int64_t H, const void* W_g,
    const float* U, int64_t B, int64_t gamma, int64_t V, const int32_t* anchor, const void* A,
    const void* Bm, dspark_dtype_t wdt, int64_t r, float temperature, const uint64_t* seeds,
    uint64_t offset, int32_t topk, int32_t* tokens, float* tok_logit, float* lse,
    int32_t* topk_idx, float* topk_prob, float* logits_out, void* ws, size_t ws_bytes,
    int32_t* status, hipStream_t stream) {
  const char* fn = "dspark_markov_propose_head";
  if (head != kHeadLinear && head != kHeadSilu && head != kHeadGated && head != kHeadRnn)
    return fail(DSPARK_EINVAL, "%s: unknown head %d", fn, head);
  if (head == kHeadGated || head == kHeadRnn) {
    if (!h || !W_g || H <= 0) return fail(DSPARK_EINVAL, "%s: the gated and RNN heads need h, W_g and H > 0", fn);
    if (H > kMaxHeadHidden) return fail(DSPARK_EUNSUPPORTED, "%s: H > %d", fn, kMaxHeadHidden);
  }
  return propose_impl(fn, head, h, H, W_g, U, B, gamma, V, anchor, A, Bm, wdt, r, temperature, seeds, offset, topk,
                      tokens, tok_logit, lse, topk_idx, topk_prob, logits_out, ws, ws_bytes, nullptr, status,
                      stream);
}

// ---------------------------------------------------------------------------
extern "C" dspark_status_t dspark_confidence_survival(
    const void* h, dspark_dtype_t dt, int64_t B, int64_t gamma, int64_t H, const void* w_c,
    float b_c, const void* w_m, const void* A, int64_t r, const int32_t* anchor,
    const int32_t* tokens, float* conf, float* survival, hipStream_t stream) {
  const char* fn = "dspark_confidence_survival";
  if (!h || !w_c || !conf || !survival) return fail(DSPARK_EINVAL, "%s: h, w_c, conf, survival must be non-NULL", fn);
  if (B <= 0 || gamma <= 0 || H <= 0) return fail(DSPARK_EINVAL, "%s: B, gamma, H must be positive", fn);
  if (B > kI32Max || H > kI32Max || B * gamma > kI32Max) return fail(DSPARK_EINVAL, "%s: sizes too large", fn);
  if (w_m && (!A || !anchor || !tokens || r <= 0))
    return fail(DSPARK_EINVAL, "%s: w_m needs A, anchor, tokens and r > 0", fn);
  if (gamma > kMaxGamma) return fail(DSPARK_EUNSUPPORTED, "%s: gamma > %d", fn, kMaxGamma);
  if (dt != DSPARK_F32 && dt != DSPARK_BF16) return fail(DSPARK_EUNSUPPORTED, "%s: unknown dtype %d", fn, (int)dt);
  if (w_m && r > kI32Max) return fail(DSPARK_EINVAL, "%s: r too large", fn);
  return hip_status(launch_confidence(h, dt == DSPARK_BF16, (int)B, (int)gamma, (int)H, w_c, b_c, w_m,
                                      A, w_m ? (int)r : 0, anchor, tokens, conf, survival, stream),
                    fn);
}

// ---------------------------------------------------------------------------
extern "C" dspark_status_t dspark_overlap_tau_workspace(int64_t N, int64_t gamma, int64_t V, size_t* bytes) {
  if (!bytes) return fail(DSPARK_EINVAL, "dspark_overlap_tau_workspace: bytes is NULL");
  if (N <= 0 || gamma <= 0 || V <= 0) return fail(DSPARK_EINVAL, "dspark_overlap_tau_workspace: sizes must be positive");
  if (gamma > kMaxGamma) return fail(DSPARK_EUNSUPPORTED, "dspark_overlap_tau_workspace: gamma > %d", kMaxGamma);
  if (N * gamma > kI32Max) return fail(DSPARK_EINVAL, "dspark_overlap_tau_workspace: sizes too large");
  *bytes = overlap_ws_bytes(N, gamma, V);
  return DSPARK_OK;
}

extern "C" dspark_status_t dspark_overlap_tau(const float* teacher, const float* draft,
                                              const int32_t* cand_idx, const float* cand_prob,
                                              int32_t k, const uint8_t* valid, int64_t N,
                                              int64_t gamma, int64_t V, float* alpha, float* tau,
                                              double* accept_rate_at, double* tau_mean, void* ws,
                                              size_t ws_bytes, int32_t* status, hipStream_t stream) {
  const char* fn = "dspark_overlap_tau";
  if (!teacher || !alpha || !tau) return fail(DSPARK_EINVAL, "%s: teacher, alpha, tau must be non-NULL", fn);
  if (N <= 0 || gamma <= 0 || V <= 0) return fail(DSPARK_EINVAL, "%s: N, gamma, V must be positive", fn);
  if (V > kI32Max || N * gamma > kI32Max) return fail(DSPARK_EINVAL, "%s: sizes too large", fn);
  if (draft) {
    if (k != 0 || cand_idx || cand_prob)
      return fail(DSPARK_EINVAL, "%s: dense mode needs k == 0 and NULL candidates", fn);
  } else {
    if (k <= 0 || !cand_idx || !cand_prob)
      return fail(DSPARK_EINVAL, "%s: candidate mode needs k > 0, cand_idx and cand_prob", fn);
    if (k > V) return fail(DSPARK_EINVAL, "%s: k > V", fn);
    if (k > kMaxCand) return fail(DSPARK_EUNSUPPORTED, "%s: k > %d", fn, kMaxCand);
  }
  if (gamma > kMaxGamma) return fail(DSPARK_EUNSUPPORTED, "%s: gamma > %d", fn, kMaxGamma);
  if (V % 4) return fail(DSPARK_EUNSUPPORTED, "%s: V %% 4 != 0", fn);
  if (!aligned16(teacher) || (draft && !aligned16(draft)))
    return fail(DSPARK_EUNSUPPORTED, "%s: teacher/draft must be 16-byte aligned", fn);
  if (!aligned4(status)) return fail(DSPARK_EINVAL, "%s: status must be 4-byte aligned", fn);
  const size_t need = overlap_ws_bytes(N, gamma, V);
  if (!ws || ws_bytes < need)
    return fail(DSPARK_EWORKSPACE, "%s: workspace of %zu bytes needed, %zu given", fn, need, ws ? ws_bytes : 0);
  OverlapArgs a{};
  a.teacher = teacher;
  a.draft = draft;
  a.cand_idx = cand_idx;
  a.cand_prob = cand_prob;
  a.k = draft ? 0 : k;
  a.valid = valid;
  a.N = static_cast<int>(N);
  a.gamma = static_cast<int>(gamma);
  a.V = static_cast<int>(V);
  a.alpha = alpha;
  a.tau = tau;
  a.accept_rate_at = accept_rate_at;
  a.tau_mean = tau_mean;
  a.status = status;
  carve_overlap_ws(a, ws, N, gamma, V);
  return hip_status(launch_overlap_tau(a, stream), fn);
}

// ---------------------------------------------------------------------------
extern "C" dspark_status_t dspark_prefix_schedule(const float* survival, int64_t R, int64_t gamma,
                                                  const double* sps, int64_t n_sps, int32_t* lengths,
                                                  double* stats, hipStream_t stream) {
  const char* fn = "dspark_prefix_schedule";
  if (!survival || !sps || !lengths || !stats)
    return fail(DSPARK_EINVAL, "%s: survival, sps, lengths and stats must be non-NULL", fn);
  if (R <= 0 || gamma <= 0) return fail(DSPARK_EINVAL, "%s: R and gamma must be positive", fn);
  if (n_sps < R) return fail(DSPARK_EINVAL, "%s: the SPS table (%lld entries) must reach B = R = %lld", fn,
                             static_cast<long long>(n_sps), static_cast<long long>(R));
  if (gamma > kMaxGamma) return fail(DSPARK_EUNSUPPORTED, "%s: gamma > %d", fn, kMaxGamma);
  if (R > kSchedMaxCand || R * gamma > kSchedMaxCand)
    return fail(DSPARK_EUNSUPPORTED, "%s: R * gamma > %d", fn, kSchedMaxCand);
  const int64_t kmax = std::min<int64_t>(R * gamma, n_sps - R);
  return hip_status(launch_prefix_schedule(survival, static_cast<int>(R), static_cast<int>(gamma), sps,
                                           static_cast<int>(kmax), lengths, stats, stream),
                    fn);
}

// ---------------------------------------------------------------------------
extern "C" dspark_status_t dspark_apply_block_logits(const float* U, int64_t B, int64_t gamma, int64_t V,
                                                     const int32_t* prev_tokens, const void* A, const void* Bm,
                                                     dspark_dtype_t wdt, int64_t r, float* logits_out,
                                                     hipStream_t stream) {
  const char* fn = "dspark_apply_block_logits";
  if (!U || !prev_tokens || !A || !Bm || !logits_out)
    return fail(DSPARK_EINVAL, "%s: U, prev_tokens, A, Bm and logits_out must be non-NULL", fn);
  if (B <= 0 || gamma <= 0 || V <= 0 || r <= 0) return fail(DSPARK_EINVAL, "%s: B, gamma, V, r must be positive", fn);
  if (V > kI32Max || B * gamma > kI32Max / 2) return fail(DSPARK_EINVAL, "%s: sizes too large", fn);
  if (wdt != DSPARK_F32 && wdt != DSPARK_BF16) return fail(DSPARK_EUNSUPPORTED, "%s: unknown dtype %d", fn, (int)wdt);
  if (r > kMaxRank) return fail(DSPARK_EUNSUPPORTED, "%s: r > %d", fn, kMaxRank);
  const bool bf16 = wdt == DSPARK_BF16;
  // the MFMA kernel needs 16-byte rows of U and aligned tables
  const bool vec = bf16 && V % 8 == 0 && aligned16(U) && aligned16(A) && aligned16(Bm) && aligned16(logits_out);
  return hip_status(launch_block_logits(U, prev_tokens, A, Bm, vec, static_cast<int>(B * gamma), static_cast<int>(V),
                                        static_cast<int>(r), logits_out, stream, bf16),
                    fn);
}

extern "C" dspark_status_t dspark_compute_loss_workspace(int64_t B, int64_t gamma, int64_t V, size_t* bytes) {
  if (!bytes) return fail(DSPARK_EINVAL, "dspark_compute_loss_workspace: bytes is NULL");
  if (B <= 0 || gamma <= 0 || V <= 0) return fail(DSPARK_EINVAL, "dspark_compute_loss_workspace: sizes must be positive");
  if (gamma > kMaxGamma) return fail(DSPARK_EUNSUPPORTED, "dspark_compute_loss_workspace: gamma > %d", kMaxGamma);
  if (B * gamma > kI32Max) return fail(DSPARK_EINVAL, "dspark_compute_loss_workspace: sizes too large");
  *bytes = loss_ws_bytes(B, gamma, V);
  return DSPARK_OK;
}

extern "C" dspark_status_t dspark_compute_loss(const float* draft, const float* teacher, const int32_t* target,
                                               const float* conf_logit, const uint8_t* valid, int64_t B,
                                               int64_t gamma, int64_t V, float lambda_ce, float lambda_l1,
                                               float lambda_conf, float decay_gamma, int32_t conf_decay,
                                               float* per_pos, double* losses, void* ws, size_t ws_bytes,
                                               int32_t* status, hipStream_t stream) {
  const char* fn = "dspark_compute_loss";
  if (!draft || !teacher || !target || !losses)
    return fail(DSPARK_EINVAL, "%s: draft, teacher, target and losses must be non-NULL", fn);
  if (B <= 0 || gamma <= 0 || V <= 0) return fail(DSPARK_EINVAL, "%s: B, gamma, V must be positive", fn);
  if (V > kI32Max || B * gamma > kI32Max) return fail(DSPARK_EINVAL, "%s: sizes too large", fn);
  if (!std::isfinite(decay_gamma) || decay_gamma <= 0.0f)
    return fail(DSPARK_EINVAL, "%s: decay_gamma must be finite and positive", fn);
  if (!std::isfinite(lambda_ce) || !std::isfinite(lambda_l1) || !std::isfinite(lambda_conf))
    return fail(DSPARK_EINVAL, "%s: the loss weights must be finite", fn);
  if (gamma > kMaxGamma) return fail(DSPARK_EUNSUPPORTED, "%s: gamma > %d", fn, kMaxGamma);
  if (V % 4) return fail(DSPARK_EUNSUPPORTED, "%s: V %% 4 != 0", fn);
  if (!aligned16(teacher) || !aligned16(draft))
    return fail(DSPARK_EUNSUPPORTED, "%s: teacher/draft must be 16-byte aligned", fn);
  if (!aligned4(status)) return fail(DSPARK_EINVAL, "%s: status must be 4-byte aligned", fn);
  const size_t need = loss_ws_bytes(B, gamma, V);
  if (!ws || ws_bytes < need)
    return fail(DSPARK_EWORKSPACE, "%s: workspace of %zu bytes needed, %zu given", fn, need, ws ? ws_bytes : 0);
  const size_t rows = static_cast<size_t>(B * gamma);
  char* tail = static_cast<char*>(ws) + align_up(overlap_ws_bytes(B, gamma, V));
  float* alpha = reinterpret_cast<float*>(tail);
  float* lse_d = reinterpret_cast<float*>(tail + align_up(rows * 4));
  float* ov = reinterpret_cast<float*>(tail + 2 * align_up(rows * 4));
  float* tau = reinterpret_cast<float*>(tail + 3 * align_up(rows * 4));
  OverlapArgs o{};
  o.teacher = teacher;
  o.draft = draft;
  o.valid = valid;
  o.N = static_cast<int>(B);
  o.gamma = static_cast<int>(gamma);
  o.V = static_cast<int>(V);
  o.alpha = alpha;
  o.tau = tau;
  o.lse_draft = lse_d;
  o.ov_sum = ov;
  o.status = status;
  carve_overlap_ws(o, ws, B, gamma, V);
  hipError_t e = launch_overlap_tau(o, stream);
  if (e != hipSuccess) return hip_status(e, fn);
  LossArgs l{};
  l.draft = draft;
  l.target = target;
  l.conf = conf_logit;
  l.valid = valid;
  l.lse_draft = lse_d;
  l.ov_sum = ov;
  l.tau = tau;
  l.N = static_cast<int>(B);
  l.gamma = static_cast<int>(gamma);
  l.V = static_cast<int>(V);
  l.lambda_ce = lambda_ce;
  l.lambda_l1 = lambda_l1;
  l.lambda_conf = lambda_conf;
  l.decay = decay_gamma;
  l.conf_decay = conf_decay != 0;
  l.per_pos = per_pos;
  l.losses = losses;
  return hip_status(launch_loss_finish(l, stream), fn);
}

// ---------------------------------------------------------------------------
extern "C" dspark_status_t dspark_verify_workspace(int64_t B, int64_t gamma, int64_t V, size_t* bytes) {
  if (!bytes) return fail(DSPARK_EINVAL, "dspark_verify_workspace: bytes is NULL");
  if (B <= 0 || gamma <= 0 || V <= 0) return fail(DSPARK_EINVAL, "dspark_verify_workspace: sizes must be positive");
  if (gamma > kMaxGamma) return fail(DSPARK_EUNSUPPORTED, "dspark_verify_workspace: gamma > %d", kMaxGamma);
  if (B * (2 * gamma + 1) > kI32Max / 2) return fail(DSPARK_EINVAL, "dspark_verify_workspace: sizes too large");
  *bytes = verify_ws_bytes(B, gamma, V);
  return DSPARK_OK;
}

extern "C" dspark_status_t dspark_verify(const float* target_logits, const float* draft_logits,
                                         const int32_t* draft_tokens, const int32_t* lengths,
                                         const uint64_t* seeds, uint64_t offset, int64_t B, int64_t gamma,
                                         int64_t V, int32_t* accepted, int32_t* next_token, float* accept_prob,
                                         void* ws, size_t ws_bytes, hipStream_t stream) {
  const char* fn = "dspark_verify";
  if (!target_logits || !draft_logits || !draft_tokens || !seeds || !accepted || !next_token)
    return fail(DSPARK_EINVAL, "%s: target_logits, draft_logits, draft_tokens, seeds, accepted and next_token must be non-NULL", fn);
  if (B <= 0 || gamma <= 0 || V <= 0) return fail(DSPARK_EINVAL, "%s: B, gamma, V must be positive", fn);
  if (V > kI32Max / 2 || B * (2 * gamma + 1) > kI32Max / 2) return fail(DSPARK_EINVAL, "%s: sizes too large", fn);
  if (gamma > kMaxGamma) return fail(DSPARK_EUNSUPPORTED, "%s: gamma > %d", fn, kMaxGamma);
  if (V % 4) return fail(DSPARK_EUNSUPPORTED, "%s: V %% 4 != 0", fn);
  if (!aligned16(target_logits) || !aligned16(draft_logits))
    return fail(DSPARK_EUNSUPPORTED, "%s: target_logits/draft_logits must be 16-byte aligned", fn);
  const size_t need = verify_ws_bytes(B, gamma, V);
  if (!ws || ws_bytes < need)
    return fail(DSPARK_EWORKSPACE, "%s: workspace of %zu bytes needed, %zu given", fn, need, ws ? ws_bytes : 0);
  return hip_status(launch_verify(target_logits, draft_logits, draft_tokens, lengths, seeds, offset,
                                  static_cast<int>(B), static_cast<int>(gamma), static_cast<int>(V), accepted,
                                  next_token, accept_prob, ws, stream),
                    fn);
}
