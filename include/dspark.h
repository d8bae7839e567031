/*
 * dspark.h -- C ABI of the DSpark semi-autoregressive draft-proposal hot path
 * on AMD Instinct MI355X (gfx950).
 *
 * One block per request holds gamma slots: the anchor slot plus gamma-1 MASK
 * slots, each predicting one draft token.  The library runs, per block:
 *   S1  the LM-head contraction U = h . W_lm^T over the full vocabulary;
 *   S2+ the sequential Vanilla-Markov stage: U~_j = U_j + A[x_{j-1}] . Bm with
 *   S3  x_{-1} = anchor, then greedy argmax or Gumbel-max sampling of x_j;
 *   S4  optionally the k largest U~_j with their softmax (candidate set);
 *   S5  the confidence head c_j = sigmoid(w_c.h_j [+ w_m.A[x_{j-1}]] + b_c)
 *       and the prefix survival a_j = prod_{i<=j} c_i;
 *   S6  the offline overlap alpha_j = sum_v min(p_j, q_j) against a teacher
 *       distribution and tau_prob = 1 + sum_i prod_{j<=i} alpha_j.
 *
 * Sources, cited by page title and section:
 *   [P1] "Qwen3.8-Flash-Next DSpark 训练实验" (xpengzhao.github.io):
 *        评估口径/离线指标; Baseline 架构/Markov 顺序修正; Confidence head.
 *   [P4] "DSpark 论文精读：置信度调度推测解码、半自回归生成与大模型推理加速"
 *        (zzqdeco.github.io): §2.2, §2.3, §3.1.
 *   [P5] "DeepSpec 训练全流程详解（以 Qwen3 + DSpark 为例）"
 *        (wangjunjian.com): §4.3 propose.
 *
 * Conventions shared by every entry point
 *   - Array arguments are DEVICE pointers owned by the caller; the library
 *     never allocates, frees or keeps them.  Scratch memory comes only from the
 *     caller's workspace argument, sized by the matching *_workspace query.
 *   - Layouts are dense row-major.  Request-major rows: m = b*gamma + j.
 *   - Every call only enqueues work on `stream` and returns; results are valid
 *     once the caller synchronises that stream.  No call synchronises.
 *   - Calls are stateless and thread-safe; results are bit-identical from run
 *     to run (all reductions have a fixed order; no floating-point atomics).
 *   - Errors are returned as a status; no exception crosses the ABI.  All
 *     argument checks run on the host BEFORE any device work is enqueued, so
 *     an invalid call leaves the stream untouched.  dspark_last_error() gives
 *     a message for the last non-OK status of the calling thread.
 *   - Token and anchor ids must lie in [0, V); this is the caller's contract
 *     and is not checked on the device.
 *   - Device status word.  The calls whose kernels may wait for other
 *     workgroups of the same launch (dspark_markov_propose and
 *     dspark_markov_propose_head on the resident chain, dspark_overlap_tau and
 *     dspark_compute_loss on the single-launch path for few rows) take an
 *     optional `status` argument: a device pointer to one int32 (4-byte
 *     aligned) or NULL.  The call's last kernel sets it to DSPARK_OK, or to
 *     DSPARK_ETIMEOUT when one of those waits ran past its bound; the call's
 *     outputs are then invalid.  Read it after synchronising the stream.
 *     These waits rely on every workgroup of the launch being resident on
 *     the device at once.  On an otherwise idle device that holds (the host
 *     checks the occupancy before choosing such a launch); long-running
 *     kernels on other streams can keep workgroups from starting, which is
 *     the only way a wait can run out (100 ms bound per wait).
 */
#ifndef DSPARK_H
#define DSPARK_H

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  DSPARK_OK = 0,
  DSPARK_EINVAL = 1,       /* NULL where required, non-positive or too large size, inconsistent pointers */
  DSPARK_EUNSUPPORTED = 2, /* valid but not implemented: a dtype, an alignment, gamma > 16, topk > 32 ... */
  DSPARK_EWORKSPACE = 3,   /* workspace NULL or smaller than the *_workspace query returned */
  DSPARK_EHIP = 4,         /* a HIP launch failed; dspark_last_error() has the HIP error string */
  DSPARK_ETIMEOUT = 5      /* never returned by a call: the value the device status word takes when a
                              bounded wait inside a launch ran out (see the conventions above) */
} dspark_status_t;

/* Element types.  The type is a plain 32-bit integer rather than an enum, so
   that every value a caller passes is well defined for the library to read;
   values other than these two return DSPARK_EUNSUPPORTED. */
typedef int32_t dspark_dtype_t;
enum {
  DSPARK_F32 = 0,  /* IEEE binary32 */
  DSPARK_BF16 = 1  /* bfloat16 (upper half of a binary32) */
};

/* Message for the last non-OK status returned on this thread ("" if none). */
const char* dspark_last_error(void);

/* Library version string, e.g. "dspark-mi355x 0.1.0 gfx950". */
const char* dspark_version(void);

/*
 * S1 -- LM head.  [P4] §2.2 (U_1..U_gamma = W_lm [h_1..h_gamma]); [P1] the
 * frozen LM head maps the final draft hidden states to full-vocabulary logits;
 * [P5] §4.3 compute_logits(block_hidden).  No bias, no scaling.
 *
 *   h     [M, H]  dtype dt   final hidden states, row m = b*gamma + j
 *   w_lm  [V, H]  dtype dt   LM-head weight (nn.Linear layout)
 *   U     [M, V]  float32    output, U[m, v] = sum_k h[m, k] * w_lm[v, k],
 *                            accumulated in float32
 * Requirements: M, H, V > 0; V <= 2^31 - 1; M*V <= 2^40.  For DSPARK_BF16:
 * H % 8 == 0 and V % 8 == 0 (16-byte rows), else EUNSUPPORTED.
 */
dspark_status_t dspark_lm_head(const void* h, const void* w_lm, dspark_dtype_t dt,
                               int64_t M, int64_t H, int64_t V, float* U,
                               hipStream_t stream);

/*
 * S1 and S5 in one call: dspark_lm_head over M = B*gamma rows, and the
 * hidden-only confidence head with prefix survival of
 * dspark_confidence_survival (w_m == NULL), which depends on h alone.  [P4]
 * §2.2 and §3.1; [P1] Confidence head.  For bf16 with M <= 16 both run in
 * one launch (the LM head's first workgroup also computes the confidence
 * from the rows of h it already holds); otherwise each step has its own
 * launch.  Same arguments, layouts, requirements and errors as the two calls:
 *   h [B, gamma, H], w_lm [V, H], U [B, gamma, V] as for dspark_lm_head;
 *   w_c [H] dtype dt, b_c, conf and survival [B, gamma] float32 as for
 *   dspark_confidence_survival; gamma <= 16.
 */
dspark_status_t dspark_lm_head_confidence(const void* h, const void* w_lm, dspark_dtype_t dt,
                                          int64_t B, int64_t gamma, int64_t H, int64_t V,
                                          float* U, const void* w_c, float b_c, float* conf,
                                          float* survival, hipStream_t stream);

/*
 * Workspace size (bytes) needed by dspark_markov_propose for these sizes.
 * The workspace must be zero-filled before its first use (e.g. one
 * hipMemsetAsync at allocation); every call leaves the part that must start
 * at zero zeroed again.  One call at a time per workspace.
 */
dspark_status_t dspark_markov_propose_workspace(int64_t B, int64_t gamma, int64_t V,
                                                int32_t topk, size_t* bytes);

/*
 * How dspark_markov_propose will run the chain for these sizes on the current
 * device: *resident_workgroups > 0 when one resident kernel (a plain launch of
 * one workgroup per compute unit, after an occupancy check) keeps Bm on chip
 * for all positions with that many workgroups (bf16, B = 1 with r = 64, 128 or
 * 256, or B <= 16 with r = 256, when the share of Bm fits in registers and
 * LDS), 0 when it runs one step kernel per position.  Environment:
 * DSPARK_MARKOV_RESIDENT=0 disables the resident chain, DSPARK_MARKOV_WORKGROUPS=n
 * caps its workgroups (each then holds more of Bm).  Results agree with the
 * per-position path up to float32 summation order.  No device work.
 */
dspark_status_t dspark_markov_propose_plan(int64_t B, int64_t V, int64_t r, dspark_dtype_t wdt,
                                           int32_t* resident_workgroups);

/*
 * S2-S4 -- sequential Vanilla-Markov proposal.  [P1] Markov 顺序修正:
 * m_i = W_1[t_{i-1}], b_i = W_2 m_i, l_i = l_i^0 + b_i, with t_0 the anchor;
 * inference selects each token from l_i and feeds it to the next position.
 * [P4] §2.2: U~_j = U_j + b(x_{j-1}), x_j ~ softmax(U~_j).  [P5] §4.3:
 * sample_draft_tokens(base_logits, first_prev_token_ids = anchor).
 * Here W_1 = A (an embedding table) and W_2 m = m . Bm.
 *
 *   U          [B, gamma, V] float32   base logits (output of dspark_lm_head)
 *   anchor     [B]   int32             previous token of slot 0
 *   A          [V, r] dtype wdt        Markov down table W_1
 *   Bm         [r, V] dtype wdt        Markov up projection W_2 (r x V, row-major)
 *   temperature  0: greedy, x_j = argmax_v U~_j[v] (ties: lowest v).
 *                > 0: x_j = argmax_v (U~_j[v] / T + G[b, j, v]) (Gumbel-max),
 *                G = -log(-log u), u = (floor(w / 2^9) + 1/2) * 2^-23 where w is
 *                output word (v mod 4) of Philox4x32-10 (Salmon et al., SC'11)
 *                with key (lo32(seeds[b]), hi32(seeds[b])) and counter
 *                (v div 4, j, lo32(offset), hi32(offset)).
 *   seeds      [B]   uint64            per-request Philox keys (NULL iff T == 0)
 *   offset     Philox counter offset (e.g. the decoding round)
 *   topk       0 .. 32: also return the topk largest U~_j (value descending,
 *              ties to the lower index) and their softmax over that set.
 * Outputs:
 *   tokens     [B, gamma] int32        drafted tokens
 *   tok_logit  [B, gamma] float32      U~_j at the drafted token (may be NULL)
 *   lse        [B, gamma] float32      log sum_v exp U~_j[v] (may be NULL);
 *                                      exp(tok_logit - lse) is q_j(x_j) at T = 1
 *   topk_idx   [B, gamma, topk] int32  candidate ids (NULL iff topk == 0); -1 where a
 *                                      row has fewer than topk orderable values (NaN)
 *   topk_prob  [B, gamma, topk] float32 softmax of U~ over the candidates
 *   logits_out [B, gamma, V] float32   U~ itself (may be NULL; costs B*gamma*V*4
 *                                      bytes of extra writes)
 *   ws, ws_bytes  workspace of at least dspark_markov_propose_workspace() bytes,
 *                 zero-filled before its first use (see above)
 *   status     [1] int32 or NULL       device status word (see the conventions):
 *                                      DSPARK_ETIMEOUT when the resident chain (see
 *                                      dspark_markov_propose_plan) waited past its
 *                                      time bound (100 ms per position) for a
 *                                      workgroup that had not started; its tokens
 *                                      are then -1 and every output is invalid
 * On the per-position path a token of -1 marks a row with no orderable value
 * (every U~_j[v] NaN); the status stays DSPARK_OK.  Rows of A are gathered
 * with the previous token clamped into [0, V), so invalid anchors or -1
 * tokens give wrong but bounded reads.  A status pointer that is not 4-byte
 * aligned is EINVAL.
 * Requirements: B, gamma, V, r > 0; gamma <= 16; topk <= 32 and topk <= V;
 * V <= 2^31 - 1.  DSPARK_BF16: r % 32 == 0, r <= 1024, V % 8 == 0.
 * DSPARK_F32: r <= 1024.  Otherwise EUNSUPPORTED.  T must be finite and >= 0.
 */
dspark_status_t dspark_markov_propose(const float* U, int64_t B, int64_t gamma, int64_t V,
                                      const int32_t* anchor, const void* A, const void* Bm,
                                      dspark_dtype_t wdt, int64_t r,
                                      float temperature, const uint64_t* seeds, uint64_t offset,
                                      int32_t topk, int32_t* tokens, float* tok_logit, float* lse,
                                      int32_t* topk_idx, float* topk_prob, float* logits_out,
                                      void* ws, size_t ws_bytes, int32_t* status, hipStream_t stream);

/*
 * dspark_markov_propose without a workspace argument, for callers that cannot
 * allocate device memory: code under HIP graph capture, tight serving loops,
 * harnesses that forbid hipMalloc.  The call allocates nothing: its workspace
 * is a static scratch array of 64 MiB inside the library, one copy per
 * device, held until the process ends and zero-filled by a kernel on
 * `stream` at the first call on each device.
 *   - Limit: sizes whose dspark_markov_propose_workspace() exceeds 64 MiB are
 *     rejected with DSPARK_EWORKSPACE before any device work (at V = 151936
 *     with top-16: B = 64 fits, B = 256 does not).
 *   - Every call on a device shares that device's scratch, which keeps the
 *     last call's contents: calls that overlap in time on one device (other
 *     threads, other streams) race and give wrong results; calls issued in
 *     order on one stream are safe.
 *   - The top-k recompute of the per-position path reads Bm directly (no
 *     transposed copy); results equal dspark_markov_propose's with the plain
 *     workspace.
 * Every other argument, output, rule and error is dspark_markov_propose's.
 */
dspark_status_t dspark_markov_propose_noalloc(const float* U, int64_t B, int64_t gamma, int64_t V,
                                              const int32_t* anchor, const void* A, const void* Bm,
                                              dspark_dtype_t wdt, int64_t r,
                                              float temperature, const uint64_t* seeds, uint64_t offset,
                                              int32_t topk, int32_t* tokens, float* tok_logit,
                                              float* lse, int32_t* topk_idx, float* topk_prob,
                                              float* logits_out, int32_t* status, hipStream_t stream);

/*
 * Sequential-head variants of dspark_markov_propose.  [P4] §2.3 heads table:
 *   DSPARK_HEAD_SILU  (VanillaMarkov): b_j = W_up SiLU(W_down[x_{j-1}]),
 *   DSPARK_HEAD_GATED (GatedMarkovHead): g_j = sigmoid(W_g [h_j; W_down[x_{j-1}]]),
 *                     b_j = W_up (g_j * W_down[x_{j-1}]),
 *   DSPARK_HEAD_RNN   (RNNHead; the RNN head passage of "Baseline 架构"): a
 *                     state s_j of rank r, zero before the block, over the
 *                     input z_j = [s_{j-1}; W_down[x_{j-1}]; h_j]:
 *                     s_j = (1 - g_j) s_{j-1} + g_j tanh(W_cand z_j) with
 *                     g_j = sigmoid(W_gate z_j), and
 *                     b_j = W_up SiLU(W_out [s_j; W_down[x_{j-1}]; h_j]);
 *                     s_j is kept in the tables' dtype.  The passage's
 *                     gate values did not survive its extraction, so "gate
 *                     1 writes the candidate" is a chosen convention (the
 *                     other one is this head with W_gate negated),
 * with W_down = A [V, r] and W_up = Bm^T; DSPARK_HEAD_LINEAR is
 * dspark_markov_propose itself.  The r-vector the up-projection receives is
 * rounded to the tables' dtype (bf16: to nearest, ties to even), as a module
 * computing in that dtype hands it on.  The variants run one step per position
 * (no resident chain); every other argument, output and rule is that of
 * dspark_markov_propose.
 *
 *   head   DSPARK_HEAD_LINEAR (0), DSPARK_HEAD_SILU (1), DSPARK_HEAD_GATED (2)
 *          or DSPARK_HEAD_RNN (3)
 *   h      [B, gamma, H] dtype wdt   hidden state h_j of each position (gated, RNN)
 *   W_g    gated: [r, H + r] dtype wdt, gate weights over [h_j; A[x_{j-1}]];
 *          RNN: [3r, 2r + H] dtype wdt, the rows of W_gate, W_cand and W_out
 *          stacked, each over [state; A[x_{j-1}]; h_j]
 *   ws     at least dspark_markov_propose_head_workspace bytes, zero-filled
 *          before its first use
 * Requirements: those of dspark_markov_propose; gated and RNN: h, W_g
 * non-NULL, 0 < H <= 16384.  The RNN workspace also holds the state table
 * [B, gamma, r].
 */
#define DSPARK_HEAD_LINEAR 0
#define DSPARK_HEAD_SILU 1
#define DSPARK_HEAD_GATED 2
#define DSPARK_HEAD_RNN 3

dspark_status_t dspark_markov_propose_head_workspace(int32_t head, int64_t B, int64_t gamma, int64_t V,
                                                     int64_t r, dspark_dtype_t wdt, int32_t topk,
                                                     size_t* bytes);

/*
 * Workspace that also holds a transposed copy of Bm ([V, r], bf16) for the
 * exact top-k of S4 (an implementation choice: the pages fix what the top-k
 * is, not how its candidates are recomputed).  On the per-position path the
 * top-k recomputes the U~ of its candidate 8-column segments from Bm; read
 * from Bm [r, V], each segment takes 16 bytes of each of r rows, i.e. r whole
 * cache lines for 16 useful bytes per line.  With this larger workspace,
 * dspark_markov_propose and dspark_markov_propose_head store the transposed
 * Bm in the workspace's tail (from position 0's step kernel, or by a copy
 * kernel when that step cannot, e.g. with logits_out) and the recompute reads
 * whole row pieces, when that moves fewer bytes (large B; bf16, topk > 0, not
 * the resident chain).
 * The results are the same top-k (up to float32 summation order in the
 * recomputed values).
 *
 *   bytes  out: dspark_markov_propose_head_workspace(head, ...) plus, for bf16
 *          and topk > 0, r * V * 2 bytes rounded up to 256
 * Errors: those of dspark_markov_propose_head_workspace; an unknown wdt is
 * DSPARK_EUNSUPPORTED.
 */
dspark_status_t dspark_markov_propose_workspace_bmt(int32_t head, int64_t B, int64_t gamma, int64_t V,
                                                    int64_t r, dspark_dtype_t wdt, int32_t topk,
                                                    size_t* bytes);

dspark_status_t dspark_markov_propose_head(int32_t head, const void* h, int64_t H, const void* W_g,
                                           const float* U, int64_t B, int64_t gamma, int64_t V,
                                           const int32_t* anchor, const void* A, const void* Bm,
                                           dspark_dtype_t wdt, int64_t r, float temperature,
                                           const uint64_t* seeds, uint64_t offset, int32_t topk,
                                           int32_t* tokens, float* tok_logit, float* lse,
                                           int32_t* topk_idx, float* topk_prob, float* logits_out,
                                           void* ws, size_t ws_bytes, int32_t* status, hipStream_t stream);

/*
 * S5 -- confidence head and prefix survival.  [P1] Confidence head:
 * s_i = w_c^T [h_i; m_i] + b_c, a^_i = sigmoid(s_i), m_i = W_1[t_{i-1}];
 * [P5] §4.3 predict_confidence_step(block_hidden) (hidden states only);
 * [P4] §3.1 prefix survival a_{r,j} = prod_{i<=j} c_{r,i}.
 *
 *   h         [B, gamma, H] dtype dt   final hidden states
 *   w_c       [H] dtype dt, b_c        linear head H -> 1
 *   w_m       [r] dtype dt or NULL     weight of the Markov state m_j = A[x_{j-1}];
 *                                      NULL gives the hidden-only head
 *   A         [V, r] dtype dt          Markov table (ignored when w_m == NULL)
 *   anchor    [B] int32, tokens [B, gamma] int32   previous tokens (ignored
 *                                      when w_m == NULL; may then be NULL)
 *   conf      [B, gamma] float32       c_j = sigmoid(s_j)
 *   survival  [B, gamma] float32       a_j = prod_{i<=j} c_i
 * Requirements: B, gamma, H > 0; gamma <= 16; with w_m: r > 0, A, anchor and
 * tokens non-NULL.
 */
dspark_status_t dspark_confidence_survival(const void* h, dspark_dtype_t dt,
                                           int64_t B, int64_t gamma, int64_t H,
                                           const void* w_c, float b_c, const void* w_m,
                                           const void* A, int64_t r,
                                           const int32_t* anchor, const int32_t* tokens,
                                           float* conf, float* survival, hipStream_t stream);

/*
 * Workspace size (bytes) needed by dspark_overlap_tau for these sizes.
 */
dspark_status_t dspark_overlap_tau_workspace(int64_t N, int64_t gamma, int64_t V, size_t* bytes);

/*
 * S6 -- overlap and probabilistic acceptance length.  [P1] 离线指标:
 * a_i = sum_v min(p_i(v), q_i(v)) = 1 - ||p_i - q_i||_1 / 2;
 * tau_prob = 1 + sum_{i=0}^{gamma-1} prod_{j<=i} a_j per valid block; slots that
 * are not valid get a_i = 0; accept_rate@i is aggregated over valid slots;
 * for the candidate-set evaluation the draft is the softmax over the candidates
 * (zero elsewhere) while the teacher keeps its full-vocabulary softmax.
 * [P4] §3.1 and the clamp to [0, 1] of its loss code.
 *
 *   teacher    [N, gamma, V] float32   teacher logits, p = softmax(teacher)
 *   draft      [N, gamma, V] float32   draft logits, q = softmax(draft)  -- dense mode
 *              or NULL                 -- candidate mode, then:
 *   cand_idx   [N, gamma, k] int32     candidate ids (distinct, in [0, V)); an id outside
 *                                      [0, V) marks no candidate and adds nothing
 *   cand_prob  [N, gamma, k] float32   q' on the candidates
 *   k          candidate count (0 in dense mode)
 *   valid      [N, gamma] uint8 or NULL (all valid)
 * Outputs:
 *   alpha          [N, gamma] float32  clamp(sum_v min(p, q), 0, 1), 0 where invalid
 *   tau            [N] float32         tau_prob; 0 for a block with no valid slot
 *   accept_rate_at [gamma] float64 or NULL   sum valid*alpha / sum valid (0 if none)
 *   tau_mean       [1] float64 or NULL       mean tau over blocks with a valid slot
 *   ws, ws_bytes   workspace of at least dspark_overlap_tau_workspace() bytes,
 *                  zero-filled before its first use; every call leaves the
 *                  part that must start at zero zeroed again (one call at a
 *                  time per workspace).  Two paths wait inside one launch:
 *                  few rows (N * gamma <= 64) run as one launch whose chunks
 *                  wait for their row's normalisers, and in dense mode many
 *                  rows (N * gamma >= 1024, V <= 172032) run on a resident
 *                  grid (one workgroup per compute unit, after an occupancy
 *                  check) whose 16 workgroups per row exchange their chunk
 *                  states.  Such waits need every workgroup of the launch
 *                  resident; if other long work keeps some from starting, a
 *                  wait runs past its bound (100 ms; on the resident grid the
 *                  first time-out ends every later wait of the call) and tau
 *                  and tau_mean (and on the resident grid alpha) are NaN.
 *                  Environment: DSPARK_OVERLAP_RESIDENT=0 selects the
 *                  two-pass kernel for many rows instead (no waits).
 *   status         [1] int32 or NULL   device status word: DSPARK_ETIMEOUT when
 *                  such a wait ran out (outputs invalid), else DSPARK_OK
 * Requirements: N, gamma, V > 0; gamma <= 16; V % 4 == 0 (16-byte rows);
 * dense mode: k == 0 and cand_* NULL; candidate mode: 1 <= k <= 64 and cand_*
 * non-NULL.
 */
dspark_status_t dspark_overlap_tau(const float* teacher, const float* draft,
                                   const int32_t* cand_idx, const float* cand_prob, int32_t k,
                                   const uint8_t* valid, int64_t N, int64_t gamma, int64_t V,
                                   float* alpha, float* tau, double* accept_rate_at,
                                   double* tau_mean, void* ws, size_t ws_bytes, int32_t* status,
                                   hipStream_t stream);

/*
 * K5 -- hardware-aware prefix scheduler.  [P4] §3.2: request r verifying its
 * first l_r draft tokens costs 1 + l_r slots of the verification batch
 * B = sum_r (1 + l_r) and is expected to emit 1 + sum_{j<=l_r} a_{r,j}
 * tokens; the lengths maximise Theta = tau * SPS(B), found by one scan over
 * all (r, j) in descending order of a_{r,j}.  [P4] §7.2: SPS(B) is a table
 * measured offline.
 *
 *   survival  [R, gamma] float32       a_{r,j}; column j is position j + 1 of
 *                                      the block (the layout
 *                                      dspark_confidence_survival writes);
 *                                      non-increasing along each row for the
 *                                      lengths to be the optimum
 *   sps       [n_sps] float64          sps[B - 1] = verification steps per
 *                                      second at a batch of B tokens,
 *                                      B = 1..n_sps; finite and >= 0
 *   lengths   [R] int32 (out)          l_r in 0..gamma
 *   stats     [3] float64 (out)        {Theta*, tau*, B*} at the chosen cut
 * Semantics: values are clamped to [0, 1] (NaN read as 0); equal values are
 * taken in order of the flat index r * gamma + j; tau is the exact sum
 * rounded once to float64 and Theta one float64 product, so results are
 * bit-identical to any exact evaluation of the same definition; the first
 * (smallest-B) maximum wins; batches beyond n_sps are not admissible.
 * Requirements: R, gamma > 0; n_sps >= R; gamma <= 16; R * gamma <= 16384.
 */
dspark_status_t dspark_prefix_schedule(const float* survival, int64_t R, int64_t gamma,
                                       const double* sps, int64_t n_sps, int32_t* lengths,
                                       double* stats, hipStream_t stream);

/*
 * Teacher-forced block logits.  [P4] §2.3 (apply_block_logits: with the
 * reference tokens known, every position's Markov bias comes from its known
 * previous token in one batched step); [P5] §3.3 (prev_token_ids = [anchor,
 * t_1, ..., t_{gamma-1}]).  The bias is linear as in dspark_markov_propose:
 *   logits_out[b, j, v] = U[b, j, v] + sum_k A[prev_tokens[b, j], k] * Bm[k, v].
 *
 *   U            [B, gamma, V] float32   base logits (the LM head's output)
 *   prev_tokens  [B, gamma] int32        previous token of each position, in [0, V)
 *                                        (out-of-range values are clamped into it)
 *   A [V, r], Bm [r, V]  dtype wdt       Markov tables, as for dspark_markov_propose
 *   logits_out   [B, gamma, V] float32   (out) corrected logits U~
 * bf16 tables with r in {32, 64, 128, 256}, V % 8 == 0 and 16-byte aligned
 * arrays run on MFMA (Bm streamed once per tile range for up to 128 rows);
 * other shapes take a plain per-row kernel.
 * Requirements: B, gamma, V, r > 0; r <= 1024.
 */
dspark_status_t dspark_apply_block_logits(const float* U, int64_t B, int64_t gamma, int64_t V,
                                          const int32_t* prev_tokens, const void* A, const void* Bm,
                                          dspark_dtype_t wdt, int64_t r, float* logits_out,
                                          hipStream_t stream);

/*
 * Workspace size (bytes) needed by dspark_compute_loss for these sizes.
 */
dspark_status_t dspark_compute_loss_workspace(int64_t B, int64_t gamma, int64_t V, size_t* bytes);

/*
 * Training-loss forward.  [P4] §4.1: per position j, with p = softmax(teacher)
 * and q = softmax(draft),
 *   CE_j = -log q_j(target_j),  L1_j = sum_v |p_j(v) - q_j(v)|,
 *   alpha_j = clamp(1 - L1_j / 2, 0, 1),
 *   BCE_j = BCE-with-logits(conf_logit_j, alpha_j)
 *         = max(s, 0) - s * alpha + log(1 + exp(-|s|)),
 *   w_j = exp(-j / decay_gamma),
 *   total = lambda_ce * CE + lambda_l1 * L1 + lambda_conf * conf.
 * [P5] §3.4: aggregates are masked weighted sums over the total weight:
 *   CE = sum_{valid (b,j)} w_j CE_bj / sum_{valid} w_j, L1 likewise;
 *   conf = mean of BCE over valid positions (conf_decay == 0, as both code
 *   excerpts compute it) or weighted like CE (conf_decay != 0, [P1]'s prose).
 * The pages' defaults: lambda_ce 0.1, lambda_l1 0.9, lambda_conf 1.0,
 * decay_gamma 4.
 *
 *   draft, teacher  [B, gamma, V] float32, 16-byte aligned
 *   target          [B, gamma] int32 in [0, V)
 *   conf_logit      [B, gamma] float32 or NULL (no confidence term: BCE = 0)
 *   valid           [B, gamma] uint8 or NULL (all valid)
 *   per_pos         [B, gamma, 4] float32 (out, optional): CE, L1, alpha, BCE;
 *                   zeros at invalid positions
 *   losses          [4] float64 (out): total, CE, L1, conf; 0 when no position
 *                   is valid; NaN when a bounded wait of the overlap pass ran
 *                   out (only possible when other work occupies the device)
 *   ws, ws_bytes    workspace of at least dspark_compute_loss_workspace bytes,
 *                   zero-filled before its first use (a call leaves it ready)
 *   status          [1] int32 or NULL: device status word, DSPARK_ETIMEOUT when
 *                   the overlap pass's bounded wait ran out (losses are then NaN)
 * Requirements: B, gamma, V > 0; gamma <= 16; V % 4 == 0; decay_gamma > 0.
 */
dspark_status_t dspark_compute_loss(const float* draft, const float* teacher, const int32_t* target,
                                    const float* conf_logit, const uint8_t* valid, int64_t B,
                                    int64_t gamma, int64_t V, float lambda_ce, float lambda_l1,
                                    float lambda_conf, float decay_gamma, int32_t conf_decay,
                                    float* per_pos, double* losses, void* ws, size_t ws_bytes,
                                    int32_t* status, hipStream_t stream);

/*
 * Workspace size (bytes) needed by dspark_verify for these sizes.
 */
dspark_status_t dspark_verify_workspace(int64_t B, int64_t gamma, int64_t V, size_t* bytes);

/*
 * Rejection-sampling verification of drafted blocks.  [P5] §4.4
 * (verify_draft_tokens): with p_j = softmax(target row j) and q_j =
 * softmax(draft row j), drafted token x_j is accepted with probability
 * min(1, p_j(x_j) / q_j(x_j)); only the leading run of accepts counts; after
 * a rejection at n the next token is drawn from max(p_n - q_n, 0)
 * normalised, and when all L tokens are accepted from p_L.  [P4] §2.1: the
 * emitted tokens then follow the target's distribution exactly.
 *
 *   target_logits [B, gamma + 1, V] float32   row j: the target's logits for
 *                                             position j given the prefix up to
 *                                             x_{j-1} (row 0: after the anchor)
 *   draft_logits  [B, gamma, V] float32       the draft's logits at each position
 *   draft_tokens  [B, gamma] int32            drafted tokens x_j in [0, V)
 *   lengths       [B] int32 or NULL           proposal length L_b in 0..gamma
 *                                             (e.g. dspark_prefix_schedule's
 *                                             lengths; NULL: gamma)
 *   seeds [B] uint64, offset                  randomness: Philox4x32-10 under key
 *                                             (lo32 seed, hi32 seed); the
 *                                             acceptance uniform of position j
 *                                             from word 0 of counter (0, 2^30 | j,
 *                                             lo32 offset, hi32 offset),
 *                                             u = (floor(w / 2^9) + 1/2) 2^-23;
 *                                             the final draw is Gumbel-max with
 *                                             the noise of token v from word v mod 4
 *                                             of counter (floor(v / 4), 2^31 | n,
 *                                             lo32 offset, hi32 offset)
 *   accepted      [B] int32 (out)             number of accepted drafted tokens
 *   next_token    [B] int32 (out)             the token drawn after them
 *   accept_prob   [B, gamma] float32 (out, optional)  min(1, p/q) at the
 *                                             decided positions, 0 past them
 *   ws, ws_bytes  workspace of at least dspark_verify_workspace bytes
 * Decisions are taken as log u_j < min(0, log p_j(x_j) - log q_j(x_j)).  A
 * rejection whose residual has no mass (p_n equal to q_n after rounding) draws
 * from p_n.  Token ids outside [0, V) and lengths outside [0, gamma] are
 * clamped.
 * Requirements: B, gamma, V > 0; gamma <= 16; V % 4 == 0; logits 16-byte aligned.
 */
dspark_status_t dspark_verify(const float* target_logits, const float* draft_logits,
                              const int32_t* draft_tokens, const int32_t* lengths,
                              const uint64_t* seeds, uint64_t offset, int64_t B, int64_t gamma,
                              int64_t V, int32_t* accepted, int32_t* next_token, float* accept_prob,
                              void* ws, size_t ws_bytes, hipStream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* DSPARK_H */
