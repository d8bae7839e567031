// Internal launch interface between the C ABI (dspark_api.hip) and the kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace dspark {

// compute units and wall-clock rate (kHz) of the current device; zeros when
// there is none
struct DeviceInfo { int cus = 0; int clock_khz = 0; };
DeviceInfo device_info();

constexpr int kMaxRank = 1024;
constexpr int kMaxTopk = 32;
constexpr int kMaxGamma = 16;
constexpr int kMaxCand = 64;
constexpr int kMaxLists = 256;   // workgroups of the resident chain
constexpr int kResidentMaxB = 16;
constexpr size_t kSkinnyMaxLds = 64 * 1024;
constexpr int kSyncWords = 12 * 1024;   // 48 KB: the resident chain's wait tree (zero at launch)
// Wait-tree layout in the sync block (32-bit words; counters and flags each on
// their own 256-byte line): time-out flag (holds call numbers, never
// cleared), group counters, top counter, group release flags, then the group
// keys [position][group][request] (64-bit).  Groups are kFanIn workgroups.
constexpr int kFanIn = 16;
constexpr int kSyncTimeout = 0;
constexpr int kSyncGroupCnt = 64;                       // + 64 * group
constexpr int kSyncTopCnt = kSyncGroupCnt + 64 * kFanIn;
constexpr int kSyncRelease = kSyncTopCnt + 64;          // + 64 * group
constexpr int kSyncKeys = 4096;                         // word offset of the group keys
static_assert(kSyncRelease + 64 * kFanIn <= kSyncKeys, "wait-tree layout");
static_assert(kSyncKeys + 2 * kMaxGamma * kFanIn * kResidentMaxB <= kSyncWords, "wait-tree size");
constexpr int kOvSyncWords = 8192;      // 32 KB: the single-launch overlap's counters (zero at launch)
// values of the optional device status word (the header's dspark_status_t)
constexpr int32_t kStatusOk = 0;
constexpr int32_t kStatusTimeout = 5;

// Arguments of one Markov position (step + merge kernels).
struct StepArgs {
  const float* U;          // [B, gamma, V]
  const int32_t* anchor;   // [B]
  int32_t* tokens;         // [B, gamma] (written after the chain)
  // [B, gamma] argmax keys of the resident chain: (orderable score << 32) |
  // ~index, raised with atomic max; zero between calls (the finish kernel
  // clears them after reading)
  unsigned long long* best;
  unsigned* sync;          // [kSyncWords] counters, flags and group keys of the resident chain
  unsigned epoch;          // number of this call (marks a timed-out resident chain)
  const void* Mrow;        // head vectors [B][gamma][r] (dtype of A) or NULL: rows of A by previous token
  int tile_cols;           // vocabulary columns per partial (64 resident, 128 narrow bf16, a multiple of 64 wide bf16, 256 f32)
  int resident;            // 1: the chain ran as the resident kernel
  // resident chain with top-k: each workgroup's k largest order keys of U~_j
  // (value desc, index asc), sorted, [B][gamma][nlist][topk]; 0 pads
  unsigned long long* cand_key;
  int nlist;
  const void* A;           // [V, r]
  const void* Bm;          // [r, V]
  const void* BmT;         // [V, r] copy of Bm (bf16) for the top-k recompute, or NULL
  int bmt_step;            // 1: the wide step kernel of position 0 stores BmT (no transpose launch; no dump)
  int B, gamma, V, r, j;
  int sample;              // 0 greedy, 1 Gumbel-max
  float inv_temp;
  const uint64_t* seeds;   // [B]
  uint32_t off_lo, off_hi;
  // per (request, position, tile) partials, [B][gamma][P]
  float* p_score;
  int32_t* p_idx;
  float* p_x;
  float* p_m;
  float* p_s;
  int P;                   // stride of the partial arrays
  int Pn;                  // partials actually produced (set by the launcher)
  float* segmax;           // [B][gamma][S] segment maxima (top-k only, else null)
  int S;
  float* logits_out;       // [B, gamma, V] or null
  float* tok_logit;        // [B, gamma] or null
  float* lse;              // [B, gamma] or null
  int topk;
  int32_t* topk_idx;       // [B, gamma, topk]
  float* topk_prob;
  // optional: written once per call by the fold of the last position of
  // request 0 (kStatusTimeout when the resident chain's wait ran out)
  int32_t* status;
};

size_t markov_partials(int64_t V);
size_t markov_segments(int64_t V);
int markov_tile_cols(bool bf16, bool sample, int B, int gamma, int r, int V);
bool markov_resident_plan(int B, int V, int r, int max_wg, int* nwg, size_t* lds);
hipError_t launch_markov_resident(StepArgs a, unsigned* sync, int nwg, size_t lds, hipStream_t s);
hipError_t launch_markov_position(StepArgs a, bool bf16, hipStream_t s);
hipError_t launch_markov_finish(StepArgs a, bool bf16, hipStream_t s);
// bytes of the transposed Bm copy (bf16, [V, r]), and whether building it pays
// off against the top-k recompute's cache-line amplification on the
// per-position path
size_t markov_bmt_bytes(int64_t r, int64_t V);
bool markov_bmt_pays(int64_t B, int64_t gamma, int64_t V, int64_t r, int32_t topk);
// whether position 0 of the per-position chain runs the wide step kernel, which
// then stores BmT itself
bool markov_bmt_in_step(bool sample, int B, int gamma, int r, int V);

hipError_t launch_lm_head(const void* h, const void* w, bool bf16, int64_t M, int64_t H,
                          int64_t V, float* U, hipStream_t s);
bool lm_head_skinny_fits(int64_t M, int64_t H);
// with conf != NULL (bf16, M = B gamma <= 16) also the hidden-only confidence
// head and prefix survival of dspark_confidence_survival, in the same launch
hipError_t launch_lm_head_skinny(const uint16_t* h, const uint16_t* w, int64_t M, int64_t H, int64_t V,
                                 float* U, hipStream_t s, const uint16_t* w_c = nullptr, float b_c = 0.f,
                                 int gamma = 1, float* conf = nullptr, float* surv = nullptr);

constexpr int kSchedMaxCand = 16384;   // R * gamma of the prefix scheduler (keys in LDS)
hipError_t launch_prefix_schedule(const float* survival, int R, int gamma, const double* sps, int kmax,
                                  int32_t* lengths, double* stats, hipStream_t s);
hipError_t launch_confidence(const void* h, bool bf16, int B, int gamma, int H,
                             const void* w_c, float b_c, const void* w_m, const void* A, int r,
                             const int32_t* anchor, const int32_t* tokens, float* conf,
                             float* surv, hipStream_t s);

struct OverlapArgs {
  const float* teacher;
  const float* draft;
  const int32_t* cand_idx;
  const float* cand_prob;
  int k;
  const uint8_t* valid;
  int N, gamma, V;
  float* alpha;
  float* tau;
  double* accept_rate_at;
  double* tau_mean;
  double* ws_acc;        // [nblk][2*gamma + 2] per-workgroup partial sums
  int nblk;
  float* ws_split;       // [rows][nchunk][5] chunk states (split path only)
  // single-launch path for few rows: [rows][nchunk][3] 64-bit slots (teacher
  // state, draft state, chunk sum), [rows][2] tagged row normalisers, the
  // wait words
  unsigned long long* ws_fused;
  unsigned long long* ws_norm;
  unsigned* sync;        // kOvSyncWords words, zero when a call starts
  unsigned epoch;        // number of this call
  unsigned long long wait_ticks;
  int nchunk;            // workgroups per row (1: one workgroup per row)
  int chunk4;            // float4 elements per chunk (set by the launcher)
  // optional per-row outputs of the dense mode (valid rows only): the draft's
  // log-normaliser and the unclamped sum of min(p, q)
  float* lse_draft;
  float* ov_sum;
  // optional: written once per call by the workgroup that finishes tau
  // (kStatusTimeout when a wait of the single-launch path ran out)
  int32_t* status;
};

// training-loss finish: per-row CE, L1, alpha, BCE and the weighted aggregates
struct LossArgs {
  const float* draft;
  const int32_t* target;
  const float* conf;       // NULL: no confidence term
  const uint8_t* valid;    // NULL: every position valid
  const float* lse_draft;  // per row, from the overlap pass
  const float* ov_sum;     // per row, from the overlap pass
  const float* tau;        // per block, from the overlap pass (NaN: a wait ran out)
  int N, gamma, V;
  float lambda_ce, lambda_l1, lambda_conf, decay;
  int conf_decay;
  float* per_pos;          // [rows][4] or NULL
  double* losses;          // [4]
};
hipError_t launch_loss_finish(const LossArgs& a, hipStream_t s);
hipError_t launch_block_logits(const float* U, const int32_t* prev, const void* A, const void* Bm, bool vec,
                               int M, int V, int r, float* out, hipStream_t s, bool bf16);

// sequential-head variants (markov_head_prep writes m_j before each position)
constexpr int kHeadLinear = 0, kHeadSilu = 1, kHeadGated = 2, kHeadRnn = 3;
constexpr int kMaxHeadHidden = 16384;   // H of the gated and RNN heads (their input in LDS)
hipError_t launch_head_prep(const StepArgs& a, bool bf16, int head, const void* h, int H, const void* Wg, void* M,
                            hipStream_t s);

// rejection-sampling verification
int verify_chunks(int64_t rows, int64_t V);
size_t verify_ws_bytes(int64_t B, int64_t G, int64_t V);
hipError_t launch_verify(const float* target, const float* draft, const int32_t* tokens, const int32_t* lengths,
                         const uint64_t* seeds, uint64_t offset, int B, int G, int V, int32_t* accepted,
                         int32_t* next_token, float* accept_prob, void* ws, hipStream_t s);

int overlap_tau_blocks(int64_t N);
// workspace of the single-read path for many rows: [rows][16][4] tagged 64-bit
// chunk-state words, then [rows][16] float chunk sums
size_t overlap_resident_ws_bytes(int64_t rows);
int overlap_split_chunks(int64_t rows, int64_t V);
hipError_t launch_overlap_tau(OverlapArgs a, hipStream_t s);
unsigned next_epoch();

// Workspace supplied by the library instead of the caller (the no-allocation
// propose entry point): `capacity` bytes at an address that `acquire` returns
// for the current device, zero-filled (by a kernel enqueued on `s`) the first
// time it is acquired on that device.
struct ScratchProvider {
  size_t capacity;
  hipError_t (*acquire)(hipStream_t s, void** ptr);
};

}  // namespace dspark

#include "dspark.h"

// dspark_markov_propose and its variants (dspark_api.hip): every argument
// check, then the chain.  With scratch != NULL, ws and ws_bytes are ignored
// and the workspace is scratch's (calls with larger needs are rejected).
dspark_status_t propose_impl(
    const char* fn, int head_kind, const void* h, int64_t H, const void* Wg,
    const float* U, int64_t B, int64_t gamma, int64_t V, const int32_t* anchor, const void* A,
    const void* Bm, dspark_dtype_t wdt, int64_t r, float temperature, const uint64_t* seeds,
    uint64_t offset, int32_t topk, int32_t* tokens, float* tok_logit, float* lse,
    int32_t* topk_idx, float* topk_prob, float* logits_out, void* ws, size_t ws_bytes,
    const dspark::ScratchProvider* scratch, int32_t* status, hipStream_t stream);
