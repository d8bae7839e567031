// Training-loss forward of the DSpark draft head, from the per-row results of
// the overlap pass.  "DSpark 论文精读", §4.1: per position j,
// CE_j = -log q_j(x*_j), L1_j = sum_v |p_j(v) - q_j(v)| (p = softmax(teacher),
// q = softmax(draft)), the soft label alpha_j = clamp(1 - L1_j / 2, 0, 1)
// supervising the confidence logit with BCE-with-logits, position weights
// w_j = exp(-j / gamma_decay), total = l_ce CE + l_l1 L1 + l_conf conf;
// "DeepSpec 训练全流程详解", §3.4: masked weighted sums over the total weight.
//
// The overlap kernels leave, per valid row, the draft's log-normaliser L_q
// and S = sum_v min(p, q).  Since p and q each sum to one,
// sum_v |p - q| = 2 - 2 S, so L1 = 2 - 2 S and alpha = clamp(S, 0, 1); CE is
// L_q minus the draft logit at the target.  One workgroup then walks the rows
// (thread t takes rows t, t + 256, ...), writes the per-position values and
// reduces the weighted sums in float64 in a fixed order.  A NaN tau from the
// overlap pass (a bounded wait that ran out) makes every aggregate NaN.
#include "common.h"
#include "internal.h"

namespace dspark {

constexpr int kLossThreads = 256;

__global__ __launch_bounds__(kLossThreads) void loss_finish(LossArgs a) {
  constexpr int NW = kLossThreads / kWave;
  __shared__ double red[NW][6];
  __shared__ int bad_s;
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int rows = a.N * a.gamma;
  if (tid == 0) bad_s = 0;
  __syncthreads();
  double sw = 0.0, sce = 0.0, sl1 = 0.0, sbw = 0.0, sb = 0.0, nv = 0.0;
  for (int row = tid; row < rows; row += kLossThreads) {
    const int j = row % a.gamma;
    const bool v = !a.valid || a.valid[row];
    float ce = 0.f, l1 = 0.f, al = 0.f, bce = 0.f;
    if (v) {
      const float S = a.ov_sum[row];
      l1 = 2.f - 2.f * S;
      al = fminf(fmaxf(S, 0.f), 1.f);
      ce = a.lse_draft[row] - a.draft[static_cast<size_t>(row) * a.V + a.target[row]];
      if (a.conf) {
        const float s = a.conf[row];
        bce = fmaxf(s, 0.f) - s * al + log1pf(expf(-fabsf(s)));
      }
      const double wj = exp(-static_cast<double>(j) / static_cast<double>(a.decay));
      sw += wj;
      sce += wj * ce;
      sl1 += wj * l1;
      sbw += wj * bce;
      sb += bce;
      nv += 1.0;
    }
    if (a.per_pos) {
      float* o = a.per_pos + static_cast<size_t>(row) * 4;
      o[0] = ce;
      o[1] = l1;
      o[2] = al;
      o[3] = bce;
    }
  }
  for (int b = tid; b < a.N; b += kLossThreads)
    if (!(a.tau[b] == a.tau[b])) bad_s = 1;
  const double part[6] = {sw, sce, sl1, sbw, sb, nv};
#pragma unroll
  for (int i = 0; i < 6; ++i) {
    const double s = wave_sum(part[i]);
    if (lane == 0) red[w][i] = s;
  }
  __syncthreads();
  if (tid == 0) {
    double t[6] = {0.0, 0.0, 0.0, 0.0, 0.0, 0.0};
    for (int q = 0; q < NW; ++q)
      for (int i = 0; i < 6; ++i) t[i] += red[q][i];
    const double W = t[0];
    const double ce = W > 0.0 ? t[1] / W : 0.0;
    const double l1 = W > 0.0 ? t[2] / W : 0.0;
    double cf = 0.0;
    if (a.conf) cf = a.conf_decay ? (W > 0.0 ? t[3] / W : 0.0) : (t[5] > 0.0 ? t[4] / t[5] : 0.0);
    const double total = a.lambda_ce * ce + a.lambda_l1 * l1 + a.lambda_conf * cf;
    const double nan = __builtin_nan("");
    a.losses[0] = bad_s ? nan : total;
    a.losses[1] = bad_s ? nan : ce;
    a.losses[2] = bad_s ? nan : l1;
    a.losses[3] = bad_s ? nan : cf;
  }
}

hipError_t launch_loss_finish(const LossArgs& a, hipStream_t s) {
  hipLaunchKernelGGL(loss_finish, dim3(1), dim3(kLossThreads), 0, s, a);
  return hipGetLastError();
}

}  // namespace dspark
