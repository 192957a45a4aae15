// Sequence-level step of the fused-linear ORPO loss (odds-ratio preference
// loss; "Liger-Kernel 項目詳細介紹", 主要功能 / 使用方法 item 4 name it and show
// the call orpo_loss(lm_head.weight, x, target); the objective is the
// published ORPO one).  From the token losses l_i of 2B sequences of T tokens
// (chosen 0..B-1, rejected B..2B-1) it forms, in fp64 and in a fixed order:
//   a_s = -(1/n_s) sum_{i in s, valid} l_i              (mean log-probability)
//   r_p = (a_w - a_l) - (log(1 - e^{a_w}) - log(1 - e^{a_l}))
//   loss = (sum of chosen token losses) / N_chosen + beta / B * sum_p softplus(-r_p)
// and the per-token gradient factors w_i = d loss / d l_i that the fused
// linear + cross-entropy pass then applies to (softmax - onehot).  A pair with
// a sequence that has no valid token adds nothing to the odds-ratio term; in
// that term each a_s is held at or below -2^-24 (see kMaxSeqLogp).
#include "flce_internal.h"

namespace flce {

namespace {

constexpr int kOrpoThreads = 1024;
constexpr int kOrpoWaves = kOrpoThreads / 64;

__device__ __forceinline__ double wave_sum(double v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o);
  return v;
}

// fixed-order block sum (wave sums, then wave 0 adds the 16 partials)
__device__ double block_sum(double v, double* red) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  v = wave_sum(v);
  __syncthreads();
  if (lane == 0) red[wave] = v;
  __syncthreads();
  double t = 0.0;
  for (int k = 0; k < kOrpoWaves; ++k) t += red[k];
  return t;
}

// The mean log-probability a of a sequence is negative in exact arithmetic,
// but the fp32 token losses of a near-certain sequence can round to 0 or just
// below it, which would make log(1 - e^a) infinite or NaN.  The odds-ratio
// term takes a at most -2^-24: its loss and gradient factors tend to finite
// limits as a -> 0 (softplus(-r) -> 0, sigmoid(-r) / (1 - e^{a_w}) stays
// bounded), so the bound changes them only below the fp32 resolution.
constexpr double kMaxSeqLogp = -0x1p-24;

__device__ __forceinline__ double softplus(double x) { return fmax(x, 0.0) + log1p(exp(-fabs(x))); }
__device__ __forceinline__ double sigmoid(double x) {
  return x >= 0.0 ? 1.0 / (1.0 + exp(-x)) : exp(x) / (1.0 + exp(x));
}

}  // namespace

// scratch: 3 * n_seq doubles (per-sequence loss sums, valid counts, gradient coefficients)
__global__ __launch_bounds__(kOrpoThreads) void k_orpo_stats(const float* __restrict__ rowloss,
                                                             const int64_t* __restrict__ y, int64_t n_seq, int64_t T,
                                                             int64_t ign, float beta, float* __restrict__ scale,
                                                             float* __restrict__ seq_logp, float* __restrict__ loss,
                                                             double* __restrict__ scratch) {
  __shared__ double red[kOrpoWaves];
  double* ssum = scratch;
  double* scnt = scratch + n_seq;
  double* coef = scratch + 2 * n_seq;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int64_t B = n_seq / 2;

  // per-sequence sums of the valid token losses and valid counts, one wave per sequence
  for (int64_t s = wave; s < n_seq; s += kOrpoWaves) {
    double sum = 0.0, cnt = 0.0;
    for (int64_t t = lane; t < T; t += 64) {
      const int64_t i = s * T + t;
      if (y[i] != ign) {
        sum += (double)rowloss[i];
        cnt += 1.0;
      }
    }
    sum = wave_sum(sum);
    cnt = wave_sum(cnt);
    if (lane == 0) {
      ssum[s] = sum;
      scnt[s] = cnt;
    }
  }
  __syncthreads();

  // chosen-token NLL and the pairs' odds-ratio terms
  double nll = 0.0, nchosen = 0.0, orsum = 0.0;
  for (int64_t s = threadIdx.x; s < n_seq; s += kOrpoThreads) {
    const double a = scnt[s] > 0.0 ? -ssum[s] / scnt[s] : 0.0;
    if (seq_logp) seq_logp[s] = (float)a;
    coef[s] = 0.0;
    if (s < B) {
      nll += ssum[s];
      nchosen += scnt[s];
    }
  }
  __syncthreads();
  for (int64_t p = threadIdx.x; p < B; p += kOrpoThreads) {
    const int64_t sw = p, sl = B + p;
    const double nw = scnt[sw], nl = scnt[sl];
    if (nw > 0.0 && nl > 0.0) {
      const double aw = fmin(-ssum[sw] / nw, kMaxSeqLogp), al = fmin(-ssum[sl] / nl, kMaxSeqLogp);
      const double ow = -expm1(aw), ol = -expm1(al);  // 1 - e^a
      const double r = (aw - al) - (log(ow) - log(ol));
      orsum += softplus(-r);
      const double g = -sigmoid(-r) * (double)beta / (double)B;  // d (beta/B softplus(-r)) / dr
      // dr/da_w = 1 / (1 - e^{a_w}), dr/da_l = -1 / (1 - e^{a_l}), da_s/dl_i = -1/n_s
      coef[sw] = g * (1.0 / ow) * (-1.0 / nw);
      coef[sl] = g * (-1.0 / ol) * (-1.0 / nl);
    }
  }
  nll = block_sum(nll, red);
  nchosen = block_sum(nchosen, red);
  orsum = block_sum(orsum, red);
  __syncthreads();
  const double inv_nc = 1.0 / (nchosen > 0.0 ? nchosen : 1.0);
  if (threadIdx.x == 0) *loss = (float)(nll * inv_nc + (double)beta * orsum / (double)(B > 0 ? B : 1));

  // per-token gradient factors
  const int64_t n = n_seq * T;
  for (int64_t i = threadIdx.x; i < n; i += kOrpoThreads) {
    const int64_t s = i / T;
    float w = 0.f;
    if (y[i] != ign) w = (float)((s < B ? inv_nc : 0.0) + coef[s]);
    scale[i] = w;
  }
}

hipError_t launch_orpo_stats(const float* rowloss, const int64_t* y, int64_t n_seq, int64_t T, int64_t ign, float beta,
                             float* scale, float* seq_logp, float* loss, double* scratch, hipStream_t s) {
  ProfScope ps(kPhaseOrpo, s);
  hipLaunchKernelGGL(k_orpo_stats, dim3(1), dim3(kOrpoThreads), 0, s, rowloss, y, n_seq, T, ign, beta, scale,
                     seq_logp, loss, scratch);
  return hipGetLastError();
}

}  // namespace flce
