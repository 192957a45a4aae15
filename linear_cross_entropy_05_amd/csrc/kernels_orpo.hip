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

// Odds-ratio term of one pair from the sums of its sequences' valid token
// losses and their counts: returns softplus(-r) (0 if a sequence has no valid
// token) and sets the gradient coefficients d(beta/B softplus(-r))/d l_i of
// the chosen (cw) and rejected (cl) sequence's tokens (left as they are when
// the term is 0).
__device__ double pair_terms(double sum_w, double n_w, double sum_l, double n_l, float beta, int64_t B, double& cw,
                             double& cl) {
  if (!(n_w > 0.0 && n_l > 0.0)) return 0.0;
  const double aw = fmin(-sum_w / n_w, kMaxSeqLogp), al = fmin(-sum_l / n_l, kMaxSeqLogp);
  const double ow = -expm1(aw), ol = -expm1(al);  // 1 - e^a
  const double r = (aw - al) - (log(ow) - log(ol));
  const double g = -sigmoid(-r) * (double)beta / (double)B;  // d (beta/B softplus(-r)) / dr
  // dr/da_w = 1 / (1 - e^{a_w}), dr/da_l = -1 / (1 - e^{a_l}), da_s/dl_i = -1/n_s
  cw = g * (1.0 / ow) * (-1.0 / n_w);
  cl = g * (-1.0 / ol) * (-1.0 / n_l);
  return softplus(-r);
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
    orsum += pair_terms(ssum[sw], scnt[sw], ssum[sl], scnt[sl], beta, B, coef[sw], coef[sl]);
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

// ---- one pass: chunks that hold whole (chosen, rejected) pairs --------------
//
// A chunk holds pairs p0 .. p0 + np - 1: rows [0, np T) are their chosen
// sequences p0 .. (tokens p0 T ..), rows [np T, 2 np T) their rejected ones
// B + p0 .. (tokens (B + p0) T ..).  Local sequence s of the chunk is global
// sequence p0 + s (s < np) or B + p0 + s - np.

__device__ __forceinline__ int64_t orpo_src_row(int64_t r, int64_t half, int64_t T, int64_t B, int64_t p0) {
  return r < half ? p0 * T + r : (B + p0) * T + (r - half);
}

// Gathers the chunk's hidden states and targets into contiguous rows.
template <typename T>
__global__ __launch_bounds__(256) void k_orpo_gather(const T* __restrict__ X, const int64_t* __restrict__ y, int64_t H,
                                                     int64_t Tl, int64_t B, int64_t p0, int64_t np,
                                                     T* __restrict__ Xg, int64_t* __restrict__ yg) {
  constexpr int E = 16 / sizeof(T);
  const int64_t r = blockIdx.x;
  const int64_t src = orpo_src_row(r, np * Tl, Tl, B, p0);
  if (threadIdx.x == 0) yg[r] = y[src];
  const uint4* in = reinterpret_cast<const uint4*>(X + src * H);
  uint4* out = reinterpret_cast<uint4*>(Xg + r * H);
  for (int64_t i = threadIdx.x; i < H / E; i += 256) out[i] = in[i];
}

// Writes the chunk's dX rows back to their sequences' rows.
template <typename T>
__global__ __launch_bounds__(256) void k_orpo_scatter(const T* __restrict__ dXc, int64_t H, int64_t Tl, int64_t B,
                                                      int64_t p0, int64_t np, T* __restrict__ dX) {
  constexpr int E = 16 / sizeof(T);
  const int64_t r = blockIdx.x;
  const int64_t dst = orpo_src_row(r, np * Tl, Tl, B, p0);
  const uint4* in = reinterpret_cast<const uint4*>(dXc + r * H);
  uint4* out = reinterpret_cast<uint4*>(dX + dst * H);
  for (int64_t i = threadIdx.x; i < H / E; i += 256) out[i] = in[i];
}

// The chunk's sequence and pair terms (fp64, fixed order) and its tokens'
// gradient factors.  seq: [3 n_seq] doubles (loss sums, valid counts,
// coefficients) and pair: [B] doubles (softplus(-r)), indexed globally.
__global__ __launch_bounds__(kOrpoThreads) void k_orpo_chunk_stats(
    const float* __restrict__ rlc, const int64_t* __restrict__ yg, int64_t Tl, int64_t B, int64_t n_seq, int64_t p0,
    int64_t np, int64_t ign, float beta, const int32_t* __restrict__ nchosen, float* __restrict__ wc,
    float* __restrict__ seq_logp, double* __restrict__ seq, double* __restrict__ pair) {
  double* ssum = seq;
  double* scnt = seq + n_seq;
  double* coef = seq + 2 * n_seq;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  auto gseq = [&](int64_t s) { return s < np ? p0 + s : B + p0 + (s - np); };
  // per-sequence sums of the valid token losses and valid counts, one wave
  // per sequence (the same order as the two-pass statistics)
  for (int64_t s = wave; s < 2 * np; s += kOrpoWaves) {
    double sum = 0.0, cnt = 0.0;
    for (int64_t t = lane; t < Tl; t += 64) {
      const int64_t i = s * Tl + t;
      if (yg[i] != ign) {
        sum += (double)rlc[i];
        cnt += 1.0;
      }
    }
    sum = wave_sum(sum);
    cnt = wave_sum(cnt);
    if (lane == 0) {
      const int64_t g = gseq(s);
      ssum[g] = sum;
      scnt[g] = cnt;
      coef[g] = 0.0;
      if (seq_logp) seq_logp[g] = (float)(cnt > 0.0 ? -sum / cnt : 0.0);
    }
  }
  __syncthreads();
  for (int64_t p = threadIdx.x; p < np; p += kOrpoThreads) {
    const int64_t sw = p0 + p, sl = B + p0 + p;
    pair[sw] = pair_terms(ssum[sw], scnt[sw], ssum[sl], scnt[sl], beta, B, coef[sw], coef[sl]);
  }
  __syncthreads();
  const int nc = *nchosen;
  const double inv_nc = 1.0 / (double)(nc > 0 ? nc : 1);
  for (int64_t i = threadIdx.x; i < 2 * np * Tl; i += kOrpoThreads) {
    const int64_t s = i / Tl;
    float w = 0.f;
    if (yg[i] != ign) w = (float)((s < np ? inv_nc : 0.0) + coef[gseq(s)]);
    wc[i] = w;
  }
}

// loss = (sum of the chosen sequences' token losses) / N_chosen
//        + beta / B * sum_p softplus(-r_p), in a fixed order
__global__ __launch_bounds__(kOrpoThreads) void k_orpo_final(const double* __restrict__ seq,
                                                             const double* __restrict__ pair, int64_t B,
                                                             float beta, const int32_t* __restrict__ nchosen,
                                                             float* __restrict__ loss) {
  __shared__ double red[kOrpoWaves];
  double nll = 0.0, orsum = 0.0;
  for (int64_t p = threadIdx.x; p < B; p += kOrpoThreads) {
    nll += seq[p];
    orsum += pair[p];
  }
  nll = block_sum(nll, red);
  orsum = block_sum(orsum, red);
  if (threadIdx.x == 0) {
    const int nc = *nchosen;
    *loss = (float)(nll / (double)(nc > 0 ? nc : 1) + (double)beta * orsum / (double)(B > 0 ? B : 1));
  }
}

hipError_t launch_orpo_gather(const void* X, const int64_t* y, int64_t H, int64_t Tl, int64_t B, int64_t p0,
                              int64_t np, int dtype, void* Xg, int64_t* yg, hipStream_t s) {
  ProfScope ps(kPhaseOrpo, s);
  const unsigned rows = (unsigned)(2 * np * Tl);
  if (dtype == 1)
    hipLaunchKernelGGL(k_orpo_gather<__bf16>, dim3(rows), dim3(256), 0, s, static_cast<const __bf16*>(X), y, H, Tl,
                       B, p0, np, static_cast<__bf16*>(Xg), yg);
  else
    hipLaunchKernelGGL(k_orpo_gather<float>, dim3(rows), dim3(256), 0, s, static_cast<const float*>(X), y, H, Tl, B,
                       p0, np, static_cast<float*>(Xg), yg);
  return hipGetLastError();
}

hipError_t launch_orpo_scatter(const void* dXc, int64_t H, int64_t Tl, int64_t B, int64_t p0, int64_t np, int dtype,
                               void* dX, hipStream_t s) {
  ProfScope ps(kPhaseOrpo, s);
  const unsigned rows = (unsigned)(2 * np * Tl);
  if (dtype == 1)
    hipLaunchKernelGGL(k_orpo_scatter<__bf16>, dim3(rows), dim3(256), 0, s, static_cast<const __bf16*>(dXc), H, Tl, B,
                       p0, np, static_cast<__bf16*>(dX));
  else
    hipLaunchKernelGGL(k_orpo_scatter<float>, dim3(rows), dim3(256), 0, s, static_cast<const float*>(dXc), H, Tl, B,
                       p0, np, static_cast<float*>(dX));
  return hipGetLastError();
}

hipError_t launch_orpo_chunk_stats(const float* rlc, const int64_t* yg, int64_t Tl, int64_t B, int64_t p0, int64_t np,
                                   int64_t ign, float beta, const int32_t* nchosen, float* wc, float* seq_logp,
                                   double* seq, double* pair, hipStream_t s) {
  ProfScope ps(kPhaseOrpo, s);
  hipLaunchKernelGGL(k_orpo_chunk_stats, dim3(1), dim3(kOrpoThreads), 0, s, rlc, yg, Tl, B, 2 * B, p0, np, ign, beta,
                     nchosen, wc, seq_logp, seq, pair);
  return hipGetLastError();
}

hipError_t launch_orpo_final(const double* seq, const double* pair, int64_t B, float beta, const int32_t* nchosen,
                             float* loss, hipStream_t s) {
  ProfScope ps(kPhaseOrpo, s);
  hipLaunchKernelGGL(k_orpo_final, dim3(1), dim3(kOrpoThreads), 0, s, seq, pair, B, beta, nchosen, loss);
  return hipGetLastError();
}

hipError_t launch_orpo_stats(const float* rowloss, const int64_t* y, int64_t n_seq, int64_t T, int64_t ign, float beta,
                             float* scale, float* seq_logp, float* loss, double* scratch, hipStream_t s) {
  ProfScope ps(kPhaseOrpo, s);
  hipLaunchKernelGGL(k_orpo_stats, dim3(1), dim3(kOrpoThreads), 0, s, rowloss, y, n_seq, T, ign, beta, scale,
                     seq_logp, loss, scratch);
  return hipGetLastError();
}

}  // namespace flce
