// Logits-only cross-entropy, forward and backward in one pass over each row,
// with the gradient written over the logits.
//
// Method: the CrossEntropy kernel of "[論文レビュー] Liger Kernel: Efficient
// Triton Kernels for LLM Training" (主な発見): an online softmax (running max
// and rescaled sum of exponentials in a single sweep of the row) and in-place
// replacement of the logits by their gradient.  One 1024-thread workgroup per token row:
//   sweep 1  m, s over the row (online), target logit z_y  ->  lse = m + ln s
//   sweep 2  logits[v] <- (e^(z_v - lse) - [v = y]) / N   (0 on ignored rows)
// The row is fp32 and may be any length; 16-byte vector accesses are used on
// the row's 16-byte-aligned middle part.
#include <float.h>

#include "flce_internal.h"

namespace flce {

namespace {

constexpr float kLog2e = 1.4426950408889634f;
// 1024 threads per row and 16 vector loads in flight per thread: a row's two
// sweeps then follow each other closely enough that the second mostly hits
// the MALL (measured on the 8192 x 256000 fp32 logits: 4.9 -> 4.3 ms)
constexpr int kCeThreads = 1024;
constexpr int kUnroll = 16;
// The first unrolled iteration of a row (16 x 1024 vectors, 256 KiB) stays on
// chip between the sweeps: 9 x 1024 vectors (144 KiB) in LDS, the other 7 in
// registers.
constexpr int kCacheBlocks = 9;
constexpr int kCacheVec = kCacheBlocks * kCeThreads;

typedef float f32x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ float ex2(float x) { return __builtin_amdgcn_exp2f(x); }

struct Online {
  float m, s;
  __device__ __forceinline__ void add4(f32x4 x) {
    const float mx = fmaxf(fmaxf(x[0], x[1]), fmaxf(x[2], x[3]));
    if (mx > m) {
      s *= ex2((m - mx) * kLog2e);
      m = mx;
    }
    const float mb = m * kLog2e;
    s += ex2(fmaf(x[0], kLog2e, -mb)) + ex2(fmaf(x[1], kLog2e, -mb)) + ex2(fmaf(x[2], kLog2e, -mb)) +
         ex2(fmaf(x[3], kLog2e, -mb));
  }
  __device__ __forceinline__ void add1(float x) {
    if (x > m) {
      s *= ex2((m - x) * kLog2e);
      m = x;
    }
    s += ex2(fmaf(x, kLog2e, -m * kLog2e));
  }
  __device__ __forceinline__ void merge(float m2, float s2) {
    const float M = fmaxf(m, m2);
    s = s * ex2((m - M) * kLog2e) + s2 * ex2((m2 - M) * kLog2e);
    m = M;
  }
};

}  // namespace

__global__ __launch_bounds__(kCeThreads) void k_ce_rows(float* __restrict__ logits, const int64_t* __restrict__ y,
                                                        int64_t V, int64_t ign, const int32_t* __restrict__ nvalid,
                                                        float* __restrict__ rowloss) {
  __shared__ float red_m[kCeThreads / 64], red_s[kCeThreads / 64];
  __shared__ f32x4 cache[kCacheVec];  // first vectors of the row, kept for sweep 2
  __shared__ float lse_sh;
  const int64_t r = blockIdx.x;
  const int tid = threadIdx.x;
  float* row = logits + r * V;
  const int64_t t = y[r];

  // split the row into a scalar head (up to 16-byte alignment), a vector body and a scalar tail
  const int64_t mis = (int64_t)(((uintptr_t)row >> 2) & 3);
  int64_t head = mis ? 4 - mis : 0;
  if (head > V) head = V;
  const int64_t nvec = (V - head) / 4;
  const int64_t tail0 = head + 4 * nvec;
  f32x4* body = reinterpret_cast<f32x4*>(row + head);

  if (t == ign) {
    for (int64_t i = tid; i < head; i += kCeThreads) row[i] = 0.f;
    for (int64_t i = tid; i < nvec; i += kCeThreads) body[i] = f32x4{0.f, 0.f, 0.f, 0.f};
    for (int64_t i = tail0 + tid; i < V; i += kCeThreads) row[i] = 0.f;
    if (tid == 0) rowloss[r] = 0.f;
    return;
  }

  // sweep 1 (the first kCacheVec vectors of the body also go to LDS for sweep 2)
  Online o{-FLT_MAX, 0.f};
  f32x4 kept[kUnroll - kCacheBlocks];  // the rest of the first iteration, in registers
  for (int64_t i = tid; i < head; i += kCeThreads) o.add1(row[i]);
  int64_t i = tid;
  for (; i + (kUnroll - 1) * kCeThreads < nvec; i += kUnroll * kCeThreads) {
    f32x4 x[kUnroll];
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) x[u] = body[i + u * kCeThreads];
    if (i < kCacheVec) {
#pragma unroll
      for (int u = 0; u < kCacheBlocks; ++u) cache[i + u * kCeThreads] = x[u];
#pragma unroll
      for (int u = kCacheBlocks; u < kUnroll; ++u) kept[u - kCacheBlocks] = x[u];
    }
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) o.add4(x[u]);
  }
  for (; i < nvec; i += kCeThreads) o.add4(body[i]);
  for (int64_t k = tail0 + tid; k < V; k += kCeThreads) o.add1(row[k]);

#pragma unroll
  for (int off = 32; off > 0; off >>= 1) {
    const float m2 = __shfl_xor(o.m, off), s2 = __shfl_xor(o.s, off);
    o.merge(m2, s2);
  }
  if ((tid & 63) == 0) {
    red_m[tid >> 6] = o.m;
    red_s[tid >> 6] = o.s;
  }
  __syncthreads();
  if (tid == 0) {
    Online a{red_m[0], red_s[0]};
    for (int w = 1; w < kCeThreads / 64; ++w) a.merge(red_m[w], red_s[w]);
    const float lse = a.m + logf(a.s);
    const float zt = (t >= 0 && t < V) ? row[t] : 0.f;
    rowloss[r] = lse - zt;
    lse_sh = lse;
  }
  __syncthreads();

  // sweep 2
  const int n = *nvalid;
  const float inv = 1.f / (float)(n > 0 ? n : 1);
  const float lb = lse_sh * kLog2e;
  auto g1 = [&](float z, int64_t v) { return (ex2(fmaf(z, kLog2e, -lb)) - (v == t ? 1.f : 0.f)) * inv; };
  for (int64_t k = tid; k < head; k += kCeThreads) row[k] = g1(row[k], k);
  i = tid;
  for (; i + (kUnroll - 1) * kCeThreads < nvec; i += kUnroll * kCeThreads) {
    f32x4 x[kUnroll];
    if (i < kCacheVec) {
#pragma unroll
      for (int u = 0; u < kUnroll; ++u) x[u] = u < kCacheBlocks ? cache[i + u * kCeThreads] : kept[u - kCacheBlocks];
    } else {
#pragma unroll
      for (int u = 0; u < kUnroll; ++u) x[u] = body[i + u * kCeThreads];
    }
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
      const int64_t v = head + 4 * (i + u * kCeThreads);
      // gradients are not read again here: stream them past the caches
      __builtin_nontemporal_store(f32x4{g1(x[u][0], v), g1(x[u][1], v + 1), g1(x[u][2], v + 2), g1(x[u][3], v + 3)},
                                  &body[i + u * kCeThreads]);
    }
  }
  for (; i < nvec; i += kCeThreads) {
    const f32x4 x = body[i];
    const int64_t v = head + 4 * i;
    body[i] = f32x4{g1(x[0], v), g1(x[1], v + 1), g1(x[2], v + 2), g1(x[3], v + 3)};
  }
  for (int64_t k = tail0 + tid; k < V; k += kCeThreads) row[k] = g1(row[k], k);
}

hipError_t launch_ce_rows(float* logits, const int64_t* y, int64_t BT, int64_t V, int64_t ign, const int32_t* nvalid,
                          float* rowloss, hipStream_t s) {
  if (BT <= 0) return hipSuccess;
  ProfScope ps(kPhaseCeRows, s);
  hipLaunchKernelGGL(k_ce_rows, dim3((unsigned)BT), dim3(kCeThreads), 0, s, logits, y, V, ign, nvalid, rowloss);
  return hipGetLastError();
}

}  // namespace flce
