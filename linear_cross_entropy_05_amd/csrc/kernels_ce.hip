// Logits-only cross-entropy, forward and backward in one pass over each row,
// with the gradient written over the logits.
//
// Method: the CrossEntropy kernel of "[論文レビュー] Liger Kernel: Efficient
// Triton Kernels for LLM Training" (主な発見): an online softmax (running max
// and rescaled sum of exponentials in a single sweep of the row) and in-place
// replacement of the logits by their gradient.  One 512-thread workgroup per token row:
//   sweep 1  m, s over the row (online), target logit z_y  ->  lse = m + ln s
//   sweep 2  logits[v] <- (e^(z_v - lse) - [v = y]) / N   (0 on ignored rows)
// The row is fp32 and may be any length; 16-byte vector accesses are used on
// the row's 16-byte-aligned middle part.
#include <float.h>

#include "flce_internal.h"
#include "gemm_core.h"

namespace flce {

namespace {

constexpr float kLog2e = 1.4426950408889634f;
// One 512-thread workgroup per row, one row per CU at a time.  Sweep 2 needs
// the whole row again, so as much of it as fits stays on chip between the
// sweeps: per thread kRegVec 16-byte vectors in registers (two waves per SIMD
// leave 256 registers each) and kLdsVec in LDS (copied there straight from
// memory, no registers), 62 x 8 KiB = 496 KiB of a row; only the rest is read
// a second time.  Measured on 8192 x 256000 fp32 logits: 256 KiB kept 3.98 ms,
// 400 KiB (1024 threads) 3.67 ms, 496 KiB 3.61 ms.
constexpr int kCeThreads = 512;
constexpr int kRegVec = 44;
constexpr int kLdsVec = 18;  // 144 KiB of LDS
constexpr int kKeepVec = kRegVec + kLdsVec;
constexpr int kStream = 4;  // loads in flight per thread over the rest of the row

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

// Element indices within a row are 32-bit: the launcher rejects V >= 2^31.
__global__ __launch_bounds__(kCeThreads) void k_ce_rows(float* __restrict__ logits, const int64_t* __restrict__ y,
                                                        int64_t V64, int64_t ign, const int32_t* __restrict__ nvalid,
                                                        float* __restrict__ rowloss) {
  __shared__ float red_m[kCeThreads / 64], red_s[kCeThreads / 64];
  __shared__ f32x4 cache[kLdsVec * kCeThreads];  // slot u of thread i: vector i + (kRegVec + u) T of the body
  __shared__ float lse_sh;
  const int64_t r = blockIdx.x;
  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int V = (int)V64;
  float* row = logits + r * V64;
  const int64_t t64 = y[r];

  // split the row into a scalar head (up to 16-byte alignment), a vector body and a scalar tail
  const int mis = (int)(((uintptr_t)row >> 2) & 3);
  int head = mis ? 4 - mis : 0;
  if (head > V) head = V;
  const int nvec = (V - head) / 4;
  const int tail0 = head + 4 * nvec;
  f32x4* body = reinterpret_cast<f32x4*>(row + head);

  if (t64 == ign) {
    for (int i = tid; i < head; i += kCeThreads) row[i] = 0.f;
    for (int i = tid; i < nvec; i += kCeThreads) body[i] = f32x4{0.f, 0.f, 0.f, 0.f};
    for (int i = tail0 + tid; i < V; i += kCeThreads) row[i] = 0.f;
    if (tid == 0) rowloss[r] = 0.f;
    return;
  }
  // the target as a body-relative element index (out-of-range targets were
  // flagged by the count pass and match no element)
  const int t = (t64 >= 0 && t64 < V64) ? (int)t64 : -1;

  // sweep 1.  The LDS part is copied first (vectors past the body read as
  // zero and are never used), then the register part is loaded, then the
  // rest of the row streams through.  The parts kept on chip are read once,
  // with non-temporal loads; the rest is read again in sweep 2 and is left to
  // the caches (the re-read then hits the 256 MB last-level cache often
  // enough: non-temporal loads there made the call 11% slower, on the kept
  // parts and the re-read 6% faster).
  {
    const u32x4 rs = pipe::rsrc_words(body, (int64_t)nvec * 16);
    const uint32_t base = pipe::lds_addr(reinterpret_cast<const char*>(cache)) + 1024u * (uint32_t)wave;
#pragma unroll
    for (int u = 0; u < kLdsVec; ++u)
      pipe::dma16(rs, base + (uint32_t)(u * kCeThreads * 16), (uint32_t)((tid + (kRegVec + u) * kCeThreads) * 16), 0);
  }
  Online o{-FLT_MAX, 0.f};
  f32x4 kept[kRegVec];
#pragma unroll
  for (int u = 0; u < kRegVec; ++u) {
    const int v = tid + u * kCeThreads;
    kept[u] = v < nvec ? __builtin_nontemporal_load(&body[v]) : f32x4{0.f, 0.f, 0.f, 0.f};
  }
  for (int i = tid; i < head; i += kCeThreads) o.add1(row[i]);
#pragma unroll
  for (int u = 0; u < kRegVec; ++u)
    if (tid + u * kCeThreads < nvec) o.add4(kept[u]);
  int i = tid + kKeepVec * kCeThreads;
  for (; i + (kStream - 1) * kCeThreads < nvec; i += kStream * kCeThreads) {
    f32x4 x[kStream];
#pragma unroll
    for (int u = 0; u < kStream; ++u) x[u] = body[i + u * kCeThreads];
#pragma unroll
    for (int u = 0; u < kStream; ++u) o.add4(x[u]);
  }
  for (; i < nvec; i += kCeThreads) o.add4(body[i]);
  for (int k = tail0 + tid; k < V; k += kCeThreads) o.add1(row[k]);
  pipe::wait_vm<0>();  // this thread's LDS slots have landed
#pragma unroll
  for (int u = 0; u < kLdsVec; ++u)
    if (tid + (kRegVec + u) * kCeThreads < nvec) o.add4(cache[u * kCeThreads + tid]);

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
    const float zt = t >= 0 ? row[t] : 0.f;
    rowloss[r] = lse - zt;
    lse_sh = lse;
  }
  __syncthreads();

  // sweep 2: gradients over the logits; they are not read again here, so
  // they stream past the caches
  const int n = *nvalid;
  const float inv = 1.f / (float)(n > 0 ? n : 1);
  const float lb = lse_sh * kLog2e;
  auto g1 = [&](float z, int v) { return (ex2(fmaf(z, kLog2e, -lb)) - (v == t ? 1.f : 0.f)) * inv; };
  auto g4 = [&](f32x4 x, int vi) {
    const int v = head + 4 * vi;
    return f32x4{g1(x[0], v), g1(x[1], v + 1), g1(x[2], v + 2), g1(x[3], v + 3)};
  };
  for (int k = tid; k < head; k += kCeThreads) row[k] = g1(row[k], k);
#pragma unroll
  for (int u = 0; u < kRegVec; ++u) {
    const int v = tid + u * kCeThreads;
    if (v < nvec) __builtin_nontemporal_store(g4(kept[u], v), &body[v]);
  }
#pragma unroll
  for (int u = 0; u < kLdsVec; ++u) {
    const int v = tid + (kRegVec + u) * kCeThreads;
    if (v < nvec) __builtin_nontemporal_store(g4(cache[u * kCeThreads + tid], v), &body[v]);
  }
  i = tid + kKeepVec * kCeThreads;
  for (; i + (kStream - 1) * kCeThreads < nvec; i += kStream * kCeThreads) {
    f32x4 x[kStream];
#pragma unroll
    for (int u = 0; u < kStream; ++u) x[u] = __builtin_nontemporal_load(&body[i + u * kCeThreads]);
#pragma unroll
    for (int u = 0; u < kStream; ++u)
      __builtin_nontemporal_store(g4(x[u], i + u * kCeThreads), &body[i + u * kCeThreads]);
  }
  for (; i < nvec; i += kCeThreads) body[i] = g4(body[i], i);
  for (int k = tail0 + tid; k < V; k += kCeThreads) row[k] = g1(row[k], k);
}

hipError_t launch_ce_rows(float* logits, const int64_t* y, int64_t BT, int64_t V, int64_t ign, const int32_t* nvalid,
                          float* rowloss, hipStream_t s) {
  if (BT <= 0) return hipSuccess;
  ProfScope ps(kPhaseCeRows, s);
  hipLaunchKernelGGL(k_ce_rows, dim3((unsigned)BT), dim3(kCeThreads), 0, s, logits, y, V, ign, nvalid, rowloss);
  return hipGetLastError();
}

}  // namespace flce
