// Kernels of chunked fused linear + cross-entropy (FLCE), forward and
// backward, for gfx950.
//
// Method ("[論文レビュー] Liger Kernel: Efficient Triton Kernels for LLM
// Training", 提案手法 and 主な発見; "Liger-Kernel 項目詳細介紹", 技術實現): the
// tokens are processed in chunks so the full tokens x vocabulary logits never
// exist; within a chunk the softmax statistics are gathered online and the
// logits buffer is overwritten by d(loss)/d(logits); the computation is exact.
// Per chunk of `rows` tokens (c indexes the chunk's tokens, v the vocabulary,
// h the hidden units):
//   logits   Z[c,v] = x_c . w_v; per (token, 128-wide vocabulary half tile h)
//            the max M_h and sum of exp(z - M_h), taken from the fp32
//            accumulators in the GEMM epilogue; the chunk buffer receives
//            z - M_h in the element type
//   lse      lse_c = M + ln sum_h s_h e^(M_h - M) over the half tiles,
//            M = max M_h; target logit x_c . w_y (fp32 dot product);
//            per-token loss lse_c - z_{c,y_c} (0 for ignored tokens)
//   grad     G[c,v] = (e^(Z[c,v] - lse_c) - [v = y_c]) / N written over the
//            stored z - M_h
//            (0 on ignored tokens), N = number of non-ignored tokens
//   dX       dX[c,:] = G[c,:] W
//   dW       dW (+)= G^T X_chunk, fp32, stored on the first chunk
//            (dX and dW share one launch)
// and once per call: count N and check targets; loss = sum of token losses / N.
// In flce_fwd_bwd the chunks hold only the non-ignored tokens (gathered, in
// their order), so the last chunks may hold fewer rows than launched for:
// the row count comes from N in device memory (RowCount).
#include <float.h>

#include "flce_internal.h"
#include "gemm_core.h"

namespace flce {

constexpr float kLog2e = 1.4426950408889634f;
// gradient pass: threads per token row and 16-byte loads in flight per
// thread (1024 x 4 measured ~8% faster than 256 x 4 on 250 KiB rows; 2 and 4
// loads in flight tie, 8 is slower)
constexpr int kGradThreads = 1024;
constexpr int kGradUnroll = 4;

__device__ __forceinline__ float exp2_fast(float x) { return __builtin_amdgcn_exp2f(x); }

__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o));
  return v;
}
__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o);
  return v;
}

// ---- count valid targets, range check (once per call) ----------------------

// N = number of targets that are not ignore_index, and error 6 if one of them
// lies outside [0, V).  With `idx` (token compaction) also the positions:
// the non-ignored tokens' in order at idx[0 .. N), the ignored tokens' from
// the end backwards (the j-th ignored position at idx[BT - 1 - j]).  One
// workgroup, 4096 targets per pass, four consecutive ones per thread, ranks
// from a scan over the threads in order.
__global__ __launch_bounds__(1024) void k_count_valid(const int64_t* __restrict__ y, int64_t BT, int64_t V,
                                                      int64_t ign, int32_t* nvalid, int32_t* err,
                                                      int32_t* __restrict__ idx) {
  __shared__ int wtot[16], red_b[16];
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  int bad = 0;
  int64_t done = 0;  // non-ignored targets before this pass
  for (int64_t base = 0; base < BT; base += 4096) {
    const int64_t i0 = base + 4 * (int64_t)threadIdx.x;
    bool f[4];
    int cnt = 0;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      f[q] = false;
      if (i0 + q < BT) {
        const int64_t t = y[i0 + q];
        if (t != ign) {
          f[q] = true;
          bad |= (t < 0 || t >= V);
        }
      }
      cnt += f[q];
    }
    // inclusive scan of cnt over the lanes, then over the waves
    int incl = cnt;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
      const int u = __shfl_up(incl, o);
      if (lane >= o) incl += u;
    }
    if (lane == 63) wtot[w] = incl;
    __syncthreads();
    int before = 0, total = 0;
#pragma unroll
    for (int k = 0; k < 16; ++k) {
      const int u = wtot[k];
      before += k < w ? u : 0;
      total += u;
    }
    __syncthreads();  // wtot is written again by the next pass
    if (idx) {
      int64_t r = done + before + incl - cnt;  // non-ignored targets before i0
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int64_t i = i0 + q;
        if (i < BT) {
          if (f[q])
            idx[r++] = (int32_t)i;
          else
            idx[BT - 1 - (i - r)] = (int32_t)i;  // i - r ignored targets before i
        }
      }
    }
    done += total;
  }
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) bad |= __shfl_xor(bad, o);
  if (lane == 0) red_b[w] = bad;
  __syncthreads();
  if (threadIdx.x == 0) {
    int tb = 0;
    for (int i = 0; i < 16; ++i) tb |= red_b[i];
    *nvalid = (int32_t)done;
    *err = tb ? 6 : 0;
  }
}

// Rows of a chunk.  With token compaction a chunk holds the non-ignored
// tokens c0 .. c0 + max - 1 of the N in device memory, so fewer rows (or
// none) may be in use; otherwise all `max` are.
struct RowCount {
  const int32_t* n;  // N, or nullptr: all max rows
  int64_t c0, max;
  __device__ __forceinline__ int64_t get() const {
    if (!n) return max;
    const int64_t r = (int64_t)__builtin_amdgcn_readfirstlane(*n) - c0;
    return r < 0 ? 0 : (r > max ? max : r);
  }
};

// Token compaction, once per call: zero the dX rows and token losses of the
// ignored tokens (idx[N .. BT)), which no chunk visits.
template <typename T>
__global__ __launch_bounds__(256) void k_zero_ignored(const int32_t* __restrict__ idx, const int32_t* __restrict__ nvalid,
                                                      int64_t BT, int64_t H, T* __restrict__ dX,
                                                      float* __restrict__ rowloss) {
  constexpr int E = Elem<T>::chunk;
  const int64_t n = __builtin_amdgcn_readfirstlane(*nvalid);
  for (int64_t r = n + blockIdx.x; r < BT; r += gridDim.x) {
    const int64_t p = idx[r];
    T* row = dX + p * H;
    for (int64_t h = (int64_t)threadIdx.x * E; h < H; h += 256 * E)
      *reinterpret_cast<u32x4*>(row + h) = u32x4{0, 0, 0, 0};
    if (threadIdx.x == 0) rowloss[p] = 0.f;
  }
}

// Token compaction, per chunk: row r of the chunk is token idx[c0 + r]; copy
// its X row, target and token scale into contiguous arrays.
template <typename T>
__global__ __launch_bounds__(256) void k_gather_chunk(const T* __restrict__ X, const int64_t* __restrict__ y,
                                                      const float* __restrict__ scale, int64_t H,
                                                      const int32_t* __restrict__ idx, RowCount rc,
                                                      T* __restrict__ xs, int64_t* __restrict__ ys,
                                                      float* __restrict__ ss) {
  constexpr int E = Elem<T>::chunk;
  const int64_t rows = rc.get();
  for (int64_t r = blockIdx.x; r < rows; r += gridDim.x) {
    const int64_t p = idx[rc.c0 + r];
    const T* src = X + p * H;
    T* dst = xs + r * H;
    for (int64_t h = (int64_t)threadIdx.x * E; h < H; h += 256 * E)
      *reinterpret_cast<u32x4*>(dst + h) = *reinterpret_cast<const u32x4*>(src + h);
    if (threadIdx.x == 0) {
      ys[r] = y[p];
      if (scale) ss[r] = scale[p];
    }
  }
}

// The per-XCD counters of a launch's work items (take_item in gemm_core.h)
// back to zero before it.
__global__ void k_queue_reset(int* head) {
  if (threadIdx.x < kXcds) head[threadIdx.x] = 0;
}

__global__ void k_fill_zero(float* p, int64_t n) {
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += (int64_t)gridDim.x * blockDim.x)
    p[i] = 0.f;
}

// ---- logits GEMM with the softmax-statistics epilogue -----------------------

template <typename T>
struct LogitsArgs {
  Operand<T> W;  // A: [V, H], K = H contiguous
  Operand<T> X;  // B: chunk tokens [rows, H]
  int64_t V, H, nvt, ldz;
  RowCount rc;     // the chunk's rows
  int64_t nvh;     // 128-wide vocabulary half tiles: 2 nvt
  T* z;            // chunk buffer [rows, ldz]
  float2* part;    // [rows, nvh] (max, sum of exp) per half tile
  int* head;       // take_item counters: nvt x ceil(rows / 256) tiles
};

__device__ __forceinline__ void store4(Rsrc r, uint32_t off, float a, float b, float c, float d, __bf16*) {
  const bf16x2 lo = __builtin_convertvector((f32x2){a, b}, bf16x2);
  const bf16x2 hi = __builtin_convertvector((f32x2){c, d}, bf16x2);
  typedef int i32x2 __attribute__((ext_vector_type(2)));
  __builtin_amdgcn_raw_buffer_store_b64(i32x2{__builtin_bit_cast(int, lo), __builtin_bit_cast(int, hi)}, r, (int)off, 0,
                                        0);
}
__device__ __forceinline__ void store4(Rsrc r, uint32_t off, float a, float b, float c, float d, float*) {
  typedef int i32x4 __attribute__((ext_vector_type(4)));
  __builtin_amdgcn_raw_buffer_store_b128(
      i32x4{__builtin_bit_cast(int, a), __builtin_bit_cast(int, b), __builtin_bit_cast(int, c), __builtin_bit_cast(int, d)},
      r, (int)off, 0, 0);
}

__device__ __forceinline__ void store4_ptr(__bf16* p, float a, float b, float c, float d) {
  const bf16x2 lo = __builtin_convertvector((f32x2){a, b}, bf16x2);
  const bf16x2 hi = __builtin_convertvector((f32x2){c, d}, bf16x2);
  *reinterpret_cast<uint2*>(p) = uint2{__builtin_bit_cast(uint32_t, lo), __builtin_bit_cast(uint32_t, hi)};
}
__device__ __forceinline__ void store4_ptr(float* p, float a, float b, float c, float d) {
  *reinterpret_cast<f32x4*>(p) = f32x4{a, b, c, d};
}

// Stand-in logit for vocabulary entries past V in the last tile: below any
// real logit, finite, and a power of two (so m * log2e is exact for it)
constexpr float kPad = -0x1p100f;

// LDS row pitch (bytes) of the staged bf16 chunk block in the logits epilogue
constexpr int kZPitch = 264;
// cache-policy bits of a buffer store that streams past the L2 (nt): the chunk
// buffer and dW are far larger than the L2, and keeping them out leaves it
// to the GEMM operands
constexpr int kNonTemporal = 2;

template <typename T>
__global__ __launch_bounds__(256) void k_logits(LogitsArgs<T> a) {
  __shared__ __attribute__((aligned(16))) char smem[kGemmLdsBytes];
  const int64_t rows = a.rc.get();
  const int64_t nct = (rows + kTile - 1) / kTile;
  int kind;
  const int64_t tile = take_item(a.head, a.nvt * nct, 0, smem, kind);
  if (tile < 0) return;
  int64_t vt, ct;
  grouped_tile(tile, a.nvt, nct, kTileGroup, vt, ct);
  const int64_t v0 = vt * kTile, c0 = ct * kTile;
  Operand<T> X = a.X;
  X.rows = rows;  // rows past the chunk's read as zero

  f32x16 acc[4][4];
  gemm_mainloop<T, false, false>(smem, a.W, v0, X, c0, 0, a.H, acc);

  const int tid = threadIdx.x, lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wy = wave >> 1, wx = wave & 1;
  // accumulator (i, j, e) holds Z[c, v] with
  //   v = vw + 32 i + 8 (e / 4) + e % 4,  c = cw + 32 j + lane % 32
  // Each wave covers 128 vocabulary entries (a half tile h = 2 vt + wy) of
  // 128 tokens; its statistics are its own, so no data is exchanged.
  const int64_t vw = v0 + wy * 128 + 4 * (lane >> 5);
  const int64_t cw = c0 + wx * 128 + (lane & 31);
  const bool full = v0 + wy * 128 + 128 <= a.V;
  const int64_t half = 2 * vt + wy;
  const int64_t nrows = rows - c0 < kTile ? rows - c0 : kTile;
  const bool store_z = a.z != nullptr;  // forward only: statistics, no chunk buffer
  const Rsrc zr = make_rsrc(store_z ? a.z + c0 * a.ldz : a.W.base, store_z ? nrows * a.ldz * (int64_t)sizeof(T) : 0);
  const uint32_t lane_off = (uint32_t)(((wx * 128 + (lane & 31)) * a.ldz + vw) * (int64_t)sizeof(T));
  const uint32_t row32 = (uint32_t)(32 * a.ldz * (int64_t)sizeof(T));
  if (!full) {
    // Entries past V (zero rows of W) must not count.  Pushed far below any
    // logit they add exp(kPad - m) = 0 to a block's sum; a block with no
    // entry below V gets (M_h, s_h) = (kPad, 0), which the lse combine
    // weighs by exp(M_h - M) = 0, and the gradient pass zeroes those columns.
    // This lane's entries sit at vw + a compile-time offset (< 128), so one
    // 32-bit count of valid entries from vw decides them all.
    const int nvalid_v = (int)(a.V - vw < 128 ? a.V - vw : 128);
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        const bool pad = 32 * i + 8 * (e >> 2) + (e & 3) >= nvalid_v;
#pragma unroll
        for (int j = 0; j < 4; ++j)
          if (pad) acc[i][j][e] = kPad;
      }
  }
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    // max over the 128 entries of token c: 64 in this lane, 64 in lane ^ 32
    float m = acc[0][j][0];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int e = 0; e < 16; ++e) m = fmaxf(m, acc[i][j][e]);
    m = fmaxf(m, __shfl_xor(m, 32));
    const float mb = m * kLog2e;
    float sum = 0.f;
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int e = 0; e < 16; ++e) sum += exp2_fast(fmaf(acc[i][j][e], kLog2e, -mb));
    sum += __shfl_xor(sum, 32);
    if (m == kPad) sum = 0.f;  // no entry of this block lies below V
    const int64_t c = cw + 32 * j;
    if (lane < 32 && c < rows) a.part[c * a.nvh + half] = float2{m, sum};
    // z - m, rounded to the chunk's element type: the entries that carry
    // most of the softmax mass are then small numbers and keep their
    // precision.  Rows are padded to a multiple of 256, so a tile never
    // crosses into the next row; entries past V fill the padding.
    if (!store_z) continue;
    if constexpr (sizeof(T) == 2) {
      // A lane holds 16-byte pieces of one token row, so direct stores would
      // scatter 32 rows per instruction.  Stage the wave's 32 x 128 block in
      // LDS (rows 264 bytes apart: both passes below are free of bank
      // conflicts) and store two whole 256-byte row segments per instruction.
      char* st = smem + wave * (32 * kZPitch);
      const int t = lane & 31, hh = lane >> 5;
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          const f32x16& q = acc[i][j];
          const bf16x2 lo = __builtin_convertvector((f32x2){q[4 * g] - m, q[4 * g + 1] - m}, bf16x2);
          const bf16x2 hi = __builtin_convertvector((f32x2){q[4 * g + 2] - m, q[4 * g + 3] - m}, bf16x2);
          *reinterpret_cast<uint2*>(st + t * kZPitch + 2 * (32 * i + 8 * g + 4 * hh)) =
              uint2{__builtin_bit_cast(uint32_t, lo), __builtin_bit_cast(uint32_t, hi)};
        }
      const uint32_t seg_off = (uint32_t)((v0 + wy * 128 + 4 * t) * 2);
#pragma unroll
      for (int k = 0; k < 16; ++k) {
        const int r = 2 * k + hh;
        const uint2 d = *reinterpret_cast<const uint2*>(st + r * kZPitch + 8 * t);
        typedef int i32x2 __attribute__((ext_vector_type(2)));
        __builtin_amdgcn_raw_buffer_store_b64(i32x2{(int)d.x, (int)d.y}, zr,
                                              (int)((uint32_t)(wx * 128 + 32 * j + r) * (uint32_t)(a.ldz * 2) + seg_off),
                                              0, kNonTemporal);
      }
    } else {
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          const f32x16& q = acc[i][j];
          store4(zr, lane_off + j * row32 + (uint32_t)((32 * i + 8 * g) * (int64_t)sizeof(T)), q[4 * g] - m,
                 q[4 * g + 1] - m, q[4 * g + 2] - m, q[4 * g + 3] - m, (T*)nullptr);
        }
    }
  }
}

// ---- log-sum-exp over the vocabulary tiles, per-token loss --------------------

// One wave per token: combine the half-tile statistics into lse, and take the
// target's logit as the dot product x_c . w_y in fp32 (the same products the
// MFMA accumulates, summed in a different order).
// The token loss of chunk row c goes to rowloss[rowidx[c]] (token
// compaction) or rowloss[c].
template <typename T>
__global__ __launch_bounds__(256) void k_lse(const float2* __restrict__ part, int64_t nvh, const T* __restrict__ X,
                                             const T* __restrict__ W, int64_t H, int64_t V,
                                             const int64_t* __restrict__ y, int64_t ign, RowCount rc,
                                             const int32_t* __restrict__ rowidx, float* __restrict__ lse,
                                             float* __restrict__ rowloss) {
  constexpr int E = Elem<T>::chunk;
  const int lane = threadIdx.x & 63;
  const int64_t c = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (c >= rc.get()) return;
  const float2* p = part + c * nvh;
  float M = -FLT_MAX;
  for (int64_t t = lane; t < nvh; t += 64) M = fmaxf(M, p[t].x);
  M = wave_max(M);
  float S = 0.f;
  for (int64_t t = lane; t < nvh; t += 64) {
    const float2 q = p[t];
    S += q.y * exp2_fast((q.x - M) * kLog2e);
  }
  S = wave_sum(S);
  const int64_t t = y[c];
  float zt = 0.f;
  if (t != ign && t >= 0 && t < V) {
    const T* xr = X + c * H;
    const T* wr = W + t * H;
    for (int64_t h = (int64_t)lane * E; h < H; h += 64 * E) {
      const u32x4 xa = *reinterpret_cast<const u32x4*>(xr + h);
      const u32x4 wa = *reinterpret_cast<const u32x4*>(wr + h);
      if constexpr (sizeof(T) == 2) {
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          zt = fmaf(__builtin_bit_cast(float, xa[q] << 16), __builtin_bit_cast(float, wa[q] << 16), zt);
          zt = fmaf(__builtin_bit_cast(float, xa[q] & 0xffff0000u), __builtin_bit_cast(float, wa[q] & 0xffff0000u), zt);
        }
      } else {
        const f32x4 xf = __builtin_bit_cast(f32x4, xa), wf = __builtin_bit_cast(f32x4, wa);
        zt = fmaf(xf.x, wf.x, zt);
        zt = fmaf(xf.y, wf.y, zt);
        zt = fmaf(xf.z, wf.z, zt);
        zt = fmaf(xf.w, wf.w, zt);
      }
    }
  }
  zt = wave_sum(zt);
  if (lane == 0) {
    const float l = M + logf(S);
    lse[c] = l;
    rowloss[rowidx ? (int64_t)rowidx[c] : c] = (t != ign) ? l - zt : 0.f;
  }
}

// ---- gradient of the loss w.r.t. the logits, in place -------------------------

__device__ __forceinline__ float grad1(float z, float lb, int64_t v, int64_t t, int64_t V, float inv) {
  return v < V ? (exp2_fast(fmaf(z, kLog2e, -lb)) - (v == t ? 1.f : 0.f)) * inv : 0.f;
}

// The chunk holds z - M_h (M_h: max of the token's 128-wide vocabulary half
// tile h), so the probability is exp(stored + M_h - lse).
template <typename T>
__global__ __launch_bounds__(kGradThreads) void k_grad(T* __restrict__ z, int64_t ldz, int64_t V,
                                              const float* __restrict__ lse, const float2* __restrict__ part,
                                              int64_t nvh, const int64_t* __restrict__ y, int64_t ign,
                                              const int32_t* __restrict__ nvalid, const float* __restrict__ scale,
                                              RowCount rc) {
  constexpr int E = Elem<T>::chunk;
  const int64_t c = blockIdx.x;
  if (c >= rc.get()) return;
  const int64_t t = y[c];
  T* row = z + c * ldz;
  if (t == ign) {
    for (int64_t v = (int64_t)threadIdx.x * E; v < ldz; v += kGradThreads * E)
      *reinterpret_cast<u32x4*>(row + v) = u32x4{0, 0, 0, 0};
    return;
  }
  // the row's factor: 1/N for the mean, or the caller's per-token scale
  float inv;
  if (scale) {
    inv = scale[c];
  } else {
    const int n = *nvalid;
    inv = 1.f / (float)(n > 0 ? n : 1);
  }
  const float l = lse[c];
  const float2* pc = part + c * nvh;
  auto grad16 = [&](u32x4 d, int64_t v) {
    const int64_t h = v / 128;
    const float lb = (l - (h < nvh ? pc[h].x : 0.f)) * kLog2e;
    if constexpr (sizeof(T) == 2) {
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const float z0 = __builtin_bit_cast(float, d[q] << 16);
        const float z1 = __builtin_bit_cast(float, d[q] & 0xffff0000u);
        const float g0 = grad1(z0, lb, v + 2 * q, t, V, inv);
        const float g1 = grad1(z1, lb, v + 2 * q + 1, t, V, inv);
        d[q] = __builtin_bit_cast(uint32_t, __builtin_convertvector((f32x2){g0, g1}, bf16x2));
      }
    } else {
      const f32x4 zf = __builtin_bit_cast(f32x4, d);
      const f32x4 g = {grad1(zf.x, lb, v, t, V, inv), grad1(zf.y, lb, v + 1, t, V, inv),
                       grad1(zf.z, lb, v + 2, t, V, inv), grad1(zf.w, lb, v + 3, t, V, inv)};
      d = __builtin_bit_cast(u32x4, g);
    }
    return d;
  };
  // kGradUnroll 16-byte loads in flight per thread.  The chunk is read once
  // here and the gradient next by the dX and dW products from memory (both
  // far larger than the caches), so loads and stores stream past them
  // (non-temporal loads measured 6.5% faster than plain ones).
  constexpr int kU = kGradUnroll;
  int64_t v = (int64_t)threadIdx.x * E;
  for (; v + (kU - 1) * kGradThreads * E < ldz; v += kU * kGradThreads * E) {
    u32x4 d[kU];
#pragma unroll
    for (int u = 0; u < kU; ++u)
      d[u] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(row + v + u * kGradThreads * E));
#pragma unroll
    for (int u = 0; u < kU; ++u) {
      const int64_t vu = v + u * kGradThreads * E;
      __builtin_nontemporal_store(grad16(d[u], vu), reinterpret_cast<u32x4*>(row + vu));
    }
  }
  for (; v < ldz; v += kGradThreads * E)
    __builtin_nontemporal_store(grad16(__builtin_nontemporal_load(reinterpret_cast<const u32x4*>(row + v)), v),
                                reinterpret_cast<u32x4*>(row + v));
}

// ---- dX = G W ---------------------------------------------------------------

template <typename T>
struct DxArgs {
  Operand<T> G;  // chunk buffer [rows, ldz], K = V contiguous: the GEMM's B (columns c)
  Operand<T> W;  // [V, H] read K-major: the GEMM's A (rows h)
  int64_t V, H, nmt, nnt, ksplit, splits;
  RowCount rc;   // the chunk's rows (nmt: tiles over rc.max)
  T* dx;         // when not split: chunk row c goes to dx row rowidx[c] (or c)
  const int32_t* rowidx;
  float* part;   // [splits, rc.max, H] when split
};

// dX item t of a launch over (split, tile) ids: nmt x nnt tiles cover the
// chunk's `rows` rows in use, split after split.  The ids are dealt to the
// XCDs in contiguous ranges, so an XCD's concurrently running tiles are
// neighbours of one split and share operand blocks in its L2.
template <typename T>
__device__ __forceinline__ void dx_item(const DxArgs<T>& a, char* smem, int64_t t, int64_t nmt, int64_t rows) {
  const int64_t ntiles = nmt * a.nnt;
  const int64_t split = t / ntiles;
  int64_t mt, nt;
  grouped_tile(t - split * ntiles, nmt, a.nnt, 4, mt, nt);
  const int64_t m0 = mt * kTile, n0 = nt * kTile;
  const int64_t k0 = split * a.ksplit;
  const int64_t k1 = k0 + a.ksplit < a.V ? k0 + a.ksplit : a.V;
  Operand<T> G = a.G, W = a.W;
  G.rows = rows;
  if (k1 < G.cols) G.cols = k1;
  if (k1 < W.rows) W.rows = k1;

  // W^T as the A operand (rows h) and G as B (columns c): each lane then
  // holds four consecutive h of one dX row
  f32x16 acc[4][4];
  gemm_mainloop<T, true, false>(smem, W, n0, G, m0, k0, k1, acc);

  // accumulator (i, j, e): h = n0 + hw + 32 i + 8 (e / 4) + e % 4, c = m0 + cw + 32 j
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int hw = (wave >> 1) * 128 + 4 * (lane >> 5);
  const int cw = (wave & 1) * 128 + (lane & 31);
  const int mlim = (int)(rows - m0 < kTile ? rows - m0 : kTile);
  const int nlim = (int)(a.H - n0 < kTile ? a.H - n0 : kTile);
  const bool split_k = a.splits > 1;
  float* pbase = a.part + split * a.rc.max * a.H + m0 * a.H + n0;
  const uint32_t H = (uint32_t)a.H;
  const bool full = mlim == kTile && nlim == kTile;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int c = cw + 32 * j;
    if (!full && c >= mlim) continue;
    // this lane's dX row (split partials stay in chunk order)
    const int64_t drow = a.rowidx ? (int64_t)a.rowidx[m0 + c] : m0 + c;
    T* drow_base = a.dx + drow * a.H + n0;
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int h = hw + 32 * i + 8 * g;
        if (full || h < nlim) {
          const f32x16& q = acc[i][j];
          if (split_k)
            *reinterpret_cast<f32x4*>(pbase + ((uint32_t)c * H + (uint32_t)h)) =
                f32x4{q[4 * g], q[4 * g + 1], q[4 * g + 2], q[4 * g + 3]};
          else
            store4_ptr(drow_base + h, q[4 * g], q[4 * g + 1], q[4 * g + 2], q[4 * g + 3]);
        }
      }
  }
}

// dX rows = sum of the split partials [splits][rc.max][H], four consecutive
// elements per thread (H is a multiple of 4), one row per workgroup pass;
// chunk row c goes to dx row rowidx[c] (or c).  The partials are read once,
// with non-temporal loads.
template <typename T>
__global__ __launch_bounds__(256) void k_dx_reduce(const float* __restrict__ part, int64_t splits, RowCount rc,
                                                   int64_t H, const int32_t* __restrict__ rowidx,
                                                   T* __restrict__ dx) {
  const int64_t rows = rc.get(), pitch = rc.max * H;
  for (int64_t c = blockIdx.x; c < rows; c += gridDim.x) {
    const float* src = part + c * H;
    T* dst = dx + (rowidx ? (int64_t)rowidx[c] : c) * H;
    for (int64_t h = 4 * (int64_t)threadIdx.x; h < H; h += 4 * 256) {
      f32x4 s = {0.f, 0.f, 0.f, 0.f};
      for (int64_t k = 0; k < splits; ++k)
        s += __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(src + k * pitch + h));
      store4_ptr(dst + h, s[0], s[1], s[2], s[3]);
    }
  }
}

// ---- dW (+)= G^T X_chunk --------------------------------------------------------

template <typename T>
struct DwArgs {
  Operand<T> G;   // chunk buffer read K-major ([rows = K][ldz]): the GEMM's B (columns v)
  Operand<T> X;   // fp32: chunk tokens [rows = K][H], read K-major: the GEMM's A (rows h)
  Operand<T> XT;  // bf16: the chunk transposed, [H][ldxt], K-contiguous: the GEMM's A
  int64_t V, H, nvt, nht;
  RowCount rc;    // the chunk's rows: the product's K extent
  float* dw;      // [V, H]
  int first;
};

// X_c^T[h][c] = X_c[c][h] for c < rows, 0 for rows <= c < ldxt (the K tail
// of the dW product reads whole 16-byte chunks, so the padding must be
// finite).  64 x 64 tiles through LDS; both global passes are coalesced.
__global__ __launch_bounds__(256) void k_transpose_chunk(const uint16_t* __restrict__ X, RowCount rc, int64_t H,
                                                         uint16_t* __restrict__ XT, int64_t ldxt) {
  __shared__ uint16_t tile[64][66];
  const int64_t rows = rc.get();
  const int64_t c0 = (int64_t)blockIdx.x * 64, h0 = (int64_t)blockIdx.y * 64;
  const int tx = threadIdx.x & 63, ty = threadIdx.x >> 6;
#pragma unroll
  for (int r = ty; r < 64; r += 4) {
    const int64_t c = c0 + r, h = h0 + tx;
    tile[r][tx] = (c < rows && h < H) ? X[c * H + h] : (uint16_t)0;
  }
  __syncthreads();
#pragma unroll
  for (int r = ty; r < 64; r += 4) {
    const int64_t h = h0 + r, c = c0 + tx;
    if (h < H && c < ldxt) XT[h * ldxt + c] = tile[tx][r];
  }
}

// Main-loop hook of the dW product on chunks after the first: the old dW
// values of the tile are added into the accumulators during the first 16 / kPer
// stages of its K loop, kPer 32 x 32 blocks per stage (blocks kPer kt ..
// kPer kt + kPer - 1 at stage kt, block b being (b % 4, b / 4)), instead of
// being read back at the end of the tile, where all tiles of a round would
// wait for them at once.  The sum is the same old + sum of products,
// accumulated in another order.  Each lane loads the four 16-byte pieces of
// each of its blocks (four consecutive h of one dW row each); rows past V read
// as zero (buffer range), columns past H land on other dW entries that are
// read but never stored.  One block per stage needs 17 stages (chunks of more
// than 1024 tokens); two per stage, for shorter chunks, need 9 (measured: two
// per stage is 0.9% slower on 64-stage tiles, 2.7% faster than the
// read-modify-write epilogue on 16-stage ones).
template <int kPer>
struct FoldOld {
  static constexpr int kStages = 16 / kPer;
  u32x4 r;         // buffer resource over the tile's rows of dW
  uint32_t voff;   // bytes to this lane's element of block (0, 0), piece 0
  uint32_t row32;  // bytes between dW rows 32 apart
  bool on;         // uniform: a chunk after the first, with > kStages stages
  f32x4 buf[4 * kPer];

  __device__ __forceinline__ bool active() const { return on; }
  // block b: rows 32 (b / 4) + lane % 32, columns 32 (b % 4) + 8 g + 4 (lane / 32) ..
  template <int Q>
  __device__ __forceinline__ void issue() {
#pragma unroll
    for (int p = 0; p < kPer; ++p) {
      const int b = Q * kPer + p;
      const uint32_t o = voff + (uint32_t)(b >> 2) * row32 + (uint32_t)(b & 3) * 128u;
#pragma unroll
      for (int g = 0; g < 4; ++g)
        asm volatile("buffer_load_dwordx4 %0, %1, %2, 0 offen"
                     : "=v"(buf[4 * p + g])
                     : "v"(o + 32u * g), "s"(r)
                     : "memory");
    }
  }
  template <int Q>
  __device__ __forceinline__ void apply(f32x16 (&acc)[4][4]) {
    // the loads landed at the barrier before this call; route the registers
    // through an empty asm placed after it, so nothing reads them earlier
#pragma unroll
    for (int g = 0; g < 4 * kPer; ++g) asm volatile("" : "+v"(buf[g]));
#pragma unroll
    for (int p = 0; p < kPer; ++p) {
      f32x16& q = acc[(Q * kPer + p) & 3][(Q * kPer + p) >> 2];
#pragma unroll
      for (int g = 0; g < 4; ++g)
#pragma unroll
        for (int e = 0; e < 4; ++e) q[4 * g + e] += buf[4 * p + g][e];
    }
  }
};

// The loop runs stages 0 .. nk - 2 with the hook in its first kStages, so a
// fold needs nk >= kStages + 1.
template <int kPer>
constexpr int kFoldMinStages = FoldOld<kPer>::kStages + 1;

// dW tile `tile` of nvt x nht over the chunk's `rows` rows in use (its K).
template <typename T>
__device__ __forceinline__ void dw_item(const DwArgs<T>& a, char* smem, int64_t tile, int64_t rows) {
  int64_t vt, ht;
  // groups of 4 vocabulary tiles (measured ~1% faster than 8 for this product)
  grouped_tile(tile, a.nvt, a.nht, 4, vt, ht);
  const int64_t v0 = vt * kTile, h0 = ht * kTile;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int vlim = (int)(a.V - v0 < kTile ? a.V - v0 : kTile);
  const int hlim = (int)(a.H - h0 < kTile ? a.H - h0 : kTile);

  // X_chunk^T as the A operand (rows h) and G^T as B (columns v): each lane
  // then holds four consecutive h of one dW row
  f32x16 acc[4][4];
  bool folded = false;
  // K (tokens) past the chunk's rows reads as zero
  Operand<T> G = a.G;
  G.rows = rows;
  if constexpr (sizeof(T) == 2) {
    Operand<T> XT = a.XT;
    XT.cols = rows;
    const int64_t nk = (rows + pipe::kBK - 1) / pipe::kBK;
    auto run = [&](auto& fold) {
      fold.r = pipe::rsrc_words(a.dw + v0 * a.H + h0, ((int64_t)vlim * a.H - h0) * 4);
      fold.voff = (uint32_t)((((wave & 1) * 128 + (lane & 31)) * a.H + (wave >> 1) * 128 + 4 * (lane >> 5)) * 4);
      fold.row32 = (uint32_t)(32 * a.H * 4);
      gemm_mainloop<T, false, true>(smem, XT, h0, G, v0, 0, rows, acc, fold);
      folded = fold.on;
    };
    if (!a.first && nk >= kFoldMinStages<2> && nk < kFoldMinStages<1>) {
      FoldOld<2> fold;
      fold.on = true;
      run(fold);
    } else {
      FoldOld<1> fold;
      fold.on = !a.first && nk >= kFoldMinStages<1>;
      run(fold);
    }
  } else {
    Operand<T> X = a.X;
    X.rows = rows;
    gemm_mainloop<T, true, true>(smem, X, h0, G, v0, 0, rows, acc);
  }

  // accumulator (i, j, e): h = h0 + (wave / 2) 128 + 32 i + 8 (e / 4) + 4 (lane / 32) + e % 4,
  //                        v = v0 + (wave % 2) 128 + 32 j + lane % 32
  float* base = a.dw + v0 * a.H + h0;
  const uint32_t H = (uint32_t)a.H;
  // A lane holds 16-byte pieces of one dW row (v), so direct accesses would
  // touch 32 rows per instruction.  Per 32-row block, stage the wave's
  // 32 x 128 floats in LDS (16-byte chunk c of row r at chunk c ^ r: both
  // passes free of bank conflicts) and read/write two whole 512-byte row
  // segments per instruction.
  char* st = smem + wave * (32 * 512);
  const int t = lane & 31, hh = lane >> 5;
  const int hcol = (wave >> 1) * 128 + 4 * t;  // this lane's 4 columns in the staged pass
  // whole tile inside dW: no per-lane guards, so the compiler can batch the
  // LDS reads and global accesses instead of branching around each one
  const bool full = vlim == kTile && hlim == kTile;
  // half-block hb = rows 16 (hb % 2) .. + 15 of block hb / 2; lane row k of
  // it is dW row vrow + 2 k + hh
  auto row_of = [&](int hb, int k) { return (wave & 1) * 128 + 32 * (hb >> 1) + 16 * (hb & 1) + 2 * k + hh; };
  auto load_old = [&](int hb, f32x4 (&o)[8]) {
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      const int v = row_of(hb, k);
      const f32x4* p = reinterpret_cast<const f32x4*>(base + ((uint32_t)v * H + (uint32_t)hcol));
      o[k] = full ? *p : (v < vlim && hcol < hlim) ? *p : f32x4{};
    }
  };
  auto stage = [&](int j) {
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int c = 8 * i + 2 * g + hh;
        *reinterpret_cast<f32x4*>(st + t * 512 + ((c ^ t) << 4)) =
            f32x4{acc[i][j][4 * g], acc[i][j][4 * g + 1], acc[i][j][4 * g + 2], acc[i][j][4 * g + 3]};
      }
  };
  // stores half-block hb; `d` holds its old rows (added to) or is scratch
  auto store_half = [&](int hb, f32x4 (&d)[8], bool add) {
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      const int r = 16 * (hb & 1) + 2 * k + hh;
      const f32x4 z = *reinterpret_cast<const f32x4*>(st + r * 512 + ((t ^ r) << 4));
      d[k] = add ? d[k] + z : z;
    }
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      const int v = row_of(hb, k);
      if (full || (v < vlim && hcol < hlim))
        __builtin_nontemporal_store(d[k], reinterpret_cast<f32x4*>(base + ((uint32_t)v * H + (uint32_t)hcol)));
    }
  };
  f32x4 x[8], y[8];
  if (a.first || folded) {
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      stage(j);
      store_half(2 * j, x, false);
      store_half(2 * j + 1, y, false);
    }
  } else {
    // two half-blocks of old rows in flight: the rows of half-block h + 1 are
    // requested before the stores of half-block h, so waiting for them never
    // waits for those stores (loads and stores complete in issue order)
    load_old(0, x);
    load_old(1, y);
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      stage(j);
      store_half(2 * j, x, true);
      if (j < 3) load_old(2 * j + 2, x);
      store_half(2 * j + 1, y, true);
      if (j < 3) load_old(2 * j + 3, y);
    }
  }
}

// ---- dX and dW of a chunk in one launch ------------------------------------------

// Both products read the chunk's gradient and nothing the other writes, so
// they share one launch and one tile queue: each XCD's range holds its share
// of the dX items first, then its share of the dW tiles.  The dX items are
// long (K = V) and go out first, one per CU; a CU whose dX item ends takes dW
// tiles, so the XCDs' different speeds and the last, partial round of dW
// tiles spread over the whole launch instead of ending each product.
template <typename T>
struct BwdArgs {
  DxArgs<T> dx;
  DwArgs<T> dw;
  int* head;  // kXcds counters, zero at launch
};

template <typename T>
__global__ __launch_bounds__(256) void k_dx_dw(BwdArgs<T> a) {
  __shared__ __attribute__((aligned(16))) char smem[kGemmLdsBytes];
  const int64_t rows = a.dw.rc.get();
  const int64_t nmt = (rows + kTile - 1) / kTile;
  const int64_t ndx = nmt * a.dx.nnt * a.dx.splits;
  // an empty chunk after the first adds nothing to dW
  const int64_t ndw = (rows == 0 && !a.dw.first) ? 0 : a.dw.nvt * a.dw.nht;
  int kind;
  const int64_t item = take_item(a.head, ndx, ndw, smem, kind);
  if (item < 0) return;
  if (kind == 0)
    dx_item(a.dx, smem, item, nmt, rows);
  else
    dw_item(a.dw, smem, item, rows);
}

// ---- loss = sum of token losses / N ------------------------------------------------

__global__ __launch_bounds__(1024) void k_loss_final(const float* __restrict__ rowloss, int64_t BT,
                                                     const int32_t* __restrict__ nvalid, float* loss) {
  __shared__ double red[1024];
  double s = 0.0;
  for (int64_t i = threadIdx.x; i < BT; i += 1024) s += (double)rowloss[i];
  red[threadIdx.x] = s;
  __syncthreads();
  for (int o = 512; o > 0; o >>= 1) {
    if ((int)threadIdx.x < o) red[threadIdx.x] += red[threadIdx.x + o];
    __syncthreads();
  }
  if (threadIdx.x == 0) {
    const int n = *nvalid;
    *loss = (float)(red[0] / (double)(n > 0 ? n : 1));
  }
}

// ---- host side ------------------------------------------------------------------------

hipError_t launch_count_valid(const int64_t* y, int64_t BT, int64_t V, int64_t ign, int32_t* nvalid, int32_t* err,
                              hipStream_t s) {
  ProfScope ps(kPhaseCount, s);
  hipLaunchKernelGGL(k_count_valid, dim3(1), dim3(1024), 0, s, y, BT, V, ign, nvalid, err, (int32_t*)nullptr);
  return hipGetLastError();
}

hipError_t launch_compact(const Layout& L, const int64_t* y, int64_t ign, char* ws, int32_t* err, void* dX,
                          float* rowloss, hipStream_t s) {
  int32_t* nvalid = reinterpret_cast<int32_t*>(ws + L.off_nvalid);
  int32_t* idx = reinterpret_cast<int32_t*>(ws + L.off_idx);
  {
    ProfScope ps(kPhaseCount, s);
    hipLaunchKernelGGL(k_count_valid, dim3(1), dim3(1024), 0, s, y, L.BT, L.V, ign, nvalid, err, idx);
  }
  if (L.BT > 0) {
    const unsigned blocks = (unsigned)(L.BT < 1024 ? L.BT : 1024);
    ProfScope ps(kPhaseGather, s);
    if (L.dtype == 1)
      hipLaunchKernelGGL(k_zero_ignored<__bf16>, dim3(blocks), dim3(256), 0, s, idx, nvalid, L.BT, L.H,
                         static_cast<__bf16*>(dX), rowloss);
    else
      hipLaunchKernelGGL(k_zero_ignored<float>, dim3(blocks), dim3(256), 0, s, idx, nvalid, L.BT, L.H,
                         static_cast<float*>(dX), rowloss);
  }
  return hipGetLastError();
}

hipError_t launch_fill_zero(float* p, int64_t n, hipStream_t s) {
  if (n <= 0) return hipSuccess;
  int64_t blocks = (n + 255) / 256;
  if (blocks > 4096) blocks = 4096;
  ProfScope ps(kPhaseFill, s);
  hipLaunchKernelGGL(k_fill_zero, dim3((unsigned)blocks), dim3(256), 0, s, p, n);
  return hipGetLastError();
}

hipError_t launch_loss_final(const float* rowloss, int64_t BT, const int32_t* nvalid, float* loss, hipStream_t s) {
  ProfScope ps(kPhaseLoss, s);
  hipLaunchKernelGGL(k_loss_final, dim3(1), dim3(1024), 0, s, rowloss, BT, nvalid, loss);
  return hipGetLastError();
}

// Logits of one chunk with their softmax statistics (and, when z is not
// null, the chunk buffer), then lse and the per-token losses.  Xc, yc: the
// chunk's rows; row c's token loss goes to rowloss[rowidx[c]] (or [c]).
template <typename T>
static void logits_lse(const Layout& L, const T* Xc, const T* W, const int64_t* yc, int64_t ign, RowCount rc,
                       const int32_t* rowidx, char* ws, float* rowloss, T* z, hipStream_t s) {
  const int64_t H = L.H, V = L.V;
  float2* part = reinterpret_cast<float2*>(ws + L.off_part);
  float* lse = reinterpret_cast<float*>(ws + L.off_lse);
  LogitsArgs<T> la;
  la.W = Operand<T>{W, H, V, H};
  la.X = Operand<T>{Xc, H, rc.max, H};
  la.V = V;
  la.H = H;
  la.nvt = L.nvt;
  la.rc = rc;
  la.nvh = 2 * L.nvt;
  la.ldz = L.ldz;
  la.z = z;
  la.part = part;
  // the grid covers rc.max rows; the kernel counts the tiles of the rows in use
  const int64_t tiles = la.nvt * ((rc.max + kTile - 1) / kTile);
  la.head = reinterpret_cast<int*>(ws + L.off_queue);
  {
    ProfScope ps(kPhaseLogits, s);
    hipLaunchKernelGGL(k_queue_reset, dim3(1), dim3(64), 0, s, la.head);
    hipLaunchKernelGGL(k_logits<T>, dim3((unsigned)queue_grid(tiles)), dim3(kThreads), 0, s, la);
  }

  {
    ProfScope ps(kPhaseLse, s);
    hipLaunchKernelGGL(k_lse<T>, dim3((unsigned)((rc.max + 3) / 4)), dim3(256), 0, s, part, 2 * L.nvt, Xc, W, H, V, yc,
                       ign, rc, rowidx, lse, rowloss);
  }
}

template <typename T>
static hipError_t backward_impl(const Layout& L, const T* Xc, const T* W, const int64_t* yc, const float* scalec,
                                int64_t ign, RowCount rc, const int32_t* rowidx, char* ws, T* dx, float* dW,
                                bool first, hipStream_t s);

// Chunk c0 .. c0 + rows - 1 of the tokens in their order (no compaction).
template <typename T>
static hipError_t chunk_impl(const Layout& L, const T* X, const T* W, const int64_t* y, const float* scale,
                             int64_t ign, int64_t c0, int64_t rows, char* ws, float* rowloss, T* dX, float* dW,
                             bool first, hipStream_t s) {
  const RowCount rc{nullptr, 0, rows};
  logits_lse<T>(L, X + c0 * L.H, W, y + c0, ign, rc, nullptr, ws, rowloss + c0, reinterpret_cast<T*>(ws + L.off_chunk),
                s);
  return backward_impl<T>(L, X + c0 * L.H, W, y + c0, scale ? scale + c0 : nullptr, ign, rc, nullptr, ws,
                          dX + c0 * L.H, dW, first, s);
}

// Chunk of the non-ignored tokens c0 .. c0 + rows_max - 1 (token
// compaction): their rows are gathered, the products run on the rows in use,
// token losses and dX rows go back to the tokens' positions.
template <typename T>
static hipError_t chunk_compact_impl(const Layout& L, const T* X, const T* W, const int64_t* y, const float* scale,
                                     int64_t ign, int64_t c0, int64_t rows_max, char* ws, float* rowloss, T* dX,
                                     float* dW, bool first, hipStream_t s) {
  const RowCount rc{reinterpret_cast<const int32_t*>(ws + L.off_nvalid), c0, rows_max};
  const int32_t* idx = reinterpret_cast<const int32_t*>(ws + L.off_idx);
  T* xs = reinterpret_cast<T*>(ws + L.off_xs);
  int64_t* ys = reinterpret_cast<int64_t*>(ws + L.off_ys);
  float* ss = reinterpret_cast<float*>(ws + L.off_ss);
  {
    const unsigned blocks = (unsigned)(rows_max < 4096 ? rows_max : 4096);
    ProfScope ps(kPhaseGather, s);
    hipLaunchKernelGGL(k_gather_chunk<T>, dim3(blocks), dim3(256), 0, s, X, y, scale, L.H, idx, rc, xs, ys, ss);
  }
  logits_lse<T>(L, xs, W, ys, ign, rc, idx + c0, ws, rowloss, reinterpret_cast<T*>(ws + L.off_chunk), s);
  return backward_impl<T>(L, xs, W, ys, scale ? ss : nullptr, ign, rc, idx + c0, ws, dX, dW, first, s);
}

// The backward half of a chunk whose logits (z - M_h) and statistics are in
// the workspace: in-place gradient, dX rows, dW (+)=.  Xc, yc, scalec: the
// chunk's rows; chunk row c's dX row goes to dx row rowidx[c] (or c).
template <typename T>
static hipError_t backward_impl(const Layout& L, const T* Xc, const T* W, const int64_t* yc, const float* scalec,
                                int64_t ign, RowCount rc, const int32_t* rowidx, char* ws, T* dx, float* dW,
                                bool first, hipStream_t s) {
  const int64_t H = L.H, V = L.V, rows = rc.max;
  T* z = reinterpret_cast<T*>(ws + L.off_chunk);
  float2* part = reinterpret_cast<float2*>(ws + L.off_part);
  float* lse = reinterpret_cast<float*>(ws + L.off_lse);
  const int32_t* nvalid = reinterpret_cast<const int32_t*>(ws + L.off_nvalid);
  {
    ProfScope ps(kPhaseGrad, s);
    hipLaunchKernelGGL(k_grad<T>, dim3((unsigned)rows), dim3(kGradThreads), 0, s, z, L.ldz, V, lse, part, 2 * L.nvt, yc,
                       ign, nvalid, scalec, rc);
  }

  // dX = G W
  DxArgs<T> da;
  da.G = Operand<T>{z, L.ldz, rows, L.ldz};
  da.W = Operand<T>{W, H, V, H};
  da.V = V;
  da.H = H;
  da.rc = rc;
  da.nmt = (rows + kTile - 1) / kTile;
  da.nnt = (H + kTile - 1) / kTile;
  const int64_t ks = kStageK<T>;
  da.ksplit = ((V + L.splits - 1) / L.splits + ks - 1) / ks * ks;
  const int64_t splits = (V + da.ksplit - 1) / da.ksplit;
  da.splits = splits;
  da.dx = dx;
  da.rowidx = rowidx;
  da.part = reinterpret_cast<float*>(ws + L.off_dxpart);

  // dW (+)= G^T X_chunk
  DwArgs<T> wa;
  wa.G = Operand<T>{z, L.ldz, rows, L.ldz};
  wa.X = Operand<T>{Xc, H, rows, H};
  T* xt = reinterpret_cast<T*>(ws + L.off_part);  // the statistics are dead after the gradient pass
  wa.XT = Operand<T>{xt, L.ldxt, H, rows};
  wa.V = V;
  wa.H = H;
  wa.rc = rc;
  wa.nvt = L.nvt;
  wa.nht = (H + kTile - 1) / kTile;
  wa.dw = dW;
  wa.first = first ? 1 : 0;
  BwdArgs<T> ba{da, wa, reinterpret_cast<int*>(ws + L.off_queue)};
  const int64_t items = da.nmt * da.nnt * splits + wa.nvt * wa.nht;
  {
    ProfScope ps(kPhaseDxDw, s);  // bf16: the chunk transpose is counted with the products
    if constexpr (sizeof(T) == 2)
      hipLaunchKernelGGL(k_transpose_chunk, dim3((unsigned)(L.ldxt / 64), (unsigned)((H + 63) / 64)), dim3(256), 0, s,
                         reinterpret_cast<const uint16_t*>(Xc), rc, H, reinterpret_cast<uint16_t*>(xt), L.ldxt);
    hipLaunchKernelGGL(k_queue_reset, dim3(1), dim3(64), 0, s, ba.head);
    hipLaunchKernelGGL(k_dx_dw<T>, dim3((unsigned)queue_grid(items)), dim3(kThreads), 0, s, ba);
  }
  if (splits > 1) {
    const unsigned blocks = (unsigned)(rows < 8192 ? rows : 8192);
    ProfScope ps(kPhaseDxReduce, s);
    hipLaunchKernelGGL(k_dx_reduce<T>, dim3(blocks), dim3(256), 0, s, da.part, splits, rc, H, rowidx, dx);
  }
  return hipGetLastError();
}

hipError_t launch_fwd_chunk(const Layout& L, const void* X, const void* W, const int64_t* y, int64_t ign, int64_t c0,
                            int64_t rows, char* ws, float* rowloss, hipStream_t s) {
  const RowCount rc{nullptr, 0, rows};
  if (L.dtype == 1)
    logits_lse<__bf16>(L, static_cast<const __bf16*>(X) + c0 * L.H, static_cast<const __bf16*>(W), y + c0, ign, rc,
                       nullptr, ws, rowloss + c0, nullptr, s);
  else
    logits_lse<float>(L, static_cast<const float*>(X) + c0 * L.H, static_cast<const float*>(W), y + c0, ign, rc,
                      nullptr, ws, rowloss + c0, nullptr, s);
  return hipGetLastError();
}

hipError_t launch_logits_chunk(const Layout& L, const void* X, const void* W, const int64_t* y, int64_t ign, int64_t c0,
                               int64_t rows, char* ws, float* rowloss, hipStream_t s) {
  const RowCount rc{nullptr, 0, rows};
  if (L.dtype == 1)
    logits_lse<__bf16>(L, static_cast<const __bf16*>(X) + c0 * L.H, static_cast<const __bf16*>(W), y + c0, ign, rc,
                       nullptr, ws, rowloss + c0, reinterpret_cast<__bf16*>(ws + L.off_chunk), s);
  else
    logits_lse<float>(L, static_cast<const float*>(X) + c0 * L.H, static_cast<const float*>(W), y + c0, ign, rc,
                      nullptr, ws, rowloss + c0, reinterpret_cast<float*>(ws + L.off_chunk), s);
  return hipGetLastError();
}

hipError_t launch_grad_chunk(const Layout& L, const void* X, const void* W, const int64_t* y, const float* scale,
                             int64_t ign, int64_t c0, int64_t rows, char* ws, void* dX, float* dW, bool first,
                             hipStream_t s) {
  const RowCount rc{nullptr, 0, rows};
  const float* sc = scale ? scale + c0 : nullptr;
  if (L.dtype == 1)
    return backward_impl<__bf16>(L, static_cast<const __bf16*>(X) + c0 * L.H, static_cast<const __bf16*>(W), y + c0, sc,
                                 ign, rc, nullptr, ws, static_cast<__bf16*>(dX) + c0 * L.H, dW, first, s);
  return backward_impl<float>(L, static_cast<const float*>(X) + c0 * L.H, static_cast<const float*>(W), y + c0, sc, ign,
                              rc, nullptr, ws, static_cast<float*>(dX) + c0 * L.H, dW, first, s);
}

hipError_t launch_flce_chunk(const Layout& L, const void* X, const void* W, const int64_t* y, const float* scale,
                             int64_t ign, int64_t c0, int64_t rows, char* ws, float* rowloss, void* dX, float* dW,
                             bool first, hipStream_t s) {
  if (L.compact) {
    if (L.dtype == 1)
      return chunk_compact_impl<__bf16>(L, static_cast<const __bf16*>(X), static_cast<const __bf16*>(W), y, scale, ign,
                                        c0, rows, ws, rowloss, static_cast<__bf16*>(dX), dW, first, s);
    return chunk_compact_impl<float>(L, static_cast<const float*>(X), static_cast<const float*>(W), y, scale, ign, c0,
                                     rows, ws, rowloss, static_cast<float*>(dX), dW, first, s);
  }
  if (L.dtype == 1)
    return chunk_impl<__bf16>(L, static_cast<const __bf16*>(X), static_cast<const __bf16*>(W), y, scale, ign, c0, rows,
                              ws, rowloss, static_cast<__bf16*>(dX), dW, first, s);
  return chunk_impl<float>(L, static_cast<const float*>(X), static_cast<const float*>(W), y, scale, ign, c0, rows, ws,
                           rowloss, static_cast<float*>(dX), dW, first, s);
}

}  // namespace flce
