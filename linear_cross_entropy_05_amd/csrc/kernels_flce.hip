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
//   logits   Z[c,v] = x_c . w_v; per (token, 256-wide vocabulary tile t)
//            the max M_t and sum of exp(z - M_t), and the target's logit,
//            taken from the fp32 accumulators in the GEMM epilogue; the
//            chunk buffer receives z - M_t in the element type
//   lse      lse_c = M + ln sum_t s_t e^(m_t - M) over the tiles, M = max m_t;
//            per-token loss lse_c - z_{c,y_c} (0 for ignored tokens)
//   grad     G[c,v] = (e^(Z[c,v] - lse_c) - [v = y_c]) / N written over the
//            stored z - M_t
//            (0 on ignored tokens), N = number of non-ignored tokens
//   dX       dX[c,:] = G[c,:] W
//   dW       dW (+)= G^T X_chunk, fp32, stored on the first chunk
// and once per call: count N and check targets; loss = sum of token losses / N.
#include <float.h>

#include "flce_internal.h"
#include "gemm_core.h"

namespace flce {

constexpr float kLog2e = 1.4426950408889634f;

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

__global__ __launch_bounds__(1024) void k_count_valid(const int64_t* __restrict__ y, int64_t BT, int64_t V,
                                                      int64_t ign, int32_t* nvalid, int32_t* err) {
  __shared__ int red_n[16], red_b[16];
  int n = 0, bad = 0;
  for (int64_t i = threadIdx.x; i < BT; i += 1024) {
    const int64_t t = y[i];
    if (t != ign) {
      ++n;
      bad |= (t < 0 || t >= V);
    }
  }
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) {
    n += __shfl_xor(n, o);
    bad |= __shfl_xor(bad, o);
  }
  const int w = threadIdx.x >> 6;
  if ((threadIdx.x & 63) == 0) {
    red_n[w] = n;
    red_b[w] = bad;
  }
  __syncthreads();
  if (threadIdx.x == 0) {
    int tn = 0, tb = 0;
    for (int i = 0; i < 16; ++i) {
      tn += red_n[i];
      tb |= red_b[i];
    }
    *nvalid = tn;
    *err = tb ? 6 : 0;
  }
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
  const int64_t* y;
  int64_t V, H, rows, nvt, nct, ldz;
  T* z;            // chunk buffer [rows, ldz]
  float2* part;    // [rows, nvt] (max, sum of exp) per vocabulary tile
  float* zt;       // [rows] target logit
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

template <typename T>
__global__ __launch_bounds__(256) void k_logits(LogitsArgs<T> a) {
  __shared__ __attribute__((aligned(16))) char smem[kLdsBytes];
  const int64_t tile = xcd_tile(blockIdx.x, a.nvt * a.nct);
  const int64_t vt = tile / a.nct, ct = tile % a.nct;
  const int64_t v0 = vt * kTile, c0 = ct * kTile;

  f32x16 acc[4][4];
  gemm_mainloop<T, false, false>(smem, a.W, v0, a.X, c0, 0, a.H, acc);

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wy = wave >> 1, wx = wave & 1;
  // accumulator (i, j, e) holds Z[c, v] with
  //   v = vw + 32 i + 8 (e / 4) + e % 4,  c = cw + 32 j + lane % 32
  const int64_t vw = v0 + wy * 128 + 4 * (lane >> 5);
  const int64_t cw = c0 + wx * 128 + (lane & 31);
  const bool full = v0 + kTile <= a.V;

  // 1. per token: the max over this wave's 128 vocabulary entries (in-lane
  //    over 64 values, then with the lane holding the other 64)
  float mj[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    float m = -FLT_MAX;
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int e = 0; e < 16; ++e)
        if (full || vw + 32 * i + 8 * (e >> 2) + (e & 3) < a.V) m = fmaxf(m, acc[i][j][e]);
    mj[j] = fmaxf(m, __shfl_xor(m, 32));

    // the target logit, from the one lane that holds it (fp32, before rounding)
    const int64_t c = cw + 32 * j;
    if (c < a.rows) {
      const int64_t t = a.y[c] - (v0 + wy * 128);
      if (t >= 0 && t < 128 && ((t >> 2) & 1) == (lane >> 5)) {
        const int i = (int)(t >> 5), g = (int)((t >> 3) & 3), r = (int)(t & 3);
#pragma unroll
        for (int ii = 0; ii < 4; ++ii)
#pragma unroll
          for (int e = 0; e < 16; ++e)
            if (ii == i && (e >> 2) == g && (e & 3) == r) a.zt[c] = acc[ii][j][e];
      }
    }
  }

  // 2. the tile max M over both waves that hold these tokens (wy = 0, 1),
  //    through LDS; the main loop ended on a barrier, so LDS is free
  float* xm = reinterpret_cast<float*>(smem);        // [2][256] wave maxima
  float* xs = xm + 2 * kTile;                        // [2][256] wave sums
  if (lane < 32) {
#pragma unroll
    for (int j = 0; j < 4; ++j) xm[wy * kTile + wx * 128 + 32 * j + lane] = mj[j];
  }
  __syncthreads();
#pragma unroll
  for (int j = 0; j < 4; ++j) mj[j] = fmaxf(mj[j], xm[(wy ^ 1) * kTile + wx * 128 + 32 * j + (lane & 31)]);

  // 3. sum of exp(z - M) over the tile, and z - M rounded to the chunk's
  //    element type: stored relative to the tile max, the entries that carry
  //    most of the softmax mass are small numbers and keep their precision.
  //    Rows are padded to a multiple of 256, so a tile never crosses into the
  //    next row; entries past V fill the padding (zeroed later).
  const int64_t nrows = a.rows - c0 < kTile ? a.rows - c0 : kTile;
  const Rsrc zr = make_rsrc(a.z + c0 * a.ldz, nrows * a.ldz * (int64_t)sizeof(T));
  const uint32_t lane_off = (uint32_t)(((wx * 128 + (lane & 31)) * a.ldz + vw) * (int64_t)sizeof(T));
  const uint32_t row32 = (uint32_t)(32 * a.ldz * (int64_t)sizeof(T));
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const float M = mj[j];
    const float mb = M * kLog2e;
    float s = 0.f;
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int e = 0; e < 16; ++e)
        if (full || vw + 32 * i + 8 * (e >> 2) + (e & 3) < a.V) s += exp2_fast(fmaf(acc[i][j][e], kLog2e, -mb));
    s += __shfl_xor(s, 32);
    if (lane < 32) xs[wy * kTile + wx * 128 + 32 * j + lane] = s;
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const f32x16& q = acc[i][j];
        store4(zr, lane_off + j * row32 + (uint32_t)((32 * i + 8 * g) * (int64_t)sizeof(T)), q[4 * g] - M,
               q[4 * g + 1] - M, q[4 * g + 2] - M, q[4 * g + 3] - M, (T*)nullptr);
      }
  }
  __syncthreads();
  if (wy == 0 && lane < 32) {
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int64_t c = cw + 32 * j;
      if (c < a.rows) {
        const int k = wx * 128 + 32 * j + lane;
        a.part[c * a.nvt + vt] = float2{mj[j], xs[k] + xs[kTile + k]};
      }
    }
  }
}

// ---- log-sum-exp over the vocabulary tiles, per-token loss --------------------

__global__ __launch_bounds__(256) void k_lse(const float2* __restrict__ part, int64_t nvt,
                                             const float* __restrict__ zt, const int64_t* __restrict__ y,
                                             int64_t ign, int64_t rows, float* __restrict__ lse,
                                             float* __restrict__ rowloss) {
  const int lane = threadIdx.x & 63;
  const int64_t c = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (c >= rows) return;
  const float2* p = part + c * nvt;
  float M = -FLT_MAX;
  for (int64_t t = lane; t < nvt; t += 64) M = fmaxf(M, p[t].x);
  M = wave_max(M);
  float S = 0.f;
  for (int64_t t = lane; t < nvt; t += 64) {
    const float2 q = p[t];
    S += q.y * exp2_fast((q.x - M) * kLog2e);
  }
  S = wave_sum(S);
  if (lane == 0) {
    const float l = M + logf(S);
    lse[c] = l;
    rowloss[c] = (y[c] != ign) ? l - zt[c] : 0.f;
  }
}

// ---- gradient of the loss w.r.t. the logits, in place -------------------------

__device__ __forceinline__ float grad1(float z, float lb, int64_t v, int64_t t, int64_t V, float inv) {
  return v < V ? (exp2_fast(fmaf(z, kLog2e, -lb)) - (v == t ? 1.f : 0.f)) * inv : 0.f;
}

// The chunk holds z - M_t (M_t: max of the token's vocabulary tile t), so the
// probability is exp(stored + M_t - lse).
template <typename T>
__global__ __launch_bounds__(256) void k_grad(T* __restrict__ z, int64_t ldz, int64_t V,
                                              const float* __restrict__ lse, const float2* __restrict__ part,
                                              int64_t nvt, const int64_t* __restrict__ y, int64_t ign,
                                              const int32_t* __restrict__ nvalid) {
  constexpr int E = Elem<T>::chunk;
  const int64_t c = blockIdx.x;
  const int64_t t = y[c];
  T* row = z + c * ldz;
  if (t == ign) {
    for (int64_t v = (int64_t)threadIdx.x * E; v < ldz; v += 256 * E)
      *reinterpret_cast<u32x4*>(row + v) = u32x4{0, 0, 0, 0};
    return;
  }
  const int n = *nvalid;
  const float inv = 1.f / (float)(n > 0 ? n : 1);
  const float l = lse[c];
  const float2* pc = part + c * nvt;
  for (int64_t v = (int64_t)threadIdx.x * E; v < ldz; v += 256 * E) {
    u32x4 d = *reinterpret_cast<const u32x4*>(row + v);
    const int64_t tile = v / kTile;
    const float lb = (l - (tile < nvt ? pc[tile].x : 0.f)) * kLog2e;
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
    *reinterpret_cast<u32x4*>(row + v) = d;
  }
}

// ---- dX = G W ---------------------------------------------------------------

template <typename T>
struct DxArgs {
  Operand<T> G;  // A: chunk buffer [rows, ldz], K = V contiguous
  Operand<T> W;  // B: [V, H] read K-major
  int64_t V, H, rows, nmt, nnt, ksplit;
  T* dx;         // [rows, H] when not split
  float* part;   // [splits, rows, H] when split
};

template <typename T>
__global__ __launch_bounds__(256) void k_dx(DxArgs<T> a) {
  __shared__ __attribute__((aligned(16))) char smem[kLdsBytes];
  const int64_t tile = blockIdx.x;
  const int64_t mt = tile / a.nnt, nt = tile % a.nnt;
  const int64_t m0 = mt * kTile, n0 = nt * kTile;
  const int64_t k0 = (int64_t)blockIdx.y * a.ksplit;
  const int64_t k1 = k0 + a.ksplit < a.V ? k0 + a.ksplit : a.V;
  Operand<T> G = a.G, W = a.W;
  if (k1 < G.cols) G.cols = k1;
  if (k1 < W.rows) W.rows = k1;

  f32x16 acc[4][4];
  gemm_mainloop<T, false, true>(smem, G, m0, W, n0, k0, k1, acc);

  // accumulator (i, j, e) holds output row m0 + mw + 32 i + 8 (e / 4) + e % 4,
  // column n0 + nw + 32 j; offsets are taken from the tile's first row
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int mw = (wave >> 1) * 128 + 4 * (lane >> 5);
  const int nw = (wave & 1) * 128 + (lane & 31);
  const int mlim = (int)(a.rows - m0 < kTile ? a.rows - m0 : kTile);
  const int nlim = (int)(a.H - n0 < kTile ? a.H - n0 : kTile);
  const bool split = gridDim.y > 1;
  float* pbase = a.part + (int64_t)blockIdx.y * a.rows * a.H + m0 * a.H + n0;
  T* dbase = a.dx + m0 * a.H + n0;
  const uint32_t H = (uint32_t)a.H;
  const bool full = mlim == kTile && nlim == kTile;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int n = nw + 32 * j;
    if (!full && n >= nlim) continue;
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        const int m = mw + 32 * i + 8 * (e >> 2) + (e & 3);
        if (full || m < mlim) {
          const uint32_t off = (uint32_t)m * H + (uint32_t)n;
          if (split)
            pbase[off] = acc[i][j][e];
          else
            dbase[off] = (T)acc[i][j][e];
        }
      }
  }
}

template <typename T>
__global__ __launch_bounds__(256) void k_dx_reduce(const float* __restrict__ part, int64_t splits, int64_t n,
                                                   T* __restrict__ dx) {
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += (int64_t)gridDim.x * blockDim.x) {
    float s = 0.f;
    for (int64_t k = 0; k < splits; ++k) s += part[k * n + i];
    dx[i] = (T)s;
  }
}

// ---- dW (+)= G^T X_chunk --------------------------------------------------------

template <typename T>
struct DwArgs {
  Operand<T> G;  // A: chunk buffer read K-major ([rows = K][ldz = M])
  Operand<T> X;  // B: chunk tokens [rows = K][H = N], read K-major
  int64_t V, H, rows, nvt, nht;
  float* dw;     // [V, H]
  int first;
};

template <typename T>
__global__ __launch_bounds__(256) void k_dw(DwArgs<T> a) {
  __shared__ __attribute__((aligned(16))) char smem[kLdsBytes];
  const int64_t tile = xcd_tile(blockIdx.x, a.nvt * a.nht);
  const int64_t vt = tile / a.nht, ht = tile % a.nht;
  const int64_t v0 = vt * kTile, h0 = ht * kTile;

  f32x16 acc[4][4];
  gemm_mainloop<T, true, true>(smem, a.G, v0, a.X, h0, 0, a.rows, acc);

  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int vw = (wave >> 1) * 128 + 4 * (lane >> 5);
  const int hw = (wave & 1) * 128 + (lane & 31);
  const int vlim = (int)(a.V - v0 < kTile ? a.V - v0 : kTile);
  const int hlim = (int)(a.H - h0 < kTile ? a.H - h0 : kTile);
  float* base = a.dw + v0 * a.H + h0;
  const uint32_t H = (uint32_t)a.H;
  const bool full = vlim == kTile && hlim == kTile;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int h = hw + 32 * j;
    if (!full && h >= hlim) continue;
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        const int v = vw + 32 * i + 8 * (e >> 2) + (e & 3);
        if (full || v < vlim) {
          float* p = base + ((uint32_t)v * H + (uint32_t)h);
          *p = a.first ? acc[i][j][e] : *p + acc[i][j][e];
        }
      }
  }
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

static size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

static int64_t pick_splits(int64_t tiles, int64_t kstages, size_t part_bytes_per_split, size_t chunk_bytes) {
  // fewest K splits that fill the 256 CUs best, each split keeping >= 16
  // stages of K, the fp32 partials within half the chunk buffer
  constexpr int64_t kCUs = 256;
  int64_t best = 1;
  double best_cost = (double)((tiles + kCUs - 1) / kCUs);
  for (int64_t s = 2; s <= 16; ++s) {
    if (kstages / s < 16) break;
    if ((size_t)s * part_bytes_per_split > chunk_bytes / 2) break;
    const double cost = (double)((tiles * s + kCUs - 1) / kCUs) / (double)s;
    if (cost < best_cost * 0.97) {
      best = s;
      best_cost = cost;
    }
  }
  return best;
}

Layout make_layout(int64_t BT, int64_t H, int64_t V, int64_t chunk_tokens, int dtype) {
  Layout L{};
  L.BT = BT;
  L.H = H;
  L.V = V;
  L.dtype = dtype;
  L.esize = dtype == 1 ? 2 : 4;
  L.ldz = (V + kTile - 1) / kTile * kTile;
  L.nvt = (V + kTile - 1) / kTile;
  int64_t C = chunk_tokens;
  if (C <= 0) {
    // largest power of two whose chunk buffer fits in 1 GiB
    C = 1;
    while ((C * 2) * L.ldz * L.esize <= (int64_t(1) << 30)) C *= 2;
  }
  if (C > BT) C = BT;
  if (C < 1) C = 1;
  L.C = C;
  const int64_t ks = kRowBytes / L.esize;
  const int64_t tiles = ((C + kTile - 1) / kTile) * ((H + kTile - 1) / kTile);
  const size_t chunk_bytes = (size_t)C * L.ldz * L.esize;
  L.splits = pick_splits(tiles, (V + ks - 1) / ks, (size_t)C * H * 4, chunk_bytes);
  size_t o = 0;
  L.off_nvalid = o;
  o = align256(o + 16);
  L.off_zt = o;
  o = align256(o + (size_t)C * 4);
  L.off_lse = o;
  o = align256(o + (size_t)C * 4);
  L.off_rowloss = o;
  o = align256(o + (size_t)(BT > 0 ? BT : 1) * 4);
  L.off_part = o;
  o = align256(o + (size_t)C * L.nvt * 8);
  L.off_chunk = o;
  o = align256(o + chunk_bytes);
  L.off_dxpart = o;
  if (L.splits > 1) o = align256(o + (size_t)L.splits * C * H * 4);
  L.total = o;
  return L;
}

hipError_t launch_count_valid(const int64_t* y, int64_t BT, int64_t V, int64_t ign, int32_t* nvalid, int32_t* err,
                              hipStream_t s) {
  ProfScope ps(kPhaseCount, s);
  hipLaunchKernelGGL(k_count_valid, dim3(1), dim3(1024), 0, s, y, BT, V, ign, nvalid, err);
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

template <typename T>
static hipError_t chunk_impl(const Layout& L, const T* X, const T* W, const int64_t* y, int64_t ign, int64_t c0,
                             int64_t rows, char* ws, float* rowloss, T* dX, float* dW, bool first, hipStream_t s) {
  const int64_t H = L.H, V = L.V;
  T* z = reinterpret_cast<T*>(ws + L.off_chunk);
  float2* part = reinterpret_cast<float2*>(ws + L.off_part);
  float* zt = reinterpret_cast<float*>(ws + L.off_zt);
  float* lse = reinterpret_cast<float*>(ws + L.off_lse);
  const int32_t* nvalid = reinterpret_cast<const int32_t*>(ws + L.off_nvalid);
  const T* Xc = X + c0 * H;
  const int64_t* yc = y + c0;

  // logits + softmax statistics
  LogitsArgs<T> la;
  la.W = Operand<T>{W, H, V, H};
  la.X = Operand<T>{Xc, H, rows, H};
  la.y = yc;
  la.V = V;
  la.H = H;
  la.rows = rows;
  la.nvt = L.nvt;
  la.nct = (rows + kTile - 1) / kTile;
  la.ldz = L.ldz;
  la.z = z;
  la.part = part;
  la.zt = zt;
  {
    ProfScope ps(kPhaseLogits, s);
    hipLaunchKernelGGL(k_logits<T>, dim3((unsigned)(la.nvt * la.nct)), dim3(kThreads), 0, s, la);
  }

  {
    ProfScope ps(kPhaseLse, s);
    hipLaunchKernelGGL(k_lse, dim3((unsigned)((rows + 3) / 4)), dim3(256), 0, s, part, L.nvt, zt, yc, ign, rows, lse,
                       rowloss + c0);
  }
  {
    ProfScope ps(kPhaseGrad, s);
    hipLaunchKernelGGL(k_grad<T>, dim3((unsigned)rows), dim3(256), 0, s, z, L.ldz, V, lse, part, L.nvt, yc, ign,
                       nvalid);
  }

  // dX = G W
  DxArgs<T> da;
  da.G = Operand<T>{z, L.ldz, rows, L.ldz};
  da.W = Operand<T>{W, H, V, H};
  da.V = V;
  da.H = H;
  da.rows = rows;
  da.nmt = (rows + kTile - 1) / kTile;
  da.nnt = (H + kTile - 1) / kTile;
  const int64_t ks = kStageK<T>;
  da.ksplit = ((V + L.splits - 1) / L.splits + ks - 1) / ks * ks;
  const int64_t splits = (V + da.ksplit - 1) / da.ksplit;
  da.dx = dX + c0 * H;
  da.part = reinterpret_cast<float*>(ws + L.off_dxpart);
  {
    ProfScope ps(kPhaseDx, s);
    hipLaunchKernelGGL(k_dx<T>, dim3((unsigned)(da.nmt * da.nnt), (unsigned)splits), dim3(kThreads), 0, s, da);
  }
  if (splits > 1) {
    const int64_t n = rows * H;
    int64_t blocks = (n + 255) / 256;
    if (blocks > 8192) blocks = 8192;
    ProfScope ps(kPhaseDxReduce, s);
    hipLaunchKernelGGL(k_dx_reduce<T>, dim3((unsigned)blocks), dim3(256), 0, s, da.part, splits, n, da.dx);
  }

  // dW (+)= G^T X_chunk
  DwArgs<T> wa;
  wa.G = Operand<T>{z, L.ldz, rows, L.ldz};
  wa.X = Operand<T>{Xc, H, rows, H};
  wa.V = V;
  wa.H = H;
  wa.rows = rows;
  wa.nvt = L.nvt;
  wa.nht = (H + kTile - 1) / kTile;
  wa.dw = dW;
  wa.first = first ? 1 : 0;
  {
    ProfScope ps(kPhaseDw, s);
    hipLaunchKernelGGL(k_dw<T>, dim3((unsigned)(wa.nvt * wa.nht)), dim3(kThreads), 0, s, wa);
  }
  return hipGetLastError();
}

hipError_t launch_flce_chunk(const Layout& L, const void* X, const void* W, const int64_t* y, int64_t ign, int64_t c0,
                             int64_t rows, char* ws, float* rowloss, void* dX, float* dW, bool first, hipStream_t s) {
  if (L.dtype == 1)
    return chunk_impl<__bf16>(L, static_cast<const __bf16*>(X), static_cast<const __bf16*>(W), y, ign, c0, rows, ws,
                              rowloss, static_cast<__bf16*>(dX), dW, first, s);
  return chunk_impl<float>(L, static_cast<const float*>(X), static_cast<const float*>(W), y, ign, c0, rows, ws,
                           rowloss, static_cast<float*>(dX), dW, first, s);
}

}  // namespace flce
