// MFMA tile GEMM building blocks for gfx950 (CDNA4), shared by the three
// contractions of fused linear + cross-entropy:
//   logits   Z^T[v,c] = sum_h W[v,h] X[c,h]     (both operands K-contiguous)
//   dX       dX[c,h]  = sum_v G[c,v] W[v,h]     (W read K-major)
//   dW       dW[v,h] += sum_c G[c,v] X[c,h]     (G read K-major; bf16 X from a
//                                                 transposed copy, K-contiguous)
//
// A workgroup of 256 threads (4 wave64s, 2 x 2) owns a 256 x 256 output tile;
// each wave owns 128 x 128 = 4 x 4 MFMA 32x32 blocks (16 fp32 accumulators
// per lane per block, held in the AGPRs).  K advances 128 bytes per stage
// (64 bf16 or 32 fp32); one operand's tile of one stage is 32 KiB of LDS.
//
// bf16 operands use the direct-to-LDS pipeline of namespace `pipe` below
// (copies straight from HBM into a ring of five 32 KiB LDS slabs, all 160 KiB
// of gfx950 LDS; transposing LDS reads for K-major operands).  fp32 operands
// use the double-buffered (2 stages x 2 operands, 128 KiB) register-staged
// loop that follows here:
// each stage is loaded into registers (K-contiguous operands chunk by chunk;
// K-major ones as 4 x 4 blocks transposed in registers) and written to LDS
// "row-major in K" -- tile row r (an M or N index) is 128 bytes of consecutive
// K in eight 16-byte chunks, chunk c at slot (c ^ r ^ (r >> 3)) & 7, free of
// bank conflicts for the row-wise fragment reads and the transposing writes.
//
// MFMA operand mapping: for v_mfma_f32_32x32x16_bf16 lane l feeds row
// (l % 32) of its operand with the 8 K values of chunk (2 s + l / 32) of the
// current 64-deep stage (s = 0..3).  A and B use the same K assignment, so
// the contraction is exact whatever order the hardware sums the K slots in.
// The fp32 path issues four v_mfma_f32_32x32x2f32 per chunk pair, element t
// of each lane's chunk feeding the t-th instruction.  Accumulator element e of
// lane l is output row 8 (e / 4) + 4 (l / 32) + e % 4, column l % 32.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>
#include <utility>

#include "flce_host.h"

namespace flce {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x2 __attribute__((ext_vector_type(2)));

constexpr int kThreads = 256;                   // 4 waves
constexpr int kOpBytes = kTile * kRowBytes;     // one operand, one stage: 32 KiB
constexpr int kStageBytes = 2 * kOpBytes;       // A + B
constexpr int kLdsBytes = 2 * kStageBytes;      // double buffered: 128 KiB

template <typename T>
struct Elem;
template <>
struct Elem<__bf16> {
  static constexpr int chunk = 8;               // elements per 16-byte chunk
};
template <>
struct Elem<float> {
  static constexpr int chunk = 4;
};
template <typename T>
constexpr int kStageK = kRowBytes / (int)sizeof(T);  // K elements per stage

// One GEMM operand as it lies in HBM.  For a K-contiguous operand, memory
// rows are M (or N) indices and memory columns are K; for a K-major one the
// other way round.  `rows` bounds the memory rows that may be read; `cols`
// bounds the K extent of a K-contiguous operand (chunks starting at or past
// it read as zero).  Reads past the operand's last valid element return zero
// (buffer range checking); other reads past `cols` in a K-major operand land
// on M/N indices whose outputs are never stored.
template <typename T>
struct Operand {
  const T* base;
  int64_t ld;    // elements between consecutive memory rows
  int64_t rows;  // valid memory rows
  int64_t cols;  // valid memory columns
};

typedef __amdgpu_buffer_rsrc_t Rsrc;

// Buffer resource over [base, base + bytes): loads at or past `bytes` read 0,
// stores there are dropped.  Only byte offsets below 2^31 are ever used.
// Callers pass workgroup-uniform values; readfirstlane makes that explicit so
// the resource always lives in scalar registers.
__device__ __forceinline__ Rsrc make_rsrc(const void* base, int64_t bytes) {
  const int64_t n = bytes <= 0 ? 0 : (bytes > 0x7fffffff ? 0x7fffffff : bytes);
  const uint64_t p = reinterpret_cast<uint64_t>(base);
  const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)p);
  const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(p >> 32));
  const int nn = __builtin_amdgcn_readfirstlane((int)n);
  void* q = reinterpret_cast<void*>(((uint64_t)hi << 32) | lo);
  return __builtin_amdgcn_make_buffer_rsrc(q, (short)0, nn, 0x00020000);
}

__device__ __forceinline__ u32x4 bload16(Rsrc r, uint32_t voff, uint32_t soff) {
  return __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(r, (int)voff, (int)soff, 0));
}

__device__ __forceinline__ uint32_t lds_off(uint32_t r, uint32_t c) {
  return r * kRowBytes + (((c ^ r ^ (r >> 3)) & 7u) << 4);
}

// ---- global -> registers -------------------------------------------------

// K-contiguous operand, view of one 256-row tile: thread t loads chunk t % 8
// of rows t / 8 + 32 i (i = 0..7) at each stage.
template <typename T>
struct KContigLoader {
  Rsrc r;
  uint32_t voff;     // this thread's byte offset within the tile
  uint32_t row32;    // bytes between rows t / 8 + 32 i and + 32 (i + 1)
  int64_t kchunk;    // this thread's K offset within a stage (elements)
  int64_t kend;      // K bound

  __device__ __forceinline__ void init(const Operand<T>& op, int64_t mn0, int tid) {
    const int64_t nrows = op.rows - mn0 < kTile ? op.rows - mn0 : kTile;
    r = make_rsrc(op.base + mn0 * op.ld, nrows * op.ld * (int64_t)sizeof(T));
    voff = (uint32_t)(((tid >> 3) * op.ld + (tid & 7) * Elem<T>::chunk) * (int64_t)sizeof(T));
    row32 = (uint32_t)(32 * op.ld * (int64_t)sizeof(T));
    kchunk = (tid & 7) * Elem<T>::chunk;
    kend = op.cols;
  }
  __device__ __forceinline__ void load(u32x4 (&st)[8], int64_t k0) const {
    const uint32_t soff = (uint32_t)(k0 * (int64_t)sizeof(T));
    // chunks past the K bound: an offset past every resource's range reads 0
    const uint32_t v = k0 + kchunk < kend ? voff : 0x80000000u;
#pragma unroll
    for (int i = 0; i < 8; ++i) st[i] = bload16(r, v + i * row32, soff);
  }
};

// K-major operand.  bf16: thread t loads the 8 x 8 block at K rows
// 8 (t / 32) + j, MN columns 8 (t % 32) ..; fp32: the 4 x 4 blocks at K rows
// 4 (t / 64 + 4 i) + j, MN columns 4 (t % 64) .. (i = 0, 1).  The resource is
// rebuilt per stage from (k0, mn0), so offsets stay within one stage.
template <typename T>
struct KMajorLoader {
  const T* base;
  int64_t ld, rows, cols, mn0;
  uint32_t voff;

  __device__ __forceinline__ void init(const Operand<T>& op, int64_t mn0_, int tid) {
    base = op.base;
    ld = op.ld;
    rows = op.rows;
    cols = op.cols;
    mn0 = mn0_;
    if constexpr (sizeof(T) == 2)
      voff = (uint32_t)((8 * (tid >> 5) * ld + 8 * (tid & 31)) * (int64_t)sizeof(T));
    else
      voff = (uint32_t)((4 * (tid >> 6) * ld + 4 * (tid & 63)) * (int64_t)sizeof(T));
  }
  __device__ __forceinline__ void load(u32x4 (&st)[8], int64_t k0) const {
    // valid bytes from (k0, mn0) to the end of the last valid row's columns
    const int64_t nb = rows > k0 ? ((rows - k0 - 1) * ld + (cols - mn0)) * (int64_t)sizeof(T) : 0;
    const Rsrc r = make_rsrc(base + k0 * ld + mn0, nb);
    const uint32_t rowb = (uint32_t)(ld * (int64_t)sizeof(T));
    if constexpr (sizeof(T) == 2) {
#pragma unroll
      for (int j = 0; j < 8; ++j) st[j] = bload16(r, voff, j * rowb);
    } else {
#pragma unroll
      for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) st[4 * i + j] = bload16(r, voff, (16 * i + j) * rowb);
    }
  }
};

// ---- registers -> LDS ------------------------------------------------------

__device__ __forceinline__ void store_kcontig(char* lds, const u32x4 (&st)[8], int tid) {
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const int q = tid + kThreads * i;
    *reinterpret_cast<u32x4*>(lds + lds_off(q >> 3, q & 7)) = st[i];
  }
}

template <typename T>
__device__ __forceinline__ void store_kmajor(char* lds, const u32x4 (&st)[8], int tid);

template <>
__device__ __forceinline__ void store_kmajor<float>(char* lds, const u32x4 (&st)[8], int tid) {
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const int b = tid + kThreads * i;
    const int mc = b & 63, kb = b >> 6;
#pragma unroll
    for (int p = 0; p < 4; ++p) {
      const u32x4 o = {st[4 * i][p], st[4 * i + 1][p], st[4 * i + 2][p], st[4 * i + 3][p]};
      *reinterpret_cast<u32x4*>(lds + lds_off(mc * 4 + p, kb)) = o;
    }
  }
}

// ---- MFMA on one stage -------------------------------------------------------

template <typename T>
__device__ __forceinline__ f32x16 mma_chunk(u32x4 a, u32x4 b, f32x16 c);

template <>
__device__ __forceinline__ f32x16 mma_chunk<__bf16>(u32x4 a, u32x4 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a), __builtin_bit_cast(bf16x8, b),
                                                 c, 0, 0, 0);
}

template <>
__device__ __forceinline__ f32x16 mma_chunk<float>(u32x4 a, u32x4 b, f32x16 c) {
  const f32x4 af = __builtin_bit_cast(f32x4, a), bf = __builtin_bit_cast(f32x4, b);
  c = __builtin_amdgcn_mfma_f32_32x32x2f32(af.x, bf.x, c, 0, 0, 0);
  c = __builtin_amdgcn_mfma_f32_32x32x2f32(af.y, bf.y, c, 0, 0, 0);
  c = __builtin_amdgcn_mfma_f32_32x32x2f32(af.z, bf.z, c, 0, 0, 0);
  c = __builtin_amdgcn_mfma_f32_32x32x2f32(af.w, bf.w, c, 0, 0, 0);
  return c;
}

// One stage = 4 steps of 16 bf16 (8 fp32) K values.  The fragments of step
// s + 1 are read from LDS while the 16 MFMAs of step s run.
__device__ __forceinline__ void read_frags(const char* ldsA, const char* ldsB, u32x4 (&a)[4], u32x4 (&b)[4], int wy,
                                           int wx, int lane, int s) {
  const int c = 2 * s + (lane >> 5);
#pragma unroll
  for (int i = 0; i < 4; ++i) a[i] = *reinterpret_cast<const u32x4*>(ldsA + lds_off(wy * 128 + 32 * i + (lane & 31), c));
#pragma unroll
  for (int j = 0; j < 4; ++j) b[j] = *reinterpret_cast<const u32x4*>(ldsB + lds_off(wx * 128 + 32 * j + (lane & 31), c));
}

template <typename T>
__device__ __forceinline__ void mma_stage(const char* ldsA, const char* ldsB, f32x16 (&acc)[4][4], int wy,
                                          int wx, int lane) {
  u32x4 a[2][4], b[2][4];
  read_frags(ldsA, ldsB, a[0], b[0], wy, wx, lane, 0);
#pragma unroll
  for (int s = 0; s < 4; ++s) {
    if (s < 3) read_frags(ldsA, ldsB, a[(s + 1) & 1], b[(s + 1) & 1], wy, wx, lane, s + 1);
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j) acc[i][j] = mma_chunk<T>(a[s & 1][i], b[s & 1][j], acc[i][j]);
  }
}

// ---- the main loop -----------------------------------------------------------

template <typename T, bool kKMajor>
__device__ __forceinline__ void store_op(char* lds, const u32x4 (&st)[8], int tid) {
  if constexpr (kKMajor)
    store_kmajor<T>(lds, st, tid);
  else
    store_kcontig(lds, st, tid);
}

template <typename T, bool kKMajor>
using LoaderOf = typename std::conditional<kKMajor, KMajorLoader<T>, KContigLoader<T>>::type;

// acc = A[m0:m0+256, k0:k1] * B[n0:n0+256, k0:k1]^T.  The stages cover
// [k0, k0 + KS * ceil((k1 - k0) / KS)); the caller makes the K extent past
// k1 read as zero (operand bounds) or lets it land on zero padding.
template <typename T, bool kAKMajor, bool kBKMajor>
__device__ __forceinline__ void mainloop_regstage(char* smem, const Operand<T>& A, int64_t m0, const Operand<T>& B,
                                              int64_t n0, int64_t k0, int64_t k1, f32x16 (&acc)[4][4]) {
  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int wy = wave >> 1, wx = wave & 1;
  constexpr int KS = kStageK<T>;
  const int nk = (int)((k1 - k0 + KS - 1) / KS);

#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = f32x16{};
  if (nk <= 0) return;

  LoaderOf<T, kAKMajor> la;
  LoaderOf<T, kBKMajor> lb;
  la.init(A, m0, tid);
  lb.init(B, n0, tid);
  u32x4 sa[8], sb[8];
  la.load(sa, k0);
  lb.load(sb, k0);
  store_op<T, kAKMajor>(smem, sa, tid);
  store_op<T, kBKMajor>(smem + kOpBytes, sb, tid);
  __syncthreads();

  for (int kt = 0; kt < nk; ++kt) {
    char* cur = smem + (kt & 1) * kStageBytes;
    char* nxt = smem + ((kt + 1) & 1) * kStageBytes;
    const bool more = kt + 1 < nk;
    if (more) {
      const int64_t kn = k0 + (int64_t)(kt + 1) * KS;
      la.load(sa, kn);
      lb.load(sb, kn);
    }
    mma_stage<T>(cur, cur + kOpBytes, acc, wy, wx, lane);
    if (more) {
      store_op<T, kAKMajor>(nxt, sa, tid);
      store_op<T, kBKMajor>(nxt + kOpBytes, sb, tid);
    }
    __syncthreads();
  }
}

// ---- bf16 pipelined main loop -------------------------------------------------
//
// Global -> LDS copies go straight into LDS (buffer_load ... lds, 16 bytes per
// lane; a wave's instruction fills 1 KiB of LDS in lane order).  A stage is
// 64 bf16 of K, so every tile row of a K-contiguous operand is one whole
// 128-byte segment per stage: the L2 serves it as one 128-byte request (32 of
// K would be a 64-byte request, and the request rate, not bytes, is what
// limits these copies).  Two stages of 64 KiB: the copy of stage k + 2 starts
// as soon as everyone is done reading stage k and lands while stage k + 1 is
// multiplied.  Tiles in LDS:
//   K-contiguous operand: 256 rows x 128 bytes; 16-byte chunk c of row r at
//     slot c ^ ((r' >> 1) ^ (r' >> 4)) & 7, r' = r % 32 (the copying lane picks
//     the chunk that belongs at its slot).  Fragments: ds_read_b128.
//   K-major operand: 64 K rows x 512 bytes (256 MN values); 32-byte segment
//     s of K row k at position s ^ {0, 2, 5, 7}[k % 4].  Fragments: two
//     ds_read_b64_tr_b16, which hand lane i of each 16-lane group element t
//     of the 8 bytes read by lane 4 t + i / 4 of that group (so lane 4 t + q
//     points at K row t, MN columns 4 q .. 4 q + 3, and lane i receives MN
//     column i for four consecutive K rows).
// Both swizzles keep fragment reads free of LDS bank conflicts (measured with
// the SQ_LDS_BANK_CONFLICT counter).
// Each stage is four 16-MFMA steps; the fragments of step s + 1 are read
// while step s multiplies.  One barrier per stage, before its last step.
namespace pipe {

constexpr int kBK = 64;           // bf16 K per stage
constexpr int kRowB = 128;        // bytes per K-contiguous tile row per stage
constexpr int kOp = 256 * kRowB;  // 32 KiB per operand per stage
constexpr int kSlab = kOp;        // LDS ring slot: one operand tile of one stage
constexpr int kSlabs = 5;
constexpr int kRingBytes = kSlabs * kSlab;  // 160 KiB, all of the gfx950 LDS
constexpr int kLoads = 8;         // 1 KiB copies per wave per operand per stage

typedef __attribute__((address_space(3))) void* lds_void;
typedef short i16x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ uint32_t kc_sw(uint32_t r) { return ((r >> 1) ^ (r >> 4)) & 7u; }
__device__ __forceinline__ uint32_t kc_off(uint32_t r, uint32_t c) {
  return r * kRowB + (((c ^ kc_sw(r & 31u)) & 7u) << 4);
}
__device__ __forceinline__ uint32_t km_sw(uint32_t k) { return (0x7520u >> (4 * (k & 3u))) & 15u; }
__device__ __forceinline__ uint32_t km_off(uint32_t k, uint32_t n) {
  return k * 512u + ((((n >> 4) ^ km_sw(k)) & 15u) << 5) + ((n & 15u) << 1);
}

// Buffer resource as four scalar words (for the inline-asm copies below).
__device__ __forceinline__ u32x4 rsrc_words(const void* base, int64_t bytes) {
  const int64_t n = bytes <= 0 ? 0 : (bytes > 0x7fffffff ? 0x7fffffff : bytes);
  const uint64_t p = reinterpret_cast<uint64_t>(base);
  const uint32_t lo = (uint32_t)__builtin_amdgcn_readfirstlane((uint32_t)p);
  const uint32_t hi = (uint32_t)__builtin_amdgcn_readfirstlane((uint32_t)(p >> 32)) & 0xffffu;
  const uint32_t nr = (uint32_t)__builtin_amdgcn_readfirstlane((uint32_t)n);
  return u32x4{lo, hi, nr, 0x00020000u};
}

// 16 bytes per lane from the buffer straight into LDS at lds + 16 * lane.
// Written as inline asm so that the compiler does not add its own
// conservative "wait for every outstanding load" before later LDS reads: the
// pipeline places the waits itself (wait_vm), also in inline asm.  The
// bounds check of a raw buffer covers the VGPR offset, so every offset that
// can leave the operand lives there; the scalar offset only carries k0.
// m0 (the LDS destination) is set inside the same asm statement, so nothing
// here relies on it surviving; hipcc warns that it may not preserve a
// clobbered m0 for its own code, and the kernels' generated code writes and
// reads m0 only in these statements.
__device__ __forceinline__ void dma16(u32x4 r, uint32_t lds_addr, uint32_t voff, uint32_t soff) {
  asm volatile("s_mov_b32 m0, %0\n\tbuffer_load_dwordx4 %1, %2, %3 offen lds"
               :
               : "s"(lds_addr), "v"(voff), "s"(r), "s"(soff)
               : "memory", "m0");
}

// LDS byte address of a pointer into a __shared__ array, as a scalar
__device__ __forceinline__ uint32_t lds_addr(const char* p) {
  return (uint32_t)__builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)(lds_void)p);
}

// K-contiguous operand, one 256-row tile.  Copy q of wave w fills rows
// 8 w + 32 q .. + 7; lane i fills row 8 w + 32 q + i / 8, slot i % 8.
struct KcLoader {
  u32x4 r;
  uint32_t voff[kLoads];
  uint32_t kch;  // K offset (elements) of this lane's chunk, the same for every copy
  int64_t kend;
  __device__ __forceinline__ void init(const Operand<__bf16>& op, int64_t mn0, int wave, int lane) {
    const int64_t nrows = op.rows - mn0 < kTile ? op.rows - mn0 : kTile;
    r = rsrc_words(op.base + mn0 * op.ld, nrows * op.ld * 2);
    kend = op.cols;
    const uint32_t row = 8 * wave + (lane >> 3);  // < 32: the swizzle is that of every copy's row
    const uint32_t c = ((lane & 7) ^ kc_sw(row)) & 7u;
    kch = 8 * c;
#pragma unroll
    for (int q = 0; q < kLoads; ++q) voff[q] = (uint32_t)(((row + 32 * q) * op.ld + 8 * c) * 2);
  }
  // the copies of the stage starting at K offset k0; `more` false: every
  // lane reads out of bounds and the copies write zeros
  struct Stage {
    uint32_t soff;
    bool in;
  };
  __device__ __forceinline__ Stage stage(int64_t k0, bool more) const {
    return Stage{(uint32_t)(k0 * 2), more && (k0 + kBK <= kend || k0 + kch < kend)};
  }
  // copy q of this wave into the operand tile at LDS byte address `tile`
  __device__ __forceinline__ void issue(const Stage& st, uint32_t tile, int q, int wave) const {
    dma16(r, tile + 1024 * wave + 4096 * q, st.in ? voff[q] : 0x80000000u, st.soff);
  }
  __device__ __forceinline__ u32x4 frag(const char* tile, int row, int c) const {
    return *reinterpret_cast<const u32x4*>(tile + kc_off(row, c));
  }
};

// K-major operand (memory rows are K): copy q of wave w fills K rows
// 2 w + 8 q and 2 w + 8 q + 1; lane i fills K row 2 w + 8 q + i / 32, 16
// bytes at position (i % 32) / 2, half i % 2.
struct KmLoader {
  const __bf16* base;
  int64_t ld, rows, cols, mn0;
  uint32_t voff[kLoads];
  __device__ __forceinline__ void init(const Operand<__bf16>& op, int64_t mn0_, int wave, int lane) {
    base = op.base;
    ld = op.ld;
    rows = op.rows;
    cols = op.cols;
    mn0 = mn0_;
    const uint32_t k = 2 * wave + (lane >> 5);  // k % 4, hence the swizzle, is that of every copy
    const uint32_t seg = (((lane & 31) >> 1) ^ km_sw(k)) & 15u;
#pragma unroll
    for (int q = 0; q < kLoads; ++q) voff[q] = (uint32_t)(((k + 8 * q) * ld + 16 * seg + 8 * (lane & 1)) * 2);
  }
  // One resource per stage, starting at K row k0: it ends at the last element
  // of the operand, so K rows past it and MN columns past it on the last K
  // row read as zero (MN columns past the tile edge on earlier rows feed only
  // outputs that are never stored).  `more` false: an empty resource, zeros.
  struct Stage {
    u32x4 r;
  };
  __device__ __forceinline__ Stage stage(int64_t k0, bool more) const {
    const int64_t nb = (more && rows > k0) ? ((rows - k0 - 1) * ld + (cols - mn0)) * 2 : 0;
    return Stage{rsrc_words(base + (more ? k0 * ld + mn0 : 0), nb)};
  }
  __device__ __forceinline__ void issue(const Stage& st, uint32_t tile, int q, int wave) const {
    dma16(st.r, tile + 1024 * wave + 4096 * q, voff[q], 0);
  }
  // fragment of MN columns nb .. nb + 31, K rows 16 s + 8 (lane / 32) .. + 7
  __device__ __forceinline__ u32x4 frag(const char* tile, int nb, int s, int lane) const {
    const uint32_t g = lane >> 4, q = lane & 3, t = (lane >> 2) & 3;
    const uint32_t n = nb + 16 * (g & 1) + 4 * q;
    const uint32_t k = 16 * s + 8 * (g >> 1) + t;
    const i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) i16x4*)(tile + km_off(k, n)));
    const i16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) i16x4*)(tile + km_off(k + 4, n)));
    const uint2 a = __builtin_bit_cast(uint2, lo), b = __builtin_bit_cast(uint2, hi);
    return u32x4{a.x, a.y, b.x, b.y};
  }
};

template <bool kKMajor>
using LoaderT = typename std::conditional<kKMajor, KmLoader, KcLoader>::type;

// this wave's four fragments of step s (16 of K) of one operand tile: rows
// (or columns) w 128 + 32 i .. + 31
template <bool kKMajor>
__device__ __forceinline__ void load_frags(const LoaderT<kKMajor>& l, const char* tile, int s, int w, int lane,
                                           u32x4 (&f)[4]) {
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    if constexpr (kKMajor)
      f[i] = l.frag(tile, w * 128 + 32 * i, s, lane);
    else
      f[i] = l.frag(tile, w * 128 + 32 * i + (lane & 31), 2 * s + (lane >> 5));
  }
}

// fragment i of load_frags alone
template <bool kKMajor>
__device__ __forceinline__ void load_frag1(const LoaderT<kKMajor>& l, const char* tile, int s, int w, int lane, int i,
                                           u32x4& f) {
  if constexpr (kKMajor)
    f = l.frag(tile, w * 128 + 32 * i, s, lane);
  else
    f = l.frag(tile, w * 128 + 32 * i + (lane & 31), 2 * s + (lane >> 5));
}

// s_waitcnt vmcnt(N): at most N of this wave's copies still in flight
template <int N>
__device__ __forceinline__ void wait_vm() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  asm volatile("s_waitcnt vmcnt(%0)" : : "n"(N) : "memory");
}

// At most N of this wave's copies in flight and its LDS reads done, then the
// workgroup barrier.  No compiler fence: __syncthreads() would also wait for
// the copies issued after the ones this barrier is for.
template <int N>
__device__ __forceinline__ void wait_barrier() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  asm volatile("s_waitcnt vmcnt(%0) lgkmcnt(0)\n\ts_barrier" : : "n"(N) : "memory");
}

__device__ __forceinline__ uint32_t mod5(uint32_t x) { return x >= 5 ? x - 5 : x; }

// A main-loop hook that does nothing.  A hook that is active() takes part in
// the first kStages stages of the loop, which are then unrolled so that the
// stage number Q is a compile-time constant (accumulator blocks can only be
// named by constant indices without spilling them): issue<Q>() runs at the
// start of stage Q, before any of its copies, and apply<Q>(acc) right after
// its barrier, before its last 16 MFMAs.  The barrier waits for every memory
// operation of this wave but the eight copies issued after issue<Q>(), so
// loads issued there have landed when apply runs (their registers must be
// passed through an empty asm after the barrier, so that the compiler reads
// them only from there on).  An active hook needs at least kStages + 1
// stages.
struct NoHook {
  static constexpr int kStages = 0;
  __device__ __forceinline__ bool active() const { return false; }
  template <int Q>
  __device__ __forceinline__ void issue() {}
  template <int Q>
  __device__ __forceinline__ void apply(f32x16 (&)[4][4]) {}
};

template <class F, int... Q>
__device__ __forceinline__ void unroll_stages(F&& f, std::integer_sequence<int, Q...>) {
  (f(std::integral_constant<int, Q>{}), ...);
}

// One tile's pass over K.  LDS holds five 32 KiB operand slabs in a ring:
// stage k's A tile sits in slab 2k mod 5, its B tile in slab 2k + 1 mod 5.
// While stage k is multiplied, stage k + 1 is in flight or landed, and
//   * A of stage k + 2 goes to the slab B of stage k - 1 left, its eight
//     copies per wave spread over steps 0..2 of stage k (3, 3, 2);
//   * B of stage k + 2 goes to the slab A of stage k leaves, one copy per
//     two MFMAs of step 3, after the stage's only barrier.
// So one stage's copies are spread over the whole stage instead of bunched
// into its last step, and the in-order copy counter lets each wave wait for
// exactly the stage it needs (the newest eight copies stay in flight).  The
// copies are inline asm, placed by scheduling barriers: with the compiler's
// own LDS-copy builtin it would wait for every copy before each transposing
// LDS read.  Each step's fragment reads are split, the A half before the
// step's MFMAs and the B half after eight of them, so no more than 8 (K-
// contiguous) or 16 (K-major) LDS reads are outstanding at a time.
// Copies past the last stage read nothing and write zeros into free slabs.
template <bool kAKMajor, bool kBKMajor, class Hook>
__device__ __forceinline__ void mainloop(char* smem, const Operand<__bf16>& A, int64_t m0, const Operand<__bf16>& B,
                                         int64_t n0, int64_t k0, int64_t k1, f32x16 (&acc)[4][4], Hook& hook) {
  const int lane = threadIdx.x & 63, wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int wy = wave >> 1, wx = wave & 1;
  LoaderT<kAKMajor> la;
  LoaderT<kBKMajor> lb;
  la.init(A, m0, wave, lane);
  lb.init(B, n0, wave, lane);
  int nk = (int)((k1 - k0 + kBK - 1) / kBK);
  if (nk < 0) nk = 0;
  const uint32_t lds0 = lds_addr(smem);
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = f32x16{};
  if (nk <= 0) return;
  {
    const auto a0 = la.stage(k0, true);
    const auto b0 = lb.stage(k0, true);
    const auto a1 = la.stage(k0 + kBK, nk > 1);
    const auto b1 = lb.stage(k0 + kBK, nk > 1);
#pragma unroll
    for (int q = 0; q < kLoads; ++q) la.issue(a0, lds0, q, wave);
#pragma unroll
    for (int q = 0; q < kLoads; ++q) lb.issue(b0, lds0 + kSlab, q, wave);
#pragma unroll
    for (int q = 0; q < kLoads; ++q) la.issue(a1, lds0 + 2 * kSlab, q, wave);
#pragma unroll
    for (int q = 0; q < kLoads; ++q) lb.issue(b1, lds0 + 3 * kSlab, q, wave);
  }
  wait_barrier<2 * kLoads>();  // stage 0 is in

  // Where the next step's fragments are read within a step: all four of
  // an operand at once (A before the step's MFMAs, B after eight of them),
  // or, when only B is K-major (the dW product), one fragment before each of
  // MFMAs 0..3 (A) and kSpreadB..kSpreadB+3 (B).  Measured on the three
  // products: spreading the reads makes dW 1.6% faster and logits 1.1% slower.
  constexpr bool kSpreadReads = kBKMajor && !kAKMajor;
  constexpr int kSpreadB = 8;
  u32x4 fa[2][4], fb[2][4];
  uint32_t sa = 0;  // slab of A for the current stage
  load_frags<kAKMajor>(la, smem, 0, wy, lane, fa[0]);
  load_frags<kBKMajor>(lb, smem + kSlab, 0, wx, lane, fb[0]);
  // one stage with a next stage; Q >= 0: the hook's stage Q (= kt)
  auto stage = [&](int kt, auto qc) {
    constexpr int Q = decltype(qc)::value;
    if constexpr (Q >= 0) hook.template issue<Q>();
    const char* ta = smem + sa * kSlab;
    const char* tb = smem + mod5(sa + 1) * kSlab;
    const bool more = kt + 2 < nk;
    const int64_t kn = k0 + (int64_t)(kt + 2) * kBK;
    const auto sta = la.stage(kn, more);
    const uint32_t dsta = lds0 + mod5(sa + 4) * kSlab;
#pragma unroll
    for (int s = 0; s < 3; ++s) {
      if constexpr (!kSpreadReads) load_frags<kAKMajor>(la, ta, s + 1, wy, lane, fa[(s + 1) & 1]);
      __builtin_amdgcn_sched_barrier(0);
      const int nq = s < 2 ? 3 : 2;
#pragma unroll
      for (int u = 0; u < 16; ++u) {
        if constexpr (kSpreadReads) {
          if (u < 4 || (u >= kSpreadB && u < kSpreadB + 4)) {
            __builtin_amdgcn_sched_barrier(0);
            if (u < 4)
              load_frag1<kAKMajor>(la, ta, s + 1, wy, lane, u, fa[(s + 1) & 1][u]);
            else
              load_frag1<kBKMajor>(lb, tb, s + 1, wx, lane, u - kSpreadB, fb[(s + 1) & 1][u - kSpreadB]);
            __builtin_amdgcn_sched_barrier(0);
          }
        } else if (u == 8) {
          __builtin_amdgcn_sched_barrier(0);
          load_frags<kBKMajor>(lb, tb, s + 1, wx, lane, fb[(s + 1) & 1]);
          __builtin_amdgcn_sched_barrier(0);
        }
        acc[u >> 2][u & 3] = mma_chunk<__bf16>(fa[s & 1][u >> 2], fb[s & 1][u & 3], acc[u >> 2][u & 3]);
        if ((u == 3 || u == 8 || u == 13) && (u - 3) / 5 < nq) {
          __builtin_amdgcn_sched_barrier(0);
          la.issue(sta, dsta, 3 * s + (u - 3) / 5, wave);
          __builtin_amdgcn_sched_barrier(0);
        }
      }
      __builtin_amdgcn_sched_barrier(0);
    }
    // all but this stage's eight A copies landed, so stage kt + 1 is in;
    // after the barrier nobody reads stage kt any more
    wait_barrier<kLoads>();
    if constexpr (Q >= 0) hook.template apply<Q>(acc);
    const uint32_t sn = mod5(sa + 2);
    load_frags<kAKMajor>(la, smem + sn * kSlab, 0, wy, lane, fa[0]);
    load_frags<kBKMajor>(lb, smem + mod5(sn + 1) * kSlab, 0, wx, lane, fb[0]);
    __builtin_amdgcn_sched_barrier(0);
    const auto stb = lb.stage(kn, more);
    const uint32_t dstb = lds0 + sa * kSlab;
#pragma unroll
    for (int u = 0; u < 16; ++u) {
      acc[u >> 2][u & 3] = mma_chunk<__bf16>(fa[1][u >> 2], fb[1][u & 3], acc[u >> 2][u & 3]);
      if (u & 1) {
        __builtin_amdgcn_sched_barrier(0);
        lb.issue(stb, dstb, u >> 1, wave);
        __builtin_amdgcn_sched_barrier(0);
      }
    }
    __builtin_amdgcn_sched_barrier(0);
    sa = sn;
  };
  // every stage of these loops has a next stage; the last stage follows
  int kt = 0;
  if (hook.active()) {
    unroll_stages([&](auto qc) { stage(kt++, qc); }, std::make_integer_sequence<int, Hook::kStages>{});
  }
  for (; kt + 1 < nk; ++kt) stage(kt, std::integral_constant<int, -1>{});
  {
    const char* ta = smem + sa * kSlab;
    const char* tb = smem + mod5(sa + 1) * kSlab;
#pragma unroll
    for (int s = 0; s < 3; ++s) {
      load_frags<kAKMajor>(la, ta, s + 1, wy, lane, fa[(s + 1) & 1]);
      load_frags<kBKMajor>(lb, tb, s + 1, wx, lane, fb[(s + 1) & 1]);
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int u = 0; u < 16; ++u)
        acc[u >> 2][u & 3] = mma_chunk<__bf16>(fa[s & 1][u >> 2], fb[s & 1][u & 3], acc[u >> 2][u & 3]);
    }
#pragma unroll
    for (int u = 0; u < 16; ++u)
      acc[u >> 2][u & 3] = mma_chunk<__bf16>(fa[1][u >> 2], fb[1][u & 3], acc[u >> 2][u & 3]);
  }
  wait_vm<0>();
  __syncthreads();  // the slabs are free for the caller
}

}  // namespace pipe

static_assert(kLdsBytes <= pipe::kRingBytes, "LDS");
constexpr int kGemmLdsBytes = pipe::kRingBytes;

// Tile-order group size (consecutive tile rows walked column by column).
constexpr int kTileGroup = 8;

// acc = A[m0:m0+256, k0:k1) * B[n0:n0+256, k0:k1)^T: the direct-to-LDS
// pipeline for bf16, the register-staged loop for fp32.  The hook runs inside
// the bf16 loop (see pipe::NoHook); the fp32 loop takes none.
template <typename T, bool kAKMajor, bool kBKMajor, class Hook>
__device__ __forceinline__ void gemm_mainloop(char* smem, const Operand<T>& A, int64_t m0, const Operand<T>& B,
                                              int64_t n0, int64_t k0, int64_t k1, f32x16 (&acc)[4][4], Hook& hook) {
  if constexpr (sizeof(T) == 2)
    pipe::mainloop<kAKMajor, kBKMajor>(smem, A, m0, B, n0, k0, k1, acc, hook);
  else
    mainloop_regstage<T, kAKMajor, kBKMajor>(smem, A, m0, B, n0, k0, k1, acc);
}

template <typename T, bool kAKMajor, bool kBKMajor>
__device__ __forceinline__ void gemm_mainloop(char* smem, const Operand<T>& A, int64_t m0, const Operand<T>& B,
                                              int64_t n0, int64_t k0, int64_t k1, f32x16 (&acc)[4][4]) {
  pipe::NoHook none;
  gemm_mainloop<T, kAKMajor, kBKMajor>(smem, A, m0, B, n0, k0, k1, acc, none);
}

// Tile (tm, tn) of a tm-count x tn-count grid for tile id t, walking groups
// of `group` consecutive tm rows column by column: concurrently running tiles
// then share few A row-blocks and few B column-blocks (L2 reuse).
__device__ __forceinline__ void grouped_tile(int64_t t, int64_t ntm, int64_t ntn, int64_t group, int64_t& tm,
                                             int64_t& tn) {
  const int64_t per_group = group * ntn;
  const int64_t g = t / per_group;
  const int64_t first = g * group;
  const int64_t rows = ntm - first < group ? ntm - first : group;
  const int64_t l = t - g * per_group;
  tm = first + l % rows;
  tn = l / rows;
}

// Work items of one launch handed out at run time (the layout of the items
// over the XCDs is xcd_item in flce_host.h).  Each XCD's range has a counter
// in `head` (kXcds ints, zero at launch).  A workgroup takes the next item of
// its XCD's range; once that range is used up, the next item of another
// XCD's range.  The XCDs do not run equally fast (a few percent apart on the
// same tiles), so with items fixed per XCD the launch lasts as long as the
// slowest; here the faster ones take over the rest of its range.  The launch
// has more workgroups than items (queue_grid); a workgroup that finds every
// range used up gets -1 and returns.  Each item is taken exactly once (one
// atomic increment per take), and an item's result does not depend on which
// workgroup computes it.  Uses the first bytes of `smem` (free before the
// main loop) to hand thread 0's answer to the workgroup; sets `kind`.
__device__ __forceinline__ int64_t take_item(int* head, int64_t n0, int64_t n1, char* smem, int& kind) {
  if (threadIdx.x == 0) {
    const int x = (int)(blockIdx.x % kXcds);
    XcdItem it{-1, 0};
    for (int i = 0; i < kXcds && it.item < 0; ++i) {
      const int y = (x + i) % kXcds;
      it = xcd_item(n0, n1, y, atomicAdd(head + y, 1));
    }
    volatile int* sh = reinterpret_cast<volatile int*>(smem);
    sh[0] = (int)it.item;
    sh[1] = it.kind;
  }
  __syncthreads();
  const volatile int* sh = reinterpret_cast<const volatile int*>(smem);
  const int item = __builtin_amdgcn_readfirstlane(sh[0]);
  kind = __builtin_amdgcn_readfirstlane(sh[1]);
  __syncthreads();
  return item;
}

}  // namespace flce
