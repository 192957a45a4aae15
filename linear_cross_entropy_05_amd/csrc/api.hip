// C-ABI entry points that launch work: the token-chunk schedule of fused
// linear + cross-entropy.  Their argument checks and workspace layouts are in
// host_checks.cpp (plain C++, no device calls).
//
// Schedule of one flce_fwd_bwd call, all on the caller's stream:
//   count N and check targets
//   for each chunk of C tokens:  logits+statistics -> lse -> in-place grad
//                                -> dX rows of the chunk -> dW (+)=
//   loss = sum of token losses / N
// The forward-only entry point (flce_fwd) runs the first three steps of the
// same schedule with no chunk buffer: logits never leave the GEMM epilogue.
// Only one logits chunk exists at a time ("[論文レビュー] Liger Kernel:
// Efficient Triton Kernels for LLM Training", 提案手法: chunked FLCE to bound
// the memory of large-vocabulary logits).
#include <string.h>

#include <atomic>
#include <mutex>

#include "../../include/flce.h"
#include "flce_internal.h"

namespace {

// Per-device answer of "is this a gfx950" (0 unknown, 1 yes, 2 no).  Calls
// from several host threads may fill it at once; each writes the same value.
constexpr int kMaxDevices = 64;
std::atomic<int> g_device_ok[kMaxDevices];

int device_status(int dev) {
  if (dev < 0) return -1;
  if (dev < kMaxDevices) {
    const int known = g_device_ok[dev].load(std::memory_order_relaxed);
    if (known) return known == 1 ? 1 : 0;
  }
  hipDeviceProp_t p;
  if (hipGetDeviceProperties(&p, dev) != hipSuccess) return -1;
  const int ok = strncmp(p.gcnArchName, "gfx950", 6) == 0 ? 1 : 0;
  if (dev < kMaxDevices) g_device_ok[dev].store(ok ? 1 : 2, std::memory_order_relaxed);
  return ok;
}

int current_device_ok() {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess) return -1;
  return device_status(dev);
}

}  // namespace

extern "C" {

int flce_device_supported(int device) { return device_status(device); }

int flce_fwd_bwd(const void* X, const void* W, const int64_t* targets, const float* token_scale, int64_t BT,
                 int64_t H, int64_t V, int64_t ignore_index, int64_t chunk_tokens, int dtype, float* loss,
                 float* row_loss, void* dX, float* dW, void* workspace, size_t workspace_bytes, int32_t* err_flag,
                 void* stream) {
  flce::Layout L;
  const int st = flce::check_fwd_bwd(X, W, targets, token_scale, BT, H, V, chunk_tokens, dtype, loss, row_loss, dX,
                                     dW, workspace, workspace_bytes, err_flag, &L);
  if (st != FLCE_OK) return st;
  if (current_device_ok() != 1) return FLCE_ERR_DEVICE;

  hipStream_t s = static_cast<hipStream_t>(stream);
  char* ws = static_cast<char*>(workspace);
  int32_t* nvalid = reinterpret_cast<int32_t*>(ws + L.off_nvalid);
  float* rl = row_loss ? row_loss : reinterpret_cast<float*>(ws + L.off_rowloss);

  // only the non-ignored tokens go through the chunks, packed in their order
  if (flce::launch_compact(L, targets, ignore_index, ws, err_flag, dX, rl, s) != hipSuccess) return FLCE_ERR_LAUNCH;
  if (BT == 0) {
    if (flce::launch_fill_zero(dW, V * H, s) != hipSuccess) return FLCE_ERR_LAUNCH;
  }
  for (int64_t c0 = 0; c0 < BT; c0 += L.C) {
    const int64_t rows = BT - c0 < L.C ? BT - c0 : L.C;
    if (flce::launch_flce_chunk(L, X, W, targets, token_scale, ignore_index, c0, rows, ws, rl, dX, dW, c0 == 0, s) !=
        hipSuccess)
      return FLCE_ERR_LAUNCH;
  }
  if (flce::launch_loss_final(rl, BT, nvalid, loss, s) != hipSuccess) return FLCE_ERR_LAUNCH;
  return FLCE_OK;
}

int flce_fwd(const void* X, const void* W, const int64_t* targets, int64_t BT, int64_t H, int64_t V,
             int64_t ignore_index, int64_t chunk_tokens, int dtype, float* loss, float* row_loss, void* workspace,
             size_t workspace_bytes, int32_t* err_flag, void* stream) {
  flce::Layout L;
  const int st = flce::check_fwd(X, W, targets, BT, H, V, chunk_tokens, dtype, loss, row_loss, workspace,
                                 workspace_bytes, err_flag, &L);
  if (st != FLCE_OK) return st;
  if (current_device_ok() != 1) return FLCE_ERR_DEVICE;

  hipStream_t s = static_cast<hipStream_t>(stream);
  char* ws = static_cast<char*>(workspace);
  int32_t* nvalid = reinterpret_cast<int32_t*>(ws + L.off_nvalid);
  float* rl = row_loss ? row_loss : reinterpret_cast<float*>(ws + L.off_rowloss);
  if (flce::launch_count_valid(targets, BT, V, ignore_index, nvalid, err_flag, s) != hipSuccess)
    return FLCE_ERR_LAUNCH;
  for (int64_t c0 = 0; c0 < BT; c0 += L.C) {
    const int64_t rows = BT - c0 < L.C ? BT - c0 : L.C;
    if (flce::launch_fwd_chunk(L, X, W, targets, ignore_index, c0, rows, ws, rl, s) != hipSuccess)
      return FLCE_ERR_LAUNCH;
  }
  if (flce::launch_loss_final(rl, BT, nvalid, loss, s) != hipSuccess) return FLCE_ERR_LAUNCH;
  return FLCE_OK;
}

int flce_orpo(const void* X, const void* W, const int64_t* targets, int64_t n_seq, int64_t seq_len, int64_t H,
              int64_t V, int64_t ignore_index, float beta, int64_t chunk_tokens, int dtype, float* loss,
              float* seq_logp, void* dX, float* dW, void* workspace, size_t workspace_bytes, int32_t* err_flag,
              void* stream) {
  flce::OrpoLayout L;
  const int st = flce::check_orpo(X, W, targets, n_seq, seq_len, H, V, chunk_tokens, dtype, loss, seq_logp, dX, dW,
                                  workspace, workspace_bytes, err_flag, &L);
  if (st != FLCE_OK) return st;
  if (current_device_ok() != 1) return FLCE_ERR_DEVICE;

  const int64_t BT = n_seq * seq_len;
  hipStream_t s = static_cast<hipStream_t>(stream);
  char* ws = static_cast<char*>(workspace);
  int32_t* nvalid = reinterpret_cast<int32_t*>(ws + L.off_nvalid);
  if (L.one_pass) {
    // chunks of whole pairs: forward, the pairs' terms and token factors, backward
    const int64_t B = n_seq / 2;
    char* region = ws + L.off_region;
    float* rlc = reinterpret_cast<float*>(ws + L.off_rlc);
    float* wc = reinterpret_cast<float*>(ws + L.off_wc);
    double* seq = reinterpret_cast<double*>(ws + L.off_seq);
    double* pair = reinterpret_cast<double*>(ws + L.off_pair);
    void* xg = ws + L.off_xg;
    int64_t* yg = reinterpret_cast<int64_t*>(ws + L.off_yg);
    void* dxc = ws + L.off_dxc;
    if (flce::launch_count_valid(targets, BT, V, ignore_index, nvalid, err_flag, s) != hipSuccess)
      return FLCE_ERR_LAUNCH;
    // valid tokens of the chosen half (its range check repeats the one above)
    if (flce::launch_count_valid(targets, B * seq_len, V, ignore_index, nvalid + 1, nvalid + 2, s) != hipSuccess)
      return FLCE_ERR_LAUNCH;
    for (int64_t p0 = 0; p0 < B; p0 += L.pairs) {
      const int64_t np = B - p0 < L.pairs ? B - p0 : L.pairs;
      const int64_t rows = 2 * np * seq_len;
      if (flce::launch_orpo_gather(X, targets, H, seq_len, B, p0, np, dtype, xg, yg, s) != hipSuccess ||
          flce::launch_logits_chunk(L.fb, xg, W, yg, ignore_index, 0, rows, region, rlc, s) != hipSuccess ||
          flce::launch_orpo_chunk_stats(rlc, yg, seq_len, B, p0, np, ignore_index, beta, nvalid + 1, wc, seq_logp, seq,
                                        pair, s) != hipSuccess ||
          flce::launch_grad_chunk(L.fb, xg, W, yg, wc, ignore_index, 0, rows, region, dxc, dW, p0 == 0, s) !=
              hipSuccess ||
          flce::launch_orpo_scatter(dxc, H, seq_len, B, p0, np, dtype, dX, s) != hipSuccess)
        return FLCE_ERR_LAUNCH;
    }
    if (flce::launch_orpo_final(seq, pair, B, beta, nvalid + 1, loss, s) != hipSuccess) return FLCE_ERR_LAUNCH;
    return FLCE_OK;
  }
  float* rl = reinterpret_cast<float*>(ws + L.off_rowloss);
  float* scale = reinterpret_cast<float*>(ws + L.off_scale);
  double* scratch = reinterpret_cast<double*>(ws + L.off_scratch);
  char* region = ws + L.off_region;

  if (flce::launch_count_valid(targets, BT, V, ignore_index, nvalid, err_flag, s) != hipSuccess)
    return FLCE_ERR_LAUNCH;
  // token losses (forward only)
  for (int64_t c0 = 0; c0 < BT; c0 += L.fwd.C) {
    const int64_t rows = BT - c0 < L.fwd.C ? BT - c0 : L.fwd.C;
    if (flce::launch_fwd_chunk(L.fwd, X, W, targets, ignore_index, c0, rows, region, rl, s) != hipSuccess)
      return FLCE_ERR_LAUNCH;
  }
  // sequence terms, loss, per-token gradient factors
  if (flce::launch_orpo_stats(rl, targets, n_seq, seq_len, ignore_index, beta, scale, seq_logp, loss, scratch, s) !=
      hipSuccess)
    return FLCE_ERR_LAUNCH;
  // gradients: the fused pass with those factors (its token losses repeat the ones above)
  for (int64_t c0 = 0; c0 < BT; c0 += L.fb.C) {
    const int64_t rows = BT - c0 < L.fb.C ? BT - c0 : L.fb.C;
    if (flce::launch_flce_chunk(L.fb, X, W, targets, scale, ignore_index, c0, rows, region, rl, dX, dW, c0 == 0,
                                s) != hipSuccess)
      return FLCE_ERR_LAUNCH;
  }
  return FLCE_OK;
}

int ce_fwd_bwd_inplace(float* logits, const int64_t* targets, int64_t BT, int64_t V, int64_t ignore_index,
                       float* loss, float* row_loss, void* workspace, size_t workspace_bytes, int32_t* err_flag,
                       void* stream) {
  const int st = flce::check_ce(logits, targets, BT, V, loss, row_loss, workspace, workspace_bytes, err_flag);
  if (st != FLCE_OK) return st;
  if (current_device_ok() != 1) return FLCE_ERR_DEVICE;

  hipStream_t s = static_cast<hipStream_t>(stream);
  char* ws = static_cast<char*>(workspace);
  int32_t* nvalid = reinterpret_cast<int32_t*>(ws);
  float* rl = row_loss ? row_loss : reinterpret_cast<float*>(ws + 256);
  if (flce::launch_count_valid(targets, BT, V, ignore_index, nvalid, err_flag, s) != hipSuccess)
    return FLCE_ERR_LAUNCH;
  if (flce::launch_ce_rows(logits, targets, BT, V, ignore_index, nvalid, rl, s) != hipSuccess)
    return FLCE_ERR_LAUNCH;
  if (flce::launch_loss_final(rl, BT, nvalid, loss, s) != hipSuccess) return FLCE_ERR_LAUNCH;
  return FLCE_OK;
}

// ---- logits-only cross-entropy with no workspace and no allocation ----------

namespace {

// The one scratch array of ce_fwd_bwd_inplace_noalloc: the valid-token count
// (first 256 bytes) and, when the caller passes no row_loss, one float of
// token loss per row.  Each GPU the library runs on holds its own copy for
// the life of the process.
constexpr int64_t kNoAllocMaxRows = (int64_t)1 << 21;
constexpr size_t kNoAllocScratchBytes = 256 + (size_t)kNoAllocMaxRows * 4;
static __device__ __align__(256) char scratch[kNoAllocScratchBytes];

// Device address of `scratch` on each device, looked up once per device with
// that device current (the array's name is only a host-side stand-in).
std::atomic<char*> g_scratch[kMaxDevices];
std::mutex g_scratch_mu;

char* scratch_on(int dev) {
  if (dev < 0 || dev >= kMaxDevices) return nullptr;
  char* p = g_scratch[dev].load(std::memory_order_acquire);
  if (p) return p;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  p = g_scratch[dev].load(std::memory_order_relaxed);
  if (!p) {
    void* q = nullptr;
    if (hipGetSymbolAddress(&q, HIP_SYMBOL(scratch)) != hipSuccess || !q) return nullptr;
    p = static_cast<char*>(q);
    g_scratch[dev].store(p, std::memory_order_release);
  }
  return p;
}

}  // namespace

int64_t ce_noalloc_max_rows(void) { return kNoAllocMaxRows; }

int ce_fwd_bwd_inplace_noalloc(float* logits, const int64_t* targets, int64_t BT, int64_t V, int64_t ignore_index,
                               float* loss, float* row_loss, int32_t* err_flag, void* stream) {
  const int st = flce::check_ce_noalloc(logits, targets, BT, V, loss, row_loss, err_flag, kNoAllocMaxRows);
  if (st != FLCE_OK) return st;
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev >= kMaxDevices) return FLCE_ERR_DEVICE;
  if (device_status(dev) != 1) return FLCE_ERR_DEVICE;
  char* ws = scratch_on(dev);
  if (!ws) return FLCE_ERR_LAUNCH;

  hipStream_t s = static_cast<hipStream_t>(stream);
  int32_t* nvalid = reinterpret_cast<int32_t*>(ws);
  float* rl = row_loss ? row_loss : reinterpret_cast<float*>(ws + 256);
  // every scratch word read is written first in stream order (count, then
  // token losses), so nothing needs clearing between calls
  if (flce::launch_count_valid(targets, BT, V, ignore_index, nvalid, err_flag, s) != hipSuccess)
    return FLCE_ERR_LAUNCH;
  if (flce::launch_ce_rows(logits, targets, BT, V, ignore_index, nvalid, rl, s) != hipSuccess)
    return FLCE_ERR_LAUNCH;
  if (flce::launch_loss_final(rl, BT, nvalid, loss, s) != hipSuccess) return FLCE_ERR_LAUNCH;
  return FLCE_OK;
}

}  // extern "C"
