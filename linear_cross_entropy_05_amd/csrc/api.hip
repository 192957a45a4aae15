// C-ABI entry points: argument checks, workspace layout, and the token-chunk
// schedule of fused linear + cross-entropy.
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

#include "../../include/flce.h"
#include "flce_internal.h"

namespace {

constexpr int kMaxDevices = 64;
int g_device_ok[kMaxDevices];  // 0 unknown, 1 gfx950, 2 other

int device_status(int dev) {
  if (dev < 0) return -1;
  if (dev < kMaxDevices && g_device_ok[dev]) return g_device_ok[dev] == 1 ? 1 : 0;
  hipDeviceProp_t p;
  if (hipGetDeviceProperties(&p, dev) != hipSuccess) return -1;
  const int ok = strncmp(p.gcnArchName, "gfx950", 6) == 0 ? 1 : 0;
  if (dev < kMaxDevices) g_device_ok[dev] = ok ? 1 : 2;
  return ok;
}

int current_device_ok() {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess) return -1;
  return device_status(dev);
}

bool aligned(const void* p, uintptr_t a) { return ((uintptr_t)p & (a - 1)) == 0; }

// The kernels address one 256-row tile of an operand, or of the chunk buffer,
// through a buffer resource with 32-bit byte offsets whose range is capped at
// 2^31 - 1 bytes: a 256-row tile of W or X ([.., H]), of the chunk buffer
// ([.., V rounded up to 256]) and of the transposed token chunk ([H, C
// rounded up to 64], bf16) must fit.  Larger shapes are rejected rather than
// computed with dropped accesses.
bool tiles_fit(const flce::Layout& L, bool chunk_buffer) {
  constexpr int64_t kMax = INT32_MAX;
  const int64_t rows = 256;
  if (rows * L.H * L.esize > kMax) return false;
  if (chunk_buffer && rows * L.ldz * L.esize > kMax) return false;
  if (chunk_buffer && L.dtype == FLCE_BF16 && rows * L.ldxt * 2 > kMax) return false;
  return true;
}

}  // namespace

extern "C" {

const char* flce_status_str(int status) {
  switch (status) {
    case FLCE_OK: return "ok";
    case FLCE_ERR_ARG: return "invalid argument (null pointer or bad size)";
    case FLCE_ERR_DTYPE: return "unsupported dtype";
    case FLCE_ERR_WORKSPACE: return "workspace too small";
    case FLCE_ERR_DEVICE: return "current device is not gfx950";
    case FLCE_ERR_LAUNCH: return "kernel launch failed";
    case FLCE_ERR_TARGET: return "target outside [0, V) that is not ignore_index";
    case FLCE_ERR_SHAPE:
      return "unsupported shape (H must be a multiple of 8 for bf16, 4 for fp32; 256 rows of W, of the logits "
             "chunk and of the transposed token chunk must each fit in 2^31 bytes)";
    case FLCE_ERR_ALIGN: return "misaligned pointer";
    default: return "unknown status";
  }
}

int flce_device_supported(int device) { return device_status(device); }

int64_t flce_chunk_tokens(int64_t BT, int64_t H, int64_t V, int64_t chunk_tokens, int dtype) {
  if (BT < 0 || H <= 0 || V <= 0 || (dtype != FLCE_F32 && dtype != FLCE_BF16)) return 0;
  return flce::make_layout(BT, H, V, chunk_tokens, dtype).C;
}

size_t flce_workspace_bytes(int64_t BT, int64_t H, int64_t V, int64_t chunk_tokens, int dtype) {
  if (BT < 0 || H <= 0 || V <= 0 || (dtype != FLCE_F32 && dtype != FLCE_BF16)) return 0;
  return flce::make_layout(BT, H, V, chunk_tokens, dtype).total;
}

int flce_fwd_bwd(const void* X, const void* W, const int64_t* targets, const float* token_scale, int64_t BT,
                 int64_t H, int64_t V, int64_t ignore_index, int64_t chunk_tokens, int dtype, float* loss,
                 float* row_loss, void* dX, float* dW, void* workspace, size_t workspace_bytes, int32_t* err_flag,
                 void* stream) {
  if (dtype != FLCE_F32 && dtype != FLCE_BF16) return FLCE_ERR_DTYPE;
  if (BT < 0 || H <= 0 || V <= 0 || BT > INT32_MAX || V > INT32_MAX) return FLCE_ERR_ARG;
  if (!W || !loss || !dW || !workspace || !err_flag) return FLCE_ERR_ARG;
  if (BT > 0 && (!X || !targets || !dX)) return FLCE_ERR_ARG;
  if (H % (dtype == FLCE_BF16 ? 8 : 4) != 0) return FLCE_ERR_SHAPE;
  if (!aligned(W, 16) || (X && !aligned(X, 16)) || (targets && !aligned(targets, 8)) || !aligned(workspace, 256) ||
      !aligned(dW, 16) || (dX && !aligned(dX, 16)) || (row_loss && !aligned(row_loss, 4)) ||
      (token_scale && !aligned(token_scale, 4)))
    return FLCE_ERR_ALIGN;
  const flce::Layout L = flce::make_layout(BT, H, V, chunk_tokens, dtype);
  if (!tiles_fit(L, true)) return FLCE_ERR_SHAPE;
  if (workspace_bytes < L.total) return FLCE_ERR_WORKSPACE;
  if (current_device_ok() != 1) return FLCE_ERR_DEVICE;

  hipStream_t s = static_cast<hipStream_t>(stream);
  char* ws = static_cast<char*>(workspace);
  int32_t* nvalid = reinterpret_cast<int32_t*>(ws + L.off_nvalid);
  float* rl = row_loss ? row_loss : reinterpret_cast<float*>(ws + L.off_rowloss);

  if (flce::launch_count_valid(targets, BT, V, ignore_index, nvalid, err_flag, s) != hipSuccess)
    return FLCE_ERR_LAUNCH;
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

size_t flce_fwd_workspace_bytes(int64_t BT, int64_t H, int64_t V, int64_t chunk_tokens, int dtype) {
  if (BT < 0 || H <= 0 || V <= 0 || (dtype != FLCE_F32 && dtype != FLCE_BF16)) return 0;
  return flce::make_fwd_layout(BT, H, V, chunk_tokens, dtype).total;
}

int flce_fwd(const void* X, const void* W, const int64_t* targets, int64_t BT, int64_t H, int64_t V,
             int64_t ignore_index, int64_t chunk_tokens, int dtype, float* loss, float* row_loss, void* workspace,
             size_t workspace_bytes, int32_t* err_flag, void* stream) {
  if (dtype != FLCE_F32 && dtype != FLCE_BF16) return FLCE_ERR_DTYPE;
  if (BT < 0 || H <= 0 || V <= 0 || BT > INT32_MAX || V > INT32_MAX) return FLCE_ERR_ARG;
  if (!W || !loss || !workspace || !err_flag) return FLCE_ERR_ARG;
  if (BT > 0 && (!X || !targets)) return FLCE_ERR_ARG;
  if (H % (dtype == FLCE_BF16 ? 8 : 4) != 0) return FLCE_ERR_SHAPE;
  if (!aligned(W, 16) || (X && !aligned(X, 16)) || (targets && !aligned(targets, 8)) || !aligned(workspace, 256) ||
      (row_loss && !aligned(row_loss, 4)))
    return FLCE_ERR_ALIGN;
  const flce::Layout L = flce::make_fwd_layout(BT, H, V, chunk_tokens, dtype);
  if (!tiles_fit(L, false)) return FLCE_ERR_SHAPE;
  if (workspace_bytes < L.total) return FLCE_ERR_WORKSPACE;
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

namespace {
struct OrpoLayout {
  size_t off_nvalid, off_rowloss, off_scale, off_scratch, off_region, total;
  flce::Layout fwd, fb;
};
size_t a256(size_t x) { return (x + 255) & ~(size_t)255; }
OrpoLayout orpo_layout(int64_t n_seq, int64_t seq_len, int64_t H, int64_t V, int64_t chunk_tokens, int dtype) {
  OrpoLayout L{};
  const int64_t BT = n_seq * seq_len;
  L.fwd = flce::make_fwd_layout(BT, H, V, chunk_tokens, dtype);
  L.fb = flce::make_layout(BT, H, V, chunk_tokens, dtype);
  size_t o = 0;
  L.off_nvalid = o;
  o = a256(o + 16);
  L.off_rowloss = o;
  o = a256(o + (size_t)BT * 4);
  L.off_scale = o;
  o = a256(o + (size_t)BT * 4);
  L.off_scratch = o;
  o = a256(o + (size_t)n_seq * 3 * 8);
  L.off_region = o;
  L.total = o + (L.fwd.total > L.fb.total ? L.fwd.total : L.fb.total);
  return L;
}
}  // namespace

size_t flce_orpo_workspace_bytes(int64_t n_seq, int64_t seq_len, int64_t H, int64_t V, int64_t chunk_tokens,
                                 int dtype) {
  if (n_seq < 2 || n_seq % 2 || seq_len <= 0 || H <= 0 || V <= 0 || (dtype != FLCE_F32 && dtype != FLCE_BF16))
    return 0;
  return orpo_layout(n_seq, seq_len, H, V, chunk_tokens, dtype).total;
}

int flce_orpo(const void* X, const void* W, const int64_t* targets, int64_t n_seq, int64_t seq_len, int64_t H,
              int64_t V, int64_t ignore_index, float beta, int64_t chunk_tokens, int dtype, float* loss,
              float* seq_logp, void* dX, float* dW, void* workspace, size_t workspace_bytes, int32_t* err_flag,
              void* stream) {
  if (dtype != FLCE_F32 && dtype != FLCE_BF16) return FLCE_ERR_DTYPE;
  if (n_seq < 2 || n_seq % 2 || seq_len <= 0 || H <= 0 || V <= 0 || V > INT32_MAX || n_seq > INT32_MAX ||
      seq_len > INT32_MAX / n_seq)
    return FLCE_ERR_ARG;
  if (!X || !W || !targets || !loss || !dX || !dW || !workspace || !err_flag) return FLCE_ERR_ARG;
  if (H % (dtype == FLCE_BF16 ? 8 : 4) != 0) return FLCE_ERR_SHAPE;
  if (!aligned(W, 16) || !aligned(X, 16) || !aligned(targets, 8) || !aligned(workspace, 256) || !aligned(dW, 16) ||
      !aligned(dX, 16) || (seq_logp && !aligned(seq_logp, 4)))
    return FLCE_ERR_ALIGN;
  const int64_t BT = n_seq * seq_len;
  const OrpoLayout L = orpo_layout(n_seq, seq_len, H, V, chunk_tokens, dtype);
  if (!tiles_fit(L.fb, true) || !tiles_fit(L.fwd, false)) return FLCE_ERR_SHAPE;
  if (workspace_bytes < L.total) return FLCE_ERR_WORKSPACE;
  if (current_device_ok() != 1) return FLCE_ERR_DEVICE;

  hipStream_t s = static_cast<hipStream_t>(stream);
  char* ws = static_cast<char*>(workspace);
  int32_t* nvalid = reinterpret_cast<int32_t*>(ws + L.off_nvalid);
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

size_t ce_workspace_bytes(int64_t BT, int64_t V) {
  if (BT < 0 || V <= 0) return 0;
  return 256 + (((size_t)(BT > 0 ? BT : 1) * 4 + 255) & ~(size_t)255);
}

int ce_fwd_bwd_inplace(float* logits, const int64_t* targets, int64_t BT, int64_t V, int64_t ignore_index,
                       float* loss, float* row_loss, void* workspace, size_t workspace_bytes, int32_t* err_flag,
                       void* stream) {
  if (BT < 0 || V <= 0 || BT > INT32_MAX || V > INT32_MAX) return FLCE_ERR_ARG;
  if (!loss || !workspace || !err_flag) return FLCE_ERR_ARG;
  if (BT > 0 && (!logits || !targets)) return FLCE_ERR_ARG;
  if ((logits && !aligned(logits, 4)) || (targets && !aligned(targets, 8)) || !aligned(workspace, 256) ||
      (row_loss && !aligned(row_loss, 4)))
    return FLCE_ERR_ALIGN;
  if (workspace_bytes < ce_workspace_bytes(BT, V)) return FLCE_ERR_WORKSPACE;
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

}  // extern "C"
