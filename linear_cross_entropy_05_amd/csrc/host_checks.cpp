// Host-only part of the C ABI: argument checks, the chunk rule, workspace
// layouts, status strings and size queries.  No HIP header and no device
// call: libflce links this unit, and a CPU test builds it with the address
// and undefined-behaviour sanitizers and runs the library's host-check cases
// through it.
#include "flce_host.h"

#include "../../include/flce.h"

namespace flce {

namespace {

size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

bool aligned(const void* p, uintptr_t a) { return ((uintptr_t)p & (a - 1)) == 0; }

bool dtype_ok(int dtype) { return dtype == FLCE_F32 || dtype == FLCE_BF16; }

// Token count, hidden size and vocabulary each below 2^31: the layout
// arithmetic below then stays far from int64 overflow.
bool sizes_ok(int64_t BT, int64_t H, int64_t V) {
  return BT >= 0 && H > 0 && V > 0 && BT <= INT32_MAX && H <= INT32_MAX && V <= INT32_MAX;
}

// Fewest K splits of the dX product that fill the 256 CUs best, each split
// keeping >= 16 stages of K, the fp32 partials within half the chunk buffer
// or 128 MiB, whichever is larger (small chunks would otherwise leave most
// CUs idle).
int64_t pick_splits(int64_t tiles, int64_t kstages, size_t part_bytes_per_split, size_t chunk_bytes) {
  constexpr int64_t kCUs = 256;
  const size_t cap = chunk_bytes / 2 > ((size_t)128 << 20) ? chunk_bytes / 2 : ((size_t)128 << 20);
  int64_t best = 1;
  double best_cost = (double)((tiles + kCUs - 1) / kCUs);
  for (int64_t s = 2; s <= 16; ++s) {
    if (kstages / s < 16) break;
    if ((size_t)s * part_bytes_per_split > cap) break;
    const double cost = (double)((tiles * s + kCUs - 1) / kCUs) / (double)s;
    if (cost < best_cost * 0.97) {
      best = s;
      best_cost = cost;
    }
  }
  return best;
}

}  // namespace

Layout make_layout(int64_t BT, int64_t H, int64_t V, int64_t chunk_tokens, int dtype, bool compact) {
  Layout L{};
  L.BT = BT;
  L.H = H;
  L.V = V;
  L.dtype = dtype;
  L.esize = dtype == FLCE_BF16 ? 2 : 4;
  L.ldz = (V + kTile - 1) / kTile * kTile;
  L.nvt = (V + kTile - 1) / kTile;
  int64_t C = chunk_tokens;
  if (C <= 0) {
    // as few chunks as keep the chunk buffer within 1 GiB, of equal size
    // rounded up to whole 256-token tiles (each chunk after the first costs
    // a read-modify-write of the fp32 dW)
    const int64_t cmax = ((int64_t)1 << 30) / (L.ldz * L.esize);
    if (cmax < kTile || BT <= cmax) {
      C = cmax < 1 ? 1 : cmax;
    } else {
      const int64_t nch = (BT + cmax - 1) / cmax;
      C = ((BT + nch - 1) / nch + kTile - 1) / kTile * kTile;
      const int64_t cmax_tiles = cmax / kTile * kTile;
      if (C > cmax_tiles) C = cmax_tiles;
    }
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
  L.off_queue = o + 64;
  o = align256(o + 96);
  L.off_lse = o;
  o = align256(o + (size_t)C * 4);
  L.off_rowloss = o;
  o = align256(o + (size_t)(BT > 0 ? BT : 1) * 4);
  L.compact = compact;
  if (compact) {
    L.off_idx = o;
    o = align256(o + (size_t)(BT > 0 ? BT : 1) * 4);
    L.off_ys = o;
    o = align256(o + (size_t)C * 8);
    L.off_ss = o;
    o = align256(o + (size_t)C * 4);
    L.off_xs = o;
    o = align256(o + (size_t)C * H * L.esize);
  }
  L.off_part = o;
  L.ldxt = (C + 63) / 64 * 64;
  {
    const size_t stats = (size_t)C * 2 * L.nvt * 8;
    const size_t xt = dtype == FLCE_BF16 ? (size_t)H * L.ldxt * 2 : 0;
    o = align256(o + (stats > xt ? stats : xt));
  }
  L.off_chunk = o;
  o = align256(o + chunk_bytes);
  L.off_dxpart = o;
  if (L.splits > 1) o = align256(o + (size_t)L.splits * C * H * 4);
  L.total = o;
  return L;
}

Layout make_fwd_layout(int64_t BT, int64_t H, int64_t V, int64_t chunk_tokens, int dtype) {
  Layout L{};
  L.BT = BT;
  L.H = H;
  L.V = V;
  L.dtype = dtype;
  L.esize = dtype == FLCE_BF16 ? 2 : 4;
  L.ldz = (V + kTile - 1) / kTile * kTile;
  L.nvt = (V + kTile - 1) / kTile;
  int64_t C = chunk_tokens;
  if (C <= 0) {
    // no logits are kept: a pass is bounded only by its statistics
    // (8 bytes per token and half tile), at most 256 MiB
    C = ((int64_t)1 << 28) / (2 * L.nvt * 8);
  }
  if (C > BT) C = BT;
  if (C < 1) C = 1;
  L.C = C;
  L.splits = 1;
  size_t o = 0;
  L.off_nvalid = o;
  L.off_queue = o + 64;
  o = align256(o + 96);
  L.off_lse = o;
  o = align256(o + (size_t)C * 4);
  L.off_rowloss = o;
  o = align256(o + (size_t)(BT > 0 ? BT : 1) * 4);
  L.off_part = o;
  o = align256(o + (size_t)C * 2 * L.nvt * 8);
  L.off_chunk = o;
  L.off_dxpart = o;
  L.total = o;
  return L;
}

OrpoLayout make_orpo_layout(int64_t n_seq, int64_t seq_len, int64_t H, int64_t V, int64_t chunk_tokens, int dtype) {
  OrpoLayout L{};
  const int64_t BT = n_seq * seq_len;
  const int64_t B = n_seq / 2;
  // the chunk size fused linear + cross-entropy would take for this batch
  const int64_t C = make_layout(BT, H, V, chunk_tokens, dtype, false).C;
  L.pairs = C / (2 * seq_len);
  if (L.pairs > B) L.pairs = B;
  L.one_pass = L.pairs >= 1;
  size_t o = 0;
  L.off_nvalid = o;
  o = align256(o + 16);
  if (L.one_pass) {
    const int64_t esize = dtype == FLCE_BF16 ? 2 : 4;
    L.Cp = 2 * L.pairs * seq_len;
    L.fb = make_layout(L.Cp, H, V, L.Cp, dtype, false);
    L.off_rlc = o;
    o = align256(o + (size_t)L.Cp * 4);
    L.off_wc = o;
    o = align256(o + (size_t)L.Cp * 4);
    L.off_seq = o;
    o = align256(o + (size_t)n_seq * 3 * 8);
    L.off_pair = o;
    o = align256(o + (size_t)(B > 0 ? B : 1) * 8);
    L.off_xg = o;
    o = align256(o + (size_t)L.Cp * H * esize);
    L.off_yg = o;
    o = align256(o + (size_t)L.Cp * 8);
    L.off_dxc = o;
    o = align256(o + (size_t)L.Cp * H * esize);
    L.off_region = o;
    L.total = o + L.fb.total;
  } else {
    L.fwd = make_fwd_layout(BT, H, V, chunk_tokens, dtype);
    L.fb = make_layout(BT, H, V, chunk_tokens, dtype, false);
    L.off_rowloss = o;
    o = align256(o + (size_t)BT * 4);
    L.off_scale = o;
    o = align256(o + (size_t)BT * 4);
    L.off_scratch = o;
    o = align256(o + (size_t)n_seq * 3 * 8);
    L.off_region = o;
    L.total = o + (L.fwd.total > L.fb.total ? L.fwd.total : L.fb.total);
  }
  return L;
}

size_t ce_layout_bytes(int64_t BT) { return 256 + align256((size_t)(BT > 0 ? BT : 1) * 4); }

bool tiles_fit(const Layout& L, bool chunk_buffer) {
  constexpr int64_t kMax = INT32_MAX;
  const int64_t rows = kTile;
  if (rows * L.H * L.esize > kMax) return false;
  if (chunk_buffer && rows * L.ldz * L.esize > kMax) return false;
  if (chunk_buffer && L.dtype == FLCE_BF16 && rows * L.ldxt * 2 > kMax) return false;
  // the fp32 dW rows of a 256-row tile (read back by the dW product)
  if (chunk_buffer && rows * L.H * 4 > kMax) return false;
  // tile ids of one launch (int32, with room for the launch's extra workgroups)
  const int64_t ct = (L.C + kTile - 1) / kTile, ht = (L.H + kTile - 1) / kTile;
  if (L.nvt * ct > (1 << 30) || (chunk_buffer && L.nvt * ht > (1 << 30))) return false;
  return true;
}

int check_fwd_bwd(const void* X, const void* W, const int64_t* targets, const float* token_scale, int64_t BT,
                  int64_t H, int64_t V, int64_t chunk_tokens, int dtype, const float* loss, const float* row_loss,
                  const void* dX, const float* dW, const void* workspace, size_t workspace_bytes,
                  const int32_t* err_flag, Layout* out) {
  if (!dtype_ok(dtype)) return FLCE_ERR_DTYPE;
  if (!sizes_ok(BT, H, V)) return FLCE_ERR_ARG;
  if (!W || !loss || !dW || !workspace || !err_flag) return FLCE_ERR_ARG;
  if (BT > 0 && (!X || !targets || !dX)) return FLCE_ERR_ARG;
  if (H % (dtype == FLCE_BF16 ? 8 : 4) != 0) return FLCE_ERR_SHAPE;
  if (!aligned(W, 16) || (X && !aligned(X, 16)) || (targets && !aligned(targets, 8)) || !aligned(workspace, 256) ||
      !aligned(dW, 16) || (dX && !aligned(dX, 16)) || (row_loss && !aligned(row_loss, 4)) ||
      (token_scale && !aligned(token_scale, 4)))
    return FLCE_ERR_ALIGN;
  const Layout L = make_layout(BT, H, V, chunk_tokens, dtype, true);
  if (!tiles_fit(L, true)) return FLCE_ERR_SHAPE;
  if (workspace_bytes < L.total) return FLCE_ERR_WORKSPACE;
  *out = L;
  return FLCE_OK;
}

int check_fwd(const void* X, const void* W, const int64_t* targets, int64_t BT, int64_t H, int64_t V,
              int64_t chunk_tokens, int dtype, const float* loss, const float* row_loss, const void* workspace,
              size_t workspace_bytes, const int32_t* err_flag, Layout* out) {
  if (!dtype_ok(dtype)) return FLCE_ERR_DTYPE;
  if (!sizes_ok(BT, H, V)) return FLCE_ERR_ARG;
  if (!W || !loss || !workspace || !err_flag) return FLCE_ERR_ARG;
  if (BT > 0 && (!X || !targets)) return FLCE_ERR_ARG;
  if (H % (dtype == FLCE_BF16 ? 8 : 4) != 0) return FLCE_ERR_SHAPE;
  if (!aligned(W, 16) || (X && !aligned(X, 16)) || (targets && !aligned(targets, 8)) || !aligned(workspace, 256) ||
      (row_loss && !aligned(row_loss, 4)))
    return FLCE_ERR_ALIGN;
  const Layout L = make_fwd_layout(BT, H, V, chunk_tokens, dtype);
  if (!tiles_fit(L, false)) return FLCE_ERR_SHAPE;
  if (workspace_bytes < L.total) return FLCE_ERR_WORKSPACE;
  *out = L;
  return FLCE_OK;
}

int check_orpo(const void* X, const void* W, const int64_t* targets, int64_t n_seq, int64_t seq_len, int64_t H,
               int64_t V, int64_t chunk_tokens, int dtype, const float* loss, const float* seq_logp, const void* dX,
               const float* dW, const void* workspace, size_t workspace_bytes, const int32_t* err_flag,
               OrpoLayout* out) {
  if (!dtype_ok(dtype)) return FLCE_ERR_DTYPE;
  if (n_seq < 2 || n_seq % 2 || seq_len <= 0 || n_seq > INT32_MAX || seq_len > INT32_MAX / n_seq ||
      !sizes_ok(n_seq * seq_len, H, V))
    return FLCE_ERR_ARG;
  if (!X || !W || !targets || !loss || !dX || !dW || !workspace || !err_flag) return FLCE_ERR_ARG;
  if (H % (dtype == FLCE_BF16 ? 8 : 4) != 0) return FLCE_ERR_SHAPE;
  if (!aligned(W, 16) || !aligned(X, 16) || !aligned(targets, 8) || !aligned(workspace, 256) || !aligned(dW, 16) ||
      !aligned(dX, 16) || (seq_logp && !aligned(seq_logp, 4)))
    return FLCE_ERR_ALIGN;
  const OrpoLayout L = make_orpo_layout(n_seq, seq_len, H, V, chunk_tokens, dtype);
  if (!tiles_fit(L.fb, true) || (!L.one_pass && !tiles_fit(L.fwd, false))) return FLCE_ERR_SHAPE;
  if (workspace_bytes < L.total) return FLCE_ERR_WORKSPACE;
  *out = L;
  return FLCE_OK;
}

int check_ce(const float* logits, const int64_t* targets, int64_t BT, int64_t V, const float* loss,
             const float* row_loss, const void* workspace, size_t workspace_bytes, const int32_t* err_flag) {
  if (!sizes_ok(BT, 1, V)) return FLCE_ERR_ARG;
  if (!loss || !workspace || !err_flag) return FLCE_ERR_ARG;
  if (BT > 0 && (!logits || !targets)) return FLCE_ERR_ARG;
  if ((logits && !aligned(logits, 4)) || (targets && !aligned(targets, 8)) || !aligned(workspace, 256) ||
      (row_loss && !aligned(row_loss, 4)))
    return FLCE_ERR_ALIGN;
  if (workspace_bytes < ce_layout_bytes(BT)) return FLCE_ERR_WORKSPACE;
  return FLCE_OK;
}

int check_ce_noalloc(const float* logits, const int64_t* targets, int64_t BT, int64_t V, const float* loss,
                     const float* row_loss, const int32_t* err_flag, int64_t max_rows) {
  if (!sizes_ok(BT, 1, V)) return FLCE_ERR_ARG;
  if (BT > max_rows) return FLCE_ERR_SCRATCH;
  if (!loss || !err_flag) return FLCE_ERR_ARG;
  if (BT > 0 && (!logits || !targets)) return FLCE_ERR_ARG;
  if ((logits && !aligned(logits, 4)) || (targets && !aligned(targets, 8)) || (row_loss && !aligned(row_loss, 4)))
    return FLCE_ERR_ALIGN;
  return FLCE_OK;
}

}  // namespace flce

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
      return "unsupported shape (H must be a multiple of 8 for bf16, 4 for fp32; 256 rows of W, of the fp32 dW, of "
             "the logits chunk and of the transposed token chunk must each fit in 2^31 bytes)";
    case FLCE_ERR_ALIGN: return "misaligned pointer";
    case FLCE_ERR_SCRATCH: return "more rows than the static scratch of the no-allocation entry point holds";
    default: return "unknown status";
  }
}

int64_t flce_chunk_tokens(int64_t BT, int64_t H, int64_t V, int64_t chunk_tokens, int dtype) {
  if (!flce::sizes_ok(BT, H, V) || !flce::dtype_ok(dtype)) return 0;
  return flce::make_layout(BT, H, V, chunk_tokens, dtype, true).C;
}

size_t flce_workspace_bytes(int64_t BT, int64_t H, int64_t V, int64_t chunk_tokens, int dtype) {
  if (!flce::sizes_ok(BT, H, V) || !flce::dtype_ok(dtype)) return 0;
  return flce::make_layout(BT, H, V, chunk_tokens, dtype, true).total;
}

size_t flce_fwd_workspace_bytes(int64_t BT, int64_t H, int64_t V, int64_t chunk_tokens, int dtype) {
  if (!flce::sizes_ok(BT, H, V) || !flce::dtype_ok(dtype)) return 0;
  return flce::make_fwd_layout(BT, H, V, chunk_tokens, dtype).total;
}

size_t flce_orpo_workspace_bytes(int64_t n_seq, int64_t seq_len, int64_t H, int64_t V, int64_t chunk_tokens,
                                 int dtype) {
  if (n_seq < 2 || n_seq % 2 || seq_len <= 0 || n_seq > INT32_MAX || seq_len > INT32_MAX / n_seq ||
      !flce::sizes_ok(n_seq * seq_len, H, V) || !flce::dtype_ok(dtype))
    return 0;
  return flce::make_orpo_layout(n_seq, seq_len, H, V, chunk_tokens, dtype).total;
}

size_t ce_workspace_bytes(int64_t BT, int64_t V) {
  if (!flce::sizes_ok(BT, 1, V)) return 0;
  return flce::ce_layout_bytes(BT);
}

}  // extern "C"
