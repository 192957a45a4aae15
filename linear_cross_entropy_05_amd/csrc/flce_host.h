// Host side of the C-ABI entry points that touches no device: argument
// checks, the chunk rule and the workspace layouts.  Plain C++ with no HIP
// header, so the same unit is compiled into libflce and, with the address and
// undefined-behaviour sanitizers, into a CPU test program.
#pragma once

#include <stddef.h>
#include <stdint.h>

namespace flce {

constexpr int kTile = 256;      // output tile edge (M and N) of the MFMA products
constexpr int kRowBytes = 128;  // K bytes per tile row per pipeline stage

// Tile ranges of a GEMM launch.  Workgroups are dealt round-robin over the
// chip's kXcds XCDs (workgroup b runs on XCD b % kXcds), and the tile ids
// [0, total) of a launch are split into kXcds contiguous ranges, one per XCD,
// so that the tiles an XCD runs at once are neighbours sharing operand blocks
// in its L2: range x starts at xcd_first(total, x) and holds
// xcd_len(total, x) tiles.  (constexpr, so also callable from device code.)
constexpr int kXcds = 8;
constexpr int64_t xcd_len(int64_t total, int64_t x) { return total / kXcds + (x < total % kXcds ? 1 : 0); }
constexpr int64_t xcd_first(int64_t total, int64_t x) {
  return x * (total / kXcds) + (x < total % kXcds ? x : total % kXcds);
}
// Work items of a launch taken at run time from per-XCD counters (take_item
// in gemm_core.h): n0 items of kind 0 and n1 of kind 1 (n1 = 0 for a launch
// of one kind).  The range of XCD y holds its share of kind 0 (items
// xcd_first(n0, y) .. + xcd_len(n0, y) - 1) and then its share of kind 1;
// position v of it is the item below, or item -1 past the range.  Over all
// XCDs and positions each item of each kind appears exactly once.
struct XcdItem {
  int64_t item;
  int kind;
};
constexpr XcdItem xcd_item(int64_t n0, int64_t n1, int64_t y, int64_t v) {
  const int64_t l0 = xcd_len(n0, y), l1 = xcd_len(n1, y);
  if (v < l0) return XcdItem{xcd_first(n0, y) + v, 0};
  if (v < l0 + l1) return XcdItem{xcd_first(n1, y) + (v - l0), 1};
  return XcdItem{-1, 0};
}
// Workgroups of such a launch of `total` items: one eighth more than the
// items, as many for each XCD (the surplus finds every range used up).
constexpr int64_t queue_grid(int64_t total) {
  return kXcds * ((total + kXcds - 1) / kXcds + ((total + kXcds - 1) / kXcds + 7) / 8);
}

// Workspace of one flce_fwd_bwd call: where each scratch array lives.  The
// chunk buffer holds one chunk's logits, then (in place) their gradient; it
// is the only large array.  Offsets are in bytes from the workspace base,
// each 256-byte aligned.
struct Layout {
  int64_t BT, H, V;
  int dtype;        // 0 fp32, 1 bf16
  int64_t C;        // tokens per chunk
  int64_t ldz;      // elements between chunk rows (V rounded up to 256)
  int64_t nvt;      // vocabulary tiles of the logits GEMM (ceil(V / 256)); statistics per half tile
  int64_t splits;   // K splits of the dX GEMM
  int64_t esize;    // bytes per element of X, W and the chunk
  int64_t ldxt;     // bf16: elements between rows of the transposed token chunk X_c^T [H, ldxt]
  // X_c^T shares the statistics region (off_part): the statistics are dead
  // once the gradient pass has run, and X_c^T is only read by the dW product
  size_t off_nvalid, off_lse, off_rowloss, off_part, off_chunk, off_dxpart, total;
  // eight int32 work-item counters (take_item) of the logits launch and of
  // the dX + dW launch (zeroed before each), inside the 256 bytes that start
  // at off_nvalid
  size_t off_queue;
  // Token compaction (flce_fwd_bwd): only the non-ignored tokens go through
  // the chunks, packed in their order.  idx [BT] int32 holds their positions,
  // then those of the ignored tokens; each chunk's rows of X, targets and
  // token scales are gathered into xs [C, H], ys [C] int64 and ss [C] fp32.
  // Without compaction the four offsets are 0 and the regions absent.
  bool compact;
  size_t off_idx, off_ys, off_ss, off_xs;
};

// compact: the layout of flce_fwd_bwd (token compaction); false for the
// passes that process every token of a chunk (ORPO)
Layout make_layout(int64_t BT, int64_t H, int64_t V, int64_t chunk_tokens, int dtype, bool compact);
// Forward only: no chunk buffer; off_chunk == off_dxpart == total.
Layout make_fwd_layout(int64_t BT, int64_t H, int64_t V, int64_t chunk_tokens, int dtype);

// Workspace of flce_orpo.  One pass when a chunk can hold at least one
// whole (chosen, rejected) pair: chunks of `pairs` pairs (Cp = 2 pairs
// seq_len tokens) gathered into contiguous rows, each run forward, then its
// pair terms and token factors, then backward.  Otherwise two passes over
// the whole batch: forward only (token losses), sequence terms, then the
// fused pass with the token factors.
struct OrpoLayout {
  bool one_pass;
  int64_t pairs, Cp;
  size_t off_nvalid;  // int32 [0] N, [1] valid chosen tokens, [2] error flag of the second count
  // two passes
  size_t off_rowloss, off_scale, off_scratch;
  // one pass: chunk token losses and factors, 3 n_seq + B doubles, gathered
  // rows, targets and dX rows
  size_t off_rlc, off_wc, off_seq, off_pair, off_xg, off_yg, off_dxc;
  size_t off_region, total;
  Layout fwd, fb;  // two passes: both; one pass: fb is the chunk's layout
};
OrpoLayout make_orpo_layout(int64_t n_seq, int64_t seq_len, int64_t H, int64_t V, int64_t chunk_tokens, int dtype);

// Bytes of the logits-only cross-entropy workspace: the valid-token count
// and, when the caller passes no row_loss, BT floats of token losses.
size_t ce_layout_bytes(int64_t BT);

// The kernels address one 256-row tile of an operand (or of the chunk
// buffer, of the transposed token chunk, or of the fp32 dW) through 32-bit
// byte offsets below 2^31, and number a launch's tiles with 32-bit ids
// (at most 2^30 tiles): false if these sizes would not fit.
bool tiles_fit(const Layout& L, bool chunk_buffer);

// Checks an entry point makes before it touches a device.  Each returns
// FLCE_OK or the status the entry point returns (flce_status in flce.h),
// and, on FLCE_OK, the layout the call will use.
int check_fwd_bwd(const void* X, const void* W, const int64_t* targets, const float* token_scale, int64_t BT,
                  int64_t H, int64_t V, int64_t chunk_tokens, int dtype, const float* loss, const float* row_loss,
                  const void* dX, const float* dW, const void* workspace, size_t workspace_bytes,
                  const int32_t* err_flag, Layout* L);
int check_fwd(const void* X, const void* W, const int64_t* targets, int64_t BT, int64_t H, int64_t V,
              int64_t chunk_tokens, int dtype, const float* loss, const float* row_loss, const void* workspace,
              size_t workspace_bytes, const int32_t* err_flag, Layout* L);
int check_orpo(const void* X, const void* W, const int64_t* targets, int64_t n_seq, int64_t seq_len, int64_t H,
               int64_t V, int64_t chunk_tokens, int dtype, const float* loss, const float* seq_logp, const void* dX,
               const float* dW, const void* workspace, size_t workspace_bytes, const int32_t* err_flag,
               OrpoLayout* L);
int check_ce(const float* logits, const int64_t* targets, int64_t BT, int64_t V, const float* loss,
             const float* row_loss, const void* workspace, size_t workspace_bytes, const int32_t* err_flag);
// the logits-only cross-entropy with no workspace: at most max_rows rows
int check_ce_noalloc(const float* logits, const int64_t* targets, int64_t BT, int64_t V, const float* loss,
                     const float* row_loss, const int32_t* err_flag, int64_t max_rows);

}  // namespace flce
