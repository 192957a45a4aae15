// Internal interface between the C-ABI entry points and the kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace flce {

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
};

Layout make_layout(int64_t BT, int64_t H, int64_t V, int64_t chunk_tokens, int dtype);
// Forward only: no chunk buffer; off_chunk == off_dxpart == total.
Layout make_fwd_layout(int64_t BT, int64_t H, int64_t V, int64_t chunk_tokens, int dtype);

// Kernel kinds, in the order flce_profile_end reports them.
enum Phase {
  kPhaseCount = 0,  // count valid targets, range check
  kPhaseLogits,     // logits GEMM + softmax statistics
  kPhaseLse,        // log-sum-exp combine, per-token loss
  kPhaseGrad,       // in-place gradient of the logits
  kPhaseDx,         // dX GEMM
  kPhaseDxReduce,   // sum of dX split partials
  kPhaseDw,         // dW GEMM
  kPhaseLoss,       // final mean
  kPhaseCeRows,     // logits-only cross-entropy rows
  kPhaseFill,       // zero fill
  kPhaseOrpo,       // ORPO sequence statistics and token gradient factors
  kNumPhases
};

// Brackets one launch with event records while profiling is on.
class ProfScope {
 public:
  ProfScope(int phase, hipStream_t s);
  ~ProfScope();

 private:
  long idx_;
  hipStream_t s_;
};

// Launchers (all asynchronous on `s`; they return the launch status).
hipError_t launch_count_valid(const int64_t* y, int64_t BT, int64_t V, int64_t ignore_index, int32_t* nvalid,
                              int32_t* err, hipStream_t s);
hipError_t launch_fill_zero(float* p, int64_t n, hipStream_t s);
// scale: NULL (gradient factor 1/N) or per-token gradient factors [BT]
hipError_t launch_flce_chunk(const Layout& L, const void* X, const void* W, const int64_t* y, const float* scale,
                             int64_t ignore_index, int64_t c0, int64_t rows, char* ws, float* rowloss, void* dX,
                             float* dW, bool first, hipStream_t s);
hipError_t launch_fwd_chunk(const Layout& L, const void* X, const void* W, const int64_t* y, int64_t ignore_index,
                            int64_t c0, int64_t rows, char* ws, float* rowloss, hipStream_t s);
hipError_t launch_loss_final(const float* rowloss, int64_t BT, const int32_t* nvalid, float* loss, hipStream_t s);
hipError_t launch_orpo_stats(const float* rowloss, const int64_t* y, int64_t n_seq, int64_t T, int64_t ign, float beta,
                             float* scale, float* seq_logp, float* loss, double* scratch, hipStream_t s);
hipError_t launch_ce_rows(float* logits, const int64_t* y, int64_t BT, int64_t V, int64_t ignore_index,
                          const int32_t* nvalid, float* rowloss, hipStream_t s);

}  // namespace flce
