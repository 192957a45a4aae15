// Internal interface between the C-ABI entry points and the kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "flce_host.h"

namespace flce {

// Kernel kinds, in the order flce_profile_end reports them.
enum Phase {
  kPhaseCount = 0,  // count valid targets, range check
  kPhaseLogits,     // logits GEMM + softmax statistics
  kPhaseLse,        // log-sum-exp combine, per-token loss
  kPhaseGrad,       // in-place gradient of the logits
  kPhaseDxDw,       // dX and dW GEMMs (one launch; bf16: with the chunk transpose)
  kPhaseDxReduce,   // sum of dX split partials
  kPhaseLoss,       // final mean
  kPhaseCeRows,     // logits-only cross-entropy rows
  kPhaseFill,       // zero fill
  kPhaseOrpo,       // ORPO sequence statistics and token gradient factors
  kPhaseGather,     // token compaction: ignored rows zeroed, chunk rows gathered
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
// Token compaction (a layout with L.compact), once per call before the
// chunks: N, the target check, the positions of the non-ignored tokens (then
// the ignored ones) and zeros in the ignored tokens' dX rows and losses.
hipError_t launch_compact(const Layout& L, const int64_t* y, int64_t ignore_index, char* ws, int32_t* err, void* dX,
                          float* rowloss, hipStream_t s);
// One chunk, forward and backward.  Without compaction: tokens c0 .. c0 +
// rows - 1.  With it (L.compact, after launch_compact): the non-ignored
// tokens c0 .. c0 + rows - 1 in their order, of which those below N exist.
// scale: NULL (gradient factor 1/N) or per-token gradient factors [BT]
hipError_t launch_flce_chunk(const Layout& L, const void* X, const void* W, const int64_t* y, const float* scale,
                             int64_t ignore_index, int64_t c0, int64_t rows, char* ws, float* rowloss, void* dX,
                             float* dW, bool first, hipStream_t s);
// The two halves of launch_flce_chunk: logits with their statistics and
// the chunk buffer (z - M_h), lse and token losses; then, from those, the
// in-place gradient with factors `scale` (NULL: 1/N), dX rows and dW (+)=.
hipError_t launch_logits_chunk(const Layout& L, const void* X, const void* W, const int64_t* y, int64_t ignore_index,
                               int64_t c0, int64_t rows, char* ws, float* rowloss, hipStream_t s);
hipError_t launch_grad_chunk(const Layout& L, const void* X, const void* W, const int64_t* y, const float* scale,
                             int64_t ignore_index, int64_t c0, int64_t rows, char* ws, void* dX, float* dW, bool first,
                             hipStream_t s);
hipError_t launch_fwd_chunk(const Layout& L, const void* X, const void* W, const int64_t* y, int64_t ignore_index,
                            int64_t c0, int64_t rows, char* ws, float* rowloss, hipStream_t s);
hipError_t launch_loss_final(const float* rowloss, int64_t BT, const int32_t* nvalid, float* loss, hipStream_t s);
hipError_t launch_orpo_stats(const float* rowloss, const int64_t* y, int64_t n_seq, int64_t T, int64_t ign, float beta,
                             float* scale, float* seq_logp, float* loss, double* scratch, hipStream_t s);
// One-pass ORPO over chunks of whole (chosen, rejected) pairs p0 .. p0 + np - 1
// of sequences of Tl tokens (B pairs in all): gather the chunk's rows,
// scatter its dX rows back, the chunk's sequence / pair terms and token
// factors, and the final loss.
hipError_t launch_orpo_gather(const void* X, const int64_t* y, int64_t H, int64_t Tl, int64_t B, int64_t p0,
                              int64_t np, int dtype, void* Xg, int64_t* yg, hipStream_t s);
hipError_t launch_orpo_scatter(const void* dXc, int64_t H, int64_t Tl, int64_t B, int64_t p0, int64_t np, int dtype,
                               void* dX, hipStream_t s);
hipError_t launch_orpo_chunk_stats(const float* rlc, const int64_t* yg, int64_t Tl, int64_t B, int64_t p0, int64_t np,
                                   int64_t ign, float beta, const int32_t* nchosen, float* wc, float* seq_logp,
                                   double* seq, double* pair, hipStream_t s);
hipError_t launch_orpo_final(const double* seq, const double* pair, int64_t B, float beta, const int32_t* nchosen,
                             float* loss, hipStream_t s);
hipError_t launch_ce_rows(float* logits, const int64_t* y, int64_t BT, int64_t V, int64_t ignore_index,
                          const int32_t* nvalid, float* rowloss, hipStream_t s);

}  // namespace flce
