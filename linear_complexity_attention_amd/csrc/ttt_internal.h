// Host-side launchers of the TTT kernels; the C ABI (ttt_api.cpp) schedules them.
#pragma once
#include <hip/hip_runtime.h>
#include <stddef.h>
#include "common.h"

namespace ttt {

enum { INNER_LINEAR = 0, INNER_MLP = 1, INNER_SWIGLU = 2 };
enum { LOSS_MSE = 0, LOSS_DOT = 1 };
enum { BF_ROWMAJOR = 0, BF_TRANSPOSED = 1, BF_MLP3 = 2 };

// Everything a kernel of one update batch (the whole sequence in full-batch
// mode, one chunk in causal mode) needs to know.
struct Problem {
  int B, H, N, d, hid;    // hid: hidden width (d for LINEAR)
  int inner, loss, nm;    // nm: matrices of the inner model
  int bf16;               // q/k/v/o are bf16 (else fp32)
  const void* q; const void* k; const void* v; void* o;
  const float* eta_tok;   // [B,H,N] or null
  float eta_scale;
  const float* stats;     // [P][d][2] (mu, rstd) or null (no key norm)
  long long msz;          // elements per matrix (d*hid, or d*d)
};

// ---- key statistics --------------------------------------------------------
// partial (count, mean, M2) per (pair, slice, channel) -> part[P][S][3][d]
void launch_stats_partial(const Problem& pb, int S, float* part, hipStream_t st);
// Chan's parallel combination of the slices -> stats[P][d][2]
void launch_stats_final(const Problem& pb, int S, const float* part, float eps, float* stats,
                        hipStream_t st);

// ---- generic (fp32 arithmetic, any dtype, every inner model / loss) ------
// G for tokens [t0, t0+nt) of every pair -> gbuf[P][nt][d] (fp32, eta folded in)
void launch_gen_grad_out(const Problem& pb, const WRef& W, int t0, int nt, float* gbuf, hipStream_t st);
// partial dW over S token splits of [t0, t0+nt) -> part[S][P][nm][msz]
void launch_gen_dW(const Problem& pb, const WRef& W, int t0, int nt, const float* gbuf, int S,
                   float* part, hipStream_t st);
// O = F_W(Q) for every token.  Full-batch mode (chunk == 0): every token reads
// state 1; causal mode: chunk 0 reads w0, chunk c >= 1 reads state c at
// states + (c-1)*state_stride (layout [P][nm][msz]).
void launch_gen_query(const Problem& pb, const WRef& w0, const float* states, long long state_stride,
                      int nchunks, int chunk, hipStream_t st);

// ---- weight update (shared by every path) ----------------------------------
// Wnew = Wcur - sum_s part[s]; optional column re-norm to W0's column norms;
// writes the fp32 state (layout [P][nm][msz]), optionally W_out and a bf16
// operand copy (layout chosen by `bf_layout`, see update.hip).
struct UpdateArgs {
  WRef cur, w0;
  const float* part;            // gradient partials (already scaled by eta and the loss constant)
  int part_mode;                // PART_SPLITS: part[s][p][nm][msz], s < S
                                // PART_STREAMK: slot (i*J + p - first_pair(i)) of workgroup i
  int S; long long part_pair_stride;
  int sk_G, sk_J, sk_tpp;       // stream-K geometry of the gradient kernel
  float* next;                  // [P][nm][msz] fp32
  float* out[3];                // W_out matrices [B,H,in,out] or null
  bf16* bf;                     // bf16 operand copy or null
  int bf_layout;
  int renorm;
};
enum { PART_SPLITS = 0, PART_STREAMK = 1 };
void launch_update(const Problem& pb, const UpdateArgs& a, hipStream_t st);
// bf16 operand copy of a weight state without an update (W0 for the first
// gradient pass of the MFMA kernels)
void launch_convert_bf16(const Problem& pb, const WRef& W, bf16* dst, int bf_layout, hipStream_t st);

// ---- MFMA fast paths --------------------------------------------------------
// GELU-MLP, d = 64, h in {64,128,256}, bf16: fused forward/backward of one
// update batch (tokens [t0, t0+nt)) on bf16 MFMA, stream-K over the pairs'
// tiles; partials land in BF_MLP3-ordered slots (see mfma_grad_geometry).
bool mfma_full_supported(const Problem& pb);
void mfma_grad_geometry(const Problem& pb, int nt, int* G, int* J, int* tiles_per_pair);
void launch_mfma_full_grad(const Problem& pb, const bf16* wbf, int t0, int nt, float scale, float* part,
                           hipStream_t st);
// readout O = F_W(Q) on bf16 MFMA; wstates: bf16 BF_MLP3 states, state s at
// wstates + s*state_stride (state 0 = W0); full batch reads state 1, causal
// chunk c reads state c.
bool mfma_query_supported(const Problem& pb);
void launch_mfma_query(const Problem& pb, const bf16* wstates, long long state_stride, int nchunks, int chunk,
                       hipStream_t st);

// ---- finiteness check ------------------------------------------------------
void launch_zero_flag(int* flag, hipStream_t st);
void launch_check_finite(const Problem& pb, float* const* wfinal, long long wcount, int* flag,
                         hipStream_t st);

}  // namespace ttt
