// Host-side launchers of the TTT kernels; the C ABI (ttt_api.cpp) schedules them.
#pragma once
#include <hip/hip_runtime.h>
#include <stddef.h>
#include "common.h"

namespace ttt {

enum { INNER_LINEAR = 0, INNER_MLP = 1, INNER_SWIGLU = 2 };
enum { LOSS_MSE = 0, LOSS_DOT = 1 };

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
// Wnew = Wcur - sum(partials); optional column re-norm to W0's column norms;
// writes the fp32 state (layout [P][nm][msz]) and optionally W_out.
struct UpdateArgs {
  WRef cur, w0;
  const float* part;            // gradient partials (already scaled by eta and the loss constant)
  int part_mode;                // PART_SPLITS: part[s][p][nm][msz], s < S
                                // PART_STREAMK: slot (i*J + p - first_pair(i)) of workgroup i,
                                // laid out in the MFMA gradient kernel's register order
                                // (see k_update_streamk)
  int S; long long part_pair_stride;
  int sk_G, sk_J, sk_tpp;       // stream-K geometry of the gradient kernel
  float* next;                  // [P][nm][msz] fp32
  float* out[3];                // W_out matrices [B,H,in,out] or null
  int renorm;
};
enum { PART_SPLITS = 0, PART_STREAMK = 1 };

// Stream-K split of the MFMA gradient kernel.  The (pair, 32-token tile) space
// is laid on a cost line on which pair p occupies U = tpp + kSkAlpha units: a
// prologue slot of kSkAlpha units (the cost of staging a pair's weights and
// statistics, in tiles) followed by its tpp tiles.  Workgroup q of G takes the
// line range [q C / G, (q + 1) C / G), C = P U, i.e. the tiles in it: ranges
// that cross a pair boundary, and so pay a second prologue, get fewer tiles.
constexpr int kSkAlpha = 6;
// flattened tile index (pair * tpp + tile) of the first tile at or after line position u
__host__ __device__ inline long long sk_tile_at(long long u, int tpp) {
  const long long U = tpp + kSkAlpha, p = u / U, t = u % U - kSkAlpha;
  return p * tpp + (t > 0 ? t : 0);
}
// workgroup whose line range holds position u
__host__ __device__ inline long long sk_group_of(long long u, long long G, long long C) { return ((u + 1) * G - 1) / C; }
// first pair of workgroup q's range (its partial slot j holds pair first + j)
__host__ __device__ inline long long sk_first_pair(long long q, long long G, long long C, int tpp) {
  return (q * C / G) / (tpp + kSkAlpha);
}
void launch_update(const Problem& pb, const UpdateArgs& a, hipStream_t st);

// ---- MFMA fast paths --------------------------------------------------------
// GELU-MLP, d = 64, h in {64,128,256}, bf16 tensors: fused forward/backward of
// one update batch (tokens [t0, t0+nt)) at the fp32 weights W, stream-K over the
// pairs' 32-token tiles; the key statistics are merged from the per-slice
// partials `spart` (S_stats slices, null: no key norm); partial slots as in
// mfma_grad_geometry.
bool mfma_full_supported(const Problem& pb);
// producer (= consumer) waves of the gradient kernel for hidden width hid; the
// hidden units are split over them in slices of hid / mfma_grad_waves(hid).
// Measured alternatives at width 256: 8 + 8 waves ran 5 % slower (the extra
// reads of the shared LDS tiles cost more than the added latency hiding), and
// 4 producers + 8 consumers (the consumers also computing V_hat) 2.2x slower
// (at three waves per SIMD the consumers spill registers).
constexpr int mfma_grad_waves(int /*hid*/) { return 4; }
void mfma_grad_geometry(const Problem& pb, int nt, int* G, int* J, int* tiles_per_pair);
void launch_mfma_full_grad(const Problem& pb, const WRef& W, int t0, int nt, float scale, const float* spart,
                           int S_stats, float eps, float* part, hipStream_t st);
// readout O = F_W(Q) on bf16 MFMA from fp32 states: full batch reads state 1,
// causal chunk c reads state c (state 0 = w0, state s >= 1 at
// states + (s-1)*state_stride, layout [P][nm][msz]).
bool mfma_query_supported(const Problem& pb);
void launch_mfma_query(const Problem& pb, const WRef& w0, const float* states, long long state_stride, int nchunks,
                       int chunk, hipStream_t st);

// SwiGLU fast weights + negative dot loss (LaCT), bf16 tensors, d in {64,128},
// h in {128,256}, no key norm: gradient of one update batch with hi/lo-split
// bf16 MFMA operands (fp32-level accuracy), partials part[S][P][3][msz]
bool lact_supported(const Problem& pb);
int lact_grad_splits(const Problem& pb, int nt);
void launch_lact_grad(const Problem& pb, const WRef& W, int t0, int nt, int S, float scale, float* part,
                      hipStream_t st);
// SwiGLU readout on bf16 MFMA (state addressing as launch_mfma_query)
bool lact_readout_supported(const Problem& pb);
void launch_lact_readout(const Problem& pb, const WRef& w0, const float* states, long long state_stride,
                         int nchunks, int chunk, hipStream_t st);

// compute units of the current device (cached per device; 256 if unknown)
int device_cu_count();

// ---- finiteness check ------------------------------------------------------
void launch_zero_flag(int* flag, hipStream_t st);
void launch_check_finite(const Problem& pb, float* const* wfinal, long long wcount, int* flag,
                         hipStream_t st);

}  // namespace ttt
