// Host-side launchers of the TTT kernels; the C ABI (ttt_api.cpp) schedules them.
#pragma once
#include <hip/hip_runtime.h>
#include <stddef.h>
#include "common.h"
#include "ttt.h"

namespace ttt {

enum { INNER_LINEAR = 0, INNER_MLP = 1, INNER_SWIGLU = 2, INNER_GLU = 3, INNER_DWCONV = 4 };
enum { LOSS_MSE = 0, LOSS_DOT = 1 };

// Everything a kernel of one update batch (the whole sequence in full-batch
// mode, one chunk in causal mode) needs to know.
// A problem covers heads [h0, h0 + H) of tensors with Hs heads; its pairs
// p = b H + h (b < B, h < H) are numbered compactly (weight states, partials
// and statistics use p), and row(p) gives the pair's row of the [B, Hs, N, d]
// tensors, of eta_tok and of W_out.
struct Problem {
  int B, H, N, d, hid;    // hid: hidden width (d for LINEAR and GLU)
  int inner, loss, nm;    // nm: matrices of the inner model
  int bf16;               // q/k/v/o are bf16 (else fp32)
  const void* q; const void* k; const void* v; void* o;
  const float* eta_tok;   // [B,Hs,N] or null
  float eta_scale;
  const float* stats;     // [P][d][2] (mu, rstd) or null (no key norm)
  long long msz;          // elements per matrix (d*hid, d*d, or d*k*k)
  int Hs, h0;             // heads of the tensors, first head of this problem
  int gh, gw, ck;         // DWCONV: token raster and kernel size
  __host__ __device__ long long row(long long p) const { return (p / H) * Hs + h0 + p % H; }
  __host__ __device__ bool full_heads() const { return Hs == H && h0 == 0; }
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
  int sk_direct;                // the gradient kernel applied the step to every whole pair: skip those
  float* next;                  // [P][nm][msz] fp32 (may alias cur: every element is read, then written, by one thread)
  float* out[3];                // W_out matrices [B,H,in,out] or null
  int renorm;
  unsigned mask;                // bit i: matrix i is updated (others: next = cur, momentum untouched)
  int rule;                     // RULE_*: GD subtracts the partials; MOMENTUM and MUON fold them into mom
  float beta;                   // momentum coefficient
  float* mom;                   // [P][nm][msz] momentum (MOMENTUM, MUON) or null
  int mom_only;                 // MUON: update mom and copy cur to next; the Muon step follows
};
enum { RULE_GD = 0, RULE_MOMENTUM = 1, RULE_MUON = 2 };
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
// Grid of the stream-K split for P pairs of tpp tiles: G = min(target, P*tpp)
// workgroups (never more workgroups than tiles) and J, the partial slots each
// workgroup owns: a range of ceil(C / G) line units touches at most J pairs.
__host__ __device__ inline void sk_geometry(long long P, int tpp, long long target, int* G, int* J) {
  const long long total = P * tpp;
  const long long g = target < total ? target : total;
  const long long U = tpp + kSkAlpha, per = (P * U + g - 1) / g;
  *G = (int)g;
  *J = (int)((per + U - 1) / U + 1);
}
// first and last workgroup whose tile range holds a tile of pair p (the ones
// holding its first and its last tile on the cost line)
__host__ __device__ inline void sk_pair_groups(long long p, int tpp, long long G, long long C, long long* q0,
                                               long long* q1) {
  const long long U = tpp + kSkAlpha;
  *q0 = sk_group_of(p * U + kSkAlpha, G, C);
  *q1 = sk_group_of(p * U + kSkAlpha + tpp - 1, G, C);
}
// partial slot of pair p written by workgroup q (q0 <= q <= q1): a workgroup
// after q0 starts inside p, so p is its first pair (slot q J); q0 may have
// started in an earlier pair
__host__ __device__ inline long long sk_slot(long long p, long long q, long long q0, long long G, long long C, int tpp,
                                             int J) {
  return q * J + (q == q0 ? p - sk_first_pair(q0, G, C, tpp) : 0);
}
// Register order of the MFMA gradient kernel's stream-K partials (d = 64,
// GELU MLP, hidden width hid split over its 4 waves in slices of HP = hid/4
// units, NHB = HP/16 blocks of 16 units).  Float4 j of a pair's partial
// (j < 32 hid) holds elements (row + i, col), i = 0..3, of matrix mat:
//   dW1 part, j < 16 hid:  float4 ((qq*4 + cb)*NHB + hb)*64 + l -> dW1[16cb + 4g + i][qq*HP + 16hb + r]
//   dW2 part:              float4 ((qq*NHB + hb)*4 + cb)*64 + l -> dW2[qq*HP + 16hb + 4g + i][16cb + r]
// with l = 16g + r.
struct SkElem { int mat, row, col; };
__host__ __device__ inline SkElem sk_part_elem(int hid, int j) {
  const int hp = hid / 4, nhb = hp / 16, half = 16 * hid;
  const int mat = j >= half ? 1 : 0, jj = j - mat * half;
  const int l = jj & 63, blk = jj >> 6, g = l >> 4, r = l & 15;
  if (mat == 0) {
    const int hb = blk % nhb, cb = (blk / nhb) & 3, qq = blk / (4 * nhb);
    return SkElem{0, 16 * cb + 4 * g, qq * hp + 16 * hb + r};
  }
  const int cb = blk & 3, hb = (blk >> 2) % nhb, qq = blk / (4 * nhb);
  return SkElem{1, qq * hp + 16 * hb + 4 * g, 16 * cb + r};
}
// The stream-K update kernel's workgroup x takes partial float4s [256x, 256x +
// 256), four consecutive 64-float4 blocks of one matrix, which hold the
// matrix block rows [row0, row0 + rows) x columns [col0, col0 + cols) (W1:
// 64/NHB rows of HP columns; W2: 16 whole rows); rs is the matrix row stride.
struct SkBlock { int mat, row0, col0, rows, cols, rs; };
__host__ __device__ inline SkBlock sk_update_block(int hid, int x) {
  const int hp = hid / 4, nhb = hp / 16, half = 16 * hid;
  const int mat = 256 * x >= half ? 1 : 0;
  const int blk0 = (256 * x - mat * half) >> 6;
  if (mat == 0) {
    const int u0 = blk0 / nhb;                     // qq * 4 + first cb
    return SkBlock{0, 16 * (u0 & 3), (u0 >> 2) * hp, 64 / nhb, hp, hid};
  }
  return SkBlock{1, 16 * (blk0 >> 2), 0, 16, 64, 64};
}
void launch_update(const Problem& pb, const UpdateArgs& a, hipStream_t st);
// column re-norm of a.next in place (matrices in a.mask), writing a.out
void launch_renorm(const Problem& pb, const UpdateArgs& a, hipStream_t st);

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
// Direct step: a workgroup whose range holds a whole pair applies the plain
// gradient step to it itself, W* = W - dW, writing `next` (the [P][2][d*hid]
// fp32 state, natural layouts) and, when given, the caller's W_out matrices
// (rows pb.row(p)); it stores the pair's partial like any slot and, after a
// barrier, all its threads apply the step from it.  The update kernel then
// skips those pairs (UpdateArgs::sk_direct), and is not launched when no pair
// is split.  With one_round the grid is one workgroup per pair, every pair
// is whole; it is taken when the pairs fill between half and all of the
// workgroup slots in one round (many short pairs: the split-N partials and
// the update kernel would outweigh the work).
// With readout set (every pair whole), the workgroup reads out its pair
// itself instead: its consumer waves put W* from their accumulators into LDS
// (and W_out), no partial and no state is written, and after a barrier all
// its waves compute O = F_W*(Q) of the pair's tokens (no readout kernel).
struct GradDirect { float* next; float* out[2]; int readout; };
bool mfma_grad_direct_fits(const Problem& pb);
// pairs of the stream-K split whose tiles more than one workgroup holds
long long mfma_grad_split_pairs(const Problem& pb, int nt);
void launch_mfma_full_grad(const Problem& pb, const WRef& W, int t0, int nt, float scale, const float* spart,
                           int S_stats, float eps, float* part, const GradDirect* direct, bool one_round,
                           hipStream_t st);
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

// ---- Muon: Newton-Schulz orthogonalisation of the momentum matrices --------
// For every (pair, updated matrix): X = mom / (||mom||_F + 1e-7) on the wide
// orientation, ns_steps quintic iterations, then next -= scale * X (back in the
// [in, out] orientation); W_out is written when out[i] is set.  xa, xb: two
// [P][nm][m*n] buffers, ga, gb: two [P][nm][m*m] buffers (m = min(in, out),
// n = max(in, out)).
size_t muon_scratch_floats(const Problem& pb);
void launch_muon(const Problem& pb, const float* mom, float* next, float* const* out, unsigned mask, float scale,
                 int ns_steps, float* scratch, hipStream_t st);

// ---- simplified GLU on bf16 MFMA (d = 64, bf16 tensors) ----------------------
// partials part[S][P][2][d*d] of the update batch [t0, t0 + nt); readout from
// the state (layout [P][2][d*d]); head ranges via Problem::row
bool glu_supported(const Problem& pb);
int glu_grad_splits(const Problem& pb, int nt);
// spart: the key-statistics slices (S_stats per pair), merged by the kernel
// itself; null: pb.stats (finished statistics) or no key norm
void launch_glu_grad(const Problem& pb, const WRef& W, int t0, int nt, int S, const float* spart, int S_stats,
                     float eps, float* part, hipStream_t st);
void launch_glu_query(const Problem& pb, const float* state, hipStream_t st);

// ---- depthwise-convolution inner model (full batch) --------------------------
// partial dw over S token splits -> part[S][P][1][d*ck*ck]; readout from the
// state at `state` (layout [P][d*ck*ck])
int dwconv_grad_splits(const Problem& pb);
void launch_dwconv_grad(const Problem& pb, const WRef& W, int S, float* part, hipStream_t st);
void launch_dwconv_query(const Problem& pb, const float* state, hipStream_t st);

// ---- outer-loop backward (full batch, one step, linear / GELU MLP) ----------
// wstar_states: W* of every pair ([P][nm][msz]); S: token splits of the
// weight reductions (part holds S * P * nm * msz floats); dO32, gG, gF:
// [P][N][d] fp32; U, dpair: [P][nm][msz]; knp: [P][S_kn][2][d]; dq, dk, dv:
// fp32 [B,Hs,N,d]; deta fp32 [B,Hs,N] or null; dW0[i] in W0's layout
// ([H,in,out] summed over the batch when w0_shared, else [B,H,in,out]) or null.
int bwd_kn_splits(const Problem& pb);
// dW0 in the caller's layout from the per-pair [P][nm][msz] gradient (summed
// over the batch for a shared W0), then the key-norm backward of dk in place
void launch_bwd_tail(const Problem& pb, const float* dpair, int w0_shared, float* const* dW0, float* dk, int S_kn,
                     float* knp, hipStream_t st);
// the fp32-MFMA backward of the GELU MLP (d, h multiples of 16, W0 16-byte aligned)
struct BwdMfmaSizes {
  long long tok_d, tok_h, wsz;   // floats of a [P][N][d], a [P][N][h] and a [P][2][d h] buffer
  int KS;                        // token slices of the reductions over N
};
struct BwdMfmaBufs {
  float *X, *Q, *dO, *G, *F, *Fd;             // [P][N][d]
  float *Z, *A, *dA, *dZ, *Zd, *Ad, *Ab;      // [P][N][h]
  float *part;                                // [KS][P][2][d h]
  float *dW, *Ws, *U;                         // [P][2][d h]
  float *knp;                                 // key-norm partials
};
// one fp32 inner step of the GELU MLP on tokens [t0, t0 + nt) on the same
// matrix-core products: X [P][nt][d], Z, A, dZ [P][nt][h], F, G [P][nt][d];
// dA optional ([P][nt][h], else dZ overwrites it)
struct StepMfmaBufs {
  float *X, *Z, *A, *dA, *dZ, *F, *G;
};
bool step_mfma_shape(const Problem& pb);
bool step_mfma_aligned(const WRef& W);
int step_mfma_splits(const Problem& pb, int nt);
void launch_step_mfma(const Problem& pb, const WRef& W, int t0, int nt, const StepMfmaBufs& sb, float* part, int KS,
                      hipStream_t st);
bool bwd_mfma_supported(const Problem& pb, const WRef& w0);
void bwd_mfma_sizes(const Problem& pb, BwdMfmaSizes* s);
void launch_backward_mfma(const Problem& pb, const WRef& w0, const void* dO, const BwdMfmaBufs& bb, float* dq,
                          float* dk, float* dv, float* deta, float* const* dW0, int w0_shared, int S_kn,
                          hipStream_t st);
void launch_backward(const Problem& pb, const WRef& w0, const float* wstar_states, const void* dO, int S,
                     float* part, float* dO32, float* U, float* gG, float* gF, float* dpair, float* knp, int S_kn,
                     float* dq, float* dk, float* dv, float* deta, float* const* dW0, int w0_shared,
                     hipStream_t st);

// compute units of the current device (cached per device; 256 if unknown)
int device_cu_count();

// scratch bytes per device behind ttt_forward_noalloc (every benchmarked
// configuration fits; the largest, ViT-S at r = 4, needs 145 MiB)
constexpr size_t kNoallocScratchBytes = size_t(192) << 20;
// record a printf-style message as the handle's last error (h == NULL: the
// thread's create error) and return code
int set_error(ttt_handle* h, int code, const char* fmt, ...);
// ttt_forward that creates no stream or event: the head ranges of a request
// use the handle's second stream only if an earlier ttt_forward created it,
// and otherwise run one after another on the caller's stream
int forward_no_create(ttt_handle* h, const void* q, const void* k, const void* v, const ttt_weights* W0,
                      const ttt_eta* eta, int loss, int inner, int chunk, void* o, const ttt_weights_out* W_out,
                      void* workspace, size_t ws_bytes, void* stream);

// ---- finiteness check ------------------------------------------------------
void launch_zero_flag(int* flag, hipStream_t st);
// n floats at p set to zero by a fill kernel (no memset node under graph capture)
void launch_fill_zero(float* p, long long n, hipStream_t st);
// n elements of pb.o and wcount elements at each non-null wfinal[i]
void launch_check_finite(const Problem& pb, long long n, float* const* wfinal, long long wcount, int* flag,
                         hipStream_t st);

}  // namespace ttt
