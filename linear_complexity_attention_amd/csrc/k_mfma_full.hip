// MFMA kernels of the GELU-MLP inner model, head dimension 64, hidden width
// 64/128/256 (gfx950, wave64, v_mfma_f32_16x16x32_{bf16,f16}, fp32 accumulate).
//
// k_mfma_grad: steps (i)-(ii) of one inner update (ViT3 summary page, section
// 02), fused per 32-token tile:
//     K_hat = (K - mu) * rstd                     key instance norm (TvS page)
//     Z  = K_hat W1,  A = gelu(Z),  V_hat = A W2   forward on the keys
//     G' = eta_n (V - V_hat) [MSE]  |  eta_n V [dot]     the negated loss gradient
//                                                       per token (the sign, the
//                                                       MSE constant 2/(n_b d) and
//                                                       the scalar eta are applied
//                                                       to the partials)
//     dW2 -= A^T G',  dA = G' W2^T,  dZ = dA * gelu'(Z),  dW1 -= K_hat^T dZ
// Each wave owns a slice of the hidden units (its slice of Z, A, dA, dZ, dW1,
// dW2, with the weight fragments of that slice held in registers).  The tiles
// shared by all waves sit in LDS, XOR-swizzled so that every access is free
// of bank conflicts: K and V as [token][channel]; A and G' as [unit][token],
// tokens of a row stored in the order the MFMA output packs them (so one lane
// writes its 8 tokens at once).  Operands that need the other orientation are
// fetched with the transposing LDS read ds_read_b64_tr_b16.  A, G' and dZ are
// f16 (A and dZ come out of the packed-f16 GELU), and so is the normalised key
// tile (|K_hat| <= sqrt(N)); raw keys (no key norm) stay bf16.  The token range
// of all (b, h) pairs is cut evenly over the grid ("stream-K"): a workgroup
// that crosses a pair boundary writes one fp32 partial per pair it touched;
// the update kernel adds them in a fixed order, so results are run-to-run
// identical.
//
// k_mfma_query: step (iii), O = gelu(Q W1*) W2*, with tokens on the MFMA lane
// axis so that both products chain through registers (details at the kernel).
//
// GELU and gelu' are evaluated two elements at a time in packed f16 from a
// polynomial fit of the normal CDF (see gelu_chains below); the fp32 kernels use
// the exact erf form.
#include <type_traits>

#include "ttt_internal.h"

namespace ttt {

namespace {

constexpr int D = 64;
constexpr int TT = 32;            // tokens per tile
constexpr int LDK = 64;           // [token][channel] tile row stride (bf16), swizzled by kswz
constexpr int LDT = 32;           // [unit][token] tile row stride (bf16), swizzled by tswz

typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) s16x4* lds_s16x4_ptr;

__device__ __forceinline__ f32x4 mfma16(const bf16x8& a, const bf16x8& b, const f32x4& c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

// Transposing LDS read: the 16 lanes of each quarter-wave each name an 8-byte
// row piece; lane i receives element (i % 4) of the pieces of lanes
// i/4, 4 + i/4, 8 + i/4 and 12 + i/4 (in that order).
__device__ __forceinline__ bf16x4 ld_tr(const bf16* p) {
  s16x4 v = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4_ptr)((__attribute__((address_space(3))) char*)p));
  return __builtin_bit_cast(bf16x4, v);
}

// Packed-f16 GELU.  With a clamp point c, zh = sqrt(2) Z / c, w = clamp(zh,
// -sqrt(2), sqrt(2)) and v = w^2 - 1 (in [-1, 1]),
//     c Phi(Z) = c/2 + w P(v) / sqrt(2),     gelu'(Z) = 1/2 + w Q(v) / sqrt(2)
// where P, Q are Lawson (minimax) fits in v, whose small coefficients keep f16
// Horner accurate; then zh * c Phi(Z) = sqrt(2) gelu(Z).  Two elements per
// instruction and no transcendental.  The weights that produce Z are staged
// pre-scaled by sqrt(2)/c, so the MFMA delivers zh; the activation
// A' = sqrt(2) gelu(Z) is consumed by products whose other operand (or result)
// carries the compensating 1/sqrt(2).
// Where no w is needed (the readout), the same P is evaluated on the
// unclamped zh and the clamp moves to the output, where the last FMA's clamp
// bit does it for free:
//     Phi(Z) = clamp01(1/2 + zh P(zh^2 - 1) / (sqrt(2) c)),  zh Phi(Z) = (sqrt(2)/c) gelu(Z).
// Beyond the fit interval the degree-9 odd polynomial leaves [0, 1] with the
// sign of Z and never comes back (checked for every finite f16 zh; once v^k
// overflows, the infinities carry that sign), so Phi is exactly 0 or 1 there.
// Two fits (coefficients of v^0, v^1, ...):
//   GeluFitG: c = 3.5, P of degree 4, Q of degree 5, max |error| 5.7e-3 on
//             gelu (|Z| < 4; beyond, the result's relative error is 1e-3),
//             2.4e-3 on gelu'; for the gradient kernel (gelu' needs the wider
//             clamp point: it approaches 1 only slowly);
//   GeluFit4: c = 3.125, P of degree 4, output clamp, max |error| 2.6e-3 on
//             gelu beyond the f16 rounding of the result (relative 5e-4),
//             over every finite f16 zh; for the readout, which needs no gelu'.
// The gradient kernel keeps the input clamp: its w feeds gelu' as well, and
// packed max and min issue slower than an FMA (measured), so moving the clamp
// of w to the waves that evaluate gelu' cost more than it saved.
typedef _Float16 f16;
typedef f16 h2 __attribute__((ext_vector_type(2)));
typedef f16 f16x4 __attribute__((ext_vector_type(4)));
typedef f16 f16x8 __attribute__((ext_vector_type(8)));
typedef float f2 __attribute__((ext_vector_type(2)));
constexpr float kSqrt2 = 1.41421356237f;
constexpr float kRSqrt2 = 0.70710678119f;
struct GeluFitG {
  static constexpr float c = 3.5f;
  static constexpr int NP = 5, NQ = 6;
  static constexpr float P[5] = {2.440403834f, -1.086301905f, 0.665899315f, -0.464786102f, 0.196728345f};
  static constexpr float Q[6] = {0.764969678f, -0.512306439f, 0.450549349f, -0.42596567f, 0.42093503f, -0.196860224f};
};
struct GeluFit4 {
  static constexpr float c = 3.125f;
  static constexpr int NP = 5, NQ = 1;
  static constexpr float P[5] = {2.14908049f, -0.897445747f, 0.478055487f, -0.263695363f, 0.094819101f};
  static constexpr float Q[1] = {0.f};
};
constexpr float kZScale = kSqrt2 / GeluFitG::c;         // W1 staging scale of the gradient kernel
constexpr float kZScaleQ = kSqrt2 / GeluFit4::c;       // ... and of the readout
constexpr float kW2ScaleQ = 1.f / kZScaleQ;            // W2 staging scale of the readout (c/sqrt(2))
__device__ __forceinline__ h2 hh(float x) { return h2{(f16)x, (f16)x}; }
__device__ __forceinline__ h2 cvt_h2(float x0, float x1) { return __builtin_convertvector(f2{x0, x1}, h2); }
// The Horner chains of NC element pairs are advanced together: a dependent
// packed-f16 FMA must wait a cycle after its producer, independent ones need
// not, so interleaving the chains keeps the VALU issuing every cycle.
//   z[2c], z[2c+1] = zh of pair c  ->  a[c] = sqrt(2) gelu(Z)  (and, if wout,
//   wout[c] = w, from which gelu_deriv_chains gives gelu'(Z))
template <class F, int NC>
__device__ __forceinline__ void gelu_chains(const float* z, h2* a, h2* wout) {
  h2 zh[NC], w[NC], v[NC], p[NC];
#pragma unroll
  for (int c = 0; c < NC; ++c) zh[c] = cvt_h2(z[2 * c], z[2 * c + 1]);
#pragma unroll
  for (int c = 0; c < NC; ++c) w[c] = __builtin_elementwise_max(zh[c], hh(-kSqrt2));
#pragma unroll
  for (int c = 0; c < NC; ++c) w[c] = __builtin_elementwise_min(w[c], hh(kSqrt2));
#pragma unroll
  for (int c = 0; c < NC; ++c) v[c] = __builtin_elementwise_fma(w[c], w[c], hh(-1.0f));
#pragma unroll
  for (int c = 0; c < NC; ++c)
    p[c] = __builtin_elementwise_fma(hh(F::P[F::NP - 1] * kRSqrt2), v[c], hh(F::P[F::NP - 2] * kRSqrt2));
#pragma unroll
  for (int k = F::NP - 3; k >= 0; --k)
#pragma unroll
    for (int c = 0; c < NC; ++c) p[c] = __builtin_elementwise_fma(p[c], v[c], hh(F::P[k] * kRSqrt2));
#pragma unroll
  for (int c = 0; c < NC; ++c) {
    a[c] = zh[c] * __builtin_elementwise_fma(w[c], p[c], hh(0.5f * F::c));
    if (wout) wout[c] = w[c];
  }
}
//   z[2c], z[2c+1] = zh of pair c  ->  a[c] = (sqrt(2)/c) gelu(Z), output-clamped form
template <class F, int NC>
__device__ __forceinline__ void gelu_chains_oc(const float* z, h2* a) {
  constexpr float s = kRSqrt2 / F::c;
  h2 zh[NC], v[NC], p[NC];
#pragma unroll
  for (int c = 0; c < NC; ++c) zh[c] = cvt_h2(z[2 * c], z[2 * c + 1]);
#pragma unroll
  for (int c = 0; c < NC; ++c) v[c] = __builtin_elementwise_fma(zh[c], zh[c], hh(-1.0f));
#pragma unroll
  for (int c = 0; c < NC; ++c)
    p[c] = __builtin_elementwise_fma(hh(F::P[F::NP - 1] * s), v[c], hh(F::P[F::NP - 2] * s));
#pragma unroll
  for (int k = F::NP - 3; k >= 0; --k)
#pragma unroll
    for (int c = 0; c < NC; ++c) p[c] = __builtin_elementwise_fma(p[c], v[c], hh(F::P[k] * s));
#pragma unroll
  for (int c = 0; c < NC; ++c) {
    // max-then-min against 0 and 1 becomes the FMA's clamp bit
    const h2 phi = __builtin_elementwise_min(
        __builtin_elementwise_max(__builtin_elementwise_fma(zh[c], p[c], hh(0.5f)), hh(0.f)), hh(1.f));
    a[c] = zh[c] * phi;
  }
}
//   w[c] (clamped zh of pair c)  ->  gp[c] = gelu'(Z)
template <class F, int NC>
__device__ __forceinline__ void gelu_deriv_chains(const h2* w, h2* gp) {
  h2 v[NC], q[NC];
#pragma unroll
  for (int c = 0; c < NC; ++c) v[c] = __builtin_elementwise_fma(w[c], w[c], hh(-1.0f));
#pragma unroll
  for (int c = 0; c < NC; ++c)
    q[c] = __builtin_elementwise_fma(hh(F::Q[F::NQ - 1] * kRSqrt2), v[c], hh(F::Q[F::NQ - 2] * kRSqrt2));
#pragma unroll
  for (int k = F::NQ - 3; k >= 0; --k)
#pragma unroll
    for (int c = 0; c < NC; ++c) q[c] = __builtin_elementwise_fma(q[c], v[c], hh(F::Q[k] * kRSqrt2));
#pragma unroll
  for (int c = 0; c < NC; ++c) gp[c] = __builtin_elementwise_fma(w[c], q[c], hh(0.5f));
}

// element-type generic helpers (bf16 or f16 MFMA operands)
template <typename T> struct Vec;
template <> struct Vec<bf16> { typedef bf16x8 v8; typedef bf16x4 v4; };
template <> struct Vec<f16> { typedef f16x8 v8; typedef f16x4 v4; };
__device__ __forceinline__ f32x4 mfma16(const f16x8& a, const f16x8& b, const f32x4& c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
}
template <typename T>
__device__ __forceinline__ typename Vec<T>::v4 ld_trt(const T* p) {
  s16x4 v = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4_ptr)((__attribute__((address_space(3))) char*)p));
  return __builtin_bit_cast(typename Vec<T>::v4, v);
}
template <typename T>
__device__ __forceinline__ typename Vec<T>::v8 ld8t(const T* p) { return *reinterpret_cast<const typename Vec<T>::v8*>(p); }
template <typename V8, typename V4>
__device__ __forceinline__ V8 cat44t(const V4& x, const V4& y) {
  V8 r;
#pragma unroll
  for (int i = 0; i < 4; ++i) { r[i] = x[i]; r[4 + i] = y[i]; }
  return r;
}

__device__ __forceinline__ bf16x8 ld8(const bf16* p) { return *reinterpret_cast<const bf16x8*>(p); }
__device__ __forceinline__ bf16x8 cat44(const bf16x4& x, const bf16x4& y) { return cat44t<bf16x8>(x, y); }
__device__ __forceinline__ f16x8 cat44(const f16x4& x, const f16x4& y) { return cat44t<f16x8>(x, y); }
__device__ __forceinline__ bf16x4 pack4(const f32x4& x) {
  bf16x4 r;
#pragma unroll
  for (int i = 0; i < 4; ++i) r[i] = (bf16)x[i];
  return r;
}
__device__ __forceinline__ f16x4 pack4h(const f32x4& x) {
  const h2 a = cvt_h2(x[0], x[1]), b = cvt_h2(x[2], x[3]);
  return f16x4{a.x, a.y, b.x, b.y};
}
// XOR swizzles of the LDS tiles (column index in 2-byte elements).  Row `row`
// of a [token][channel] tile stores channel c at c ^ kswz(row); row `row` of a
// [unit][token] tile stores token column t at t ^ tswz(row).  Both were chosen
// by measuring SQ_LDS_BANK_CONFLICT on every access pattern of the gradient
// kernel (row reads and writes of 8 or 16 bytes per lane, and the transposing
// reads); with them none of those patterns has a bank conflict.  kswz moves
// whole 8-element pieces, so 16-byte accesses stay contiguous; tswz also moves
// 4-element halves, so 16-byte accesses to [unit][token] tiles are split into
// two 8-byte ones.
__device__ __forceinline__ int kswz(int row) { return ((row >> 3) & 1) * 8 + ((row >> 1) & 1) * 16 + ((row >> 2) & 1) * 32; }
__device__ __forceinline__ int tswz(int row) { return ((row >> 3) & 1) * 4 + ((row >> 1) & 1) * 8 + ((row >> 2) & 1) * 16; }

// storage column of token t inside a 32-token [unit][token] row: the 8 tokens
// of MFMA lane group g (4g..4g+3 and 16+4g..16+4g+3) are contiguous at 8g.
__device__ __forceinline__ int tok_col(int t) { return t < 16 ? 8 * (t >> 2) + (t & 3) : 8 * ((t - 16) >> 2) + 4 + (t & 3); }


// One wave's share [a_, b_) of a pair's tokens (wave-uniform bounds, a_ < b_
// or empty): O = gelu(Q W1*) W2* with the weights staged in LDS as the readout
// stages them (w1s: W1 [c][h] bf16 scaled by sqrt(2)/c, rows of HID + 16;
// w2s: W2 [h][c] f16 scaled by c/sqrt(2), rows of 80) and, with STAGE_O, the
// wave's 2 KB output staging block sb; QTB 16-token blocks per full pass.
template <int HID, int QTB, bool STAGE_O>
__device__ __forceinline__ void readout_share(const bf16* w1s, const f16* w2s, bf16* sb, const bf16* qp, bf16* op,
                                              int a_, int b_, int lane) {
  constexpr int L1 = HID + 16, L2 = 80;
  const int r = lane & 15, g = lane >> 4;
  // rows past the wave's share read the share's last row (their O rows are
  // not stored), so the loads need no branch
  auto load_q = [&](int pos, bf16x8 (&q)[QTB][2]) {
#pragma unroll
    for (int tb = 0; tb < QTB; ++tb)
#pragma unroll
      for (int ks = 0; ks < 2; ++ks) {
        const int n = min(pos + 16 * tb + r, b_ - 1);
        q[tb][ks] = ld8(qp + (long long)n * D + 32 * ks + 8 * g);
      }
  };
  // one pass over NTB 16-token blocks starting at pos
  auto pass = [&](auto ntb_c, int pos, const bf16x8 (&q)[QTB][2]) {
    constexpr int NTB = decltype(ntb_c)::value;
    f32x4 o[4][NTB];
#pragma unroll
    for (int cb = 0; cb < 4; ++cb)
#pragma unroll
      for (int tb = 0; tb < NTB; ++tb) o[cb][tb] = f32x4{0, 0, 0, 0};
#pragma unroll
    for (int hc = 0; hc < HID / 32; ++hc) {
      f32x4 z[2][NTB];
#pragma unroll
      for (int u = 0; u < 2; ++u)
#pragma unroll
        for (int tb = 0; tb < NTB; ++tb) z[u][tb] = f32x4{0, 0, 0, 0};
      // issue priority while this wave has MFMAs to issue, so that the MFMA
      // pipe is fed ahead of the other waves' GELU arithmetic (measured: 2 %)
      __builtin_amdgcn_s_setprio(1);
#pragma unroll
      for (int ks = 0; ks < 2; ++ks)
#pragma unroll
        for (int u = 0; u < 2; ++u) {
          // W1^T operand: W1[c = 32 ks + 8 g + j][h = 32 hc + 16 u + r]
          const bf16x4 lo = ld_tr(&w1s[(32 * ks + 8 * g + (r >> 2)) * L1 + 32 * hc + 16 * u + 4 * (r & 3)]);
          const bf16x4 hi = ld_tr(&w1s[(32 * ks + 8 * g + 4 + (r >> 2)) * L1 + 32 * hc + 16 * u + 4 * (r & 3)]);
          const bf16x8 a = cat44(lo, hi);
#pragma unroll
          for (int tb = 0; tb < NTB; ++tb) z[u][tb] = mfma16(a, q[tb][ks], z[u][tb]);
        }
      // activation operand: hidden k-slots j < 4 -> u = 0, i = j; j >= 4 -> u = 1, i = j - 4
      __builtin_amdgcn_s_setprio(0);
      f16x8 ab[NTB];
#pragma unroll
      for (int tb = 0; tb < NTB; ++tb) {
        const float zz[8] = {z[0][tb][0], z[0][tb][1], z[0][tb][2], z[0][tb][3],
                             z[1][tb][0], z[1][tb][1], z[1][tb][2], z[1][tb][3]};
        h2 x[4];
        gelu_chains_oc<GeluFit4, 4>(zz, x);
        ab[tb] = f16x8{x[0].x, x[0].y, x[1].x, x[1].y, x[2].x, x[2].y, x[3].x, x[3].y};
      }
      __builtin_amdgcn_s_setprio(1);
#pragma unroll
      for (int cb = 0; cb < 4; ++cb) {
        // W2^T operand: W2[h = 32 hc + tau(g, j)][c = 16 cb + r]
        const f16x4 lo = ld_trt(&w2s[(32 * hc + 4 * g + (r >> 2)) * L2 + 16 * cb + 4 * (r & 3)]);
        const f16x4 hi = ld_trt(&w2s[(32 * hc + 16 + 4 * g + (r >> 2)) * L2 + 16 * cb + 4 * (r & 3)]);
        const f16x8 a = f16x8{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
#pragma unroll
        for (int tb = 0; tb < NTB; ++tb) o[cb][tb] = mfma16(a, ab[tb], o[cb][tb]);
      }
    }
    // a row past the share holds the share's last row (its Q was clamped),
    // so storing it there rewrites identical values: no branch
#pragma unroll
    for (int tb = 0; tb < NTB; ++tb) {
      if constexpr (STAGE_O) {
        // lane (g, r) holds channels 16 cb + 4 g .. + 3 of token r; through
        // the wave's LDS block, lane l then takes channels 8 (l & 7) .. + 7
        // of token (l >> 3) + 8 k (the wave's own LDS operations are done
        // in order: no barrier)
#pragma unroll
        for (int cb = 0; cb < 4; ++cb)
          *reinterpret_cast<bf16x4*>(sb + r * D + (((2 * cb + (g >> 1)) ^ (r & 7)) << 3) + 4 * (g & 1)) =
              pack4(o[cb][tb]);
#pragma unroll
        for (int k = 0; k < 2; ++k) {
          const int t = (lane >> 3) + 8 * k, c = lane & 7;
          const bf16x8 v = *reinterpret_cast<const bf16x8*>(sb + t * D + ((c ^ (t & 7)) << 3));
          const int n = min(pos + 16 * tb + t, b_ - 1);
          *reinterpret_cast<bf16x8*>(op + (long long)n * D + 8 * c) = v;
        }
      } else {
        const int n = min(pos + 16 * tb + r, b_ - 1);
#pragma unroll
        for (int cb = 0; cb < 4; ++cb)
          *reinterpret_cast<bf16x4*>(op + (long long)n * D + 16 * cb + 4 * g) = pack4(o[cb][tb]);
      }
    }
  };
  // Q of the next piece is loaded while the current one is computed; the two
  // register sets alternate and every piece inside the loop is a full pass,
  // so no path back to the loop head leaves a load unconsumed (that would
  // make the compiler wait for every outstanding load and store before each
  // prefetch).  The share's last piece, when shorter than a pass, takes the
  // shortest pass that covers it (16 or 32 tokens; the share of the last wave
  // of a segment may end inside a 16-token unit) and leaves the loop; all
  // these branches are on wave-uniform scalars.
  constexpr int STEP = 16 * QTB;
  bf16x8 qa[QTB][2], qb[QTB][2];
  auto tail = [&](int pos, const bf16x8 (&q)[QTB][2]) {
    const int rem = b_ - pos;
    if (rem <= 16) pass(std::integral_constant<int, 1>{}, pos, q);
    else if (QTB == 2 || rem <= 32) pass(std::integral_constant<int, 2>{}, pos, q);
    else pass(std::integral_constant<int, QTB>{}, pos, q);   // rows past the share are clamped
  };
  int pos = a_;
  if (pos < b_) load_q(pos, qa);
  while (pos < b_) {
    if (b_ - pos < STEP) { tail(pos, qa); break; }
    load_q(pos + STEP, qb);          // past the share it re-reads the share's last row
    pass(std::integral_constant<int, QTB>{}, pos, qa);
    pos += STEP;
    if (pos >= b_) break;
    if (b_ - pos < STEP) { tail(pos, qb); break; }
    load_q(pos + STEP, qa);
    pass(std::integral_constant<int, QTB>{}, pos, qb);
    pos += STEP;
  }
}

// producer (and consumer) waves of the gradient kernel for hidden width HID
template <int HID> constexpr int kGradWaves = mfma_grad_waves(HID);
// workgroups per CU: at width 64 the kernel fits twice (both its LDS and, under
// this bound, its registers), at 128 and 256 once
template <int HID> constexpr int kGradBlocksPerCU = HID == 64 ? 2 : 1;

// Index of tile i's buffer in a ring of N.  Taken through readfirstlane so
// that the compiler treats it as an opaque uniform value: otherwise loop
// strength reduction turns every LDS address into its own induction variable.
template <int N>
__device__ __forceinline__ int ring(int i) { return __builtin_amdgcn_readfirstlane(i % N); }

// ---------------------------------------------------------------------------
// Chan et al.'s pairwise combination of (count, mean, M2) statistics: fold
// (nb, mb, m2b) into (cn, mean, m2); empty parts are skipped.
__device__ __forceinline__ void chan_merge(float& cn, float& mean, float& m2, float nb, float mb, float m2b) {
  if (nb > 0.f) {
    const float nt = cn + nb, delta = mb - mean, f = nb * __builtin_amdgcn_rcpf(nt);
    mean += delta * f;
    m2 += m2b + delta * delta * cn * f;
    cn = nt;
  }
}

// Fused forward/backward of one update batch, producer/consumer form.
//
// A workgroup has 2 NW waves: NW producers and NW consumers (NW = 4 or 8);
// producer q and consumer q own the same HP = HID/NW hidden units and share a
// SIMD (waves w and w + 4 land on the same SIMD), so the producer's VALU-heavy
// GELU and the consumer's MFMA-heavy weight-gradient products overlap there.  Tiles of 32 tokens flow
// through a three-stage pipeline, one barrier per stage:
//   phase k, producers: Z' = K_hat W1 sqrt(2)/c and the packed GELU of tile k
//            -> A' (At[k%3]) and the clamped w (Gp[k%3]); V_hat and G' of tile k-1
//            (G' -> Gc[(k-1)%2]); then stage K_hat, V, eta of tile k+1 (loaded
//            from the end of the phase before) and request tile k+2;
//   phase k, consumers: backward of tile k-2: dW2 += A'^T G', dA = G' W2^T,
//            dZ = dA gelu'(Z) (gelu' from w), dW1 += K_hat^T dZ.
// The gelu' polynomial runs on the consumers: the producers' GELU arithmetic
// is the critical path, the consumers have slack.
// Buffers: K tiles x4, V tiles x3, A' x3, w x3, G' x2.
template <int HID, int LOSS, bool KNORM, int NW, bool DIRECT>
__global__ void __launch_bounds__(128 * NW, kGradBlocksPerCU<HID> * NW / 2)   // threads, waves per SIMD
k_mfma_grad(Problem pb, WRef W, int t0, int nt, int J, float scale, const float* __restrict__ spart, int S_stats,
            float eps, float* __restrict__ part, GradDirect dw) {
  typedef typename std::conditional<KNORM, f16, bf16>::type KT;
  typedef typename Vec<KT>::v8 k8;
  constexpr int NTH = 128 * NW;        // threads
  constexpr int HP = HID / NW;         // hidden units per producer / consumer
  constexpr int NHB = HP / 16;         // 16-wide hidden blocks per wave
  constexpr int NKH = HID / 32;        // k-steps over the hidden width
  constexpr int SCH = 32 / NW;         // channels staged per producer thread
  constexpr int NB2 = 8 / NW;          // V_hat / G' blocks (16 tokens x 16 channels) per producer
  static_assert(NHB >= 1, "at least one 16-wide hidden block per wave");
  constexpr int NK = 4, NV = 3, NA = 3, NG = 2;
  __shared__ __attribute__((aligned(16))) KT Kr[NK][TT * LDK];
  __shared__ __attribute__((aligned(16))) bf16 Vr[NV][TT * LDK];
  __shared__ __attribute__((aligned(16))) f16 At[NA][HID * LDT];
  __shared__ __attribute__((aligned(16))) h2 Gp[NA][NW * NHB * 64 * 4];
  __shared__ __attribute__((aligned(16))) f16 Gc[NG][D * LDT];
  __shared__ float eta_s[NV][TT];
  __shared__ __attribute__((aligned(16))) float kst[KNORM ? D : 1][2];   // key rstd, -mean * rstd per channel
  __shared__ float kpart[KNORM ? NTH / 64 : 1][3][KNORM ? D : 1];       // slice groups (count, mean, M2)

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);   // wave index, provably uniform
  const int q = w & (NW - 1);
  const bool producer = w < NW;
  const int r = lane & 15, g = lane >> 4;
  const int h0 = q * HP;
  const int P = pb.B * pb.H;
  const int tpp = (nt + TT - 1) / TT;
  const long long G = gridDim.x, C = (long long)P * (tpp + kSkAlpha);
  const long long begin = sk_tile_at((long long)blockIdx.x * C / G, tpp);
  const long long end = sk_tile_at((long long)(blockIdx.x + 1) * C / G, tpp);
  const int p_first = (int)sk_first_pair(blockIdx.x, G, C, tpp);

  long long x = begin;
  while (x < end) {
    const int p = (int)(x / tpp);
    const int bb = p / pb.H, hh_ = p % pb.H;
    const int tile0 = (int)(x - (long long)p * tpp);
    const long long seg_end = end < (long long)(p + 1) * tpp ? end : (long long)(p + 1) * tpp;
    const int n = (int)(seg_end - x);                 // tiles of this segment
    const float* W1 = W.mat(0, bb, hh_);

    // producer staging: thread -> (token row st, channels sc .. sc + SCH - 1) of a
    // tile; tile 0's keys and values are loaded first, under the prologue
    typedef __bf16 stg_t __attribute__((ext_vector_type(SCH)));
    const int st = tid / (D / SCH), sc = (tid % (D / SCH)) * SCH;
    const bf16* kp = (const bf16*)pb.k + ((long long)p * pb.N + t0) * D;
    const bf16* vp = (const bf16*)pb.v + ((long long)p * pb.N + t0) * D;
    stg_t kreg = {}, vreg = {};
    auto prefetch = [&](int i) {              // segment-relative tile i
      const int nn = (tile0 + i) * TT + st;
      if (i < n && nn < nt) {
        kreg = *reinterpret_cast<const stg_t*>(kp + (long long)nn * D + sc);
        vreg = *reinterpret_cast<const stg_t*>(vp + (long long)nn * D + sc);
      }
    };
    if (producer) prefetch(0);

    // ---- segment prologue (all waves): the pair's weights and key statistics.
    // W1 * sqrt(2)/c and -W2 / sqrt(2) are staged in LDS, in their natural
    // [in][out] layouts, over the A' / w buffers (unused until phase 0),
    // with coalesced 16-byte loads; the producers then take their MFMA
    // fragments with transposing reads, the consumers theirs with plain
    // 16-byte reads.  The key statistics are merged from the per-slice
    // (count, mean, M2) partials with Chan's formula, first by 2 NW groups of
    // 64 threads (slices s = group, group + 2 NW, ...), then by one thread per
    // channel.
    constexpr int L1 = HID + 16, L2 = 80;                // row strides of the staged W1, W2
    KT* w1s = reinterpret_cast<KT*>(&At[0][0]);
    f16* w2s = reinterpret_cast<f16*>(&Gp[0][0]);
    static_assert(D * L1 <= NA * HID * LDT, "W1 staging exceeds the A' buffers");
    static_assert(HID * L2 <= NA * NW * NHB * 64 * 4 * 2, "W2 staging exceeds the w buffers");
    {
      constexpr int NL = D * HID / (NTH * 4);           // float4 loads per thread and matrix
      float4 a1[NL], a2[NL];
#pragma unroll
      for (int j = 0; j < NL; ++j) {
        a1[j] = reinterpret_cast<const float4*>(W1)[tid + NTH * j];
        a2[j] = reinterpret_cast<const float4*>(W.mat(1, bb, hh_))[tid + NTH * j];
      }
      if (KNORM) {                    // slices grp, grp + NG, ...: loads of 4 slices in flight at once
        constexpr int NG = NTH / 64, U = 4;
        const int c = tid & 63, grp = tid >> 6;
        const float* sp = spart + (long long)p * S_stats * 3 * D + c;
        float cn = 0.f, mean = 0.f, m2 = 0.f;
        for (int s0 = grp; s0 < S_stats; s0 += NG * U) {
          float nb[U], mb[U], m2b[U];
#pragma unroll
          for (int u = 0; u < U; ++u) {
            const int sl = s0 + NG * u;
            nb[u] = 0.f; mb[u] = 0.f; m2b[u] = 0.f;
            if (sl < S_stats) { nb[u] = sp[sl * 3 * D]; mb[u] = sp[sl * 3 * D + D]; m2b[u] = sp[sl * 3 * D + 2 * D]; }
          }
#pragma unroll
          for (int u = 0; u < U; ++u) chan_merge(cn, mean, m2, nb[u], mb[u], m2b[u]);
        }
        kpart[grp][0][c] = cn;
        kpart[grp][1][c] = mean;
        kpart[grp][2][c] = m2;
      }
#pragma unroll
      for (int j = 0; j < NL; ++j) {
        const int e = 4 * (tid + NTH * j);
        const int c1 = e / HID, h1 = e % HID;            // W1 [c][h]
        const int h2_ = e / D, c2 = e % D;                // W2 [h][c]
        typedef typename Vec<KT>::v4 kt4;
        *reinterpret_cast<kt4*>(&w1s[c1 * L1 + h1]) =
            kt4{(KT)(a1[j].x * kZScale), (KT)(a1[j].y * kZScale), (KT)(a1[j].z * kZScale), (KT)(a1[j].w * kZScale)};
        *reinterpret_cast<f16x4*>(&w2s[h2_ * L2 + c2]) =
            f16x4{(f16)(a2[j].x * -kRSqrt2), (f16)(a2[j].y * -kRSqrt2), (f16)(a2[j].z * -kRSqrt2),
                  (f16)(a2[j].w * -kRSqrt2)};
      }
    }
    __syncthreads();                                   // staged weights, slice-group statistics
    if (KNORM && tid < D) {
      float cn = 0.f, mean = 0.f, m2 = 0.f;
#pragma unroll
      for (int gi = 0; gi < NTH / 64; ++gi) chan_merge(cn, mean, m2, kpart[gi][0][tid], kpart[gi][1][tid], kpart[gi][2][tid]);
      // K_hat = fma(k, rstd, -mean * rstd) with rstd cut to 16 significant
      // bits: the product of a bf16 key (8 bits) and rstd is then exact, so a
      // key equal to a bf16-representable mean (a single token, a constant
      // channel) normalises to exactly 0, as (k - mean) * rstd does.
      const float rs = __uint_as_float(__float_as_uint(__builtin_amdgcn_rsqf(m2 / fmaxf(cn, 1.f) + eps)) & 0xffffff00u);
      kst[tid][0] = rs;
      kst[tid][1] = -mean * rs;
    }
    if (KNORM) __syncthreads();                        // kst is read by every staging thread

    if (producer) {
      // ---------------- producer ----------------
      // issue priority over the consumer of the same SIMD: the producer's GELU
      // waits on its own Z' MFMAs, which must not queue behind the consumer's
      __builtin_amdgcn_s_setprio(2);
      // W1' as the B operand of Z' = K_hat W1' (k = channel, n = hidden)
      k8 w1r[NHB][2];
#pragma unroll
      for (int hb = 0; hb < NHB; ++hb)
#pragma unroll
        for (int ks = 0; ks < 2; ++ks) {
          const int row = 32 * ks + 8 * g + (r >> 2), col = h0 + 16 * hb + 4 * (r & 3);
          w1r[hb][ks] = cat44(ld_trt(&w1s[row * L1 + col]), ld_trt(&w1s[(row + 4) * L1 + col]));
        }
      // V_hat / G' blocks of this producer: channel block cb2, token halves
      // tb2 = 0, 1 (NW = 4) or tb2 = q / 4 (NW = 8)
      const int cb2 = q & 3;
      auto tbh = [&](int b) { return NB2 == 2 ? b : q >> 2; };
      // -W2 / sqrt(2) as the B operand of -V_hat = A' (-W2 / sqrt(2)) (k = hidden, n = channel): column block cb2
      f16x8 w2g[LOSS == LOSS_MSE ? NKH : 1];
      if (LOSS == LOSS_MSE) {
#pragma unroll
        for (int ks = 0; ks < NKH; ++ks) {
          const int row = 32 * ks + 8 * g + (r >> 2), col = 16 * cb2 + 4 * (r & 3);
          w2g[ks] = cat44(ld_trt(&w2s[row * L2 + col]), ld_trt(&w2s[(row + 4) * L2 + col]));
        }
      }
      const float* ep = pb.eta_tok ? pb.eta_tok + (long long)p * pb.N + t0 : nullptr;
      typedef KT stgk_t __attribute__((ext_vector_type(SCH)));
      // per-lane LDS offsets (elements), the same for every tile; what varies
      // with the tile, the hidden block or the k-step is a uniform addend
      const int r4 = r >> 2, r3 = r & 3;
      const int offSt = st * LDK + (sc ^ kswz(st));                          // staging writes
      const int offK0 = r * LDK + ((8 * g) ^ kswz(r));                        // Z' operand, ks = 0 (+16 tb LDK)
      const int offK1 = r * LDK + ((32 + 8 * g) ^ kswz(r));                   // ks = 1
      const int offAw0 = (h0 + r) * LDT + ((8 * g) ^ tswz(r));                // A' writes (+16 hb LDT)
      const int offAw1 = (h0 + r) * LDT + ((8 * g + 4) ^ tswz(r));
      int offTr[2][2];                                                        // A' transposed reads (+32 ks LDT)
#pragma unroll
      for (int tb2 = 0; tb2 < 2; ++tb2)
#pragma unroll
        for (int o = 0; o < 2; ++o) {
          const int ar = 8 * g + r4 + 4 * o;
          offTr[tb2][o] = ar * LDT + (tok_col(16 * tb2 + 4 * r3) ^ tswz(ar));
        }
      const int offV = (4 * g + r4) * LDK + ((16 * cb2 + 4 * r3) ^ kswz(4 * g + r4));   // V reads (+16 tb2 LDK)
      const int offGc0 = (16 * cb2 + r) * LDT + ((8 * g) ^ tswz(r));          // G' writes, tb2 = 0
      const int offGc1 = (16 * cb2 + r) * LDT + ((8 * g + 4) ^ tswz(r));      // tb2 = 1
      // Rows past the end of the batch: their eta is 0, so their G' row is 0
      // and they add exactly nothing to dW1 and dW2, provided their keys and
      // values are finite.  Raw keys and values there are zeros or an earlier
      // tile's; normalised keys are zeroed (-mean * rstd alone can exceed the
      // f16 range when the variance is tiny).  Only a pair's last tile has such
      // rows, so full tiles skip the test.
      auto stage = [&](int i) {
        const int nn = (tile0 + i) * TT + st;
        if constexpr (KNORM) {
          stgk_t kh;
#pragma unroll
          for (int j = 0; j < SCH; ++j) kh[j] = (KT)__builtin_fmaf((float)kreg[j], kst[sc + j][0], kst[sc + j][1]);
          if ((tile0 + i + 1) * TT > nt && nn >= nt) kh = stgk_t{};
          *reinterpret_cast<stgk_t*>(&Kr[ring<NK>(i)][offSt]) = kh;
        } else {
          *reinterpret_cast<stg_t*>(&Kr[ring<NK>(i)][offSt]) = kreg;
        }
        *reinterpret_cast<stg_t*>(&Vr[ring<NV>(i)][offSt]) = vreg;
        if (sc == 0) eta_s[ring<NV>(i)][st] = nn < nt ? (ep ? ep[nn] : 1.0f) : 0.0f;
      };
      // forward of tile i in chunks of two hidden blocks: Z' (MFMA) ...
      constexpr int HB2 = NHB < 2 ? NHB : 2;
      constexpr int NCH = NHB / HB2;
      auto fwd_gemm = [&](int i, int hc, f32x4 (&z)[2][HB2]) {
        const KT* kt0 = Kr[ring<NK>(i)] + offK0;
        const KT* kt1 = Kr[ring<NK>(i)] + offK1;
#pragma unroll
        for (int tb = 0; tb < 2; ++tb)
#pragma unroll
          for (int hb = 0; hb < HB2; ++hb) z[tb][hb] = f32x4{0, 0, 0, 0};
#pragma unroll
        for (int ks = 0; ks < 2; ++ks)
#pragma unroll
          for (int tb = 0; tb < 2; ++tb) {
            const k8 a = ld8t((ks ? kt1 : kt0) + 16 * tb * LDK);
#pragma unroll
            for (int hb = 0; hb < HB2; ++hb) z[tb][hb] = mfma16(a, w1r[hc + hb][ks], z[tb][hb]);
          }
      };
      // ... then GELU: A' -> At, w -> Gp
      auto fwd_act = [&](int i, int hc, const f32x4 (&z)[2][HB2]) {
        f16* at0 = At[ring<NA>(i)] + offAw0;
        f16* at1 = At[ring<NA>(i)] + offAw1;
        h2* gpo = Gp[ring<NA>(i)] + lane * 4;
#pragma unroll
        for (int hb = 0; hb < HB2; ++hb) {
          const float zz[8] = {z[0][hb][0], z[0][hb][1], z[0][hb][2], z[0][hb][3],
                               z[1][hb][0], z[1][hb][1], z[1][hb][2], z[1][hb][3]};
          h2 av[4], gp[4];
          gelu_chains<GeluFitG, 4>(zz, av, gp);
          *reinterpret_cast<f16x4*>(at0 + 16 * (hc + hb) * LDT) = f16x4{av[0].x, av[0].y, av[1].x, av[1].y};
          *reinterpret_cast<f16x4*>(at1 + 16 * (hc + hb) * LDT) = f16x4{av[2].x, av[2].y, av[3].x, av[3].y};
          h2* gq = gpo + (q * NHB + hc + hb) * 256;
          *reinterpret_cast<f16x8*>(gq) =
              f16x8{gp[0].x, gp[0].y, gp[1].x, gp[1].y, gp[2].x, gp[2].y, gp[3].x, gp[3].y};
        }
      };
      // V - V_hat of tile i, token half tb2, channel block cb2: two MFMA chains,
      // one starting from V ...
      auto gp_issue = [&](int i, int tb2, f32x4& v0, f32x4& v1) {
        const bf16x4 vq = ld_trt(Vr[ring<NV>(i)] + offV + 16 * tb2 * LDK);
        v0 = f32x4{0, 0, 0, 0};
        v1 = f32x4{(float)vq[0], (float)vq[1], (float)vq[2], (float)vq[3]};
        if (LOSS == LOSS_MSE) {
          // A'[t = 16 tb2 + r][h = 32 ks + 8 g + j]
          const f16* alo = At[ring<NA>(i)] + offTr[tb2][0];
          const f16* ahi = At[ring<NA>(i)] + offTr[tb2][1];
#pragma unroll
          for (int ks = 0; ks < NKH; ++ks) {
            const f16x4 lo = ld_trt(alo + 32 * ks * LDT);
            const f16x4 hi = ld_trt(ahi + 32 * ks * LDT);
            if (ks & 1) v1 = mfma16(cat44(lo, hi), w2g[ks], v1);
            else v0 = mfma16(cat44(lo, hi), w2g[ks], v0);
          }
        }
      };
      // ... and G' = eta (V - V_hat) [MSE] or eta V [dot] -> Gc.  A full tile
      // without per-token rates has eta = 1 on every row.
      auto gp_fin = [&](int i, int tb2, const f32x4& v0, const f32x4& v1) {
        f32x4 gv = v0 + v1;
        if (ep || (tile0 + i + 1) * TT > nt) {
#pragma unroll
          for (int j = 0; j < 4; ++j) gv[j] *= eta_s[ring<NV>(i)][16 * tb2 + 4 * g + j];
        }
        *reinterpret_cast<f16x4*>(Gc[ring<NG>(i)] + (tb2 ? offGc1 : offGc0)) = pack4h(gv);
      };

      stage(0);
      prefetch(1);
      __syncthreads();
      // phase 0: forward of tile 0.  Each phase stages the next tile at its end,
      // from loads issued at the end of the phase before (a whole phase earlier)
#pragma unroll
      for (int c = 0; c < NCH; ++c) {
        f32x4 z[2][HB2];
        fwd_gemm(0, c * HB2, z);
        fwd_act(0, c * HB2, z);
      }
      if (1 < n) { stage(1); prefetch(2); }
      __syncthreads();
      // phases 1 .. n-1: forward of tile k interleaved with V_hat / G' of tile k-1,
      // so that the V_hat MFMA chains run under the GELU arithmetic
      for (int k = 1; k < n; ++k) {
        f32x4 va0, va1, vb0, vb1;
        f32x4 z[2][HB2];
        fwd_gemm(k, 0, z);
        gp_issue(k - 1, tbh(0), va0, va1);
        fwd_act(k, 0, z);
        if (NCH > 1) fwd_gemm(k, HB2, z);
        gp_fin(k - 1, tbh(0), va0, va1);
        if (NB2 > 1) gp_issue(k - 1, tbh(1), vb0, vb1);
        if (NCH > 1) fwd_act(k, HB2, z);
        if (NB2 > 1) gp_fin(k - 1, tbh(1), vb0, vb1);
        if (k + 1 < n) { stage(k + 1); prefetch(k + 2); }
        __syncthreads();
      }
      // phase n: V_hat / G' of the last tile; phase n+1: the consumers' last backward
#pragma unroll
      for (int b = 0; b < NB2; ++b) {
        f32x4 v0, v1;
        gp_issue(n - 1, tbh(b), v0, v1);
        gp_fin(n - 1, tbh(b), v0, v1);
      }
      __syncthreads();
      __syncthreads();
    } else {
      // ---------------- consumer ----------------
      // -W2 / sqrt(2) as the B operand of dA' = G' (-W2 / sqrt(2))^T (k = channel, n = hidden),
      // from the staged copy (overwritten from phase 0 on)
      f16x8 w2r[NHB][2];
#pragma unroll
      for (int hb = 0; hb < NHB; ++hb)
#pragma unroll
        for (int ks = 0; ks < 2; ++ks) w2r[hb][ks] = *reinterpret_cast<const f16x8*>(&w2s[(h0 + 16 * hb + r) * L2 + 32 * ks + 8 * g]);
      f32x4 acc1[4][NHB], acc2[NHB][4];
#pragma unroll
      for (int a = 0; a < 4; ++a)
#pragma unroll
        for (int b = 0; b < NHB; ++b) { acc1[a][b] = f32x4{0, 0, 0, 0}; acc2[b][a] = f32x4{0, 0, 0, 0}; }
      // per-lane LDS offsets (elements), as in the producer
      const int r4 = r >> 2, r3 = r & 3;
      const int offR0 = r * LDT + ((8 * g) ^ tswz(r));         // unit-major rows, token half 0 (+16 cb LDT)
      const int offR1 = r * LDT + ((8 * g + 4) ^ tswz(r));     // token half 1
      int offGt[2][2];                                          // G' transposed reads (+32 ks LDT)
#pragma unroll
      for (int tb = 0; tb < 2; ++tb)
#pragma unroll
        for (int o = 0; o < 2; ++o) {
          const int gr = 8 * g + r4 + 4 * o;
          offGt[tb][o] = gr * LDT + (tok_col(16 * tb + 4 * r3) ^ tswz(gr));
        }
      int offKt[4];                                             // K_hat transposed reads (+16 LDK for hi)
#pragma unroll
      for (int cb = 0; cb < 4; ++cb) offKt[cb] = (4 * g + r4) * LDK + ((16 * cb + 4 * r3) ^ kswz(4 * g + r4));
      auto backward = [&](int i) {
        const f16* gc = Gc[ring<NG>(i)];
        const f16* at = At[ring<NA>(i)] + h0 * LDT;
        const h2* gpi = Gp[ring<NA>(i)] + lane * 4;
        const KT* kt = Kr[ring<NK>(i)];
        // pass 1: dW2 += A'^T G' (G' as the B operand: k = token, n = channel)
        {
          f16x8 gb[4];
#pragma unroll
          for (int cb = 0; cb < 4; ++cb)
            gb[cb] = cat44(*reinterpret_cast<const f16x4*>(gc + offR0 + 16 * cb * LDT),
                           *reinterpret_cast<const f16x4*>(gc + offR1 + 16 * cb * LDT));
#pragma unroll
          for (int hb = 0; hb < NHB; ++hb) {
            // A'^T (m = hidden, k = token) from the unit-major tile
            const f16x8 aa = cat44(*reinterpret_cast<const f16x4*>(at + offR0 + 16 * hb * LDT),
                                   *reinterpret_cast<const f16x4*>(at + offR1 + 16 * hb * LDT));
#pragma unroll
            for (int cb = 0; cb < 4; ++cb) acc2[hb][cb] = mfma16(aa, gb[cb], acc2[hb][cb]);
          }
        }
        // pass 2: dA' = G' (-W2 / sqrt(2))^T (G' as the A operand: m = token, k = channel),
        // dZ' = dA' gelu'(Z)
        k8 dz[NHB];
        {
          f16x8 ga[2][2];
#pragma unroll
          for (int ks = 0; ks < 2; ++ks)
#pragma unroll
            for (int tb = 0; tb < 2; ++tb) {
              ga[ks][tb] = cat44(ld_trt(gc + offGt[tb][0] + 32 * ks * LDT), ld_trt(gc + offGt[tb][1] + 32 * ks * LDT));
            }
#pragma unroll
          for (int hb = 0; hb < NHB; ++hb) {
            f32x4 da[2] = {f32x4{0, 0, 0, 0}, f32x4{0, 0, 0, 0}};
#pragma unroll
            for (int ks = 0; ks < 2; ++ks)
#pragma unroll
              for (int tb = 0; tb < 2; ++tb) da[tb] = mfma16(ga[ks][tb], w2r[hb][ks], da[tb]);
            const f16x8 wv = *reinterpret_cast<const f16x8*>(gpi + (q * NHB + hb) * 256);
            const h2 wc[4] = {h2{wv[0], wv[1]}, h2{wv[2], wv[3]}, h2{wv[4], wv[5]}, h2{wv[6], wv[7]}};
            h2 gd[4];
            gelu_deriv_chains<GeluFitG, 4>(wc, gd);
            const h2 d0 = cvt_h2(da[0][0], da[0][1]) * gd[0], d1 = cvt_h2(da[0][2], da[0][3]) * gd[1];
            const h2 d2 = cvt_h2(da[1][0], da[1][1]) * gd[2], d3 = cvt_h2(da[1][2], da[1][3]) * gd[3];
            dz[hb][0] = (KT)(float)d0.x; dz[hb][1] = (KT)(float)d0.y; dz[hb][2] = (KT)(float)d1.x;
            dz[hb][3] = (KT)(float)d1.y; dz[hb][4] = (KT)(float)d2.x; dz[hb][5] = (KT)(float)d2.y;
            dz[hb][6] = (KT)(float)d3.x; dz[hb][7] = (KT)(float)d3.y;
          }
        }
        // pass 3: dW1 += K_hat^T dZ (K_hat^T as the A operand: m = channel, k = token)
#pragma unroll
        for (int cb = 0; cb < 4; ++cb) {
          const k8 ka = cat44(ld_trt(kt + offKt[cb]), ld_trt(kt + offKt[cb] + 16 * LDK));
#pragma unroll
          for (int hb = 0; hb < NHB; ++hb) acc1[cb][hb] = mfma16(ka, dz[hb], acc1[cb][hb]);
        }
      };
      __syncthreads();                           // the producers' prologue
      for (int k = 0; k < n + 2; ++k) {
        if (k >= 2) backward(k - 2);
        __syncthreads();
      }
      // partial of this (workgroup, pair) segment, [dW1 part | dW2 part], each
      // stored in register order: float4 ((q*4 + cb)*NHB + hb)*64 + lane holds
      // dW1[16cb + 4g + i][h0 + 16hb + r], float4 ((q*NHB + hb)*4 + cb)*64 + lane
      // holds dW2[h0 + 16hb + 4g + i][16cb + r] (i = 0..3), so every store
      // instruction writes 1 KB contiguously.  With G' the negated gradient,
      // acc2 holds A'^T G' = -sqrt(2) A^T G and acc1 holds K_hat^T dZ' =
      // K_hat^T dZ / sqrt(2).
      const float scale1 = scale * kSqrt2, scale2 = -scale * kRSqrt2;
      if (DIRECT && dw.readout && tile0 == 0 && n == tpp) {
        // fused readout of a whole pair: W* = W - dW straight from the
        // accumulators into the readout's LDS copies (over the A' and w
        // buffers, free once every wave has passed the loop's last barrier),
        // and to W_out; one row block at a time, the lane index opaque so that
        // none of this index arithmetic is hoisted into the main loop (the
        // step without the fused readout goes through the partial instead:
        // the extra global stores here spill registers in the main loop)
        int lane_o = lane;
        asm volatile("" : "+v"(lane_o));
        const int rr = lane_o & 15, gg = lane_o >> 4;
        constexpr int QL1 = HID + 16, QL2 = 80;
        bf16* w1q = reinterpret_cast<bf16*>(&At[0][0]);
        f16* w2q = reinterpret_cast<f16*>(&Gp[0][0]);
        const float* W2c = W.mat(1, bb, hh_);
        float* o1 = dw.out[0] ? dw.out[0] + pb.row(p) * D * HID : nullptr;
        float* o2 = dw.out[1] ? dw.out[1] + pb.row(p) * D * HID : nullptr;
#pragma unroll
        for (int cb = 0; cb < 4; ++cb) {
          float v[NHB][4];
#pragma unroll
          for (int hb = 0; hb < NHB; ++hb)
#pragma unroll
            for (int i = 0; i < 4; ++i) v[hb][i] = W1[(16 * cb + 4 * gg + i) * HID + h0 + 16 * hb + rr];
#pragma unroll
          for (int hb = 0; hb < NHB; ++hb)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
              const int c = 16 * cb + 4 * gg + i, hh = h0 + 16 * hb + rr;
              const float x = v[hb][i] - scale1 * acc1[cb][hb][i];
              w1q[c * QL1 + hh] = (bf16)(x * kZScaleQ);
              if (o1) o1[c * HID + hh] = x;
            }
          __builtin_amdgcn_sched_barrier(0);
        }
#pragma unroll
        for (int hb = 0; hb < NHB; ++hb) {
          float v[4][4];
#pragma unroll
          for (int cb = 0; cb < 4; ++cb)
#pragma unroll
            for (int i = 0; i < 4; ++i) v[cb][i] = W2c[(h0 + 16 * hb + 4 * gg + i) * D + 16 * cb + rr];
#pragma unroll
          for (int cb = 0; cb < 4; ++cb)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
              const int hh = h0 + 16 * hb + 4 * gg + i, c = 16 * cb + rr;
              const float x = v[cb][i] - scale2 * acc2[hb][cb][i];
              w2q[hh * QL2 + c] = (f16)(x * kW2ScaleQ);
              if (o2) o2[hh * D + c] = x;
            }
          __builtin_amdgcn_sched_barrier(0);
        }
      } else {
        f32x4* out = reinterpret_cast<f32x4*>(part + ((long long)blockIdx.x * J + (p - p_first)) * (2LL * D * HID));
#pragma unroll
        for (int cb = 0; cb < 4; ++cb)
#pragma unroll
          for (int hb = 0; hb < NHB; ++hb) out[((q * 4 + cb) * NHB + hb) * 64 + lane] = scale1 * acc1[cb][hb];
#pragma unroll
        for (int hb = 0; hb < NHB; ++hb)
#pragma unroll
          for (int cb = 0; cb < 4; ++cb) out[D * HID / 4 + ((q * NHB + hb) * 4 + cb) * 64 + lane] = scale2 * acc2[hb][cb];
      }
    }
    if (DIRECT && tile0 == 0 && n == tpp) {
      // this segment is the whole pair
      __syncthreads();
      constexpr int QL1 = HID + 16, QL2 = 80;
      static_assert(D * QL1 * sizeof(bf16) <= sizeof(At) && HID * QL2 * sizeof(f16) <= sizeof(Gp),
                    "the readout's weight copies fit the A' and w buffers");
      if (!dw.readout) {
        // direct step: every thread of the workgroup takes float4s of the
        // pair's partial, which this workgroup just wrote (L2-resident), and
        // applies W* = W - dW to the 4 weights each maps to (partial layout
        // above), in the natural layouts W1 [c][h] and W2 [h][c]
        const float4* pin =
            reinterpret_cast<const float4*>(part + ((long long)blockIdx.x * J + (p - p_first)) * (2LL * D * HID));
        const float* Wm[2] = {W1, W.mat(1, bb, hh_)};
        float* nx = dw.next + (long long)p * 2 * D * HID;
        constexpr int HALF = D * HID / 4;
        // float4 jj of the partial -> element offset of its i = 0 weight in
        // matrix jj / HALF and the stride over i
        auto map = [&](int jj, int& mat, int& base, int& step) {
          mat = jj >= HALF ? 1 : 0;
          const int jl = jj - mat * HALF, l = jl & 63, blk = jl >> 6, gg = l >> 4, rr = l & 15;
          if (mat == 0) {
            const int hb = blk % NHB, cb = (blk / NHB) & 3, qq = blk / (4 * NHB);
            base = (16 * cb + 4 * gg) * HID + qq * HP + 16 * hb + rr;
            step = HID;
          } else {
            const int cb = blk & 3, hb = (blk >> 2) % NHB, qq = blk / (4 * NHB);
            base = (qq * HP + 16 * hb + 4 * gg) * D + 16 * cb + rr;
            step = D;
          }
        };
        // eight float4s per thread at a time, every load of the batch issued
        // before its stores (the stores may alias the loads in the compiler's
        // view, so a plain loop would wait for each iteration's loads)
        // the thread index passes through an empty asm statement, so that the
        // compiler cannot hoist the (segment-invariant) index arithmetic below
        // to the kernel entry and keep it in registers through the main loops
        int tid_o = tid;
        asm volatile("" : "+v"(tid_o));
        constexpr int PER = 2 * HALF / NTH, UB = PER < 8 ? PER : 8;
        static_assert(2 * HALF % (NTH * UB) == 0, "the partial splits evenly into batches");
        for (int j0 = 0; j0 < PER; j0 += UB) {
          float4 dv[UB];
          float wv[UB][4];
          int mat[UB], base[UB], step[UB];
#pragma unroll
          for (int u = 0; u < UB; ++u) {
            const int jj = tid_o + NTH * (j0 + u);
            map(jj, mat[u], base[u], step[u]);
            dv[u] = pin[jj];
#pragma unroll
            for (int i = 0; i < 4; ++i) wv[u][i] = Wm[mat[u]][base[u] + i * step[u]];
          }
#pragma unroll
          for (int u = 0; u < UB; ++u) {
            float* nm = nx + mat[u] * D * HID;
            float* om = dw.out[mat[u]] ? dw.out[mat[u]] + pb.row(p) * D * HID : nullptr;
            const float d4[4] = {dv[u].x, dv[u].y, dv[u].z, dv[u].w};
#pragma unroll
            for (int i = 0; i < 4; ++i) {
              const int e = base[u] + i * step[u];
              const float x = wv[u][i] - d4[i];
              nm[e] = x;
              if (om) om[e] = x;
            }
          }
        }
      } else {
        // fused readout: the consumers have put W* into LDS in the readout's
        // layouts (over the A' and w buffers); O = F_W*(Q) of the pair's
        // tokens, split over all 2 NW waves in 16-token units (the readout
        // kernel's pass loop); the output staging blocks go over the key tiles
        static_assert(2 * NW * 16 * D * sizeof(bf16) <= sizeof(Kr), "output staging fits the key tiles");
        const int wq = __builtin_amdgcn_readfirstlane(tid >> 6);
        const int units = (pb.N + 15) >> 4;
        const int a_ = __builtin_amdgcn_readfirstlane(16 * (wq * units / (2 * NW)));
        const int b_ = __builtin_amdgcn_readfirstlane(min(pb.N, 16 * ((wq + 1) * units / (2 * NW))));
        const bf16* qp = (const bf16*)pb.q + (long long)p * pb.N * D;
        bf16* op = (bf16*)pb.o + (long long)p * pb.N * D;
        bf16* sb = reinterpret_cast<bf16*>(&Kr[0][0]) + wq * 16 * D;
        // the lane index passes through an empty asm statement so that the
        // readout's per-lane offsets are not hoisted into the main loops
        int lane_o = lane;
        asm volatile("" : "+v"(lane_o));
        readout_share<HID, (HID == 64 ? 1 : 2), (HID <= 128)>(reinterpret_cast<const bf16*>(&At[0][0]),
                                                             reinterpret_cast<const f16*>(&Gp[0][0]), sb, qp, op,
                                                             a_, b_, lane_o);
        __syncthreads();                      // LDS is the next segment's
      }
    }
    x = seg_end;
  }
}

// ---------------------------------------------------------------------------
// O = gelu(Q W1*) W2* with tokens on the MFMA n axis.
//
// One workgroup per CU (16 waves; 8 at width 64).  The (pair, token) space is
// cut into equal contiguous ranges, one per workgroup; a range covers one or
// more weight states (pair, chunk).  The workgroup stages each state's weights
// in LDS in their natural layouts (read transposed by the MFMA operand loads),
// the first two at once into two buffers, and splits the state's tokens over
// the waves in 16-token units, so every wave gets the same work to within 16
// tokens.  A wave walks its tokens 32 at a time (64 at width 64; shorter for
// the last piece) and prefetches the next piece's Q while computing.
//
// The first product runs on bf16 (Q is bf16); the second on f16, fed straight
// from the packed-f16 GELU: W1 is staged scaled by sqrt(2)/c, so the MFMA
// yields zh = sqrt(2) Z / c, and the output-clamped GELU gives zh Phi(Z) =
// (sqrt(2)/c) gelu(Z); W2 is staged scaled by c/sqrt(2) to compensate.
// Workgroup -> range mapping is XCD-aware: consecutive ranges (which share a
// pair's weights) are given to workgroups of the same XCD.
// waves per workgroup and 16-token blocks per pass: 16 waves of 32-token passes
// at widths 128 and 256; 8 waves of 64-token passes at width 64, where a pass
// is short and the wider one keeps more Q loads in flight (measured)
template <int HID> constexpr int kQW = HID == 64 ? 8 : 16;
template <int HID> constexpr int kQTB = HID == 64 ? 4 : 2;
template <int HID>
__global__ void __launch_bounds__(kQW<HID> * 64, 1)
k_mfma_query(Problem pb, WRef w0, const float* __restrict__ states, long long state_stride, int chunk, int span) {
  constexpr int QW = kQW<HID>, QTB = kQTB<HID>;
  constexpr int NTHR = QW * 64;
  constexpr int L1 = HID + 16;           // [c][h] row stride (16 mod 128: conflict-free transposed reads)
  constexpr int L2 = 80;                 // [h][c] row stride
  __shared__ __attribute__((aligned(16))) bf16 w1b[2][D * L1];
  __shared__ __attribute__((aligned(16))) f16 w2b[2][HID * L2];
  // per-wave staging of a 16-token output block (16 rows of 128 bytes, the
  // 16-byte chunks of row t XOR-permuted by t & 7), so that each output store
  // writes 8 whole rows (1 KB) instead of 32 bytes of 16 rows; at width 256
  // the weight buffers leave no room for it
  constexpr bool kStageO = HID <= 128;
  __shared__ __attribute__((aligned(16))) bf16 ob[kStageO ? QW : 1][kStageO ? 16 * D : 8];
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int r = lane & 15, g = lane >> 4;
  const int N = pb.N;
  const long long T = (long long)pb.B * pb.H * N;
  const int G = gridDim.x;
  const int L = (G % 8 == 0) ? (int)(blockIdx.x % 8) * (G / 8) + (int)(blockIdx.x / 8) : (int)blockIdx.x;
  long long t = (long long)L * T / G;
  const long long t_end = (long long)(L + 1) * T / G;

  // segment of the range starting at token tt: pair p, tokens [n0, n1) of it,
  // all read from one state (full batch: state 1, after the update; causal
  // chunk c: state c)
  struct Seg { int p, n0, n1, state; };
  auto seg_at = [&](long long tt) {
    Seg sg;
    sg.p = (int)(tt / N);
    sg.n0 = (int)(tt - (long long)sg.p * N);
    const int c = sg.n0 / span;
    sg.n1 = (int)min((long long)min(N, (c + 1) * span), sg.n0 + (t_end - tt));
    sg.state = chunk ? c : 1;
    return sg;
  };
  auto wptr = [&](const Seg& sg, int m) -> const float* {
    if (sg.state == 0) return w0.mat(m, sg.p / pb.H, sg.p % pb.H);
    return states + (sg.state - 1) * state_stride + (long long)sg.p * 2 * D * HID + (long long)m * D * HID;
  };
  // the weights of up to two segments are staged in LDS (two buffers), their
  // loads in flight together: a range that crosses a pair boundary pays one
  // staging latency, not two
  constexpr int NL = HID * D / (NTHR * 4);       // float4 loads per thread and matrix
  static_assert(HID * D % (NTHR * 4) == 0, "weights split evenly over the threads");
  auto stage_store = [&](int buf, const float4 (&a)[NL], const float4 (&b)[NL]) {
#pragma unroll
    for (int j = 0; j < NL; ++j) {
      const int e = 4 * (tid + NTHR * j);
      const int c1 = e / HID, h1 = e % HID;         // W1 [c][h]
      const int h2_ = e / D, c2 = e % D;             // W2 [h][c]
      *reinterpret_cast<bf16x4*>(&w1b[buf][c1 * L1 + h1]) = bf16x4{
          (bf16)(a[j].x * kZScaleQ), (bf16)(a[j].y * kZScaleQ), (bf16)(a[j].z * kZScaleQ), (bf16)(a[j].w * kZScaleQ)};
      *reinterpret_cast<f16x4*>(&w2b[buf][h2_ * L2 + c2]) =
          f16x4{(f16)(b[j].x * kW2ScaleQ), (f16)(b[j].y * kW2ScaleQ), (f16)(b[j].z * kW2ScaleQ), (f16)(b[j].w * kW2ScaleQ)};
    }
  };
  auto stage_load = [&](const Seg& sg, float4 (&a)[NL], float4 (&b)[NL]) {
    const float4* W1 = reinterpret_cast<const float4*>(wptr(sg, 0));
    const float4* W2 = reinterpret_cast<const float4*>(wptr(sg, 1));
#pragma unroll
    for (int j = 0; j < NL; ++j) { a[j] = W1[tid + NTHR * j]; b[j] = W2[tid + NTHR * j]; }
  };
  if (t < t_end) {
    const Seg s0 = seg_at(t);
    const long long t1 = t + (s0.n1 - s0.n0);
    float4 a0[NL], b0[NL], a1[NL], b1[NL];
    stage_load(s0, a0, b0);
    if (t1 < t_end) stage_load(seg_at(t1), a1, b1);
    stage_store(0, a0, b0);
    if (t1 < t_end) stage_store(1, a1, b1);
    __syncthreads();
  }

  for (int si = 0; t < t_end; ++si) {
    const Seg sg = seg_at(t);
    const int p = sg.p, n0 = sg.n0, n1 = sg.n1;
    const int buf = si & 1;
    if (si >= 2) {                       // third and later segments: stage in place
      float4 a[NL], b[NL];
      stage_load(sg, a, b);
      __syncthreads();                   // every wave is done with segment si - 2
      stage_store(buf, a, b);
      __syncthreads();
    }
    // the segment's work, with the buffer a compile-time constant (LDS
    // addresses stay lane offset + immediate)
    auto segment = [&](auto bufc) {
    constexpr int BUF = decltype(bufc)::value;
    const bf16* w1s = w1b[BUF];
    const f16* w2s = w2b[BUF];

    const int units = (n1 - n0 + 15) >> 4;
    // the wave's share (wave-uniform: kept in scalar registers, so the loop
    // below branches on scalars, not on exec masks)
    const int wu = __builtin_amdgcn_readfirstlane(w);
    const int a_ = __builtin_amdgcn_readfirstlane(n0 + 16 * (wu * units / QW));
    const int b_ = __builtin_amdgcn_readfirstlane(min(n1, n0 + 16 * ((wu + 1) * units / QW)));
    const bf16* qp = (const bf16*)pb.q + (long long)p * N * D;
    bf16* op = (bf16*)pb.o + (long long)p * N * D;
    readout_share<HID, QTB, kStageO>(w1s, w2s, kStageO ? ob[w] : nullptr, qp, op, a_, b_, lane);
    };
    if (buf == 0) segment(std::integral_constant<int, 0>{});
    else segment(std::integral_constant<int, 1>{});
    t += n1 - n0;
  }
}

template <int HID, bool DIRECT>
void launch_grad_hd(const Problem& pb, const WRef& W, int t0, int nt, int G, int J, float scale,
                    const float* spart, int S_stats, float eps, float* part, const GradDirect& dw, hipStream_t st) {
  constexpr int NW = kGradWaves<HID>;
  const dim3 grid(G), block(128 * NW);
  if (pb.loss == LOSS_MSE) {
    if (spart)
      hipLaunchKernelGGL((k_mfma_grad<HID, LOSS_MSE, true, NW, DIRECT>), grid, block, 0, st, pb, W, t0, nt, J, scale,
                         spart, S_stats, eps, part, dw);
    else
      hipLaunchKernelGGL((k_mfma_grad<HID, LOSS_MSE, false, NW, DIRECT>), grid, block, 0, st, pb, W, t0, nt, J, scale,
                         spart, S_stats, eps, part, dw);
  } else {
    if (spart)
      hipLaunchKernelGGL((k_mfma_grad<HID, LOSS_DOT, true, NW, DIRECT>), grid, block, 0, st, pb, W, t0, nt, J, scale,
                         spart, S_stats, eps, part, dw);
    else
      hipLaunchKernelGGL((k_mfma_grad<HID, LOSS_DOT, false, NW, DIRECT>), grid, block, 0, st, pb, W, t0, nt, J, scale,
                         spart, S_stats, eps, part, dw);
  }
}
template <int HID>
void launch_grad_h(const Problem& pb, const WRef& W, int t0, int nt, int G, int J, float scale,
                   const float* spart, int S_stats, float eps, float* part, const GradDirect& dw, hipStream_t st) {
  if (dw.next) launch_grad_hd<HID, true>(pb, W, t0, nt, G, J, scale, spart, S_stats, eps, part, dw, st);
  else launch_grad_hd<HID, false>(pb, W, t0, nt, G, J, scale, spart, S_stats, eps, part, dw, st);
}

}  // namespace

bool mfma_full_supported(const Problem& pb) {
  return pb.bf16 && pb.inner == INNER_MLP && pb.d == D && (pb.hid == 64 || pb.hid == 128 || pb.hid == 256);
}

bool mfma_query_supported(const Problem& pb) { return mfma_full_supported(pb); }

// grid of the stream-K gradient kernel: one workgroup per CU (two for hidden
// width 64, whose workgroups fit twice), never more workgroups than tiles
void mfma_grad_geometry(const Problem& pb, int nt, int* G, int* J, int* tiles_per_pair) {
  const int P = pb.B * pb.H;
  const int tpp = (nt + TT - 1) / TT;
  *tiles_per_pair = tpp;
  sk_geometry(P, tpp, (long long)device_cu_count() * (pb.hid == 64 ? kGradBlocksPerCU<64> : 1), G, J);
}

// one pair per workgroup in a single round that fills at least half the
// slots (measured on the ViT-S shape, 384 pairs of 196 tokens: at width 64,
// one round of 384 of 512 slots, 49 -> 43 us per step; at width 256 the two
// rounds of 384 over 256 slots only matched the stream-K split)
bool mfma_grad_direct_fits(const Problem& pb) {
  const long long slots = (long long)device_cu_count() * (pb.hid == 64 ? kGradBlocksPerCU<64> : 1);
  const long long P = (long long)pb.B * pb.H;
  return 2 * P >= slots && P <= slots;
}

long long mfma_grad_split_pairs(const Problem& pb, int nt) {
  int G, J, tpp;
  mfma_grad_geometry(pb, nt, &G, &J, &tpp);
  const long long P = (long long)pb.B * pb.H, C = P * (tpp + kSkAlpha);
  long long split = 0;
  for (long long p = 0; p < P; ++p) {
    long long q0, q1;
    sk_pair_groups(p, tpp, G, C, &q0, &q1);
    split += q0 != q1;
  }
  return split;
}

void launch_mfma_full_grad(const Problem& pb, const WRef& W, int t0, int nt, float scale, const float* spart,
                           int S_stats, float eps, float* part, const GradDirect* direct, bool one_round,
                           hipStream_t st) {
  int G, J, tpp;
  GradDirect dw{nullptr, {nullptr, nullptr}, 0};
  if (direct) dw = *direct;
  if (one_round) {
    // G = pairs: on the stream-K cost line every workgroup's range is then
    // exactly one pair's tiles
    G = pb.B * pb.H;
    J = 1;
  } else {
    mfma_grad_geometry(pb, nt, &G, &J, &tpp);
  }
  switch (pb.hid) {
    case 64: launch_grad_h<64>(pb, W, t0, nt, G, J, scale, spart, S_stats, eps, part, dw, st); break;
    case 128: launch_grad_h<128>(pb, W, t0, nt, G, J, scale, spart, S_stats, eps, part, dw, st); break;
    default: launch_grad_h<256>(pb, W, t0, nt, G, J, scale, spart, S_stats, eps, part, dw, st); break;
  }
}

void launch_mfma_query(const Problem& pb, const WRef& w0, const float* states, long long state_stride, int nchunks,
                       int chunk, hipStream_t st) {
  (void)nchunks;
  const int span = chunk ? (chunk < pb.N ? chunk : pb.N) : pb.N;
  // one workgroup per CU, fewer when there are not 128 tokens for each (with
  // many short pairs every CU is worth using: a workgroup's time is mostly
  // the staging of the weights of the pairs it touches, one per segment)
  const long long T = (long long)pb.B * pb.H * pb.N;
  long long G = device_cu_count();
  if (G > (T + 127) / 128) G = (T + 127) / 128;
  if (G < 1) G = 1;
  switch (pb.hid) {
    case 64: hipLaunchKernelGGL((k_mfma_query<64>), dim3((unsigned)G), dim3(kQW<64> * 64), 0, st, pb, w0, states, state_stride, chunk, span); break;
    case 128: hipLaunchKernelGGL((k_mfma_query<128>), dim3((unsigned)G), dim3(kQW<128> * 64), 0, st, pb, w0, states, state_stride, chunk, span); break;
    default: hipLaunchKernelGGL((k_mfma_query<256>), dim3((unsigned)G), dim3(kQW<256> * 64), 0, st, pb, w0, states, state_stride, chunk, span); break;
  }
}

}  // namespace ttt
