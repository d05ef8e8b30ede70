// bf16 MFMA kernels of the GELU-MLP inner model, head dimension 64, hidden
// width 64/128/256 (gfx950, wave64, v_mfma_f32_16x16x32_bf16, fp32 accumulate).
//
// k_mfma_grad: steps (i)-(ii) of one inner update (ViT3 summary page, section
// 02), fused per 32-token tile:
//     K_hat = (K - mu) * rstd                     key instance norm (TvS page)
//     Z  = K_hat W1,  A = gelu(Z),  V_hat = A W2   forward on the keys
//     G' = eta_n (V_hat - V)   [MSE]  |  -eta_n V  [dot]   (constant 2/(n_b d) and
//                                                         the scalar eta folded at the end)
//     dW2 += A^T G',  dA = G' W2^T,  dZ = dA * gelu'(Z),  dW1 += K_hat^T dZ
// Each of the 4 waves owns a quarter of the hidden units (its slice of Z, A,
// dA, dZ, dW1, dW2); the two products that mix hidden units (V_hat = A W2 and
// the K_hat^T / G'^T operands) go through LDS.  The token range of all (b, h)
// pairs is cut evenly over the grid ("stream-K"): a workgroup that crosses a
// pair boundary writes one fp32 partial per pair it touched, and the update
// kernel adds them in a fixed order, so the result is run-to-run identical.
//
// k_mfma_query: step (iii), O = gelu(Q W1*) W2*, with tokens on the MFMA lane
// axis so that both products chain through registers; W1*, W2* sit in LDS.
//
// GELU here is z * sigma(y(z)), y = z (a + b z^2 + c z^4), a logistic fit of
// the normal CDF (max |error| 3.7e-5 on gelu, 9.3e-5 on gelu', far below the
// bf16 rounding of the MFMA operands); the fp32 kernels use the exact erf form.
#include "ttt_internal.h"

namespace ttt {

namespace {

constexpr int D = 64;
constexpr int TT = 32;            // tokens per tile
constexpr int NWAVE = 4;
constexpr int NTHR = NWAVE * 64;
// LDS row strides (bf16 elements), padded against bank conflicts
constexpr int KRS = D + 8;        // [T][D] tiles
constexpr int KCS = TT + 4;       // [D][T] tiles

__device__ __forceinline__ f32x4 mfma16(const bf16x8& a, const bf16x8& b, const f32x4& c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

// logistic fit of Phi: y = z (A + B t + C t^2), t = z^2, pre-scaled by -log2(e)
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kGa = 1.59484567f, kGb = 7.40075326e-2f, kGc = -6.94974947e-4f;
constexpr float kPa = -kGa * kLog2e, kPb = -kGb * kLog2e, kPc = -kGc * kLog2e;
constexpr float kDa = kGa, kDb = 3.0f * kGb, kDc = 5.0f * kGc;

__device__ __forceinline__ float sig_of(float zc, float t) {
  const float p = __builtin_fmaf(t, __builtin_fmaf(t, kPc, kPb), kPa);
  const float e = __builtin_amdgcn_exp2f(zc * p);
  return __builtin_amdgcn_rcpf(1.0f + e);
}

__device__ __forceinline__ float gelu_fast(float z) {
  const float zc = __builtin_amdgcn_fmed3f(z, -9.0f, 9.0f);
  return z * sig_of(zc, zc * zc);
}

__device__ __forceinline__ void gelu_fast2(float z, float& a, float& gp) {
  const float zc = __builtin_amdgcn_fmed3f(z, -9.0f, 9.0f);
  const float t = zc * zc;
  const float s = sig_of(zc, t);
  a = z * s;
  const float yd = __builtin_fmaf(t, __builtin_fmaf(t, kDc, kDb), kDa);
  const float ss = __builtin_fmaf(-s, s, s);
  gp = __builtin_fmaf(zc * yd, ss, s);
}

__device__ __forceinline__ bf16x8 ld8(const bf16* p) { return *reinterpret_cast<const bf16x8*>(p); }
__device__ __forceinline__ bf16x4 ld4(const bf16* p) { return *reinterpret_cast<const bf16x4*>(p); }
__device__ __forceinline__ bf16x8 cat44(const bf16x4& x, const bf16x4& y) {
  bf16x8 r;
#pragma unroll
  for (int i = 0; i < 4; ++i) { r[i] = x[i]; r[4 + i] = y[i]; }
  return r;
}
__device__ __forceinline__ bf16x8 pack8(const f32x4& x, const f32x4& y) {
  bf16x8 r;
#pragma unroll
  for (int i = 0; i < 4; ++i) { r[i] = (bf16)x[i]; r[4 + i] = (bf16)y[i]; }
  return r;
}

// bf16 copy of one pair's weights (layout BF_MLP3): [W1t (h x d) | W2 (h x d) | W2t (d x h)]
struct Bf3 {
  const bf16* w1t; const bf16* w2; const bf16* w2t;
};
__device__ __forceinline__ Bf3 bf3_of(const bf16* base, int p, int hid) {
  const long long m = (long long)D * hid;
  const bf16* b = base + (long long)p * 3 * m;
  return {b, b + m, b + 2 * m};
}

// ---------------------------------------------------------------------------
template <int HID, int LOSS>
__global__ void __launch_bounds__(NTHR, 1)
k_mfma_grad(Problem pb, const bf16* __restrict__ wbf, int t0, int nt, int J, float scale,
            float* __restrict__ part) {
  constexpr int HW = HID / NWAVE;      // hidden units per wave
  constexpr int NHB = HW / 16;         // 16-wide hidden blocks per wave
  constexpr int NKH = HID / 32;        // k-steps over the hidden width
  constexpr int ATS = HID + 8;
  __shared__ __attribute__((aligned(16))) bf16 Kr[TT * KRS];
  __shared__ __attribute__((aligned(16))) bf16 Kc[D * KCS];
  __shared__ __attribute__((aligned(16))) bf16 Vc[D * KCS];
  __shared__ __attribute__((aligned(16))) bf16 Gr[TT * KRS];
  __shared__ __attribute__((aligned(16))) bf16 Gc[D * KCS];
  __shared__ __attribute__((aligned(16))) bf16 At[LOSS == LOSS_MSE ? TT * ATS : 8];
  __shared__ float eta_s[TT];

  const int tid = threadIdx.x;
  const int lane = tid & 63, w = tid >> 6;
  const int r = lane & 15, g = lane >> 4;
  const int h0 = w * HW;
  // staging role: token row st, channels 8*sc .. 8*sc+7
  const int st = tid >> 3, sc = tid & 7;

  const int P = pb.B * pb.H;
  const int tpp = (nt + TT - 1) / TT;
  const long long total = (long long)P * tpp;
  const long long G = gridDim.x;
  const long long begin = (long long)blockIdx.x * total / G;
  const long long end = (long long)(blockIdx.x + 1) * total / G;
  const int p_first = (int)(begin / tpp);

  const bf16* kin = (const bf16*)pb.k;
  const bf16* vin = (const bf16*)pb.v;

  long long x = begin;
  while (x < end) {
    const int p = (int)(x / tpp);
    const int tile0 = (int)(x - (long long)p * tpp);
    const long long seg_end = end < (long long)(p + 1) * tpp ? end : (long long)(p + 1) * tpp;
    const int tile1 = (int)(seg_end - (long long)p * tpp);

    // ---- per-pair constants: weight fragments (registers) and key statistics
    const Bf3 wb = bf3_of(wbf, p, HID);
    bf16x8 w1r[NHB][2], w2r[NHB][2], w2c[NKH];
#pragma unroll
    for (int hb = 0; hb < NHB; ++hb)
#pragma unroll
      for (int ks = 0; ks < 2; ++ks) {
        w1r[hb][ks] = ld8(wb.w1t + (long long)(h0 + 16 * hb + r) * D + 32 * ks + 8 * g);
        w2r[hb][ks] = ld8(wb.w2 + (long long)(h0 + 16 * hb + r) * D + 32 * ks + 8 * g);
      }
    if (LOSS == LOSS_MSE) {
#pragma unroll
      for (int ks = 0; ks < NKH; ++ks) w2c[ks] = ld8(wb.w2t + (long long)(16 * w + r) * HID + 32 * ks + 8 * g);
    }
    float mu[8], rs[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) { mu[j] = 0.f; rs[j] = 1.f; }
    if (pb.stats) {
      const float* s = pb.stats + ((long long)p * D + 8 * sc) * 2;
#pragma unroll
      for (int j = 0; j < 8; ++j) { mu[j] = s[2 * j]; rs[j] = s[2 * j + 1]; }
    }
    const bf16* kp = kin + ((long long)p * pb.N + t0) * D;
    const bf16* vp = vin + ((long long)p * pb.N + t0) * D;
    const float* ep = pb.eta_tok ? pb.eta_tok + (long long)p * pb.N + t0 : nullptr;

    f32x4 acc1[4][NHB], acc2[NHB][4];
#pragma unroll
    for (int a = 0; a < 4; ++a)
#pragma unroll
      for (int b = 0; b < NHB; ++b) { acc1[a][b] = f32x4{0, 0, 0, 0}; acc2[b][a] = f32x4{0, 0, 0, 0}; }

    // prefetch of the first tile's rows
    bf16x8 kreg = {}, vreg = {};
    {
      const int n = tile0 * TT + st;
      if (n < nt) { kreg = ld8(kp + (long long)n * D + 8 * sc); vreg = ld8(vp + (long long)n * D + 8 * sc); }
    }

    for (int tile = tile0; tile < tile1; ++tile) {
      const int n = tile * TT + st;
      const bool live = n < nt;
      // ---- stage K_hat (both layouts), V (channel-major), eta
      {
        bf16x8 kh;
#pragma unroll
        for (int j = 0; j < 8; ++j) kh[j] = live ? (bf16)(((float)kreg[j] - mu[j]) * rs[j]) : (bf16)0.f;
        *reinterpret_cast<bf16x8*>(&Kr[st * KRS + 8 * sc]) = kh;
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          Kc[(8 * sc + j) * KCS + st] = kh[j];
          Vc[(8 * sc + j) * KCS + st] = live ? vreg[j] : (bf16)0.f;
        }
        if (sc == 0) eta_s[st] = live ? (ep ? ep[n] : 1.0f) : 0.0f;
      }
      // prefetch the next tile (lands while this one computes)
      {
        const int nn = (tile + 1) * TT + st;
        if (tile + 1 < tile1 && nn < nt) {
          kreg = ld8(kp + (long long)nn * D + 8 * sc);
          vreg = ld8(vp + (long long)nn * D + 8 * sc);
        }
      }
      __syncthreads();

      // ---- Z = K_hat W1 (this wave's hidden slice), A = gelu(Z), gp = gelu'(Z)
      f32x4 z[2][NHB];
#pragma unroll
      for (int tb = 0; tb < 2; ++tb)
#pragma unroll
        for (int hb = 0; hb < NHB; ++hb) z[tb][hb] = f32x4{0, 0, 0, 0};
#pragma unroll
      for (int ks = 0; ks < 2; ++ks)
#pragma unroll
        for (int tb = 0; tb < 2; ++tb) {
          const bf16x8 a = ld8(&Kr[(16 * tb + r) * KRS + 32 * ks + 8 * g]);
#pragma unroll
          for (int hb = 0; hb < NHB; ++hb) z[tb][hb] = mfma16(a, w1r[hb][ks], z[tb][hb]);
        }
      f32x4 gp[2][NHB];
      bf16x8 apk[NHB];
#pragma unroll
      for (int hb = 0; hb < NHB; ++hb) {
        f32x4 av[2];
#pragma unroll
        for (int tb = 0; tb < 2; ++tb)
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            float a_, g_;
            gelu_fast2(z[tb][hb][i], a_, g_);
            av[tb][i] = a_;
            gp[tb][hb][i] = g_;
          }
        apk[hb] = pack8(av[0], av[1]);
      }
      if (LOSS == LOSS_MSE) {
        // A^T -> LDS in token-major layout for V_hat = A W2
#pragma unroll
        for (int hb = 0; hb < NHB; ++hb)
#pragma unroll
          for (int j = 0; j < 8; ++j) {
            const int t = (j < 4) ? 4 * g + j : 16 + 4 * g + (j - 4);
            At[t * ATS + h0 + 16 * hb + r] = apk[hb][j];
          }
      }
      __syncthreads();

      // ---- G' for (t = 16 tb + 4 g + i, c = 16 w + r)
      {
        f32x4 gv[2];
        if (LOSS == LOSS_MSE) {
          f32x4 vh[2] = {f32x4{0, 0, 0, 0}, f32x4{0, 0, 0, 0}};
#pragma unroll
          for (int ks = 0; ks < NKH; ++ks)
#pragma unroll
            for (int tb = 0; tb < 2; ++tb)
              vh[tb] = mfma16(ld8(&At[(16 * tb + r) * ATS + 32 * ks + 8 * g]), w2c[ks], vh[tb]);
#pragma unroll
          for (int tb = 0; tb < 2; ++tb) {
            const bf16x4 vv = ld4(&Vc[(16 * w + r) * KCS + 16 * tb + 4 * g]);
#pragma unroll
            for (int i = 0; i < 4; ++i) gv[tb][i] = eta_s[16 * tb + 4 * g + i] * (vh[tb][i] - (float)vv[i]);
          }
        } else {
#pragma unroll
          for (int tb = 0; tb < 2; ++tb) {
            const bf16x4 vv = ld4(&Vc[(16 * w + r) * KCS + 16 * tb + 4 * g]);
#pragma unroll
            for (int i = 0; i < 4; ++i) gv[tb][i] = -eta_s[16 * tb + 4 * g + i] * (float)vv[i];
          }
        }
#pragma unroll
        for (int tb = 0; tb < 2; ++tb) {
          bf16x4 gq;
#pragma unroll
          for (int i = 0; i < 4; ++i) gq[i] = (bf16)gv[tb][i];
          *reinterpret_cast<bf16x4*>(&Gc[(16 * w + r) * KCS + 16 * tb + 4 * g]) = gq;
#pragma unroll
          for (int i = 0; i < 4; ++i) Gr[(16 * tb + 4 * g + i) * KRS + 16 * w + r] = gq[i];
        }
      }
      __syncthreads();

      // ---- dW2 += A^T G'
#pragma unroll
      for (int cb = 0; cb < 4; ++cb) {
        const bf16x8 b = cat44(ld4(&Gc[(16 * cb + r) * KCS + 4 * g]), ld4(&Gc[(16 * cb + r) * KCS + 16 + 4 * g]));
#pragma unroll
        for (int hb = 0; hb < NHB; ++hb) acc2[hb][cb] = mfma16(apk[hb], b, acc2[hb][cb]);
      }
      // ---- dA = G' W2^T, dZ = dA * gelu'(Z)
      bf16x8 dzp[NHB];
      {
        f32x4 da[2][NHB];
#pragma unroll
        for (int tb = 0; tb < 2; ++tb)
#pragma unroll
          for (int hb = 0; hb < NHB; ++hb) da[tb][hb] = f32x4{0, 0, 0, 0};
#pragma unroll
        for (int ks = 0; ks < 2; ++ks)
#pragma unroll
          for (int tb = 0; tb < 2; ++tb) {
            const bf16x8 a = ld8(&Gr[(16 * tb + r) * KRS + 32 * ks + 8 * g]);
#pragma unroll
            for (int hb = 0; hb < NHB; ++hb) da[tb][hb] = mfma16(a, w2r[hb][ks], da[tb][hb]);
          }
#pragma unroll
        for (int hb = 0; hb < NHB; ++hb) {
          f32x4 d0, d1;
#pragma unroll
          for (int i = 0; i < 4; ++i) { d0[i] = da[0][hb][i] * gp[0][hb][i]; d1[i] = da[1][hb][i] * gp[1][hb][i]; }
          dzp[hb] = pack8(d0, d1);
        }
      }
      // ---- dW1 += K_hat^T dZ
#pragma unroll
      for (int cb = 0; cb < 4; ++cb) {
        const bf16x8 a = cat44(ld4(&Kc[(16 * cb + r) * KCS + 4 * g]), ld4(&Kc[(16 * cb + r) * KCS + 16 + 4 * g]));
#pragma unroll
        for (int hb = 0; hb < NHB; ++hb) acc1[cb][hb] = mfma16(a, dzp[hb], acc1[cb][hb]);
      }
      __syncthreads();
    }

    // ---- partial of this (workgroup, pair) segment
    float* out = part + ((long long)blockIdx.x * J + (p - p_first)) * (2LL * D * HID);
#pragma unroll
    for (int cb = 0; cb < 4; ++cb)
#pragma unroll
      for (int hb = 0; hb < NHB; ++hb)
#pragma unroll
        for (int i = 0; i < 4; ++i)
          out[(16 * cb + 4 * g + i) * HID + h0 + 16 * hb + r] = scale * acc1[cb][hb][i];
#pragma unroll
    for (int hb = 0; hb < NHB; ++hb)
#pragma unroll
      for (int cb = 0; cb < 4; ++cb)
#pragma unroll
        for (int i = 0; i < 4; ++i)
          out[(long long)D * HID + (h0 + 16 * hb + 4 * g + i) * D + 16 * cb + r] = scale * acc2[hb][cb][i];
    x = seg_end;
  }
}

// ---------------------------------------------------------------------------
// O = gelu(Q W1*) W2* with tokens on the MFMA n axis.  One workgroup = one
// pair's token range; W1t and W2t of the pair's state are staged in LDS.
constexpr int QTOK = 64;                 // tokens per wave iteration
template <int HID>
__global__ void __launch_bounds__(NTHR, 2)
k_mfma_query(Problem pb, const bf16* __restrict__ wstates, long long state_stride, int chunk, int span,
             int groups, int tok_per_wg) {
  constexpr int W1S = D + 8;             // W1t rows [HID][D]
  constexpr int W2S = HID + 4;           // W2t rows [D][HID]
  __shared__ __attribute__((aligned(16))) bf16 w1s[HID * W1S];
  __shared__ __attribute__((aligned(16))) bf16 w2s[D * W2S];
  const int p = blockIdx.y;
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int r = lane & 15, g = lane >> 4;
  // blockIdx.x = (batch of tokens c, group inside it); full batch: one batch of N
  const int c = blockIdx.x / groups, grp = blockIdx.x % groups;
  const int c0 = c * span;
  const int n0 = c0 + grp * tok_per_wg;
  const int n1 = min(min(pb.N, c0 + span), n0 + tok_per_wg);
  if (n0 >= n1) return;
  // full batch reads state 1 (after the update); causal chunk c reads state c
  const int state = chunk ? c : 1;
  const Bf3 wb = bf3_of(wstates + state * state_stride, p, HID);
  for (int e = tid * 8; e < HID * D; e += NTHR * 8) {
    const int hh = e / D, cc = e % D;
    *reinterpret_cast<bf16x8*>(&w1s[hh * W1S + cc]) = ld8(wb.w1t + e);
  }
  for (int e = tid * 8; e < HID * D; e += NTHR * 8) {
    const int cc = e / HID, hh = e % HID;
    *reinterpret_cast<bf16x8*>(&w2s[cc * W2S + hh]) = ld8(wb.w2t + e);
  }
  __syncthreads();
  const bf16* qp = (const bf16*)pb.q + (long long)p * pb.N * D;
  bf16* op = (bf16*)pb.o + (long long)p * pb.N * D;
  for (int base = n0 + w * QTOK; base < n1; base += NWAVE * QTOK) {
    bf16x8 qb[4][2];
#pragma unroll
    for (int tb = 0; tb < 4; ++tb)
#pragma unroll
      for (int ks = 0; ks < 2; ++ks) {
        const int n = base + 16 * tb + r;
        qb[tb][ks] = n < n1 ? ld8(qp + (long long)n * D + 32 * ks + 8 * g) : bf16x8{};
      }
    f32x4 o[4][4];
#pragma unroll
    for (int cb = 0; cb < 4; ++cb)
#pragma unroll
      for (int tb = 0; tb < 4; ++tb) o[cb][tb] = f32x4{0, 0, 0, 0};
#pragma unroll 2
    for (int hc = 0; hc < HID / 32; ++hc) {
      f32x4 zt[2][4];
#pragma unroll
      for (int u = 0; u < 2; ++u)
#pragma unroll
        for (int tb = 0; tb < 4; ++tb) zt[u][tb] = f32x4{0, 0, 0, 0};
#pragma unroll
      for (int ks = 0; ks < 2; ++ks)
#pragma unroll
        for (int u = 0; u < 2; ++u) {
          const bf16x8 a = ld8(&w1s[(32 * hc + 16 * u + r) * W1S + 32 * ks + 8 * g]);
#pragma unroll
          for (int tb = 0; tb < 4; ++tb) zt[u][tb] = mfma16(a, qb[tb][ks], zt[u][tb]);
        }
      bf16x8 ab[4];
#pragma unroll
      for (int tb = 0; tb < 4; ++tb) {
        f32x4 a0, a1;
#pragma unroll
        for (int i = 0; i < 4; ++i) { a0[i] = gelu_fast(zt[0][tb][i]); a1[i] = gelu_fast(zt[1][tb][i]); }
        ab[tb] = pack8(a0, a1);
      }
#pragma unroll
      for (int cb = 0; cb < 4; ++cb) {
        const bf16x8 a = cat44(ld4(&w2s[(16 * cb + r) * W2S + 32 * hc + 4 * g]),
                               ld4(&w2s[(16 * cb + r) * W2S + 32 * hc + 16 + 4 * g]));
#pragma unroll
        for (int tb = 0; tb < 4; ++tb) o[cb][tb] = mfma16(a, ab[tb], o[cb][tb]);
      }
    }
#pragma unroll
    for (int tb = 0; tb < 4; ++tb) {
      const int n = base + 16 * tb + r;
      if (n < n1) {
#pragma unroll
        for (int cb = 0; cb < 4; ++cb) {
          bf16x4 v;
#pragma unroll
          for (int i = 0; i < 4; ++i) v[i] = (bf16)o[cb][tb][i];
          *reinterpret_cast<bf16x4*>(op + (long long)n * D + 16 * cb + 4 * g) = v;
        }
      }
    }
  }
}

template <int HID>
void launch_grad_h(const Problem& pb, const bf16* wbf, int t0, int nt, int G, int J, float scale, float* part,
                   hipStream_t st) {
  if (pb.loss == LOSS_MSE)
    hipLaunchKernelGGL((k_mfma_grad<HID, LOSS_MSE>), dim3(G), dim3(NTHR), 0, st, pb, wbf, t0, nt, J, scale, part);
  else
    hipLaunchKernelGGL((k_mfma_grad<HID, LOSS_DOT>), dim3(G), dim3(NTHR), 0, st, pb, wbf, t0, nt, J, scale, part);
}

}  // namespace

bool mfma_full_supported(const Problem& pb) {
  return pb.bf16 && pb.inner == INNER_MLP && pb.d == D && (pb.hid == 64 || pb.hid == 128 || pb.hid == 256);
}

bool mfma_query_supported(const Problem& pb) { return mfma_full_supported(pb); }

// grid of the stream-K gradient kernel: at most one workgroup per CU and
// never more workgroups than tiles
void mfma_grad_geometry(const Problem& pb, int nt, int* G, int* J, int* tiles_per_pair) {
  const int P = pb.B * pb.H;
  const int tpp = (nt + TT - 1) / TT;
  *tiles_per_pair = tpp;
  const long long total = (long long)P * tpp;
  long long g = 256;
  if (g > total) g = total;
  *G = (int)g;
  // pairs a workgroup can touch: its tile count spans at most this many
  const long long per = (total + g - 1) / g;
  *J = (int)((per + tpp - 1) / tpp + 1);
}

void launch_mfma_full_grad(const Problem& pb, const bf16* wbf, int t0, int nt, float scale, float* part,
                           hipStream_t st) {
  int G, J, tpp;
  mfma_grad_geometry(pb, nt, &G, &J, &tpp);
  switch (pb.hid) {
    case 64: launch_grad_h<64>(pb, wbf, t0, nt, G, J, scale, part, st); break;
    case 128: launch_grad_h<128>(pb, wbf, t0, nt, G, J, scale, part, st); break;
    default: launch_grad_h<256>(pb, wbf, t0, nt, G, J, scale, part, st); break;
  }
}

void launch_mfma_query(const Problem& pb, const bf16* wstates, long long state_stride, int nchunks, int chunk,
                       hipStream_t st) {
  const int span = chunk ? (chunk < pb.N ? chunk : pb.N) : pb.N;
  const int tpw = NWAVE * QTOK * 4;
  const int groups = (span + tpw - 1) / tpw;
  dim3 grid(groups * nchunks, pb.B * pb.H);
  switch (pb.hid) {
    case 64: hipLaunchKernelGGL((k_mfma_query<64>), grid, dim3(NTHR), 0, st, pb, wstates, state_stride, chunk, span, groups, tpw); break;
    case 128: hipLaunchKernelGGL((k_mfma_query<128>), grid, dim3(NTHR), 0, st, pb, wstates, state_stride, chunk, span, groups, tpw); break;
    default: hipLaunchKernelGGL((k_mfma_query<256>), grid, dim3(NTHR), 0, st, pb, wstates, state_stride, chunk, span, groups, tpw); break;
  }
}

}  // namespace ttt
