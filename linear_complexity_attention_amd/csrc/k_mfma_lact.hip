// bf16 MFMA kernels of the large-chunk causal TTT layer with SwiGLU fast
// weights and the negative dot-product loss (LaCT analysis page, sections "Fast
// weights as memory of the current context", "Nonlinear memory complements
// local attention" and "Order of operations excludes leaking the future").
//
// Per chunk c of C tokens, at the fast weights W_c (fp32):
//     Z1 = K W1, Z3 = K W3, s = silu(Z1), Hh = s * Z3
//     G  = -eta_n V                                  (dot loss, per-token rates)
//     dW2 = Hh^T G,  dH = G W2^T,  dZ1 = dH * Z3 * silu'(Z1),  dZ3 = dH * s
//     dW1 = K^T dZ1, dW3 = K^T dZ3
// and the readout O_c = (silu(Q_c W1) * (Q_c W3)) W2 at the same W_c.
//
// Precision.  The chunk recurrence W_{c+1} = renorm(W_c - dW_c) feeds every
// step's rounding into the next one and amplifies it (at the config's rates a
// 1e-3 relative perturbation of W0 grows to >0.2 over 16 chunks), so the
// gradient products keep fp32-level accuracy on bf16 MFMA: an operand that is
// not exactly representable in bf16 is split as x = hi + lo (two bf16 values,
// ~16 significant bits) and its product takes two MFMAs.  K and V are bf16
// inputs and exact; the per-token rates are folded into Hh and into dH after
// the product, so every gradient GEMM has one exact operand.  The readout is
// not fed back and uses plain bf16 operands.
//
// Gradient kernel layout: workgroup = (token split, 64 hidden units, pair);
// each of its 4 waves owns 16 hidden units and accumulates the matching slices
// of dW1, dW3 (d x 16) and dW2 (16 x d) in registers; K and V tiles sit in LDS
// as [token][channel] and are read row-wise (b128) or transposed
// (ds_read_b64_tr_b16).  Partials of the token splits are reduced by the
// update kernel in a fixed order.
#include "ttt_internal.h"

namespace ttt {

namespace {

constexpr int TT = 32;            // tokens per tile
constexpr int NW = 4;             // waves per gradient workgroup
constexpr int HS = NW * 16;       // hidden units per gradient workgroup

typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) s16x4* lds_s16x4_ptr;

__device__ __forceinline__ f32x4 mfma16(const bf16x8& a, const bf16x8& b, const f32x4& c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}
// transposing LDS read (see k_mfma_full.hip for the lane mapping)
__device__ __forceinline__ bf16x4 ld_tr(const bf16* p) {
  s16x4 v = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4_ptr)((__attribute__((address_space(3))) char*)p));
  return __builtin_bit_cast(bf16x4, v);
}
__device__ __forceinline__ bf16x8 ld8(const bf16* p) { return *reinterpret_cast<const bf16x8*>(p); }
__device__ __forceinline__ bf16x8 cat44(const bf16x4& x, const bf16x4& y) {
  bf16x8 r;
#pragma unroll
  for (int i = 0; i < 4; ++i) { r[i] = x[i]; r[4 + i] = y[i]; }
  return r;
}
// x = hi + lo with hi = bf16(x), lo = bf16(x - hi)
__device__ __forceinline__ void split(float x, bf16& hi, bf16& lo) {
  hi = (bf16)x;
  lo = (bf16)(x - (float)hi);
}
__device__ __forceinline__ float sigm(float z) {
  return __builtin_amdgcn_rcpf(1.0f + __builtin_amdgcn_exp2f(-1.4426950408889634f * z));
}

// ---------------------------------------------------------------------------
template <int D, int HID>
__global__ void __launch_bounds__(NW * 64, 1)
k_lact_grad(Problem pb, WRef W, int t0, int nt, int S, float scale, float* __restrict__ part) {
  constexpr int NTHR = NW * 64;
  constexpr int NKS = D / 32;          // k-steps over the head dimension
  constexpr int NCB = D / 16;          // 16-wide channel blocks
  constexpr int LDK = D + 16;          // [token][channel] row stride (bf16)
  constexpr int SCH = D * TT / NTHR;   // channels staged per thread (16 or 8)
  constexpr int SPR = D / SCH;
  __shared__ __attribute__((aligned(16))) bf16 Kr[TT * LDK];
  __shared__ __attribute__((aligned(16))) bf16 Vr[TT * LDK];
  __shared__ float eta_s[TT];

  const int s = blockIdx.x, hs = blockIdx.y, p = blockIdx.z;
  const int bb = p / pb.H, hh = p % pb.H;
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int r = lane & 15, g = lane >> 4;
  const int hcol = hs * HS + 16 * w + r;           // this lane's hidden unit (B operand / n index)
  const int st = tid / SPR, sc = (tid % SPR) * SCH;
  const int L = ((nt + S - 1) / S + TT - 1) / TT * TT;
  const int n0 = s * L, n1 = min(nt, n0 + L);

  // ---- weight fragments, split into hi/lo bf16
  const float* W1 = W.mat(0, bb, hh);
  const float* W2 = W.mat(1, bb, hh);
  const float* W3 = W.mat(2, bb, hh);
  bf16x8 w1h[NKS], w1l[NKS], w3h[NKS], w3l[NKS], w2h[NKS], w2l[NKS];
#pragma unroll
  for (int ks = 0; ks < NKS; ++ks) {
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const int c = 32 * ks + 8 * g + j;
      bf16 a, b;
      split(W1[c * HID + hcol], a, b); w1h[ks][j] = a; w1l[ks][j] = b;
      split(W3[c * HID + hcol], a, b); w3h[ks][j] = a; w3l[ks][j] = b;
      split(W2[hcol * D + c], a, b); w2h[ks][j] = a; w2l[ks][j] = b;
    }
    __builtin_amdgcn_sched_barrier(0);
  }
  f32x4 a1[NCB], a3[NCB], a2[NCB];
#pragma unroll
  for (int cb = 0; cb < NCB; ++cb) { a1[cb] = f32x4{0, 0, 0, 0}; a3[cb] = a1[cb]; a2[cb] = a1[cb]; }

  const bf16* kp = (const bf16*)pb.k + ((long long)p * pb.N + t0) * D;
  const bf16* vp = (const bf16*)pb.v + ((long long)p * pb.N + t0) * D;
  const float* ep = pb.eta_tok ? pb.eta_tok + (long long)p * pb.N + t0 : nullptr;

  // K, V and the per-token rate of this thread's staging row, one tile ahead
  // (one wave per SIMD: nothing else would hide the load latency)
  bf16x8 kv[SCH / 8], vv[SCH / 8];
  float ev = 0.f;
  auto fetch = [&](int tt) {
    const int n = tt + st;
    const bool live = tt < n1 && n < n1;
#pragma unroll
    for (int u = 0; u < SCH / 8; ++u) {
      kv[u] = live ? ld8(kp + (long long)n * D + sc + 8 * u) : bf16x8{};
      vv[u] = live ? ld8(vp + (long long)n * D + sc + 8 * u) : bf16x8{};
    }
    if (sc == 0) ev = live ? (ep ? ep[n] : 1.0f) : 0.0f;
  };
  fetch(n0);
  for (int tt = n0; tt < n1; tt += TT) {
    // ---- stage K, V ([token][channel]) and the per-token rates, fetch the next tile
#pragma unroll
    for (int u = 0; u < SCH / 8; ++u) {
      *reinterpret_cast<bf16x8*>(&Kr[st * LDK + sc + 8 * u]) = kv[u];
      *reinterpret_cast<bf16x8*>(&Vr[st * LDK + sc + 8 * u]) = vv[u];
    }
    if (sc == 0) eta_s[st] = ev;
    fetch(tt + TT);
    __syncthreads();

    // ---- Z1 = K W1, Z3 = K W3, dHv = V W2^T (this wave's 16 hidden units)
    f32x4 z1[2], z3[2], dv[2];
#pragma unroll
    for (int tb = 0; tb < 2; ++tb) { z1[tb] = f32x4{0, 0, 0, 0}; z3[tb] = z1[tb]; dv[tb] = z1[tb]; }
#pragma unroll
    for (int ks = 0; ks < NKS; ++ks)
#pragma unroll
      for (int tb = 0; tb < 2; ++tb) {
        const bf16x8 ka = ld8(&Kr[(16 * tb + r) * LDK + 32 * ks + 8 * g]);
        const bf16x8 va = ld8(&Vr[(16 * tb + r) * LDK + 32 * ks + 8 * g]);
        z1[tb] = mfma16(ka, w1h[ks], z1[tb]);
        z1[tb] = mfma16(ka, w1l[ks], z1[tb]);
        z3[tb] = mfma16(ka, w3h[ks], z3[tb]);
        z3[tb] = mfma16(ka, w3l[ks], z3[tb]);
        dv[tb] = mfma16(va, w2h[ks], dv[tb]);
        dv[tb] = mfma16(va, w2l[ks], dv[tb]);
      }
    // ---- elementwise: lane holds tokens 16 tb + 4 g + i of hidden unit hcol;
    // packing (tb 0, i 0..3 | tb 1, i 0..3) is the token order of the
    // token-contracted MFMAs below
    bf16x8 hph, hpl, d1h, d1l, d3h, d3l;
#pragma unroll
    for (int tb = 0; tb < 2; ++tb)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float e = eta_s[16 * tb + 4 * g + i];
        const float x1 = z1[tb][i], x3 = z3[tb][i];
        const float sg = sigm(x1);
        const float si = x1 * sg;
        const float dh = -e * dv[tb][i];
        const float hp = -e * (si * x3);
        const float q1 = dh * x3 * (sg * (1.0f + x1 * (1.0f - sg)));
        const float q3 = dh * si;
        const int k = 4 * tb + i;
        bf16 a, b;
        split(hp, a, b); hph[k] = a; hpl[k] = b;
        split(q1, a, b); d1h[k] = a; d1l[k] = b;
        split(q3, a, b); d3h[k] = a; d3l[k] = b;
      }
    // ---- token-contracted products
#pragma unroll
    for (int cb = 0; cb < NCB; ++cb) {
      // V[t = tau(g, j)][c = 16 cb + r] and K[...] in the transposed orientation
      const bf16x8 vb = cat44(ld_tr(&Vr[(4 * g + (r >> 2)) * LDK + 16 * cb + 4 * (r & 3)]),
                              ld_tr(&Vr[(16 + 4 * g + (r >> 2)) * LDK + 16 * cb + 4 * (r & 3)]));
      const bf16x8 kb = cat44(ld_tr(&Kr[(4 * g + (r >> 2)) * LDK + 16 * cb + 4 * (r & 3)]),
                              ld_tr(&Kr[(16 + 4 * g + (r >> 2)) * LDK + 16 * cb + 4 * (r & 3)]));
      a2[cb] = mfma16(hph, vb, a2[cb]);          // dW2[h][c]  (m = h, n = c)
      a2[cb] = mfma16(hpl, vb, a2[cb]);
      a1[cb] = mfma16(kb, d1h, a1[cb]);          // dW1[c][h]  (m = c, n = h)
      a1[cb] = mfma16(kb, d1l, a1[cb]);
      a3[cb] = mfma16(kb, d3h, a3[cb]);
      a3[cb] = mfma16(kb, d3l, a3[cb]);
    }
    __syncthreads();
  }

  // ---- partial of this token split: [dW1 (d x h) | dW2 (h x d) | dW3 (d x h)]
  const long long msz = (long long)D * HID;
  float* out = part + ((long long)s * (pb.B * pb.H) + p) * 3 * msz;
  const int h0 = hs * HS + 16 * w;
#pragma unroll
  for (int cb = 0; cb < NCB; ++cb)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int c = 16 * cb + 4 * g + i;
      out[c * HID + hcol] = scale * a1[cb][i];
      out[2 * msz + c * HID + hcol] = scale * a3[cb][i];
      out[msz + (long long)(h0 + 4 * g + i) * D + 16 * cb + r] = scale * a2[cb][i];
    }
}

// ---------------------------------------------------------------------------
// Readout O = (silu(Q W1) * (Q W3)) W2, tokens on the MFMA n axis.  The hidden
// width is walked in halves: each half of W1, W3 ([c][h]) and W2 ([h][c]) is
// staged in LDS as bf16; O accumulates in registers across the halves.
constexpr int RW = 8;                    // waves per readout workgroup
constexpr int RTOK = 32;                 // tokens per wave
template <int D, int HID>
__global__ void __launch_bounds__(RW * 64, 1)
k_lact_readout(Problem pb, WRef w0, const float* __restrict__ states, long long state_stride, int chunk, int span,
               int groups) {
  constexpr int NTHR = RW * 64;
  constexpr int HH = 128;                // hidden units per staged half
  constexpr int NKS = D / 32, NCB = D / 16;
  constexpr int L1 = HH + 16;            // [c][h] rows
  constexpr int L2 = D + 16;             // [h][c] rows
  __shared__ __attribute__((aligned(16))) bf16 w1s[D * L1];
  __shared__ __attribute__((aligned(16))) bf16 w3s[D * L1];
  __shared__ __attribute__((aligned(16))) bf16 w2s[HH * L2];
  // per-wave staging of a 16-token output block (16 rows of D bf16, the
  // 16-byte chunks of row t XOR-permuted by t & 7), so that each output store
  // writes whole rows (1 KB contiguous) instead of 32 bytes of 16 rows
  __shared__ __attribute__((aligned(16))) bf16 ob[RW][16 * D];
  // XCD-aware work mapping: workgroups are dealt to the 8 XCDs round-robin, so
  // the work index L gives consecutive L (the groups of one (pair, chunk),
  // which read the same weight state) to workgroups of one XCD and its L2
  const int nb = gridDim.x * gridDim.y, bid = blockIdx.y * gridDim.x + blockIdx.x;
  const int L = nb % 8 == 0 ? (bid % 8) * (nb / 8) + bid / 8 : bid;
  const int p = L / gridDim.x, bx = L % gridDim.x;
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int r = lane & 15, g = lane >> 4;
  const int c = bx / groups, grp = bx % groups;
  const int c0 = c * span;
  const int n0 = c0 + grp * (RW * RTOK);
  const int n1 = min(min(pb.N, c0 + span), n0 + RW * RTOK);
  if (n0 >= n1) return;
  const int state = chunk ? c : 1;
  const int bb = p / pb.H, hh = p % pb.H;
  const float *W1, *W2, *W3;
  const long long msz = (long long)D * HID;
  if (state == 0) { W1 = w0.mat(0, bb, hh); W2 = w0.mat(1, bb, hh); W3 = w0.mat(2, bb, hh); }
  else {
    const float* base = states + (state - 1) * state_stride + (long long)p * 3 * msz;
    W1 = base; W2 = base + msz; W3 = base + 2 * msz;
  }
  const bf16* qp = (const bf16*)pb.q + (long long)p * pb.N * D;
  bf16* op = (bf16*)pb.o + (long long)p * pb.N * D;
  const int base = n0 + w * RTOK;
  bf16x8 qb[2][NKS];
#pragma unroll
  for (int tb = 0; tb < 2; ++tb)
#pragma unroll
    for (int ks = 0; ks < NKS; ++ks) {
      const int n = base + 16 * tb + r;
      qb[tb][ks] = n < n1 ? ld8(qp + (long long)n * D + 32 * ks + 8 * g) : bf16x8{};
    }
  f32x4 o[NCB][2];
#pragma unroll
  for (int cb = 0; cb < NCB; ++cb) { o[cb][0] = f32x4{0, 0, 0, 0}; o[cb][1] = o[cb][0]; }

  for (int half = 0; half < HID / HH; ++half) {
    const int hb0 = half * HH;
    if (half) __syncthreads();
    // the half's weights, in batches of SB float4 per matrix and thread: the
    // loads of a batch are all in flight before the first conversion waits
    constexpr int NIT = D * HH / (NTHR * 4), SB = NIT < 4 ? NIT : 4;
    static_assert(D * HH % (NTHR * 4) == 0 && NIT % SB == 0, "staging splits evenly");
#pragma unroll
    for (int k0 = 0; k0 < NIT; k0 += SB) {
      float4 a[SB], b[SB], m[SB];
#pragma unroll
      for (int k = 0; k < SB; ++k) {
        const int e = tid * 4 + (k0 + k) * NTHR * 4;
        const int cc = e / HH, hx = e % HH;                    // W1, W3 [c][h] rows
        const int hy = e / D, cy = e % D;                      // W2 [h][c] rows
        a[k] = *reinterpret_cast<const float4*>(W1 + cc * HID + hb0 + hx);
        b[k] = *reinterpret_cast<const float4*>(W3 + cc * HID + hb0 + hx);
        m[k] = *reinterpret_cast<const float4*>(W2 + (long long)(hb0 + hy) * D + cy);
      }
#pragma unroll
      for (int k = 0; k < SB; ++k) {
        const int e = tid * 4 + (k0 + k) * NTHR * 4;
        const int cc = e / HH, hx = e % HH;
        const int hy = e / D, cy = e % D;
        *reinterpret_cast<bf16x4*>(&w1s[cc * L1 + hx]) = bf16x4{(bf16)a[k].x, (bf16)a[k].y, (bf16)a[k].z, (bf16)a[k].w};
        *reinterpret_cast<bf16x4*>(&w3s[cc * L1 + hx]) = bf16x4{(bf16)b[k].x, (bf16)b[k].y, (bf16)b[k].z, (bf16)b[k].w};
        *reinterpret_cast<bf16x4*>(&w2s[hy * L2 + cy]) = bf16x4{(bf16)m[k].x, (bf16)m[k].y, (bf16)m[k].z, (bf16)m[k].w};
      }
    }
    __syncthreads();
    if (base < n1) {
#pragma unroll 1
      for (int hc = 0; hc < HH / 32; ++hc) {
        f32x4 z1[2][2], z3[2][2];
#pragma unroll
        for (int u = 0; u < 2; ++u)
#pragma unroll
          for (int tb = 0; tb < 2; ++tb) { z1[u][tb] = f32x4{0, 0, 0, 0}; z3[u][tb] = z1[u][tb]; }
#pragma unroll
        for (int ks = 0; ks < NKS; ++ks)
#pragma unroll
          for (int u = 0; u < 2; ++u) {
            const int row = 32 * ks + 8 * g + (r >> 2), col = 32 * hc + 16 * u + 4 * (r & 3);
            const bf16x8 a1 = cat44(ld_tr(&w1s[row * L1 + col]), ld_tr(&w1s[(row + 4) * L1 + col]));
            const bf16x8 a3 = cat44(ld_tr(&w3s[row * L1 + col]), ld_tr(&w3s[(row + 4) * L1 + col]));
#pragma unroll
            for (int tb = 0; tb < 2; ++tb) {
              z1[u][tb] = mfma16(a1, qb[tb][ks], z1[u][tb]);
              z3[u][tb] = mfma16(a3, qb[tb][ks], z3[u][tb]);
            }
          }
        bf16x8 hb[2];
#pragma unroll
        for (int tb = 0; tb < 2; ++tb)
#pragma unroll
          for (int u = 0; u < 2; ++u)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
              const float x1 = z1[u][tb][i];
              hb[tb][4 * u + i] = (bf16)(x1 * sigm(x1) * z3[u][tb][i]);
            }
#pragma unroll
        for (int cb = 0; cb < NCB; ++cb) {
          const int col = 16 * cb + 4 * (r & 3);
          const bf16x8 a = cat44(ld_tr(&w2s[(32 * hc + 4 * g + (r >> 2)) * L2 + col]),
                                 ld_tr(&w2s[(32 * hc + 16 + 4 * g + (r >> 2)) * L2 + col]));
#pragma unroll
          for (int tb = 0; tb < 2; ++tb) o[cb][tb] = mfma16(a, hb[tb], o[cb][tb]);
        }
      }
    }
  }
  // lane (g, r) holds channels 16 cb + 4 g .. + 3 of token r; through the
  // wave's LDS block, lane l then takes the 16-byte chunk l % (D / 8) of token
  // l / (D / 8) + k 64 / (D / 8) (the wave's own LDS operations are done in
  // order: no barrier)
  constexpr int ROWC = D / 8, RPI = 64 / ROWC;
  bf16* sb = ob[w];
#pragma unroll
  for (int tb = 0; tb < 2; ++tb) {
#pragma unroll
    for (int cb = 0; cb < NCB; ++cb) {
      bf16x4 v;
#pragma unroll
      for (int i = 0; i < 4; ++i) v[i] = (bf16)o[cb][tb][i];
      *reinterpret_cast<bf16x4*>(sb + r * D + (((2 * cb + (g >> 1)) ^ (r & 7)) << 3) + 4 * (g & 1)) = v;
    }
#pragma unroll
    for (int k = 0; k < 16 / RPI; ++k) {
      const int t = lane / ROWC + RPI * k, c = lane % ROWC;
      const bf16x8 v = *reinterpret_cast<const bf16x8*>(sb + t * D + ((c ^ (t & 7)) << 3));
      const int n = base + 16 * tb + t;
      if (n < n1) *reinterpret_cast<bf16x8*>(op + (long long)n * D + 8 * c) = v;
    }
  }
}

}  // namespace

bool lact_supported(const Problem& pb) {
  return pb.bf16 && pb.inner == INNER_SWIGLU && pb.loss == LOSS_DOT && (pb.d == 64 || pb.d == 128) &&
         (pb.hid == 128 || pb.hid == 256);
}

bool lact_readout_supported(const Problem& pb) {
  return pb.bf16 && pb.inner == INNER_SWIGLU && (pb.d == 64 || pb.d == 128) && (pb.hid == 128 || pb.hid == 256);
}

int lact_grad_splits(const Problem& pb, int nt) {
  const long long other = (long long)pb.B * pb.H * (pb.hid / HS);
  long long s = (256 + other - 1) / other;
  const long long tiles = (nt + TT - 1) / TT;
  if (s > tiles) s = tiles;
  return (int)(s < 1 ? 1 : s);
}

template <int D, int HID>
static void lact_grad_launch(const Problem& pb, const WRef& W, int t0, int nt, int S, float scale, float* part,
                             hipStream_t st) {
  dim3 grid(S, HID / HS, pb.B * pb.H);
  hipLaunchKernelGGL((k_lact_grad<D, HID>), grid, dim3(NW * 64), 0, st, pb, W, t0, nt, S, scale, part);
}

void launch_lact_grad(const Problem& pb, const WRef& W, int t0, int nt, int S, float scale, float* part,
                      hipStream_t st) {
  if (pb.d == 128) {
    if (pb.hid == 256) lact_grad_launch<128, 256>(pb, W, t0, nt, S, scale, part, st);
    else lact_grad_launch<128, 128>(pb, W, t0, nt, S, scale, part, st);
  } else {
    if (pb.hid == 256) lact_grad_launch<64, 256>(pb, W, t0, nt, S, scale, part, st);
    else lact_grad_launch<64, 128>(pb, W, t0, nt, S, scale, part, st);
  }
}

template <int D, int HID>
static void lact_readout_launch(const Problem& pb, const WRef& w0, const float* states, long long state_stride,
                                int nchunks, int chunk, hipStream_t st) {
  const int span = chunk ? (chunk < pb.N ? chunk : pb.N) : pb.N;
  const int groups = (span + RW * RTOK - 1) / (RW * RTOK);
  dim3 grid(groups * nchunks, pb.B * pb.H);
  hipLaunchKernelGGL((k_lact_readout<D, HID>), grid, dim3(RW * 64), 0, st, pb, w0, states, state_stride, chunk,
                     span, groups);
}

void launch_lact_readout(const Problem& pb, const WRef& w0, const float* states, long long state_stride,
                         int nchunks, int chunk, hipStream_t st) {
  if (pb.d == 128) {
    if (pb.hid == 256) lact_readout_launch<128, 256>(pb, w0, states, state_stride, nchunks, chunk, st);
    else lact_readout_launch<128, 128>(pb, w0, states, state_stride, nchunks, chunk, st);
  } else {
    if (pb.hid == 256) lact_readout_launch<64, 256>(pb, w0, states, state_stride, nchunks, chunk, st);
    else lact_readout_launch<64, 128>(pb, w0, states, state_stride, nchunks, chunk, st);
  }
}

}  // namespace ttt
