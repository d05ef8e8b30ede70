// bf16 MFMA kernels of the simplified gated linear unit of the ViT3 block
// (ViT3 summary page, section 03 guideline 6 and section 04):
//     U = X W1,  Z = X W2,  F = U * silu(Z)            (two d x d maps, d = 64)
// One full-batch step (section 02):
//     G  = eta_n 2/(N d) (F - V) [MSE]   |   -eta_n V [dot]
//     dU = G * silu(Z),  dZ = G * U * silu'(Z),  dW1 = X^T dU,  dW2 = X^T dZ
// and the readout O = (Q W1*) * silu(Q W2*).
//
// Layout (v_mfma_f32_16x16x32_bf16, wave64): tokens are the M axis of the
// forward products, so the lane holding U, Z of (token, unit) also holds the
// matching V and eta and does the elementwise work; each of the 4 waves owns
// 16 of the 64 hidden units (its B-operand weight fragments stay in
// registers).  dU, dZ go to LDS as [unit][token] rows and X is staged a second
// time as [channel][token] rows, so both operands of dW = X^T dU are read 8
// tokens at a time (one 16-byte read per lane).  Token splits of each pair
// write fp32 partials [S][P][2][d*d], reduced by the update kernel in a fixed
// order.  The single full-batch step is not a recurrence, so plain bf16
// operands (fp32 accumulation) meet the bf16 tolerance.
#include "ttt_internal.h"

namespace ttt {

namespace {

constexpr int D = 64;
constexpr int TT = 32;               // tokens per tile
constexpr int NW = 4;                // waves: 16 hidden units each
constexpr int LX = D + 8;            // [token][channel] row stride (bf16)
constexpr int LT = TT + 8;           // [channel|unit][token] row stride (bf16)

__device__ __forceinline__ f32x4 mfma16(const bf16x8& a, const bf16x8& b, const f32x4& c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ float sigm(float z) {
  return __builtin_amdgcn_rcpf(1.0f + __builtin_amdgcn_exp2f(-1.4426950408889634f * z));
}

// B-operand fragments of W[c][16 jb + r] (c = 32 ks + 8 g + e) in bf16
__device__ __forceinline__ void load_wfrag(const float* W, int jb, int r, int g, bf16x8 (&f)[2]) {
#pragma unroll
  for (int ks = 0; ks < 2; ++ks)
#pragma unroll
    for (int e = 0; e < 8; ++e) f[ks][e] = (bf16)W[(32 * ks + 8 * g + e) * D + 16 * jb + r];
}

// partial dW1, dW2 of token split blockIdx.x of pair blockIdx.y
__global__ void __launch_bounds__(NW * 64) k_glu_grad(Problem pb, WRef W, int t0, int nt, int S,
                                                      float* __restrict__ part) {
  __shared__ __attribute__((aligned(16))) bf16 Xs[TT * LX];     // [token][channel]
  __shared__ __attribute__((aligned(16))) bf16 Xt[D * LT];      // [channel][token]
  __shared__ __attribute__((aligned(16))) bf16 Vs[TT * LX];     // [token][channel]
  __shared__ __attribute__((aligned(16))) bf16 dUs[D * LT];     // [unit][token]
  __shared__ __attribute__((aligned(16))) bf16 dZs[D * LT];
  __shared__ float es[TT];
  const int s = blockIdx.x, p = blockIdx.y;
  const int b = p / pb.H, h = p % pb.H;
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int r = lane & 15, g = lane >> 4;
  const long long prow = pb.row(p);
  const bf16* kp = (const bf16*)pb.k + (prow * pb.N + t0) * D;
  const bf16* vp = (const bf16*)pb.v + (prow * pb.N + t0) * D;
  const float* ep = pb.eta_tok ? pb.eta_tok + prow * pb.N + t0 : nullptr;
  const bool mse = pb.loss == LOSS_MSE;
  const float cm = 2.0f / ((float)nt * (float)D);
  bf16x8 w1f[2], w2f[2];
  load_wfrag(W.mat(0, b, h), w, r, g, w1f);
  load_wfrag(W.mat(1, b, h), w, r, g, w2f);
  // staging: thread -> (token st, channels 8 sc8 .. 8 sc8 + 7)
  const int st = tid >> 3, sc = (tid & 7) * 8;
  float mu[8], rs[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    mu[e] = pb.stats ? pb.stats[((size_t)p * D + sc + e) * 2] : 0.f;
    rs[e] = pb.stats ? pb.stats[((size_t)p * D + sc + e) * 2 + 1] : 1.f;
  }
  f32x4 a1[4], a2[4];   // dW1, dW2 blocks [channel block cb][unit block w]
#pragma unroll
  for (int cb = 0; cb < 4; ++cb) { a1[cb] = f32x4{0, 0, 0, 0}; a2[cb] = f32x4{0, 0, 0, 0}; }
  const int tiles = (nt + TT - 1) / TT;
  const int per = (tiles + S - 1) / S;
  const int k0 = s * per, k1 = min(tiles, k0 + per);
  for (int kt = k0; kt < k1; ++kt) {
    const int n = kt * TT + st;
    bf16x8 xv = {}, vv = {};
    if (n < nt) {
      xv = *reinterpret_cast<const bf16x8*>(kp + (long long)n * D + sc);
      vv = *reinterpret_cast<const bf16x8*>(vp + (long long)n * D + sc);
      if (pb.stats) {
#pragma unroll
        for (int e = 0; e < 8; ++e) xv[e] = (bf16)(((float)xv[e] - mu[e]) * rs[e]);
      }
    }
    __syncthreads();                                   // the previous tile's reads are done
    *reinterpret_cast<bf16x8*>(&Xs[st * LX + sc]) = xv;
    *reinterpret_cast<bf16x8*>(&Vs[st * LX + sc]) = vv;
#pragma unroll
    for (int e = 0; e < 8; ++e) Xt[(sc + e) * LT + st] = xv[e];
    if (tid < TT) es[tid] = kt * TT + tid < nt ? pb.eta_scale * (ep ? ep[kt * TT + tid] : 1.f) : 0.f;
    __syncthreads();
    // U, Z of (16 tokens x this wave's 16 units), two token blocks
#pragma unroll
    for (int tb = 0; tb < 2; ++tb) {
      f32x4 u = {0, 0, 0, 0}, z = {0, 0, 0, 0};
#pragma unroll
      for (int ks = 0; ks < 2; ++ks) {
        const bf16x8 xa = *reinterpret_cast<const bf16x8*>(&Xs[(16 * tb + r) * LX + 32 * ks + 8 * g]);
        u = mfma16(xa, w1f[ks], u);
        z = mfma16(xa, w2f[ks], z);
      }
      // lane holds (token 16 tb + 4 g + i, unit 16 w + r)
      bf16x4 du, dz;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int t = 16 * tb + 4 * g + i, j = 16 * w + r;
        const float vt = (float)Vs[t * LX + j], et = es[t];
        const float sg = sigm(z[i]), si = z[i] * sg;
        const float gr = mse ? et * cm * (u[i] * si - vt) : -et * vt;
        du[i] = (bf16)(gr * si);
        dz[i] = (bf16)(gr * u[i] * sg * (1.0f + z[i] * (1.0f - sg)));
      }
      *reinterpret_cast<bf16x4*>(&dUs[(16 * w + r) * LT + 16 * tb + 4 * g]) = du;
      *reinterpret_cast<bf16x4*>(&dZs[(16 * w + r) * LT + 16 * tb + 4 * g]) = dz;
    }
    __syncthreads();
    // dW1 += X^T dU, dW2 += X^T dZ for (channel block cb, unit block w), k = 32 tokens
    const bf16x8 bu = *reinterpret_cast<const bf16x8*>(&dUs[(16 * w + r) * LT + 8 * g]);
    const bf16x8 bz = *reinterpret_cast<const bf16x8*>(&dZs[(16 * w + r) * LT + 8 * g]);
#pragma unroll
    for (int cb = 0; cb < 4; ++cb) {
      const bf16x8 xa = *reinterpret_cast<const bf16x8*>(&Xt[(16 * cb + r) * LT + 8 * g]);
      a1[cb] = mfma16(xa, bu, a1[cb]);
      a2[cb] = mfma16(xa, bz, a2[cb]);
    }
  }
  // lane holds dW[c = 16 cb + 4 g + i][j = 16 w + r]
  float* o = part + ((long long)s * pb.B * pb.H + p) * 2 * D * D;
#pragma unroll
  for (int cb = 0; cb < 4; ++cb)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int c = 16 * cb + 4 * g + i, j = 16 * w + r;
      o[c * D + j] = a1[cb][i];
      o[D * D + c * D + j] = a2[cb][i];
    }
}

// O = (Q W1*) * silu(Q W2*) for 128 tokens of pair blockIdx.y from the
// state (layout [P][2][d*d]); O is staged in LDS for row-wise stores
constexpr int kQTiles = 4;
__global__ void __launch_bounds__(NW * 64) k_glu_query(Problem pb, const float* __restrict__ state) {
  __shared__ __attribute__((aligned(16))) bf16 Qs[TT * LX];
  __shared__ __attribute__((aligned(16))) bf16 Os[TT * LX];
  const int p = blockIdx.y;
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int r = lane & 15, g = lane >> 4;
  const long long prow = pb.row(p);
  const bf16* qp = (const bf16*)pb.q + prow * pb.N * D;
  bf16* op = (bf16*)pb.o + prow * pb.N * D;
  const float* Ws = state + (long long)p * 2 * D * D;
  bf16x8 w1f[2], w2f[2];
  load_wfrag(Ws, w, r, g, w1f);
  load_wfrag(Ws + D * D, w, r, g, w2f);
  const int st = tid >> 3, sc = (tid & 7) * 8;
  for (int kt = blockIdx.x * kQTiles; kt < min((pb.N + TT - 1) / TT, (blockIdx.x + 1) * kQTiles); ++kt) {
    const int n = kt * TT + st;
    const bf16x8 qv = n < pb.N ? *reinterpret_cast<const bf16x8*>(qp + (long long)n * D + sc) : bf16x8{};
    __syncthreads();
    *reinterpret_cast<bf16x8*>(&Qs[st * LX + sc]) = qv;
    __syncthreads();
#pragma unroll
    for (int tb = 0; tb < 2; ++tb) {
      f32x4 u = {0, 0, 0, 0}, z = {0, 0, 0, 0};
#pragma unroll
      for (int ks = 0; ks < 2; ++ks) {
        const bf16x8 qa = *reinterpret_cast<const bf16x8*>(&Qs[(16 * tb + r) * LX + 32 * ks + 8 * g]);
        u = mfma16(qa, w1f[ks], u);
        z = mfma16(qa, w2f[ks], z);
      }
#pragma unroll
      for (int i = 0; i < 4; ++i) Os[(16 * tb + 4 * g + i) * LX + 16 * w + r] = (bf16)(u[i] * z[i] * sigm(z[i]));
    }
    __syncthreads();
    if (n < pb.N) *reinterpret_cast<bf16x8*>(op + (long long)n * D + sc) = *reinterpret_cast<const bf16x8*>(&Os[st * LX + sc]);
  }
}

}  // namespace

bool glu_supported(const Problem& pb) { return pb.bf16 && pb.inner == INNER_GLU && pb.d == D; }

int glu_grad_splits(const Problem& pb, int nt) {
  const long long P = (long long)pb.B * pb.H;
  long long s = (4LL * device_cu_count() + P - 1) / P;
  const long long tiles = (nt + TT - 1) / TT;
  const long long maxs = (tiles + 3) / 4;         // at least 4 tiles per split
  if (s > maxs) s = maxs;
  if (s < 1) s = 1;
  return (int)s;
}

void launch_glu_grad(const Problem& pb, const WRef& W, int t0, int nt, int S, float* part, hipStream_t st) {
  hipLaunchKernelGGL(k_glu_grad, dim3(S, pb.B * pb.H), dim3(NW * 64), 0, st, pb, W, t0, nt, S, part);
}

void launch_glu_query(const Problem& pb, const float* state, hipStream_t st) {
  const int tiles = (pb.N + TT - 1) / TT;
  hipLaunchKernelGGL(k_glu_query, dim3((tiles + kQTiles - 1) / kQTiles, pb.B * pb.H), dim3(NW * 64), 0, st, pb,
                     state);
}

}  // namespace ttt
