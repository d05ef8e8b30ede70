// Outer-loop backward of the TTT layer (ViT3 summary page, section 02: the
// inner update is differentiable and is trained end to end with the outer
// network, a gradient of a gradient; section 03 guideline 1: the value
// projection learns through the loss's mixed second derivative).  Full batch,
// one gradient step, linear and GELU-MLP inner models, fp32 arithmetic.
//
// With W* = W0 - g(W0), g = dL/dW, and dO the gradient of an outer loss S
// with respect to O = F_W*(Q):
//   readout backward:   U = dS/dW*, dQ = dS/dQ                  (k_bwd_readout_tok
//                       and the generic dW kernel run on (Q, dO))
//   through the step:   phi = <g(W0, K_hat, V, eta), U> = sum_n <G_n, F_dot_n>,
//                       F_dot the tangent of the inner model along U;
//                       dW0 = U - dphi/dW0, dK_hat = -dphi/dK_hat,
//                       dV = -dphi/dV, deta_n = -dphi/deta_n  (k_bwd_key_tok per
//                       token, k_bwd_wbar per hidden slice, k_bwd_dw0)
//   key norm:           dK = rstd (dK_hat - mean dK_hat - K_hat mean(dK_hat K_hat))
//                                                             (k_bwd_kn_*)
// MLP terms (Z = X W1, A = gelu(Z), F = A W2; Z_dot = X U1, A_dot = gelu'(Z)
// Z_dot, F_dot = A_dot W2 + A U2; G the loss gradient; F_bar = 2 c eta F_dot
// for MSE, 0 for the dot loss):
//   A_dot_bar = G W2^T, A_bar = G U2^T + F_bar W2^T,
//   Z_dot_bar = gelu'(Z) A_dot_bar, Z_bar = gelu''(Z) Z_dot A_dot_bar + gelu'(Z) A_bar,
//   dphi/dX = Z_dot_bar U1^T + Z_bar W1^T, dphi/dW1 = X^T Z_bar,
//   dphi/dW2 = A_dot^T G + A^T F_bar.
// Linear: F_dot = X U, dphi/dX = G U^T + F_bar W^T, dphi/dW = X^T F_bar.
// These are the reference-speed kernels (LDS-staged fp32 loops over 16-token
// tiles, like the generic forward kernels).
#include "ttt_internal.h"

namespace ttt {

namespace {

constexpr int kThreads = 256;
constexpr int kTok = 16;
constexpr int kSlice = 32;
constexpr int kMaxD = 128;
constexpr int kMaxH = 512;

__device__ __forceinline__ float gelu_second(float z) {
  return 0.39894228040143268f * __expf(-0.5f * z * z) * (2.0f - z * z);
}

template <typename T>
__device__ __forceinline__ void load_rows(const T* base, long long row, int N, int d, int t0, int cnt, float* dst) {
  for (int i = threadIdx.x; i < kTok * d; i += kThreads) {
    const int t = i / d, c = i % d;
    dst[i] = t < cnt ? to_f32<T>(base[(row * N + t0 + t) * d + c]) : 0.f;
  }
}

// dO rows of every pair -> fp32 [P][N][d] (the layout the generic dW kernel reads)
template <typename T>
__global__ void __launch_bounds__(kThreads) k_bwd_rows_f32(Problem pb, const T* __restrict__ src, float* __restrict__ dst) {
  const int p = blockIdx.y;
  const long long n = (long long)pb.N * pb.d;
  const T* s = src + pb.row(p) * n;
  float* o = dst + (long long)p * n;
  for (long long i = blockIdx.x * (long long)kThreads + threadIdx.x; i < n; i += (long long)gridDim.x * kThreads)
    o[i] = to_f32<T>(s[i]);
}

// dQ for 16 tokens of pair blockIdx.y at the updated weights W*:
// MLP: dQ = (gelu'(Q W1*) (dO W2*^T)) W1*^T;  linear: dQ = dO W*^T
template <typename T>
__global__ void __launch_bounds__(kThreads) k_bwd_readout_tok(Problem pb, WRef Ws, const float* __restrict__ dO32,
                                                             float* __restrict__ dq) {
  const int p = blockIdx.y, b = p / pb.H, h = p % pb.H;
  const int t0 = blockIdx.x * kTok, cnt = min(kTok, pb.N - t0);
  const int d = pb.d, hid = pb.hid;
  __shared__ float qs[kTok * kMaxD], gs[kTok * kMaxD], zb[kTok * kMaxH];
  load_rows<T>((const T*)pb.q, pb.row(p), pb.N, d, t0, cnt, qs);
  for (int i = threadIdx.x; i < kTok * d; i += kThreads) {
    const int t = i / d;
    gs[i] = t < cnt ? dO32[((long long)p * pb.N + t0) * d + i] : 0.f;
  }
  __syncthreads();
  const float* W1 = Ws.mat(0, b, h);
  float* out = dq + (pb.row(p) * pb.N + t0) * d;
  if (pb.inner == INNER_LINEAR) {
    for (int i = threadIdx.x; i < cnt * d; i += kThreads) {
      const int t = i / d, c = i % d;
      float s = 0.f;
      for (int cc = 0; cc < d; ++cc) s += gs[t * d + cc] * W1[(size_t)c * d + cc];
      out[i] = s;
    }
    return;
  }
  const float* W2 = Ws.mat(1, b, h);
  for (int i = threadIdx.x; i < kTok * hid; i += kThreads) {
    const int t = i / hid, j = i % hid;
    float z = 0.f, a = 0.f;
    for (int c = 0; c < d; ++c) {
      z += qs[t * d + c] * W1[(size_t)c * hid + j];
      a += gs[t * d + c] * W2[(size_t)j * d + c];
    }
    zb[i] = gelu_exact_prime(z) * a;
  }
  __syncthreads();
  for (int i = threadIdx.x; i < cnt * d; i += kThreads) {
    const int t = i / d, c = i % d;
    float s = 0.f;
    for (int j = 0; j < hid; ++j) s += zb[t * hid + j] * W1[(size_t)c * hid + j];
    out[i] = s;
  }
}

// Per-token terms of phi for 16 tokens of pair blockIdx.y at W0 along U:
// dv = -dphi/dV, deta = -dphi/deta (nullable), dkh = -dphi/dX (fp32, written
// at the pair's row of dk), and G, F_bar for the weight reduction (fp32
// [P][N][d]).
template <typename T>
__global__ void __launch_bounds__(kThreads) k_bwd_key_tok(Problem pb, WRef W0, const float* __restrict__ U,
                                                         float* __restrict__ dv, float* __restrict__ deta,
                                                         float* __restrict__ dkh, float* __restrict__ gG,
                                                         float* __restrict__ gF) {
  const int p = blockIdx.y, b = p / pb.H, h = p % pb.H;
  const int t0 = blockIdx.x * kTok, cnt = min(kTok, pb.N - t0);
  const int d = pb.d, hid = pb.hid, N = pb.N;
  const bool mlp = pb.inner == INNER_MLP;
  const float c2 = 2.0f / ((float)N * (float)d);
  const bool mse = pb.loss == LOSS_MSE;
  __shared__ float xs[kTok * kMaxD], vs[kTok * kMaxD], fs[kTok * kMaxD], fds[kTok * kMaxD];
  __shared__ float Gs[kTok * kMaxD], Fbs[kTok * kMaxD];
  __shared__ float zs[kTok * kMaxH], zds[kTok * kMaxH];
  __shared__ float es[kTok], red[kTok][kThreads / kTok];
  const long long prow = pb.row(p);
  // X = K_hat (normalised on the way), V, eta
  for (int i = threadIdx.x; i < kTok * d; i += kThreads) {
    const int t = i / d, c = i % d;
    float x = 0.f, vv = 0.f;
    if (t < cnt) {
      x = to_f32<T>(((const T*)pb.k)[(prow * N + t0 + t) * d + c]);
      if (pb.stats) x = (x - pb.stats[((size_t)p * d + c) * 2]) * pb.stats[((size_t)p * d + c) * 2 + 1];
      vv = to_f32<T>(((const T*)pb.v)[(prow * N + t0 + t) * d + c]);
    }
    xs[i] = x;
    vs[i] = vv;
  }
  if (threadIdx.x < kTok) {
    const int n = t0 + threadIdx.x;
    es[threadIdx.x] = threadIdx.x < cnt ? pb.eta_scale * (pb.eta_tok ? pb.eta_tok[prow * N + n] : 1.f) : 0.f;
  }
  __syncthreads();
  const float* W1 = W0.mat(0, b, h);
  const float* W2 = mlp ? W0.mat(1, b, h) : nullptr;
  const float* U1 = U + (long long)p * pb.nm * pb.msz;
  const float* U2 = U1 + pb.msz;
  // forward and tangent: F (MSE only), F_dot
  if (mlp) {
    for (int i = threadIdx.x; i < kTok * hid; i += kThreads) {
      const int t = i / hid, j = i % hid;
      float z = 0.f, zd = 0.f;
      for (int c = 0; c < d; ++c) {
        z += xs[t * d + c] * W1[(size_t)c * hid + j];
        zd += xs[t * d + c] * U1[(size_t)c * hid + j];
      }
      zs[i] = z;
      zds[i] = zd;
    }
    __syncthreads();
    for (int i = threadIdx.x; i < kTok * d; i += kThreads) {
      const int t = i / d, c = i % d;
      float f = 0.f, fd = 0.f;
      for (int j = 0; j < hid; ++j) {
        const float z = zs[t * hid + j], a = gelu_exact(z), ad = gelu_exact_prime(z) * zds[t * hid + j];
        f += a * W2[(size_t)j * d + c];
        fd += ad * W2[(size_t)j * d + c] + a * U2[(size_t)j * d + c];
      }
      fs[i] = f;
      fds[i] = fd;
    }
  } else {
    for (int i = threadIdx.x; i < kTok * d; i += kThreads) {
      const int t = i / d, c = i % d;
      float f = 0.f, fd = 0.f;
      for (int cc = 0; cc < d; ++cc) {
        f += xs[t * d + cc] * W1[(size_t)cc * d + c];
        fd += xs[t * d + cc] * U1[(size_t)cc * d + c];
      }
      fs[i] = f;
      fds[i] = fd;
    }
  }
  __syncthreads();
  // G, F_bar, and the per-token outputs dV, deta
  constexpr int LPT = kThreads / kTok;    // lanes per token for the deta row sums
  {
    const int t = threadIdx.x / LPT, l = threadIdx.x % LPT;
    float acc = 0.f;
    for (int c = l; c < d; c += LPT) {
      const int i = t * d + c;
      const float e = es[t], fd = fds[i], vv = vs[i];
      float g, fb, vb;
      if (mse) {
        g = e * c2 * (fs[i] - vv);
        fb = c2 * e * fd;
        vb = -fb;
        acc += c2 * fd * (fs[i] - vv);
      } else {
        g = -e * vv;
        fb = 0.f;
        vb = -e * fd;
        acc += -fd * vv;
      }
      Gs[i] = g;
      Fbs[i] = fb;
      if (t < cnt) {
        const long long o = ((long long)p * N + t0 + t) * d + c;
        gG[o] = g;
        gF[o] = fb;
        dv[(prow * N + t0 + t) * d + c] = -vb;
      }
    }
    red[t][l] = acc;
  }
  __syncthreads();
  if (deta && threadIdx.x < cnt) {
    float s = 0.f;
    for (int l = 0; l < LPT; ++l) s += red[threadIdx.x][l];
    deta[prow * N + t0 + threadIdx.x] = -s;
  }
  float* dk = dkh + (prow * N + t0) * d;
  if (!mlp) {
    // dphi/dX = G U^T + F_bar W^T
    for (int i = threadIdx.x; i < cnt * d; i += kThreads) {
      const int t = i / d, c = i % d;
      float s = 0.f;
      for (int cc = 0; cc < d; ++cc) s += Gs[t * d + cc] * U1[(size_t)c * d + cc] + Fbs[t * d + cc] * W1[(size_t)c * d + cc];
      dk[i] = -s;
    }
    return;
  }
  // Z_dot_bar and Z_bar per (token, hidden), in place of Z_dot and Z
  for (int i = threadIdx.x; i < kTok * hid; i += kThreads) {
    const int t = i / hid, j = i % hid;
    float adb = 0.f, ab = 0.f;
    for (int c = 0; c < d; ++c) {
      const float g = Gs[t * d + c];
      adb += g * W2[(size_t)j * d + c];
      ab += g * U2[(size_t)j * d + c] + Fbs[t * d + c] * W2[(size_t)j * d + c];
    }
    const float z = zs[i], zd = zds[i], gp = gelu_exact_prime(z);
    zds[i] = gp * adb;
    zs[i] = gelu_second(z) * zd * adb + gp * ab;
  }
  __syncthreads();
  // dphi/dX = Z_dot_bar U1^T + Z_bar W1^T
  for (int i = threadIdx.x; i < cnt * d; i += kThreads) {
    const int t = i / d, c = i % d;
    float s = 0.f;
    for (int j = 0; j < hid; ++j)
      s += zds[t * hid + j] * U1[(size_t)c * hid + j] + zs[t * hid + j] * W1[(size_t)c * hid + j];
    dk[i] = -s;
  }
}

// dphi/dW partials over token split s for a slice of 32 output columns:
// MLP: dW1[c][j] += X[c] Z_bar[j], dW2[j][c] += A_dot[j] G[c] + A[j] F_bar[c];
// linear: dW[c][c'] += X[c] F_bar[c'].  grid = (slices, S, P); part [S][P][nm][msz]
template <typename T>
__global__ void __launch_bounds__(kThreads) k_bwd_wbar(Problem pb, WRef W0, const float* __restrict__ U,
                                                      const float* __restrict__ gG, const float* __restrict__ gF,
                                                      int S, float* __restrict__ part) {
  const int slice = blockIdx.x, s = blockIdx.y, p = blockIdx.z;
  const int b = p / pb.H, h = p % pb.H;
  const int d = pb.d, N = pb.N;
  const bool mlp = pb.inner == INNER_MLP;
  const int outw = mlp ? pb.hid : d;
  const int j0 = slice * kSlice, js = min(kSlice, outw - j0);
  const int L = (N + S - 1) / S, n0 = s * L, n1 = min(N, n0 + L);
  __shared__ float xs[kTok * kMaxD], gs[kTok * kMaxD], fbs[kTok * kMaxD];
  __shared__ float zb[kTok * kSlice], ad[kTok * kSlice], aa[kTok * kSlice];
  constexpr int R = kMaxD * kSlice / kThreads;
  float acc1[R], acc2[R];
#pragma unroll
  for (int r = 0; r < R; ++r) { acc1[r] = 0.f; acc2[r] = 0.f; }
  const float* W1 = W0.mat(0, b, h);
  const float* W2 = mlp ? W0.mat(1, b, h) : nullptr;
  const float* U1 = U + (long long)p * pb.nm * pb.msz;
  const float* U2 = U1 + pb.msz;
  const int hid = pb.hid;
  const long long prow = pb.row(p);
  for (int tt = n0; tt < n1; tt += kTok) {
    const int cnt = min(kTok, n1 - tt);
    for (int i = threadIdx.x; i < kTok * d; i += kThreads) {
      const int t = i / d, c = i % d;
      float x = 0.f, g = 0.f, f = 0.f;
      if (t < cnt) {
        x = to_f32<T>(((const T*)pb.k)[(prow * N + tt + t) * d + c]);
        if (pb.stats) x = (x - pb.stats[((size_t)p * d + c) * 2]) * pb.stats[((size_t)p * d + c) * 2 + 1];
        g = gG[((long long)p * N + tt) * d + i];
        f = gF[((long long)p * N + tt) * d + i];
      }
      xs[i] = x;
      gs[i] = g;
      fbs[i] = f;
    }
    __syncthreads();
    if (mlp) {
      for (int i = threadIdx.x; i < kTok * js; i += kThreads) {
        const int t = i / js, jj = i % js, j = j0 + jj;
        float z = 0.f, zd = 0.f, adb = 0.f, ab = 0.f;
        for (int c = 0; c < d; ++c) {
          z += xs[t * d + c] * W1[(size_t)c * hid + j];
          zd += xs[t * d + c] * U1[(size_t)c * hid + j];
          adb += gs[t * d + c] * W2[(size_t)j * d + c];
          ab += gs[t * d + c] * U2[(size_t)j * d + c] + fbs[t * d + c] * W2[(size_t)j * d + c];
        }
        const float gp = gelu_exact_prime(z);
        const bool live = t < cnt;
        zb[t * kSlice + jj] = live ? gelu_second(z) * zd * adb + gp * ab : 0.f;
        ad[t * kSlice + jj] = live ? gp * zd : 0.f;
        aa[t * kSlice + jj] = live ? gelu_exact(z) : 0.f;
      }
      __syncthreads();
    }
#pragma unroll
    for (int r = 0; r < R; ++r) {
      const int e = threadIdx.x + kThreads * r;
      const int c = e / kSlice, jj = e % kSlice;     // W1 / linear W entry [c][j0 + jj]
      if (c < d && jj < js) {
        float s1 = 0.f;
        for (int t = 0; t < cnt; ++t)
          s1 += xs[t * d + c] * (mlp ? zb[t * kSlice + jj] : fbs[t * d + j0 + jj]);
        acc1[r] += s1;
      }
      if (mlp) {                                     // W2 entry [j0 + jj2][c2]
        const int jj2 = e / d, c2 = e % d;
        if (jj2 < js) {
          float s2 = 0.f;
          for (int t = 0; t < cnt; ++t) s2 += ad[t * kSlice + jj2] * gs[t * d + c2] + aa[t * kSlice + jj2] * fbs[t * d + c2];
          acc2[r] += s2;
        }
      }
    }
    __syncthreads();
  }
  float* base = part + ((size_t)s * (pb.B * pb.H) + p) * pb.nm * pb.msz;
#pragma unroll
  for (int r = 0; r < R; ++r) {
    const int e = threadIdx.x + kThreads * r;
    const int c = e / kSlice, jj = e % kSlice;
    if (c < d && jj < js) base[(size_t)c * outw + j0 + jj] = acc1[r];
    if (mlp) {
      const int jj2 = e / d, c2 = e % d;
      if (jj2 < js) base[pb.msz + (size_t)(j0 + jj2) * d + c2] = acc2[r];
    }
  }
}

// sum of S partials, in split order: out[p][e] = sum_s part[s][p][e]  (grid over P*wsz)
__global__ void __launch_bounds__(kThreads) k_sum_splits(const float* __restrict__ part, int S, long long n,
                                                        float sign, const float* __restrict__ base,
                                                        float* __restrict__ out) {
  const long long i = blockIdx.x * (long long)kThreads + threadIdx.x;
  if (i >= n) return;
  float s = 0.f;
  for (int k = 0; k < S; ++k) s += part[k * n + i];
  out[i] = (base ? base[i] : 0.f) + sign * s;
}

// dW0 in the caller's layout: shared W0 ([H, in, out]) gets the sum over the
// batch (in batch order), a per-batch W0 its pair's own gradient.
__global__ void __launch_bounds__(kThreads) k_bwd_dw0(Problem pb, const float* __restrict__ dpair, int shared,
                                                     float* __restrict__ o0, float* __restrict__ o1) {
  const int i = blockIdx.y;   // matrix
  float* out = i == 0 ? o0 : o1;
  if (!out) return;
  const long long msz = pb.msz;
  const long long e = blockIdx.x * (long long)kThreads + threadIdx.x;
  if (e >= (shared ? (long long)pb.H : (long long)pb.B * pb.H) * msz) return;
  const long long wsz = (long long)pb.nm * msz;
  if (shared) {
    const int h = (int)(e / msz);
    const long long o = e % msz;
    float s = 0.f;
    for (int b = 0; b < pb.B; ++b) s += dpair[((long long)b * pb.H + h) * wsz + i * msz + o];
    out[(long long)(pb.h0 + h) * msz + o] = s;
  } else {
    const int p = (int)(e / msz);
    const long long o = e % msz;
    out[pb.row(p) * msz + o] = dpair[(long long)p * wsz + i * msz + o];
  }
}

// key-norm backward, pass 1: per (pair, slice, channel) sums of dK_hat and
// dK_hat * K_hat over a token slice -> kp[P][S][2][d]
template <typename T>
__global__ void __launch_bounds__(kThreads) k_bwd_kn_sums(Problem pb, const float* __restrict__ dkh, int S,
                                                         float* __restrict__ kp) {
  const int s = blockIdx.x, p = blockIdx.y;
  const int d = pb.d, N = pb.N;
  const int L = (N + S - 1) / S, n0 = s * L, n1 = min(N, n0 + L);
  const int R = kThreads / d;            // row lanes (d <= 128 -> >= 2)
  const int c = threadIdx.x % d, r = threadIdx.x / d;
  const long long prow = pb.row(p);
  const float mu = pb.stats[((size_t)p * d + c) * 2], rs = pb.stats[((size_t)p * d + c) * 2 + 1];
  float s1 = 0.f, s2 = 0.f;
  if (r < R)
    for (int n = n0 + r; n < n1; n += R) {
      const long long o = (prow * N + n) * d + c;
      const float g = dkh[o], kh = (to_f32<T>(((const T*)pb.k)[o]) - mu) * rs;
      s1 += g;
      s2 += g * kh;
    }
  __shared__ float red[2][kThreads];
  red[0][threadIdx.x] = r < R ? s1 : 0.f;
  red[1][threadIdx.x] = r < R ? s2 : 0.f;
  __syncthreads();
  if (threadIdx.x < d) {
    float a = 0.f, bsum = 0.f;
    for (int rr = 0; rr < R; ++rr) { a += red[0][rr * d + threadIdx.x]; bsum += red[1][rr * d + threadIdx.x]; }
    float* o = kp + (((size_t)p * S + s) * 2) * d;
    o[threadIdx.x] = a;
    o[d + threadIdx.x] = bsum;
  }
}

// pass 2, in place: dk = rstd (dK_hat - sum1 / N - K_hat sum2 / N)
template <typename T>
__global__ void __launch_bounds__(kThreads) k_bwd_kn_apply(Problem pb, const float* __restrict__ kp, int S,
                                                          float* __restrict__ dk) {
  const int p = blockIdx.y;
  const int d = pb.d, N = pb.N;
  const long long prow = pb.row(p);
  const long long n_el = (long long)N * d;
  for (long long i = blockIdx.x * (long long)kThreads + threadIdx.x; i < n_el; i += (long long)gridDim.x * kThreads) {
    const int c = (int)(i % d);
    float s1 = 0.f, s2 = 0.f;
    for (int s = 0; s < S; ++s) {
      const float* o = kp + (((size_t)p * S + s) * 2) * d;
      s1 += o[c];
      s2 += o[d + c];
    }
    const float mu = pb.stats[((size_t)p * d + c) * 2], rs = pb.stats[((size_t)p * d + c) * 2 + 1];
    const long long o = prow * n_el + i;
    const float kh = (to_f32<T>(((const T*)pb.k)[o]) - mu) * rs;
    dk[o] = rs * (dk[o] - s1 / (float)N - kh * s2 / (float)N);
  }
}

}  // namespace

int bwd_kn_splits(const Problem& pb) {
  long long s = 4LL * device_cu_count() / ((long long)pb.B * pb.H);
  const long long maxs = (pb.N + 63) / 64;
  if (s > maxs) s = maxs;
  if (s < 1) s = 1;
  return (int)s;
}

void launch_backward(const Problem& pb, const WRef& w0, const float* wstar_states, const void* dO, int S,
                     float* part, float* dO32, float* U, float* gG, float* gF, float* dpair, float* knp, int S_kn,
                     float* dq, float* dk, float* dv, float* deta, float* const* dW0, int w0_shared,
                     hipStream_t st) {
  const int P = pb.B * pb.H;
  const long long pw = (long long)P * pb.nm * pb.msz;
  WRef ws{};
  for (int i = 0; i < 3; ++i) ws.m[i] = wstar_states + (long long)(i < pb.nm ? i : 0) * pb.msz;
  ws.sb = (long long)pb.H * pb.nm * pb.msz;
  ws.sh = (long long)pb.nm * pb.msz;
  const dim3 tiles((pb.N + kTok - 1) / kTok, P);
  const unsigned nblk = (unsigned)((pw + kThreads - 1) / kThreads);
  // readout backward: dO as fp32 rows, dQ, then U = dS/dW* through the generic dW kernel on (Q, dO)
  if (pb.bf16) {
    hipLaunchKernelGGL(k_bwd_rows_f32<bf16>, dim3(64, P), dim3(kThreads), 0, st, pb, (const bf16*)dO, dO32);
    hipLaunchKernelGGL(k_bwd_readout_tok<bf16>, tiles, dim3(kThreads), 0, st, pb, ws, dO32, dq);
  } else {
    hipLaunchKernelGGL(k_bwd_rows_f32<float>, dim3(64, P), dim3(kThreads), 0, st, pb, (const float*)dO, dO32);
    hipLaunchKernelGGL(k_bwd_readout_tok<float>, tiles, dim3(kThreads), 0, st, pb, ws, dO32, dq);
  }
  Problem pq = pb;
  pq.k = pb.q;
  pq.stats = nullptr;
  launch_gen_dW(pq, ws, 0, pb.N, dO32, S, part, st);
  hipLaunchKernelGGL(k_sum_splits, dim3(nblk), dim3(kThreads), 0, st, part, S, pw, 1.0f, (const float*)nullptr, U);
  // through the step: per-token terms, then the weight reduction
  const int outw = pb.inner == INNER_MLP ? pb.hid : pb.d;
  const dim3 wgrid((outw + kSlice - 1) / kSlice, S, P);
  if (pb.bf16) {
    hipLaunchKernelGGL(k_bwd_key_tok<bf16>, tiles, dim3(kThreads), 0, st, pb, w0, U, dv, deta, dk, gG, gF);
    hipLaunchKernelGGL(k_bwd_wbar<bf16>, wgrid, dim3(kThreads), 0, st, pb, w0, U, gG, gF, S, part);
  } else {
    hipLaunchKernelGGL(k_bwd_key_tok<float>, tiles, dim3(kThreads), 0, st, pb, w0, U, dv, deta, dk, gG, gF);
    hipLaunchKernelGGL(k_bwd_wbar<float>, wgrid, dim3(kThreads), 0, st, pb, w0, U, gG, gF, S, part);
  }
  // dW0 of each pair = U - dphi/dW0, then the caller's layout and the key norm
  hipLaunchKernelGGL(k_sum_splits, dim3(nblk), dim3(kThreads), 0, st, part, S, pw, -1.0f, (const float*)U, dpair);
  launch_bwd_tail(pb, dpair, w0_shared, dW0, dk, S_kn, knp, st);
}

void launch_bwd_tail(const Problem& pb, const float* dpair, int w0_shared, float* const* dW0, float* dk, int S_kn,
                     float* knp, hipStream_t st) {
  const int P = pb.B * pb.H;
  const long long nout = (w0_shared ? (long long)pb.H : (long long)P) * pb.msz;
  hipLaunchKernelGGL(k_bwd_dw0, dim3((unsigned)((nout + kThreads - 1) / kThreads), pb.nm), dim3(kThreads), 0, st, pb,
                     dpair, w0_shared, dW0[0], pb.nm > 1 ? dW0[1] : nullptr);
  // key norm: dK from dK_hat in place
  if (pb.stats) {
    const dim3 g1(S_kn, P);
    const dim3 g2((unsigned)std::min<long long>(((long long)pb.N * pb.d + kThreads - 1) / kThreads, 256), P);
    if (pb.bf16) {
      hipLaunchKernelGGL(k_bwd_kn_sums<bf16>, g1, dim3(kThreads), 0, st, pb, dk, S_kn, knp);
      hipLaunchKernelGGL(k_bwd_kn_apply<bf16>, g2, dim3(kThreads), 0, st, pb, knp, S_kn, dk);
    } else {
      hipLaunchKernelGGL(k_bwd_kn_sums<float>, g1, dim3(kThreads), 0, st, pb, dk, S_kn, knp);
      hipLaunchKernelGGL(k_bwd_kn_apply<float>, g2, dim3(kThreads), 0, st, pb, knp, S_kn, dk);
    }
  }
}

}  // namespace ttt
