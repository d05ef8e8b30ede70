// Generic TTT-layer kernels: fp32 arithmetic on fp32 or bf16 tensors, every
// matrix inner model (linear, GELU MLP, SwiGLU, the simplified GLU of the ViT3
// page), both losses, any d <= 128 and h <= 512.  They serve the fp32 configuration (exact erf GELU, fp32 sums) and
// every shape the MFMA kernels do not cover.  Plain LDS-staged loops: the
// bf16 MFMA kernels are the fast path.
//
// The three steps of one inner update (ViT3 summary page, section 02):
//   (i)   forward on the keys       V_hat = F_W(K_hat)
//   (ii)  loss gradient, backward   G = dL/dV_hat, dW by hand
//   (iii) readout on the queries    O = F_W*(Q)
// with the losses of section 03 guideline 1 / the LaCT page (MSE mean over the
// n_b*d entries, negative dot product), per-token rates eta_n folded into G.
#include "ttt_internal.h"

namespace ttt {

namespace {

constexpr int kThreads = 256;
constexpr int kTok = 16;     // tokens per workgroup tile
constexpr int kSlice = 32;   // hidden columns per dW workgroup
constexpr int kMaxD = 128;
constexpr int kMaxH = 512;

__device__ __forceinline__ float eta_of(const Problem& pb, int p, int n) {
  float e = pb.eta_scale;
  if (pb.eta_tok) e *= pb.eta_tok[(size_t)pb.row(p) * pb.N + n];
  return e;
}

// Row n of pair p of a [B,H,N,d] tensor into LDS, as fp32; keys are
// instance-normalised on the way when statistics are given.
template <typename T>
__device__ __forceinline__ void stage_rows(const Problem& pb, const T* base, int p, int t0, int nt,
                                           const float* stats, float* dst /*[kTok][d]*/) {
  const int d = pb.d;
  for (int i = threadIdx.x; i < kTok * d; i += kThreads) {
    const int t = i / d, c = i % d;
    float x = 0.f;
    if (t < nt) {
      x = to_f32<T>(base[((size_t)pb.row(p) * pb.N + t0 + t) * d + c]);
      if (stats) {
        const float* s = stats + ((size_t)p * d + c) * 2;
        x = (x - s[0]) * s[1];
      }
    }
    dst[t * d + c] = x;
  }
}

// Hidden activations of the inner model for kTok staged rows x:
//   MLP: act = gelu(x W1);  SwiGLU: act = silu(x W1) * (x W3);
//   GLU: act = (x W1) * silu(x Wg) (Wg passed as W3), which is F itself.
__device__ __forceinline__ void hidden_fwd(const Problem& pb, const float* W1, const float* W3,
                                           const float* x, float* act) {
  const int d = pb.d, hid = pb.hid;
  for (int i = threadIdx.x; i < kTok * hid; i += kThreads) {
    const int t = i / hid, j = i % hid;
    float z1 = 0.f, z3 = 0.f;
    for (int c = 0; c < d; ++c) {
      const float xv = x[t * d + c];
      z1 += xv * W1[(size_t)c * hid + j];
      if (W3) z3 += xv * W3[(size_t)c * hid + j];
    }
    act[i] = pb.inner == INNER_SWIGLU ? z1 * sigmoid_f(z1) * z3
           : pb.inner == INNER_GLU    ? z1 * z3 * sigmoid_f(z3)
                                      : gelu_exact(z1);
  }
}

// out[t][c] = F_W(x_t)[c] for the staged rows.
__device__ __forceinline__ void inner_out(const Problem& pb, const WRef& W, int b, int h,
                                          const float* x, float* act, float* out) {
  const int d = pb.d;
  if (pb.inner == INNER_LINEAR) {
    const float* Wl = W.mat(0, b, h);
    for (int i = threadIdx.x; i < kTok * d; i += kThreads) {
      const int t = i / d, c = i % d;
      float s = 0.f;
      for (int cc = 0; cc < d; ++cc) s += x[t * d + cc] * Wl[(size_t)cc * d + c];
      out[i] = s;
    }
    return;
  }
  const float* W1 = W.mat(0, b, h);
  const float* W2 = W.mat(1, b, h);
  if (pb.inner == INNER_GLU) {            // no output projection: F = act
    hidden_fwd(pb, W1, W2, x, out);
    return;
  }
  const float* W3 = pb.inner == INNER_SWIGLU ? W.mat(2, b, h) : nullptr;
  hidden_fwd(pb, W1, W3, x, act);
  __syncthreads();
  const int hid = pb.hid;
  for (int i = threadIdx.x; i < kTok * d; i += kThreads) {
    const int t = i / d, c = i % d;
    float s = 0.f;
    for (int j = 0; j < hid; ++j) s += act[t * hid + j] * W2[(size_t)j * d + c];
    out[i] = s;
  }
}

// (i)+(ii, first half): G = dL/dV_hat for tokens [t0, t0+nt) of pair blockIdx.y.
template <typename T>
__global__ void __launch_bounds__(kThreads) k_gen_grad_out(Problem pb, WRef W, int t0, int nt,
                                                           float* __restrict__ gbuf) {
  const int p = blockIdx.y, b = p / pb.H, h = p % pb.H;
  const int tt = blockIdx.x * kTok;
  const int cnt = min(kTok, nt - tt);
  const int d = pb.d;
  __shared__ float xs[kTok * kMaxD];
  __shared__ float vh[kTok * kMaxD];
  __shared__ float act[kTok * kMaxH];
  float* g = gbuf + ((size_t)p * nt + tt) * d;
  if (pb.loss == LOSS_DOT) {   // G_n = -eta_n v_n: no forward needed
    for (int i = threadIdx.x; i < cnt * d; i += kThreads) {
      const int t = i / d, c = i % d, n = t0 + tt + t;
      g[i] = -eta_of(pb, p, n) * to_f32<T>(((const T*)pb.v)[((size_t)pb.row(p) * pb.N + n) * d + c]);
    }
    return;
  }
  stage_rows<T>(pb, (const T*)pb.k, p, t0 + tt, cnt, pb.stats, xs);
  __syncthreads();
  inner_out(pb, W, b, h, xs, act, vh);
  __syncthreads();
  const float scale = 2.0f / ((float)nt * (float)d);
  for (int i = threadIdx.x; i < cnt * d; i += kThreads) {
    const int t = i / d, c = i % d, n = t0 + tt + t;
    const float vv = to_f32<T>(((const T*)pb.v)[((size_t)pb.row(p) * pb.N + n) * d + c]);
    g[i] = eta_of(pb, p, n) * scale * (vh[i] - vv);
  }
}

// (ii, second half): partial dW of one hidden slice over one token split.
// grid = (slices, S, P).  part layout [S][P][nm][msz].
template <typename T>
__global__ void __launch_bounds__(kThreads) k_gen_dW(Problem pb, WRef W, int t0, int nt,
                                                     const float* __restrict__ gbuf, int S,
                                                     float* __restrict__ part) {
  const int slice = blockIdx.x, s = blockIdx.y, p = blockIdx.z;
  const int b = p / pb.H, h = p % pb.H;
  const int d = pb.d;
  const int outw = pb.inner == INNER_LINEAR ? d : pb.hid;   // columns being sliced
  const int j0 = slice * kSlice;
  const int js = min(kSlice, outw - j0);
  const int L = (nt + S - 1) / S;
  const int n0 = s * L, n1 = min(nt, n0 + L);
  __shared__ float xs[kTok * kMaxD];
  __shared__ float gs[kTok * kMaxD];
  __shared__ float aa[kTok * kSlice];   // A (MLP) / Hh (SwiGLU)
  __shared__ float d1[kTok * kSlice];   // dZ (MLP) / dZ1 (SwiGLU)
  __shared__ float d3[kTok * kSlice];   // dZ3 (SwiGLU)
  // accumulator entries owned by this thread: e = threadIdx.x + 256*r over d*kSlice
  float acc1[kMaxD * kSlice / kThreads], acc2[kMaxD * kSlice / kThreads], acc3[kMaxD * kSlice / kThreads];
  constexpr int R = kMaxD * kSlice / kThreads;
#pragma unroll
  for (int r = 0; r < R; ++r) { acc1[r] = 0.f; acc2[r] = 0.f; acc3[r] = 0.f; }
  const float* W1 = W.mat(0, b, h);
  const bool glu = pb.inner == INNER_GLU;
  // GLU: its gate matrix (matrix 1) takes the place of W3, and there is no W2
  const float* W2 = pb.inner == INNER_LINEAR || glu ? nullptr : W.mat(1, b, h);
  const float* W3 = pb.inner == INNER_SWIGLU ? W.mat(2, b, h) : glu ? W.mat(1, b, h) : nullptr;
  const int hid = pb.hid;
  for (int tt = n0; tt < n1; tt += kTok) {
    const int cnt = min(kTok, n1 - tt);
    stage_rows<T>(pb, (const T*)pb.k, p, t0 + tt, cnt, pb.stats, xs);
    for (int i = threadIdx.x; i < kTok * d; i += kThreads) {
      const int t = i / d;
      gs[i] = t < cnt ? gbuf[((size_t)p * nt + tt) * d + i] : 0.f;
    }
    __syncthreads();
    if (pb.inner != INNER_LINEAR) {
      for (int i = threadIdx.x; i < kTok * js; i += kThreads) {
        const int t = i / js, jj = i % js, j = j0 + jj;
        float z1 = 0.f, z3 = 0.f, da = 0.f;
        for (int c = 0; c < d; ++c) {
          z1 += xs[t * d + c] * W1[(size_t)c * hid + j];
          if (W3) z3 += xs[t * d + c] * W3[(size_t)c * hid + j];
          if (W2) da += gs[t * d + c] * W2[(size_t)j * d + c];
        }
        const bool live = t < cnt;
        if (glu) {              // F = U * silu(Zg): dU = G silu(Zg), dZg = G U silu'(Zg)
          const float sg = sigmoid_f(z3), gj = gs[t * d + j];
          d1[t * kSlice + jj] = live ? gj * z3 * sg : 0.f;
          d3[t * kSlice + jj] = live ? gj * z1 * sg * (1.f + z3 * (1.f - sg)) : 0.f;
        } else if (pb.inner == INNER_MLP) {
          aa[t * kSlice + jj] = live ? gelu_exact(z1) : 0.f;
          d1[t * kSlice + jj] = live ? da * gelu_exact_prime(z1) : 0.f;
        } else {
          const float sg = sigmoid_f(z1), si = z1 * sg;
          aa[t * kSlice + jj] = live ? si * z3 : 0.f;
          d1[t * kSlice + jj] = live ? da * z3 * sg * (1.f + z1 * (1.f - sg)) : 0.f;
          d3[t * kSlice + jj] = live ? da * si : 0.f;
        }
      }
    }
    __syncthreads();
#pragma unroll
    for (int r = 0; r < R; ++r) {
      const int e = threadIdx.x + kThreads * r;
      // dW1[c][j] (and dW3, and the linear dW) entries: e -> (c = e / kSlice, jj = e % kSlice)
      const int c = e / kSlice, jj = e % kSlice;
      if (c < d && jj < js) {
        float s1 = 0.f, s3 = 0.f;
        for (int t = 0; t < cnt; ++t) {
          const float xv = xs[t * d + c];
          if (pb.inner == INNER_LINEAR) s1 += xv * gs[t * d + j0 + jj];
          else {
            s1 += xv * d1[t * kSlice + jj];
            if (W3) s3 += xv * d3[t * kSlice + jj];
          }
        }
        acc1[r] += s1;
        acc3[r] += s3;
      }
      // dW2[j][c] entries: e -> (jj = e / d, c = e % d)
      if (W2) {
        const int jj2 = e / d, c2 = e % d;
        if (jj2 < js) {
          float s2 = 0.f;
          for (int t = 0; t < cnt; ++t) s2 += aa[t * kSlice + jj2] * gs[t * d + c2];
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
    if (c < d && jj < js) {
      base[(size_t)c * outw + j0 + jj] = acc1[r];
      if (W3) base[(glu ? 1 : 2) * pb.msz + (size_t)c * outw + j0 + jj] = acc3[r];
    }
    if (W2) {
      const int jj2 = e / d, c2 = e % d;
      if (jj2 < js) base[pb.msz + (size_t)(j0 + jj2) * d + c2] = acc2[r];
    }
  }
}

// (iii) readout: O = F_W(Q).  grid = (groups of kTok tokens per chunk, chunks, P).
// Full-batch mode (chunk == 0): every token reads the updated state 1.
// Causal mode: chunk 0 reads W0, chunk c >= 1 reads state c (the weights left
// by chunks 0..c-1); state c lives at states + (c-1)*state_stride, [P][nm][msz].
template <typename T>
__global__ void __launch_bounds__(kThreads) k_gen_query(Problem pb, WRef w0, const float* __restrict__ states,
                                                        long long state_stride, int chunk) {
  const int g = blockIdx.x, c = blockIdx.y, p = blockIdx.z;
  const int b = p / pb.H, h = p % pb.H;
  const int c0 = chunk ? c * chunk : 0;
  const int c1 = chunk ? min(pb.N, c0 + chunk) : pb.N;
  const int tt = c0 + g * kTok;
  if (tt >= c1) return;
  const int cnt = min(kTok, c1 - tt);
  const int d = pb.d;
  __shared__ float xs[kTok * kMaxD];
  __shared__ float os[kTok * kMaxD];
  __shared__ float act[kTok * kMaxH];
  WRef W = w0;
  const int state = chunk ? c : 1;
  if (state > 0) {
    const float* base = states + (state - 1) * state_stride;
    const int P = pb.B * pb.H;
    (void)P;
    W.m[0] = base;
    W.m[1] = base + pb.msz;
    W.m[2] = base + 2 * pb.msz;
    W.sb = (long long)pb.H * pb.nm * pb.msz;
    W.sh = (long long)pb.nm * pb.msz;
  }
  stage_rows<T>(pb, (const T*)pb.q, p, tt, cnt, nullptr, xs);
  __syncthreads();
  inner_out(pb, W, b, h, xs, act, os);
  __syncthreads();
  T* o = (T*)pb.o + ((size_t)pb.row(p) * pb.N + tt) * d;
  for (int i = threadIdx.x; i < cnt * d; i += kThreads) o[i] = from_f32<T>(os[i]);
}

__global__ void k_check_finite(const void* o, int bf, long long n, const float* w0, const float* w1,
                               const float* w2, long long wn, int* flag) {
  long long i = blockIdx.x * (long long)blockDim.x + threadIdx.x;
  const long long stride = (long long)gridDim.x * blockDim.x;
  bool bad = false;
  for (long long j = i; j < n; j += stride) {
    const float x = bf ? (float)((const bf16*)o)[j] : ((const float*)o)[j];
    bad |= !isfinite(x);
  }
  const float* ws[3] = {w0, w1, w2};
  for (int m = 0; m < 3; ++m)
    if (ws[m])
      for (long long j = i; j < wn; j += stride) bad |= !isfinite(ws[m][j]);
  if (bad) atomicOr(flag, 1);
}

__global__ void k_zero_flag(int* flag) { if (threadIdx.x == 0) *flag = 0; }

__global__ void __launch_bounds__(256) k_fill_zero(float* p, long long n) {
  for (long long i = blockIdx.x * 256LL + threadIdx.x; i < n; i += (long long)gridDim.x * 256) p[i] = 0.f;
}

}  // namespace

void launch_zero_flag(int* flag, hipStream_t st) {
  hipLaunchKernelGGL(k_zero_flag, dim3(1), dim3(64), 0, st, flag);
}

void launch_fill_zero(float* p, long long n, hipStream_t st) {
  long long blocks = (n + 255) / 256;
  if (blocks > 4096) blocks = 4096;
  if (blocks < 1) blocks = 1;
  hipLaunchKernelGGL(k_fill_zero, dim3((unsigned)blocks), dim3(256), 0, st, p, n);
}

void launch_gen_grad_out(const Problem& pb, const WRef& W, int t0, int nt, float* gbuf, hipStream_t st) {
  dim3 grid((nt + kTok - 1) / kTok, pb.B * pb.H);
  if (pb.bf16) hipLaunchKernelGGL(k_gen_grad_out<bf16>, grid, dim3(kThreads), 0, st, pb, W, t0, nt, gbuf);
  else hipLaunchKernelGGL(k_gen_grad_out<float>, grid, dim3(kThreads), 0, st, pb, W, t0, nt, gbuf);
}

void launch_gen_dW(const Problem& pb, const WRef& W, int t0, int nt, const float* gbuf, int S, float* part,
                   hipStream_t st) {
  const int outw = pb.inner == INNER_LINEAR ? pb.d : pb.hid;
  dim3 grid((outw + kSlice - 1) / kSlice, S, pb.B * pb.H);
  if (pb.bf16) hipLaunchKernelGGL(k_gen_dW<bf16>, grid, dim3(kThreads), 0, st, pb, W, t0, nt, gbuf, S, part);
  else hipLaunchKernelGGL(k_gen_dW<float>, grid, dim3(kThreads), 0, st, pb, W, t0, nt, gbuf, S, part);
}

void launch_gen_query(const Problem& pb, const WRef& w0, const float* states, long long state_stride,
                      int nchunks, int chunk, hipStream_t st) {
  const int span = chunk ? chunk : pb.N;
  dim3 grid((span + kTok - 1) / kTok, nchunks, pb.B * pb.H);
  if (pb.bf16)
    hipLaunchKernelGGL(k_gen_query<bf16>, grid, dim3(kThreads), 0, st, pb, w0, states, state_stride, chunk);
  else
    hipLaunchKernelGGL(k_gen_query<float>, grid, dim3(kThreads), 0, st, pb, w0, states, state_stride, chunk);
}

void launch_check_finite(const Problem& pb, long long n, float* const* wfinal, long long wcount, int* flag,
                         hipStream_t st) {
  hipLaunchKernelGGL(k_check_finite, dim3(1024), dim3(256), 0, st, pb.o, pb.bf16, n, wfinal[0], wfinal[1],
                     wfinal[2], wcount, flag);
}

}  // namespace ttt
