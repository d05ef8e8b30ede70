// Depthwise-convolution inner model of the ViT3 block (ViT3 summary page,
// section 03 guideline 6, the inner-model table, section 04 and its glossary
// entry "DWConv"): the fast weight is a per-channel k x k kernel w[c] that
// cross-correlates channel c of the token raster (token t = i gw + j, zero
// padding of r = (k - 1) / 2):
//     F(x)[t, c] = sum_{a, b} w[c][a k + b] x[(i + a - r) gw + (j + b - r), c]
// One full-batch step (steps (i)-(ii) of section 02):
//     G = eta_n 2/(N d) (F(K_hat) - V)  [MSE]   |   -eta_n V  [dot]
//     dw[c][a k + b] = sum_t G[t, c] K_hat[shift_{a,b}(t), c]
// and the readout (iii) O = F_{w*}(Q).  Per token and channel this is k^2
// multiply-adds per product, against 2 bytes read per bf16 element: the
// kernels are bound by HBM (the neighbours come from the L1/L2 caches), so
// they are plain fp32 loops with lanes along the channels (coalesced rows)
// and no matrix cores.
#include "ttt_internal.h"

namespace ttt {

namespace {

constexpr int kWaves = 4;
constexpr int kMaxC = 128;          // channels: lane c and c + 64
constexpr int kQTok = 64;           // tokens per readout workgroup

template <typename T>
__device__ __forceinline__ float ldf(const T* p) { return to_f32<T>(*p); }

// partial dw of token split s of pair p -> part[(s P + p) msz + c k^2 + tap]
// grid = (S, P), 256 threads: wave w takes tokens n0 + w, n0 + w + 4, ...
template <typename T, int K>
__global__ void __launch_bounds__(kWaves * 64) k_dw_grad(Problem pb, WRef W, int S, float mse_scale,
                                                         float* __restrict__ part) {
  constexpr int KK = K * K, R = (K - 1) / 2;
  const int s = blockIdx.x, p = blockIdx.y;
  const int b = p / pb.H, h = p % pb.H;
  const int d = pb.d, gw = pb.gw, gh = pb.gh, N = pb.N;
  const long long prow = pb.row(p);
  const T* kp = (const T*)pb.k + prow * N * d;
  const T* vp = (const T*)pb.v + prow * N * d;
  const float* ep = pb.eta_tok ? pb.eta_tok + prow * N : nullptr;
  const float* w = W.mat(0, b, h);
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  const int L = (N + S - 1) / S, n0 = s * L, n1 = min(N, n0 + L);
  const bool mse = pb.loss == LOSS_MSE;
  float acc[2][KK], wr[2][KK], mu[2] = {0.f, 0.f}, rs[2] = {1.f, 1.f};
#pragma unroll
  for (int u = 0; u < 2; ++u) {
    const int c = lane + 64 * u;
#pragma unroll
    for (int t = 0; t < KK; ++t) { acc[u][t] = 0.f; wr[u][t] = (mse && c < d) ? w[c * KK + t] : 0.f; }
    if (pb.stats && c < d) { mu[u] = pb.stats[((size_t)p * d + c) * 2]; rs[u] = pb.stats[((size_t)p * d + c) * 2 + 1]; }
  }
  for (int n = n0 + wv; n < n1; n += kWaves) {
    const int i = n / gw, j = n % gw;
    const float et = pb.eta_scale * (ep ? ep[n] : 1.f);
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      const int c = lane + 64 * u;
      if (c >= d) continue;
      float nb[KK];
#pragma unroll
      for (int a = 0; a < K; ++a)
#pragma unroll
        for (int bb = 0; bb < K; ++bb) {
          const int ii = i + a - R, jj = j + bb - R;
          const bool in = ii >= 0 && ii < gh && jj >= 0 && jj < gw;
          nb[a * K + bb] = in ? (ldf(kp + ((long long)ii * gw + jj) * d + c) - mu[u]) * rs[u] : 0.f;
        }
      const float vv = ldf(vp + (long long)n * d + c);
      float g;
      if (mse) {
        float f = 0.f;
#pragma unroll
        for (int t = 0; t < KK; ++t) f = fmaf(wr[u][t], nb[t], f);
        g = et * mse_scale * (f - vv);
      } else {
        g = -et * vv;
      }
#pragma unroll
      for (int t = 0; t < KK; ++t) acc[u][t] = fmaf(g, nb[t], acc[u][t]);
    }
  }
  // the four waves' sums, added in wave order
  __shared__ float red[kWaves][kMaxC][KK];
#pragma unroll
  for (int u = 0; u < 2; ++u)
#pragma unroll
    for (int t = 0; t < KK; ++t) red[wv][lane + 64 * u][t] = acc[u][t];
  __syncthreads();
  const long long msz = pb.msz;
  float* out = part + ((long long)s * pb.B * pb.H + p) * msz;
  for (int e = threadIdx.x; e < d * KK; e += kWaves * 64) {
    const int c = e / KK, t = e % KK;
    float v = 0.f;
#pragma unroll
    for (int q = 0; q < kWaves; ++q) v += red[q][c][t];
    out[e] = v;
  }
}

// O = F_w(Q) from the state (layout [P][d k^2]).  grid = (ceil(N / 64), P)
template <typename T, int K>
__global__ void __launch_bounds__(kWaves * 64) k_dw_query(Problem pb, const float* __restrict__ state) {
  constexpr int KK = K * K, R = (K - 1) / 2;
  const int p = blockIdx.y;
  const int d = pb.d, gw = pb.gw, gh = pb.gh, N = pb.N;
  const long long prow = pb.row(p);
  const T* qp = (const T*)pb.q + prow * N * d;
  T* op = (T*)pb.o + prow * N * d;
  const float* w = state + (long long)p * pb.msz;
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  float wr[2][KK];
#pragma unroll
  for (int u = 0; u < 2; ++u)
#pragma unroll
    for (int t = 0; t < KK; ++t) wr[u][t] = lane + 64 * u < d ? w[(lane + 64 * u) * KK + t] : 0.f;
  const int n0 = blockIdx.x * kQTok, n1 = min(N, n0 + kQTok);
  for (int n = n0 + wv; n < n1; n += kWaves) {
    const int i = n / gw, j = n % gw;
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      const int c = lane + 64 * u;
      if (c >= d) continue;
      float f = 0.f;
#pragma unroll
      for (int a = 0; a < K; ++a)
#pragma unroll
        for (int bb = 0; bb < K; ++bb) {
          const int ii = i + a - R, jj = j + bb - R;
          if (ii >= 0 && ii < gh && jj >= 0 && jj < gw)
            f = fmaf(wr[u][a * K + bb], ldf(qp + ((long long)ii * gw + jj) * d + c), f);
        }
      op[(long long)n * d + c] = from_f32<T>(f);
    }
  }
}

template <typename T>
void grad_k(const Problem& pb, const WRef& W, int S, float scale, float* part, hipStream_t st) {
  const dim3 grid(S, pb.B * pb.H), block(kWaves * 64);
  switch (pb.ck) {
    case 1: hipLaunchKernelGGL((k_dw_grad<T, 1>), grid, block, 0, st, pb, W, S, scale, part); break;
    case 3: hipLaunchKernelGGL((k_dw_grad<T, 3>), grid, block, 0, st, pb, W, S, scale, part); break;
    case 5: hipLaunchKernelGGL((k_dw_grad<T, 5>), grid, block, 0, st, pb, W, S, scale, part); break;
    default: hipLaunchKernelGGL((k_dw_grad<T, 7>), grid, block, 0, st, pb, W, S, scale, part); break;
  }
}

template <typename T>
void query_k(const Problem& pb, const float* state, hipStream_t st) {
  const dim3 grid((pb.N + kQTok - 1) / kQTok, pb.B * pb.H), block(kWaves * 64);
  switch (pb.ck) {
    case 1: hipLaunchKernelGGL((k_dw_query<T, 1>), grid, block, 0, st, pb, state); break;
    case 3: hipLaunchKernelGGL((k_dw_query<T, 3>), grid, block, 0, st, pb, state); break;
    case 5: hipLaunchKernelGGL((k_dw_query<T, 5>), grid, block, 0, st, pb, state); break;
    default: hipLaunchKernelGGL((k_dw_query<T, 7>), grid, block, 0, st, pb, state); break;
  }
}

}  // namespace

// token splits: about four workgroups per CU over all pairs, at least 128
// tokens each
int dwconv_grad_splits(const Problem& pb) {
  const long long P = (long long)pb.B * pb.H;
  long long s = (4LL * device_cu_count() + P - 1) / P;
  const long long maxs = (pb.N + 127) / 128;
  if (s > maxs) s = maxs;
  if (s < 1) s = 1;
  return (int)s;
}

void launch_dwconv_grad(const Problem& pb, const WRef& W, int S, float* part, hipStream_t st) {
  const float scale = 2.0f / ((float)pb.N * (float)pb.d);
  if (pb.bf16) grad_k<bf16>(pb, W, S, scale, part, st);
  else grad_k<float>(pb, W, S, scale, part, st);
}

void launch_dwconv_query(const Problem& pb, const float* state, hipStream_t st) {
  if (pb.bf16) query_k<bf16>(pb, state, st);
  else query_k<float>(pb, state, st);
}

}  // namespace ttt
