// Key instance-normalisation statistics (Test-Time Training vs Sleep page,
// section "Side one": keys carry a constant shift that must be removed before
// the inner optimisation).  Per (batch, head, channel), over the N tokens:
// mean and 1/sqrt(biased variance + eps).
//
// Every workgroup reduces one token slice of one (b, h) pair to (count, mean,
// M2) per channel, so the whole chip streams K once from HBM; the slices are
// merged with Chan's parallel-variance formula, either by the gradient kernel
// itself (MFMA path) or by a tiny second kernel (generic path).
#include "ttt_internal.h"

namespace ttt {

namespace {

constexpr int kThreads = 256;

template <typename T>
__device__ __forceinline__ void load8(const T* p, float* x);
template <>
__device__ __forceinline__ void load8<bf16>(const bf16* p, float* x) {
  bf16x8 v = *reinterpret_cast<const bf16x8*>(p);
#pragma unroll
  for (int i = 0; i < 8; ++i) x[i] = (float)v[i];
}
template <>
__device__ __forceinline__ void load8<float>(const float* p, float* x) {
  float4 a = reinterpret_cast<const float4*>(p)[0];
  float4 b = reinterpret_cast<const float4*>(p)[1];
  x[0] = a.x; x[1] = a.y; x[2] = a.z; x[3] = a.w; x[4] = b.x; x[5] = b.y; x[6] = b.z; x[7] = b.w;
}

// d % 8 == 0: each thread owns 8 consecutive channels of one token row; the
// workgroup walks the slice R = 256/(d/8) rows at a time, four rows in flight
// per thread.  One pass: sums of (k - s) and (k - s)^2 around the pair's first
// key row s (so the variance does not cancel), turned into (count, mean, M2).
template <typename T>
__global__ void __launch_bounds__(kThreads) k_stats_partial_v8(const T* __restrict__ k, int N, int d,
                                                               int S, float* __restrict__ part, int H, int Hs,
                                                               int h0) {
  const int s = blockIdx.x, p = blockIdx.y;
  const long long prow = (long long)(p / H) * Hs + h0 + p % H;   // the pair's row of k
  const int L = (N + S - 1) / S;
  const int n0 = s * L, n1 = min(N, n0 + L);
  const int groups = d >> 3;
  const int R = kThreads / groups;
  const int cg = threadIdx.x % groups, r = threadIdx.x / groups;
  const bool active = r < R;
  const T* base = k + (size_t)prow * N * d + cg * 8;
  __shared__ float red[2][kThreads][8];
  float sh[8], s1[8], s2[8];
  load8<T>(base, sh);                       // shift: the pair's first key row
#pragma unroll
  for (int i = 0; i < 8; ++i) { s1[i] = 0.f; s2[i] = 0.f; }
  if (active) {
    int n = n0 + r;
    for (; n + 3 * R < n1; n += 4 * R) {
      float x[4][8];
#pragma unroll
      for (int u = 0; u < 4; ++u) load8<T>(base + (size_t)(n + u * R) * d, x[u]);
#pragma unroll
      for (int u = 0; u < 4; ++u)
#pragma unroll
        for (int i = 0; i < 8; ++i) { const float t = x[u][i] - sh[i]; s1[i] += t; s2[i] += t * t; }
    }
    for (; n < n1; n += R) {
      float x[8];
      load8<T>(base + (size_t)n * d, x);
#pragma unroll
      for (int i = 0; i < 8; ++i) { const float t = x[i] - sh[i]; s1[i] += t; s2[i] += t * t; }
    }
  }
#pragma unroll
  for (int i = 0; i < 8; ++i) { red[0][threadIdx.x][i] = s1[i]; red[1][threadIdx.x][i] = s2[i]; }
  __syncthreads();
  const int cnt = max(n1 - n0, 0);
  if (threadIdx.x < d) {
    const int c = threadIdx.x, g = c >> 3, j = c & 7;
    float a1 = 0.f, a2 = 0.f;
    for (int rr = 0; rr < R; ++rr) { a1 += red[0][rr * groups + g][j]; a2 += red[1][rr * groups + g][j]; }
    float shift[8];
    load8<T>(k + (size_t)prow * N * d + g * 8, shift);
    const float m1 = cnt ? a1 / (float)cnt : 0.f;
    float* o = part + ((size_t)p * S + s) * 3 * d;
    o[c] = (float)cnt;
    o[d + c] = shift[j] + m1;
    o[2 * d + c] = fmaxf(a2 - a1 * m1, 0.f);
  }
}

// any d <= 256: thread = (channel, row lane)
template <typename T>
__global__ void __launch_bounds__(kThreads) k_stats_partial_scalar(const T* __restrict__ k, int N, int d,
                                                                   int S, float* __restrict__ part, int H, int Hs,
                                                                   int h0) {
  const int s = blockIdx.x, p = blockIdx.y;
  const long long prow = (long long)(p / H) * Hs + h0 + p % H;
  const int L = (N + S - 1) / S;
  const int n0 = s * L, n1 = min(N, n0 + L);
  const int R = kThreads / d;
  const int c = threadIdx.x % d, r = threadIdx.x / d;
  const bool active = r < R;
  const T* base = k + (size_t)prow * N * d + c;
  __shared__ float red[kThreads];
  __shared__ float mean_s[256];
  float acc = 0.f;
  if (active)
    for (int n = n0 + r; n < n1; n += R) acc += to_f32<T>(base[(size_t)n * d]);
  red[threadIdx.x] = active ? acc : 0.f;
  __syncthreads();
  const int cnt = max(n1 - n0, 0);
  if (threadIdx.x < d) {
    float sum = 0.f;
    for (int rr = 0; rr < R; ++rr) sum += red[rr * d + threadIdx.x];
    mean_s[threadIdx.x] = cnt ? sum / (float)cnt : 0.f;
  }
  __syncthreads();
  const float m = mean_s[c];
  acc = 0.f;
  if (active)
    for (int n = n0 + r; n < n1; n += R) { float t = to_f32<T>(base[(size_t)n * d]) - m; acc += t * t; }
  __syncthreads();
  red[threadIdx.x] = active ? acc : 0.f;
  __syncthreads();
  if (threadIdx.x < d) {
    float m2 = 0.f;
    for (int rr = 0; rr < R; ++rr) m2 += red[rr * d + threadIdx.x];
    float* o = part + ((size_t)p * S + s) * 3 * d;
    o[threadIdx.x] = (float)cnt;
    o[d + threadIdx.x] = mean_s[threadIdx.x];
    o[2 * d + threadIdx.x] = m2;
  }
}

// Chan et al.'s pairwise combination of (count, mean, M2) statistics, in
// double precision: (n, mean, m2) absorbs (nb, mb, m2b); empty parts are skipped.
__device__ __forceinline__ void chan_d(double& n, double& mean, double& m2, double nb, double mb, double m2b) {
  if (nb == 0.0) return;
  const double nt = n + nb, delta = mb - mean;
  mean += delta * nb / nt;
  m2 += m2b + delta * delta * n * nb / nt;
  n = nt;
}

// One wave per (pair, channel): lane l merges slices l, l + 64, ... in order,
// then the 64 lane results are merged by a fixed butterfly (xor 32, 16, ..., 1),
// so the result is the same on every run.  stats[p][c] = (mean, rstd).
__global__ void __launch_bounds__(256) k_stats_final(const float* __restrict__ part, int P, int S, int d, float eps,
                                                     float* __restrict__ stats) {
  const int wv = (blockIdx.x * blockDim.x + threadIdx.x) >> 6, lane = threadIdx.x & 63;
  if (wv >= P * d) return;
  const int p = wv / d, c = wv % d;
  double n = 0.0, mean = 0.0, m2 = 0.0;
  for (int s = lane; s < S; s += 64) {
    const float* o = part + ((size_t)p * S + s) * 3 * d;
    chan_d(n, mean, m2, o[c], o[d + c], o[2 * d + c]);
  }
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) {
    const double nb = __shfl_xor(n, off), mb = __shfl_xor(mean, off), m2b = __shfl_xor(m2, off);
    chan_d(n, mean, m2, nb, mb, m2b);
  }
  if (lane == 0) {
    const double var = n > 0.0 ? m2 / n : 0.0;
    stats[(size_t)wv * 2] = (float)mean;
    stats[(size_t)wv * 2 + 1] = (float)(1.0 / sqrt(var + (double)eps));
  }
}

}  // namespace

void launch_stats_partial(const Problem& pb, int S, float* part, hipStream_t st) {
  const int P = pb.B * pb.H;
  dim3 grid(S, P);
  if (pb.d % 8 == 0 && pb.d <= 128) {
    if (pb.bf16)
      hipLaunchKernelGGL(k_stats_partial_v8<bf16>, grid, dim3(kThreads), 0, st, (const bf16*)pb.k, pb.N, pb.d, S, part, pb.H, pb.Hs, pb.h0);
    else
      hipLaunchKernelGGL(k_stats_partial_v8<float>, grid, dim3(kThreads), 0, st, (const float*)pb.k, pb.N, pb.d, S, part, pb.H, pb.Hs, pb.h0);
  } else {
    if (pb.bf16)
      hipLaunchKernelGGL(k_stats_partial_scalar<bf16>, grid, dim3(kThreads), 0, st, (const bf16*)pb.k, pb.N, pb.d, S, part, pb.H, pb.Hs, pb.h0);
    else
      hipLaunchKernelGGL(k_stats_partial_scalar<float>, grid, dim3(kThreads), 0, st, (const float*)pb.k, pb.N, pb.d, S, part, pb.H, pb.Hs, pb.h0);
  }
}

void launch_stats_final(const Problem& pb, int S, const float* part, float eps, float* stats, hipStream_t st) {
  const int P = pb.B * pb.H;
  const int n = P * pb.d;
  hipLaunchKernelGGL(k_stats_final, dim3((n + 3) / 4), dim3(256), 0, st, part, P, S, pb.d, eps, stats);
}

}  // namespace ttt
