// Muon update rule of the large-chunk TTT layer (LaCT analysis page, section
// "Nonlinear memory complements local attention": the matrix gradient is
// turned into an orthogonalised matrix by Newton-Schulz iterations before the
// update, and L2 normalisation follows).  The iteration is the quintic one of
// the published Muon optimiser:
//     X = M / (||M||_F + 1e-7),   ns_steps times:  A = X X^T,
//     X <- a X + (b A + c A A) X,  (a, b, c) = (3.4445, -4.7750, 2.0315)
// on the wide orientation of M (rows <= cols; a tall matrix is transposed and
// back), then W -= scale * X.  Every product is a small dense GEMM per (pair,
// matrix) -- m x m x n and m x m x m with m = min(in, out) <= 128 -- run in
// fp32 (the chunk recurrence amplifies rounding, see k_mfma_lact.hip) by one
// batched LDS-tiled kernel: 32 x 32 output tiles, so one launch covers every
// (pair, matrix) at once.
#include "ttt_internal.h"

namespace ttt {

namespace {

constexpr float kNsA = 3.4445f, kNsB = -4.7750f, kNsC = 2.0315f;
constexpr int kT = 32;            // output tile and k-step of the batched GEMM

__device__ __forceinline__ void mat_shape(const Problem& pb, int i, int& rows, int& cols) {
  if (pb.inner == INNER_LINEAR) { rows = pb.d; cols = pb.d; return; }
  if (i == 1) { rows = pb.hid; cols = pb.d; }   // W2 [h, d]
  else { rows = pb.d; cols = pb.hid; }          // W1, W3 [d, h]
}

__device__ __forceinline__ float block_sum(float v, float* red) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v += __shfl_xor(v, o);
  const int w = threadIdx.x >> 6, nw = blockDim.x >> 6;
  if ((threadIdx.x & 63) == 0) red[w] = v;
  __syncthreads();
  float t = 0.f;
  for (int i = 0; i < nw; ++i) t += red[i];
  return t;
}

// X0 = M / (||M||_F + 1e-7) in the wide orientation.  grid = (nm, P)
__global__ void __launch_bounds__(256) k_ns_init(Problem pb, const float* __restrict__ mom, unsigned mask,
                                                 float* __restrict__ x) {
  const int i = blockIdx.x, p = blockIdx.y;
  if (!((mask >> i) & 1u)) return;
  int rows, cols;
  mat_shape(pb, i, rows, cols);
  const long long msz = pb.msz;
  const float* m = mom + ((long long)p * pb.nm + i) * msz;
  float* xo = x + ((long long)p * pb.nm + i) * msz;
  __shared__ float red[4];
  float ss = 0.f;
  for (long long e = threadIdx.x; e < msz; e += blockDim.x) ss += m[e] * m[e];
  const float inv = 1.0f / (sqrtf(block_sum(ss, red)) + 1e-7f);
  const bool tall = rows > cols;
  for (long long e = threadIdx.x; e < msz; e += blockDim.x) {
    const int r = (int)(e / cols), c = (int)(e % cols);
    xo[tall ? (long long)c * rows + r : e] = m[e] * inv;
  }
}

// C = alpha * A op(B) + beta * D for every (pair, matrix) in the mask:
// A [M][K], op(B) = B [K][Nc] or (transB) B^T with B [Nc][K], C, D [M][Nc];
// all row-major, contiguous, batch entry z = p * nm + i at z * stride.
// grid = (ceil(Nc / 32), ceil(M / 32), nm * P), 256 threads, 2 x 2 outputs each.
__global__ void __launch_bounds__(256) k_bgemm(int nm, unsigned mask, int M, int Nc, int K, float alpha,
                                               const float* __restrict__ A, long long sA,
                                               const float* __restrict__ B, long long sB, int transB, float beta,
                                               const float* __restrict__ D, long long sD, float* __restrict__ C,
                                               long long sC) {
  const int z = blockIdx.z, i = z % nm;
  if (!((mask >> i) & 1u)) return;
  const int r0 = blockIdx.y * kT, c0 = blockIdx.x * kT;
  A += z * sA; B += z * sB; C += z * sC;
  if (D) D += z * sD;
  __shared__ float As[kT][kT + 1];
  __shared__ float Bs[kT][kT + 1];   // Bs[k][j]
  const int tx = threadIdx.x % 16, ty = threadIdx.x / 16;
  float acc[2][2] = {{0.f, 0.f}, {0.f, 0.f}};
  for (int k0 = 0; k0 < K; k0 += kT) {
    for (int t = threadIdx.x; t < kT * kT; t += 256) {
      const int rr = t / kT, cc = t % kT;
      // A tile: row r0 + rr, column k0 + cc (coalesced along k)
      As[rr][cc] = (r0 + rr < M && k0 + cc < K) ? A[(long long)(r0 + rr) * K + k0 + cc] : 0.f;
      if (transB)   // B [Nc][K]: row c0 + rr, column k0 + cc -> Bs[k][j]
        Bs[cc][rr] = (c0 + rr < Nc && k0 + cc < K) ? B[(long long)(c0 + rr) * K + k0 + cc] : 0.f;
      else          // B [K][Nc]: row k0 + rr, column c0 + cc
        Bs[rr][cc] = (k0 + rr < K && c0 + cc < Nc) ? B[(long long)(k0 + rr) * Nc + c0 + cc] : 0.f;
    }
    __syncthreads();
#pragma unroll 8
    for (int kk = 0; kk < kT; ++kk) {
      const float a0 = As[2 * ty][kk], a1 = As[2 * ty + 1][kk];
      const float b0 = Bs[kk][2 * tx], b1 = Bs[kk][2 * tx + 1];
      acc[0][0] = fmaf(a0, b0, acc[0][0]);
      acc[0][1] = fmaf(a0, b1, acc[0][1]);
      acc[1][0] = fmaf(a1, b0, acc[1][0]);
      acc[1][1] = fmaf(a1, b1, acc[1][1]);
    }
    __syncthreads();
  }
#pragma unroll
  for (int u = 0; u < 2; ++u)
#pragma unroll
    for (int v = 0; v < 2; ++v) {
      const int r = r0 + 2 * ty + u, c = c0 + 2 * tx + v;
      if (r < M && c < Nc) {
        const long long e = (long long)r * Nc + c;
        C[e] = alpha * acc[u][v] + (D ? beta * D[e] : 0.f);
      }
    }
}

// next -= scale * X (back in the [in, out] orientation), W_out if requested.
// grid = (nm, P)
__global__ void __launch_bounds__(256) k_muon_apply(Problem pb, const float* __restrict__ x, unsigned mask,
                                                    float scale, float* __restrict__ next, float* o0, float* o1,
                                                    float* o2) {
  const int i = blockIdx.x, p = blockIdx.y;
  int rows, cols;
  mat_shape(pb, i, rows, cols);
  const long long msz = pb.msz;
  float* w = next + ((long long)p * pb.nm + i) * msz;
  float* out = i == 0 ? o0 : i == 1 ? o1 : o2;
  if (out) out += pb.row(p) * msz;
  const bool upd = (mask >> i) & 1u;
  const float* xi = x + ((long long)p * pb.nm + i) * msz;
  const bool tall = rows > cols;
  for (long long e = threadIdx.x; e < msz; e += blockDim.x) {
    float v = w[e];
    if (upd) {
      const int r = (int)(e / cols), c = (int)(e % cols);
      v -= scale * xi[tall ? (long long)c * rows + r : e];
      w[e] = v;
    }
    if (out) out[e] = v;
  }
}

}  // namespace

size_t muon_scratch_floats(const Problem& pb) {
  const long long m = pb.inner == INNER_LINEAR ? pb.d : (pb.d < pb.hid ? pb.d : pb.hid);
  return (size_t)pb.B * pb.H * pb.nm * (2 * pb.msz + 2 * m * m);
}

void launch_muon(const Problem& pb, const float* mom, float* next, float* const* out, unsigned mask, float scale,
                 int ns_steps, float* scratch, hipStream_t st) {
  const int P = pb.B * pb.H, nm = pb.nm;
  const int m = pb.inner == INNER_LINEAR ? pb.d : (pb.d < pb.hid ? pb.d : pb.hid);
  const int n = (int)(pb.msz / m);
  const long long sx = pb.msz, sg = (long long)m * m;
  float* xa = scratch;
  float* xb = xa + (size_t)P * nm * sx;
  float* ga = xb + (size_t)P * nm * sx;
  float* gb = ga + (size_t)P * nm * sg;
  hipLaunchKernelGGL(k_ns_init, dim3(nm, P), dim3(256), 0, st, pb, mom, mask, xa);
  const unsigned zb = (unsigned)(nm * P);
  const dim3 gmm((m + kT - 1) / kT, (m + kT - 1) / kT, zb), gmn((n + kT - 1) / kT, (m + kT - 1) / kT, zb);
  for (int s = 0; s < ns_steps; ++s) {
    // A = X X^T
    hipLaunchKernelGGL(k_bgemm, gmm, dim3(256), 0, st, nm, mask, m, m, n, 1.0f, xa, sx, xa, sx, 1, 0.0f,
                       (const float*)nullptr, 0LL, ga, sg);
    // Bm = c A A + b A
    hipLaunchKernelGGL(k_bgemm, gmm, dim3(256), 0, st, nm, mask, m, m, m, kNsC, ga, sg, ga, sg, 0, kNsB,
                       (const float*)ga, sg, gb, sg);
    // X' = Bm X + a X
    hipLaunchKernelGGL(k_bgemm, gmn, dim3(256), 0, st, nm, mask, m, n, m, 1.0f, gb, sg, xa, sx, 0, kNsA,
                       (const float*)xa, sx, xb, sx);
    float* t = xa; xa = xb; xb = t;
  }
  hipLaunchKernelGGL(k_muon_apply, dim3(nm, P), dim3(256), 0, st, pb, xa, mask, scale, next, out[0], out[1], out[2]);
}

}  // namespace ttt
