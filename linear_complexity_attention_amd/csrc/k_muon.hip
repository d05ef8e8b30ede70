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

// sum of squares of slice s (kNormSlice elements) of every (pair, matrix):
// part[(p nm + i) nsl + s].  grid = (nsl, nm, P)
constexpr int kNormSlice = 4096;
__global__ void __launch_bounds__(256) k_ns_norm(Problem pb, const float* __restrict__ mom, unsigned mask, int nsl,
                                                 float* __restrict__ part) {
  const int s = blockIdx.x, i = blockIdx.y, p = blockIdx.z;
  if (!((mask >> i) & 1u)) return;
  const long long msz = pb.msz;
  const float* m = mom + ((long long)p * pb.nm + i) * msz;
  __shared__ float red[4];
  float ss = 0.f;
  const long long e1 = min(msz, (long long)(s + 1) * kNormSlice);
  for (long long e = (long long)s * kNormSlice + threadIdx.x; e < e1; e += blockDim.x) ss += m[e] * m[e];
  const float t = block_sum(ss, red);
  if (threadIdx.x == 0) part[((long long)p * pb.nm + i) * nsl + s] = t;
}

__device__ __forceinline__ float inv_norm(const float* part, int nsl) {
  float t = 0.f;
  for (int k = 0; k < nsl; ++k) t += part[k];
  return 1.0f / (sqrtf(t) + 1e-7f);
}

// X0 = M / (||M||_F + 1e-7) in the wide orientation, through 32 x 32 LDS
// tiles so that both the read of M and the (transposed) write of X are
// row-wise.  grid = (tiles of M, nm, P)
__global__ void __launch_bounds__(256) k_ns_init(Problem pb, const float* __restrict__ mom, unsigned mask,
                                                 const float* __restrict__ npart, int nsl, float* __restrict__ x) {
  const int i = blockIdx.y, p = blockIdx.z;
  if (!((mask >> i) & 1u)) return;
  int rows, cols;
  mat_shape(pb, i, rows, cols);
  const int tcols = (cols + 31) / 32;
  const int tr = blockIdx.x / tcols, tc = blockIdx.x % tcols;
  if (tr * 32 >= rows) return;
  const long long msz = pb.msz;
  const float* m = mom + ((long long)p * pb.nm + i) * msz;
  float* xo = x + ((long long)p * pb.nm + i) * msz;
  const float inv = inv_norm(npart + ((long long)p * pb.nm + i) * nsl, nsl);
  __shared__ float tile[32][33];
  const int lx = threadIdx.x % 32, ly = threadIdx.x / 32;      // 32 x 8
  for (int yy = ly; yy < 32; yy += 8) {
    const int r = tr * 32 + yy, c = tc * 32 + lx;
    tile[yy][lx] = (r < rows && c < cols) ? m[(long long)r * cols + c] * inv : 0.f;
  }
  __syncthreads();
  if (rows > cols) {            // tall: X[c][r] = M[r][c], written along r
    for (int yy = ly; yy < 32; yy += 8) {
      const int c = tc * 32 + yy, r = tr * 32 + lx;
      if (c < cols && r < rows) xo[(long long)c * rows + r] = tile[lx][yy];
    }
  } else {
    for (int yy = ly; yy < 32; yy += 8) {
      const int r = tr * 32 + yy, c = tc * 32 + lx;
      if (r < rows && c < cols) xo[(long long)r * cols + c] = tile[yy][lx];
    }
  }
}

// C = alpha * A op(B) + beta * D for every (pair, matrix) in the mask:
// A [M][K], op(B) = B [K][Nc] or (transB) B^T with B [Nc][K], C, D [M][Nc];
// all row-major, contiguous, batch entry z = p * nm + i at z * stride.
// 32 x 32 output tiles (so a launch has P * nm * (M/32) * (Nc/32) workgroups)
// and up to 256 of K staged in LDS at once (A and B^T as [row][k], B as
// [k][col], 70 KB), each operand in its stored orientation so that the LDS
// stores are 16 bytes; the workgroup pays one global round trip per 256 of K
// instead of one per k-step.  Wave w computes the 16 x 16 block (16 (w / 2), 16 (w % 2)) on
// v_mfma_f32_16x16x4f32 (fp32 operands and sums): lane l supplies
// A[16 (w / 2) + l % 16][4 s + l / 16] and B[4 s + l / 16][16 (w % 2) + l % 16]
// and holds the result rows 4 (l / 16) + e, column l % 16.
// grid = (ceil(Nc / 32), ceil(M / 32), nm * P), 256 threads.
constexpr int kBT = 32, kBK = 256, kBP = kBT + 4;
__global__ void __launch_bounds__(256) k_bgemm(int nm, unsigned mask, int M, int Nc, int K, float alpha,
                                               const float* __restrict__ A, long long sA,
                                               const float* __restrict__ B, long long sB, int transB, float beta,
                                               const float* __restrict__ D, long long sD, float* __restrict__ C,
                                               long long sC) {
  const int z = blockIdx.z, i = z % nm;
  if (!((mask >> i) & 1u)) return;
  const int r0 = blockIdx.y * kBT, c0 = blockIdx.x * kBT;
  A += z * sA; B += z * sB; C += z * sC;
  if (D) D += z * sD;
  // [row][k] rows of kBK + 4 floats: the fragment reads (16 rows x 4 k per
  // wave) fall on 64 distinct banks
  constexpr int LA = kBK + 4, NB = kBK * kBP > kBT * LA ? kBK * kBP : kBT * LA;
  __shared__ __attribute__((aligned(16))) float smem[kBT * LA + NB];
  float(*As)[LA] = reinterpret_cast<float(*)[LA]>(smem);                 // A [row][k]
  float(*Bt)[LA] = reinterpret_cast<float(*)[LA]>(smem + kBT * LA);      // B^T [col][k] (transB)
  float(*Bs)[kBP] = reinterpret_cast<float(*)[kBP]>(smem + kBT * LA);    // B [k][col]
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int wi = w >> 1, wj = w & 1;
  f32x4 acc[2] = {{0.f, 0.f, 0.f, 0.f}, {0.f, 0.f, 0.f, 0.f}};
  // float4 loads need 16-byte aligned rows and batch entries
  const bool vec = K % 4 == 0 && Nc % 4 == 0 && sA % 4 == 0 && sB % 4 == 0;
  for (int k0 = 0; k0 < K; k0 += kBK) {
    const int kc = min(kBK, K - k0);
    if (vec && kc % 4 == 0) {
      // float4 loads, all of a thread's loads in flight before the LDS stores:
      // A (and B^T) rows along k into [row][k], B [K][Nc] rows into [k][col]
      constexpr int NV = kBT * kBK / 4 / 256;      // float4 per thread and operand (8)
      const int k4 = kc / 4;
      // out-of-range elements are read at the batch entry's first element and
      // masked after the load, so that no load waits under a branch of its own
      float4 av[NV], bv[NV];
      bool aok[NV], bok[NV];
#pragma unroll
      for (int u = 0; u < NV; ++u) {
        const int f = threadIdx.x + 256 * u;
        const bool fin = f < kBT * k4;
        const int rr = fin ? f / k4 : 0, kk = fin ? 4 * (f % k4) : 0;
        aok[u] = fin && r0 + rr < M;
        av[u] = *reinterpret_cast<const float4*>(A + (aok[u] ? (long long)(r0 + rr) * K + k0 + kk : 0LL));
        long long bo;
        if (transB) {
          bok[u] = fin && c0 + rr < Nc;
          bo = (long long)(c0 + rr) * K + k0 + kk;
        } else {
          const int kr = f / (kBT / 4), cc = 4 * (f % (kBT / 4));
          bok[u] = fin && c0 + cc < Nc;
          bo = (long long)(k0 + kr) * Nc + c0 + cc;
        }
        bv[u] = *reinterpret_cast<const float4*>(B + (bok[u] ? bo : 0LL));
      }
#pragma unroll
      for (int u = 0; u < NV; ++u) {
        if (!aok[u]) av[u] = float4{0.f, 0.f, 0.f, 0.f};
        if (!bok[u]) bv[u] = float4{0.f, 0.f, 0.f, 0.f};
      }
#pragma unroll
      for (int u = 0; u < NV; ++u) {
        const int f = threadIdx.x + 256 * u;
        if (f < kBT * k4) {
          const int rr = f / k4, kk = 4 * (f % k4);
          *reinterpret_cast<float4*>(&As[rr][kk]) = av[u];
          if (transB) {
            *reinterpret_cast<float4*>(&Bt[rr][kk]) = bv[u];
          } else {
            const int kr = f / (kBT / 4), cc = 4 * (f % (kBT / 4));
            *reinterpret_cast<float4*>(&Bs[kr][cc]) = bv[u];
          }
        }
      }
    } else {
      for (int t = threadIdx.x; t < kBT * kc; t += 256) {
        const int rr = t / kc, kk = t % kc;
        As[rr][kk] = (r0 + rr < M) ? A[(long long)(r0 + rr) * K + k0 + kk] : 0.f;
        if (transB) Bt[rr][kk] = (c0 + rr < Nc) ? B[(long long)(c0 + rr) * K + k0 + kk] : 0.f;
      }
      if (!transB)
        for (int t = threadIdx.x; t < kBT * kc; t += 256) {
          const int kr = t / kBT, cc = t % kBT;
          Bs[kr][cc] = (c0 + cc < Nc) ? B[(long long)(k0 + kr) * Nc + c0 + cc] : 0.f;
        }
    }
    // k rows up to the next multiple of 4 are zero (the MFMA takes 4 of k)
    const int kc4 = (kc + 3) & ~3;
    for (int t = threadIdx.x; t < (kc4 - kc) * kBT; t += 256) {
      const int kk = kc + t / kBT, x = t % kBT;
      As[x][kk] = 0.f;
      if (transB) Bt[x][kk] = 0.f;
      else Bs[kk][x] = 0.f;
    }
    __syncthreads();
    // eight k-steps' fragments are read before their MFMAs, which alternate
    // between two accumulators
    const int kq = lane >> 4, ca = 16 * wi + (lane & 15), cb = 16 * wj + (lane & 15);
    auto bfrag = [&](int k) { return transB ? Bt[cb][k] : Bs[k][cb]; };
    int s4 = 0;
    for (; s4 + 32 <= kc4; s4 += 32) {
      float a[8], b[8];
#pragma unroll
      for (int u = 0; u < 8; ++u) { a[u] = As[ca][s4 + 4 * u + kq]; b[u] = bfrag(s4 + 4 * u + kq); }
#pragma unroll
      for (int u = 0; u < 8; ++u) acc[u & 1] = __builtin_amdgcn_mfma_f32_16x16x4f32(a[u], b[u], acc[u & 1], 0, 0, 0);
    }
    for (; s4 < kc4; s4 += 4)
      acc[0] = __builtin_amdgcn_mfma_f32_16x16x4f32(As[ca][s4 + kq], bfrag(s4 + kq), acc[0], 0, 0, 0);
    __syncthreads();
  }
  // D's four values are loaded together (at the entry's first element when
  // out of range) before the stores
  float dv[4] = {0.f, 0.f, 0.f, 0.f};
  const int c = c0 + 16 * wj + (lane & 15);
  if (D) {
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int r = r0 + 16 * wi + 4 * (lane >> 4) + e;
      dv[e] = D[r < M && c < Nc ? (long long)r * Nc + c : 0LL];
    }
#pragma unroll
    for (int e = 0; e < 4; ++e) dv[e] *= beta;
  }
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    const int r = r0 + 16 * wi + 4 * (lane >> 4) + e;
    if (r < M && c < Nc) C[(long long)r * Nc + c] = alpha * (acc[0][e] + acc[1][e]) + dv[e];
  }
}

// next -= scale * X (back in the [in, out] orientation), W_out if requested;
// 32 x 32 LDS tiles as in k_ns_init.  grid = (tiles of W, nm, P)
__global__ void __launch_bounds__(256) k_muon_apply(Problem pb, const float* __restrict__ x, unsigned mask,
                                                    float scale, float* __restrict__ next, float* o0, float* o1,
                                                    float* o2) {
  const int i = blockIdx.y, p = blockIdx.z;
  int rows, cols;
  mat_shape(pb, i, rows, cols);
  const int tcols = (cols + 31) / 32;
  const int tr = blockIdx.x / tcols, tc = blockIdx.x % tcols;
  if (tr * 32 >= rows) return;
  const long long msz = pb.msz;
  float* w = next + ((long long)p * pb.nm + i) * msz;
  float* out = i == 0 ? o0 : i == 1 ? o1 : o2;
  if (out) out += pb.row(p) * msz;
  const bool upd = (mask >> i) & 1u;
  const float* xi = x + ((long long)p * pb.nm + i) * msz;
  __shared__ float tile[32][33];   // the X values of this tile of W, [row][col] of W
  const int lx = threadIdx.x % 32, ly = threadIdx.x / 32;
  if (upd) {
    if (rows > cols) {            // X [cols][rows]: read along r
      for (int yy = ly; yy < 32; yy += 8) {
        const int c = tc * 32 + yy, r = tr * 32 + lx;
        tile[lx][yy] = (c < cols && r < rows) ? xi[(long long)c * rows + r] : 0.f;
      }
    } else {
      for (int yy = ly; yy < 32; yy += 8) {
        const int r = tr * 32 + yy, c = tc * 32 + lx;
        tile[yy][lx] = (r < rows && c < cols) ? xi[(long long)r * cols + c] : 0.f;
      }
    }
  }
  __syncthreads();
  for (int yy = ly; yy < 32; yy += 8) {
    const int r = tr * 32 + yy, c = tc * 32 + lx;
    if (r < rows && c < cols) {
      const long long e = (long long)r * cols + c;
      float v = w[e];
      if (upd) {
        v -= scale * tile[yy][lx];
        w[e] = v;
      }
      if (out) out[e] = v;
    }
  }
}

}  // namespace

static int norm_slices(const Problem& pb) { return (int)((pb.msz + kNormSlice - 1) / kNormSlice); }

size_t muon_scratch_floats(const Problem& pb) {
  const long long m = pb.inner == INNER_LINEAR ? pb.d : (pb.d < pb.hid ? pb.d : pb.hid);
  return (size_t)pb.B * pb.H * pb.nm * (2 * pb.msz + 2 * m * m + norm_slices(pb));
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
  float* npart = gb + (size_t)P * nm * sg;
  const int nsl = norm_slices(pb);
  // tiles of the largest [in, out] matrix of the model (every matrix is d x h or h x d)
  const int side_r = pb.inner == INNER_LINEAR ? pb.d : (pb.d > pb.hid ? pb.d : pb.hid);
  const unsigned wtiles = (unsigned)(((side_r + 31) / 32) * ((side_r + 31) / 32));
  hipLaunchKernelGGL(k_ns_norm, dim3(nsl, nm, P), dim3(256), 0, st, pb, mom, mask, nsl, npart);
  hipLaunchKernelGGL(k_ns_init, dim3(wtiles, nm, P), dim3(256), 0, st, pb, mom, mask, (const float*)npart, nsl, xa);
  const unsigned zb = (unsigned)(nm * P);
  const dim3 gmm((m + kBT - 1) / kBT, (m + kBT - 1) / kBT, zb), gmn((n + kBT - 1) / kBT, (m + kBT - 1) / kBT, zb);
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
  hipLaunchKernelGGL(k_muon_apply, dim3(wtiles, nm, P), dim3(256), 0, st, pb, xa, mask, scale, next, out[0], out[1],
                     out[2]);
}

}  // namespace ttt
