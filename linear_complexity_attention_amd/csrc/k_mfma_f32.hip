// GELU-MLP products on the fp32 matrix cores (d and h multiples of 16):
// batched products over whole pairs plus elementwise passes, every product on
// v_mfma_f32_16x16x4f32 (exact fp32 products, fp32 sums), for the two fp32
// paths of the layer:
//  - one inner step on a token range at the fp32 weights (ViT3 summary page,
//    section 02, steps (i)-(ii)), for the multi-step requests (epochs, chunks,
//    section 03 guideline 2) that cannot use the bf16 fused kernel: its
//    token-sliced partials feed the ordinary update kernels;
//  - the outer-loop backward, the same gradient of a gradient as the token-tile
//    kernels of k_backward.hip (section 02: the inner update is differentiable
//    and trained end to end; section 03 guideline 1: the value projection
//    learns through the loss's mixed second derivative).
//
// Per pair, with X = K_hat, Z = X W1, A = gelu(Z), F = A W2 and the loss
// gradient G (MSE: 2/(N d) eta (F - V); dot: -eta V):
//   step         dW2 = A^T G, dA = G W2^T, dZ = gelu'(Z) dA, dW1 = X^T dZ,
//                W* = W0 - dW
//   readout      Zq = Q W1*, Aq = gelu(Zq), U2 = Aq^T dO, dZq = gelu'(Zq) (dO W2*^T),
//                U1 = Q^T dZq, dQ = dZq W1*^T
//   through the step, phi = sum_n <G_n, F_dot_n> along U:
//                Z_dot = X U1, A_dot = gelu'(Z) Z_dot, F_dot = A_dot W2 + A U2,
//                F_bar = 2/(N d) eta F_dot (MSE; 0 for the dot loss),
//                A_dot_bar = G W2^T (= dA), A_bar = G U2^T + F_bar W2^T,
//                Z_dot_bar = gelu'(Z) A_dot_bar (= dZ),
//                Z_bar = gelu''(Z) Z_dot A_dot_bar + gelu'(Z) A_bar,
//                dphi/dX = Z_dot_bar U1^T + Z_bar W1^T,
//                dphi/dW1 = X^T Z_bar, dphi/dW2 = A_dot^T G + A^T F_bar,
//                dV = -dphi/dV, deta = -dphi/deta (per token)
//   outputs      dW0 = U - dphi/dW0, dK_hat = -dphi/dX (then the key-norm backward)
//
// The products of a pair are small ([N x d] x [d x h] and their transposes),
// so one kernel takes all pairs at once (grid z = pair) in 64 x 64 output
// tiles; the reductions over the tokens split K and add the slices in order.
#include <algorithm>
#include <cstdio>
#include <cstdlib>

#include "ttt_internal.h"

namespace ttt {

namespace {

constexpr int kT = 256;                 // threads per workgroup
constexpr int BM = 64, BN = 64, BK = 16;
constexpr int LS = 80;                  // LDS row stride (floats): 16 mod 64, conflict-free fragment reads

__device__ __forceinline__ f32x4 mfma_f32(float a, float b, const f32x4& c) {
  return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ float gelu_second_f(float z) {
  return 0.39894228040143268f * __expf(-0.5f * z * z) * (2.0f - z * z);
}

// C[p] (+)= alpha A[p] B[p] for every pair p = blockIdx.z / KS, K slice blockIdx.z % KS.
// Operand element (r, c) of pair p sits at ptr + (p / H) sb + (p % H) sh + r ld + c;
// TA: A is stored [K][M]; TB: B is stored [N][K].  The stored rows of every
// operand are 16-byte aligned and their contiguous extent is a multiple of 4
// (d or h): the token axis is always a row index.  With KS > 1, slice s writes
// C + s cstride (plain store) for the in-order sum afterwards.
struct Op {
  const float* p;
  long long sb, sh;
  int ld;
};
struct OutOp {
  float* p;
  long long sb, sh, cstride;
  int ld;
};
// Elementwise epilogues on the product v (= alpha A B, plus C when
// accumulating); z, zd, da and out2 share C's layout:
//   EPI_STORE  C = v
//   EPI_GELU   C = v, out2 = gelu(v)
//   EPI_GP     C = v, out2 = v gelu'(z)   (out2 == C: only the product is kept)
//   EPI_ZBAR   C = gelu''(z) zd da + gelu'(z) v
enum { EPI_STORE = 0, EPI_GELU = 1, EPI_GP = 2, EPI_ZBAR = 3 };
struct Epi {
  const float *z, *zd, *da;
  float* out2;
};

// LDS tile element (k, x) of a [BK][64] tile: rows of 80 floats, the column
// XOR-ed with 16 (k / 4), so that the transposing scalar stores (four k rows
// per thread) and the fragment reads (four k rows x 16 columns per wave) both
// fall on 64 distinct banks; four consecutive columns stay consecutive.
__device__ __forceinline__ int sw(int k, int x) { return k * LS + (x ^ ((k >> 2) << 4)); }

constexpr int CS = BM + 4;   // row stride (floats) of the output tile staged in LDS

template <bool TA, bool TB, int EPI>
__global__ void __launch_bounds__(kT) k_gemm_f32(int H, int M, int N, int K, int KS, Op A, Op B, OutOp C,
                                                 float alpha, int accumulate, Epi ep) {
  // operand tiles; after the main loop the output tile [BM][CS] reuses them
  __shared__ __attribute__((aligned(16))) float smem[4 * BK * LS];
  static_assert(BM * CS <= 4 * BK * LS, "output tile exceeds the operand tiles");
  float(*As)[BK * LS] = reinterpret_cast<float(*)[BK * LS]>(smem);                // [k][m]
  float(*Bs)[BK * LS] = reinterpret_cast<float(*)[BK * LS]>(smem + 2 * BK * LS);  // [k][n]
  const int p = blockIdx.z / KS, ks = blockIdx.z % KS;
  const long long pa = (long long)(p / H), ph = (long long)(p % H);
  const float* a = A.p + pa * A.sb + ph * A.sh;
  const float* b = B.p + pa * B.sb + ph * B.sh;
  float* c = C.p + pa * C.sb + ph * C.sh + (long long)ks * C.cstride;
  const int m0 = blockIdx.y * BM, n0 = blockIdx.x * BN;
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int wm = w >> 1, wn = w & 1;
  // this slice's k range, in whole BK tiles
  const int nkt = (K + BK - 1) / BK;
  const int kt0 = (int)((long long)ks * nkt / KS), kt1 = (int)((long long)(ks + 1) * nkt / KS);
  float4 ra, rb;
  // An out-of-range element is read at the operand's first element and masked
  // after the load.  Written as a conditional load, it was compiled into a
  // select between the global address and a private one holding the zero, as
  // four flat loads, which the LDS waits of the MFMA loop count as well: the
  // next tile's loads then stalled every fragment read.
  auto ld4 = [](const float* base, long long off, bool ok) {
    const float4 v = *reinterpret_cast<const float4*>(base + (ok ? off : 0));
    return ok ? v : make_float4(0.f, 0.f, 0.f, 0.f);
  };
  auto load = [&](int k0) {
    if (!TA) {   // A[m][k]: thread -> row m, four k
      const int m = m0 + (tid >> 2), k = k0 + 4 * (tid & 3);
      ra = ld4(a, (long long)m * A.ld + k, m < M && k < K);
    } else {     // stored [k][m]: thread -> row k, four m
      const int k = k0 + (tid >> 4), m = m0 + 4 * (tid & 15);
      ra = ld4(a, (long long)k * A.ld + m, k < K && m < M);
    }
    if (!TB) {   // B[k][n]: thread -> row k, four n
      const int k = k0 + (tid >> 4), n = n0 + 4 * (tid & 15);
      rb = ld4(b, (long long)k * B.ld + n, k < K && n < N);
    } else {     // stored [n][k]: thread -> row n, four k
      const int n = n0 + (tid >> 2), k = k0 + 4 * (tid & 3);
      rb = ld4(b, (long long)n * B.ld + k, n < N && k < K);
    }
  };
  auto store = [&](int buf) {
    if (!TA) {
      const int m = tid >> 2, k = 4 * (tid & 3);
      As[buf][sw(k + 0, m)] = ra.x;
      As[buf][sw(k + 1, m)] = ra.y;
      As[buf][sw(k + 2, m)] = ra.z;
      As[buf][sw(k + 3, m)] = ra.w;
    } else {
      *reinterpret_cast<float4*>(&As[buf][sw(tid >> 4, 4 * (tid & 15))]) = ra;
    }
    if (!TB) {
      *reinterpret_cast<float4*>(&Bs[buf][sw(tid >> 4, 4 * (tid & 15))]) = rb;
    } else {
      const int n = tid >> 2, k = 4 * (tid & 3);
      Bs[buf][sw(k + 0, n)] = rb.x;
      Bs[buf][sw(k + 1, n)] = rb.y;
      Bs[buf][sw(k + 2, n)] = rb.z;
      Bs[buf][sw(k + 3, n)] = rb.w;
    }
  };
  // wave (wm, wn) owns the 32 x 32 block at (32 wm, 32 wn): 2 x 2 MFMA tiles.
  // Fragments: lane l holds A[16 i + l % 16][4 s + l / 16] and
  // B[4 s + l / 16][16 j + l % 16]; the result rows 4 (l / 16) + e, column l % 16.
  f32x4 acc[2][2];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};
  const int kk = lane >> 4, col = lane & 15;
  if (kt0 < kt1) {
    load(kt0 * BK);
    store(0);
    __syncthreads();
    for (int kt = kt0; kt < kt1; ++kt) {
      const int buf = (kt - kt0) & 1;
      if (kt + 1 < kt1) load((kt + 1) * BK);
#pragma unroll
      for (int s = 0; s < BK / 4; ++s) {
        float fa[2], fb[2];
#pragma unroll
        for (int i = 0; i < 2; ++i) fa[i] = As[buf][sw(4 * s + kk, 32 * wm + 16 * i + col)];
#pragma unroll
        for (int j = 0; j < 2; ++j) fb[j] = Bs[buf][sw(4 * s + kk, 32 * wn + 16 * j + col)];
#pragma unroll
        for (int i = 0; i < 2; ++i)
#pragma unroll
          for (int j = 0; j < 2; ++j) acc[i][j] = mfma_f32(fa[i], fb[j], acc[i][j]);
      }
      if (kt + 1 < kt1) store(buf ^ 1);
      __syncthreads();
    }
  }
  // Epilogue through LDS: the accumulators go to the [64][CS] output tile,
  // then thread t takes columns 4 (t % 16) .. + 3 of rows t / 16 + 16 k, so
  // that every load and store of C and of the epilogue operands is 16 bytes
  // and a wave covers 4 whole tile rows (stores straight from the MFMA layout
  // write 64-byte pieces of rows).  The inputs of the 4 rows are loaded
  // before any is used, at the tile's first element when out of range.
  // Requires 16-byte aligned rows of C and of the epilogue operands and N a
  // multiple of 4 (checked by the launcher).
  const long long tb = (c - C.p) + (long long)m0 * C.ld + n0;   // the tile's first element
  constexpr int NIN = EPI == EPI_ZBAR ? 3 : (EPI == EPI_GP ? 1 : 0);
  __syncthreads();   // every wave has read its last fragments
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int e = 0; e < 4; ++e)
        smem[(32 * wm + 16 * i + 4 * (lane >> 4) + e) * CS + 32 * wn + 16 * j + (lane & 15)] = acc[i][j][e];
  __syncthreads();
  const int nn = 4 * (tid & 15), rr = tid >> 4;
  const bool colok = n0 + nn < N;
  const float4 z4 = make_float4(0.f, 0.f, 0.f, 0.f);
  float4 pv[4], x0[4], x1[4], x2[4];
  int offv[4];
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    const int mm = rr + 16 * k;
    const bool ok = colok && m0 + mm < M;
    offv[k] = ok ? mm * C.ld + nn : -1;
    const long long q = tb + (ok ? mm * C.ld + nn : 0);
    pv[k] = accumulate ? *reinterpret_cast<const float4*>(C.p + q) : z4;
    if constexpr (NIN >= 1) x0[k] = *reinterpret_cast<const float4*>(ep.z + q);
    if constexpr (NIN >= 3) {
      x1[k] = *reinterpret_cast<const float4*>(ep.zd + q);
      x2[k] = *reinterpret_cast<const float4*>(ep.da + q);
    }
  }
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    if (offv[k] < 0) continue;
    const long long q = tb + offv[k];
    const float4 a4 = *reinterpret_cast<const float4*>(&smem[(rr + 16 * k) * CS + nn]);
    const float av[4] = {a4.x, a4.y, a4.z, a4.w};
    const float pp[4] = {pv[k].x, pv[k].y, pv[k].z, pv[k].w};
    float v[4], o2[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) v[u] = accumulate ? pp[u] + alpha * av[u] : alpha * av[u];
    if constexpr (EPI == EPI_STORE) {
      *reinterpret_cast<float4*>(C.p + q) = make_float4(v[0], v[1], v[2], v[3]);
    } else if constexpr (EPI == EPI_GELU) {
      *reinterpret_cast<float4*>(C.p + q) = make_float4(v[0], v[1], v[2], v[3]);
#pragma unroll
      for (int u = 0; u < 4; ++u) o2[u] = gelu_exact(v[u]);
      *reinterpret_cast<float4*>(ep.out2 + q) = make_float4(o2[0], o2[1], o2[2], o2[3]);
    } else if constexpr (EPI == EPI_GP) {
      const float zz[4] = {x0[k].x, x0[k].y, x0[k].z, x0[k].w};
#pragma unroll
      for (int u = 0; u < 4; ++u) o2[u] = v[u] * gelu_exact_prime(zz[u]);
      if (ep.out2 != C.p) *reinterpret_cast<float4*>(C.p + q) = make_float4(v[0], v[1], v[2], v[3]);
      *reinterpret_cast<float4*>(ep.out2 + q) = make_float4(o2[0], o2[1], o2[2], o2[3]);
    } else {
      const float zz[4] = {x0[k].x, x0[k].y, x0[k].z, x0[k].w};
      const float zd[4] = {x1[k].x, x1[k].y, x1[k].z, x1[k].w};
      const float da[4] = {x2[k].x, x2[k].y, x2[k].z, x2[k].w};
#pragma unroll
      for (int u = 0; u < 4; ++u) o2[u] = gelu_second_f(zz[u]) * zd[u] * da[u] + gelu_exact_prime(zz[u]) * v[u];
      *reinterpret_cast<float4*>(C.p + q) = make_float4(o2[0], o2[1], o2[2], o2[3]);
    }
  }
}

// ---------------------------------------------------------------------------
// elementwise passes over [P][N][x] buffers (pair-major)

// token rows t0 .. t0 + nt of a [B, Hs, N, d] tensor -> fp32 [P][nt][d];
// keys normalised with the statistics when given
template <typename T>
__global__ void __launch_bounds__(kT) k_rows_f32(Problem pb, const T* __restrict__ src, const float* __restrict__ stats,
                                                 int t0, int nt, float* __restrict__ dst) {
  const int p = blockIdx.y, d = pb.d;
  const long long n = (long long)nt * d;
  const T* s = src + pb.row(p) * (long long)pb.N * d + (long long)t0 * d;
  float* o = dst + (long long)p * n;
  for (long long i = blockIdx.x * (long long)kT + threadIdx.x; i < n; i += (long long)gridDim.x * kT) {
    float x = to_f32<T>(s[i]);
    if (stats) {
      const int ch = (int)(i % d);
      x = (x - stats[((size_t)p * d + ch) * 2]) * stats[((size_t)p * d + ch) * 2 + 1];
    }
    o[i] = x;
  }
}

// the loss gradient of tokens t0 .. t0 + nt: G = 2/(nt d) eta (F - V) [MSE],
// -eta V [dot] -> [P][nt][d]
template <typename T>
__global__ void __launch_bounds__(kT) k_loss_grad(Problem pb, int t0, int nt, const float* __restrict__ F,
                                                  float* __restrict__ G) {
  const int p = blockIdx.y, d = pb.d, N = pb.N;
  const long long n = (long long)nt * d, prow = pb.row(p);
  const T* v = (const T*)pb.v + (prow * N + t0) * d;
  const float c2 = 2.0f / ((float)nt * (float)d);
  const bool mse = pb.loss == LOSS_MSE;
  for (long long i = blockIdx.x * (long long)kT + threadIdx.x; i < n; i += (long long)gridDim.x * kT) {
    const int t = t0 + (int)(i / d);
    const float e = pb.eta_scale * (pb.eta_tok ? pb.eta_tok[prow * N + t] : 1.f);
    const float vv = to_f32<T>(v[i]);
    G[(long long)p * n + i] = mse ? e * c2 * (F[(long long)p * n + i] - vv) : -e * vv;
  }
}

// Per token, with the tangent F_dot: F_bar = 2/(N d) eta F_dot (MSE, in place of
// F_dot; the dot loss has none), dV = -dphi/dV and deta = -dphi/deta.  One
// wave per token: lanes over the channels, then a fixed-order row sum.
template <typename T>
__global__ void __launch_bounds__(kT) k_phi_tok(Problem pb, const float* __restrict__ F, float* __restrict__ Fd,
                                                float* __restrict__ dv, float* __restrict__ deta) {
  const int p = blockIdx.y, d = pb.d, N = pb.N;
  const int t = blockIdx.x * (kT / 64) + (threadIdx.x >> 6), lane = threadIdx.x & 63;
  if (t >= N) return;
  const long long prow = pb.row(p), n = (long long)N * d;
  const long long ro = (long long)p * n + (long long)t * d;
  const T* v = (const T*)pb.v + prow * n + (long long)t * d;
  const float c2 = 2.0f / ((float)N * (float)d);
  const float e = pb.eta_scale * (pb.eta_tok ? pb.eta_tok[prow * N + t] : 1.f);
  const bool mse = pb.loss == LOSS_MSE;
  float acc = 0.f;
  for (int ch = lane; ch < d; ch += 64) {
    const float fd = Fd[ro + ch], vv = to_f32<T>(v[ch]);
    if (mse) {
      const float fb = c2 * e * fd;
      acc += c2 * fd * (F[ro + ch] - vv);
      Fd[ro + ch] = fb;
      dv[prow * n + (long long)t * d + ch] = fb;
    } else {
      acc -= fd * vv;
      dv[prow * n + (long long)t * d + ch] = e * fd;
    }
  }
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) acc += __shfl_xor(acc, off);
  if (deta && lane == 0) deta[prow * N + t] = -acc;
}

// W* = W0 - dW per pair ([P][2][d h] state layout; W0 through WRef)
__global__ void __launch_bounds__(kT) k_wstar(Problem pb, WRef w0, const float* __restrict__ dW, float* __restrict__ ws) {
  const int p = blockIdx.y, i = blockIdx.z;
  const long long msz = pb.msz;
  const float* src = w0.mat(i, p / pb.H, p % pb.H);
  const long long o = ((long long)p * 2 + i) * msz;
  for (long long e = blockIdx.x * (long long)kT + threadIdx.x; e < msz; e += (long long)gridDim.x * kT)
    ws[o + e] = src[e] - dW[o + e];
}

// out[e] = base[e] + sign * sum_s part[s][e], the slices added in order
__global__ void __launch_bounds__(kT) k_sum_slices(const float* __restrict__ part, int S, long long n, float sign,
                                                   const float* __restrict__ base, float* __restrict__ out) {
  for (long long i = blockIdx.x * (long long)kT + threadIdx.x; i < n; i += (long long)gridDim.x * kT) {
    float s = 0.f;
    for (int k = 0; k < S; ++k) s += part[k * n + i];
    out[i] = (base ? base[i] : 0.f) + sign * s;
  }
}

unsigned ew_blocks(long long n) { return (unsigned)std::min<long long>((n + kT - 1) / kT, 4096); }

// token slices of the reductions over N: about four workgroups per CU in all
int red_slices(long long tiles, int N) {
  long long s = (4LL * device_cu_count() + tiles - 1) / tiles;
  const long long maxs = (N + 255) / 256;          // at least 256 tokens per slice
  if (s > maxs) s = maxs;
  return (int)(s < 1 ? 1 : s);
}

}  // namespace

bool bwd_mfma_supported(const Problem& pb, const WRef& w0) {
  if (pb.inner != INNER_MLP || pb.d % 16 != 0 || pb.hid % 16 != 0) return false;
  // W0 is read with 16-byte loads
  for (int i = 0; i < 2; ++i)
    if (reinterpret_cast<uintptr_t>(w0.m[i]) % 16 != 0) return false;
  return w0.sb % 4 == 0 && w0.sh % 4 == 0;
}

// floats of the workspace regions, in the order launch_backward_mfma uses them
void bwd_mfma_sizes(const Problem& pb, BwdMfmaSizes* s) {
  const long long P = (long long)pb.B * pb.H;
  s->tok_d = P * pb.N * pb.d;
  s->tok_h = P * pb.N * pb.hid;
  s->wsz = P * 2 * pb.msz;
  const long long tiles_w = (long long)P * ((pb.d + BM - 1) / BM) * ((pb.hid + BN - 1) / BN);
  s->KS = red_slices(tiles_w, pb.N);
}

namespace {

template <bool TA, bool TB, int EPI = EPI_STORE>
void gemm(int P, int H, int M, int N, int K, int KS, const Op& A, const Op& B, const OutOp& C, bool acc,
          hipStream_t st, float alpha = 1.0f, const Epi& ep = Epi{}) {
  const dim3 grid((N + BN - 1) / BN, (M + BM - 1) / BM, P * KS);
  // The epilogue's 16-byte accesses need every row of C (and of the epilogue
  // operands, which share C's layout) 16-byte aligned and N a multiple of 4.
  // Every call meets this: C is workspace (256-byte aligned) or the
  // caller's dq / dk (16-byte aligned, checked at the boundary), and the row
  // lengths and strides are multiples of d or h, which this path requires to
  // be multiples of 16.  A call that broke it would be a bug here, not a
  // caller's error, so it stops the process rather than fault the GPU.
  auto al16 = [](const void* p) { return reinterpret_cast<uintptr_t>(p) % 16 == 0; };
  const bool vec = N % 4 == 0 && C.ld % 4 == 0 && C.sb % 4 == 0 && C.sh % 4 == 0 && C.cstride % 4 == 0 &&
                   al16(C.p) && (!ep.z || al16(ep.z)) && (!ep.zd || al16(ep.zd)) && (!ep.da || al16(ep.da)) &&
                   (!ep.out2 || al16(ep.out2));
  if (!vec) {
    std::fprintf(stderr, "ttt: fp32 product with an unaligned output (internal error)\n");
    std::abort();
  }
  hipLaunchKernelGGL((k_gemm_f32<TA, TB, EPI>), grid, dim3(kT), 0, st, H, M, N, K, KS, A, B, C, alpha, acc ? 1 : 0,
                     ep);
}

// pair-major [P][rows][ld] buffer as an operand
Op pm(const float* p, long long per_pair, int H, int ld) { return Op{p, per_pair * H, per_pair, ld}; }
OutOp pmo(float* p, long long per_pair, int H, int ld, long long cstride = 0) {
  return OutOp{p, per_pair * H, per_pair, cstride, ld};
}

}  // namespace

bool step_mfma_shape(const Problem& pb) { return pb.inner == INNER_MLP && pb.d % 16 == 0 && pb.hid % 16 == 0; }

bool step_mfma_aligned(const WRef& W) {
  for (int i = 0; i < 2; ++i)
    if (reinterpret_cast<uintptr_t>(W.m[i]) % 16 != 0) return false;
  return W.sb % 4 == 0 && W.sh % 4 == 0;
}

int step_mfma_splits(const Problem& pb, int nt) {
  const long long P = (long long)pb.B * pb.H;
  return red_slices(P * ((pb.d + BM - 1) / BM) * ((pb.hid + BN - 1) / BN), nt);
}

// One inner step on tokens [t0, t0 + nt) of every pair at the weights W:
//   X = K_hat rows, Z = X W1 and A = gelu(Z), F = A W2 (MSE), G, dW2 = A^T G,
//   dA = G W2^T and dZ = gelu'(Z) dA, dW1 = X^T dZ
// The weight gradients go to part as KS token slices [KS][P][2][d h] (the
// layout of the token-split partials the update kernels sum); dA is kept only
// when sb.dA is given (else dZ overwrites it in place).
void launch_step_mfma(const Problem& pb, const WRef& W, int t0, int nt, const StepMfmaBufs& sb, float* part, int KS,
                      hipStream_t st) {
  const int P = pb.B * pb.H, H = pb.H, d = pb.d, h = pb.hid;
  const long long nd = (long long)nt * d, nh = (long long)nt * h, msz = pb.msz, wpp = 2 * msz;
  const long long cs = (long long)P * wpp;
  const dim3 rows(64, P);
  const Op W1{W.m[0], W.sb, W.sh, h}, W2{W.m[1], W.sb, W.sh, d};
  if (pb.bf16)
    hipLaunchKernelGGL(k_rows_f32<bf16>, rows, dim3(kT), 0, st, pb, (const bf16*)pb.k, pb.stats, t0, nt, sb.X);
  else
    hipLaunchKernelGGL(k_rows_f32<float>, rows, dim3(kT), 0, st, pb, (const float*)pb.k, pb.stats, t0, nt, sb.X);
  const Op X = pm(sb.X, nd, H, d);
  gemm<false, false, EPI_GELU>(P, H, nt, h, d, 1, X, W1, pmo(sb.Z, nh, H, h), false, st, 1.0f,
                               Epi{nullptr, nullptr, nullptr, sb.A});                               // Z, A
  if (pb.loss == LOSS_MSE) gemm<false, false>(P, H, nt, d, h, 1, pm(sb.A, nh, H, h), W2, pmo(sb.F, nd, H, d), false, st);
  if (pb.bf16) hipLaunchKernelGGL(k_loss_grad<bf16>, rows, dim3(kT), 0, st, pb, t0, nt, sb.F, sb.G);
  else hipLaunchKernelGGL(k_loss_grad<float>, rows, dim3(kT), 0, st, pb, t0, nt, sb.F, sb.G);
  const Op G = pm(sb.G, nd, H, d);
  const OutOp o1{part, wpp * H, wpp, cs, h}, o2{part + msz, wpp * H, wpp, cs, d};
  gemm<true, false>(P, H, h, d, nt, KS, pm(sb.A, nh, H, h), G, o2, false, st);                      // dW2 slices
  float* dA = sb.dA ? sb.dA : sb.dZ;
  gemm<false, true, EPI_GP>(P, H, nt, h, d, 1, G, W2, pmo(dA, nh, H, h), false, st, 1.0f,
                            Epi{sb.Z, nullptr, nullptr, sb.dZ});                                    // dA, dZ
  gemm<true, false>(P, H, d, h, nt, KS, X, pm(sb.dZ, nh, H, h), o1, false, st);                     // dW1 slices
}

void launch_backward_mfma(const Problem& pb, const WRef& w0, const void* dO, const BwdMfmaBufs& bb, float* dq,
                          float* dk, float* dv, float* deta, float* const* dW0, int w0_shared, int S_kn,
                          hipStream_t st) {
  const int P = pb.B * pb.H, H = pb.H, N = pb.N, d = pb.d, h = pb.hid;
  BwdMfmaSizes sz;
  bwd_mfma_sizes(pb, &sz);
  const int KS = sz.KS;
  const long long nd = (long long)N * d, nh = (long long)N * h, msz = pb.msz;
  const long long wpp = 2 * msz;                               // state floats per pair
  const bool mse = pb.loss == LOSS_MSE;
  const dim3 rows(64, P);
  // operands of the weights: W0 through its strides, W*, U, dW as [P][2][msz]
  const Op W1{w0.m[0], w0.sb, w0.sh, h}, W2{w0.m[1], w0.sb, w0.sh, d};
  auto st1 = [&](const float* base) { return Op{base, wpp * H, wpp, h}; };        // matrix 0: [d][h]
  auto st2 = [&](const float* base) { return Op{base + msz, wpp * H, wpp, d}; };  // matrix 1: [h][d]
  auto so1 = [&](float* base, long long cs) { return OutOp{base, wpp * H, wpp, cs, h}; };
  auto so2 = [&](float* base, long long cs) { return OutOp{base + msz, wpp * H, wpp, cs, d}; };
  const long long cs = (long long)P * wpp;                     // K-slice stride of the weight partials

  // token rows as fp32: Q, dO (X = K_hat comes with the step)
  if (pb.bf16) {
    hipLaunchKernelGGL(k_rows_f32<bf16>, rows, dim3(kT), 0, st, pb, (const bf16*)pb.q, (const float*)nullptr, 0, N, bb.Q);
    hipLaunchKernelGGL(k_rows_f32<bf16>, rows, dim3(kT), 0, st, pb, (const bf16*)dO, (const float*)nullptr, 0, N, bb.dO);
  } else {
    hipLaunchKernelGGL(k_rows_f32<float>, rows, dim3(kT), 0, st, pb, (const float*)pb.q, (const float*)nullptr, 0, N,
                       bb.Q);
    hipLaunchKernelGGL(k_rows_f32<float>, rows, dim3(kT), 0, st, pb, (const float*)dO, (const float*)nullptr, 0, N,
                       bb.dO);
  }
  const Op X = pm(bb.X, nd, H, d), Q = pm(bb.Q, nd, H, d), dOp = pm(bb.dO, nd, H, d);

  // ---- the step at W0 (Z, A, F, G, dA, dZ kept for the terms of phi), W*
  launch_step_mfma(pb, w0, 0, N, StepMfmaBufs{bb.X, bb.Z, bb.A, bb.dA, bb.dZ, bb.F, bb.G}, bb.part, KS, st);
  const Op G = pm(bb.G, nd, H, d);
  hipLaunchKernelGGL(k_sum_slices, dim3(ew_blocks(cs)), dim3(kT), 0, st, bb.part, KS, cs, 1.0f,
                     (const float*)nullptr, bb.dW);
  hipLaunchKernelGGL(k_wstar, dim3((unsigned)std::min<long long>((msz + kT - 1) / kT, 64), P, 2), dim3(kT), 0, st, pb,
                     w0, bb.dW, bb.Ws);

  // ---- the readout backward at W*: U = dS/dW*, dQ
  gemm<false, false, EPI_GELU>(P, H, N, h, d, 1, Q, st1(bb.Ws), pmo(bb.Zd, nh, H, h), false, st, 1.0f,
                               Epi{nullptr, nullptr, nullptr, bb.Ad});                              // Zq, Aq (in Zd, Ad)
  gemm<true, false>(P, H, h, d, N, KS, pm(bb.Ad, nh, H, h), dOp, so2(bb.part, cs), false, st);  // U2 slices
  gemm<false, true, EPI_GP>(P, H, N, h, d, 1, dOp, st2(bb.Ws), pmo(bb.Ab, nh, H, h), false, st, 1.0f,
                            Epi{bb.Zd, nullptr, nullptr, bb.Ab});                                  // dZq (in Ab)
  gemm<true, false>(P, H, d, h, N, KS, Q, pm(bb.Ab, nh, H, h), so1(bb.part, cs), false, st);    // U1 slices
  hipLaunchKernelGGL(k_sum_slices, dim3(ew_blocks(cs)), dim3(kT), 0, st, bb.part, KS, cs, 1.0f,
                     (const float*)nullptr, bb.U);
  // dQ = dZq W1*^T, written at the pair's rows of dq
  {
    const OutOp dqo{dq + (long long)pb.h0 * nd, (long long)pb.Hs * nd, nd, 0, d};
    gemm<false, true>(P, H, N, d, h, 1, pm(bb.Ab, nh, H, h), st1(bb.Ws), dqo, false, st);
  }

  // ---- through the step: tangent along U, phi's per-token and weight terms
  gemm<false, false, EPI_GP>(P, H, N, h, d, 1, X, st1(bb.U), pmo(bb.Zd, nh, H, h), false, st, 1.0f,
                             Epi{bb.Z, nullptr, nullptr, bb.Ad});                                  // Z_dot, A_dot
  gemm<false, false>(P, H, N, d, h, 1, pm(bb.Ad, nh, H, h), W2, pmo(bb.Fd, nd, H, d), false, st);
  gemm<false, false>(P, H, N, d, h, 1, pm(bb.A, nh, H, h), st2(bb.U), pmo(bb.Fd, nd, H, d), true, st);  // F_dot
  if (pb.bf16) hipLaunchKernelGGL(k_phi_tok<bf16>, dim3((N + 3) / 4, P), dim3(kT), 0, st, pb, bb.F, bb.Fd, dv, deta);
  else hipLaunchKernelGGL(k_phi_tok<float>, dim3((N + 3) / 4, P), dim3(kT), 0, st, pb, bb.F, bb.Fd, dv, deta);
  const Op Fb = pm(bb.Fd, nd, H, d);    // F_bar (MSE)
  // A_bar = G U2^T + F_bar W2^T, then Z_bar in its place
  const Epi zbar{bb.Z, bb.Zd, bb.dA, nullptr};
  if (mse) {
    gemm<false, true>(P, H, N, h, d, 1, G, st2(bb.U), pmo(bb.Ab, nh, H, h), false, st);
    gemm<false, true, EPI_ZBAR>(P, H, N, h, d, 1, Fb, W2, pmo(bb.Ab, nh, H, h), true, st, 1.0f, zbar);
  } else {
    gemm<false, true, EPI_ZBAR>(P, H, N, h, d, 1, G, st2(bb.U), pmo(bb.Ab, nh, H, h), false, st, 1.0f, zbar);
  }
  // dK_hat = -(Z_dot_bar U1^T + Z_bar W1^T), at the pair's rows of dk
  {
    const OutOp dko{dk + (long long)pb.h0 * nd, (long long)pb.Hs * nd, nd, 0, d};
    gemm<false, true>(P, H, N, d, h, 1, pm(bb.dZ, nh, H, h), st1(bb.U), dko, false, st, -1.0f);
    gemm<false, true>(P, H, N, d, h, 1, pm(bb.Ab, nh, H, h), W1, dko, true, st, -1.0f);
  }
  // dphi/dW1 = X^T Z_bar; dphi/dW2 = A_dot^T G + A^T F_bar
  gemm<true, false>(P, H, d, h, N, KS, X, pm(bb.Ab, nh, H, h), so1(bb.part, cs), false, st);
  gemm<true, false>(P, H, h, d, N, KS, pm(bb.Ad, nh, H, h), G, so2(bb.part, cs), false, st);
  if (mse) gemm<true, false>(P, H, h, d, N, KS, pm(bb.A, nh, H, h), Fb, so2(bb.part, cs), true, st);
  // dW0 per pair = U - dphi/dW0 (in dW), then the caller's layout
  hipLaunchKernelGGL(k_sum_slices, dim3(ew_blocks(cs)), dim3(kT), 0, st, bb.part, KS, cs, -1.0f, (const float*)bb.U,
                     bb.dW);
  launch_bwd_tail(pb, bb.dW, w0_shared, dW0, dk, S_kn, bb.knp, st);
}

}  // namespace ttt
