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

typedef __attribute__((__vector_size__(2 * sizeof(__bf16)))) __bf16 bf16x2;

constexpr int D = 64;
constexpr int TT = 64;               // tokens per tile
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

// Staging map: thread t moves channels 8 (t % 8) .. + 7 of the adjacent tile
// tokens 2 (t / 8) and 2 (t / 8) + 1 (two 16-byte loads per tensor; a wave's
// loads cover whole 128-byte token rows).
//
// X^T is kept in LDS as [channel][token] rows whose 8-token groups are
// permuted per row: group G of channel c sits at group G ^ swz(c),
// swz(c) = (c / 8) & 6.  Then both the packed two-token stores of the staging
// map and the 16-byte MFMA operand reads (16 channels, one group) fall on 64
// distinct LDS banks.
__device__ __forceinline__ int xt_col(int c, int t) { return ((((t >> 3) ^ ((c >> 3) & 6))) << 3) | (t & 7); }

struct TileRegs {
  bf16x8 x[2], v[2];
  float e;
};

// partial dW1, dW2 of token split blockIdx.x of pair blockIdx.y (tiles
// [s T / S, (s + 1) T / S) of the T tiles).  The K, V and eta of the next two
// tiles are loaded into registers while the current tile is computed, so each
// workgroup keeps two tiles (32 KiB) of loads in flight.  Three workgroups
// per CU (LDS); the register budget is held to three waves per SIMD to match.
// (mean, rstd) of one channel from the key-statistics slices of its pair, sp =
// [S][3][d] (count, mean, M2): Chan et al.'s pairwise combination in double
// precision, slices in order (loads of eight slices in flight)
__device__ float2 merge_key_slices(const float* __restrict__ sp, int S, int d, int c, float eps) {
  double n = 0.0, mean = 0.0, m2 = 0.0;
  for (int s0 = 0; s0 < S; s0 += 8) {
    float a[8], b[8], e[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const float* o = sp + (size_t)min(s0 + u, S - 1) * 3 * d + c;
      a[u] = o[0];
      b[u] = o[d];
      e[u] = o[2 * d];
    }
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      if (s0 + u >= S || a[u] == 0.f) continue;
      const double nb = a[u], nt = n + nb, delta = (double)b[u] - mean;
      mean += delta * nb / nt;
      m2 += (double)e[u] + delta * delta * n * nb / nt;
      n = nt;
    }
  }
  const double var = n > 0.0 ? m2 / n : 0.0;
  return float2{(float)mean, (float)(1.0 / sqrt(var + (double)eps))};
}

template <int LOSS>
__global__ void __launch_bounds__(NW * 64) __attribute__((amdgpu_waves_per_eu(3, 3))) k_glu_grad(Problem pb, WRef W, int t0, int nt, int S,
                                                      const float* __restrict__ spart, int S_stats, float eps,
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
  constexpr bool mse = LOSS == LOSS_MSE;     // the loss is a template parameter: no select between both forms
  const float cm = 2.0f / ((float)nt * (float)D);
  bf16x8 w1f[2], w2f[2];
  load_wfrag(W.mat(0, b, h), w, r, g, w1f);
  load_wfrag(W.mat(1, b, h), w, r, g, w2f);
  const int st = 2 * (tid >> 3), sc = (tid & 7) * 8;
  // key statistics (mean, rstd), merged here from the pair's slices (or read
  // finished), channel c at [c % 8][c / 8] so that the eight channel groups of
  // a wave read eight consecutive entries
  __shared__ float2 nrm[D];
  if (tid < D)
    nrm[(tid & 7) * 8 + (tid >> 3)] =
        spart ? merge_key_slices(spart + (size_t)p * S_stats * 3 * D, S_stats, D, tid, eps)
              : pb.stats ? reinterpret_cast<const float2*>(pb.stats)[(size_t)p * D + tid] : float2{0.f, 1.f};
  // Rows past the batch load the batch's last row (every load is issued on
  // every path, so the compiler's waits stay exact); their eta is 0, which
  // zeroes their dU and dZ and so their share of dW.
  auto fetch = [&](int kt, TileRegs& t) {
#pragma unroll
    for (int q = 0; q < 2; ++q) {
      const int n = min(kt * TT + st + q, nt - 1);
      t.x[q] = *reinterpret_cast<const bf16x8*>(kp + (long long)n * D + sc);
      t.v[q] = *reinterpret_cast<const bf16x8*>(vp + (long long)n * D + sc);
    }
    const int n = kt * TT + (tid & (TT - 1));
    const float e = pb.eta_scale * (ep ? ep[min(n, nt - 1)] : 1.f);
    t.e = n < nt ? e : 0.f;
  };
  f32x4 a1[4], a2[4];   // dW1, dW2 blocks [channel block cb][unit block w]
#pragma unroll
  for (int cb = 0; cb < 4; ++cb) { a1[cb] = f32x4{0, 0, 0, 0}; a2[cb] = f32x4{0, 0, 0, 0}; }
  const int tiles = (nt + TT - 1) / TT;
  const int k0 = (int)((long long)s * tiles / S), k1 = (int)((long long)(s + 1) * tiles / S);
  // one tile: its registers -> LDS, refill them with tile kt + 2, compute
  auto step = [&](int kt, TileRegs& cur) {
    __syncthreads();                                   // the previous tile's LDS reads are done
    bf16x8 xv[2] = {cur.x[0], cur.x[1]};
    if (pb.stats) {
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const float2 m = nrm[e * 8 + (sc >> 3)];
#pragma unroll
        for (int q = 0; q < 2; ++q) xv[q][e] = (bf16)(((float)xv[q][e] - m.x) * m.y);
      }
    }
#pragma unroll
    for (int q = 0; q < 2; ++q) {
      *reinterpret_cast<bf16x8*>(&Xs[(st + q) * LX + sc]) = xv[q];
      *reinterpret_cast<bf16x8*>(&Vs[(st + q) * LX + sc]) = cur.v[q];
    }
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      bf16x2 pr;
      pr[0] = xv[0][e];
      pr[1] = xv[1][e];
      *reinterpret_cast<bf16x2*>(&Xt[(sc + e) * LT + xt_col(sc + e, st)]) = pr;
    }
    if (tid < TT) es[tid] = cur.e;
    if (kt + 2 < k1) fetch(kt + 2, cur);
    __syncthreads();
    // U, Z of (16 tokens x this wave's 16 units), four token blocks
#pragma unroll
    for (int tb = 0; tb < TT / 16; ++tb) {
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
    // dW1 += X^T dU, dW2 += X^T dZ for (channel block cb, unit block w), 32 tokens per product
#pragma unroll
    for (int kk = 0; kk < TT / 32; ++kk) {
      const bf16x8 bu = *reinterpret_cast<const bf16x8*>(&dUs[(16 * w + r) * LT + 32 * kk + 8 * g]);
      const bf16x8 bz = *reinterpret_cast<const bf16x8*>(&dZs[(16 * w + r) * LT + 32 * kk + 8 * g]);
#pragma unroll
      for (int cb = 0; cb < 4; ++cb) {
        const int c = 16 * cb + r;
        const bf16x8 xa = *reinterpret_cast<const bf16x8*>(&Xt[c * LT + xt_col(c, 32 * kk + 8 * g)]);
        a1[cb] = mfma16(xa, bu, a1[cb]);
        a2[cb] = mfma16(xa, bz, a2[cb]);
      }
    }
  };
  // two tiles of loads in flight: ra and rb alternate
  TileRegs ra, rb;
  if (k0 < k1) fetch(k0, ra);
  if (k0 + 1 < k1) fetch(k0 + 1, rb);
  for (int kt = k0; kt < k1; kt += 2) {
    step(kt, ra);
    if (kt + 1 < k1) step(kt + 1, rb);
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

// O = (Q W1*) * silu(Q W2*) for tiles [s T / S, (s + 1) T / S) of pair
// blockIdx.y from the state (layout [P][2][d*d]).  Q of the next two tiles
// is loaded while the current one is computed; O is staged in LDS for
// row-wise 16-byte stores.  Registers are held to eight waves per SIMD, so
// eight workgroups fit a CU (LDS 18 KiB each) and the grid is one round.
__global__ void __launch_bounds__(NW * 64) __attribute__((amdgpu_waves_per_eu(8, 8))) k_glu_query(Problem pb, const float* __restrict__ state, int S) {
  __shared__ __attribute__((aligned(16))) bf16 Qs[TT * LX];
  __shared__ __attribute__((aligned(16))) bf16 Os[TT * LX];
  const int s = blockIdx.x, p = blockIdx.y;
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
  struct QRegs { bf16x8 q[2]; };
  auto fetch = [&](int kt, QRegs& t) {
#pragma unroll
    for (int q = 0; q < 2; ++q) {
      const int n = kt * TT + st + 32 * q;
      t.q[q] = n < pb.N ? *reinterpret_cast<const bf16x8*>(qp + (long long)n * D + sc) : bf16x8{};
    }
  };
  const int tiles = (pb.N + TT - 1) / TT;
  const int k0 = (int)((long long)s * tiles / S), k1 = (int)((long long)(s + 1) * tiles / S);
  auto step = [&](int kt, QRegs& cur) {
    __syncthreads();                                   // Qs and Os of the previous tile are consumed
#pragma unroll
    for (int q = 0; q < 2; ++q) *reinterpret_cast<bf16x8*>(&Qs[(st + 32 * q) * LX + sc]) = cur.q[q];
    if (kt + 2 < k1) fetch(kt + 2, cur);
    __syncthreads();
#pragma unroll
    for (int tb = 0; tb < TT / 16; ++tb) {
      f32x4 u = {0, 0, 0, 0}, z = {0, 0, 0, 0};
      // U^T = W1^T Q^T: the lane holds units 16 w + 4 g .. + 3 of token 16 tb + r
#pragma unroll
      for (int ks = 0; ks < 2; ++ks) {
        const bf16x8 qa = *reinterpret_cast<const bf16x8*>(&Qs[(16 * tb + r) * LX + 32 * ks + 8 * g]);
        u = mfma16(w1f[ks], qa, u);
        z = mfma16(w2f[ks], qa, z);
      }
      bf16x4 ov;
#pragma unroll
      for (int i = 0; i < 4; ++i) ov[i] = (bf16)(u[i] * z[i] * sigm(z[i]));
      *reinterpret_cast<bf16x4*>(&Os[(16 * tb + r) * LX + 16 * w + 4 * g]) = ov;
    }
    __syncthreads();
#pragma unroll
    for (int q = 0; q < 2; ++q) {
      const int n = kt * TT + st + 32 * q;
      if (n < pb.N)
        *reinterpret_cast<bf16x8*>(op + (long long)n * D + sc) = *reinterpret_cast<const bf16x8*>(&Os[(st + 32 * q) * LX + sc]);
    }
  };
  QRegs ra, rb;
  if (k0 < k1) fetch(k0, ra);
  if (k0 + 1 < k1) fetch(k0 + 1, rb);
  for (int kt = k0; kt < k1; kt += 2) {
    step(kt, ra);
    if (kt + 1 < k1) step(kt + 1, rb);
  }
}

}  // namespace

bool glu_supported(const Problem& pb) { return pb.bf16 && pb.inner == INNER_GLU && pb.d == D; }

// token splits per pair: one round of workgroups over the chip (the LDS of
// the gradient kernel, about 46 KiB, fits three per CU), at least two tiles
// per split so that the prefetch overlaps
int glu_grad_splits(const Problem& pb, int nt) {
  const long long P = (long long)pb.B * pb.H;
  long long s = 3LL * device_cu_count() / P;
  const long long tiles = (nt + TT - 1) / TT;
  const long long maxs = (tiles + 1) / 2;
  if (s > maxs) s = maxs;
  if (s < 1) s = 1;
  return (int)s;
}

void launch_glu_grad(const Problem& pb, const WRef& W, int t0, int nt, int S, const float* spart, int S_stats,
                     float eps, float* part, hipStream_t st) {
  if (pb.loss == LOSS_MSE)
    hipLaunchKernelGGL(k_glu_grad<LOSS_MSE>, dim3(S, pb.B * pb.H), dim3(NW * 64), 0, st, pb, W, t0, nt, S, spart,
                       S_stats, eps, part);
  else
    hipLaunchKernelGGL(k_glu_grad<LOSS_DOT>, dim3(S, pb.B * pb.H), dim3(NW * 64), 0, st, pb, W, t0, nt, S, spart,
                       S_stats, eps, part);
}

// one round of readout workgroups over the chip (eight per CU), each over a
// balanced range of at least two tiles of its pair
void launch_glu_query(const Problem& pb, const float* state, hipStream_t st) {
  const long long P = (long long)pb.B * pb.H;
  const long long tiles = (pb.N + TT - 1) / TT;
  long long S = 8LL * device_cu_count() / P;
  if (S > (tiles + 1) / 2) S = (tiles + 1) / 2;
  if (S < 1) S = 1;
  hipLaunchKernelGGL(k_glu_query, dim3((unsigned)S, (unsigned)P), dim3(NW * 64), 0, st, pb, state, (int)S);
}

}  // namespace ttt
