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
// kernels are bound by HBM, so they are plain fp32 loops with lanes along the
// channels (coalesced rows) and no matrix cores.
//
// Main path: each workgroup stages an 8 x 8 token tile of the raster plus its
// halo of (k - 1) / 2 tokens into LDS (fp32, keys already normalised, zeros
// outside the raster), issuing all of its loads at once, then takes every tap
// from LDS.  A fallback reads the neighbours straight from global memory for
// channel counts or kernel sizes whose tile does not fit the LDS budget.
#include "ttt_internal.h"

namespace ttt {

namespace {

constexpr int kWaves = 4;
constexpr int kMaxC = 128;          // channels: lane c and c + 64
constexpr int kQTok = 64;           // tokens per readout workgroup

template <typename T>
__device__ __forceinline__ float ldf(const T* p) { return to_f32<T>(*p); }

// ---------------------------------------------------------------------------
// LDS-tiled kernels
// ---------------------------------------------------------------------------
constexpr int kTile = 8;                          // tile side in tokens
constexpr int kTileTok = kTile * kTile;
constexpr int kTokPerWave = kTileTok / kWaves;    // 16
constexpr size_t kTileLdsMax = 64 * 1024;         // sp^2 d * 4 bytes <= 64 KiB

// 16-byte loads per thread that stage a (8 + K - 1)^2 window of d <= 64 U
// channels: sp^2 (d / 8) / 256 rounded up (at most 8 within the LDS budget)
template <int K, int U>
constexpr int stage_iters() { return ((kTile + K - 1) * (kTile + K - 1) * 8 * U + kWaves * 64 - 1) / (kWaves * 64); }

size_t tile_lds_bytes(int d, int K) {
  const size_t sp = kTile + K - 1;
  return sp * sp * (size_t)d * sizeof(float);
}
// the gradient also stages the tile's V rows (element size es) and eta
size_t grad_lds_bytes(int d, int K, size_t es) { return tile_lds_bytes(d, K) + kTileTok * (d * es + sizeof(float)); }

// d in {8, 16, 32, 64, 128}: eight channels per 16-byte load and a fixed
// channel group per thread (d / 8 divides the workgroup size)
bool tiled_ok(const Problem& pb) {
  return pb.d % 8 == 0 && pb.d <= 128 && (kWaves * 64) % (pb.d / 8) == 0 &&
         grad_lds_bytes(pb.d, pb.ck, pb.bf16 ? 2 : 4) <= kTileLdsMax;
}

template <typename T>
__device__ __forceinline__ void load8(const T* p, float* x);
template <>
__device__ __forceinline__ void load8<bf16>(const bf16* p, float* x) {
  const bf16x8 v = *reinterpret_cast<const bf16x8*>(p);
#pragma unroll
  for (int i = 0; i < 8; ++i) x[i] = (float)v[i];
}
template <>
__device__ __forceinline__ void load8<float>(const float* p, float* x) {
  const float4 a = reinterpret_cast<const float4*>(p)[0], b = reinterpret_cast<const float4*>(p)[1];
  x[0] = a.x; x[1] = a.y; x[2] = a.z; x[3] = a.w; x[4] = b.x; x[5] = b.y; x[6] = b.z; x[7] = b.w;
}

// Raster rows ti0 - R .. ti0 + 7 + R, columns tj0 - R .. tj0 + 7 + R of one
// pair's [N][d] rows -> tile[pos][d] (pos = row-major in the (8 + k - 1)^2
// window) as (x - mu) * rs per channel; window positions outside the raster
// hold 0, the convolution's zero padding.  Thread t owns channels
// 8 (t % (d / 8)) .. + 7, whose mu / rs it holds.  All loads are issued
// before the first is used: a position outside the raster reads the pair's
// first row and is zeroed afterwards, so that no load sits under a branch
// of its own (each would be waited for before the next is issued).
template <typename T, int K, int U>
__device__ __forceinline__ void stage_tile(const T* __restrict__ src, int gh, int gw, int d, int ti0, int tj0,
                                           const float* mu, const float* rs, float* __restrict__ tile) {
  constexpr int SP = kTile + K - 1, R = (K - 1) / 2;
  constexpr int IT = stage_iters<K, U>();
  const int groups = d >> 3, total = SP * SP * groups;
  float x[IT][8];
  bool in[IT];
#pragma unroll
  for (int it = 0; it < IT; ++it) {
    const int e = threadIdx.x + it * kWaves * 64;
    const int pos = e / groups, cg = e % groups;
    const int ii = ti0 + pos / SP - R, jj = tj0 + pos % SP - R;
    in[it] = e < total && ii >= 0 && ii < gh && jj >= 0 && jj < gw;
    load8<T>(src + (in[it] ? ((long long)ii * gw + jj) * d + cg * 8 : 0LL), x[it]);
  }
#pragma unroll
  for (int it = 0; it < IT; ++it) {
    const int e = threadIdx.x + it * kWaves * 64;
    if (e >= total) break;
#pragma unroll
    for (int i = 0; i < 8; ++i) x[it][i] = in[it] ? (x[it][i] - mu[i]) * rs[i] : 0.f;
    float4* dst = reinterpret_cast<float4*>(tile + (size_t)e * 8);   // pos * d + cg * 8 == 8 e
    dst[0] = make_float4(x[it][0], x[it][1], x[it][2], x[it][3]);
    dst[1] = make_float4(x[it][4], x[it][5], x[it][6], x[it][7]);
  }
}

// partial dw over the tiles s, s + S, ... of pair p -> part[(s P + p) msz + c k^2 + tap].
// grid = (S, P), 256 threads, dynamic LDS grad_lds_bytes(d, k, sizeof(T)), d <= 64 U.
// Wave w takes the tile's tokens w, w + 4, ..., lane l channels l + 64 u.
template <typename T, int K, int U>
__global__ void __launch_bounds__(kWaves * 64) k_dw_grad_tile(Problem pb, WRef W, int S, float mse_scale,
                                                              float* __restrict__ part) {
  constexpr int KK = K * K, SP = kTile + K - 1;
  extern __shared__ float tile[];   // key window, then V rows [64][d] (T), then eta [64]
  const int s = blockIdx.x, p = blockIdx.y;
  const int b = p / pb.H, h = p % pb.H;
  const int d = pb.d, gw = pb.gw, gh = pb.gh;
  const long long prow = pb.row(p);
  const T* kp = (const T*)pb.k + prow * pb.N * d;
  const T* vp = (const T*)pb.v + prow * pb.N * d;
  const float* ep = pb.eta_tok ? pb.eta_tok + prow * pb.N : nullptr;
  const float* w = W.mat(0, b, h);
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  const bool mse = pb.loss == LOSS_MSE;
  const int cg = threadIdx.x % (d >> 3);
  float smu[8], srs[8];
  if (pb.stats) {
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int c = cg * 8 + i;
      smu[i] = pb.stats[((size_t)p * d + c) * 2];
      srs[i] = pb.stats[((size_t)p * d + c) * 2 + 1];
    }
  } else {
#pragma unroll
    for (int i = 0; i < 8; ++i) { smu[i] = 0.f; srs[i] = 1.f; }
  }
  float acc[U][KK], wr[U][KK];
#pragma unroll
  for (int u = 0; u < U; ++u) {
    const int c = lane + 64 * u;
#pragma unroll
    for (int t = 0; t < KK; ++t) { acc[u][t] = 0.f; wr[u][t] = (mse && c < d) ? w[c * KK + t] : 0.f; }
  }
  T* vs = reinterpret_cast<T*>(tile + SP * SP * d);
  float* es = reinterpret_cast<float*>(vs + kTileTok * d);
  const int tw = (gw + kTile - 1) / kTile, ntiles = tw * ((gh + kTile - 1) / kTile);
  for (int tix = s; tix < ntiles; tix += S) {
    const int ti0 = (tix / tw) * kTile, tj0 = (tix % tw) * kTile;
    __syncthreads();   // the previous tile's taps have been read
    {
      // V rows of the tile's 64 tokens (16-byte loads, zeros outside the
      // raster) and their eta, issued together with the key window's loads
      constexpr int IV = kTileTok * 8 * U / (kWaves * 64);
      const int groups = d >> 3;
      bf16x8 vb[IV];
      float4 vf[IV][2];
#pragma unroll
      for (int it = 0; it < IV; ++it) {
        const int e = threadIdx.x + it * kWaves * 64, tt = e / groups;
        const int i = ti0 + tt / kTile, j = tj0 + tt % kTile;
        const bool ok = e < kTileTok * groups && i < gh && j < gw;
        // outside the raster: read the pair's first row, zeroed below
        const T* src = vp + (ok ? ((long long)i * gw + j) * d + (e % groups) * 8 : 0LL);
        if constexpr (sizeof(T) == 2) {
          vb[it] = *reinterpret_cast<const bf16x8*>(src);
          if (!ok) vb[it] = bf16x8{};
        } else {
          vf[it][0] = reinterpret_cast<const float4*>(src)[0];
          vf[it][1] = reinterpret_cast<const float4*>(src)[1];
          if (!ok) vf[it][0] = vf[it][1] = make_float4(0.f, 0.f, 0.f, 0.f);
        }
      }
      float ev = 0.f;
      if (threadIdx.x < kTileTok) {
        const int i = ti0 + threadIdx.x / kTile, j = tj0 + threadIdx.x % kTile;
        if (i < gh && j < gw) ev = pb.eta_scale * (ep ? ep[(long long)i * gw + j] : 1.f);
      }
      stage_tile<T, K, U>(kp, gh, gw, d, ti0, tj0, smu, srs, tile);
#pragma unroll
      for (int it = 0; it < IV; ++it) {
        const int e = threadIdx.x + it * kWaves * 64;
        if (e >= kTileTok * groups) break;
        if constexpr (sizeof(T) == 2) {
          *reinterpret_cast<bf16x8*>(vs + (size_t)e * 8) = vb[it];
        } else {
          reinterpret_cast<float4*>(vs + (size_t)e * 8)[0] = vf[it][0];
          reinterpret_cast<float4*>(vs + (size_t)e * 8)[1] = vf[it][1];
        }
      }
      if (threadIdx.x < kTileTok) es[threadIdx.x] = ev;
    }
    __syncthreads();
#pragma unroll 1
    for (int m = 0; m < kTokPerWave; ++m) {
      const int tt = wv + kWaves * m, ti = tt / kTile, tj = tt % kTile;
      if (ti0 + ti >= gh || tj0 + tj >= gw) continue;
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const int c = lane + 64 * u;
        if (c >= d) continue;
        float nb[KK];
#pragma unroll
        for (int a = 0; a < K; ++a)
#pragma unroll
          for (int bb = 0; bb < K; ++bb) nb[a * K + bb] = tile[((ti + a) * SP + tj + bb) * d + c];
        const float vv = to_f32<T>(vs[tt * d + c]), et = es[tt];
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
  }
  // the four waves' sums, added in wave order (the tile buffer holds
  // 4 d k^2 floats: (8 + k - 1)^2 >= 4 k^2 for k <= 7)
  __syncthreads();
  float* red = tile;
#pragma unroll
  for (int u = 0; u < U; ++u) {
    const int c = lane + 64 * u;
    if (c < d)
#pragma unroll
      for (int t = 0; t < KK; ++t) red[((size_t)wv * d + c) * KK + t] = acc[u][t];
  }
  __syncthreads();
  float* out = part + ((long long)s * pb.B * pb.H + p) * pb.msz;
  const int dk = d * KK;
  for (int e = threadIdx.x; e < dk; e += kWaves * 64) {
    float v = 0.f;
#pragma unroll
    for (int q = 0; q < kWaves; ++q) v += red[q * dk + e];
    out[e] = v;
  }
}

// O = F_w(Q) for one 8 x 8 tile of pair p.  grid = (tiles, P), dynamic LDS
// tile_lds_bytes(d, k).
template <typename T, int K, int U>
__global__ void __launch_bounds__(kWaves * 64) k_dw_query_tile(Problem pb, const float* __restrict__ state) {
  constexpr int KK = K * K, SP = kTile + K - 1;
  extern __shared__ float tile[];
  const int tix = blockIdx.x, p = blockIdx.y;
  const int d = pb.d, gw = pb.gw, gh = pb.gh;
  const long long prow = pb.row(p);
  const T* qp = (const T*)pb.q + prow * pb.N * d;
  T* op = (T*)pb.o + prow * pb.N * d;
  const float* w = state + (long long)p * pb.msz;
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  const int tw = (gw + kTile - 1) / kTile;
  const int ti0 = (tix / tw) * kTile, tj0 = (tix % tw) * kTile;
  float wr[U][KK];
#pragma unroll
  for (int u = 0; u < U; ++u)
#pragma unroll
    for (int t = 0; t < KK; ++t) wr[u][t] = lane + 64 * u < d ? w[(lane + 64 * u) * KK + t] : 0.f;
  float zero[8], one[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) { zero[i] = 0.f; one[i] = 1.f; }
  stage_tile<T, K, U>(qp, gh, gw, d, ti0, tj0, zero, one, tile);
  __syncthreads();
#pragma unroll 4
  for (int m = 0; m < kTokPerWave; ++m) {
    const int tt = wv + kWaves * m, ti = tt / kTile, tj = tt % kTile;
    if (ti0 + ti >= gh || tj0 + tj >= gw) continue;
    const long long n = (long long)(ti0 + ti) * gw + tj0 + tj;
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int c = lane + 64 * u;
      if (c >= d) continue;
      float f = 0.f;
#pragma unroll
      for (int a = 0; a < K; ++a)
#pragma unroll
        for (int bb = 0; bb < K; ++bb) f = fmaf(wr[u][a * K + bb], tile[((ti + a) * SP + tj + bb) * d + c], f);
      op[n * d + c] = from_f32<T>(f);
    }
  }
}

// ---------------------------------------------------------------------------
// Fallback kernels: neighbours straight from global memory
// ---------------------------------------------------------------------------

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
  // Lanes past d repeat channel d - 1 (their sums are never written), and
  // neighbours outside the raster are read at the nearest raster position
  // and zeroed, so that no load sits under a branch of its own (each would
  // be waited for before the next is issued).
  float acc[2][KK], wr[2][KK], mu[2] = {0.f, 0.f}, rs[2] = {1.f, 1.f};
#pragma unroll
  for (int u = 0; u < 2; ++u) {
    const int c = min(lane + 64 * u, d - 1);
#pragma unroll
    for (int t = 0; t < KK; ++t) acc[u][t] = 0.f;
    if (mse) {
#pragma unroll
      for (int t = 0; t < KK; ++t) wr[u][t] = w[c * KK + t];
    } else {
#pragma unroll
      for (int t = 0; t < KK; ++t) wr[u][t] = 0.f;
    }
    if (pb.stats) { mu[u] = pb.stats[((size_t)p * d + c) * 2]; rs[u] = pb.stats[((size_t)p * d + c) * 2 + 1]; }
  }
  for (int n = n0 + wv; n < n1; n += kWaves) {
    const int i = n / gw, j = n % gw;
    const float et = pb.eta_scale * (ep ? ep[n] : 1.f);
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      if (64 * u >= d) break;
      const int c = min(lane + 64 * u, d - 1);
      float nb[KK];
#pragma unroll
      for (int a = 0; a < K; ++a)
#pragma unroll
        for (int bb = 0; bb < K; ++bb) {
          const int ii = i + a - R, jj = j + bb - R;
          const bool in = ii >= 0 && ii < gh && jj >= 0 && jj < gw;
          const int iic = min(max(ii, 0), gh - 1), jjc = min(max(jj, 0), gw - 1);
          const float x = ldf(kp + ((long long)iic * gw + jjc) * d + c);
          nb[a * K + bb] = in ? (x - mu[u]) * rs[u] : 0.f;
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
  // lanes past d repeat channel d - 1 and store nothing; neighbours outside
  // the raster are read at the nearest raster position and left out of the
  // sum, so that the loads of a token are all in flight together
  float wr[2][KK];
#pragma unroll
  for (int u = 0; u < 2; ++u)
#pragma unroll
    for (int t = 0; t < KK; ++t) wr[u][t] = w[min(lane + 64 * u, d - 1) * KK + t];
  const int n0 = blockIdx.x * kQTok, n1 = min(N, n0 + kQTok);
  for (int n = n0 + wv; n < n1; n += kWaves) {
    const int i = n / gw, j = n % gw;
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      if (64 * u >= d) break;
      const int c = min(lane + 64 * u, d - 1);
      float x[KK];
#pragma unroll
      for (int a = 0; a < K; ++a)
#pragma unroll
        for (int bb = 0; bb < K; ++bb) {
          const int iic = min(max(i + a - R, 0), gh - 1), jjc = min(max(j + bb - R, 0), gw - 1);
          x[a * K + bb] = ldf(qp + ((long long)iic * gw + jjc) * d + c);
        }
      float f = 0.f;
#pragma unroll
      for (int a = 0; a < K; ++a)
#pragma unroll
        for (int bb = 0; bb < K; ++bb) {
          const int ii = i + a - R, jj = j + bb - R;
          const bool in = ii >= 0 && ii < gh && jj >= 0 && jj < gw;
          f = in ? fmaf(wr[u][a * K + bb], x[a * K + bb], f) : f;
        }
      if (lane + 64 * u < d) op[(long long)n * d + c] = from_f32<T>(f);
    }
  }
}

int tile_count(const Problem& pb) { return ((pb.gh + kTile - 1) / kTile) * ((pb.gw + kTile - 1) / kTile); }

template <typename T, int K>
void grad_tile(const Problem& pb, const WRef& W, int S, float scale, float* part, hipStream_t st) {
  const dim3 grid(S, pb.B * pb.H), block(kWaves * 64);
  const size_t lds = grad_lds_bytes(pb.d, K, sizeof(T));
  if (pb.d > 64) hipLaunchKernelGGL((k_dw_grad_tile<T, K, 2>), grid, block, lds, st, pb, W, S, scale, part);
  else hipLaunchKernelGGL((k_dw_grad_tile<T, K, 1>), grid, block, lds, st, pb, W, S, scale, part);
}

template <typename T, int K>
void query_tile(const Problem& pb, const float* state, hipStream_t st) {
  const dim3 grid(tile_count(pb), pb.B * pb.H), block(kWaves * 64);
  const size_t lds = tile_lds_bytes(pb.d, K);
  if (pb.d > 64) hipLaunchKernelGGL((k_dw_query_tile<T, K, 2>), grid, block, lds, st, pb, state);
  else hipLaunchKernelGGL((k_dw_query_tile<T, K, 1>), grid, block, lds, st, pb, state);
}

template <typename T>
void grad_k(const Problem& pb, const WRef& W, int S, float scale, float* part, hipStream_t st) {
  const dim3 grid(S, pb.B * pb.H), block(kWaves * 64);
  if (tiled_ok(pb)) {
    switch (pb.ck) {
      case 1: grad_tile<T, 1>(pb, W, S, scale, part, st); break;
      case 3: grad_tile<T, 3>(pb, W, S, scale, part, st); break;
      case 5: grad_tile<T, 5>(pb, W, S, scale, part, st); break;
      default: grad_tile<T, 7>(pb, W, S, scale, part, st); break;
    }
    return;
  }
  switch (pb.ck) {
    case 1: hipLaunchKernelGGL((k_dw_grad<T, 1>), grid, block, 0, st, pb, W, S, scale, part); break;
    case 3: hipLaunchKernelGGL((k_dw_grad<T, 3>), grid, block, 0, st, pb, W, S, scale, part); break;
    case 5: hipLaunchKernelGGL((k_dw_grad<T, 5>), grid, block, 0, st, pb, W, S, scale, part); break;
    default: hipLaunchKernelGGL((k_dw_grad<T, 7>), grid, block, 0, st, pb, W, S, scale, part); break;
  }
}

template <typename T>
void query_k(const Problem& pb, const float* state, hipStream_t st) {
  if (tiled_ok(pb)) {
    switch (pb.ck) {
      case 1: query_tile<T, 1>(pb, state, st); break;
      case 3: query_tile<T, 3>(pb, state, st); break;
      case 5: query_tile<T, 5>(pb, state, st); break;
      default: query_tile<T, 7>(pb, state, st); break;
    }
    return;
  }
  const dim3 grid((pb.N + kQTok - 1) / kQTok, pb.B * pb.H), block(kWaves * 64);
  switch (pb.ck) {
    case 1: hipLaunchKernelGGL((k_dw_query<T, 1>), grid, block, 0, st, pb, state); break;
    case 3: hipLaunchKernelGGL((k_dw_query<T, 3>), grid, block, 0, st, pb, state); break;
    case 5: hipLaunchKernelGGL((k_dw_query<T, 5>), grid, block, 0, st, pb, state); break;
    default: hipLaunchKernelGGL((k_dw_query<T, 7>), grid, block, 0, st, pb, state); break;
  }
}

}  // namespace

// Workgroups per pair of the gradient.  Tiled path: one 8 x 8 tile each, up
// to about eight workgroups per CU over all pairs (then several tiles each).
// Fallback: about four workgroups per CU, at least 128 tokens each.
int dwconv_grad_splits(const Problem& pb) {
  const long long P = (long long)pb.B * pb.H;
  if (tiled_ok(pb)) {
    long long s = (8LL * device_cu_count() + P - 1) / P;
    if (s > tile_count(pb)) s = tile_count(pb);
    return (int)(s < 1 ? 1 : s);
  }
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
