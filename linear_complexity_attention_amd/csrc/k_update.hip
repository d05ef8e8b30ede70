// Weight update of the inner model: second stage of the split-N gradient
// reduction, the gradient step, and the optional L2 re-normalisation.
//
//   W_next = W_cur - sum_s partial_s        (eta is already inside the partials,
//                                            ViT3 summary page, section 02 update)
//   renorm: every output column of every [in, out] matrix is rescaled to the L2
//           norm that column has in W0 (LaCT analysis page, section "Nonlinear
//           memory complements local attention": L2 normalisation after the update)
//
// The partials are summed in a fixed order, so the result is bit-reproducible.
// Besides the fp32 state the kernel can emit the caller's W_out.
#include "ttt_internal.h"

namespace ttt {

namespace {

constexpr int kCols = 64;
constexpr int kLanes = 4;                        // row lanes per column (re-norm kernel)

// first and last workgroup of the stream-K gradient kernel that touched pair p
// (the workgroups holding its first and last tile on the cost line), and the
// line length C
__device__ __forceinline__ void sk_range(const UpdateArgs& a, int P, int p, long long& q0, long long& q1,
                                         long long& C) {
  const long long U = a.sk_tpp + kSkAlpha;
  C = (long long)P * U;
  q0 = sk_group_of(p * U + kSkAlpha, a.sk_G, C);
  q1 = sk_group_of(p * U + kSkAlpha + a.sk_tpp - 1, a.sk_G, C);
}

// partial slot of pair p written by workgroup q (q0 <= q <= q1): a workgroup
// after q0 starts inside p, so p is its first pair (slot q J); q0 may have
// started in an earlier pair
__device__ __forceinline__ long long sk_slot(const UpdateArgs& a, int p, long long q, long long q0, long long C) {
  return q * a.sk_J + (q == q0 ? p - sk_first_pair(q0, a.sk_G, C, a.sk_tpp) : 0);
}

__device__ __forceinline__ void mat_dims(const Problem& pb, int i, int& rows, int& cols) {
  if (pb.inner == INNER_LINEAR) { rows = pb.d; cols = pb.d; return; }
  if (i == 1) { rows = pb.hid; cols = pb.d; }   // W2 [h, d]
  else { rows = pb.d; cols = pb.hid; }          // W1, W3 [d, h]
}

// No re-norm: every element is independent.  grid = (chunks of 1024 elements
// of one pair's [nm][msz] block, P); each thread updates 4 consecutive floats.
__global__ void __launch_bounds__(256) k_update_flat(Problem pb, UpdateArgs a) {
  const int p = blockIdx.y;
  const int b = p / pb.H, h = p % pb.H;
  const long long wsz = (long long)pb.nm * pb.msz;
  const long long e = ((long long)blockIdx.x * 256 + threadIdx.x) * 4;
  if (e >= wsz) return;
  const int i = (int)(e / pb.msz);
  const long long o = e - (long long)i * pb.msz;           // offset inside matrix i (msz % 4 == 0)
  float4 w = *reinterpret_cast<const float4*>(a.cur.mat(i, b, h) + o);
  auto sub = [&](const float* q) {
    const float4 d = *reinterpret_cast<const float4*>(q + e);
    w.x -= d.x; w.y -= d.y; w.z -= d.z; w.w -= d.w;
  };
  if (a.part_mode == PART_SPLITS) {           // four splits' loads in flight, subtracted in split order
    const float* pp = a.part + (size_t)p * wsz;
    for (int s = 0; s < a.S; s += 4) {
      float4 d[4];
#pragma unroll
      for (int u = 0; u < 4; ++u)
        if (s + u < a.S) d[u] = *reinterpret_cast<const float4*>(pp + (s + u) * a.part_pair_stride + e);
#pragma unroll
      for (int u = 0; u < 4; ++u)
        if (s + u < a.S) { w.x -= d[u].x; w.y -= d[u].y; w.z -= d[u].z; w.w -= d[u].w; }
    }
  } else {
    long long q0, q1, C;
    sk_range(a, pb.B * pb.H, p, q0, q1, C);
    for (long long q = q0; q <= q1; ++q) sub(a.part + sk_slot(a, p, q, q0, C) * wsz);
  }
  *reinterpret_cast<float4*>(a.next + (size_t)p * wsz + e) = w;
  if (a.out[i]) *reinterpret_cast<float4*>(a.out[i] + (size_t)p * pb.msz + o) = w;
}

// Update from the MFMA gradient kernel's stream-K partials, which are stored in
// its register order (d = 64, GELU MLP, hidden width HID split over its waves
// in slices of HP units, NHB = HP/16 blocks of 16):
//   dW1 part: float4 ((qq*4 + cb)*NHB + hb)*64 + l  ->  dW1[16cb + 4g + i][qq*HP + 16hb + r]
//   dW2 part: float4 ((qq*NHB + hb)*4 + cb)*64 + l  ->  dW2[qq*HP + 16hb + 4g + i][16cb + r]
// with l = 16g + r, i = 0..3.  Thread = one float4 of the partial: it sums that
// float4 over the pair's slots (coalesced) and updates the 4 weights it maps to.
// grid = (D*HID/2 / 256, P).
template <int HID, int HP>
__global__ void __launch_bounds__(256) k_update_streamk(Problem pb, UpdateArgs a) {
  constexpr int D = 64, NHB = HP / 16, HALF = D * HID / 4;   // float4s per matrix
  const int p = blockIdx.y;
  const int b = p / pb.H, h = p % pb.H;
  const int j = blockIdx.x * 256 + threadIdx.x;
  if (j >= 2 * HALF) return;
  const int mat = j >= HALF ? 1 : 0;
  const int jj = j - mat * HALF;
  const int l = jj & 63, blk = jj >> 6, g = l >> 4, r = l & 15;
  int base, step;                 // element offset of i = 0 inside the matrix, stride over i
  if (mat == 0) {
    const int hb = blk % NHB, cb = (blk / NHB) & 3, qq = blk / (4 * NHB);
    base = (16 * cb + 4 * g) * HID + qq * HP + 16 * hb + r;
    step = HID;
  } else {
    const int cb = blk & 3, hb = (blk >> 2) % NHB, qq = blk / (4 * NHB);
    base = (qq * HP + 16 * hb + 4 * g) * D + 16 * cb + r;
    step = D;
  }
  const long long wsz = 2LL * D * HID;
  // W_cur's four values first, so that their loads overlap the partials'
  const float* cur = a.cur.mat(mat, b, h);
  float c4[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) c4[i] = cur[base + i * step];
  long long q0, q1, C;
  sk_range(a, pb.B * pb.H, p, q0, q1, C);
  // the pair's slots, four loads in flight at a time, added in workgroup order
  float4 sum = {0.f, 0.f, 0.f, 0.f};
  for (long long q = q0; q <= q1; q += 4) {
    float4 d[4];
#pragma unroll
    for (int u = 0; u < 4; ++u)
      if (q + u <= q1) d[u] = reinterpret_cast<const float4*>(a.part + sk_slot(a, p, q + u, q0, C) * wsz)[j];
#pragma unroll
    for (int u = 0; u < 4; ++u)
      if (q + u <= q1) { sum.x += d[u].x; sum.y += d[u].y; sum.z += d[u].z; sum.w += d[u].w; }
  }
  float* nxt = a.next + (size_t)p * wsz + (size_t)mat * D * HID;
  float* out = a.out[mat] ? a.out[mat] + (size_t)p * D * HID : nullptr;
  const float s4[4] = {sum.x, sum.y, sum.z, sum.w};
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int e = base + i * step;
    const float w = c4[i] - s4[i];
    nxt[e] = w;
    if (out) out[e] = w;
  }
}

// Re-norm after the flat update: every output column of next is rescaled to
// the L2 norm of the same column of W0.  grid = (column blocks of 16, nm, P);
// thread = (column, row lane), 64 row lanes per column, each holding its rows'
// values in registers between the norm reduction and the rescale (rows past
// RMAX * 64 are read again for the rescale).
constexpr int kRCols = 16, kRLanes = 64;
template <int RMAX>
__global__ void __launch_bounds__(kRCols * kRLanes) k_renorm(Problem pb, UpdateArgs a) {
  const int i = blockIdx.y, p = blockIdx.z;
  const int b = p / pb.H, h = p % pb.H;
  int rows, cols;
  mat_dims(pb, i, rows, cols);
  const int cl = threadIdx.x % kRCols, lane = threadIdx.x / kRCols;
  const int j = blockIdx.x * kRCols + cl;
  const bool live = j < cols;
  const float* w0 = a.w0.mat(i, b, h);
  float* nxt = a.next + ((size_t)p * pb.nm + i) * pb.msz;
  constexpr int kWaves = kRCols * kRLanes / 64;   // each wave holds 4 row lanes of every column
  __shared__ float red[2][kWaves][kRCols];
  float v[RMAX];
  float nn = 0.f, nr = 0.f;
#pragma unroll
  for (int k = 0; k < RMAX; ++k) {
    const int r = lane + kRLanes * k;
    v[k] = 0.f;
    if (live && r < rows) {
      const size_t e = (size_t)r * cols + j;
      v[k] = nxt[e];
      const float w0v = w0[e];
      nn += v[k] * v[k];
      nr += w0v * w0v;
    }
  }
  if (live)                                  // rows beyond the register block: read twice
    for (int r = lane + kRLanes * RMAX; r < rows; r += kRLanes) {
      const size_t e = (size_t)r * cols + j;
      const float x = nxt[e], w0v = w0[e];
      nn += x * x;
      nr += w0v * w0v;
    }
  // column sums: the 4 row lanes of a column inside a wave (wave lanes cl,
  // cl + 16, cl + 32, cl + 48), then the waves through LDS
  nn += __shfl_xor(nn, 16); nr += __shfl_xor(nr, 16);
  nn += __shfl_xor(nn, 32); nr += __shfl_xor(nr, 32);
  if ((lane & 3) == 0) { red[0][lane >> 2][cl] = nn; red[1][lane >> 2][cl] = nr; }
  __syncthreads();
  if (!live) return;
  float sn = 0.f, sr = 0.f;
#pragma unroll
  for (int l = 0; l < kWaves; ++l) { sn += red[0][l][cl]; sr += red[1][l][cl]; }
  const float scale = sqrtf(sr) / fmaxf(sqrtf(sn), 1e-12f);
  float* out = a.out[i] ? a.out[i] + (size_t)p * pb.msz : nullptr;
#pragma unroll
  for (int k = 0; k < RMAX; ++k) {
    const int r = lane + kRLanes * k;
    if (r < rows) {
      const size_t e = (size_t)r * cols + j;
      nxt[e] = v[k] * scale;
      if (out) out[e] = v[k] * scale;
    }
  }
  for (int r = lane + kRLanes * RMAX; r < rows; r += kRLanes) {
    const size_t e = (size_t)r * cols + j;
    const float x = nxt[e] * scale;
    nxt[e] = x;
    if (out) out[e] = x;
  }
}

static void launch_renorm(const Problem& pb, const UpdateArgs& a, hipStream_t st) {
  const int P = pb.B * pb.H;
  const int side = pb.inner == INNER_LINEAR ? pb.d : (pb.hid > pb.d ? pb.hid : pb.d);   // max rows, max cols
  dim3 g((side + kRCols - 1) / kRCols, pb.nm, P);
  if (side <= 2 * kRLanes) hipLaunchKernelGGL(k_renorm<2>, g, dim3(kRCols * kRLanes), 0, st, pb, a);
  else if (side <= 4 * kRLanes) hipLaunchKernelGGL(k_renorm<4>, g, dim3(kRCols * kRLanes), 0, st, pb, a);
  else hipLaunchKernelGGL(k_renorm<8>, g, dim3(kRCols * kRLanes), 0, st, pb, a);
}

// Update and re-norm in one kernel for shapes the float4 path cannot take.
// grid = (column blocks, nm, P); thread = (column, row lane).
__global__ void __launch_bounds__(kCols * kLanes) k_update_renorm(Problem pb, UpdateArgs a) {
  const int i = blockIdx.y, p = blockIdx.z;
  const int b = p / pb.H, h = p % pb.H;
  int rows, cols;
  mat_dims(pb, i, rows, cols);
  const int j = blockIdx.x * kCols + threadIdx.x % kCols;
  const int lane = threadIdx.x / kCols;
  const bool live = j < cols;
  const float* cur = a.cur.mat(i, b, h);
  const float* w0 = a.w0.mat(i, b, h);
  const long long wsz = (long long)pb.nm * pb.msz;
  float* nxt = a.next + (size_t)p * wsz + (size_t)i * pb.msz;
  long long q0 = 0, q1 = -1, C = 1;
  if (a.part_mode == PART_STREAMK) sk_range(a, pb.B * pb.H, p, q0, q1, C);
  __shared__ float red[2][kLanes][kCols];
  float nn = 0.f, nr = 0.f;
  if (live)
    for (int r = lane; r < rows; r += kLanes) {
      const size_t e = (size_t)r * cols + j;
      float w = cur[e];
      if (a.part_mode == PART_SPLITS) {
        const float* pp = a.part + (size_t)p * wsz + (size_t)i * pb.msz + e;
        for (int s = 0; s < a.S; ++s) w -= pp[s * a.part_pair_stride];
      } else {
        for (long long q = q0; q <= q1; ++q) w -= a.part[sk_slot(a, p, q, q0, C) * wsz + (size_t)i * pb.msz + e];
      }
      nxt[e] = w;
      nn += w * w;
      const float w0v = w0[e];
      nr += w0v * w0v;
    }
  red[0][lane][threadIdx.x % kCols] = nn;
  red[1][lane][threadIdx.x % kCols] = nr;
  __syncthreads();
  float sn = 0.f, sr = 0.f;
  for (int l = 0; l < kLanes; ++l) { sn += red[0][l][threadIdx.x % kCols]; sr += red[1][l][threadIdx.x % kCols]; }
  const float scale = a.renorm ? sqrtf(sr) / fmaxf(sqrtf(sn), 1e-12f) : 1.f;
  if (!live) return;
  float* out = a.out[i] ? a.out[i] + (size_t)p * pb.msz : nullptr;
  for (int r = lane; r < rows; r += kLanes) {
    const size_t e = (size_t)r * cols + j;
    const float w = nxt[e] * scale;
    nxt[e] = w;
    if (out) out[e] = w;
  }
}

}  // namespace

void launch_update(const Problem& pb, const UpdateArgs& a, hipStream_t st) {
  const int P = pb.B * pb.H;
  if (a.part_mode == PART_STREAMK) {
    // partials of the MFMA gradient kernel (GELU MLP, d = 64)
    UpdateArgs f = a;
    if (a.renorm)
      for (int i = 0; i < 3; ++i) f.out[i] = nullptr;   // the re-norm pass writes W_out
    const dim3 grid((unsigned)((pb.d * pb.hid / 2 + 255) / 256), P);
    switch (pb.hid) {
      case 64: hipLaunchKernelGGL((k_update_streamk<64, 64 / mfma_grad_waves(64)>), grid, dim3(256), 0, st, pb, f); break;
      case 128: hipLaunchKernelGGL((k_update_streamk<128, 128 / mfma_grad_waves(128)>), grid, dim3(256), 0, st, pb, f); break;
      default: hipLaunchKernelGGL((k_update_streamk<256, 256 / mfma_grad_waves(256)>), grid, dim3(256), 0, st, pb, f); break;
    }
    if (a.renorm) launch_renorm(pb, a, st);
    return;
  }
  // the flat kernel moves float4s: every matrix base and stride must keep 16-byte alignment
  bool aligned = pb.msz % 4 == 0 && a.cur.sb % 4 == 0 && a.cur.sh % 4 == 0;
  for (int i = 0; i < pb.nm; ++i) aligned = aligned && (reinterpret_cast<uintptr_t>(a.cur.m[i]) % 16 == 0) &&
                                          (!a.out[i] || reinterpret_cast<uintptr_t>(a.out[i]) % 16 == 0);
  if (aligned) {
    const long long wsz = (long long)pb.nm * pb.msz;
    dim3 grid((unsigned)((wsz / 4 + 255) / 256), P);
    if (!a.renorm) {
      hipLaunchKernelGGL(k_update_flat, grid, dim3(256), 0, st, pb, a);
      return;
    }
    UpdateArgs f = a;             // the re-norm pass writes W_out
    for (int i = 0; i < 3; ++i) f.out[i] = nullptr;
    hipLaunchKernelGGL(k_update_flat, grid, dim3(256), 0, st, pb, f);
    launch_renorm(pb, a, st);
    return;
  }
  const int maxcols = pb.inner == INNER_LINEAR ? pb.d : (pb.hid > pb.d ? pb.hid : pb.d);
  dim3 grid((maxcols + kCols - 1) / kCols, pb.nm, P);
  hipLaunchKernelGGL(k_update_renorm, grid, dim3(kCols * kLanes), 0, st, pb, a);
}

}  // namespace ttt
