// Weight update of the inner model: second stage of the split-N gradient
// reduction, the gradient step, and the optional L2 re-normalisation.
//
//   W_next = W_cur - sum_s partial_s        (eta is already inside the partials,
//                                            ViT3 summary page, section 02 update)
//   momentum (LaCT analysis page, update rules): M = beta M + sum_s partial_s,
//           W_next = W_cur - M; Muon folds the partials into M the same way and
//           leaves the step to the Newton-Schulz kernels (k_muon.hip)
//   matrices outside the update mask keep W_cur (Test-Time Training vs Sleep
//   page, "Side one": only the first layer adjusted)
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

// first and last workgroup of the stream-K gradient kernel that touched pair
// p, and the cost-line length C
__device__ __forceinline__ void sk_range(const UpdateArgs& a, int P, int p, long long& q0, long long& q1,
                                         long long& C) {
  C = (long long)P * (a.sk_tpp + kSkAlpha);
  sk_pair_groups(p, a.sk_tpp, a.sk_G, C, &q0, &q1);
}

__device__ __forceinline__ long long slot_of(const UpdateArgs& a, int p, long long q, long long q0, long long C) {
  return sk_slot(p, q, q0, a.sk_G, C, a.sk_tpp, a.sk_J);
}

__device__ __forceinline__ void mat_dims(const Problem& pb, int i, int& rows, int& cols) {
  if (pb.inner == INNER_LINEAR) { rows = pb.d; cols = pb.d; return; }
  if (pb.inner == INNER_DWCONV) { rows = pb.d; cols = pb.ck * pb.ck; return; }   // kernel [d][k*k]
  if (i == 1) { rows = pb.hid; cols = pb.d; }   // W2 [h, d]
  else { rows = pb.d; cols = pb.hid; }          // W1, W3 [d, h]
}

// No re-norm: every element is independent.  grid = (blocks of 64 float4s of
// one pair's [nm][msz] block, P), 256 threads: lane l owns float4 64 x + l;
// wave w sums the splits [w S / 4, (w + 1) S / 4) in split order with eight
// loads in flight, and wave 0 adds the four wave sums in wave order and
// applies the rule.
__global__ void __launch_bounds__(256) k_update_flat(Problem pb, UpdateArgs a) {
  const int p = blockIdx.y;
  const int b = p / pb.H, h = p % pb.H;
  const long long wsz = (long long)pb.nm * pb.msz;
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  const long long e = ((long long)blockIdx.x * 64 + lane) * 4;
  const bool in = e < wsz;
  const int i = in ? (int)(e / pb.msz) : 0;
  const bool upd = in && ((a.mask >> i) & 1u);
  float4 g = {0.f, 0.f, 0.f, 0.f};
  auto take = [&](const float4& d) { g.x += d.x; g.y += d.y; g.z += d.z; g.w += d.w; };
  if (upd && a.part_mode == PART_SPLITS) {
    const float* pp = a.part + (size_t)p * wsz + e;
    const int s0 = (int)((long long)wv * a.S / 4), s1 = (int)((long long)(wv + 1) * a.S / 4);
    for (int s = s0; s < s1; s += 8) {
      float4 d[8];
#pragma unroll
      for (int u = 0; u < 8; ++u)
        if (s + u < s1) d[u] = *reinterpret_cast<const float4*>(pp + (s + u) * a.part_pair_stride);
#pragma unroll
      for (int u = 0; u < 8; ++u)
        if (s + u < s1) take(d[u]);
    }
  } else if (upd && wv == 0) {
    long long q0, q1, C;
    sk_range(a, pb.B * pb.H, p, q0, q1, C);
    for (long long q = q0; q <= q1; ++q) take(*reinterpret_cast<const float4*>(a.part + slot_of(a, p, q, q0, C) * wsz + e));
  }
  __shared__ float4 red[4][64];
  red[wv][lane] = g;
  __syncthreads();
  if (wv != 0 || !in) return;
#pragma unroll
  for (int q = 1; q < 4; ++q) { const float4 d = red[q][lane]; g.x += d.x; g.y += d.y; g.z += d.z; g.w += d.w; }
  const long long o = e - (long long)i * pb.msz;           // offset inside matrix i (msz % 4 == 0)
  const float4 wc = *reinterpret_cast<const float4*>(a.cur.mat(i, b, h) + o);
  float4 w = wc;
  if (upd) {
    if (a.rule == RULE_GD) {
      w.x = wc.x - g.x; w.y = wc.y - g.y; w.z = wc.z - g.z; w.w = wc.w - g.w;
    } else {
      // the momentum rules fold the summed partials into M (Muon leaves the step to its kernels)
      float4* mp = reinterpret_cast<float4*>(a.mom + (size_t)p * wsz + e);
      float4 m = *mp;
      m.x = a.beta * m.x + g.x; m.y = a.beta * m.y + g.y; m.z = a.beta * m.z + g.z; m.w = a.beta * m.w + g.w;
      *mp = m;
      if (!a.mom_only) { w.x = wc.x - m.x; w.y = wc.y - m.y; w.z = wc.z - m.z; w.w = wc.w - m.w; }
    }
  }
  *reinterpret_cast<float4*>(a.next + (size_t)p * wsz + e) = w;
  if (a.out[i]) *reinterpret_cast<float4*>(a.out[i] + (size_t)pb.row(p) * pb.msz + o) = w;
}

// Update from the MFMA gradient kernel's stream-K partials, which are stored in
// its register order (sk_part_elem: float4 j holds four consecutive rows of
// one column).  Thread = one float4 of the partial: it sums that float4 over
// the pair's slots (coalesced reads, slots in workgroup order).  The 256
// float4s of a workgroup cover a block of whole matrix row segments
// (sk_update_block: W1 rows 16 cb0 .. + 64/NHB, columns qq HP .. + HP; W2 16
// whole rows).  The sums go through an LDS copy of that block, so that W_cur,
// the momentum, the next state and W_out are read and written as float4s
// along the rows (a direct store of the register order writes 64-byte pieces
// of 4 rows per instruction).  The arithmetic, and so the result, is that of
// the element-wise update.  Both index maps are pinned on the host.
// grid = (D*HID/2 / 256, P).
template <int HID, int HP>
__global__ void __launch_bounds__(256) k_update_streamk(Problem pb, UpdateArgs a) {
  constexpr int D = 64, NHB = HP / 16, HALF = D * HID / 4;   // float4s per matrix
  static_assert(HALF % 256 == 0 && HP == HID / 4, "a workgroup's float4s lie in one matrix");
  constexpr int LD0 = HP + 4, LD1 = D + 4;                  // LDS row strides (floats) of the W1 / W2 blocks
  constexpr int TILE = (64 / NHB) * LD0 > 16 * LD1 ? (64 / NHB) * LD0 : 16 * LD1;
  __shared__ __attribute__((aligned(16))) float tile[TILE];
  const int p = blockIdx.y;
  const int b = p / pb.H, h = p % pb.H;
  const int j = (int)blockIdx.x * 256 + (int)threadIdx.x;   // float4 of the partial
  const SkBlock blk = sk_update_block(HID, (int)blockIdx.x); // uniform
  const SkElem el = sk_part_elem(HID, j);
  const int mat = blk.mat;
  const int lrw = el.row - blk.row0, lcw = el.col - blk.col0;   // this thread's sums: rows lrw + 0..3, column lcw
  const int LD = mat == 0 ? LD0 : LD1;
  // this thread's float4 of the block in row order
  const int lr = (int)threadIdx.x / (blk.cols / 4), lc = 4 * ((int)threadIdx.x % (blk.cols / 4));
  const int e = (blk.row0 + lr) * blk.rs + blk.col0 + lc;
  const float* cur = a.cur.mat(mat, b, h);
  float* out = a.out[mat] ? a.out[mat] + (size_t)pb.row(p) * D * HID : nullptr;
  // W_cur first, so that its load overlaps the partials'
  const bool v4 = ((reinterpret_cast<uintptr_t>(cur) | reinterpret_cast<uintptr_t>(out)) & 15) == 0;   // uniform
  float wc[4];
  if (v4) {
    const float4 t = *reinterpret_cast<const float4*>(cur + e);
    wc[0] = t.x; wc[1] = t.y; wc[2] = t.z; wc[3] = t.w;
  } else {
#pragma unroll
    for (int i = 0; i < 4; ++i) wc[i] = cur[e + i];
  }
  const bool upd = (a.mask >> mat) & 1u;
  long long q0, q1, C;
  sk_range(a, pb.B * pb.H, p, q0, q1, C);
  if (a.sk_direct && q0 == q1) return;   // one workgroup held the whole pair and wrote its step (uniform)
  if (!upd) q1 = q0 - 1;          // a matrix outside the mask keeps W_cur
  // the pair's slots, four loads in flight at a time, added in workgroup order
  const long long wsz = 2LL * D * HID;
  float4 sum = {0.f, 0.f, 0.f, 0.f};
  for (long long q = q0; q <= q1; q += 4) {
    float4 d[4];
#pragma unroll
    for (int u = 0; u < 4; ++u)
      if (q + u <= q1) d[u] = reinterpret_cast<const float4*>(a.part + slot_of(a, p, q + u, q0, C) * wsz)[j];
#pragma unroll
    for (int u = 0; u < 4; ++u)
      if (q + u <= q1) { sum.x += d[u].x; sum.y += d[u].y; sum.z += d[u].z; sum.w += d[u].w; }
  }
  tile[(lrw + 0) * LD + lcw] = sum.x;
  tile[(lrw + 1) * LD + lcw] = sum.y;
  tile[(lrw + 2) * LD + lcw] = sum.z;
  tile[(lrw + 3) * LD + lcw] = sum.w;
  __syncthreads();
  const float4 s = *reinterpret_cast<const float4*>(&tile[lr * LD + lc]);
  const float s4[4] = {s.x, s.y, s.z, s.w};
  float* nxt = a.next + (size_t)p * wsz + (size_t)mat * D * HID;
  float* mom = (upd && a.rule != RULE_GD) ? a.mom + (size_t)p * wsz + (size_t)mat * D * HID : nullptr;
  float w[4];
  if (mom) {
    const float4 t = *reinterpret_cast<const float4*>(mom + e);
    const float m4[4] = {a.beta * t.x + s4[0], a.beta * t.y + s4[1], a.beta * t.z + s4[2], a.beta * t.w + s4[3]};
    *reinterpret_cast<float4*>(mom + e) = float4{m4[0], m4[1], m4[2], m4[3]};
#pragma unroll
    for (int i = 0; i < 4; ++i) w[i] = a.mom_only ? wc[i] : wc[i] - m4[i];
  } else {
#pragma unroll
    for (int i = 0; i < 4; ++i) w[i] = wc[i] - s4[i];
  }
  *reinterpret_cast<float4*>(nxt + e) = float4{w[0], w[1], w[2], w[3]};
  if (out) {
    if (v4) {
      *reinterpret_cast<float4*>(out + e) = float4{w[0], w[1], w[2], w[3]};
    } else {
#pragma unroll
      for (int i = 0; i < 4; ++i) out[e + i] = w[i];
    }
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
  // the register block's loads are issued together: row and column are
  // clamped into the matrix and the out-of-range values are masked after the
  // loads, so no load sits under its own branch (a wait after each of them)
  const int jc = live ? j : cols - 1;
  float v[RMAX], v0[RMAX];
#pragma unroll
  for (int k = 0; k < RMAX; ++k) {
    const int r = lane + kRLanes * k;
    const size_t e = (size_t)(r < rows ? r : rows - 1) * cols + jc;
    v[k] = nxt[e];
    v0[k] = w0[e];
  }
  float nn = 0.f, nr = 0.f;
#pragma unroll
  for (int k = 0; k < RMAX; ++k) {
    const bool in = live && lane + kRLanes * k < rows;
    v[k] = in ? v[k] : 0.f;
    const float w0v = in ? v0[k] : 0.f;
    nn += v[k] * v[k];
    nr += w0v * w0v;
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
  // matrices outside the update mask kept W_cur, whose columns already have
  // W0's norms: they are only copied to W_out
  const float scale = ((a.mask >> i) & 1u) ? sqrtf(sr) / fmaxf(sqrtf(sn), 1e-12f) : 1.0f;
  float* out = a.out[i] ? a.out[i] + (size_t)pb.row(p) * pb.msz : nullptr;
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

}  // namespace

void launch_renorm(const Problem& pb, const UpdateArgs& a, hipStream_t st) {
  const int P = pb.B * pb.H;
  const int side = pb.inner == INNER_LINEAR ? pb.d : (pb.hid > pb.d ? pb.hid : pb.d);   // max rows, max cols
  dim3 g((side + kRCols - 1) / kRCols, pb.nm, P);
  if (side <= 2 * kRLanes) hipLaunchKernelGGL(k_renorm<2>, g, dim3(kRCols * kRLanes), 0, st, pb, a);
  else if (side <= 4 * kRLanes) hipLaunchKernelGGL(k_renorm<4>, g, dim3(kRCols * kRLanes), 0, st, pb, a);
  else hipLaunchKernelGGL(k_renorm<8>, g, dim3(kRCols * kRLanes), 0, st, pb, a);
}

namespace {

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
  const bool upd = (a.mask >> i) & 1u;
  const bool gd = a.rule == RULE_GD;
  float* mom = (upd && !gd) ? a.mom + (size_t)p * wsz + (size_t)i * pb.msz : nullptr;
  float nn = 0.f, nr = 0.f;
  if (live)
    for (int r = lane; r < rows; r += kLanes) {
      const size_t e = (size_t)r * cols + j;
      const float wc = cur[e];
      float w = wc, g = 0.f;
      if (upd) {
        if (a.part_mode == PART_SPLITS) {
          const float* pp = a.part + (size_t)p * wsz + (size_t)i * pb.msz + e;
          for (int s = 0; s < a.S; ++s) {
            if (gd) w -= pp[s * a.part_pair_stride];
            else g += pp[s * a.part_pair_stride];
          }
        } else {
          for (long long q = q0; q <= q1; ++q) {
            const float d = a.part[slot_of(a, p, q, q0, C) * wsz + (size_t)i * pb.msz + e];
            if (gd) w -= d;
            else g += d;
          }
        }
      }
      if (mom) {
        const float m = a.beta * mom[e] + g;
        mom[e] = m;
        if (!a.mom_only) w = wc - m;
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
  const float scale = (a.renorm && upd) ? sqrtf(sr) / fmaxf(sqrtf(sn), 1e-12f) : 1.f;
  if (!live) return;
  float* out = a.out[i] ? a.out[i] + (size_t)pb.row(p) * pb.msz : nullptr;
  for (int r = lane; r < rows; r += kLanes) {
    const size_t e = (size_t)r * cols + j;
    const float w = nxt[e] * scale;
    nxt[e] = w;
    if (out) out[e] = w;
  }
}

}  // namespace

void launch_update(const Problem& pb, const UpdateArgs& a_in, hipStream_t st) {
  const int P = pb.B * pb.H;
  UpdateArgs a = a_in;
  if (a.mom_only) {               // Muon: only M is updated here; the step, re-norm and W_out follow
    a.renorm = 0;
    for (int i = 0; i < 3; ++i) a.out[i] = nullptr;
  }
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
    dim3 grid((unsigned)((wsz / 4 + 63) / 64), P);
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
  const int maxcols = pb.inner == INNER_LINEAR ? pb.d
                    : pb.inner == INNER_DWCONV ? pb.ck * pb.ck
                    : (pb.hid > pb.d ? pb.hid : pb.d);
  dim3 grid((maxcols + kCols - 1) / kCols, pb.nm, P);
  hipLaunchKernelGGL(k_update_renorm, grid, dim3(kCols * kLanes), 0, st, pb, a);
}

}  // namespace ttt
