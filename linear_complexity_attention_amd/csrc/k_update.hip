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
// Besides the fp32 state the kernel can emit the caller's W_out and a bf16
// copy laid out for the MFMA kernels (see bf16_index below).
#include "ttt_internal.h"

namespace ttt {

namespace {

constexpr int kCols = 64;
constexpr int kLanes = 4;

// bf16 operand layouts:
//   BF_ROWMAJOR   : [in][out] like the fp32 matrix
//   BF_TRANSPOSED : [out][in]
//   BF_MLP3       : GELU-MLP MFMA operands, per pair [W1^T (h x d) | W2 (h x d) | W2^T (d x h)]
__device__ __forceinline__ long long bf16_index(int layout, int r, int c, int rows, int cols) {
  return layout == BF_TRANSPOSED ? (long long)c * rows + r : (long long)r * cols + c;
}

__device__ __forceinline__ void store_bf(bf16* pair_base, int layout, int i, long long msz, int r, int c,
                                         int rows, int cols, float w) {
  const bf16 v = (bf16)w;
  if (layout == BF_MLP3) {
    if (i == 0) pair_base[(long long)c * rows + r] = v;            // W1^T [h][d]
    else {
      pair_base[msz + (long long)r * cols + c] = v;                 // W2   [h][d]
      pair_base[2 * msz + (long long)c * rows + r] = v;             // W2^T [d][h]
    }
    return;
  }
  pair_base[i * msz + bf16_index(layout, r, c, rows, cols)] = v;
}

__device__ __forceinline__ int bf_pair_mats(int layout, int nm) { return layout == BF_MLP3 ? 3 : nm; }

__device__ __forceinline__ void mat_dims(const Problem& pb, int i, int& rows, int& cols) {
  if (pb.inner == INNER_LINEAR) { rows = pb.d; cols = pb.d; return; }
  if (i == 1) { rows = pb.hid; cols = pb.d; }   // W2 [h, d]
  else { rows = pb.d; cols = pb.hid; }          // W1, W3 [d, h]
}

// grid = (column blocks, nm, P); thread = (column, row lane)
__global__ void __launch_bounds__(kCols * kLanes) k_update(Problem pb, UpdateArgs a) {
  const int i = blockIdx.y, p = blockIdx.z;
  const int b = p / pb.H, h = p % pb.H;
  int rows, cols;
  mat_dims(pb, i, rows, cols);
  const int j = blockIdx.x * kCols + threadIdx.x % kCols;
  const int lane = threadIdx.x / kCols;
  const bool live = j < cols;
  const float* cur = a.cur.mat(i, b, h);
  const float* w0 = a.w0.mat(i, b, h);
  float* nxt = a.next + ((size_t)p * pb.nm + i) * pb.msz;
  // stream-K: workgroups [wg0, wg1] of the gradient kernel touched pair p
  long long wg0 = 0, wg1 = -1, sk_total = 0;
  if (a.part_mode == PART_STREAMK) {
    sk_total = (long long)pb.B * pb.H * a.sk_tpp;
    const long long xa = (long long)p * a.sk_tpp, xb = xa + a.sk_tpp - 1;
    wg0 = ((xa + 1) * a.sk_G - 1) / sk_total;
    wg1 = ((xb + 1) * a.sk_G - 1) / sk_total;
  }
  __shared__ float red[2][kLanes][kCols];
  float nn = 0.f, nr = 0.f;
  if (live)
    for (int r = lane; r < rows; r += kLanes) {
      const size_t e = (size_t)r * cols + j;
      float w = cur[e];
      if (a.part) {
        if (a.part_mode == PART_SPLITS) {
          const float* pp = a.part + (size_t)p * pb.nm * pb.msz + (size_t)i * pb.msz;
          for (int s = 0; s < a.S; ++s) w -= pp[s * a.part_pair_stride + e];
        } else {
          for (long long q = wg0; q <= wg1; ++q) {
            const long long first = ((q * sk_total) / a.sk_G) / a.sk_tpp;
            const float* pp = a.part + (q * a.sk_J + (p - first)) * pb.nm * pb.msz + (size_t)i * pb.msz;
            w -= pp[e];
          }
        }
      }
      nxt[e] = w;
      nn += w * w;
      const float w0v = w0[e];
      nr += w0v * w0v;
    }
  float scale = 1.f;
  if (a.renorm) {
    red[0][lane][threadIdx.x % kCols] = nn;
    red[1][lane][threadIdx.x % kCols] = nr;
    __syncthreads();
    float sn = 0.f, sr = 0.f;
    for (int l = 0; l < kLanes; ++l) { sn += red[0][l][threadIdx.x % kCols]; sr += red[1][l][threadIdx.x % kCols]; }
    scale = sqrtf(sr) / fmaxf(sqrtf(sn), 1e-12f);
  }
  if (!live) return;
  float* out = a.out[i] ? a.out[i] + (size_t)p * pb.msz : nullptr;
  bf16* bfo = a.bf ? a.bf + (size_t)p * bf_pair_mats(a.bf_layout, pb.nm) * pb.msz : nullptr;
  for (int r = lane; r < rows; r += kLanes) {
    const size_t e = (size_t)r * cols + j;
    float w = nxt[e];
    if (a.renorm) { w *= scale; nxt[e] = w; }
    if (out) out[e] = w;
    if (bfo) store_bf(bfo, a.bf_layout, i, pb.msz, r, j, rows, cols, w);
  }
}

__global__ void __launch_bounds__(256) k_convert_bf16(Problem pb, WRef W, bf16* dst, int layout) {
  const int i = blockIdx.y, p = blockIdx.z;
  const int b = p / pb.H, h = p % pb.H;
  int rows, cols;
  mat_dims(pb, i, rows, cols);
  const float* src = W.mat(i, b, h);
  bf16* o = dst + (size_t)p * bf_pair_mats(layout, pb.nm) * pb.msz;
  for (long long e = blockIdx.x * 256 + threadIdx.x; e < (long long)rows * cols; e += (long long)gridDim.x * 256) {
    const int r = (int)(e / cols), c = (int)(e % cols);
    store_bf(o, layout, i, pb.msz, r, c, rows, cols, src[e]);
  }
}

}  // namespace

void launch_update(const Problem& pb, const UpdateArgs& a, hipStream_t st) {
  const int maxcols = pb.inner == INNER_LINEAR ? pb.d : (pb.hid > pb.d ? pb.hid : pb.d);
  dim3 grid((maxcols + kCols - 1) / kCols, pb.nm, pb.B * pb.H);
  hipLaunchKernelGGL(k_update, grid, dim3(kCols * kLanes), 0, st, pb, a);
}

void launch_convert_bf16(const Problem& pb, const WRef& W, bf16* dst, int layout, hipStream_t st) {
  dim3 grid(8, pb.nm, pb.B * pb.H);
  hipLaunchKernelGGL(k_convert_bf16, grid, dim3(256), 0, st, pb, W, dst, layout);
}

}  // namespace ttt
