// Measurement helpers for bench.py (not part of the TTT library):
//  - an MFMA peak micro-benchmark: every wave issues long chains of
//    independent v_mfma_f32_32x32x16_bf16 with no memory traffic, so the
//    achieved rate is the chip's bf16 matrix-core throughput at the clock it
//    sustains under that load (measured: the 32x32x16 form reaches it with 4
//    chains per wave; 16x16x32 needs 16 chains to come within 15 % of it);
//  - a shader-clock probe: one wave reads the shader cycle counter
//    (s_memtime) and the constant 100 MHz counter (s_memrealtime) around a
//    busy loop; their ratio is the shader clock at that moment;
//  - an MFMA / VALU overlap probe: per iteration a wave issues 16
//    v_mfma_f32_16x16x32_bf16 on 16 independent accumulators and/or NV
//    packed-f16 FMAs on 8 independent chains, either in the same wave or split
//    over two waves of a SIMD (even waves MFMA, odd waves VALU); no memory
//    traffic.  Comparing the times shows how much VALU work hides under the
//    matrix cores.
#include <hip/hip_runtime.h>

typedef __attribute__((__vector_size__(8 * sizeof(__bf16)))) __bf16 bf16x8;
typedef __attribute__((__vector_size__(16 * sizeof(float)))) float f32x16;

constexpr int kChains = 4;

__global__ void __launch_bounds__(256) k_mfma_peak(int iters, float* __restrict__ sink,
                                                   unsigned long long* __restrict__ clk) {
  const unsigned long long c0 = __builtin_amdgcn_s_memtime(), r0 = __builtin_amdgcn_s_memrealtime();
  bf16x8 a, b;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    a[i] = (__bf16)(1e-3f * (threadIdx.x + i));
    b[i] = (__bf16)(1e-3f * (blockIdx.x + i));
  }
  f32x16 acc[kChains];
#pragma unroll
  for (int c = 0; c < kChains; ++c)
#pragma unroll
    for (int j = 0; j < 16; ++j) acc[c][j] = 0.f;
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int c = 0; c < kChains; ++c) acc[c] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, acc[c], 0, 0, 0);
  }
  float s = 0.f;
#pragma unroll
  for (int c = 0; c < kChains; ++c)
#pragma unroll
    for (int j = 0; j < 16; ++j) s += acc[c][j];
  if (s == 12345.f) sink[blockIdx.x * 256 + threadIdx.x] = s;   // keeps the chains alive
  if (blockIdx.x == 0 && threadIdx.x == 0) {    // shader clock while this block ran
    clk[0] = __builtin_amdgcn_s_memtime() - c0;
    clk[1] = __builtin_amdgcn_s_memrealtime() - r0;
  }
}

__global__ void k_clock_probe(int spins, unsigned long long* __restrict__ out) {
  const unsigned long long c0 = __builtin_amdgcn_s_memtime();
  const unsigned long long r0 = __builtin_amdgcn_s_memrealtime();
  float x = (float)threadIdx.x;
  for (int i = 0; i < spins; ++i) x = __builtin_fmaf(x, 0.999f, 0.5f);
  const unsigned long long c1 = __builtin_amdgcn_s_memtime();
  const unsigned long long r1 = __builtin_amdgcn_s_memrealtime();
  if (threadIdx.x == 0) {
    out[0] = c1 - c0;
    out[1] = r1 - r0;
    out[2] = (unsigned long long)(x == 1.2345f);
  }
}

typedef _Float16 h2v __attribute__((ext_vector_type(2)));
typedef float f32x4v __attribute__((ext_vector_type(4)));

// MODE 0: MFMA only; 1: VALU only; 2: both in each wave; 3: even waves MFMA,
// odd waves VALU.  NV packed FMAs per iteration.
template <int MODE, int NV>
__global__ void __launch_bounds__(512) k_overlap(int iters, float* __restrict__ sink) {
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  bf16x8 a, b;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    a[i] = (__bf16)(1e-3f * (lane + i));
    b[i] = (__bf16)(2e-3f * (lane - i));
  }
  f32x4v c[16];
#pragma unroll
  for (int j = 0; j < 16; ++j) c[j] = f32x4v{0.f, 0.f, 0.f, 0.f};
  h2v x[8];
  const h2v m = h2v{(_Float16)0.999f, (_Float16)0.999f}, add = h2v{(_Float16)0.001f, (_Float16)0.001f};
#pragma unroll
  for (int j = 0; j < 8; ++j) x[j] = h2v{(_Float16)(0.01f * j), (_Float16)(0.02f * lane)};
  const bool do_m = MODE == 0 || MODE == 2 || (MODE == 3 && (wv & 1) == 0);
  const bool do_v = MODE == 1 || MODE == 2 || (MODE == 3 && (wv & 1) == 1);
  for (int it = 0; it < iters; ++it) {
    if (do_m) {
#pragma unroll
      for (int j = 0; j < 16; ++j) c[j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c[j], 0, 0, 0);
    }
    if (do_v) {
#pragma unroll
      for (int u = 0; u < NV / 8; ++u)
#pragma unroll
        for (int j = 0; j < 8; ++j) x[j] = __builtin_elementwise_fma(x[j], m, add);
    }
  }
  float s = 0.f;
#pragma unroll
  for (int j = 0; j < 16; ++j) s += c[j][0] + c[j][1] + c[j][2] + c[j][3];
#pragma unroll
  for (int j = 0; j < 8; ++j) s += (float)x[j][0] + (float)x[j][1];
  if (s == 12345.f) sink[blockIdx.x * blockDim.x + threadIdx.x] = s;   // keeps the chains alive
}

extern "C" {

// One overlap-probe launch: case 0..6 = (waves per SIMD, mode, NV)
//   0: 1, MFMA only          1: 1, VALU only (NV 64)     2: 1, both (NV 32)
//   3: 1, both (NV 64)       4: 2, MFMA only             5: 2, split MFMA | VALU (NV 64)
//   6: 2, both (NV 64)
// blocks = CUs; threads = 256 per wave per SIMD.  sink: blocks * 512 floats.
int bench_overlap_launch(int which, int blocks, int iters, float* sink, void* stream) {
  hipStream_t st = (hipStream_t)stream;
  switch (which) {
    case 0: hipLaunchKernelGGL((k_overlap<0, 64>), dim3(blocks), dim3(256), 0, st, iters, sink); break;
    case 1: hipLaunchKernelGGL((k_overlap<1, 64>), dim3(blocks), dim3(256), 0, st, iters, sink); break;
    case 2: hipLaunchKernelGGL((k_overlap<2, 32>), dim3(blocks), dim3(256), 0, st, iters, sink); break;
    case 3: hipLaunchKernelGGL((k_overlap<2, 64>), dim3(blocks), dim3(256), 0, st, iters, sink); break;
    case 4: hipLaunchKernelGGL((k_overlap<0, 64>), dim3(blocks), dim3(512), 0, st, iters, sink); break;
    case 5: hipLaunchKernelGGL((k_overlap<3, 64>), dim3(blocks), dim3(512), 0, st, iters, sink); break;
    default: hipLaunchKernelGGL((k_overlap<2, 64>), dim3(blocks), dim3(512), 0, st, iters, sink); break;
  }
  return (int)hipGetLastError();
}

// flops of one k_mfma_peak launch: blocks * 4 waves * iters * chains * 32*32*16*2
double bench_mfma_peak_flops(int blocks, int iters) {
  return (double)blocks * 4.0 * iters * kChains * 32.0 * 32.0 * 16.0 * 2.0;
}

// clk: 2 device uint64 (shader cycles and 100 MHz ticks of block 0)
int bench_mfma_peak_launch(int blocks, int iters, float* sink, unsigned long long* clk, void* stream) {
  hipLaunchKernelGGL(k_mfma_peak, dim3(blocks), dim3(256), 0, (hipStream_t)stream, iters, sink, clk);
  return (int)hipGetLastError();
}

// out: 3 device uint64 (shader cycles, 100 MHz ticks, unused)
int bench_clock_probe_launch(int spins, unsigned long long* out, void* stream) {
  hipLaunchKernelGGL(k_clock_probe, dim3(1), dim3(64), 0, (hipStream_t)stream, spins, out);
  return (int)hipGetLastError();
}

}
