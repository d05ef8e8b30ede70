// Measurement helpers for bench.py (not part of the TTT library):
//  - an MFMA peak micro-benchmark: every wave issues long chains of
//    independent v_mfma_f32_32x32x16_bf16 with no memory traffic, so the
//    achieved rate is the chip's bf16 matrix-core throughput at the clock it
//    sustains under that load (measured: the 32x32x16 form reaches it with 4
//    chains per wave; 16x16x32 needs 16 chains to come within 15 % of it);
//  - a shader-clock probe: one wave reads the shader cycle counter
//    (s_memtime) and the constant 100 MHz counter (s_memrealtime) around a
//    busy loop; their ratio is the shader clock at that moment.
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

extern "C" {

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
