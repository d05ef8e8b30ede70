// Device-side helpers shared by the TTT kernels (gfx950, wave64).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace ttt {

typedef __bf16 bf16;
typedef __attribute__((__vector_size__(8 * sizeof(__bf16)))) __bf16 bf16x8;
typedef __attribute__((__vector_size__(4 * sizeof(__bf16)))) __bf16 bf16x4;
typedef __attribute__((__vector_size__(4 * sizeof(float)))) float f32x4;
typedef __attribute__((__vector_size__(16 * sizeof(float)))) float f32x16;

// Where the fp32 weights of one (b, h) pair live: matrix i of pair (b, h)
// starts at m[i] + b*sb + h*sh.  Covers both the caller's W0 (three separate
// buffers, optionally shared over the batch) and the library's weight states.
struct WRef {
  const float* m[3];
  long long sb, sh;
  __device__ __host__ const float* mat(int i, int b, int h) const { return m[i] + b * sb + h * sh; }
};

template <typename T> __device__ __forceinline__ float to_f32(T x);
template <> __device__ __forceinline__ float to_f32<float>(float x) { return x; }
template <> __device__ __forceinline__ float to_f32<bf16>(bf16 x) { return (float)x; }

template <typename T> __device__ __forceinline__ T from_f32(float x);
template <> __device__ __forceinline__ float from_f32<float>(float x) { return x; }
template <> __device__ __forceinline__ bf16 from_f32<bf16>(float x) { return (bf16)x; }  // RNE

// Exact-erf GELU and its derivative in fp32 (device erff), used wherever fp32
// accuracy matters (generic kernels, the fp32 configuration).
__device__ __forceinline__ float gelu_exact(float z) { return 0.5f * z * (1.0f + erff(z * 0.70710678118654752f)); }
__device__ __forceinline__ float gelu_exact_prime(float z) {
  return 0.5f * (1.0f + erff(z * 0.70710678118654752f)) + z * 0.39894228040143268f * __expf(-0.5f * z * z);
}
__device__ __forceinline__ float sigmoid_f(float z) { return 1.0f / (1.0f + __expf(-z)); }

// Key statistics of one (pair, channel): mean and 1/sqrt(var + eps).
struct KeyStat { float mu, rstd; };

}  // namespace ttt
