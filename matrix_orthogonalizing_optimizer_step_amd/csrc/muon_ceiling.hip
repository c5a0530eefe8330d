// The 16-bit MFMA rate this device sustains with no memory traffic at all:
// every wave issues v_mfma_f32_32x32x16_{f16,bf16} back to back on eight
// register accumulators, with operands drawn once from a hash so that the data
// switch the way real operands do.  Under a full MFMA load the clock is set by
// the power the datapath draws, and that depends on the data: with random
// operands the clock settles far below its nominal value, with a zero operand
// it runs close to it, and bf16 operands (fewer mantissa bits) draw less than
// fp16.  A profiling aid: this is the practical ceiling the GEMMs of each
// operand type are held to, beside the dense peak at the nominal clock.
#include <hip/hip_runtime.h>

#include "../../include/muon.h"

namespace {

typedef _Float16 f16x8_t __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));

constexpr int kCeilThreads = 256;
constexpr int kCeilAcc = 8;

// The next hashed value in [-1, 1) with 10 random bits.
__device__ __forceinline__ float next_value(unsigned& h) {
  h = h * 1664525u + 1013904223u;
  return static_cast<float>((h >> 16) & 2047u) * (1.0f / 1024.0f) - 1.0f;
}

template <typename V>
__device__ __forceinline__ f32x16_t mfma(const V& a, const V& b, const f32x16_t& c) {
  if constexpr (__is_same(V, f16x8_t)) {
    return __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b, c, 0, 0, 0);
  } else {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
  }
}

template <typename V, typename E>
__device__ __forceinline__ void mfma_ceiling_body(float* sink, int rounds) {
  V a[4], b[4];
  unsigned h = threadIdx.x * 2654435761u + blockIdx.x * 40503u + 12345u;
  for (int j = 0; j < 4; ++j)
    for (int i = 0; i < 8; ++i) {
      a[j][i] = static_cast<E>(next_value(h));
      b[j][i] = static_cast<E>(next_value(h));
    }
  f32x16_t acc[kCeilAcc];
  for (int k = 0; k < kCeilAcc; ++k)
    for (int r = 0; r < 16; ++r) acc[k][r] = 0.0f;
  for (int it = 0; it < rounds; ++it) {
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int k = 0; k < kCeilAcc; ++k) acc[k] = mfma<V>(a[j], b[(j + k) & 3], acc[k]);
  }
  float s = 0.0f;
  for (int k = 0; k < kCeilAcc; ++k)
    for (int r = 0; r < 16; ++r) s += acc[k][r];
  sink[static_cast<size_t>(blockIdx.x) * kCeilThreads + threadIdx.x] = s;  // keeps the products live
}

__global__ __launch_bounds__(kCeilThreads) void mfma_ceiling_f16_kernel(float* sink, int rounds) {
  mfma_ceiling_body<f16x8_t, _Float16>(sink, rounds);
}

__global__ __launch_bounds__(kCeilThreads) void mfma_ceiling_bf16_kernel(float* sink, int rounds) {
  mfma_ceiling_body<bf16x8_t, __bf16>(sink, rounds);
}

}  // namespace

extern "C" muon_status muon_mfma_ceiling(int blocks, int rounds, muon_dtype dtype, float* sink, void* stream) {
  if (blocks < 1 || blocks > (1 << 20) || rounds < 1 || sink == nullptr) return MUON_ERR_INVALID_ARG;
  if (dtype != MUON_F16 && dtype != MUON_BF16) return MUON_ERR_INVALID_ARG;
  const hipStream_t s = static_cast<hipStream_t>(stream);
  if (dtype == MUON_F16) {
    hipLaunchKernelGGL(mfma_ceiling_f16_kernel, dim3(blocks), dim3(kCeilThreads), 0, s, sink, rounds);
  } else {
    hipLaunchKernelGGL(mfma_ceiling_bf16_kernel, dim3(blocks), dim3(kCeilThreads), 0, s, sink, rounds);
  }
  return hipGetLastError() == hipSuccess ? MUON_OK : MUON_ERR_HIP;
}
