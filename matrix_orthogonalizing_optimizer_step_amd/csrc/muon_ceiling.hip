// The 16-bit MFMA rate this device sustains with no memory traffic at all:
// every wave issues v_mfma_f32_32x32x16_f16 back to back on eight register
// accumulators, with operands drawn once from a hash so that the data switch
// the way real operands do (constant operands draw less power and let the
// clock run higher).  A profiling aid: under a full MFMA load the clock is set
// by the power limit, so this is the practical ceiling the GEMMs are held to,
// beside the dense peak at the nominal clock.
#include <hip/hip_runtime.h>

#include "../../include/muon.h"

namespace {

typedef _Float16 f16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));

constexpr int kCeilThreads = 256;
constexpr int kCeilAcc = 8;

__global__ __launch_bounds__(kCeilThreads) void mfma_ceiling_kernel(float* sink, int rounds) {
  f16x8_t a[4], b[4];
  unsigned h = threadIdx.x * 2654435761u + blockIdx.x * 40503u + 12345u;
  for (int j = 0; j < 4; ++j)
    for (int i = 0; i < 8; ++i) {  // values in [-1, 1) with 10 random bits
      h = h * 1664525u + 1013904223u;
      a[j][i] = static_cast<_Float16>(static_cast<float>((h >> 16) & 2047u) * (1.0f / 1024.0f) - 1.0f);
      h = h * 1664525u + 1013904223u;
      b[j][i] = static_cast<_Float16>(static_cast<float>((h >> 16) & 2047u) * (1.0f / 1024.0f) - 1.0f);
    }
  f32x16_t acc[kCeilAcc];
  for (int k = 0; k < kCeilAcc; ++k)
    for (int r = 0; r < 16; ++r) acc[k][r] = 0.0f;
  for (int it = 0; it < rounds; ++it) {
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int k = 0; k < kCeilAcc; ++k)
        acc[k] = __builtin_amdgcn_mfma_f32_32x32x16_f16(a[j], b[(j + k) & 3], acc[k], 0, 0, 0);
  }
  float s = 0.0f;
  for (int k = 0; k < kCeilAcc; ++k)
    for (int r = 0; r < 16; ++r) s += acc[k][r];
  sink[static_cast<size_t>(blockIdx.x) * kCeilThreads + threadIdx.x] = s;  // keeps the products live
}

}  // namespace

extern "C" muon_status muon_mfma_ceiling(int blocks, int rounds, float* sink, void* stream) {
  if (blocks < 1 || blocks > (1 << 20) || rounds < 1 || sink == nullptr) return MUON_ERR_INVALID_ARG;
  hipLaunchKernelGGL(mfma_ceiling_kernel, dim3(blocks), dim3(kCeilThreads), 0, static_cast<hipStream_t>(stream),
                     sink, rounds);
  return hipGetLastError() == hipSuccess ? MUON_OK : MUON_ERR_HIP;
}
