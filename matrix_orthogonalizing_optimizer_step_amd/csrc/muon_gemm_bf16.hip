// The MFMA GEMM kernels with bf16 operands, one per epilogue kind.
#include "muon_gemm_mfma.h"

namespace muon {

hipError_t launch_gemm_bf16(const GemmArgs& a, int batch, int kind, hipStream_t s) {
  return launch_gemm_mfma<kOpBF16>(a, batch, kind, s);
}

}  // namespace muon
