// The MFMA GEMM kernels with f16 operands, one per epilogue kind.
#include "muon_gemm_mfma.h"

namespace muon {

hipError_t launch_gemm_f16(const GemmArgs& a, int batch, int kind, hipStream_t s) {
  return launch_gemm_mfma<kOpF16>(a, batch, kind, s);
}

}  // namespace muon
