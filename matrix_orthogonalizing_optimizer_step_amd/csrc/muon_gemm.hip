// Host side of the GEMM: which kernel and epilogue a launch needs.
#include "muon_internal.h"

namespace muon {

int gemm_tile(int op) { return op == kOpF32 ? kCheckTile : kMfmaTile; }

int epi_kind(const GemmArgs& g) {
  const bool e16 = g.E16 != nullptr, q = g.q16 != nullptr;
  if (g.final_mode) {
    if (g.sym || q || g.out16 != nullptr || g.outT16 != nullptr || g.part_out != nullptr) return -1;
    return e16 ? kEpiFinE16 : kEpiFin;
  }
  if (g.out16 == nullptr) return -1;
  if (g.sym) {
    if (g.outT16 != nullptr) return -1;
    if (q) return e16 ? kEpiSymE16Q : -1;  // a fresh Q comes with Z' only
    return e16 ? kEpiSymE16 : kEpiSym;
  }
  // general products write X and X^T and have no diagonal term
  if (g.outT16 == nullptr || q || g.part_out != nullptr) return -1;
  if (g.gamma_c != 0.0f || g.gamma_a != 0.0f) return -1;
  return e16 ? kEpiGenE16 : kEpiGen;
}

hipError_t launch_gemm(const GemmArgs& a, int batch, int op, hipStream_t s) {
  if (op == kOpF32) return launch_gemm_f32(a, batch, s);
  const int kind = epi_kind(a);
  if (kind < 0) return hipErrorInvalidValue;
  return op == kOpBF16 ? launch_gemm_bf16(a, batch, kind, s) : launch_gemm_f16(a, batch, kind, s);
}

}  // namespace muon
