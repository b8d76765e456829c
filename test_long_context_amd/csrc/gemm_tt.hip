// GEMM instantiations for the TT operand layout (see gemm_impl.hpp).
#include "gemm_impl.hpp"

namespace ttt {

hipError_t gemm_tt(DT dt, Epi e, int cfg, const GemmArgs& g, hipStream_t st) {
  if (dt == DT::BF16) return gemm_by_epi<bf16, false, true>(e, cfg, g, st);
  return gemm_by_epi<float, false, true>(e, cfg, g, st);
}

}  // namespace ttt
