// GEMM instantiations for the NN operand layout (see gemm_impl.hpp).
#include "gemm_impl.hpp"

namespace ttt {

hipError_t gemm_nn(DT dt, Epi e, int cfg, const GemmArgs& g, hipStream_t st) {
  if (dt == DT::BF16) {
    if (e == Epi::PARTIAL_BF16) return gemm_cfg<bf16, true, false, (int)Epi::PARTIAL_BF16, false>(cfg, g, st);
    return gemm_by_epi<bf16, true, false>(e, cfg, g, st);
  }
  return gemm_by_epi<float, true, false>(e, cfg, g, st);
}

}  // namespace ttt
