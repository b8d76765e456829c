// GEMM instantiations for the NT operand layout (see gemm_impl.hpp).
#include "gemm_impl.hpp"

namespace ttt {

hipError_t gemm_nt(DT dt, Epi e, int cfg, const GemmArgs& g, hipStream_t st) {
  if (g.B2) {
    // two-term split of B (fast weights) in the forward products
    if (dt != DT::BF16) return hipErrorInvalidValue;
    const int c = cfg;
    if (e == Epi::SWIGLU) return gemm_cfg<bf16, true, true, (int)Epi::SWIGLU, true>(c, g, st);
    if (e == Epi::ADD_F32) return gemm_cfg<bf16, true, true, (int)Epi::ADD_F32, true>(c, g, st);
    if (e == Epi::PARTIAL) return gemm_cfg<bf16, true, true, (int)Epi::PARTIAL, true>(c, g, st);
    if (e == Epi::PARTIAL_BF16) return gemm_cfg<bf16, true, true, (int)Epi::PARTIAL_BF16, true>(c, g, st);
    return hipErrorInvalidValue;
  }
  if (dt == DT::BF16 && e == Epi::PARTIAL_BF16)
    return gemm_cfg<bf16, true, true, (int)Epi::PARTIAL_BF16, false>(cfg, g, st);
  if (dt == DT::BF16 && e == Epi::STORE_F32_LSE)
    return gemm_cfg<bf16, true, true, (int)Epi::STORE_F32_LSE, false>(cfg, g, st);
  if (dt == DT::BF16) return gemm_by_epi<bf16, true, true>(e, cfg, g, st);
  return gemm_by_epi<float, true, true>(e, cfg, g, st);
}

}  // namespace ttt
