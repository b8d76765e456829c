// GEMM dispatch: picks the operand-layout instantiation and a tile
// configuration for the shape (see gemm_impl.hpp for the kernel).
#include "gemm_impl.hpp"

namespace ttt {

int gemm_k_granule(DT) { return 64; }

// Tile choice from measured sweeps at the 3B shapes: 256 x 256 tiles (8
// waves) once there are enough of them to cover the CUs; 128 x 128 for the
// rest and for the short-K dW products (whose epilogue dominates).
int gemm_pick_cfg(DT dt, bool ak, bool bk, const GemmArgs& g) {
  if (dt != DT::BF16) return 0;
  const long splits = g.kchunk > 0 ? (g.K + g.kchunk - 1) / g.kchunk : 1;
  const long nb = g.batch > 1 ? g.batch : 1;
  auto tiles = [&](int bm, int bn) { return ((g.M + bm - 1) / bm) * (long)((g.N + bn - 1) / bn) * splits * nb; };
  if (ak && bk) return tiles(256, 256) >= 256 ? 5 : 1;
  if (ak) return tiles(256, 256) >= 192 ? 5 : 1;
  return 1;
}

hipError_t gemm(DT dt, bool a_kmajor, bool b_kmajor, Epi epi, const GemmArgs& g, hipStream_t st) {
  if (g.M <= 0 || g.N <= 0) return hipSuccess;
  const int cfg = g.tile > 0 ? g.tile : gemm_pick_cfg(dt, a_kmajor, b_kmajor, g);
  if (a_kmajor && b_kmajor) return gemm_nt(dt, epi, cfg, g, st);
  if (a_kmajor) return gemm_nn(dt, epi, cfg, g, st);
  if (!b_kmajor) return gemm_tn(dt, epi, cfg, g, st);
  return gemm_tt(dt, epi, cfg, g, st);
}

}  // namespace ttt
