// Kernel-level entry points (include/ttt_kernels.h): host-side shape checks,
// then one launch (family) on the caller's stream.
#include <stdint.h>

#include "../../include/ttt_kernels.h"
#include "kernels.hpp"

using namespace ttt;

namespace {
bool al16(const void* p) { return ((uintptr_t)p & 15) == 0; }
bool dt_ok(int32_t d) { return d == TTT_F32 || d == TTT_BF16; }
DT to_dt(int32_t d) { return d == TTT_BF16 ? DT::BF16 : DT::F32; }
}  // namespace

extern "C" ttt_status tttk_gemm(int32_t dtype, int32_t a_kmajor, int32_t b_kmajor, int32_t epi,
                                const void* A, int64_t lda, const void* B, int64_t ldb, const void* B2,
                                int32_t M, int32_t N, int32_t K, void* C, int64_t ldc, void* C2,
                                void* C3, const void* X, float scale, int32_t kchunk, int32_t tile,
                                uint32_t seed, void* stream) {
  if (!dt_ok(dtype) || epi < 0 || (epi > TTTK_EPI_PARTIAL && epi != TTTK_EPI_STORE_F32_LSE) || M < 0 || N < 0 ||
      K < 0)
    return TTT_ERR_INVALID_ARG;
  if (epi == TTTK_EPI_STORE_F32_LSE && (dtype != TTT_BF16 || !a_kmajor || !b_kmajor || !C2 || B2))
    return TTT_ERR_INVALID_ARG;
  if (!A || !B || !C || !al16(A) || !al16(B)) return TTT_ERR_INVALID_ARG;
  if (tile < 0 || tile > 6) return TTT_ERR_INVALID_ARG;
  // contiguous dimensions: K for k-major operands, M / N otherwise
  const int64_t ca = a_kmajor ? K : M, cb = b_kmajor ? K : N;
  if (ca % 8 || cb % 8 || lda % 8 || ldb % 8) return TTT_ERR_UNSUPPORTED;
  if ((a_kmajor ? lda < K : lda < M) || (b_kmajor ? ldb < K : ldb < N)) return TTT_ERR_INVALID_ARG;
  if (epi == TTTK_EPI_SWIGLU && (N % 32 || !C2)) return TTT_ERR_INVALID_ARG;
  if (epi == TTTK_EPI_SWIGLU_BWD && (N % 16 || !X || ldc < 2 * N)) return TTT_ERR_INVALID_ARG;
  if (epi == TTTK_EPI_SGD && !C2) return TTT_ERR_INVALID_ARG;
  if (seed && (epi != TTTK_EPI_SGD || dtype != TTT_BF16 || C3 || C2 == C)) return TTT_ERR_INVALID_ARG;
  if (epi == TTTK_EPI_PARTIAL && kchunk > 0 && kchunk % gemm_k_granule(to_dt(dtype))) return TTT_ERR_INVALID_ARG;
  if (B2 && (dtype != TTT_BF16 || !a_kmajor || !b_kmajor ||
             (epi != TTTK_EPI_SWIGLU && epi != TTTK_EPI_ADD_F32 && epi != TTTK_EPI_PARTIAL) || !al16(B2)))
    return TTT_ERR_INVALID_ARG;
  GemmArgs g{};
  g.A = A;
  g.B = B;
  g.B2 = B2;
  g.M = M;
  g.N = N;
  g.K = K;
  g.lda = lda;
  g.ldb = ldb;
  g.C = C;
  g.ldc = ldc;
  g.C2 = C2;
  g.C3 = C3;
  g.X = X;
  g.scale = scale;
  g.kchunk = epi == TTTK_EPI_PARTIAL ? kchunk : 0;
  g.tile = tile;
  g.seed = seed;
  if (gemm(to_dt(dtype), a_kmajor != 0, b_kmajor != 0, (Epi)epi, g, (hipStream_t)stream) != hipSuccess)
    return TTT_ERR_HIP;
  return TTT_OK;
}

namespace {
ttt_status attn_check(int32_t dtype, int32_t n, int32_t H, int32_t Hk, int32_t dh, int32_t cap,
                      int32_t window, int64_t pos0) {
  if (!dt_ok(dtype) || n < 0 || H < 1 || Hk < 1 || H % Hk || window < 1 || pos0 < 0) return TTT_ERR_INVALID_ARG;
  if (dh != 16 && dh != 64 && dh != 128) return TTT_ERR_UNSUPPORTED;
  if (cap < 64 || (cap & (cap - 1))) return TTT_ERR_UNSUPPORTED;
  // every key a query sees must still be in the store
  if ((int64_t)window + n > (int64_t)cap + 1) return TTT_ERR_UNSUPPORTED;
  return TTT_OK;
}
}  // namespace

namespace {
int fwd_splits(int32_t n, int32_t H, int32_t dh, int32_t window, int32_t ksplit) {
  if (ksplit > 0) return ksplit;
  AttnArgs a{};
  a.n = n;
  a.H = H;
  a.dh = dh;
  a.window = window;
  return attn_fwd2_splits(a);
}
}  // namespace

extern "C" int64_t tttk_attn_fwd_workspace(int32_t n, int32_t H, int32_t dh, int32_t window, int32_t ksplit) {
  if (n <= 0 || H < 1 || ksplit < 0 || ksplit > 4) return 0;
  const int s = fwd_splits(n, H, dh, window, ksplit);
  if (s <= 1) return 0;
  return (int64_t)4 * s * ((int64_t)n * H * dh + 2LL * H * n);
}

extern "C" ttt_status tttk_attn_fwd(int32_t dtype, const void* q, const void* k, const void* v, const void* vt,
                                    void* o, float* lse, int32_t n, int32_t H, int32_t Hk, int32_t dh,
                                    int32_t cap, int32_t window, int64_t pos0, int32_t variant, int32_t ksplit,
                                    void* work, void* stream) {
  ttt_status s = attn_check(dtype, n, H, Hk, dh, cap, window, pos0);
  if (s != TTT_OK) return s;
  if (!q || !k || !v || !o || variant < 0 || variant > 4 || ksplit < 0 || ksplit > 4) return TTT_ERR_INVALID_ARG;
  AttnArgs a{};
  a.q = q;
  a.k = k;
  a.v = v;
  a.o = o;
  a.lse = lse;
  a.n = n;
  a.H = H;
  a.Hk = Hk;
  a.dh = dh;
  a.cap = cap;
  a.window = window;
  a.pos0 = pos0;
  a.scale = 1.f / sqrtf((float)dh);
  a.vt = vt;
  hipError_t e;
  if (variant == 1 || (variant == 0 && !attn_fwd2_supported(to_dt(dtype), a))) {
    e = attn_fwd(to_dt(dtype), a, (hipStream_t)stream);
  } else {
    if (!attn_fwd2_supported(to_dt(dtype), a)) return TTT_ERR_UNSUPPORTED;
    if (!al16(q) || !al16(k) || !al16(v) || !al16(vt) || !al16(o)) return TTT_ERR_INVALID_ARG;
    const int ks = fwd_splits(n, H, dh, window, ksplit);
    if (ks > 1 && n > 0) {
      if (!work || !al16(work)) return TTT_ERR_INVALID_ARG;
      a.ksplit = ks;
      a.opart = (float*)work;
      a.mlpart = a.opart + (long)ks * n * H * dh;
    }
    e = attn_fwd2(to_dt(dtype), a, (hipStream_t)stream, variant == 0 ? 0 : variant - 1);
    if (e == hipSuccess) e = attn_fwd2_combine(a, (hipStream_t)stream);
  }
  return e == hipSuccess ? TTT_OK : TTT_ERR_HIP;
}

namespace {
bool use_bwd2(int32_t dtype, int32_t dh, int32_t variant) {
  return variant == 2 || (variant == 0 && dtype == TTT_BF16 && (dh == 64 || dh == 128));
}
AttnArgs bwd_shape(int32_t n, int32_t H, int32_t Hk, int32_t dh, int32_t window) {
  AttnArgs a{};
  a.n = n;
  a.H = H;
  a.Hk = Hk;
  a.dh = dh;
  a.window = window;
  return a;
}
}  // namespace

extern "C" int64_t tttk_attn_bwd_workspace(int32_t dtype, int32_t n, int32_t H, int32_t Hk, int32_t dh,
                                           int32_t window, int32_t variant) {
  if (n <= 0 || H < 1 || Hk < 1 || H % Hk || !use_bwd2(dtype, dh, variant)) return 0;
  const AttnArgs a = bwd_shape(n, H, Hk, dh, window);
  return (int64_t)4 * n * dh * ((int64_t)attn_bwd2_dq_parts(a) * H + 2LL * attn_bwd2_kv_parts(a) * Hk);
}

extern "C" ttt_status tttk_attn_bwd(int32_t dtype, const void* q, const void* k, const void* v,
                                    const float* lse, const void* dO, const float* D, float* dq, float* dk,
                                    float* dv, int32_t n, int32_t H, int32_t Hk, int32_t dh, int32_t cap,
                                    int32_t window, int64_t pos0, int32_t variant, void* work, void* stream) {
  ttt_status s = attn_check(dtype, n, H, Hk, dh, cap, window, pos0);
  if (s != TTT_OK) return s;
  if (!q || !k || !v || !lse || !dO || !D || !dq || !dk || !dv || variant < 0 || variant > 2)
    return TTT_ERR_INVALID_ARG;
  AttnArgs a{};
  a.q = q;
  a.k = k;
  a.v = v;
  a.lse = (float*)lse;
  a.n = n;
  a.H = H;
  a.Hk = Hk;
  a.dh = dh;
  a.cap = cap;
  a.window = window;
  a.pos0 = pos0;
  a.scale = 1.f / sqrtf((float)dh);
  a.dO = dO;
  a.D = D;
  hipStream_t st = (hipStream_t)stream;
  if (use_bwd2(dtype, dh, variant)) {
    if (!attn_bwd2_supported(to_dt(dtype), a)) return TTT_ERR_UNSUPPORTED;
    if (n == 0) return TTT_OK;
    if (!work || !al16(work)) return TTT_ERR_INVALID_ARG;
    const int qp = attn_bwd2_dq_parts(a), kp = attn_bwd2_kv_parts(a);
    a.kv_fill = true;  // the part sums below add every part of every key
    float* wq = (float*)work;
    float* wk = wq + (long)qp * n * H * dh;
    float* wv = wk + (long)kp * n * Hk * dh;
    a.dq = wq;
    a.dk = wk;
    a.dv = wv;
    if (attn_bwd_dq2(to_dt(dtype), a, st) != hipSuccess) return TTT_ERR_HIP;
    if (attn_bwd_dkdv2(to_dt(dtype), a, st) != hipSuccess) return TTT_ERR_HIP;
    if (sum_parts_f32(wq, qp, (long)n * H * dh, dq, st) != hipSuccess) return TTT_ERR_HIP;
    if (sum_parts_f32(wk, kp, (long)n * Hk * dh, dk, st) != hipSuccess) return TTT_ERR_HIP;
    if (sum_parts_f32(wv, kp, (long)n * Hk * dh, dv, st) != hipSuccess) return TTT_ERR_HIP;
    return TTT_OK;
  }
  a.dq = dq;
  a.dk = dk;
  a.dv = dv;
  if (attn_bwd_dq(to_dt(dtype), a, st) != hipSuccess) return TTT_ERR_HIP;
  if (attn_bwd_dkdv(to_dt(dtype), a, st) != hipSuccess) return TTT_ERR_HIP;
  return TTT_OK;
}

extern "C" ttt_status tttk_ce(int32_t dtype, const float* logits, int32_t n, int32_t nt, int32_t V,
                              const int32_t* labels, float scale, float* loss, void* dz, int* err,
                              void* stream) {
  if (!dt_ok(dtype) || !logits || !labels || !loss || !dz || !err || n < 0 || nt < 0 || nt > n || V < 2)
    return TTT_ERR_INVALID_ARG;
  if (V % 8 || !al16(logits)) return TTT_ERR_UNSUPPORTED;
  return ce_fwd_bwd(to_dt(dtype), logits, n, nt, V, labels, scale, loss, dz, err, (hipStream_t)stream) ==
                 hipSuccess
             ? TTT_OK
             : TTT_ERR_HIP;
}

extern "C" ttt_status tttk_dw_sgd(int32_t nprob, const tttk_dw_problem* probs, int32_t K, float lr, int32_t grid,
                                  void* stream) {
  if (nprob < 1 || nprob > 2 || !probs || K < 0 || grid < 0) return TTT_ERR_INVALID_ARG;
  DwUpdate u[2];
  for (int i = 0; i < nprob; ++i) {
    const tttk_dw_problem& p = probs[i];
    if (!p.A || !p.B || !p.W || !p.Hi || p.M < 1 || p.N < 1) return TTT_ERR_INVALID_ARG;
    u[i] = DwUpdate{p.A, (long)p.lda, p.B, (long)p.ldb, p.W, p.Hi, p.Lo, (long)p.ldw, p.M, p.N};
    if (!dw_sgd_supported(u[i])) return TTT_ERR_UNSUPPORTED;
  }
  return dw_sgd(u, nprob, K, lr, grid, (hipStream_t)stream) == hipSuccess ? TTT_OK : TTT_ERR_HIP;
}

extern "C" ttt_status tttk_ce_lse(const float* logits, const void* parts, int32_t n, int32_t nt, int32_t V,
                                  const int32_t* labels, float scale, float* loss, void* dz, int* err, void* stream) {
  if (!logits || !parts || !labels || !loss || !dz || !err || n < 0 || nt < 0 || nt > n || V < 1)
    return TTT_ERR_INVALID_ARG;
  if (V % 4) return TTT_ERR_UNSUPPORTED;
  return ce_fwd_bwd_lse(DT::BF16, logits, (const float2*)parts, n, nt, V, labels, scale, loss, dz, err,
                        (hipStream_t)stream) == hipSuccess
             ? TTT_OK
             : TTT_ERR_HIP;
}
