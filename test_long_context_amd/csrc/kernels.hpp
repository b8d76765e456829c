// Internal launchers of the TTT-E2E gfx950 kernels (host-callable).
// Every launcher enqueues on the given stream and returns hipSuccess or the
// launch error; shape requirements are validated by the engine before the
// first launch.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "gemm_args.hpp"  // GEMM family: C = A B^T variants, epilogues, GemmArgs

namespace ttt {

enum class DT : int { F32 = 0, BF16 = 1 };
inline size_t dt_size(DT t) { return t == DT::F32 ? 4 : 2; }


hipError_t gemm(DT dt, bool a_kmajor, bool b_kmajor, Epi epi, const GemmArgs& g, hipStream_t st);

// Fused weight-gradient contraction and fp32 SGD step (bf16 operands):
//   W[m, n] -= lr * sum_k A[k * lda + m] B[k * ldb + n],
//   Hi = RNE(W) (bf16), Lo = RNE(W - Hi) (bf16, optional)
// for one or two problems of the same K in one persistent launch (grid 0 =
// two workgroups per CU). Needs M, N multiples of 16, lda, ldb multiples of
// 8, ldw of 4, A, B, W 16-byte and Hi, Lo 8-byte aligned (dw_sgd_supported).
struct DwUpdate {
  const void* A;
  long lda;
  const void* B;
  long ldb;
  float* W;
  void* Hi;
  void* Lo;
  long ldw;
  int M, N;
};
bool dw_sgd_supported(const DwUpdate& u);
hipError_t dw_sgd(const DwUpdate* u, int n, int K, float lr, int grid, hipStream_t st);
// Tile K granule that split-K chunks must be a multiple of.
int gemm_k_granule(DT dt);

// -------------------------------------------------------- elementwise / norm
// h[t, :] = embed[tok[t], :] (as float); bad ids set *err |= 1 and give zeros.
hipError_t embed_gather(DT dt, const int32_t* tok, int n, const void* embed, int d, float* h,
                        int V, int* err, hipStream_t st);
// y (T) = g * x * r, r = rsqrt(mean(x^2) + eps); x float [n, d]; r float [n].
// x = x_in + sum of nsplit partials ([nsplit][n][d], pending split-K
// residual updates; parts may be null when nsplit = 0); x_out and save
// (either may be null) receive x; y = RMSNorm(x) * g, r = 1 / rms.
hipError_t rmsnorm_fwd_fused(DT dt, const float* x_in, const float* parts, int nsplit, float* x_out, float* save,
                             const float* g, int n, int d, float eps, void* y, float* r, hipStream_t st);
// ... with the partial sums stored in bf16
hipError_t rmsnorm_fwd_fused(DT dt, const float* x_in, const __bf16* parts, int nsplit, float* x_out, float* save,
                             const float* g, int n, int d, float eps, void* y, float* r, hipStream_t st);
hipError_t rmsnorm_fwd(DT dt, const float* x, const float* g, int n, int d, float eps, void* y,
                       float* r, hipStream_t st);
// dh[t] += rmsnorm_bwd(dy[t]) where dy = sum over nsplit partials of
// [n, d] (stride n*d), float or, with dy_bf16, bf16; writes dh (float) and
// dh_t (T copy).
hipError_t rmsnorm_bwd(DT dt, const void* dy, bool dy_bf16, int nsplit, const float* x, const float* g,
                       const float* r, int n, int d, float* dh, void* dh_t, int accumulate,
                       hipStream_t st);
// Apply RoPE to q and k of a fused qkv buffer [n, (H + 2Hk) dh] (T) at
// positions pos0 + t; write q (T) [n, H dh]; write k, v into the key/value
// store [Hk][cap][dh] at slot (pos & (cap - 1)) for rows whose position is
// >= min_store_pos; optionally also into a full-length buffer.
hipError_t rope_scatter(DT dt, const void* qkv, int n, int H, int Hk, int dh, int64_t pos0,
                        const float2* rope_tab, void* q, void* kstore, void* vstore, void* vtstore,
                        int cap, int64_t min_store_pos, hipStream_t st);
// dQKV (T) [n, (H+2Hk) dh] from dq [n, H dh] (float), dk, dv [n, Hk dh]
// (float): inverse rotation of dq and dk. dq_parts partial sums of dq;
// kv_parts of dk and dv, or, with kv_run > 0, attn_bwd2_kv_block_parts(n,
// kv_window, H / Hk, kv_run, t / 128) of those of position t.
hipError_t rope_bwd_pack(DT dt, const float* dq, int dq_parts, const float* dk, const float* dv, int kv_parts,
                         int kv_run, int kv_window, int n, int H, int Hk, int dh, int64_t pos0,
                         const float2* rope_tab, void* dqkv, hipStream_t st);
// The same from bf16 partial sums.
hipError_t rope_bwd_pack(DT dt, const __bf16* dq, int dq_parts, const __bf16* dk, const __bf16* dv, int kv_parts,
                         int kv_run, int kv_window, int n, int H, int Hk, int dh, int64_t pos0,
                         const float2* rope_tab, void* dqkv, hipStream_t st);
// Fused softmax cross-entropy over the vocabulary for rows with a target
// (rows < nt): loss[t] = lse - z[t, label]; dz (T) = (softmax - onehot) * scale;
// rows >= nt get dz = 0. Also flags non-finite losses in *err (bit 2).
hipError_t ce_fwd_bwd(DT dt, const float* logits, int n, int nt, int V, const int32_t* labels,
                      float scale, float* loss, void* dz, int* err, hipStream_t st);
// The same from the logits' per-64-column (max, sum exp) partials (float2
// [n][ceil(V / 64)], Epi::STORE_F32_LSE): one read of the logits, one write
// of dz. bf16 dz, V a multiple of 4.
hipError_t ce_fwd_bwd_lse(DT dt, const float* logits, const float2* parts, int n, int nt, int V,
                          const int32_t* labels, float scale, float* loss, void* dz, int* err, hipStream_t st);
// D[h][t] = sum_j dO[t, h, j] O[t, h, j].
hipError_t attn_rowdot(DT dt, const void* dO, const void* O, int n, int H, int dh, float* D,
                       hipStream_t st);
hipError_t copy_f32(const float* src, float* dst, size_t n, hipStream_t st);
hipError_t cast_to(DT dt, const float* src, void* dst, size_t n, hipStream_t st);
hipError_t cast_from(DT dt, const void* src, float* dst, size_t n, hipStream_t st);
hipError_t fill_i32(int* p, int v, size_t n, hipStream_t st);
hipError_t fill_f32(float* p, float v, size_t n, hipStream_t st);
hipError_t fill_zero_bytes(void* p, size_t nbytes, hipStream_t st);

// ------------------------------------------------------------------- attention
// Position of ring slot s in the transposed value store: inside each block
// of 16 slots, bits 2 and 3 are swapped, so that the eight keys one lane
// feeds to a 32x32x16 MFMA contraction (keys 4g .. 4g+3 and 8+4g .. 11+4g of
// a 16-key block) are eight consecutive positions.
__host__ __device__ __forceinline__ long vt_slot(long s) {
  return (s & ~15L) | (s & 3) | ((s & 4) << 1) | ((s & 8) >> 1);
}

struct AttnArgs {
  const void* q;      // [n, H, dh] (T) queries at positions pos0 + i
  const void* k;      // key store [Hk][cap][dh] (T)
  const void* v;      // value store [Hk][cap][dh] (T)
  const void* vt;     // transposed value store [Hk][dh][cap] (T), slots at vt_slot(), or null
  void* o;            // [n, H, dh] (T)
  float* lse;         // [H][n] (may be null)
  int n, H, Hk, dh, cap, window;
  int64_t pos0;
  float scale;
  // backward only
  const void* dO;     // [n, H, dh] (T)
  const float* D;     // [H][n]
  float* dq;          // [n, H, dh] float
  float* dk;          // [n, Hk, dh] float, keys of this call's own positions
  float* dv;
  // second-generation backward: its per-part dq / dk / dv partial sums are
  // stored as bf16 (at the same element offsets, in the same buffers) when set
  bool parts_bf16;
  // second-generation dK / dV: also write zeros into the partial sums that
  // no run of a key block reaches (for consumers that add all
  // attn_bwd2_kv_parts() parts of every key; the RoPE backward instead adds
  // each key block's own attn_bwd2_kv_block_parts())
  bool kv_fill;
  // forward key-range split (second-generation forward): ksplit parts, each
  // an unnormalised output [n, H, dh] in opart and (max, sum) in mlpart
  // [ksplit][2][H][n] (log2 domain), merged by a combine pass
  int ksplit;
  float* opart;
  float* mlpart;
};
hipError_t attn_fwd(DT dt, const AttnArgs& a, hipStream_t st);
// Second-generation forward (bf16, head_dim 64/128, needs a.vt).
bool attn_fwd2_supported(DT dt, const AttnArgs& a);
// qb: 0 = chosen from the shape, 1 / 2 = 32 / 64 queries per wave.
// With a.ksplit > 1 (and a.opart, a.mlpart), the key range is split over
// that many workgroups per query block; attn_fwd2_combine then writes o and
// lse (a no-op without a split).
hipError_t attn_fwd2(DT dt, const AttnArgs& a, hipStream_t st, int qb = 0);
hipError_t attn_fwd2_combine(const AttnArgs& a, hipStream_t st);
// Key-range split that fills the CUs for this shape (1 = none).
int attn_fwd2_splits(const AttnArgs& a);
hipError_t attn_bwd_dq(DT dt, const AttnArgs& a, hipStream_t st);
hipError_t attn_bwd_dkdv(DT dt, const AttnArgs& a, hipStream_t st);
// Second-generation backward (bf16, head_dim 64/128). dq receives
// attn_bwd2_dq_parts(a) partial sums ([parts][n][H][dh]); dk and dv receive
// attn_bwd2_kv_parts(a) partial sums ([parts][n][Hk][dh]): each 128-key
// block's (query head, query tile) pairs are cut into at most
// max(H / Hk, ATTN_BWD2_MAX_KV_PARTS) runs of about equal length, one
// workgroup and one part each (parts a block's runs do not reach are written
// as zeros).
bool attn_bwd2_supported(DT dt, const AttnArgs& a);
int attn_bwd2_dq_parts(const AttnArgs& a);
// Upper bound of attn_bwd2_dq_parts().
constexpr int ATTN_BWD2_MAX_DQ_PARTS = 8;
int attn_bwd2_kv_parts(const AttnArgs& a);
// attn_bwd2_kv_parts() <= max(H / Hk, ATTN_BWD2_MAX_KV_PARTS).
constexpr int ATTN_BWD2_MAX_KV_PARTS = 8;
// Run length (query-tile pairs per workgroup) of the dK / dV kernel for a.
int attn_bwd2_kv_run(const AttnArgs& a);
// Query tiles of 64 that see key block kb (keys 128 kb .. 128 kb + 127 of a
// call of n positions): from the block's first key up to the last query that
// sees its last key.
__host__ __device__ inline int attn_bwd2_kv_block_tiles(int n, int window, int kb) {
  const int64_t k0 = (int64_t)kb * 128, lim = k0 + 127 + window;
  const int64_t q_end = lim < (int64_t)n ? lim : (int64_t)n;
  return (int)((q_end - k0 + 63) / 64);
}
// Partial sums that key block kb receives from the dK / dV kernel (runs of
// `run` pairs over its grp query heads' tiles).
__host__ __device__ inline int attn_bwd2_kv_block_parts(int n, int window, int grp, int run, int kb) {
  return (grp * attn_bwd2_kv_block_tiles(n, window, kb) + run - 1) / run;
}
hipError_t attn_bwd_dq2(DT dt, const AttnArgs& a, hipStream_t st);
hipError_t attn_bwd_dkdv2(DT dt, const AttnArgs& a, hipStream_t st);
// dst[i] = sum_p parts[p * count + i]
hipError_t sum_parts_f32(const float* parts, int nparts, long count, float* dst, hipStream_t st);

// ---------------------------------------------------------------- decode
// y = W x for one fp32 row x (W [N][K] of storage type wdt); with g given,
// x is first RMS-normalised with gain g. Epilogues: STORE, ADD_F32 (y +=),
// SWIGLU (W rows 16-interleaved (gate, up); y [N/2] = silu(gate) * up).
// ROPE is the epilogue of gemv_qkv_rope only.
enum class GvEpi : int { STORE = 0, ADD_F32, SWIGLU, ROPE };
hipError_t gemv(DT wdt, const void* W, const float* x, const float* g, float eps, int N, int K, GvEpi epi,
                float* y, hipStream_t st);
// The fused q/k/v projection of one token (W [(H + 2 Hk) dh][K] of type dt,
// x RMS-normalised with gain g) whose epilogue applies RoPE and stores: each
// pair of rows (j, j + dh / 2) of a head is rotated at position *pos (q and
// k heads) and written to q (fp32), the key ring, or the value ring and its
// transpose (slot *pos & (cap - 1)).
hipError_t gemv_qkv_rope(DT dt, const void* W, const float* x, const float* g, float eps, int H, int Hk, int dh,
                         int K, const int64_t* pos, const float2* rope_tab, float* q, void* kstore, void* vstore,
                         void* vtstore, int cap, hipStream_t st);
// One query per head at position *pos over the window; part: [H][nsplit][dh + 2]
// with nsplit = decode_attn_splits(...) (vtstore, the transposed value store,
// may be null: then the lane-parallel kernel runs).
int decode_attn_splits(DT dt, int H, int Hk, int dh, int window, bool has_vt);
hipError_t decode_attn(DT dt, const float* q, const void* kstore, const void* vstore, const void* vtstore, int H,
                       int Hk, int dh, int cap, int window, const int64_t* pos, float* part, float* o,
                       hipStream_t st);
hipError_t embed_row(DT dt, const int32_t* tok, const void* embed, int d, int V, float* h, int* err,
                     hipStream_t st);
hipError_t bump_pos(int64_t* pos, hipStream_t st);
hipError_t set_pos(int64_t* pos, int64_t value, hipStream_t st);

// ---------------------------------------------------------------- E2-TTT
// Per (head, chunk) scalars: KW_t = eta_t A_t, KM_t = eta_t beta~_t and the
// chunk coefficients (gamma~_0, beta_1 A_1, beta~_0).
hipError_t e2_scalars(const float* eta, const float* beta, const float* gamma, int H, int64_t T,
                      int C, float* KW, float* KM, float* coef, hipStream_t st);

}  // namespace ttt
