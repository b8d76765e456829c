// TTT-E2E engine: owns the context state on one GPU and schedules the
// kernels of the inner loop on the caller's stream. Implements include/ttt.h.
//
// Phases of ttt_prefill (all on the caller's stream):
//   prefix  -- blocks 0 .. s-1 and the attention + static MLP of block s do not
//              depend on any fast weight, so they run once over the sequence
//              in slabs of up to `slab` positions (large GEMMs); their keys and
//              values go to the per-layer rings, and the residual stream at the
//              input of block s's dynamic MLP is kept for every position.
//   loop    -- for each mini-batch: block s's dynamic MLP, blocks s+1 .. L-1
//              (attention over the ring window, static MLP, dynamic MLP), final
//              norm, lm_head, fused softmax-CE + dz, then the backward into the
//              dynamic MLP weights, whose dW products apply the fp32 SGD update
//              W -= alpha dW in their epilogue (bf16 working copy re-rounded
//              from the fp32 master).
//
// Several sequences (n_seq = B > 1) run side by side, each with its own key/
// value rings, residual stream and fast weights: the loop's activations hold
// the B mini-batches one after another (rows j n .. j n + n - 1 belong to
// sequence j), so the products with frozen weights see M = B n rows, the
// products with fast weights run as one batched launch of B products, and
// the position-dependent kernels (RoPE, attention, cross-entropy) run once
// per sequence on its slice.
#include <math.h>
#include <string.h>

#include <algorithm>
#include <cstdio>
#include <cstdlib>
#include <string>
#include <vector>

#include "../../include/ttt.h"
#include "kernels.hpp"

using namespace ttt;

namespace {

struct Buf {
  void* p = nullptr;
  size_t n = 0;
};

int64_t next_pow2(int64_t x) {
  int64_t p = 1;
  while (p < x) p <<= 1;
  return p;
}

}  // namespace

struct ttt_ctx {
  ttt_config cfg{};
  DT dt = DT::BF16;
  size_t es = 2;
  int L = 0, d = 0, H = 0, Hk = 0, dh = 0, F = 0, Fd = 0, V = 0, k = 0, b = 0, nd = 0, s = 0;
  int64_t max_seq = 0, cap = 0, slab = 0;
  int QKV = 0;  // (H + 2 Hk) dh
  int B = 1;            // sequences side by side
  size_t ring_seq = 0;  // elements of one sequence's slice of a layer's ring (Hk cap dh)
  int64_t pos = 0;
  std::string err;
  std::vector<void*> allocs;

  // weights
  void* embed = nullptr;
  void* lm_head = nullptr;
  float* final_norm = nullptr;
  std::vector<float*> attn_norm, mlp_norm, dyn_norm;
  std::vector<void*> wqkv, wo, w12, w3;       // static, storage dtype
  std::vector<float*> m12, m3;               // dynamic fp32 masters (interleaved W1|W2), [B] each
  std::vector<void*> dw12, dw3;              // dynamic working copies (== master for f32)
  std::vector<void*> dw12_lo, dw3_lo;        // bf16: low terms, master ~= working + low
  std::vector<void*> w0_12, w0_3;            // W0 snapshot (storage dtype, interleaved)
  std::vector<void*> kring, vring;           // per layer [B][Hk][cap][dh]
  std::vector<void*> vtring;                 // per layer [B][Hk][dh][cap] (values transposed)
  float2* rope = nullptr;                    // [max_seq][dh/2] (cos, sin)

  // prefix / shared activations
  float* hres = nullptr;   // [B][max_seq, d] residual stream (input of block s's dynamic MLP)
  float* rbuf = nullptr;   // [slab]
  void* xn = nullptr;      // [slab, d]
  void* qkv = nullptr;     // [slab, QKV]
  void* qb = nullptr;      // [slab, H dh]
  void* ob = nullptr;      // [slab, H dh]
  void* hmid = nullptr;    // [slab, max(F, Fd)]

  // loop (per dynamic block i = l - s; every [b, ...] buffer holds B b rows)
  std::vector<float*> h_att, h_mlp, h_dyn, r_att, r_mlp, r_dyn, lse;
  std::vector<void*> q_l, o_l, h12_s, xn_d, h12_d, hm_d;
  float* h_f = nullptr;
  float* r_f = nullptr;
  float* logits = nullptr;                   // [b, V]
  float2* lse_part = nullptr;                // bf16: [b, ceil(V / 64)] (max, sum exp) of the logits' 64-column groups
  void* dz = nullptr;                        // [b, V]
  // backward
  float* gh = nullptr;                       // [b, d] gradient of the residual stream
  void* gh_t = nullptr;                      // [b, d]
  void* dh12 = nullptr;                      // [b, 2 max(F, Fd)]
  float* part = nullptr;                     // [max_split, b, d]
  int max_split = 1;
  void* dO = nullptr;                        // [b, H dh]
  float* Dbuf = nullptr;                     // [H, b]
  float* dq = nullptr;                       // [parts][b, H dh] (partial sums)
  float* apart = nullptr;                    // forward key-split partial outputs [4][b, H dh]
  float* aml = nullptr;                      // ... and their (max, sum) [4][2][H][b]
  float* dk = nullptr;                       // [b, Hk dh]
  float* dv = nullptr;
  void* dqkv = nullptr;                      // [b, QKV]
  int* d_err = nullptr;
  int64_t* d_pos = nullptr;
  float* dec = nullptr;                      // decode scratch
  int dec_split = 1;
  int32_t* d_tok = nullptr;                  // decode input token
  int32_t* tokhist = nullptr;                // [B][max_seq] every token consumed (prefill and decode)
  float* dloss = nullptr;                    // [b] losses of a decode-time update (when the caller passes none)
  int64_t trained = 0;                       // positions below it were used, with their targets, by an update
  // fast-weight updates run on side streams, overlapping the rest of the
  // backward; their inputs are per dynamic block so that the main stream
  // never overwrites what an update still reads. A block's two update
  // products (dW3 on side2, dW12 on side) run side by side, so one's
  // epilogue traffic overlaps the other's products.
  hipStream_t side = nullptr;
  hipStream_t side2 = nullptr;
  hipEvent_t ev_w3 = nullptr;                // side2: the last dW3 update is done
  std::vector<hipEvent_t> ev_dyn;            // per dynamic block: its dW inputs are ready
  std::vector<hipEvent_t> ev_upd;            // per dynamic block: its update is done
  hipEvent_t ev_join = nullptr;              // side stream done with the prefill
  std::vector<void*> ghd_t;                  // [b, d] gradient into each dynamic MLP (storage dtype)
  std::vector<void*> dh12d;                  // [b, 2 Fd] SwiGLU pre-activation gradients per dynamic block
  bool fused_update = false;                 // bf16: both update products in one dw_sgd launch
  bool upd_main = false;                     // update products on the caller's stream instead of side streams
  bool upd_at_attn = false;                  // launch a block's update when its attention backward starts
  bool upd_split = false;                    // ... its dW3 product at once and only dW12 then
  bool upd_after_dq = false;                 // ... after the query-side attention backward instead
  bool sr_round = false;                     // bf16: one stochastically rounded working copy, no low term
  bool fwd_parts_bf16 = false;               // bf16: the forward's split-K partial sums stored in bf16
  int upd_grid = 0;                          // its workgroups (0: two per CU)
  hipStream_t dstream = nullptr;             // decode graph capture stream
  hipGraphExec_t dgraph = nullptr;           // captured decode blocks

  // live per-class timing (ttt_timing_enable / ttt_timing_read)
  struct TRec {
    int kind;
    hipEvent_t a, b;
    double flops, bytes;
  };
  uint32_t tmask = 0;
  std::vector<hipEvent_t> evpool;
  size_t evused = 0;
  std::vector<TRec> trecs;
  hipEvent_t ev() {
    if (evused == evpool.size()) {
      hipEvent_t e = nullptr;
      if (hipEventCreate(&e) != hipSuccess) return nullptr;
      evpool.push_back(e);
    }
    return evpool[evused++];
  }
};

namespace {

ttt_status fail(ttt_ctx* c, ttt_status s, const std::string& msg) {
  if (c) c->err = msg;
  return s;
}

#define HIPCHK(c, call)                                                               \
  do {                                                                                \
    hipError_t e_ = (call);                                                           \
    if (e_ != hipSuccess)                                                             \
      return fail(c, TTT_ERR_HIP, std::string(#call) + ": " + hipGetErrorString(e_)); \
  } while (0)

// Records HIP events around one launch when its class is being timed.
struct Timed {
  ttt_ctx* c;
  hipStream_t st;
  int kind;
  double fl, by;
  hipEvent_t a = nullptr, b = nullptr;
  Timed(ttt_ctx* c_, hipStream_t st_, int kind_, double fl_, double by_)
      : c(c_), st(st_), kind(kind_), fl(fl_), by(by_) {
    if (c->tmask & (1u << kind)) {
      a = c->ev();
      b = c->ev();
      if (a && b) (void)hipEventRecord(a, st);
      else a = b = nullptr;
    }
  }
  ~Timed() {
    if (a) {
      (void)hipEventRecord(b, st);
      c->trecs.push_back({kind, a, b, fl, by});
    }
  }
};

#define TCALL(kind, fl, by, call)       \
  do {                                  \
    Timed t_(c, st, (kind), (fl), (by)); \
    HIPCHK(c, call);                    \
  } while (0)

constexpr int KC_GP = TTT_KC_GEMM_PREFIX, KC_AP = TTT_KC_ATTN_PREFIX, KC_GL = TTT_KC_GEMM_LOOP,
              KC_AL = TTT_KC_ATTN_LOOP, KC_LM = TTT_KC_LMHEAD, KC_CE = TTT_KC_CE,
              KC_AB = TTT_KC_ATTN_BWD, KC_SGD = TTT_KC_DW_SGD, KC_OT = TTT_KC_OTHER;

inline double gfl(double m, double n, double k) { return 2.0 * m * n * k; }

// sum over queries at positions p0 .. p0+n-1 of the number of visible keys
double window_pairs(int64_t p0, int n, int k) {
  double s = 0;
  for (int i = 0; i < n; ++i) s += (double)std::min<int64_t>(p0 + i + 1, k);
  return s;
}

bool dalloc(ttt_ctx* c, void** p, size_t bytes) {
  if (bytes == 0) bytes = 16;
  if (hipMalloc(p, bytes) != hipSuccess) {
    (void)hipGetLastError();
    *p = nullptr;
    return false;
  }
  c->allocs.push_back(*p);
  return true;
}

template <typename P>
bool dalloc_t(ttt_ctx* c, P** p, size_t bytes) {
  void* v = nullptr;
  bool ok = dalloc(c, &v, bytes);
  *p = (P*)v;
  return ok;
}

// Effective window (a window longer than any stream cannot see more keys),
// prefix slab and ring capacity of a config.
int64_t eff_window(const ttt_config& c) {
  return std::min<int64_t>(c.window, std::max<int64_t>(c.max_seq, c.minibatch));
}
void ring_shape(const ttt_config& c, int64_t* slab, int64_t* cap) {
  int64_t s = c.prefix_slab > 0 ? std::min<int64_t>(c.prefix_slab, c.max_seq)
                                : std::min<int64_t>(c.max_seq, 16384);
  s = std::max<int64_t>(s, c.minibatch);
  *slab = s;
  *cap = next_pow2(std::max<int64_t>(eff_window(c) + s, 128));
}

ttt_status validate(const ttt_config* cfg) {
  if (!cfg) return TTT_ERR_INVALID_ARG;
  const ttt_config& c = *cfg;
  if (c.dtype != TTT_F32 && c.dtype != TTT_BF16) return TTT_ERR_INVALID_ARG;
  if (c.reduction != TTT_LOSS_MEAN && c.reduction != TTT_LOSS_SUM) return TTT_ERR_INVALID_ARG;
  if (c.n_layers < 1 || c.d_model < 1 || c.n_heads < 1 || c.n_kv_heads < 1 || c.head_dim < 1 ||
      c.ffn_hidden < 1 || c.dyn_ffn_hidden < 1 || c.vocab < 2 || c.minibatch < 1 ||
      c.max_seq < 2 || c.n_dynamic < 0 || c.n_dynamic > c.n_layers || c.prefix_slab < 0 || c.n_seq < 0 ||
      c.n_seq > 64)
    return TTT_ERR_INVALID_ARG;
  if (c.window < c.minibatch) return TTT_ERR_INVALID_ARG;  // k >= b
  if (!(c.alpha >= 0.f) || !isfinite(c.alpha) || !(c.rms_eps > 0.f) || !(c.rope_theta > 1.f))
    return TTT_ERR_INVALID_ARG;
  if (c.n_heads % c.n_kv_heads) return TTT_ERR_INVALID_ARG;
  if (!(c.head_dim == 16 || c.head_dim == 64 || c.head_dim == 128)) return TTT_ERR_UNSUPPORTED;
  if (c.d_model % 16 || c.ffn_hidden % 32 || c.dyn_ffn_hidden % 32 || c.vocab % 8)
    return TTT_ERR_UNSUPPORTED;
  if (c.d_model > 8192) return TTT_ERR_UNSUPPORTED;  // a residual row stays in one workgroup's registers
  if ((int64_t)c.max_seq > (int64_t(1) << 30)) return TTT_ERR_UNSUPPORTED;
  if ((int64_t)c.vocab * c.d_model > (int64_t(1) << 31)) return TTT_ERR_UNSUPPORTED;
  // one key head's slice of a ring is addressed with 32-bit byte offsets
  int64_t slab = 0, cap = 0;
  ring_shape(c, &slab, &cap);
  const int64_t es = c.dtype == TTT_BF16 ? 2 : 4;
  if (cap * c.head_dim * es >= (int64_t(1) << 31)) return TTT_ERR_UNSUPPORTED;
  return TTT_OK;
}

ttt_status check_device(ttt_ctx* c) {
  int n = 0;
  if (hipGetDeviceCount(&n) != hipSuccess || n < 1) {
    (void)hipGetLastError();
    return fail(c, TTT_ERR_NO_DEVICE, "no HIP device");
  }
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return fail(c, TTT_ERR_NO_DEVICE, "hipGetDevice failed");
  hipDeviceProp_t pr;
  if (hipGetDeviceProperties(&pr, dev) != hipSuccess) return fail(c, TTT_ERR_NO_DEVICE, "no properties");
  if (strncmp(pr.gcnArchName, "gfx950", 6) != 0)
    return fail(c, TTT_ERR_NO_DEVICE, std::string("device is ") + pr.gcnArchName + ", need gfx950");
  return TTT_OK;
}

// Copy src [F, d] into rows of the 16-interleaved fused layout (gate rows at
// 32 j + w, up rows at 32 j + 16 + w).
hipError_t interleave(void* dst, const void* src, int F, int d, size_t es, int which, hipStream_t st) {
  const size_t blk = (size_t)16 * d * es;
  return hipMemcpy2DAsync((char*)dst + which * blk, 2 * blk, src, blk, blk, F / 16,
                          hipMemcpyDeviceToDevice, st);
}
hipError_t deinterleave(void* dst, const void* src, int F, int d, size_t es, int which, hipStream_t st) {
  const size_t blk = (size_t)16 * d * es;
  return hipMemcpy2DAsync(dst, blk, (const char*)src + which * blk, 2 * blk, blk, F / 16,
                          hipMemcpyDeviceToDevice, st);
}

int choose_split(int tiles, int K) {
  // aim for >= 2 workgroups per CU on the 256-CU part
  int s = (512 + tiles - 1) / tiles;
  s = std::min(s, std::max(1, K / 256));
  return std::max(1, std::min(s, 16));
}

GemmArgs ga(const void* A, long lda, const void* B, long ldb, int M, int N, int K, void* C, long ldc) {
  GemmArgs g{};
  g.A = A;
  g.B = B;
  g.M = M;
  g.N = N;
  g.K = K;
  g.lda = lda;
  g.ldb = ldb;
  g.C = C;
  g.ldc = ldc;
  g.scale = 1.f;
  g.kchunk = 0;
  return g;
}

// One product per sequence with the sequence's own fast weights, in one
// launch: product j reads A + j sA, B (and its low term) + j sB and writes
// C + j sC, C2 (and C3) + j sC2, with X + j sX (elements).
struct Bat {
  int n = 1;
  long sA = 0, sB = 0, sC = 0, sC2 = 0, sX = 0;
};
void set_batch(GemmArgs& g, const Bat& b) {
  if (b.n <= 1) return;
  g.batch = b.n;
  g.sA = b.sA;
  g.sB = b.sB;
  g.sC = b.sC;
  g.sC2 = b.sC2;
  g.sX = b.sX;
}

// C (float partials) = A [M, K] (k-major) * B (k-row-major [K, N]), split-K;
// *nsplit receives the number of partial slices written. Batched (bt.n > 1):
// product j's rows follow product j - 1's inside each slice, so the slices
// hold bt.n M rows, as for one product of that many rows.
ttt_status gemm_nn_split(ttt_ctx* c, int kind, const void* A, long lda, const void* B, long ldb, int M,
                         int N, int K, float* part, int* nsplit, hipStream_t st, const Bat& bt = Bat{}) {
  // bf16: 256 x 256 tiles, K split so that the grid is about one workgroup
  // per CU (measured at the 3B dX shapes: better than more, smaller tiles)
  const int gran = gemm_k_granule(c->dt);
  int s;
  if (c->dt == DT::BF16) {
    const int tiles = ((M + 255) / 256) * ((N + 255) / 256) * bt.n;
    s = std::max(1, std::min(256 / tiles, K / 512));
  } else {
    s = choose_split(((M + 127) / 128) * ((N + 127) / 128) * bt.n, K);
  }
  s = std::min(s, c->max_split);
  int chunk = (K + s - 1) / s;
  chunk = (chunk + gran - 1) / gran * gran;
  s = (K + chunk - 1) / chunk;
  GemmArgs g = ga(A, lda, B, ldb, M, N, K, part, N);
  g.kchunk = chunk;
  if (bt.n > 1) {
    Bat b2 = bt;
    b2.sC = (long)M * N;
    set_batch(g, b2);
    g.split_ld = (long)bt.n * M * N;
  }
  if (c->dt == DT::BF16) g.tile = 5;
  *nsplit = s;
  // bf16: the gradient partials are stored in bf16 (half the traffic of
  // writing them here and reading them back in the RMSNorm backward)
  const Epi e = c->dt == DT::BF16 ? Epi::PARTIAL_BF16 : Epi::PARTIAL;
  TCALL(kind, gfl(M, N, K) * bt.n, 0, gemm(c->dt, true, false, e, g, st));
  return TTT_OK;
}

#define RUN(x)                      \
  do {                              \
    ttt_status r_ = (x);            \
    if (r_ != TTT_OK) return r_;    \
  } while (0)

hipError_t attn_fwd_any(DT dt, const AttnArgs& a, hipStream_t st) {
  return attn_fwd2_supported(dt, a) ? attn_fwd2(dt, a, st) : attn_fwd(dt, a, st);
}

// Sequence j's slice of a per-sequence buffer of `per` elements of es bytes.
inline void* sq(void* p, int j, size_t per, size_t es) {
  return p ? (void*)((char*)p + (size_t)j * per * es) : nullptr;
}
inline float* sqf(float* p, int j, size_t per) { return p ? p + (size_t)j * per : nullptr; }
// floats of one sequence's dk (or dv) partial sums: up to
// ATTN_BWD2_MAX_KV_PARTS parts of the second-generation backward, H / Hk of
// the first
inline size_t kv_part_elems(const ttt_ctx* c) {
  return (size_t)std::max(c->H / c->Hk, ATTN_BWD2_MAX_KV_PARTS) * c->b * c->Hk * c->dh;
}

AttnArgs attn_args(ttt_ctx* c, int l, int j, const void* q, void* o, float* lse, int n, int64_t p0) {
  AttnArgs a{};
  a.q = q;
  a.k = sq(c->kring[l], j, c->ring_seq, c->es);
  a.v = sq(c->vring[l], j, c->ring_seq, c->es);
  a.vt = sq(c->vtring[l], j, c->ring_seq, c->es);
  a.o = o;
  a.lse = lse;
  a.n = n;
  a.H = c->H;
  a.Hk = c->Hk;
  a.dh = c->dh;
  a.cap = (int)c->cap;
  a.window = c->k;
  a.pos0 = p0;
  a.scale = 1.f / sqrtf((float)c->dh);
  return a;
}

// ------------------------------------------------------------ prefix phase
// Positions [pb, pe) of sequence j (tok: its token of position 0 onwards).
ttt_status run_prefix(ttt_ctx* c, int j, const int32_t* tok, int64_t pb, int64_t pe, hipStream_t st) {
  const int d = c->d, H = c->H, Hk = c->Hk, dh = c->dh, QKV = c->QKV, F = c->F;
  const float eps = c->cfg.rms_eps;
  const size_t rs = c->ring_seq, es = c->es;
  for (int64_t p0 = pb; p0 < pe; p0 += c->slab) {
    const int n = (int)std::min<int64_t>(c->slab, pe - p0);
    float* h = c->hres + ((size_t)j * c->max_seq + p0) * d;
    TCALL(KC_OT, 0, 0, embed_gather(c->dt, tok + p0, n, c->embed, d, h, c->V, c->d_err, st));
    for (int l = 0; l <= c->s; ++l) {
      TCALL(KC_OT, 0, 0, rmsnorm_fwd(c->dt, h, c->attn_norm[l], n, d, eps, c->xn, c->rbuf, st));
      TCALL(KC_GP, gfl(n, QKV, d), 0,
            gemm(c->dt, true, true, Epi::STORE, ga(c->xn, d, c->wqkv[l], d, n, QKV, d, c->qkv, QKV), st));
      TCALL(KC_OT, 0, 0, rope_scatter(c->dt, c->qkv, n, H, Hk, dh, p0, c->rope, c->qb, sq(c->kring[l], j, rs, es),
                                      sq(c->vring[l], j, rs, es), sq(c->vtring[l], j, rs, es), (int)c->cap, 0, st));
      AttnArgs a = attn_args(c, l, j, c->qb, c->ob, nullptr, n, p0);
      TCALL(KC_AP, 4.0 * H * dh * window_pairs(p0, n, c->k), 0, attn_fwd_any(c->dt, a, st));
      TCALL(KC_GP, gfl(n, d, H * dh), 0,
            gemm(c->dt, true, true, Epi::ADD_F32, ga(c->ob, (long)H * dh, c->wo[l], (long)H * dh, n, d, H * dh, h, d), st));
      TCALL(KC_OT, 0, 0, rmsnorm_fwd(c->dt, h, c->mlp_norm[l], n, d, eps, c->xn, c->rbuf, st));
      GemmArgs g = ga(c->xn, d, c->w12[l], d, n, 2 * F, d, nullptr, 2 * F);
      g.C2 = c->hmid;
      TCALL(KC_GP, gfl(n, 2 * F, d), 0, gemm(c->dt, true, true, Epi::SWIGLU, g, st));
      TCALL(KC_GP, gfl(n, d, F), 0,
            gemm(c->dt, true, true, Epi::ADD_F32, ga(c->hmid, F, c->w3[l], F, n, d, F, h, d), st));
    }
  }
  return TTT_OK;
}

// ------------------------------------------------------------ loop phase
// Residual-stream product C[M, N] += A B^T at a mini-batch's row count: too
// few output tiles to fill the CUs, so K is split and the partial sums are
// left in c->part for the next fused RMSNorm to add (returns their count).
// Batched (bt.n > 1, M rows per product): each slice holds bt.n M rows.
ttt_status gemm_resid(ttt_ctx* c, int kind, const void* A, long lda, const void* B, long ldb, const void* B2, int M,
                      int N, int K, int* np, hipStream_t st, const Bat& bt = Bat{}) {
  const int gran = gemm_k_granule(c->dt);
  int s = 1;
  if (c->dt == DT::BF16) {
    const int bm = 256, bn = B2 ? 128 : 256;
    const int tiles = ((M + bm - 1) / bm) * ((N + bn - 1) / bn) * bt.n;
    s = std::max(1, std::min(256 / tiles, K / 512));
  }
  s = std::min(s, c->max_split);
  int chunk = (K + s - 1) / s;
  chunk = (chunk + gran - 1) / gran * gran;
  s = (K + chunk - 1) / chunk;
  GemmArgs g = ga(A, lda, B, ldb, M, N, K, c->part, N);
  g.B2 = B2;
  g.kchunk = chunk;
  if (bt.n > 1) {
    Bat b2 = bt;
    b2.sC = (long)M * N;
    set_batch(g, b2);
    g.split_ld = (long)bt.n * M * N;
  }
  if (c->dt == DT::BF16) g.tile = 5;
  *np = s;
  TCALL(kind, gfl(M, N, K) * (B2 ? 2.0 : 1.0) * bt.n, 0,
        gemm(c->dt, true, true, c->fwd_parts_bf16 ? Epi::PARTIAL_BF16 : Epi::PARTIAL, g, st));
  return TTT_OK;
}

// Fused RMSNorm of the residual stream xr plus the np pending split-K
// partial sums in c->part (bf16 or fp32, as gemm_resid stored them).
hipError_t rms_fwd_parts(ttt_ctx* c, const float* xr, int np, float* save, const float* gain, int n, int d, float eps,
                         void* y, float* r, hipStream_t st) {
  if (c->fwd_parts_bf16)
    return rmsnorm_fwd_fused(c->dt, xr, (const __bf16*)c->part, np, nullptr, save, gain, n, d, eps, y, r, st);
  return rmsnorm_fwd_fused(c->dt, xr, (const float*)c->part, np, nullptr, save, gain, n, d, eps, y, r, st);
}

// Forward of the mini-batch [a0, a0 + n) of every sequence.
ttt_status loop_forward(ttt_ctx* c, int64_t a0, int n, hipStream_t st) {
  const int d = c->d, H = c->H, Hk = c->Hk, dh = c->dh, QKV = c->QKV, s = c->s, F = c->F, Fd = c->Fd;
  const int B = c->B, nb = B * n;
  const size_t es = c->es, rs = c->ring_seq;
  const float eps = c->cfg.rms_eps;
  // the residual stream lives in the buffers saved for the backward: xr is
  // the latest one, and each fused RMSNorm adds the pending partial sums to
  // it and saves the result as the next
  const float* xr = nullptr;
  int np = 0;  // split-K partial sums of the last residual product, pending in c->part
  for (int l = s; l < c->L; ++l) {
    const int i = l - s;
    if (l > s) {
      // attention sublayer (adds the pending dynamic-MLP output of block l-1)
      TCALL(KC_OT, 0, 0, rms_fwd_parts(c, xr, np, c->h_att[i], c->attn_norm[l], nb, d, eps,
                                            c->xn, c->r_att[i], st));
      xr = c->h_att[i];
      TCALL(KC_GL, gfl(nb, QKV, d), 0,
            gemm(c->dt, true, true, Epi::STORE, ga(c->xn, d, c->wqkv[l], d, nb, QKV, d, c->qkv, QKV), st));
      for (int j = 0; j < B; ++j) {
        void* q = sq(c->q_l[i], j, (size_t)n * H * dh, es);
        TCALL(KC_OT, 0, 0, rope_scatter(c->dt, sq(c->qkv, j, (size_t)n * QKV, es), n, H, Hk, dh, a0, c->rope, q,
                                        sq(c->kring[l], j, rs, es), sq(c->vring[l], j, rs, es),
                                        sq(c->vtring[l], j, rs, es), (int)c->cap, 0, st));
        AttnArgs a = attn_args(c, l, j, q, sq(c->o_l[i], j, (size_t)n * H * dh, es),
                               sqf(c->lse[i], j, (size_t)H * n), n, a0);
        if (attn_fwd2_supported(c->dt, a)) {
          a.ksplit = std::min(4, attn_fwd2_splits(a));
          a.opart = sqf(c->apart, j, (size_t)4 * c->b * H * dh);
          a.mlpart = sqf(c->aml, j, (size_t)4 * 2 * H * c->b);
        }
        TCALL(KC_AL, 4.0 * H * dh * window_pairs(a0, n, c->k), 0, attn_fwd_any(c->dt, a, st));
        TCALL(KC_OT, 0, 0, attn_fwd2_combine(a, st));
      }
      RUN(gemm_resid(c, KC_GL, c->o_l[i], (long)H * dh, c->wo[l], (long)H * dh, nullptr, nb, d, H * dh, &np, st));
      // static MLP sublayer
      TCALL(KC_OT, 0, 0, rms_fwd_parts(c, xr, np, c->h_mlp[i], c->mlp_norm[l], nb, d, eps,
                                            c->xn, c->r_mlp[i], st));
      xr = c->h_mlp[i];
      GemmArgs g = ga(c->xn, d, c->w12[l], d, nb, 2 * F, d, c->h12_s[i], 2 * F);
      g.C2 = c->hmid;
      TCALL(KC_GL, gfl(nb, 2 * F, d), 0, gemm(c->dt, true, true, Epi::SWIGLU, g, st));
      RUN(gemm_resid(c, KC_GL, c->hmid, F, c->w3[l], F, nullptr, nb, d, F, &np, st));
      // the previous mini-batch's update of this block (side stream) reads
      // xn_d and the saved activations written from here on
      HIPCHK(c, hipStreamWaitEvent(st, c->ev_upd[i], 0));
      TCALL(KC_OT, 0, 0, rms_fwd_parts(c, xr, np, c->h_dyn[i], c->dyn_norm[i], nb, d, eps,
                                            c->xn_d[i], c->r_dyn[i], st));
      xr = c->h_dyn[i];
    } else {
      // block s: the residual stream comes from the hoisted prefix
      HIPCHK(c, hipStreamWaitEvent(st, c->ev_upd[i], 0));
      for (int j = 0; j < B; ++j)
        TCALL(KC_OT, 0, 0, rmsnorm_fwd_fused(c->dt, c->hres + ((size_t)j * c->max_seq + a0) * d, (const float*)nullptr, 0, nullptr,
                                              sqf(c->h_dyn[i], j, (size_t)n * d), c->dyn_norm[i], n, d, eps,
                                              sq(c->xn_d[i], j, (size_t)n * d, es), sqf(c->r_dyn[i], j, n), st));
      xr = c->h_dyn[i];
    }
    // dynamic MLP sublayer under each sequence's current fast weights
    // (bf16: the fp32 master enters as two bf16 terms, working + low: one
    // step moves W by less than half a bf16 ulp, so RNE(master) alone would
    // round most updates back to the old weights, coherently)
    GemmArgs g = ga(c->xn_d[i], d, c->dw12[i], d, n, 2 * Fd, d, c->h12_d[i], 2 * Fd);
    g.C2 = c->hm_d[i];
    g.B2 = c->sr_round ? nullptr : c->dw12_lo[i];
    Bat b12;
    b12.n = B;
    b12.sA = (long)n * d;
    b12.sB = 2L * Fd * d;
    b12.sC = (long)n * 2 * Fd;
    b12.sC2 = (long)n * Fd;
    set_batch(g, b12);
    TCALL(KC_GL, gfl(nb, 2 * Fd, d), 0, gemm(c->dt, true, true, Epi::SWIGLU, g, st));
    Bat b3;
    b3.n = B;
    b3.sA = (long)n * Fd;
    b3.sB = (long)d * Fd;
    RUN(gemm_resid(c, KC_GL, c->hm_d[i], Fd, c->dw3[i], Fd, c->sr_round ? nullptr : c->dw3_lo[i], n, d, Fd, &np, st,
                   b3));
  }
  TCALL(KC_OT, 0, 0, rms_fwd_parts(c, xr, np, c->h_f, c->final_norm, nb, d, eps, c->xn,
                                        c->r_f, st));
  {
    // bf16: the epilogue also leaves each row's per-64-column (max, sum exp)
    // for the single-pass cross-entropy
    GemmArgs g = ga(c->xn, d, c->lm_head, d, nb, c->V, d, c->logits, c->V);
    g.C2 = c->lse_part;
    TCALL(KC_LM, gfl(nb, c->V, d), 0,
          gemm(c->dt, true, true, c->dt == DT::BF16 ? Epi::STORE_F32_LSE : Epi::STORE_F32, g, st));
  }
  return TTT_OK;
}

// Softmax CE + logit gradient of each sequence's mini-batch [a0, a0 + n)
// (the first nt rows have labels, read from the token history): bf16 from
// the lm_head epilogue's partials (one read of the logits), fp32 with the
// two-pass kernel. Sequence j's losses go to loss0 + j ldl.
ttt_status run_ce(ttt_ctx* c, int64_t a0, int n, int nt, float scale, float* loss0, int64_t ldl, hipStream_t st) {
  const size_t ng = (c->V + 63) / 64;
  for (int j = 0; j < c->B; ++j) {
    const int32_t* labels = c->tokhist + (size_t)j * c->max_seq + a0 + 1;
    float* logits = c->logits + (size_t)j * n * c->V;
    float* loss = loss0 + (size_t)j * ldl;
    void* dz = sq(c->dz, j, (size_t)n * c->V, c->es);
    if (c->dt == DT::BF16)
      TCALL(KC_CE, 0, (double)n * c->V * (4.0 + c->es),
            ce_fwd_bwd_lse(c->dt, logits, c->lse_part + (size_t)j * n * ng, n, nt, c->V, labels, scale, loss, dz,
                           c->d_err, st));
    else
      TCALL(KC_CE, 0, (double)n * c->V * (4.0 + c->es),
            ce_fwd_bwd(c->dt, logits, n, nt, c->V, labels, scale, loss, dz, c->d_err, st));
  }
  return TTT_OK;
}

// Seed of one update product's stochastic rounding (never 0): distinct for
// every mini-batch, dynamic block and product.
uint32_t sr_seed(int64_t step, int block, int which) {
  return (uint32_t)((((uint64_t)step * 64 + (uint64_t)block) * 2 + (uint64_t)which) * 0x9E3779B1ull) | 1u;
}

// The update products of dynamic block i (dW3 = dY^T Hmid and dW12 = dH12^T U,
// with W -= alpha dW in the epilogue) on the side streams, once the main
// stream has queued everything that reads the block's old weights.
// part: 3 = both products, 1 = dW3 only, 2 = dW12 only (dW12 completes the
// block's update event, so it must come last).
ttt_status launch_update(ttt_ctx* c, int i, int64_t a0, int n, hipStream_t st, int part = 3) {
  const int d = c->d, Fd = c->Fd, B = c->B;
  const float lr = c->cfg.alpha;
  const double upd_bytes = 8.0 + (c->dt == DT::F32 ? 0.0 : (double)c->es);  // master r/w + working copy
  void* gt = c->ghd_t[i];
  // dW3 = dY^T Hmid and dW12 = dH12^T U, with W -= alpha dW in the epilogue,
  // on the side stream once this block's products with the old W are queued
  hipStream_t us1 = c->upd_main ? st : c->side, us2 = c->upd_main ? st : c->side2;
  HIPCHK(c, hipEventRecord(c->ev_dyn[i], st));
  HIPCHK(c, hipStreamWaitEvent(us1, c->ev_dyn[i], 0));
  if (c->dt == DT::BF16 && c->fused_update) {
    if (!(part & 2)) return TTT_OK;
    // both products in one persistent launch (shapes checked at init;
    // single-sequence contexts only)
    hipStream_t st = us1;
    const DwUpdate u[2] = {
        DwUpdate{c->dh12d[i], 2L * Fd, c->xn_d[i], d, c->m12[i], c->dw12[i], c->dw12_lo[i], d, 2 * Fd, d},
        DwUpdate{gt, d, c->hm_d[i], Fd, c->m3[i], c->dw3[i], c->dw3_lo[i], Fd, d, Fd}};
    TCALL(KC_SGD, gfl(2 * Fd, d, n) + gfl(d, Fd, n), 3.0 * Fd * d * upd_bytes,
          dw_sgd(u, 2, n, lr, c->upd_grid, st));
    HIPCHK(c, hipEventRecord(c->ev_upd[i], st));
  } else {
    HIPCHK(c, hipStreamWaitEvent(us2, c->ev_dyn[i], 0));
    if (part & 1) {
      hipStream_t st = us2;
      GemmArgs g = ga(gt, d, c->hm_d[i], Fd, d, Fd, n, c->m3[i], Fd);
      g.C2 = c->dw3[i];
      g.C3 = c->sr_round ? nullptr : c->dw3_lo[i];
      g.seed = c->sr_round ? sr_seed(a0 / c->b, i, 0) : 0u;
      g.scale = lr;
      Bat bt;
      bt.n = B;
      bt.sA = (long)n * d;
      bt.sB = (long)n * Fd;
      bt.sC = bt.sC2 = (long)d * Fd;
      set_batch(g, bt);
      TCALL(KC_SGD, gfl(d, Fd, n) * B, (double)d * Fd * upd_bytes * B,
            gemm(c->dt, false, false, Epi::SGD, g, st));
      HIPCHK(c, hipEventRecord(c->ev_w3, st));
    }
    if (part & 2) {
      hipStream_t st = us1;
      GemmArgs g2 = ga(c->dh12d[i], 2 * Fd, c->xn_d[i], d, 2 * Fd, d, n, c->m12[i], d);
      g2.C2 = c->dw12[i];
      g2.C3 = c->sr_round ? nullptr : c->dw12_lo[i];
      g2.seed = c->sr_round ? sr_seed(a0 / c->b, i, 1) : 0u;
      g2.scale = lr;
      Bat bt;
      bt.n = B;
      bt.sA = (long)n * 2 * Fd;
      bt.sB = (long)n * d;
      bt.sC = bt.sC2 = 2L * Fd * d;
      set_batch(g2, bt);
      TCALL(KC_SGD, gfl(2 * Fd, d, n) * B, 2.0 * Fd * d * upd_bytes * B,
            gemm(c->dt, false, false, Epi::SGD, g2, st));
      // the block's update is done once both products are
      HIPCHK(c, hipStreamWaitEvent(st, c->ev_w3, 0));
      HIPCHK(c, hipEventRecord(c->ev_upd[i], st));
    }
  }
  return TTT_OK;
}

ttt_status loop_backward(ttt_ctx* c, int64_t a0, int n, hipStream_t st) {
  const int d = c->d, H = c->H, Hk = c->Hk, dh = c->dh, QKV = c->QKV, s = c->s, F = c->F, Fd = c->Fd;
  const int B = c->B, nb = B * n;
  const size_t es = c->es;
  const float lr = c->cfg.alpha;
  const double upd_bytes = 8.0 + (c->dt == DT::F32 ? 0.0 : (double)c->es);  // master r/w + working copy
  int ns = 1;
  const int nd = c->nd;
  // lm_head^T and the final norm
  RUN(gemm_nn_split(c, KC_LM, c->dz, c->V, c->lm_head, d, nb, d, c->V, c->part, &ns, st));
  TCALL(KC_OT, 0, 0, rmsnorm_bwd(c->dt, c->part, c->dt == DT::BF16, ns, c->h_f, c->final_norm, c->r_f, nb, d, c->gh, c->ghd_t[nd - 1], 0, st));
  for (int l = c->L - 1; l >= s; --l) {
    const int i = l - s;
    void* gt = c->ghd_t[i];
    // dynamic MLP: dHmid = dY W3 with the SwiGLU backward in the epilogue
    {
      GemmArgs g = ga(gt, d, c->dw3[i], Fd, n, Fd, d, c->dh12d[i], 2 * Fd);
      g.X = c->h12_d[i];
      Bat bt;
      bt.n = B;
      bt.sA = (long)n * d;
      bt.sB = (long)d * Fd;
      bt.sC = (long)n * 2 * Fd;
      bt.sX = (long)n * 2 * Fd;
      set_batch(g, bt);
      TCALL(KC_GL, gfl(nb, Fd, d), 0, gemm(c->dt, true, false, Epi::SWIGLU_BWD, g, st));
    }
    if (l > s) {
      Bat bt;
      bt.n = B;
      bt.sA = (long)n * 2 * Fd;
      bt.sB = 2L * Fd * d;
      RUN(gemm_nn_split(c, KC_GL, c->dh12d[i], 2 * Fd, c->dw12[i], d, n, d, 2 * Fd, c->part, &ns, st, bt));
    }
    // the update of this block when its attention backward starts, so that
    // it runs beside the attention backward and the next products rather
    // than this block's data-gradient products (with the epilogue's
    // streamed master: 2246-2249 against 2262-2264 ms per 3B step after the
    // query-side kernel and 2269-2271 here, one box; block s has no
    // attention backward in the loop; TTT_UPDATE_AT=now launches here, =dq
    // after the query-side kernel, =split dW3 here and dW12 at the
    // attention backward)
    if (!c->upd_at_attn || l == s) RUN(launch_update(c, i, a0, n, st));
    else if (c->upd_split) RUN(launch_update(c, i, a0, n, st, 1));
    if (l == s) break;
    TCALL(KC_OT, 0, 0, rmsnorm_bwd(c->dt, c->part, c->dt == DT::BF16, ns, c->h_dyn[i], c->dyn_norm[i], c->r_dyn[i], nb, d, c->gh, c->gh_t, 1, st));
    // static MLP
    {
      GemmArgs g = ga(c->gh_t, d, c->w3[l], F, nb, F, d, c->dh12, 2 * F);
      g.X = c->h12_s[i];
      TCALL(KC_GL, gfl(nb, F, d), 0, gemm(c->dt, true, false, Epi::SWIGLU_BWD, g, st));
      RUN(gemm_nn_split(c, KC_GL, c->dh12, 2 * F, c->w12[l], d, nb, d, 2 * F, c->part, &ns, st));
      TCALL(KC_OT, 0, 0, rmsnorm_bwd(c->dt, c->part, c->dt == DT::BF16, ns, c->h_mlp[i], c->mlp_norm[l], c->r_mlp[i], nb, d, c->gh, c->gh_t, 1, st));
    }
    // attention
    {
      TCALL(KC_GL, gfl(nb, H * dh, d), 0,
            gemm(c->dt, true, false, Epi::STORE, ga(c->gh_t, d, c->wo[l], (long)H * dh, nb, H * dh, d, c->dO, (long)H * dh), st));
      bool upd_done = false;
      if (c->upd_at_attn && !c->upd_after_dq) {
        RUN(launch_update(c, i, a0, n, st, c->upd_split ? 2 : 3));
        upd_done = true;
      }
      for (int j = 0; j < B; ++j) {
        const size_t qe = (size_t)n * H * dh;
        void* dO = sq(c->dO, j, qe, es);
        void* o = sq(c->o_l[i], j, qe, es);
        float* D = sqf(c->Dbuf, j, (size_t)H * n);
        TCALL(KC_OT, 0, 0, attn_rowdot(c->dt, dO, o, n, H, dh, D, st));
        AttnArgs a = attn_args(c, l, j, sq(c->q_l[i], j, qe, es), o, sqf(c->lse[i], j, (size_t)H * n), n, a0);
        a.dO = dO;
        a.D = D;
        a.dq = sqf(c->dq, j, (size_t)ATTN_BWD2_MAX_DQ_PARTS * c->b * H * dh);
        a.dk = sqf(c->dk, j, kv_part_elems(c));
        a.dv = sqf(c->dv, j, kv_part_elems(c));
        int qp = 1, kp = 1, krun = 0;
        const bool bwd2 = attn_bwd2_supported(c->dt, a);
        // the second-generation kernels' partial sums in bf16 (like the
        // split-K data-gradient products'): the RoPE backward that adds
        // them reads half the bytes
        a.parts_bf16 = bwd2;
        if (bwd2) {
          qp = attn_bwd2_dq_parts(a);
          kp = attn_bwd2_kv_parts(a);
          krun = attn_bwd2_kv_run(a);
          TCALL(KC_AB, 4.0 * H * dh * window_pairs(a0, n, c->k), 0, attn_bwd_dq2(c->dt, a, st));
        if (c->upd_at_attn && !upd_done && j == B - 1) {
          RUN(launch_update(c, i, a0, n, st, c->upd_split ? 2 : 3));
          upd_done = true;
        }
          TCALL(KC_AB, 4.0 * H * dh * 0.5 * n * (n + 1.0), 0, attn_bwd_dkdv2(c->dt, a, st));
        } else {
          TCALL(KC_AB, 4.0 * H * dh * window_pairs(a0, n, c->k), 0, attn_bwd_dq(c->dt, a, st));
          TCALL(KC_AB, 4.0 * H * dh * 0.5 * n * (n + 1.0), 0, attn_bwd_dkdv(c->dt, a, st));
        }
        if (a.parts_bf16)
          TCALL(KC_OT, 0, 0, rope_bwd_pack(c->dt, (const __bf16*)a.dq, qp, (const __bf16*)a.dk, (const __bf16*)a.dv, kp, krun, a.window, n, H,
                                           Hk, dh, a0, c->rope, sq(c->dqkv, j, (size_t)n * QKV, es), st));
        else
          TCALL(KC_OT, 0, 0, rope_bwd_pack(c->dt, a.dq, qp, a.dk, a.dv, kp, krun, a.window, n, H, Hk, dh, a0, c->rope,
                                           sq(c->dqkv, j, (size_t)n * QKV, es), st));
      }
      if (c->upd_at_attn && !upd_done) RUN(launch_update(c, i, a0, n, st, c->upd_split ? 2 : 3));
      RUN(gemm_nn_split(c, KC_GL, c->dqkv, QKV, c->wqkv[l], d, nb, d, QKV, c->part, &ns, st));
      TCALL(KC_OT, 0, 0, rmsnorm_bwd(c->dt, c->part, c->dt == DT::BF16, ns, c->h_att[i], c->attn_norm[l], c->r_att[i], nb, d, c->gh, c->ghd_t[i - 1], 1, st));
    }
  }
  // the next mini-batch's forward waits for each block's update just before
  // it first touches that block's update inputs (loop_forward)
  return TTT_OK;
}

// Decode blocks of one token: reads the token from d_tok and the position
// from d_pos (device memory, so the sequence can be captured once and
// replayed); leaves the final residual row in dec[0 .. d).
ttt_status decode_blocks(ttt_ctx* c, hipStream_t st) {
  const int d = c->d, H = c->H, Hk = c->Hk, dh = c->dh;
  const float eps = c->cfg.rms_eps;
  float* h = c->dec;
  float* qkv = h + d;
  float* q = qkv + c->QKV;
  float* o = q + (size_t)H * dh;
  float* hm = o + (size_t)H * dh;
  float* part = hm + std::max(c->F, c->Fd);
  HIPCHK(c, embed_row(c->dt, c->d_tok, c->embed, d, c->V, h, c->d_err, st));
  for (int l = 0; l < c->L; ++l) {
    HIPCHK(c, gemv_qkv_rope(c->dt, c->wqkv[l], h, c->attn_norm[l], eps, H, Hk, dh, d, c->d_pos, c->rope, q,
                            c->kring[l], c->vring[l], c->vtring[l], (int)c->cap, st));
    HIPCHK(c, decode_attn(c->dt, q, c->kring[l], c->vring[l], c->vtring[l], H, Hk, dh, (int)c->cap, c->k, c->d_pos,
                          part, o, st));
    HIPCHK(c, gemv(c->dt, c->wo[l], o, nullptr, 0.f, d, H * dh, GvEpi::ADD_F32, h, st));
    HIPCHK(c, gemv(c->dt, c->w12[l], h, c->mlp_norm[l], eps, 2 * c->F, d, GvEpi::SWIGLU, hm, st));
    HIPCHK(c, gemv(c->dt, c->w3[l], hm, nullptr, 0.f, d, c->F, GvEpi::ADD_F32, h, st));
    if (l >= c->s) {
      // the dynamic MLP under the current fast weights: the stochastically
      // rounded bf16 working copy the prefill's forward uses (half the bytes
      // of the masters), or the fp32 masters when the working copy is the
      // two-term form (its high term alone would round updates away)
      const int i = l - c->s;
      const bool wc = c->sr_round;
      HIPCHK(c, gemv(wc ? DT::BF16 : DT::F32, wc ? c->dw12[i] : c->m12[i], h, c->dyn_norm[i], eps, 2 * c->Fd, d,
                     GvEpi::SWIGLU, hm, st));
      HIPCHK(c, gemv(wc ? DT::BF16 : DT::F32, wc ? c->dw3[i] : c->m3[i], hm, nullptr, 0.f, d, c->Fd,
                     GvEpi::ADD_F32, h, st));
    }
  }
  return TTT_OK;
}

ttt_status capture_decode(ttt_ctx* c) {
  if (!c->dstream) HIPCHK(c, hipStreamCreateWithFlags(&c->dstream, hipStreamNonBlocking));
  HIPCHK(c, hipStreamBeginCapture(c->dstream, hipStreamCaptureModeThreadLocal));
  const ttt_status r = decode_blocks(c, c->dstream);
  hipGraph_t g = nullptr;
  const hipError_t e = hipStreamEndCapture(c->dstream, &g);
  if (r != TTT_OK) {
    if (g) (void)hipGraphDestroy(g);
    return r;
  }
  if (e != hipSuccess) return fail(c, TTT_ERR_HIP, std::string("decode capture: ") + hipGetErrorString(e));
  const hipError_t e2 = hipGraphInstantiate(&c->dgraph, g, nullptr, nullptr, 0);
  (void)hipGraphDestroy(g);
  if (e2 != hipSuccess) {
    c->dgraph = nullptr;
    return fail(c, TTT_ERR_HIP, std::string("decode graph: ") + hipGetErrorString(e2));
  }
  return TTT_OK;
}

}  // namespace

// ==================================================================== C ABI
extern "C" {

ttt_status ttt_init(const ttt_config* cfg, const ttt_weights* w, void* stream, ttt_ctx** out) {
  if (!out) return TTT_ERR_INVALID_ARG;
  *out = nullptr;
  ttt_status vs = validate(cfg);
  if (vs != TTT_OK) return vs;
  if (!w || !w->embed || !w->lm_head || !w->final_norm || !w->attn_norm || !w->wq || !w->wk || !w->wv ||
      !w->wo || !w->mlp_norm || !w->w1 || !w->w2 || !w->w3)
    return TTT_ERR_INVALID_ARG;
  const int nd0 = cfg->n_dynamic ? cfg->n_dynamic : cfg->n_layers - (3 * cfg->n_layers) / 4;
  if (nd0 > 0 && (!w->dyn_norm || !w->dyn_w1 || !w->dyn_w2 || !w->dyn_w3)) return TTT_ERR_INVALID_ARG;
  for (int l = 0; l < cfg->n_layers; ++l)
    if (!w->attn_norm[l] || !w->wq[l] || !w->wk[l] || !w->wv[l] || !w->wo[l] || !w->mlp_norm[l] ||
        !w->w1[l] || !w->w2[l] || !w->w3[l])
      return TTT_ERR_INVALID_ARG;
  for (int i = 0; i < nd0; ++i)
    if (!w->dyn_norm[i] || !w->dyn_w1[i] || !w->dyn_w2[i] || !w->dyn_w3[i]) return TTT_ERR_INVALID_ARG;

  ttt_ctx* c = new ttt_ctx();
  ttt_status ds = check_device(c);
  if (ds != TTT_OK) {
    delete c;
    return ds;
  }
  hipStream_t st = (hipStream_t)stream;
  c->cfg = *cfg;
  c->dt = cfg->dtype == TTT_BF16 ? DT::BF16 : DT::F32;
  c->es = dt_size(c->dt);
  c->L = cfg->n_layers;
  c->d = cfg->d_model;
  c->H = cfg->n_heads;
  c->Hk = cfg->n_kv_heads;
  c->dh = cfg->head_dim;
  c->F = cfg->ffn_hidden;
  c->Fd = cfg->dyn_ffn_hidden;
  c->V = cfg->vocab;
  c->k = (int)eff_window(*cfg);
  c->b = cfg->minibatch;
  c->nd = nd0;
  c->s = c->L - c->nd;
  c->max_seq = cfg->max_seq;
  c->QKV = (c->H + 2 * c->Hk) * c->dh;
  ring_shape(*cfg, &c->slab, &c->cap);
  c->max_split = 16;
  c->B = cfg->n_seq > 0 ? cfg->n_seq : 1;
  c->ring_seq = (size_t)c->Hk * c->cap * c->dh;
  // bf16 working copy of the fast weights: one copy rounded stochastically
  // from the fp32 master (default), or, with TTT_WEIGHT_ROUNDING=nearest, the
  // master rounded to nearest plus a low term (two bf16 terms in the forward)
  {
    const char* wr = getenv("TTT_WEIGHT_ROUNDING");
    c->sr_round = c->dt == DT::BF16 && !(wr && strcmp(wr, "nearest") == 0);
    // the forward's residual products leave their split-K partial sums in
    // bf16 (as the backward's data gradients do), fp32 with
    // TTT_FWD_PARTIALS=f32
    const char* fp = getenv("TTT_FWD_PARTIALS");
    c->fwd_parts_bf16 = c->dt == DT::BF16 && !(fp && strcmp(fp, "f32") == 0);
  }
  const size_t es = c->es;
  const int d = c->d, L = c->L, nd = c->nd, B = c->B, b = c->b * c->B;  // b: loop rows (B mini-batches)
  const int64_t S = c->slab;
  const int Fm = std::max(c->F, c->Fd);

  bool ok = true;
  auto A = [&](void** p, size_t bytes) { ok = ok && dalloc(c, p, bytes); };
  auto Af = [&](float** p, size_t n) { ok = ok && dalloc_t(c, p, n * 4); };

  A(&c->embed, (size_t)c->V * d * es);
  if (w->lm_head == w->embed) c->lm_head = c->embed;
  else A(&c->lm_head, (size_t)c->V * d * es);
  Af(&c->final_norm, d);
  c->attn_norm.resize(L);
  c->mlp_norm.resize(L);
  c->wqkv.resize(L);
  c->wo.resize(L);
  c->w12.resize(L);
  c->w3.resize(L);
  c->kring.resize(L);
  c->vring.resize(L);
  c->vtring.resize(L);
  for (int l = 0; l < L && ok; ++l) {
    Af(&c->attn_norm[l], d);
    Af(&c->mlp_norm[l], d);
    A(&c->wqkv[l], (size_t)c->QKV * d * es);
    A(&c->wo[l], (size_t)d * c->H * c->dh * es);
    A(&c->w12[l], (size_t)2 * c->F * d * es);
    A(&c->w3[l], (size_t)d * c->F * es);
    A(&c->kring[l], B * c->ring_seq * es);
    A(&c->vring[l], B * c->ring_seq * es);
    if (c->dt == DT::BF16) A(&c->vtring[l], B * c->ring_seq * es);
  }
  c->dyn_norm.resize(nd);
  c->m12.resize(nd);
  c->m3.resize(nd);
  c->dw12.resize(nd);
  c->dw3.resize(nd);
  c->dw12_lo.assign(nd, nullptr);
  c->dw3_lo.assign(nd, nullptr);
  c->w0_12.resize(nd);
  c->w0_3.resize(nd);
  for (int i = 0; i < nd && ok; ++i) {
    Af(&c->dyn_norm[i], d);
    Af(&c->m12[i], (size_t)B * 2 * c->Fd * d);
    Af(&c->m3[i], (size_t)B * d * c->Fd);
    if (c->dt == DT::F32) {
      c->dw12[i] = c->m12[i];
      c->dw3[i] = c->m3[i];
    } else {
      A(&c->dw12[i], (size_t)B * 2 * c->Fd * d * es);
      A(&c->dw3[i], (size_t)B * d * c->Fd * es);
      if (!c->sr_round) {
        A(&c->dw12_lo[i], (size_t)B * 2 * c->Fd * d * es);
        A(&c->dw3_lo[i], (size_t)B * d * c->Fd * es);
      }
    }
    A(&c->w0_12[i], (size_t)2 * c->Fd * d * es);
    A(&c->w0_3[i], (size_t)d * c->Fd * es);
  }
  {
    void* p = nullptr;
    A(&p, (size_t)c->max_seq * (c->dh / 2) * sizeof(float2));
    c->rope = (float2*)p;
  }
  Af(&c->hres, (size_t)B * c->max_seq * d);
  Af(&c->rbuf, (size_t)S);
  A(&c->xn, (size_t)S * d * es);
  A(&c->qkv, (size_t)S * c->QKV * es);
  A(&c->qb, (size_t)S * c->H * c->dh * es);
  A(&c->ob, (size_t)S * c->H * c->dh * es);
  A(&c->hmid, (size_t)S * Fm * es);
  c->h_att.resize(nd);
  c->h_mlp.resize(nd);
  c->h_dyn.resize(nd);
  c->r_att.resize(nd);
  c->r_mlp.resize(nd);
  c->r_dyn.resize(nd);
  c->lse.resize(nd);
  c->q_l.resize(nd);
  c->o_l.resize(nd);
  c->h12_s.resize(nd);
  c->xn_d.resize(nd);
  c->h12_d.resize(nd);
  c->hm_d.resize(nd);
  for (int i = 0; i < nd && ok; ++i) {
    Af(&c->h_att[i], (size_t)b * d);
    Af(&c->h_mlp[i], (size_t)b * d);
    Af(&c->h_dyn[i], (size_t)b * d);
    Af(&c->r_att[i], b);
    Af(&c->r_mlp[i], b);
    Af(&c->r_dyn[i], b);
    Af(&c->lse[i], (size_t)c->H * b);
    A(&c->q_l[i], (size_t)b * c->H * c->dh * es);
    A(&c->o_l[i], (size_t)b * c->H * c->dh * es);
    A(&c->h12_s[i], (size_t)b * 2 * c->F * es);
    A(&c->xn_d[i], (size_t)b * d * es);
    A(&c->h12_d[i], (size_t)b * 2 * c->Fd * es);
    A(&c->hm_d[i], (size_t)b * c->Fd * es);
  }
  Af(&c->h_f, (size_t)b * d);
  Af(&c->r_f, b);
  Af(&c->logits, (size_t)b * c->V);
  if (c->dt == DT::BF16) {
    void* p = nullptr;
    A(&p, (size_t)b * ((c->V + 63) / 64) * sizeof(float2));
    c->lse_part = (float2*)p;
  }
  A(&c->dz, (size_t)b * c->V * es);
  Af(&c->gh, (size_t)b * d);
  A(&c->gh_t, (size_t)b * d * es);
  A(&c->dh12, (size_t)b * 2 * Fm * es);
  Af(&c->part, (size_t)c->max_split * b * d);
  A(&c->dO, (size_t)b * c->H * c->dh * es);
  Af(&c->Dbuf, (size_t)c->H * b);
  // room for the partial sums of the second-generation backward (at most
  // ATTN_BWD2_MAX_DQ_PARTS key splits of dq, ATTN_BWD2_MAX_KV_PARTS runs of
  // dk / dv)
  Af(&c->dq, (size_t)ATTN_BWD2_MAX_DQ_PARTS * b * c->H * c->dh);
  Af(&c->apart, (size_t)4 * b * c->H * c->dh);
  Af(&c->aml, (size_t)4 * 2 * c->H * b);
  Af(&c->dk, (size_t)c->B * kv_part_elems(c));
  Af(&c->dv, (size_t)c->B * kv_part_elems(c));
  A(&c->dqkv, (size_t)b * c->QKV * es);
  c->ghd_t.assign(nd, nullptr);
  c->dh12d.assign(nd, nullptr);
  for (int i = 0; i < nd && ok; ++i) {
    A(&c->ghd_t[i], (size_t)b * d * es);
    A(&c->dh12d[i], (size_t)b * 2 * c->Fd * es);
  }
  if (ok && hipStreamCreateWithFlags(&c->side, hipStreamNonBlocking) != hipSuccess) ok = false;
  if (ok && hipStreamCreateWithFlags(&c->side2, hipStreamNonBlocking) != hipSuccess) ok = false;
  if (ok && hipEventCreateWithFlags(&c->ev_w3, hipEventDisableTiming) != hipSuccess) ok = false;
  c->ev_dyn.assign(nd, nullptr);
  c->ev_upd.assign(nd, nullptr);
  for (int i = 0; i < nd && ok; ++i)
    if (hipEventCreateWithFlags(&c->ev_upd[i], hipEventDisableTiming) != hipSuccess) ok = false;
  for (int i = 0; i < nd && ok; ++i)
    if (hipEventCreateWithFlags(&c->ev_dyn[i], hipEventDisableTiming) != hipSuccess) ok = false;
  if (ok && hipEventCreateWithFlags(&c->ev_join, hipEventDisableTiming) != hipSuccess) ok = false;
  {
    void* p = nullptr;
    A(&p, 64);
    c->d_err = (int*)p;
    A(&p, 64);
    c->d_pos = (int64_t*)p;
    A(&p, 64);
    c->d_tok = (int32_t*)p;
    A(&p, (size_t)B * c->max_seq * sizeof(int32_t));
    c->tokhist = (int32_t*)p;
  }
  Af(&c->dloss, (size_t)c->b);
  c->dec_split = decode_attn_splits(c->dt, c->H, c->Hk, c->dh, c->k, c->dt == DT::BF16);
  // bf16 update products: two GEMM launches with the SGD epilogue on two
  // side streams (default), or, with TTT_UPDATE_KERNEL=fused, both in one
  // persistent wave-specialised launch (dw_sgd; TTT_UPDATE_GRID sets its
  // grid). The fused launch passes the same parity tests but is slower at
  // the 3B shape (about 470 vs 340 us per block in isolation): its MFMA
  // waves, one per SIMD, wait for every K step's operand loads.
  {
    const char* uk = getenv("TTT_UPDATE_KERNEL");
    c->fused_update = c->dt == DT::BF16 && B == 1 && !c->sr_round && uk && strcmp(uk, "fused") == 0;
    const char* ua = getenv("TTT_UPDATE_AT");
    // default "attn": when the block's attention backward starts
    c->upd_at_attn = !(ua && strcmp(ua, "now") == 0);
    c->upd_split = ua && strcmp(ua, "split") == 0;
    c->upd_after_dq = ua && strcmp(ua, "dq") == 0;
    const char* us = getenv("TTT_UPDATE_STREAM");
    c->upd_main = us && strcmp(us, "main") == 0;
    const char* ug = getenv("TTT_UPDATE_GRID");
    c->upd_grid = ug ? std::max(0, atoi(ug)) : 0;
  }
  Af(&c->dec, (size_t)4 * (c->QKV + 2 * Fm + 2 * d + c->H * c->dh) +
                  (size_t)c->H * c->dec_split * (c->dh + 2));
  if (!ok) {
    ttt_destroy(c);
    return TTT_ERR_OOM;
  }

  // ---- upload / repack
  auto fin = [&](ttt_status s) {
    if (s != TTT_OK) {
      ttt_destroy(c);
      return s;
    }
    *out = c;
    return TTT_OK;
  };
#define UP(call)                                            \
  do {                                                      \
    if ((call) != hipSuccess) {                             \
      (void)hipGetLastError();                              \
      return fin(TTT_ERR_HIP);                              \
    }                                                       \
  } while (0)
  const hipMemcpyKind D2D = hipMemcpyDeviceToDevice;
  UP(hipMemcpyAsync(c->embed, w->embed, (size_t)c->V * d * es, D2D, st));
  if (c->lm_head != c->embed) UP(hipMemcpyAsync(c->lm_head, w->lm_head, (size_t)c->V * d * es, D2D, st));
  UP(cast_from(c->dt, w->final_norm, c->final_norm, d, st));
  const size_t qsz = (size_t)c->H * c->dh * d * es, ksz = (size_t)c->Hk * c->dh * d * es;
  for (int l = 0; l < L; ++l) {
    UP(cast_from(c->dt, w->attn_norm[l], c->attn_norm[l], d, st));
    UP(cast_from(c->dt, w->mlp_norm[l], c->mlp_norm[l], d, st));
    UP(hipMemcpyAsync(c->wqkv[l], w->wq[l], qsz, D2D, st));
    UP(hipMemcpyAsync((char*)c->wqkv[l] + qsz, w->wk[l], ksz, D2D, st));
    UP(hipMemcpyAsync((char*)c->wqkv[l] + qsz + ksz, w->wv[l], ksz, D2D, st));
    UP(hipMemcpyAsync(c->wo[l], w->wo[l], (size_t)d * c->H * c->dh * es, D2D, st));
    UP(interleave(c->w12[l], w->w1[l], c->F, d, es, 0, st));
    UP(interleave(c->w12[l], w->w2[l], c->F, d, es, 1, st));
    UP(hipMemcpyAsync(c->w3[l], w->w3[l], (size_t)d * c->F * es, D2D, st));
    UP(fill_zero_bytes(c->kring[l], B * c->ring_seq * es, st));
    UP(fill_zero_bytes(c->vring[l], B * c->ring_seq * es, st));
    if (c->vtring[l]) UP(fill_zero_bytes(c->vtring[l], B * c->ring_seq * es, st));
  }
  for (int i = 0; i < nd; ++i) {
    UP(cast_from(c->dt, w->dyn_norm[i], c->dyn_norm[i], d, st));
    UP(interleave(c->w0_12[i], w->dyn_w1[i], c->Fd, d, es, 0, st));
    UP(interleave(c->w0_12[i], w->dyn_w2[i], c->Fd, d, es, 1, st));
    UP(hipMemcpyAsync(c->w0_3[i], w->dyn_w3[i], (size_t)d * c->Fd * es, D2D, st));
  }
  // RoPE table: angle = pos * theta^(-2j/dh) in float64, stored as fp32 (cos, sin).
  {
    const int half = c->dh / 2;
    std::vector<float2> tab((size_t)c->max_seq * half);
    std::vector<double> inv(half);
    for (int j = 0; j < half; ++j) inv[j] = 1.0 / pow((double)c->cfg.rope_theta, 2.0 * j / c->dh);
    for (int64_t p = 0; p < c->max_seq; ++p)
      for (int j = 0; j < half; ++j) {
        const double ang = (double)p * inv[j];
        tab[(size_t)p * half + j] = make_float2((float)cos(ang), (float)sin(ang));
      }
    UP(hipMemcpyAsync(c->rope, tab.data(), tab.size() * sizeof(float2), hipMemcpyHostToDevice, st));
    UP(hipStreamSynchronize(st));
  }
  UP(fill_i32(c->d_err, 0, 16, st));
  UP(hipStreamSynchronize(st));
  ttt_status rs = ttt_reset(c, stream);
  if (rs != TTT_OK) return fin(rs);
  UP(hipStreamSynchronize(st));
#undef UP
  return fin(TTT_OK);
}

ttt_status ttt_reset(ttt_ctx* c, void* stream) {
  if (!c) return TTT_ERR_INVALID_ARG;
  hipStream_t st = (hipStream_t)stream;
  const size_t es = c->es;
  for (int i = 0; i < c->nd; ++i) {
    const size_t n12 = (size_t)2 * c->Fd * c->d, n3 = (size_t)c->d * c->Fd;
    for (int j = 0; j < c->B; ++j) {
      HIPCHK(c, cast_from(c->dt, c->w0_12[i], c->m12[i] + j * n12, n12, st));
      HIPCHK(c, cast_from(c->dt, c->w0_3[i], c->m3[i] + j * n3, n3, st));
      if (c->dt != DT::F32) {
        // W0 is exact in the storage dtype: working copy = W0, low term = 0
        HIPCHK(c, hipMemcpyAsync(sq(c->dw12[i], j, n12, es), c->w0_12[i], n12 * es, hipMemcpyDeviceToDevice, st));
        HIPCHK(c, hipMemcpyAsync(sq(c->dw3[i], j, n3, es), c->w0_3[i], n3 * es, hipMemcpyDeviceToDevice, st));
      }
    }
    if (c->dw12_lo[i]) HIPCHK(c, fill_zero_bytes(c->dw12_lo[i], c->B * n12 * es, st));
    if (c->dw3_lo[i]) HIPCHK(c, fill_zero_bytes(c->dw3_lo[i], c->B * n3 * es, st));
  }
  c->pos = 0;
  c->trained = 0;
  return TTT_OK;
}

ttt_status ttt_prefill(ttt_ctx* c, const int32_t* tok, int64_t T, float* loss, float* last_logits,
                       void* stream) {
  if (!c) return TTT_ERR_INVALID_ARG;
  if (!tok || !loss) return fail(c, TTT_ERR_INVALID_ARG, "null tokens or loss");
  if (T < 2 || T > c->max_seq) return fail(c, TTT_ERR_INVALID_ARG, "T outside [2, max_seq]");
  if (c->pos != 0) return fail(c, TTT_ERR_STATE, "prefill needs position 0 (call ttt_reset)");
  hipStream_t st = (hipStream_t)stream;
  // sequence j's tokens go to row j of the token history; every later step
  // reads them from there
  HIPCHK(c, hipMemcpy2DAsync(c->tokhist, (size_t)c->max_seq * sizeof(int32_t), tok, (size_t)T * sizeof(int32_t),
                             (size_t)T * sizeof(int32_t), c->B, hipMemcpyDeviceToDevice, st));
  ttt_status r = TTT_OK;
  for (int j = 0; j < c->B; ++j) {
    r = run_prefix(c, j, c->tokhist + (size_t)j * c->max_seq, 0, T, st);
    if (r != TTT_OK) return r;
  }
  const float red_sum = c->cfg.reduction == TTT_LOSS_SUM;
  for (int64_t a0 = 0; a0 < T; a0 += c->b) {
    const int n = (int)std::min<int64_t>(c->b, T - a0);
    r = loop_forward(c, a0, n, st);
    if (r != TTT_OK) return r;
    if (a0 + n == T && last_logits)
      HIPCHK(c, hipMemcpy2DAsync(last_logits, (size_t)c->V * 4, c->logits + (size_t)(n - 1) * c->V,
                                 (size_t)n * c->V * 4, (size_t)c->V * 4, c->B, hipMemcpyDeviceToDevice, st));
    const int nt = (int)(std::min<int64_t>(a0 + n, T - 1) - a0);
    if (nt <= 0) continue;
    const float scale = red_sum ? 1.f : 1.f / nt;
    r = run_ce(c, a0, n, nt, scale, loss + a0, T - 1, st);
    if (r != TTT_OK) return r;
    r = loop_backward(c, a0, n, st);
    if (r != TTT_OK) return r;
  }
  // the caller's stream sees every update
  HIPCHK(c, hipEventRecord(c->ev_join, c->side));
  HIPCHK(c, hipStreamWaitEvent(st, c->ev_join, 0));
  HIPCHK(c, set_pos(c->d_pos, T, st));
  c->pos = T;
  c->trained = T - 1;  // position T - 1 has no target yet
  return TTT_OK;
}

ttt_status ttt_decode_step(ttt_ctx* c, const int32_t* token, float* logits, void* stream) {
  if (!c) return TTT_ERR_INVALID_ARG;
  if (!token || !logits) return fail(c, TTT_ERR_INVALID_ARG, "null token or logits");
  if (c->B > 1) return fail(c, TTT_ERR_UNSUPPORTED, "decode runs on single-sequence contexts (n_seq 1)");
  if (c->pos < 1 || c->pos >= c->max_seq)
    return fail(c, TTT_ERR_STATE, "decode needs a prefilled context with position < max_seq");
  hipStream_t st = (hipStream_t)stream;
  HIPCHK(c, hipMemcpyAsync(c->d_tok, token, sizeof(int32_t), hipMemcpyDeviceToDevice, st));
  HIPCHK(c, hipMemcpyAsync(c->tokhist + c->pos, token, sizeof(int32_t), hipMemcpyDeviceToDevice, st));
  const char* eg = getenv("TTT_DECODE_GRAPH");
  const bool use_graph = !(eg && eg[0] == '0');
  if (use_graph) {
    if (!c->dgraph) {
      ttt_status r = capture_decode(c);
      if (r != TTT_OK) return r;
    }
    HIPCHK(c, hipGraphLaunch(c->dgraph, st));
  } else {
    ttt_status r = decode_blocks(c, st);
    if (r != TTT_OK) return r;
  }
  HIPCHK(c, gemv(c->dt, c->lm_head, c->dec, c->final_norm, c->cfg.rms_eps, c->V, c->d, GvEpi::STORE, logits, st));
  HIPCHK(c, bump_pos(c->d_pos, st));
  ++c->pos;
  return TTT_OK;
}

ttt_status ttt_decode_step_update(ttt_ctx* c, const int32_t* token, float* logits, float* loss,
                                  int32_t* updated, void* stream) {
  if (!c) return TTT_ERR_INVALID_ARG;
  if (updated) *updated = 0;
  if (!token || !logits) return fail(c, TTT_ERR_INVALID_ARG, "null token or logits");
  if (c->B > 1) return fail(c, TTT_ERR_UNSUPPORTED, "decode runs on single-sequence contexts (n_seq 1)");
  if (c->pos < 1 || c->pos >= c->max_seq)
    return fail(c, TTT_ERR_STATE, "decode needs a prefilled context with position < max_seq");
  hipStream_t st = (hipStream_t)stream;
  const int64_t p = c->pos, u = c->trained;
  if (p - u >= c->b) {
    // the b positions [u, u + b) have all their targets (the last is at
    // most this token): the inner-loop step on them, as a prefill
    // mini-batch would run it
    const int n = c->b;
    HIPCHK(c, hipMemcpyAsync(c->tokhist + p, token, sizeof(int32_t), hipMemcpyDeviceToDevice, st));
    ttt_status r = run_prefix(c, 0, c->tokhist, u, u + n, st);
    if (r != TTT_OK) return r;
    r = loop_forward(c, u, n, st);
    if (r != TTT_OK) return r;
    const float scale = c->cfg.reduction == TTT_LOSS_SUM ? 1.f : 1.f / n;
    r = run_ce(c, u, n, n, scale, loss ? loss : c->dloss, 0, st);
    if (r != TTT_OK) return r;
    r = loop_backward(c, u, n, st);
    if (r != TTT_OK) return r;
    HIPCHK(c, hipEventRecord(c->ev_join, c->side));
    HIPCHK(c, hipStreamWaitEvent(st, c->ev_join, 0));
    c->trained = u + n;
    if (updated) *updated = 1;
  }
  return ttt_decode_step(c, token, logits, stream);
}

ttt_status ttt_get_fast_weights_seq(ttt_ctx* c, int32_t seq, int32_t i, float* w1, float* w2, float* w3,
                                    void* stream) {
  if (!c) return TTT_ERR_INVALID_ARG;
  if (i < 0 || i >= c->nd || !w1 || !w2 || !w3) return fail(c, TTT_ERR_INVALID_ARG, "bad dyn index or null");
  if (seq < 0 || seq >= c->B) return fail(c, TTT_ERR_INVALID_ARG, "sequence index outside [0, n_seq)");
  hipStream_t st = (hipStream_t)stream;
  const size_t n12 = (size_t)2 * c->Fd * c->d, n3 = (size_t)c->d * c->Fd;
  HIPCHK(c, deinterleave(w1, c->m12[i] + seq * n12, c->Fd, c->d, 4, 0, st));
  HIPCHK(c, deinterleave(w2, c->m12[i] + seq * n12, c->Fd, c->d, 4, 1, st));
  HIPCHK(c, hipMemcpyAsync(w3, c->m3[i] + seq * n3, n3 * 4, hipMemcpyDeviceToDevice, st));
  return TTT_OK;
}

ttt_status ttt_get_fast_weights(ttt_ctx* c, int32_t i, float* w1, float* w2, float* w3, void* stream) {
  return ttt_get_fast_weights_seq(c, 0, i, w1, w2, w3, stream);
}

ttt_status ttt_sync(ttt_ctx* c, void* stream) {
  if (!c) return TTT_ERR_INVALID_ARG;
  hipStream_t st = (hipStream_t)stream;
  HIPCHK(c, hipStreamSynchronize(st));
  int flags = 0;
  HIPCHK(c, hipMemcpy(&flags, c->d_err, sizeof(int), hipMemcpyDeviceToHost));
  if (flags) {
    HIPCHK(c, fill_i32(c->d_err, 0, 1, st));
    HIPCHK(c, hipStreamSynchronize(st));
    if (flags & 1) return fail(c, TTT_ERR_TOKEN_RANGE, "token id outside [0, vocab)");
    if (flags & 4) return fail(c, TTT_ERR_NONFINITE, "non-finite loss");
  }
  return TTT_OK;
}

ttt_status ttt_timing_enable(ttt_ctx* c, uint32_t mask) {
  if (!c) return TTT_ERR_INVALID_ARG;
  HIPCHK(c, hipDeviceSynchronize());
  c->tmask = mask;
  c->trecs.clear();
  c->evused = 0;
  return TTT_OK;
}

ttt_status ttt_timing_read(ttt_ctx* c, int32_t kind, double* ms, int64_t* launches, double* flops,
                           double* bytes) {
  if (!c) return TTT_ERR_INVALID_ARG;
  if (kind < 0 || kind >= TTT_KC_COUNT) return fail(c, TTT_ERR_INVALID_ARG, "bad kernel class");
  HIPCHK(c, hipDeviceSynchronize());
  double t = 0, f = 0, b = 0;
  int64_t nl = 0;
  for (const auto& r : c->trecs) {
    if (r.kind != kind) continue;
    float e = 0.f;
    HIPCHK(c, hipEventElapsedTime(&e, r.a, r.b));
    t += e;
    f += r.flops;
    b += r.bytes;
    ++nl;
  }
  if (ms) *ms = t;
  if (launches) *launches = nl;
  if (flops) *flops = f;
  if (bytes) *bytes = b;
  return TTT_OK;
}

int64_t ttt_position(const ttt_ctx* c) { return c ? c->pos : -1; }

const char* ttt_last_error(const ttt_ctx* c) { return c ? c->err.c_str() : "null context"; }

void ttt_destroy(ttt_ctx* c) {
  if (!c) return;
  (void)hipDeviceSynchronize();
  for (hipEvent_t e : c->evpool) (void)hipEventDestroy(e);
  if (c->dgraph) (void)hipGraphExecDestroy(c->dgraph);
  if (c->dstream) (void)hipStreamDestroy(c->dstream);
  for (hipEvent_t e : c->ev_dyn)
    if (e) (void)hipEventDestroy(e);
  for (hipEvent_t e : c->ev_upd)
    if (e) (void)hipEventDestroy(e);
  if (c->ev_join) (void)hipEventDestroy(c->ev_join);
  if (c->ev_w3) (void)hipEventDestroy(c->ev_w3);
  if (c->side) (void)hipStreamDestroy(c->side);
  if (c->side2) (void)hipStreamDestroy(c->side2);
  for (void* p : c->allocs) (void)hipFree(p);
  delete c;
}

}  // extern "C"
