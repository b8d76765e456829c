"""TTT-E2E inner loop on AMD MI355X (gfx950): Python binding of libttt.so.

Argument marshalling only: every step of the path runs in the HIP library
(include/ttt.h); torch provides device memory and the current stream. The
binding raises if the library is missing or a call fails -- there is no
fallback path.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional

PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(PKG, "libttt.so")

TTT_OK = 0
STATUS = {0: "TTT_OK", -1: "TTT_ERR_INVALID_ARG", -2: "TTT_ERR_UNSUPPORTED", -3: "TTT_ERR_OOM",
          -4: "TTT_ERR_HIP", -5: "TTT_ERR_STATE", -6: "TTT_ERR_TOKEN_RANGE",
          -7: "TTT_ERR_NONFINITE", -8: "TTT_ERR_NO_DEVICE"}


class TTTError(RuntimeError):
    def __init__(self, code: int, msg: str = ""):
        self.code = code
        super().__init__(f"{STATUS.get(code, code)}: {msg}")


class Config(ctypes.Structure):
    _fields_ = [("n_layers", ctypes.c_int32), ("d_model", ctypes.c_int32),
                ("n_heads", ctypes.c_int32), ("n_kv_heads", ctypes.c_int32),
                ("head_dim", ctypes.c_int32), ("ffn_hidden", ctypes.c_int32),
                ("dyn_ffn_hidden", ctypes.c_int32), ("vocab", ctypes.c_int32),
                ("window", ctypes.c_int32), ("minibatch", ctypes.c_int32),
                ("n_dynamic", ctypes.c_int32), ("max_seq", ctypes.c_int32),
                ("alpha", ctypes.c_float), ("rms_eps", ctypes.c_float),
                ("rope_theta", ctypes.c_float), ("dtype", ctypes.c_int32),
                ("reduction", ctypes.c_int32), ("prefix_slab", ctypes.c_int32),
                ("n_seq", ctypes.c_int32)]


_PP = ctypes.POINTER(ctypes.c_void_p)


class DwProblem(ctypes.Structure):
    """tttk_dw_problem (include/ttt_kernels.h)."""
    _fields_ = [("A", ctypes.c_void_p), ("lda", ctypes.c_int64), ("B", ctypes.c_void_p),
                ("ldb", ctypes.c_int64), ("W", ctypes.c_void_p), ("Hi", ctypes.c_void_p),
                ("Lo", ctypes.c_void_p), ("ldw", ctypes.c_int64), ("M", ctypes.c_int32),
                ("N", ctypes.c_int32)]


class Weights(ctypes.Structure):
    _fields_ = [("embed", ctypes.c_void_p), ("lm_head", ctypes.c_void_p),
                ("final_norm", ctypes.c_void_p)] + [
        (n, _PP) for n in ("attn_norm", "wq", "wk", "wv", "wo", "mlp_norm", "w1", "w2", "w3",
                           "dyn_norm", "dyn_w1", "dyn_w2", "dyn_w3")]


_lib = None


def lib() -> ctypes.CDLL:
    """Loads libttt.so (built by `python -m test_long_context_amd.build`)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it with "
                               "`python -m test_long_context_amd.build`")
        L = ctypes.CDLL(LIB_PATH)
        vp, i32, i64, st = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_int
        L.ttt_init.argtypes = [ctypes.POINTER(Config), ctypes.POINTER(Weights), vp, ctypes.POINTER(vp)]
        L.ttt_prefill.argtypes = [vp, vp, i64, vp, vp, vp]
        L.ttt_decode_step.argtypes = [vp, vp, vp, vp]
        L.ttt_decode_step_update.argtypes = [vp, vp, vp, vp, ctypes.POINTER(i32), vp]
        L.ttt_get_fast_weights.argtypes = [vp, i32, vp, vp, vp, vp]
        L.ttt_get_fast_weights_seq.argtypes = [vp, i32, i32, vp, vp, vp, vp]
        L.ttt_reset.argtypes = [vp, vp]
        L.ttt_sync.argtypes = [vp, vp]
        L.ttt_position.argtypes = [vp]
        L.ttt_position.restype = i64
        L.ttt_last_error.argtypes = [vp]
        L.ttt_last_error.restype = ctypes.c_char_p
        L.ttt_destroy.argtypes = [vp]
        L.ttt_destroy.restype = None
        L.e2ttt_chunk_scan.argtypes = [vp, vp, vp, vp, vp, vp, vp, i32, i64, i32, i32, vp]
        L.e2ttt_chunk_scan_noalloc.argtypes = [vp, vp, vp, vp, vp, vp, vp, i32, i64, i32, i32, vp]
        L.lact_chunk_scan.argtypes = [vp, vp, vp, vp, vp, vp, i32, i64, i32, i32, vp]
        L.e2ttt_mixer_forward.argtypes = [vp, vp, vp, ctypes.c_float, ctypes.c_float, ctypes.c_float, vp, vp, vp,
                                          i32, i64, i32, i32, i32, vp]
        L.e2ttt_mixer_swiglu_forward.argtypes = [vp, vp, vp, ctypes.c_float, ctypes.c_float, ctypes.c_float,
                                                 vp, vp, vp, vp, vp, vp, vp, i32, i64, i32, i32, i32, i32, vp]
        L.e2ttt_mixer_gelu_forward.argtypes = [vp, vp, vp, ctypes.c_float, ctypes.c_float, ctypes.c_float,
                                               vp, vp, vp, vp, vp, i32, i64, i32, i32, i32, i32, vp]
        L.e2ttt_hybrid_forward.argtypes = [vp, vp, vp, vp, vp, ctypes.c_float, ctypes.c_float, ctypes.c_float,
                                           ctypes.c_float, i32, vp, vp, vp, vp, vp, vp, i32, vp, i32, i64, i32, i32,
                                           i32, vp]
        L.e2ttt_chunk_scan_noalloc_max_bytes.argtypes = []
        L.e2ttt_chunk_scan_noalloc_max_bytes.restype = i64
        L.ttt_timing_enable.argtypes = [vp, ctypes.c_uint32]
        dp, lp = ctypes.POINTER(ctypes.c_double), ctypes.POINTER(ctypes.c_int64)
        L.ttt_timing_read.argtypes = [vp, i32, dp, lp, dp, dp]
        f32 = ctypes.c_float
        L.tttk_gemm.argtypes = [i32, i32, i32, i32, vp, i64, vp, i64, vp, i32, i32, i32, vp, i64, vp, vp,
                                vp, f32, i32, i32, ctypes.c_uint32, vp]
        L.tttk_attn_fwd.argtypes = [i32, vp, vp, vp, vp, vp, vp, i32, i32, i32, i32, i32, i32, i64, i32, i32, vp,
                                    vp]
        L.tttk_attn_fwd_workspace.argtypes = [i32, i32, i32, i32, i32]
        L.tttk_attn_fwd_workspace.restype = i64
        L.tttk_attn_bwd.argtypes = [i32, vp, vp, vp, vp, vp, vp, vp, vp, vp, i32, i32, i32, i32, i32, i32,
                                    i64, i32, vp, vp]
        L.tttk_attn_bwd_workspace.argtypes = [i32, i32, i32, i32, i32, i32, i32]
        L.tttk_attn_bwd_workspace.restype = i64
        L.tttk_ce.argtypes = [i32, vp, i32, i32, i32, vp, f32, vp, vp, vp, vp]
        L.tttk_ce_lse.argtypes = [vp, vp, i32, i32, i32, vp, f32, vp, vp, vp, vp]
        L.tttk_dw_sgd.argtypes = [i32, ctypes.POINTER(DwProblem), i32, f32, i32, vp]
        for f in ("ttt_init", "ttt_prefill", "ttt_decode_step", "ttt_decode_step_update", "ttt_get_fast_weights",
                  "ttt_get_fast_weights_seq",
                  "ttt_reset", "ttt_sync", "e2ttt_chunk_scan", "e2ttt_chunk_scan_noalloc", "lact_chunk_scan", "e2ttt_mixer_forward",
                  "e2ttt_mixer_swiglu_forward", "e2ttt_mixer_gelu_forward", "e2ttt_hybrid_forward",
                  "ttt_timing_enable", "ttt_timing_read", "tttk_gemm", "tttk_attn_fwd", "tttk_attn_bwd", "tttk_ce", "tttk_ce_lse",
                  "tttk_dw_sgd"):
            getattr(L, f).restype = st
        _lib = L
    return _lib


def _stream(stream=None):
    import torch
    if stream is not None:
        return ctypes.c_void_p(stream)
    if torch.cuda.is_available():
        return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    return ctypes.c_void_p(None)


def make_config(c: dict, max_seq: Optional[int] = None) -> Config:
    return Config(n_layers=c["n_layers"], d_model=c["d_model"], n_heads=c["n_heads"],
                  n_kv_heads=c["n_kv_heads"], head_dim=c["head_dim"], ffn_hidden=c["ffn_hidden"],
                  dyn_ffn_hidden=c["dyn_ffn_hidden"], vocab=c["vocab"], window=c["window"],
                  minibatch=c["minibatch"], n_dynamic=c.get("n_dynamic", 0),
                  max_seq=int(max_seq if max_seq is not None else c.get("max_seq", c["seq"])),
                  alpha=float(c["alpha"]), rms_eps=float(c["rms_eps"]),
                  rope_theta=float(c["rope_theta"]), dtype=0 if c["dtype"] == "f32" else 1,
                  reduction=0 if c.get("reduction", "mean") == "mean" else 1,
                  prefix_slab=int(c.get("prefix_slab", 0)), n_seq=int(c.get("n_seq", 0)))


def _ptr(t) -> int:
    if t is None:
        return 0
    if not t.is_contiguous():
        raise ValueError("tensors passed to the library must be contiguous")
    return t.data_ptr()


def _arr(ptrs):
    a = (ctypes.c_void_p * max(1, len(ptrs)))(*ptrs)
    return a, ctypes.cast(a, _PP)


class TTT:
    """One inner-loop context on the current GPU (see include/ttt.h)."""

    def __init__(self, cfg: dict, weights: dict, max_seq: Optional[int] = None, stream=None):
        self.cfg = dict(cfg)
        self._keep = []
        W = Weights(embed=_ptr(weights["embed"]), lm_head=_ptr(weights["lm_head"]),
                    final_norm=_ptr(weights["final_norm"]))
        for f in ("attn_norm", "wq", "wk", "wv", "wo", "mlp_norm", "w1", "w2", "w3"):
            a, p = _arr([_ptr(x[f]) for x in weights["layers"]])
            self._keep.append(a)
            setattr(W, f, p)
        for f, k in (("dyn_norm", "norm"), ("dyn_w1", "w1"), ("dyn_w2", "w2"), ("dyn_w3", "w3")):
            a, p = _arr([_ptr(x[k]) for x in weights["dyn"]])
            self._keep.append(a)
            setattr(W, f, p)
        self.c_cfg = make_config(cfg, max_seq)
        h = ctypes.c_void_p()
        st = lib().ttt_init(ctypes.byref(self.c_cfg), ctypes.byref(W), _stream(stream), ctypes.byref(h))
        if st != TTT_OK:
            raise TTTError(st, "ttt_init")
        self.h = h

    def _chk(self, st, what):
        if st != TTT_OK:
            raise TTTError(st, f"{what}: {lib().ttt_last_error(self.h).decode()}")

    @property
    def n_seq(self) -> int:
        return max(1, int(self.cfg.get("n_seq", 0)))

    def prefill(self, tokens, loss=None, last_logits=None, stream=None):
        """tokens: [T] (one sequence) or [n_seq, T]; returns the losses,
        [T - 1] or [n_seq, T - 1]."""
        import torch
        B = self.n_seq
        T = tokens.shape[-1]
        if tokens.numel() != B * T or (B > 1 and tokens.dim() != 2):
            raise ValueError(f"tokens must hold {B} row(s) of T ids, got shape {tuple(tokens.shape)}")
        if loss is None:
            loss = torch.empty(*((B,) if B > 1 else ()), T - 1, dtype=torch.float32, device=tokens.device)
        if loss.numel() != B * (T - 1) or (last_logits is not None and last_logits.numel() != B * self.cfg["vocab"]):
            raise ValueError("loss must hold n_seq (T - 1) values and last_logits n_seq vocab")
        self._chk(lib().ttt_prefill(self.h, _ptr(tokens), T, _ptr(loss), _ptr(last_logits),
                                    _stream(stream)), "ttt_prefill")
        return loss

    def decode_step(self, token, logits=None, stream=None):
        import torch
        if logits is None:
            logits = torch.empty(self.cfg["vocab"], dtype=torch.float32, device=token.device)
        self._chk(lib().ttt_decode_step(self.h, _ptr(token), _ptr(logits), _stream(stream)),
                  "ttt_decode_step")
        return logits

    def decode_step_update(self, token, logits=None, loss=None, stream=None):
        """Decode with test-time updates (ttt_decode_step_update): returns
        (logits, loss or None); loss holds the b losses of an update made
        before this token's decode."""
        import torch
        if logits is None:
            logits = torch.empty(self.cfg["vocab"], dtype=torch.float32, device=token.device)
        if loss is None:
            loss = torch.empty(self.cfg["minibatch"], dtype=torch.float32, device=token.device)
        upd = ctypes.c_int32(0)
        self._chk(lib().ttt_decode_step_update(self.h, _ptr(token), _ptr(logits), _ptr(loss), ctypes.byref(upd),
                                               _stream(stream)), "ttt_decode_step_update")
        return logits, (loss if upd.value else None)

    def fast_weights(self, i: int, stream=None, seq: int = 0):
        import torch
        d, Fd = self.cfg["d_model"], self.cfg["dyn_ffn_hidden"]
        dev = torch.device("cuda")
        w1 = torch.empty(Fd, d, dtype=torch.float32, device=dev)
        w2 = torch.empty(Fd, d, dtype=torch.float32, device=dev)
        w3 = torch.empty(d, Fd, dtype=torch.float32, device=dev)
        self._chk(lib().ttt_get_fast_weights_seq(self.h, seq, i, _ptr(w1), _ptr(w2), _ptr(w3), _stream(stream)),
                  "ttt_get_fast_weights_seq")
        return w1, w2, w3

    def reset(self, stream=None):
        self._chk(lib().ttt_reset(self.h, _stream(stream)), "ttt_reset")

    def sync(self, stream=None):
        self._chk(lib().ttt_sync(self.h, _stream(stream)), "ttt_sync")

    # live per-kernel-class timing (HIP events on the launch stream)
    KC = ("gemm_prefix", "attn_prefix", "gemm_loop", "attn_loop", "lmhead", "ce", "attn_bwd",
          "dw_sgd", "other")

    def timing_enable(self, mask: int = (1 << 9) - 1):
        self._chk(lib().ttt_timing_enable(self.h, mask), "ttt_timing_enable")

    def timing_read(self, kind: int) -> dict:
        ms, fl, by = ctypes.c_double(), ctypes.c_double(), ctypes.c_double()
        n = ctypes.c_int64()
        self._chk(lib().ttt_timing_read(self.h, kind, ctypes.byref(ms), ctypes.byref(n), ctypes.byref(fl),
                                        ctypes.byref(by)), "ttt_timing_read")
        return dict(kind=self.KC[kind], ms=ms.value, launches=n.value, flops=fl.value, bytes=by.value)

    @property
    def position(self) -> int:
        return int(lib().ttt_position(self.h))

    def close(self):
        if getattr(self, "h", None):
            lib().ttt_destroy(self.h)
            self.h = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass


def e2ttt_chunk_scan(k, v, eta, beta, gamma, W, M, chunk: int, stream=None):
    """In-place E2-TTT chunk-end scan over all chunks (see include/ttt.h)."""
    H, T, D = k.shape
    st = lib().e2ttt_chunk_scan(_ptr(k), _ptr(v), _ptr(eta), _ptr(beta), _ptr(gamma), _ptr(W),
                                _ptr(M), H, T, D, chunk, _stream(stream))
    if st != TTT_OK:
        raise TTTError(st, "e2ttt_chunk_scan")
    return W, M


def lact_chunk_scan(k, v, eta, beta, W, M, chunk: int, stream=None):
    """In-place LaCT chunk-wise scan over all chunks (see include/ttt.h)."""
    H, T, D = k.shape
    st = lib().lact_chunk_scan(_ptr(k), _ptr(v), _ptr(eta), _ptr(beta), _ptr(W), _ptr(M), H, T, D, chunk,
                               _stream(stream))
    if st != TTT_OK:
        raise TTTError(st, "lact_chunk_scan")
    return W, M


def e2ttt_mixer_forward(x, wqkv, bias, eta_base, alpha_base, tau, W, M, heads: int, chunk: int, out=None,
                        stream=None):
    """E2-TTT token mixer, TTT path (see include/ttt.h): returns out [T, H D]."""
    import torch
    T, dm = x.shape
    H, D, _ = W.shape
    assert H == heads
    if out is None:
        out = torch.empty(T, H * D, dtype=torch.float32, device=x.device)
    st = lib().e2ttt_mixer_forward(_ptr(x), _ptr(wqkv), _ptr(bias), float(eta_base), float(alpha_base), float(tau),
                                   _ptr(W), _ptr(M), _ptr(out), H, T, D, dm, chunk, _stream(stream))
    if st != TTT_OK:
        raise TTTError(st, "e2ttt_mixer_forward")
    return out


def e2ttt_mixer_swiglu_forward(x, wqkv, bias, eta_base, alpha_base, tau, state: dict, heads: int, chunk: int,
                               out=None, stream=None):
    """E2-TTT token mixer, TTT path with the SwiGLU fast-weight net (see
    include/ttt.h); state: w1, w2 [H, Dh, D], w3 [H, D, Dh] and momenta m1,
    m2, m3 (float), updated in place. Returns out [T, H D]."""
    import torch
    T, dm = x.shape
    H, Dh, D = state["w1"].shape
    assert H == heads
    if out is None:
        out = torch.empty(T, H * D, dtype=torch.float32, device=x.device)
    st = lib().e2ttt_mixer_swiglu_forward(_ptr(x), _ptr(wqkv), _ptr(bias), float(eta_base), float(alpha_base),
                                          float(tau), *(_ptr(state[n]) for n in ("w1", "w2", "w3", "m1", "m2", "m3")),
                                          _ptr(out), H, T, D, Dh, dm, chunk, _stream(stream))
    if st != TTT_OK:
        raise TTTError(st, "e2ttt_mixer_swiglu_forward")
    return out


def e2ttt_mixer_gelu_forward(x, wqkv, bias, eta_base, alpha_base, tau, state: dict, heads: int, chunk: int,
                             out=None, stream=None):
    """E2-TTT token mixer, TTT path with the GELU fast-weight net (see
    include/ttt.h); state: w1 [H, Dh, D], w2 [H, D, Dh] and momenta m1, m2
    (float), updated in place. Returns out [T, H D]."""
    import torch
    T, dm = x.shape
    H, Dh, D = state["w1"].shape
    assert H == heads
    if out is None:
        out = torch.empty(T, H * D, dtype=torch.float32, device=x.device)
    st = lib().e2ttt_mixer_gelu_forward(_ptr(x), _ptr(wqkv), _ptr(bias), float(eta_base), float(alpha_base),
                                        float(tau), *(_ptr(state[n]) for n in ("w1", "w2", "m1", "m2")),
                                        _ptr(out), H, T, D, Dh, dm, chunk, _stream(stream))
    if st != TTT_OK:
        raise TTTError(st, "e2ttt_mixer_gelu_forward")
    return out


def e2ttt_hybrid_forward(x, wqkv, bias, wgate, bgate, eta_base, alpha_base, tau, rope_theta, window: int,
                         state: dict, heads: int, chunk: int, out=None, stream=None):
    """Hybrid token-mixer block (see include/ttt.h): state is dict(W, M)
    (linear fast weight), dict(w1, w2, w3, m1, m2, m3) (SwiGLU net) or
    dict(w1, w2, m1, m2) (GELU net), updated in place. Returns out [T, H D]."""
    import torch
    T, dm = x.shape
    if "W" in state:
        H, D, _ = state["W"].shape
        Dh = 0
        ptrs = [_ptr(state["W"]), 0, 0, _ptr(state["M"]), 0, 0]
    elif "w3" not in state:
        H, Dh, D = state["w1"].shape
        ptrs = [_ptr(state["w1"]), _ptr(state["w2"]), 0, _ptr(state["m1"]), _ptr(state["m2"]), 0]
    else:
        H, Dh, D = state["w1"].shape
        ptrs = [_ptr(state[n]) for n in ("w1", "w2", "w3", "m1", "m2", "m3")]
    assert H == heads
    if out is None:
        out = torch.empty(T, H * D, dtype=torch.float32, device=x.device)
    st = lib().e2ttt_hybrid_forward(_ptr(x), _ptr(wqkv), _ptr(bias), _ptr(wgate), _ptr(bgate), float(eta_base),
                                    float(alpha_base), float(tau), float(rope_theta), int(window), *ptrs, Dh,
                                    _ptr(out), H, T, D, dm, chunk, _stream(stream))
    if st != TTT_OK:
        raise TTTError(st, "e2ttt_hybrid_forward")
    return out


def e2ttt_chunk_scan_noalloc(k, v, eta, beta, gamma, W, M, chunk: int, stream=None):
    """e2ttt_chunk_scan without device allocation (fixed work buffer; see
    include/ttt.h)."""
    H, T, D = k.shape
    st = lib().e2ttt_chunk_scan_noalloc(_ptr(k), _ptr(v), _ptr(eta), _ptr(beta), _ptr(gamma), _ptr(W),
                                        _ptr(M), H, T, D, chunk, _stream(stream))
    if st != TTT_OK:
        raise TTTError(st, "e2ttt_chunk_scan_noalloc")
    return W, M


def e2ttt_chunk_scan_noalloc_max_bytes() -> int:
    return int(lib().e2ttt_chunk_scan_noalloc_max_bytes())


# ---------------------------------------------------------------- kernel level
EPI = dict(store=0, store_f32=1, add_f32=2, swiglu=3, swiglu_bwd=4, sgd=5, partial=6, store_f32_lse=8)


def _dt(t) -> int:
    import torch
    return 1 if t.dtype == torch.bfloat16 else 0


def _check(st, what):
    if st != TTT_OK:
        raise TTTError(st, what)


def gemm(A, B, M, N, K, epi, C, *, a_kmajor=True, b_kmajor=True, lda=None, ldb=None, ldc=None,
         B2=None, C2=None, C3=None, X=None, scale=1.0, kchunk=0, tile=0, seed=0, stream=None):
    """One GEMM-family launch (include/ttt_kernels.h, tttk_gemm)."""
    lda = lda if lda is not None else (K if a_kmajor else M)
    ldb = ldb if ldb is not None else (K if b_kmajor else N)
    ldc = ldc if ldc is not None else N
    _check(lib().tttk_gemm(_dt(A), int(a_kmajor), int(b_kmajor), EPI[epi], _ptr(A), lda, _ptr(B), ldb,
                           _ptr(B2), M, N, K, _ptr(C), ldc, _ptr(C2), _ptr(C3), _ptr(X), float(scale),
                           int(kchunk), int(tile), int(seed), _stream(stream)), "tttk_gemm")


def attn_fwd_workspace(n, H, dh, window, ksplit=0):
    """Bytes of device workspace tttk_attn_fwd needs (include/ttt_kernels.h)."""
    return int(lib().tttk_attn_fwd_workspace(n, H, dh, window, int(ksplit)))


def attn_fwd(q, k, v, o, lse, n, H, Hk, dh, cap, window, pos0, vt=None, variant=0, ksplit=1, work=None,
             stream=None):
    _check(lib().tttk_attn_fwd(_dt(q), _ptr(q), _ptr(k), _ptr(v), _ptr(vt), _ptr(o), _ptr(lse), n, H, Hk, dh,
                               cap, window, pos0, int(variant), int(ksplit), _ptr(work), _stream(stream)),
           "tttk_attn_fwd")


def attn_bwd_workspace(dtype, n, H, Hk, dh, window, variant=0):
    """Bytes of device workspace tttk_attn_bwd needs (include/ttt_kernels.h);
    dtype is a torch dtype."""
    import torch
    code = 1 if dtype == torch.bfloat16 else 0
    return int(lib().tttk_attn_bwd_workspace(code, n, H, Hk, dh, window, int(variant)))


def attn_bwd(q, k, v, lse, dO, D, dq, dk, dv, n, H, Hk, dh, cap, window, pos0, variant=0, work=None,
             stream=None):
    _check(lib().tttk_attn_bwd(_dt(q), _ptr(q), _ptr(k), _ptr(v), _ptr(lse), _ptr(dO), _ptr(D), _ptr(dq),
                               _ptr(dk), _ptr(dv), n, H, Hk, dh, cap, window, pos0, int(variant), _ptr(work),
                               _stream(stream)),
           "tttk_attn_bwd")


def ce(logits, n, nt, V, labels, scale, loss, dz, err, stream=None):
    _check(lib().tttk_ce(_dt(dz), _ptr(logits), n, nt, V, _ptr(labels), float(scale), _ptr(loss), _ptr(dz),
                         _ptr(err), _stream(stream)), "tttk_ce")


def dw_sgd(problems, K: int, lr: float, grid: int = 0, stream=None):
    """Fused weight-gradient products with the fp32 SGD step (tttk_dw_sgd):
    problems is a list of dicts with A, lda, B, ldb, W, Hi, Lo, ldw, M, N."""
    arr = (DwProblem * len(problems))()
    for i, p in enumerate(problems):
        arr[i] = DwProblem(A=_ptr(p["A"]), lda=p["lda"], B=_ptr(p["B"]), ldb=p["ldb"], W=_ptr(p["W"]),
                           Hi=_ptr(p["Hi"]), Lo=_ptr(p.get("Lo")), ldw=p["ldw"], M=p["M"], N=p["N"])
    _check(lib().tttk_dw_sgd(len(problems), arr, int(K), float(lr), int(grid), _stream(stream)), "tttk_dw_sgd")


def ce_lse(logits, parts, n, nt, V, labels, scale, loss, dz, err, stream=None):
    _check(lib().tttk_ce_lse(_ptr(logits), _ptr(parts), n, nt, V, _ptr(labels), float(scale), _ptr(loss), _ptr(dz),
                             _ptr(err), _stream(stream)), "tttk_ce_lse")
