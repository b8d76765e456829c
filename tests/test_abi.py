"""Host-side checks of the C ABI (CPU only: no compute calls)."""
import ctypes

import pytest
import torch

import synth
import test_long_context_amd as tla
from tests.util import header_functions

HAS_GPU = torch.cuda.is_available()


def test_library_exports_every_declared_function():
    lib = tla.lib()
    names = header_functions()
    assert {"ttt_init", "ttt_prefill", "ttt_decode_step", "e2ttt_chunk_scan"} <= set(names)
    for n in names:
        assert hasattr(lib, n), n


def _init(cfg_overrides, ptr=1, max_seq=256):
    c = synth.config("tiny", **cfg_overrides)
    cfg = tla.make_config(c, max_seq=max_seq)
    L = c["n_layers"]
    nd = c["n_dynamic"] or L - (3 * L) // 4
    arrs = []

    def arr(n):
        a = (ctypes.c_void_p * max(1, n))(*([ptr] * n))
        arrs.append(a)
        return ctypes.cast(a, tla._PP)

    W = tla.Weights(embed=ptr, lm_head=ptr, final_norm=ptr)
    for f in ("attn_norm", "wq", "wk", "wv", "wo", "mlp_norm", "w1", "w2", "w3"):
        setattr(W, f, arr(L))
    for f in ("dyn_norm", "dyn_w1", "dyn_w2", "dyn_w3"):
        setattr(W, f, arr(nd))
    h = ctypes.c_void_p()
    return tla.lib().ttt_init(ctypes.byref(cfg), ctypes.byref(W), None, ctypes.byref(h)), h


@pytest.mark.parametrize("over,code", [
    (dict(window=8, minibatch=16), -1),          # k < b
    (dict(minibatch=0), -1),                     # b < 1
    (dict(n_kv_heads=3), -1),                    # H % Hk != 0
    (dict(alpha=float("nan")), -1),              # non-finite step size
    (dict(head_dim=32, d_model=64, n_heads=2, n_kv_heads=2), -2),  # unsupported head size
    (dict(ffn_hidden=200), -2),                  # not a multiple of 32
    (dict(vocab=250), -2),                       # not a multiple of 8
    (dict(d_model=8208), -2),                    # residual row wider than one workgroup keeps
    (dict(prefix_slab=-1), -1),                  # negative prefix slab
    (dict(n_seq=-1), -1),                        # negative sequence count
    (dict(n_seq=65), -1),                        # more sequences than a context takes
    (dict(n_seq=64), None),                      # 64 sequences side by side
    (dict(window=1 << 30), None),                # window clamped to max_seq: a 512-slot ring
    (dict(prefix_slab=64), None),                # small slab: 128-slot ring
    (dict(dtype="bf16", head_dim=128, n_heads=1, n_kv_heads=1, d_model=128), None),
])
def test_init_validates_config_before_touching_the_device(over, code):
    if code is None and HAS_GPU:
        pytest.skip("a valid config would copy from the placeholder pointers")
    st, h = _init(over)
    if code is None:
        assert st == -8   # accepted by validation; no device here
    else:
        assert st == code
    if st == 0:
        tla.lib().ttt_destroy(h)


def test_null_weights_are_rejected():
    st, _ = _init({}, ptr=0)
    assert st == -1


@pytest.mark.skipif(HAS_GPU, reason="checks the no-device path")
def test_valid_config_without_gpu_reports_no_device():
    st, _ = _init({})
    assert st == -8


def test_e2_scan_argument_checks():
    lib = tla.lib()
    f = lib.e2ttt_chunk_scan
    assert f(None, None, None, None, None, None, None, 16, 64, 128, 64, None) == -1
    assert f(1, 1, 1, 1, 1, 1, 1, 16, 64, 96, 64, None) == -2   # D unsupported
    assert f(1, 1, 1, 1, 1, 1, 1, 16, 64, 128, 60, None) == -2  # C not a multiple of 64


def test_ring_slice_of_2_gib_is_unsupported():
    """A ring whose one-key-head slice reaches 2^31 bytes (addressed with
    32-bit offsets) is refused on the host: max_seq 2^30 with a window of
    2^30 needs 2^31 slots of 16 fp32 values."""
    st, _ = _init(dict(window=1 << 30, prefix_slab=1 << 20), max_seq=1 << 30)
    assert st == -2


def test_e2_swiglu_mixer_argument_checks():
    f = tla.lib().e2ttt_mixer_swiglu_forward
    a = [16] * 10  # placeholder, 16-byte aligned pointers: rejected before any device work
    assert f(None, *a[:2], 1e-3, 0.5, 4.0, *a[:7], 2, 64, 128, 64, 64, 64, None) == -1  # null input
    assert f(*a[:3], 1e-3, 0.5, 4.0, *a[:7], 2, 64, 128, 48, 64, 64, None) == -2       # hidden not a multiple of 32
    assert f(*a[:3], 1e-3, 0.5, 4.0, *a[:7], 2, 64, 96, 64, 64, 64, None) == -2       # head size 96
    assert f(*a[:3], 1e-3, 0.5, 4.0, *a[:7], 2, 64, 128, 64, 64, 60, None) == -2      # chunk not a multiple of 64
    assert f(*a[:3], 1e-3, 0.5, 0.0, *a[:7], 2, 64, 128, 64, 64, 64, None) == -1      # tau 0


def test_e2_gelu_mixer_argument_checks():
    f = tla.lib().e2ttt_mixer_gelu_forward
    a = [16] * 10  # placeholder, 16-byte aligned pointers: rejected before any device work
    assert f(None, *a[:2], 1e-3, 0.5, 4.0, *a[:5], 2, 64, 128, 64, 64, 64, None) == -1  # null input
    assert f(*a[:3], 1e-3, 0.5, 4.0, None, *a[:4], 2, 64, 128, 64, 64, 64, None) == -1  # null W1
    assert f(*a[:3], 1e-3, 0.5, 4.0, *a[:5], 2, 64, 128, 48, 64, 64, None) == -2       # hidden not a multiple of 32
    assert f(*a[:3], 1e-3, 0.5, 4.0, *a[:5], 2, 64, 96, 64, 64, 64, None) == -2       # head size 96
    assert f(*a[:3], 1e-3, 0.5, 4.0, *a[:5], 2, 64, 128, 64, 64, 60, None) == -2      # chunk not a multiple of 64
    assert f(*a[:3], 1e-3, 0.5, 4.0, 16, 16, 16, 24, 16, 2, 64, 128, 64, 64, 64, None) == -1  # misaligned M2


def test_e2_hybrid_argument_checks():
    f = tla.lib().e2ttt_hybrid_forward
    a = [16] * 6
    base = (16, 16, 16, 16, 16, 1e-4, 0.5, 4.0, 10000.0)
    dims = (2, 64, 128, 64, 64, None)
    assert f(*base, 0, *a, 0, 16, *dims) == -1            # window 0
    assert f(*base[:8], 1.0, 16, *a, 0, 16, *dims) == -1  # rope base 1
    assert f(*base[:3], None, *base[4:], 16, *a, 0, 16, *dims) == -1  # no gate weights
    assert f(*base, 16, *a, 48, 16, *dims) == -2          # SwiGLU hidden not a multiple of 32
    assert f(*base, 16, 16, 0, 0, 0, 0, 0, -1, 16, *dims) == -1  # negative hidden
