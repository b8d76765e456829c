"""Kernel-level parity of the GEMM family (include/ttt_kernels.h, tttk_gemm)
against float64 CPU products of the same bf16 / fp32 operands.

Covers every operand layout and tile configuration at a ragged shape (several
tiles plus partial ones in M, N and K), each fused epilogue against its
definition, and the 3B-shape products of the inner loop on sampled outputs.
"""
import numpy as np
import pytest
import torch

from tests.util import say

pytestmark = pytest.mark.gpu

tla = pytest.importorskip("test_long_context_amd")
dev = "cuda"
bf = torch.bfloat16


def rnd(g, *shape, scale=0.5, dtype=bf):
    return (torch.randn(*shape, generator=g, dtype=torch.float32) * scale).to(dtype)


def logical(X, rows, K, kmajor):
    """Operand as a [rows, K] float64 CPU matrix."""
    X = X.double().cpu()
    return X.view(rows, K) if kmajor else X.view(K, rows).T


LAYOUTS = {"nt": (True, True), "nn": (True, False), "tn": (False, True), "tt": (False, False)}


@pytest.mark.parametrize("lay", sorted(LAYOUTS))
@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_gemm_layouts_tiles(lay, dtype):
    ak, bk = LAYOUTS[lay]
    M, N, K = 520, 392, 328
    g = torch.Generator().manual_seed(11)
    dt = bf if dtype == "bf16" else torch.float32
    A = rnd(g, M * K, dtype=dt)
    B = rnd(g, N * K, dtype=dt)
    ref = logical(A, M, K, ak) @ logical(B, N, K, bk).T
    Ad, Bd = A.to(dev), B.to(dev)
    tiles = (1, 2, 3, 4, 5, 6) if dtype == "bf16" else (0,)
    for t in tiles:
        say(f"gemm {lay} {dtype} tile {t} {M}x{N}x{K}")
        C = torch.full((M * N,), float("nan"), device=dev)
        tla.gemm(Ad, Bd, M, N, K, "store_f32", C, a_kmajor=ak, b_kmajor=bk, tile=t)
        err = float((C.cpu().double().view(M, N) - ref).abs().max() / ref.abs().max())
        assert err < 1e-5, (lay, dtype, t, err)


def test_gemm_epilogues():
    g = torch.Generator().manual_seed(12)
    M, N, K = 264, 160, 200
    A = rnd(g, M * K)
    B = rnd(g, N * K)
    Ad, Bd = A.to(dev), B.to(dev)
    acc = logical(A, M, K, True) @ logical(B, N, K, True).T

    # STORE: bf16 of scale * acc
    C = torch.empty(M * N, dtype=bf, device=dev)
    tla.gemm(Ad, Bd, M, N, K, "store", C, scale=0.5)
    want = (0.5 * acc).float().to(bf).double()
    assert float((C.cpu().double().view(M, N) - want).abs().max()) <= float(want.abs().max()) * 2 ** -8

    # ADD_F32
    C0 = rnd(g, M * N, dtype=torch.float32)
    C = C0.to(dev)
    tla.gemm(Ad, Bd, M, N, K, "add_f32", C)
    assert float((C.cpu().double().view(M, N) - (C0.double().view(M, N) + acc)).abs().max()) < 1e-4

    # PARTIAL over K chunks of 64: the chunks sum to the product
    nsp = (K + 63) // 64
    C = torch.empty(nsp * M * N, device=dev)
    tla.gemm(Ad, Bd, M, N, K, "partial", C, kchunk=64)
    assert float((C.cpu().double().view(nsp, M, N).sum(0) - acc).abs().max()) < 1e-4

    # SWIGLU: N columns interleaved (gate, up) in blocks of 16
    C = torch.empty(M * N, dtype=bf, device=dev)
    C2 = torch.empty(M * N // 2, dtype=bf, device=dev)
    tla.gemm(Ad, Bd, M, N, K, "swiglu", C, C2=C2)
    a = acc.view(M, N // 32, 2, 16)[:, :, 0, :].reshape(M, N // 2)
    c = acc.view(M, N // 32, 2, 16)[:, :, 1, :].reshape(M, N // 2)
    want = a / (1 + torch.exp(-a)) * c
    assert float((C2.cpu().double().view(M, N // 2) - want).abs().max()) <= float(want.abs().max()) * 2 ** -7
    assert float((C.cpu().double().view(M, N) - acc).abs().max()) <= float(acc.abs().max()) * 2 ** -8

    # SWIGLU_BWD: acc = dHmid [M, N]; X = pre-activations [M, 2N] (interleaved)
    X = rnd(g, M * 2 * N)
    C = torch.empty(M * 2 * N, dtype=bf, device=dev)
    tla.gemm(Ad, Bd, M, N, K, "swiglu_bwd", C, X=X.to(dev), ldc=2 * N)
    Xd = X.double().view(M, N // 16, 2, 16)
    av, cv = Xd[:, :, 0, :].reshape(M, N), Xd[:, :, 1, :].reshape(M, N)
    sg = 1 / (1 + torch.exp(-av))
    da = acc * cv * sg * (1 + av * (1 - sg))
    dc = acc * av * sg
    got = C.cpu().double().view(M, N // 16, 2, 16)
    for got_part, want_part in ((got[:, :, 0, :].reshape(M, N), da), (got[:, :, 1, :].reshape(M, N), dc)):
        assert float((got_part - want_part).abs().max()) <= float(want_part.abs().max()) * 2 ** -7


@pytest.mark.parametrize("lay", ["tn", "nt"])
def test_gemm_sgd_epilogue(lay):
    """W -= scale * acc on the fp32 master; C2 = bf16(W); C3 = bf16(W - C2)."""
    ak, bk = LAYOUTS[lay]
    g = torch.Generator().manual_seed(13)
    M, N, K = 392, 264, 136
    A = rnd(g, M * K)
    B = rnd(g, N * K)
    W0 = rnd(g, M * N, scale=0.02, dtype=torch.float32)
    W = W0.to(dev)
    hi = torch.empty(M * N, dtype=bf, device=dev)
    lo = torch.empty(M * N, dtype=bf, device=dev)
    tla.gemm(A.to(dev), B.to(dev), M, N, K, "sgd", W, a_kmajor=ak, b_kmajor=bk, C2=hi, C3=lo, scale=1e-3)
    acc = logical(A, M, K, ak) @ logical(B, N, K, bk).T
    want = W0.double().view(M, N) - 1e-3 * acc
    Wg = W.cpu().double().view(M, N)
    assert float((Wg - want).abs().max()) < 1e-6
    # hi is the RNE of the stored master, lo the RNE of the remainder
    Wf = W.cpu().view(M, N)
    assert torch.equal(hi.cpu().view(M, N), Wf.to(bf))
    assert torch.equal(lo.cpu().view(M, N), (Wf - Wf.to(bf).float()).to(bf))


def test_gemm_sgd_stochastic_rounding():
    """seed != 0: the master update is unchanged and the bf16 working copy is
    one of the master's two bf16 neighbours, rounded up with probability
    equal to the dropped fraction of an ulp -- unbiased where rounding to
    nearest is not. The product is zero (A = 0) so the master keeps values
    placed at known fractions 0.1, 0.3, 0.5 and 0.8 of an ulp above a bf16
    value; 32768 entries per fraction."""
    M, N, K = 256, 512, 64
    g = torch.Generator().manual_seed(17)
    base = (torch.randn(M * N, generator=g) * 0.02).to(bf).float()
    ulp = ((base.view(torch.int32) + (1 << 16)).view(torch.float32) - base).abs()
    fr = torch.tensor([0.1, 0.3, 0.5, 0.8]).repeat_interleave(M * N // 4)
    W0 = base + torch.sign(base) * fr * ulp
    W = W0.to(dev)
    A = torch.zeros(M * K, dtype=bf, device=dev)
    B = torch.zeros(N * K, dtype=bf, device=dev)
    hi = torch.empty(M * N, dtype=bf, device=dev)
    tla.gemm(A, B, M, N, K, "sgd", W, a_kmajor=False, b_kmajor=False, C2=hi, scale=1e-3, seed=12345)
    assert torch.equal(W.cpu(), W0)
    h = hi.cpu().float()
    up = (h - base).abs() > 0
    assert torch.all((h == base) | ((h - base).abs() - ulp).abs().le(0))
    for q, f in enumerate((0.1, 0.3, 0.5, 0.8)):
        sl = slice(q * M * N // 4, (q + 1) * M * N // 4)
        rate = float(up[sl].float().mean())
        n = M * N // 4
        say(f"  fraction {f}: rounded up {rate:.4f} of {n}")
        assert abs(rate - f) < 6 * (f * (1 - f) / n) ** 0.5
    # the same seed gives the same bits; another seed other bits
    hi2 = torch.empty_like(hi)
    tla.gemm(A, B, M, N, K, "sgd", W, a_kmajor=False, b_kmajor=False, C2=hi2, scale=1e-3, seed=12345)
    assert torch.equal(hi, hi2)
    tla.gemm(A, B, M, N, K, "sgd", W, a_kmajor=False, b_kmajor=False, C2=hi2, scale=1e-3, seed=777)
    assert not torch.equal(hi, hi2)


# The inner loop's products at the 3B shape (d 3072, F 8192, V 128256,
# mini-batch 1024), in the launch configuration the engine picks (tile 0),
# checked on sampled output entries.
BIG = [
    ("lm_head fwd", 1024, 128256, 3072, "nt", 0),
    ("lm_head bwd dX", 1024, 3072, 128256, "nn", 16064),
    ("dyn up bwd dX", 1024, 3072, 16384, "nn", 4096),
    ("dW3", 3072, 8192, 1024, "tn", 0),
    ("dW12", 16384, 3072, 1024, "tn", 0),
]


@pytest.mark.parametrize("name,M,N,K,lay,split", BIG)
def test_gemm_3b_shapes_sampled(name, M, N, K, lay, split):
    ak, bk = LAYOUTS[lay]
    say(f"gemm 3b {name} {M}x{N}x{K} {lay}")
    g = torch.Generator(device=dev).manual_seed(14)
    A = (torch.randn(M * K, generator=g, device=dev) * 0.5).to(bf)
    B = (torch.randn(N * K, generator=g, device=dev) * 0.5).to(bf)
    nsp = (K + split - 1) // split if split else 1
    C = torch.empty(nsp * M * N, device=dev)
    if split:
        tla.gemm(A, B, M, N, K, "partial", C, a_kmajor=ak, b_kmajor=bk, kchunk=split)
        Cm = C.view(nsp, M, N).sum(0)
    else:
        tla.gemm(A, B, M, N, K, "store_f32", C, a_kmajor=ak, b_kmajor=bk)
        Cm = C.view(M, N)
    rs = np.random.default_rng(15)
    rows = torch.as_tensor(rs.integers(0, M, 64))
    cols = torch.as_tensor(rs.integers(0, N, 64))
    rows = torch.cat([rows, torch.tensor([0, M - 1])])
    cols = torch.cat([cols, torch.tensor([N - 1, 0])])
    Ac = A.cpu().double()
    Bc = B.cpu().double()
    Am = Ac.view(M, K) if ak else Ac.view(K, M).T
    Bm = Bc.view(N, K) if bk else Bc.view(K, N).T
    want = (Am[rows] * Bm[cols]).sum(1)
    got = Cm[rows.to(dev), cols.to(dev)].cpu().double()
    # fp32 accumulation over K terms of size ~0.25: error ~ sqrt(K) * 2^-24 * |terms|
    tol = 1e-5 * max(1.0, float(want.abs().max()))
    assert float((got - want).abs().max()) < tol, (name, float((got - want).abs().max()))


@pytest.mark.parametrize("epi", ["add_f32", "partial", "swiglu"])
def test_gemm_two_term_b(epi):
    """B2 adds a second bf16 term to B (the fast weights' low part):
    C = A (B + B2)^T, for the epilogues that take it."""
    g = torch.Generator().manual_seed(16)
    M, N, K = 392, 320, 456
    A = rnd(g, M * K)
    B = rnd(g, N * K)
    B2 = rnd(g, N * K, scale=0.004)
    acc = logical(A, M, K, True) @ (logical(B, N, K, True) + logical(B2, N, K, True)).T
    Ad, Bd, B2d = A.to(dev), B.to(dev), B2.to(dev)
    for t in (0, 1, 3, 5):
        say(f"gemm two-term {epi} tile {t}")
        if epi == "add_f32":
            C = torch.zeros(M * N, device=dev)
            tla.gemm(Ad, Bd, M, N, K, epi, C, B2=B2d, tile=t)
            got = C.cpu().double().view(M, N)
        elif epi == "partial":
            nsp = (K + 127) // 128
            C = torch.empty(nsp * M * N, device=dev)
            tla.gemm(Ad, Bd, M, N, K, epi, C, B2=B2d, tile=t, kchunk=128)
            got = C.cpu().double().view(nsp, M, N).sum(0)
        else:
            C = torch.empty(M * N, dtype=bf, device=dev)
            C2 = torch.empty(M * N // 2, dtype=bf, device=dev)
            tla.gemm(Ad, Bd, M, N, K, epi, C, C2=C2, B2=B2d, tile=t)
            got = C.cpu().double().view(M, N)
            assert float((got - acc).abs().max()) <= float(acc.abs().max()) * 2 ** -8
            continue
        assert float((got - acc).abs().max() / acc.abs().max()) < 1e-5, (epi, t)


def _dw_case(g, M, N, K, lo=True, lda=None, ldb=None):
    lda, ldb = lda or M, ldb or N
    A = rnd(g, K * lda).view(K, lda)
    B = rnd(g, K * ldb).view(K, ldb)
    W0 = rnd(g, M * N, scale=0.02, dtype=torch.float32).view(M, N)
    p = dict(A=A.to(dev), lda=lda, B=B.to(dev), ldb=ldb, W=W0.to(dev), Hi=torch.empty(M, N, dtype=bf, device=dev),
             Lo=torch.empty(M, N, dtype=bf, device=dev) if lo else None, ldw=N, M=M, N=N)
    return p, A, B, W0


def _dw_check(p, A, B, W0, lr, M, N):
    acc = A[:, :M].double().T @ B[:, :N].double()
    want = W0.double() - lr * acc
    Wg = p["W"].cpu()
    err = float((Wg.double() - want).abs().max())
    assert err < 1e-6, err
    # the working copy is the RNE of the stored master, the low term the RNE of the remainder
    assert torch.equal(p["Hi"].cpu(), Wg.to(bf))
    if p["Lo"] is not None:
        assert torch.equal(p["Lo"].cpu(), (Wg - Wg.to(bf).float()).to(bf))


@pytest.mark.parametrize("K,grid", [(1024, 0), (1024, 8), (1000, 16), (328, 0), (64, 8)])
def test_dw_sgd_two_problems(K, grid):
    """tttk_dw_sgd: W -= lr A^T B for two problems in one persistent launch
    (K = 1024 and 1000: each tile's update overlapped with the next tile's
    products; other K: updated after each tile), ragged tiles in M and N,
    padded leading dimensions, one problem without the low term; grid 8 and
    16 make every workgroup visit many tiles of both problems."""
    g = torch.Generator().manual_seed(21)
    lr = 1e-3
    say(f"dw_sgd K={K} grid={grid}")
    p0, A0, B0, W00 = _dw_case(g, 400, 272, K, lda=408)
    p1, A1, B1, W01 = _dw_case(g, 272, 528, K, lo=False, ldb=536)
    tla.dw_sgd([p0, p1], K, lr, grid=grid)
    torch.cuda.synchronize()
    _dw_check(p0, A0, B0, W00, lr, 400, 272)
    _dw_check(p1, A1, B1, W01, lr, 272, 528)


def test_dw_sgd_3b_block_shapes_sampled():
    """Both products of a 3B dynamic block (dW12 [16384 x 3072] and dW3
    [3072 x 8192], K = 1024) in the engine's launch configuration, checked on
    4096 sampled entries each, plus the rounding of the working copy."""
    g = torch.Generator().manual_seed(22)
    lr = 5e-3
    K = 1024
    shapes = [(16384, 3072), (3072, 8192)]
    ps = []
    for M, N in shapes:
        A = rnd(g, K * M).view(K, M).to(dev)
        B = rnd(g, K * N).view(K, N).to(dev)
        W0 = (torch.randn(M, N, generator=g) * 0.02).to(dev)
        ps.append(dict(A=A, lda=M, B=B, ldb=N, W=W0.clone(), Hi=torch.empty(M, N, dtype=bf, device=dev),
                       Lo=torch.empty(M, N, dtype=bf, device=dev), ldw=N, M=M, N=N, W0=W0))
    tla.dw_sgd([{k: v for k, v in p.items() if k != "W0"} for p in ps], K, lr)
    torch.cuda.synchronize()
    for (M, N), p in zip(shapes, ps):
        ms = torch.randint(0, M, (4096,), generator=g)
        ns = torch.randint(0, N, (4096,), generator=g)
        a = p["A"].cpu().double()[:, ms]
        b = p["B"].cpu().double()[:, ns]
        want = p["W0"].cpu().double()[ms, ns] - lr * (a * b).sum(0)
        got = p["W"].cpu()[ms, ns]
        err = float((got.double() - want).abs().max())
        say(f"  dW+SGD {M}x{N}: max err {err:.2e}")
        assert err < 2e-6
        Wg = p["W"]
        assert torch.equal(p["Hi"], Wg.to(bf))
        assert torch.equal(p["Lo"], (Wg - Wg.to(bf).float()).to(bf))


@pytest.mark.parametrize("tile", [0, 1, 2, 3, 4, 5, 6])
def test_gemm_store_f32_lse_epilogue(tile):
    """STORE_F32_LSE: C = A B^T in fp32 and, per row and 64-column group, the
    group's (max, sum exp(x - max)) -- ragged last group and ragged rows."""
    g = torch.Generator().manual_seed(31)
    M, N, K = 264, 520, 200
    A = rnd(g, M * K)
    B = rnd(g, N * K)
    acc = logical(A, M, K, True) @ logical(B, N, K, True).T
    np_ = (N + 63) // 64
    C = torch.full((M * N,), float("nan"), device=dev)
    P = torch.full((M * np_ * 2,), float("nan"), device=dev)
    tla.gemm(A.to(dev), B.to(dev), M, N, K, "store_f32_lse", C, C2=P, tile=tile)
    assert float((C.cpu().double().view(M, N) - acc).abs().max() / acc.abs().max()) < 1e-5
    Pg = P.cpu().double().view(M, np_, 2)
    for gi in range(np_):
        blk = acc[:, 64 * gi:min(N, 64 * gi + 64)]
        mx = blk.max(dim=1).values
        sm = torch.exp(blk - mx[:, None]).sum(dim=1)
        assert float((Pg[:, gi, 0] - mx).abs().max()) < 1e-5 * float(acc.abs().max())
        assert float(((Pg[:, gi, 1] - sm) / sm).abs().max()) < 1e-5


def test_ce_from_lse_partials():
    """Single-pass CE: loss and dz from the logits and their per-64-column
    partials, against float64 (rows past nt get dz = 0)."""
    g = torch.Generator().manual_seed(32)
    n, nt, V = 37, 30, 1000
    z = torch.randn(n, V, generator=g, dtype=torch.float64) * 3
    lab = torch.randint(0, V, (nt,), generator=g, dtype=torch.int32)
    np_ = (V + 63) // 64
    parts = torch.zeros(n, np_, 2, dtype=torch.float32)
    for gi in range(np_):
        blk = z[:, 64 * gi:min(V, 64 * gi + 64)]
        mx = blk.max(dim=1).values
        parts[:, gi, 0] = mx.float()
        parts[:, gi, 1] = torch.exp(blk - mx[:, None]).sum(dim=1).float()
    loss = torch.empty(nt, device=dev)
    dz = torch.empty(n, V, dtype=bf, device=dev)
    err = torch.zeros(4, dtype=torch.int32, device=dev)
    scale = 1.0 / nt
    tla.ce_lse(z.float().to(dev), parts.to(dev), n, nt, V, lab.to(dev), scale, loss, dz, err)
    torch.cuda.synchronize()
    lse = torch.logsumexp(z[:nt], dim=1)
    want_loss = lse - z[torch.arange(nt), lab.long()]
    assert float(((loss.cpu().double() - want_loss) / want_loss).abs().max()) < 1e-5
    p = torch.softmax(z[:nt], dim=1)
    p[torch.arange(nt), lab.long()] -= 1.0
    want_dz = p * scale
    got = dz.cpu().double()
    assert float((got[:nt] - want_dz).abs().max()) <= 2 ** -8 * float(want_dz.abs().max())
    assert float(got[nt:].abs().max()) == 0.0
    assert int(err.cpu()[0]) == 0
