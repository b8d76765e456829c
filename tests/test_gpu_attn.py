"""Kernel-level parity of the sliding-window attention kernels
(include/ttt_kernels.h: tttk_attn_fwd, tttk_attn_bwd) against float64 CPU
attention written out from its definition: key t is visible to query i iff
i - window < t <= i (positions), GQA by contiguous head groups, scale
1/sqrt(dh); the backward differentiates the call's own queries and keys
(positions pos0 .. pos0 + n - 1); keys stored before pos0 are constants.

The key/value store is a ring [Hk][cap][dh] indexed by position % cap; the
cases below wrap around it, cut windows inside the call, and leave ragged
tiles.
"""
import math

import pytest
import torch

from tests.util import say

pytestmark = pytest.mark.gpu

tla = pytest.importorskip("test_long_context_amd")
dev = "cuda"
bf = torch.bfloat16

# (n, H, Hk, dh, cap, window, pos0)
CASES = [
    (150, 6, 2, 128, 512, 200, 450),   # wraps the ring, ragged n
    (150, 6, 2, 64, 512, 64, 300),     # window shorter than the call
    (130, 4, 4, 128, 512, 128, 0),     # first call: only its own keys
    (64, 3, 1, 64, 128, 40, 1000),     # window ends inside one key tile
    (256, 24, 8, 128, 8192, 4096, 5000),  # many heads, long window: the dq key range
                                          # splits into more than four parts
]


def reference(q, Kr, Vr, dO, n, H, Hk, dh, cap, window, pos0):
    """float64 forward (O, lse) and backward (dq, dk, dv) by autograd."""
    grp = H // Hk
    lo = max(0, pos0 - window + 1)
    pos = torch.arange(lo, pos0 + n)
    own = pos >= pos0
    Kall = Kr[:, pos % cap].double()          # [Hk, P, dh]
    Vall = Vr[:, pos % cap].double()
    Kown = Kall[:, own].clone().requires_grad_(True)
    Vown = Vall[:, own].clone().requires_grad_(True)
    Kc = torch.cat([Kall[:, ~own], Kown], 1)
    Vc = torch.cat([Vall[:, ~own], Vown], 1)
    qd = q.double().clone().requires_grad_(True)          # [n, H, dh]
    qp = pos0 + torch.arange(n)
    vis = (pos[None, :] <= qp[:, None]) & (pos[None, :] > qp[:, None] - window)   # [n, P]
    kk = Kc.repeat_interleave(grp, 0)                     # [H, P, dh]
    vv = Vc.repeat_interleave(grp, 0)
    s = torch.einsum("nhd,hpd->hnp", qd, kk) / math.sqrt(dh)
    s = s.masked_fill(~vis[None], float("-inf"))
    lse = torch.logsumexp(s, -1)                          # [H, n]
    p = torch.exp(s - lse[..., None])
    o = torch.einsum("hnp,hpd->nhd", p, vv)
    (o * dO.double()).sum().backward()
    D = (dO.double() * o.detach()).sum(-1).T.contiguous()  # [H, n]
    return o.detach(), lse.detach(), D, qd.grad, Kown.grad.permute(1, 0, 2), Vown.grad.permute(1, 0, 2)


def rel(a, b):
    return float((a.double() - b).abs().max() / b.abs().max())


@pytest.mark.parametrize("case", CASES)
def test_attention_fwd_bwd(case):
    n, H, Hk, dh, cap, window, pos0 = case
    g = torch.Generator().manual_seed(21)
    q = torch.randn(n, H, dh, generator=g).to(bf)
    Kr = torch.randn(Hk, cap, dh, generator=g).to(bf)
    Vr = torch.randn(Hk, cap, dh, generator=g).to(bf)
    dO = torch.randn(n, H, dh, generator=g).to(bf)
    o_ref, lse_ref, D_ref, dq_ref, dk_ref, dv_ref = reference(q, Kr, Vr, dO, n, H, Hk, dh, cap, window, pos0)

    qd, Kd, Vd, dOd = q.to(dev), Kr.to(dev), Vr.to(dev), dO.to(dev)
    # transposed values with the store's slot order inside blocks of 16
    # (bits 2 and 3 of the slot swapped; include/ttt_kernels.h)
    sl = torch.arange(cap)
    perm = (sl & ~15) | (sl & 3) | ((sl & 4) << 1) | ((sl & 8) >> 1)
    VT = torch.empty(Hk, dh, cap, dtype=bf)
    VT[:, :, perm] = Vr.transpose(1, 2)
    VTd = VT.contiguous().to(dev)
    for variant, ksplit in ((1, 1), (2, 1), (3, 1), (4, 1), (2, 2), (2, 3), (3, 4), (4, 2)):
        say(f"attn fwd variant {variant} ksplit {ksplit} case {case}")
        o = torch.full((n, H, dh), float("nan"), dtype=bf, device=dev)
        lse = torch.full((H, n), float("nan"), device=dev)
        ws = tla.attn_fwd_workspace(n, H, dh, window, ksplit)
        work = torch.empty(max(ws // 4, 1), device=dev)
        tla.attn_fwd(qd, Kd, Vd, o, lse, n, H, Hk, dh, cap, window, pos0, vt=VTd, variant=variant, ksplit=ksplit,
                     work=work)
        assert rel(o.cpu(), o_ref) < 1e-2, (variant, ksplit, rel(o.cpu(), o_ref))
        assert float((lse.cpu().double() - lse_ref).abs().max()) < 1e-2

    lse_in = lse_ref.float().to(dev)
    D_in = D_ref.float().to(dev)
    for variant in (1, 2):
        say(f"attn bwd variant {variant} case {case}")
        dq = torch.full((n, H, dh), float("nan"), device=dev)
        dk = torch.full((n, Hk, dh), float("nan"), device=dev)
        dv = torch.full((n, Hk, dh), float("nan"), device=dev)
        ws = tla.attn_bwd_workspace(bf, n, H, Hk, dh, window, variant)
        work = torch.empty(max(ws // 4, 1), device=dev)
        tla.attn_bwd(qd, Kd, Vd, lse_in, dOd, D_in, dq, dk, dv, n, H, Hk, dh, cap, window, pos0,
                     variant=variant, work=work)
        for name, got, want in (("dq", dq, dq_ref), ("dk", dk, dk_ref), ("dv", dv, dv_ref)):
            e = rel(got.cpu(), want)
            assert e < 2e-2, (variant, name, e)


@pytest.mark.parametrize("pos0", [0, 16384])
def test_attention_fwd_long_stream_sampled_rows(pos0):
    """16384 queries of 24 heads (8 key heads, dh 128) over a window of 8192
    in a 32768-slot store, the prefill's slab shape, from position 0 (the
    window ramps up) and from 16384 (full windows): sampled query rows of
    every forward variant against float64 attention over each row's own
    visible keys."""
    n, H, Hk, dh, cap, window = 16384, 24, 8, 128, 32768, 8192
    g = torch.Generator().manual_seed(23)
    q = torch.randn(n, H, dh, generator=g).to(bf)
    Kr = (torch.randn(Hk, cap, dh, generator=g) * 0.5).to(bf)
    Vr = torch.randn(Hk, cap, dh, generator=g).to(bf)
    sl = torch.arange(cap)
    perm = (sl & ~15) | (sl & 3) | ((sl & 4) << 1) | ((sl & 8) >> 1)
    VT = torch.empty(Hk, dh, cap, dtype=bf)
    VT[:, :, perm] = Vr.transpose(1, 2)
    rows = torch.tensor([0, 1, 31, 32, 63, 64, 127, 255, 256, 1000, 4095, 8190, 8191, 8192, 8200, 12345, 16320,
                         16383])
    grp = H // Hk
    ref = torch.empty(len(rows), H, dh, dtype=torch.float64)
    for r_i, r in enumerate(rows.tolist()):
        p = pos0 + r
        kp = torch.arange(max(0, p - window + 1), p + 1)
        kk = Kr[:, kp % cap].double().repeat_interleave(grp, 0)     # [H, P, dh]
        vv = Vr[:, kp % cap].double().repeat_interleave(grp, 0)
        s = torch.einsum("hd,hpd->hp", q[r].double(), kk) / math.sqrt(dh)
        ref[r_i] = torch.einsum("hp,hpd->hd", torch.softmax(s, -1), vv)
    qd, Kd, Vd, VTd = q.to(dev), Kr.to(dev), Vr.to(dev), VT.contiguous().to(dev)
    for variant, ksplit in ((1, 1), (2, 1), (3, 1), (4, 1), (2, 4)):
        o = torch.full((n, H, dh), float("nan"), dtype=bf, device=dev)
        lse = torch.empty(H, n, device=dev)
        ws = tla.attn_fwd_workspace(n, H, dh, window, ksplit)
        work = torch.empty(max(ws // 4, 1), device=dev)
        tla.attn_fwd(qd, Kd, Vd, o, lse, n, H, Hk, dh, cap, window, pos0, vt=VTd, variant=variant, ksplit=ksplit,
                     work=work)
        got = o[rows.to(dev)].cpu()
        e = rel(got, ref)
        say(f"  long stream pos0={pos0} variant {variant} ksplit {ksplit}: sampled rows rel err {e:.3e}")
        assert torch.isfinite(o).all()
        assert e < 1e-2, (variant, ksplit, e)
