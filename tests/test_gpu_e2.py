"""GPU parity of the E2-TTT chunk-end scan against the float64 oracle
(Proposition 3.1 evaluated chunk by chunk; the oracle's closed form is
itself pinned to the per-token recursion). Tolerance 1e-5 relative per
tensor (max |x - ref| / max |ref|)."""
import numpy as np
import pytest
import torch

import synth
from oracle import e2ttt as E
from tests.util import say

pytestmark = pytest.mark.gpu


def run(H, T, D, C, seed, M0=False):
    import test_long_context_amd as tla
    say(f"case: e2 H={H} T={T} D={D} C={C} M0={M0}")
    g = synth.gen_e2(H, T, D, seed)
    if M0:
        g["M"] = (synth.normal(seed, 9, H * D * D) * 0.01).to(torch.float32).view(H, D, D)
    d = {k: v.cuda() for k, v in g.items()}
    W, M = d["W"].clone(), d["M"].clone()
    tla.e2ttt_chunk_scan(d["k"], d["v"], d["eta"], d["beta"], d["gamma"], W, M, C)
    torch.cuda.synchronize()
    Wr, Mr = E.e2_closed_form(g["k"].float().numpy(), g["v"].float().numpy(), g["eta"].numpy(),
                              g["beta"].numpy(), g["gamma"].numpy(), g["W"].numpy(), g["M"].numpy(), C)
    ew = np.max(np.abs(W.cpu().numpy() - Wr)) / np.max(np.abs(Wr))
    em = np.max(np.abs(M.cpu().numpy() - Mr)) / np.max(np.abs(Mr))
    say(f"  W rel err {ew:.3e}  M rel err {em:.3e}")
    return ew, em


def test_e2_calls_on_two_streams_overlap():
    """Calls enqueued on two streams at once (each takes its own work buffer
    on its own stream, in stream order): every result is bit-identical to
    the same call made alone, over three rounds that reuse the pool."""
    import test_long_context_amd as tla
    cases = [(16, 8192, 128, 2048, 31), (8, 6000, 64, 512, 32)]
    ins, refs = [], []
    for H, T, D, C, seed in cases:
        say(f"case: e2 two streams H={H} T={T} D={D} C={C}")
        d = {k: v.cuda() for k, v in synth.gen_e2(H, T, D, seed).items()}
        W, M = d["W"].clone(), d["M"].clone()
        tla.e2ttt_chunk_scan(d["k"], d["v"], d["eta"], d["beta"], d["gamma"], W, M, C)
        torch.cuda.synchronize()
        ins.append((d, C))
        refs.append((W, M))
    streams = [torch.cuda.Stream(), torch.cuda.Stream()]
    for rnd in range(3):
        outs = []
        for (d, C), s in zip(ins, streams):
            W, M = d["W"].clone(), d["M"].clone()
            s.wait_stream(torch.cuda.current_stream())
            outs.append((W, M, s))
        for (d, C), (W, M, s) in zip(ins, outs):
            tla.e2ttt_chunk_scan(d["k"], d["v"], d["eta"], d["beta"], d["gamma"], W, M, C, stream=s.cuda_stream)
        torch.cuda.synchronize()
        for (W, M, _), (Wr, Mr) in zip(outs, refs):
            assert torch.equal(W, Wr) and torch.equal(M, Mr), rnd


def test_e2_full_workload():
    c = synth.E2_CONFIG
    ew, em = run(c["heads"], c["seq"], c["dim"], c["chunk"], c["seed"])
    assert ew < 1e-5 and em < 1e-5


@pytest.mark.parametrize("H,T,D,C,M0", [(3, 1000, 128, 256, True), (2, 200, 64, 64, True),
                                        (1, 2048 + 77, 128, 2048, False)])
def test_e2_ragged_and_small(H, T, D, C, M0):
    ew, em = run(H, T, D, C, 7, M0)
    assert ew < 1e-5 and em < 1e-5


def run_lact(H, T, D, C, seed, M0=False):
    import test_long_context_amd as tla
    say(f"case: lact H={H} T={T} D={D} C={C} M0={M0}")
    g = synth.gen_e2(H, T, D, seed)
    if M0:
        g["M"] = (synth.normal(seed, 9, H * D * D) * 0.01).to(torch.float32).view(H, D, D)
    d = {k: v.cuda() for k, v in g.items()}
    W, M = d["W"].clone(), d["M"].clone()
    tla.lact_chunk_scan(d["k"], d["v"], d["eta"], d["beta"], W, M, C)
    torch.cuda.synchronize()
    Wr, Mr = E.lact_chunked(g["k"].float().numpy(), g["v"].float().numpy(), g["eta"].numpy(),
                            g["beta"].numpy(), g["W"].numpy(), g["M"].numpy(), C)
    ew = np.max(np.abs(W.cpu().numpy() - Wr)) / np.max(np.abs(Wr))
    em = np.max(np.abs(M.cpu().numpy() - Mr)) / np.max(np.abs(Mr))
    say(f"  W rel err {ew:.3e}  M rel err {em:.3e}")
    return ew, em


def test_lact_full_workload():
    """The chunk-wise baseline (one eta-weighted update direction per chunk,
    chunk-mean momentum, no decay) on the E2 workload."""
    c = synth.E2_CONFIG
    ew, em = run_lact(c["heads"], c["seq"], c["dim"], c["chunk"], c["seed"])
    assert ew < 1e-5 and em < 1e-5


@pytest.mark.parametrize("H,T,D,C,M0", [(3, 1000, 128, 256, True), (2, 200, 64, 64, True),
                                        (1, 2048 + 77, 128, 2048, False)])
def test_lact_ragged_and_small(H, T, D, C, M0):
    ew, em = run_lact(H, T, D, C, 7, M0)
    assert ew < 1e-5 and em < 1e-5


def run_mixer(H, T, D, dm, C, seed, eta_base=1e-4, alpha_base=0.5, tau=4.0):
    """The E2-TTT token mixer's TTT path (e2ttt_mixer_forward) against the
    float64 oracle on the same bf16-valued inputs. Between the steps the
    oracle keeps q, k, v in bf16 and the scalars in float32, as the kernels
    do; the two sides differ by their arithmetic before those roundings.
    Errors: max |x - ref| / max |ref| for the outputs, W and M."""
    import test_long_context_amd as tla
    say(f"case: e2 mixer H={H} T={T} D={D} dm={dm} C={C}")
    g = synth.gen_e2_mixer(H, T, D, dm, seed)
    d = {k: v.cuda() for k, v in g.items()}
    W, M = d["W"].clone(), d["M"].clone()
    out = tla.e2ttt_mixer_forward(d["x"], d["wqkv"], d["bias"], eta_base, alpha_base, tau, W, M, H, C)
    torch.cuda.synchronize()
    Or, Wr, Mr = E.e2_mixer(g["x"].double().numpy(), g["wqkv"].double().numpy(), g["bias"].numpy(), eta_base,
                            alpha_base, tau, g["W"].numpy(), g["M"].numpy(), H, D, C)
    eo = np.max(np.abs(out.cpu().numpy().reshape(T, H, D) - Or)) / np.max(np.abs(Or))
    ew = np.max(np.abs(W.cpu().numpy() - Wr)) / np.max(np.abs(Wr))
    em = np.max(np.abs(M.cpu().numpy() - Mr)) / np.max(np.abs(Mr))
    say(f"  outputs rel err {eo:.3e}  W rel err {ew:.3e}  M rel err {em:.3e}")
    return eo, ew, em


# bf16 activations between the steps: the bf16 tolerances (2e-2 on outputs,
# 5e-2 on the state)
@pytest.mark.parametrize("H,T,D,dm,C", [(3, 1000, 128, 256, 256), (2, 200, 64, 128, 64),
                                        (1, 2048 + 77, 128, 128, 2048)])
def test_e2_mixer_small_and_ragged(H, T, D, dm, C):
    eo, ew, em = run_mixer(H, T, D, dm, C, 8)
    assert eo < 2e-2 and ew < 5e-2 and em < 5e-2


def test_e2_mixer_full_workload():
    c = synth.E2_MIXER_CONFIG
    eo, ew, em = run_mixer(c["heads"], c["seq"], c["dim"], c["d_model"], c["chunk"], c["seed"], c["eta_base"],
                           c["alpha_base"], c["tau"])
    assert eo < 2e-2 and ew < 5e-2 and em < 5e-2


# ------------------------------------------- SwiGLU fast-weight token mixer
def run_mlp_mixer(H, T, D, Dh, dm, C, seed, eta_base=3e-4, alpha_base=0.5, tau=4.0):
    """The token mixer with the SwiGLU fast-weight net
    (e2ttt_mixer_swiglu_forward) against the float64 oracle on the same
    bf16-valued inputs. The kernels round each chunk's weights and
    activations to bf16 for the products; the oracle does not. Errors: max
    |x - ref| / max |ref| for the outputs and the momenta; for the weights,
    max |W - W_ref| / max |W_ref - W0| (the change, since decay and updates
    move W far from W0)."""
    import test_long_context_amd as tla
    from oracle import e2ttt_mlp as X
    say(f"case: e2 swiglu mixer H={H} T={T} D={D} Dh={Dh} dm={dm} C={C}")
    g = synth.gen_e2_mixer(H, T, D, dm, seed)
    s0 = synth.gen_e2_mlp_state(H, D, Dh, seed)
    d = {k: v.cuda() for k, v in g.items()}
    st = {k: v.cuda().clone() for k, v in s0.items()}
    out = tla.e2ttt_mixer_swiglu_forward(d["x"], d["wqkv"], d["bias"], eta_base, alpha_base, tau, st, H, C)
    torch.cuda.synchronize()
    W = [{m: s0[w][h].double().numpy() for m, w in zip(X.MATS, ("w1", "w2", "w3"))} for h in range(H)]
    M = [{m: s0[w][h].double().numpy() for m, w in zip(X.MATS, ("m1", "m2", "m3"))} for h in range(H)]
    Or, Wr, Mr = X.e2_mlp_mixer(g["x"].double().numpy(), g["wqkv"].double().numpy(), g["bias"].numpy(),
                                eta_base, alpha_base, tau, W, M, H, D, C)
    eo = np.max(np.abs(out.cpu().numpy().reshape(T, H, D) - Or)) / np.max(np.abs(Or))
    ew, em = 0.0, 0.0
    for m, wn, mn in zip(X.MATS, ("w1", "w2", "w3"), ("m1", "m2", "m3")):
        wg, mg = st[wn].cpu().double().numpy(), st[mn].cpu().double().numpy()
        wr = np.stack([Wr[h][m] for h in range(H)])
        mr = np.stack([Mr[h][m] for h in range(H)])
        w0 = s0[wn].double().numpy()
        ew = max(ew, np.max(np.abs(wg - wr)) / np.max(np.abs(wr - w0)))
        em = max(em, np.max(np.abs(mg - mr)) / np.max(np.abs(mr)))
    say(f"  outputs rel err {eo:.3e}  W err (of the change) {ew:.3e}  M rel err {em:.3e}")
    return eo, ew, em


@pytest.mark.parametrize("H,T,D,Dh,dm,C", [(3, 1000, 128, 256, 256, 256), (2, 200, 64, 64, 128, 64),
                                           (1, 2048 + 77, 128, 128, 128, 2048)])
def test_e2_swiglu_mixer_small_and_ragged(H, T, D, Dh, dm, C):
    eo, ew, em = run_mlp_mixer(H, T, D, Dh, dm, C, 9)
    assert eo < 2e-2 and ew < 5e-2 and em < 5e-2


def test_e2_swiglu_mixer_full_workload():
    c = synth.E2_MLP_CONFIG
    eo, ew, em = run_mlp_mixer(c["heads"], c["seq"], c["dim"], c["hidden"], c["d_model"], c["chunk"], c["seed"],
                               c["eta_base"], c["alpha_base"], c["tau"])
    assert eo < 2e-2 and ew < 5e-2 and em < 5e-2


# --------------------------------------------- GELU fast-weight token mixer
def run_gelu_mixer(H, T, D, Dh, dm, C, seed, eta_base=3e-4, alpha_base=0.5, tau=4.0):
    """The token mixer with the GELU fast-weight net
    (e2ttt_mixer_gelu_forward) against the float64 oracle on the same
    bf16-valued inputs; errors as for the SwiGLU net (run_mlp_mixer)."""
    import test_long_context_amd as tla
    from oracle import e2ttt_gelu as G
    say(f"case: e2 gelu mixer H={H} T={T} D={D} Dh={Dh} dm={dm} C={C}")
    g = synth.gen_e2_mixer(H, T, D, dm, seed)
    s0 = synth.gen_e2_gelu_state(H, D, Dh, seed)
    d = {k: v.cuda() for k, v in g.items()}
    st = {k: v.cuda().clone() for k, v in s0.items()}
    out = tla.e2ttt_mixer_gelu_forward(d["x"], d["wqkv"], d["bias"], eta_base, alpha_base, tau, st, H, C)
    torch.cuda.synchronize()
    W = [{m: s0[m][h].double().numpy() for m in G.MATS} for h in range(H)]
    M = [{m: s0["m" + m[1]][h].double().numpy() for m in G.MATS} for h in range(H)]
    Or, Wr, Mr = G.e2_gelu_mixer(g["x"].double().numpy(), g["wqkv"].double().numpy(), g["bias"].numpy(),
                                 eta_base, alpha_base, tau, W, M, H, D, C)
    eo = np.max(np.abs(out.cpu().numpy().reshape(T, H, D) - Or)) / np.max(np.abs(Or))
    ew, em = 0.0, 0.0
    for m in G.MATS:
        mn = "m" + m[1]
        wg, mg = st[m].cpu().double().numpy(), st[mn].cpu().double().numpy()
        wr = np.stack([Wr[h][m] for h in range(H)])
        mr = np.stack([Mr[h][m] for h in range(H)])
        w0 = s0[m].double().numpy()
        ew = max(ew, np.max(np.abs(wg - wr)) / np.max(np.abs(wr - w0)))
        em = max(em, np.max(np.abs(mg - mr)) / np.max(np.abs(mr)))
    say(f"  outputs rel err {eo:.3e}  W err (of the change) {ew:.3e}  M rel err {em:.3e}")
    return eo, ew, em


@pytest.mark.parametrize("H,T,D,Dh,dm,C", [(3, 1000, 128, 256, 256, 256), (2, 200, 64, 64, 128, 64),
                                           (1, 2048 + 77, 128, 128, 128, 2048)])
def test_e2_gelu_mixer_small_and_ragged(H, T, D, Dh, dm, C):
    eo, ew, em = run_gelu_mixer(H, T, D, Dh, dm, C, 11)
    assert eo < 2e-2 and ew < 5e-2 and em < 5e-2


def test_e2_gelu_mixer_full_workload():
    c = synth.E2_GELU_CONFIG
    eo, ew, em = run_gelu_mixer(c["heads"], c["seq"], c["dim"], c["hidden"], c["d_model"], c["chunk"], c["seed"],
                                c["eta_base"], c["alpha_base"], c["tau"])
    assert eo < 2e-2 and ew < 5e-2 and em < 5e-2


# ------------------------------------------------- hybrid token-mixer block
def run_hybrid(H, T, D, Dh, dm, C, window, seed, eta_base, alpha_base=0.5, tau=4.0, theta=10000.0, net="swiglu"):
    """The hybrid block (e2ttt_hybrid_forward: SWA beside the TTT path, gated)
    against the float64 oracle. Errors as for the mixers: outputs and momenta
    max |x - ref| / max |ref|; weights relative to their change (SwiGLU,
    GELU nets) or to max |W| (linear). net: the fast-weight net for Dh > 0."""
    import test_long_context_amd as tla
    from oracle import e2ttt_hybrid as Y
    from oracle import e2ttt_mlp as X
    say(f"case: e2 hybrid H={H} T={T} D={D} Dh={Dh} dm={dm} C={C} window={window}")
    g = synth.gen_e2_mixer(H, T, D, dm, seed)
    gt = synth.gen_gate(H, D, dm, seed)
    d = {k: v.cuda() for k, v in g.items()}
    mats = ("w1", "w2") if net == "gelu" else X.MATS
    if Dh:
        s0 = (synth.gen_e2_gelu_state if net == "gelu" else synth.gen_e2_mlp_state)(H, D, Dh, seed)
        W = [{m: s0[m][h].double().numpy() for m in mats} for h in range(H)]
        M = [{m: s0["m" + m[1]][h].double().numpy() for m in mats} for h in range(H)]
    else:
        s0 = dict(W=g["W"], M=g["M"])
        W, M = g["W"].double().numpy(), g["M"].double().numpy()
    st = {k: v.cuda().clone() for k, v in s0.items()}
    out = tla.e2ttt_hybrid_forward(d["x"], d["wqkv"], d["bias"], gt["wgate"].cuda(), gt["bgate"].cuda(), eta_base,
                                   alpha_base, tau, theta, window, st, H, C)
    torch.cuda.synchronize()
    Or, Wr, Mr = Y.hybrid_mixer(g["x"].double().numpy(), g["wqkv"].double().numpy(), g["bias"].numpy(),
                                gt["wgate"].double().numpy(), gt["bgate"].double().numpy(), eta_base, alpha_base,
                                tau, theta, window, (W, M), H, D, C)
    eo = np.max(np.abs(out.cpu().numpy().reshape(T, H, D) - Or)) / np.max(np.abs(Or))
    if Dh:
        ew = em = 0.0
        for m in mats:
            wn, mn = m, "m" + m[1]
            wr = np.stack([Wr[h][m] for h in range(H)])
            mr = np.stack([Mr[h][m] for h in range(H)])
            ew = max(ew, np.max(np.abs(st[wn].cpu().double().numpy() - wr)) /
                     np.max(np.abs(wr - s0[wn].double().numpy())))
            em = max(em, np.max(np.abs(st[mn].cpu().double().numpy() - mr)) / np.max(np.abs(mr)))
    else:
        ew = np.max(np.abs(st["W"].cpu().numpy() - Wr)) / np.max(np.abs(Wr))
        em = np.max(np.abs(st["M"].cpu().numpy() - Mr)) / np.max(np.abs(Mr))
    say(f"  outputs rel err {eo:.3e}  W err {ew:.3e}  M rel err {em:.3e}")
    return eo, ew, em


@pytest.mark.parametrize("H,T,D,Dh,dm,C,window,eta", [(2, 300, 64, 64, 128, 64, 48, 3e-4),
                                                      (3, 1000, 128, 0, 256, 256, 100, 1e-4),
                                                      (1, 2048 + 77, 128, 128, 128, 2048, 1024, 3e-4)])
def test_e2_hybrid_small_and_ragged(H, T, D, Dh, dm, C, window, eta):
    eo, ew, em = run_hybrid(H, T, D, Dh, dm, C, window, 10, eta)
    assert eo < 2e-2 and ew < 5e-2 and em < 5e-2


@pytest.mark.parametrize("H,T,D,Dh,dm,C,window", [(2, 300, 64, 64, 128, 64, 48),
                                                  (1, 2048 + 77, 128, 128, 128, 2048, 1024)])
def test_e2_hybrid_with_gelu_net(H, T, D, Dh, dm, C, window):
    eo, ew, em = run_hybrid(H, T, D, Dh, dm, C, window, 12, 3e-4, net="gelu")
    assert eo < 2e-2 and ew < 5e-2 and em < 5e-2


def test_e2_hybrid_full_workload():
    c = synth.E2_HYBRID_CONFIG
    eo, ew, em = run_hybrid(c["heads"], c["seq"], c["dim"], c["hidden"], c["d_model"], c["chunk"], c["window"],
                            c["seed"], c["eta_base"], c["alpha_base"], c["tau"], c["rope_theta"])
    assert eo < 2e-2 and ew < 5e-2 and em < 5e-2
