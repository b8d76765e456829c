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
