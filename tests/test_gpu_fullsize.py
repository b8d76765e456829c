"""Properties of the full 128K workload (3B shapes, T = 131072, b = 1024,
k = 8192, the bench's launch configuration: 16384-position prefix slabs, a
32768-slot key/value ring reused four times, side-stream updates, split-K and
key-split partial sums, the captured decode graph). The oracle cannot run this
stream; these checks hold at any size.

* Two contexts, one prefilled with T + 1 tokens (128 full mini-batches, then a
  forward-only position), one with T + b tokens. Their first 128 mini-batches
  are the same work, so their per-token losses up to position T - 1 agree bit
  for bit (every sum on the path is taken in a fixed order).
* The first context then decodes the next tokens under the weights of 128
  updates, at positions whose ring slots have been overwritten four times.
  The second context's mini-batch 128 scores the same positions under the
  same weights through the prefill path (GEMMs, window attention over the
  ring). The decode's cross-entropy of each step matches that prequential
  loss within the bf16 loss tolerance of the parity tests.
"""
import numpy as np
import pytest
import torch

import synth
from tests.util import say

pytestmark = pytest.mark.gpu

NDEC = 4
LOSS_TOL = 2e-2


def _ce(z: np.ndarray, target: int) -> float:
    z = z.astype(np.float64)
    m = z.max()
    return float(m + np.log(np.exp(z - m).sum()) - z[target])


def test_bf16_3b_128k_decode_matches_prefill_losses_and_prefix_is_bitwise_stable():
    import test_long_context_amd as tla
    c = synth.config("3b")
    T, b = c["seq"], c["minibatch"]
    assert T == 131072 and b == 1024 and c["window"] == 8192
    say(f"case: 3b shape, T={T}, decode {NDEC} steps after T + 1 tokens; second context T + b tokens")
    w = synth.gen_weights(c, device="cuda")
    tok = synth.gen_tokens(c, n=T + b, device="cuda")

    m = tla.TTT(c, w, max_seq=T + 2 + NDEC)
    loss_a = m.prefill(tok[:T + 1])
    zs = [m.decode_step(tok[T + 1 + j:T + 2 + j]).cpu().numpy() for j in range(NDEC)]
    m.sync()
    loss_a = loss_a.cpu()
    m.close()
    say("  context A done (prefill T + 1, decode)")

    m = tla.TTT(c, w, max_seq=T + b)
    loss_b = m.prefill(tok)
    m.sync()
    loss_b = loss_b.cpu()
    m.close()
    say("  context B done (prefill T + b)")

    assert bool(torch.isfinite(loss_a).all()) and bool(torch.isfinite(loss_b).all())
    # positions 0 .. T - 1 carry a loss in both runs (T - 1 predicts token T)
    assert torch.equal(loss_a[:T], loss_b[:T])
    tk = tok.cpu().numpy()
    for j in range(NDEC):
        p = T + 1 + j  # position of the decoded token; its target is token p + 1
        assert np.all(np.isfinite(zs[j]))
        ce = _ce(zs[j], int(tk[p + 1]))
        ref = float(loss_b[p])
        e = abs(ce - ref) / abs(ref)
        say(f"  decode at position {p}: CE {ce:.5f}  prefill loss {ref:.5f}  rel err {e:.3e}")
        assert e < LOSS_TOL
