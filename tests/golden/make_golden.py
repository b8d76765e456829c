"""Writes expected values for the full-size bf16 parity tests.

Calls only the input generators (synth) and the CPU oracle. Two cases:

  * 3b_minibatch0 (default): the 3B-shape weights and the first 1025 tokens
    of its Zipf stream; the float32 oracle runs mini-batch 0 with one SGD
    step, then the forward-only position 1024 (about 10 minutes, ~30 GB RAM);
  * 1b_full: the 1B-shape weights and its whole 32768-token stream: all 32
    mini-batches and their updates (about 35 minutes, ~27 GB RAM);
  * 3b_8minibatches: the 3B-shape weights and the first 8193 tokens of its
    stream: 8 mini-batches and their updates, then the forward-only
    position 8192 (about 30 minutes, ~30 GB RAM).

Each file stores the per-token losses; for every dynamic block and matrix,
4096 seeded sample coordinates, the oracle's fast weights there after the
last update, and max |W_T - W0| over the whole matrix (the normaliser of the
update-relative error); and a fingerprint of the inputs (token ids, a few
weight values).

Usage: python tests/golden/make_golden.py [3b_minibatch0 | 1b_full | 3b_8minibatches]
"""
import os
import sys
import time

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, os.path.dirname(os.path.dirname(HERE)))

import synth  # noqa: E402
from oracle import ttt_e2e as O  # noqa: E402

NSAMPLE = 4096
CASES = {
    # name: (workload, tokens, output file)
    "3b_minibatch0": ("3b", lambda c: c["minibatch"] + 1, "ttt_3b_minibatch0.npz"),
    "1b_full": ("1b", lambda c: c["seq"], "ttt_1b_full.npz"),
    "3b_8minibatches": ("3b", lambda c: 8 * c["minibatch"] + 1, "ttt_3b_8minibatches.npz"),
}


def main(name="3b_minibatch0"):
    workload, ntok, fname = CASES[name]
    OUT = os.path.join(HERE, fname)
    c = synth.config(workload)
    t0 = time.time()
    w = synth.gen_weights(c)
    print(f"weights generated in {time.time() - t0:.0f} s", flush=True)
    tok = synth.gen_tokens(c, n=ntok(c)).numpy()
    wn = synth.weights_to_numpy(w, np.float32)
    del w
    t0 = time.time()
    out = O.ttt_inner_loop(c, wn, tok, dtype=np.float32)
    print(f"oracle ran in {time.time() - t0:.0f} s", flush=True)
    rng = np.random.default_rng(1234)
    rec = {"loss": out["loss"].astype(np.float32), "tokens": tok.astype(np.int32),
           "embed_head": wn["embed"][:4, :8].copy(), "w3_head": wn["layers"][-1]["w3"][:4, :8].copy()}
    for i, (blk, b0) in enumerate(zip(out["dyn"], wn["dyn"])):
        for k in ("w1", "w2", "w3"):
            W1, W0 = blk[k], b0[k]
            idx = rng.integers(0, W1.size, NSAMPLE)
            rec[f"d{i}_{k}_idx"] = idx.astype(np.int64)
            rec[f"d{i}_{k}_val"] = W1.reshape(-1)[idx].astype(np.float32)
            rec[f"d{i}_{k}_den"] = np.float64(np.max(np.abs(W1.astype(np.float64) - W0)))
    np.savez_compressed(OUT, **rec)
    print(f"wrote {OUT}", flush=True)


if __name__ == "__main__":
    main(*sys.argv[1:2])
