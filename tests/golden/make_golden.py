"""Writes expected values for the full-size 3B-shape parity test.

Calls only the input generators (synth) and the CPU oracle: the 3B-shape
weights and the first 1025 tokens of its Zipf stream are generated on the
host, the float32 oracle runs the inner loop over them (mini-batch 0 with one
SGD step, then the forward-only position 1024), and the file stores

  * the per-token losses of positions 0..1023;
  * for every dynamic block and matrix, 4096 seeded sample coordinates, the
    oracle's fast weights there after the step, and max |W1 - W0| over the
    whole matrix (the normaliser of the update-relative error);
  * a fingerprint of the inputs (token ids, a few weight values).

Usage: python tests/golden/make_golden.py  (about 10 minutes, ~30 GB RAM)
"""
import os
import sys
import time

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, os.path.dirname(os.path.dirname(HERE)))

import synth  # noqa: E402
from oracle import ttt_e2e as O  # noqa: E402

OUT = os.path.join(HERE, "ttt_3b_minibatch0.npz")
NSAMPLE = 4096


def main():
    c = synth.config("3b")
    t0 = time.time()
    w = synth.gen_weights(c)
    print(f"weights generated in {time.time() - t0:.0f} s", flush=True)
    tok = synth.gen_tokens(c, n=c["minibatch"] + 1).numpy()
    wn = synth.weights_to_numpy(w, np.float32)
    del w
    t0 = time.time()
    out = O.ttt_inner_loop(c, wn, tok, dtype=np.float32)
    print(f"oracle ran in {time.time() - t0:.0f} s", flush=True)
    rng = np.random.default_rng(1234)
    rec = {"loss": out["loss"].astype(np.float32), "tokens": tok.astype(np.int32),
           "embed_head": wn["embed"][:4, :8].copy(), "w3_head": wn["layers"][27]["w3"][:4, :8].copy()}
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
    main()
