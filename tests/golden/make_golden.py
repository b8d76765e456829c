"""Writes expected values for the full-size bf16 parity tests.

Calls only the input generators (synth) and the CPU oracle. Cases:

  * 3b_minibatch0 (default): the 3B-shape weights and the first 1025 tokens
    of its Zipf stream; the float32 oracle runs mini-batch 0 with one SGD
    step, then the forward-only position 1024 (about 10 minutes, ~30 GB RAM);
  * 1b_full: the 1B-shape weights and its whole 32768-token stream: all 32
    mini-batches and their updates (about 35 minutes, ~27 GB RAM);
  * 3b_8minibatches: the 3B-shape weights and the first 8193 tokens of its
    stream: 8 mini-batches and their updates, then the forward-only
    position 8192 (about 30 minutes, ~30 GB RAM);
  * 3b_decode8k: the 3B-shape weights, a TTT prefill of the first 8192
    tokens (8 mini-batches and their updates), then 3 decode steps with
    tokens 8192 .. 8194 over the full 8192-key window (about 30 minutes).
    Instead of fast-weight samples it stores, per decode step, 16384
    seeded logit samples, the 16 largest logits and max |z|;
  * 3b_16minibatches: the 3B-shape weights and the first 16385 tokens of
    its stream: 16 mini-batches and their updates (the first 8 fill the
    8192-key window, the last 8 run with the window sliding across
    mini-batch edges), the forward-only position 16384, then 3 decode
    steps with tokens 16385 .. 16387 (about 80 minutes, ~35 GB RAM).
    It stores both the loop record and the decode record.

For the loop cases the file also holds, for every dynamic matrix, the
maximum over each row and over each column of |W_T - W0| (a wrong row or
column of the GPU's update changes its maximum, whichever entries the
samples hit).

Each file stores the per-token losses; for every dynamic block and matrix,
4096 seeded sample coordinates, the oracle's fast weights there after the
last update, and max |W_T - W0| over the whole matrix (the normaliser of the
update-relative error); and a fingerprint of the inputs (token ids, a few
weight values).

Usage: python tests/golden/make_golden.py [3b_minibatch0 | 1b_full | 3b_8minibatches | 3b_decode8k |
                                           3b_16minibatches]
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
    "3b_decode8k": ("3b", lambda c: 8 * c["minibatch"] + NDEC, "ttt_3b_decode8k.npz"),
    "3b_16minibatches": ("3b", lambda c: 16 * c["minibatch"] + 1 + NDEC, "ttt_3b_16minibatches.npz"),
}
NDEC = 3          # decode steps of the decode case
NLOGIT = 16384    # sampled logits per decode step


def decode_record(zs, rec):
    """Per decode step: seeded logit samples, the 16 largest logits, max |z|."""
    rng = np.random.default_rng(4321)
    for j, z in enumerate(zs):
        idx = rng.integers(0, z.size, NLOGIT)
        top = np.argsort(-z)[:16]
        rec[f"z{j}_idx"] = idx.astype(np.int64)
        rec[f"z{j}_val"] = z[idx].astype(np.float32)
        rec[f"z{j}_top_idx"] = top.astype(np.int64)
        rec[f"z{j}_top_val"] = z[top].astype(np.float32)
        rec[f"z{j}_absmax"] = np.float64(np.max(np.abs(z)))


def loop_record(out, wn, rec, with_extrema):
    """Per-token losses and, per dynamic matrix, sampled final values, the
    normaliser max |W_T - W0| and (optionally) row and column maxima of
    |W_T - W0|."""
    rng = np.random.default_rng(1234)
    rec["loss"] = out["loss"].astype(np.float32)
    for i, (blk, b0) in enumerate(zip(out["dyn"], wn["dyn"])):
        for k in ("w1", "w2", "w3"):
            W1, W0 = blk[k], b0[k]
            idx = rng.integers(0, W1.size, NSAMPLE)
            rec[f"d{i}_{k}_idx"] = idx.astype(np.int64)
            rec[f"d{i}_{k}_val"] = W1.reshape(-1)[idx].astype(np.float32)
            dW = np.abs(W1.astype(np.float64) - W0)
            rec[f"d{i}_{k}_den"] = np.float64(np.max(dW))
            if with_extrema:
                rec[f"d{i}_{k}_rowmax"] = np.max(dW, axis=1).astype(np.float64)
                rec[f"d{i}_{k}_colmax"] = np.max(dW, axis=0).astype(np.float64)


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
    rec = {"tokens": tok.astype(np.int32), "embed_head": wn["embed"][:4, :8].copy(),
           "w3_head": wn["layers"][-1]["w3"][:4, :8].copy()}
    if name in ("3b_decode8k", "3b_16minibatches"):
        T = len(tok) - NDEC
        st = O.ttt_inner_loop(c, wn, tok[:T], dtype=np.float32, keep_state=True)
        print(f"oracle prefill ran in {time.time() - t0:.0f} s", flush=True)
        zs = [O.decode_step(st, int(tok[T + j])) for j in range(NDEC)]
        print(f"oracle ran in {time.time() - t0:.0f} s", flush=True)
        rec["prefill_len"] = np.int64(T)
        decode_record(zs, rec)
        if name == "3b_16minibatches":
            loop_record(st, wn, rec, with_extrema=True)
    else:
        out = O.ttt_inner_loop(c, wn, tok, dtype=np.float32)
        print(f"oracle ran in {time.time() - t0:.0f} s", flush=True)
        loop_record(out, wn, rec, with_extrema=(name == "1b_full"))
    np.savez_compressed(OUT, **rec)
    print(f"wrote {OUT}", flush=True)


if __name__ == "__main__":
    main(*sys.argv[1:2])
