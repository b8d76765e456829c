"""Shared helpers for the GPU tests (no method arithmetic here)."""
import os
import re

import numpy as np
import torch

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def header_functions():
    """Names of the functions declared in include/*.h."""
    names = []
    inc = os.path.join(ROOT, "include")
    for f in sorted(os.listdir(inc)):
        if f.endswith(".h"):
            txt = open(os.path.join(inc, f)).read()
            txt = re.sub(r"/\*.*?\*/", "", txt, flags=re.S)
            names += re.findall(r"^\s*(?:const\s+)?[A-Za-z_][A-Za-z0-9_\s\*]*?\b([a-z0-9_]+)\s*\(",
                                txt, flags=re.M)
    return sorted(set(n for n in names if n.startswith(("ttt_", "e2ttt_", "lact_", "tttk_"))))


def to_device(w: dict, device="cuda") -> dict:
    def mv(t):
        return t.to(device)
    out = {"embed": mv(w["embed"]), "final_norm": mv(w["final_norm"])}
    out["lm_head"] = out["embed"] if w["lm_head"] is w["embed"] else mv(w["lm_head"])
    out["layers"] = [{k: mv(v) for k, v in x.items()} for x in w["layers"]]
    out["dyn"] = [{k: mv(v) for k, v in x.items()} for x in w["dyn"]]
    return out


def rel_loss_err(gpu, ref):
    gpu = np.asarray(gpu, np.float64)
    ref = np.asarray(ref, np.float64)
    return float(np.max(np.abs(gpu - ref) / np.abs(ref)))


def dw_err(w_gpu, w_ref, w0):
    """max |W_gpu - W_ref| / max |W_ref - W0| (update-normalised)."""
    w_gpu = np.asarray(w_gpu, np.float64)
    w_ref = np.asarray(w_ref, np.float64)
    w0 = np.asarray(w0, np.float64)
    den = np.max(np.abs(w_ref - w0))
    return float(np.max(np.abs(w_gpu - w_ref)) / den) if den > 0 else float(np.max(np.abs(w_gpu - w_ref)))


def say(msg):
    print(msg, flush=True)


def ring_capacity(c: dict, max_seq: int) -> int:
    """Positions held by each layer's key/value ring, by the rule that
    include/ttt.h states for ttt_config.prefix_slab."""
    b = c["minibatch"]
    slab = c.get("prefix_slab", 0)
    slab = min(slab, max_seq) if slab > 0 else min(max_seq, 16384)
    slab = max(slab, b)
    k = min(c["window"], max(max_seq, b))
    need = max(k + slab, 128)
    return 1 << (need - 1).bit_length()
