#!/usr/bin/env python3
"""Throughput of the TTT-E2E inner loop (prefill) on one MI355X.

Workload (default): the 3B-shape model -- 28 blocks, d = 3072, 24 query / 8 KV
heads of 128, SwiGLU 8192, vocab 128256, window 8192, the last 7 blocks
updated with a dynamic SwiGLU MLP -- over a 131072-token (128K) seeded
Zipf(1.1) stream, mini-batch b = 1024, alpha = 0.005, bf16 storage with fp32
accumulation and an fp32 fast-weight master. One step = one ttt_prefill
over the whole stream (hoisted prefix + 128 mini-batches of forward, CE,
backward and SGD update) after ttt_reset; inputs are resident in HBM.

Prints one JSON line: tokens/s, the fraction of the bf16 MFMA peak reached by
the whole step (algorithmic FLOPs / time / 2.5 PFLOP/s), the live roofline of
the dominant kernel -- the fused dW + fp32 SGD update product (the largest
kernel symbol by summed duration in the step's rocprofv3 trace), timed with
HIP events on its launch streams during the timed steps, against the HBM
roofline of the update's algorithmic bytes -- the HBM rates of the
cross-entropy and update kernels, a per-class table from the warm-up step,
and the CPU oracle timed on a bounded sample of the same workload (one
steady-state mini-batch).

Counter runs (each under `rocprofv3 --pmc FETCH_SIZE`, then WRITE_SIZE):
`--copy-probe` runs a plain 1 GiB device copy (the factor that turns the
counters into bytes); `--attn-replay` runs the distinct attention-forward
launches of one step at the workload's shapes through the kernel-level entry
point (tttk_attn_fwd): every prefix slab once, then every mini-batch once.
`--pmc-summary FETCH WRITE COPY_FETCH COPY_WRITE` turns the four runs'
counter_collection CSVs into bytes per launch of one step (prefix launches
weighted by the blocks of the hoisted prefix, mini-batch launches by the
updated blocks that run attention in the loop).
"""
import csv
import hashlib
import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "TTT prefill tokens/s @128K ctx 3B-shape, 1 MI355X; % bf16 MFMA peak"
PEAK_BF16_TFLOPS = 2500.0     # MI355X dense bf16 MFMA
PEAK_FP32_TFLOPS = 157.3
PEAK_HBM_GBS = 8000.0

# timing classes of the library (ttt_kernel_class in include/ttt.h)
KC = dict(gemm_prefix=0, attn_prefix=1, gemm_loop=2, attn_loop=3, lmhead=4, ce=5, attn_bwd=6, dw_sgd=7,
          other=8)
ROOF_CLASS = "dw_sgd"                          # the fused dW + SGD update product
ATTN_CLASSES = ("attn_prefix", "attn_loop")    # the attention forward kernel
TIMED_CLASSES = (ROOF_CLASS, "ce") + ATTN_CLASSES
ROOF_SOURCES = ("test_long_context_amd/csrc/attn2.hip", "test_long_context_amd/csrc/common.hpp")
UPD_SOURCES = ("test_long_context_amd/csrc/gemm_impl.hpp", "test_long_context_amd/csrc/gemm_tn.hip",
               "test_long_context_amd/csrc/gemm.hip", "test_long_context_amd/csrc/common.hpp",
               "test_long_context_amd/csrc/gemm_args.hpp")

# HBM traffic of the update products (the roofline kernel) from rocprofv3
# --pmc FETCH_SIZE / WRITE_SIZE of --update-replay, scaled by the
# --copy-probe counters (printed by --pmc-update-summary), bytes per launch
# averaged over a block's dW12 and dW3 launches, keyed by (workload, source
# hash): valid only for the kernel source the counters were taken on.
UPD_TRAFFIC = {
    ("3b", "e5fec951678275c0"): 500006785,
}

# HBM traffic of the attention forward from rocprofv3 --pmc FETCH_SIZE /
# WRITE_SIZE (--attn-replay, scaled by the --copy-probe counters; printed by
# --pmc-summary), keyed by (workload, T, source hash): valid only for the
# kernel source the counters were taken on.
TRAFFIC = {
    ("3b", 131072, "8e2b20072160d9a6"): dict(fetch_bytes_per_launch=58315148, write_bytes_per_launch=60356575,
                                             fetch_scale=1.9999, write_scale=1.0,
                                             traffic_bytes_per_launch=176983650),
}


# MFMA busy of the same kernel (rocprofv3 SQ_VALU_MFMA_BUSY_CYCLES over the
# SIMDs x active cycles, --pmc-busy), keyed like TRAFFIC.
MFMA_BUSY = {
    ("3b", 131072, "8e2b20072160d9a6"): 0.5104,
}


def roof_source_hash(files=ROOF_SOURCES) -> str:
    h = hashlib.sha256()
    for f in files:
        with open(os.path.join(ROOT, f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def update_replay(c, tla, torch, blocks=2):
    """The update products of `blocks` dynamic blocks at the workload's
    shape, launched as the engine launches them (dW3 = dY^T Hmid, then dW12
    = dH12^T U, each a GEMM with the SGD epilogue writing the fp32 master
    and the stochastically rounded bf16 working copy)."""
    d, Fd, b = c["d_model"], c["dyn_ffn_hidden"], c["minibatch"]
    bf = torch.bfloat16
    g = torch.Generator(device="cuda").manual_seed(0)
    gt = (torch.randn(b, d, device="cuda", generator=g) * 0.1).to(bf)
    hm = (torch.randn(b, Fd, device="cuda", generator=g) * 0.1).to(bf)
    dh12 = (torch.randn(b, 2 * Fd, device="cuda", generator=g) * 0.1).to(bf)
    xn = (torch.randn(b, d, device="cuda", generator=g) * 0.1).to(bf)
    m3 = torch.randn(d, Fd, device="cuda", generator=g) * 0.02
    m12 = torch.randn(2 * Fd, d, device="cuda", generator=g) * 0.02
    h3 = torch.empty(d, Fd, dtype=bf, device="cuda")
    h12 = torch.empty(2 * Fd, d, dtype=bf, device="cuda")
    for i in range(blocks):
        tla.gemm(gt, hm, d, Fd, b, "sgd", m3, a_kmajor=False, b_kmajor=False, C2=h3, scale=c["alpha"],
                 seed=2 * i + 1)
        tla.gemm(dh12, xn, 2 * Fd, d, b, "sgd", m12, a_kmajor=False, b_kmajor=False, C2=h12, scale=c["alpha"],
                 seed=2 * i + 2)
    torch.cuda.synchronize()
    print(json.dumps(dict(launches=2 * blocks)), flush=True)


def update_isolated_us(c, tla, torch, reps=5):
    """Average duration (us) of one update launch on an otherwise idle GPU:
    a block's dW3 and dW12 products with the SGD epilogue, as the engine
    launches them, timed with events over `reps` pairs after one warm-up
    pair (run after the timed region: context for the in-step figure, which
    shares the chip with the main stream)."""
    d, Fd, b = c["d_model"], c["dyn_ffn_hidden"], c["minibatch"]
    bf = torch.bfloat16
    g = torch.Generator(device="cuda").manual_seed(0)
    gt = (torch.randn(b, d, device="cuda", generator=g) * 0.1).to(bf)
    hm = (torch.randn(b, Fd, device="cuda", generator=g) * 0.1).to(bf)
    dh12 = (torch.randn(b, 2 * Fd, device="cuda", generator=g) * 0.1).to(bf)
    xn = (torch.randn(b, d, device="cuda", generator=g) * 0.1).to(bf)
    m3 = torch.randn(d, Fd, device="cuda", generator=g) * 0.02
    m12 = torch.randn(2 * Fd, d, device="cuda", generator=g) * 0.02
    h3 = torch.empty(d, Fd, dtype=bf, device="cuda")
    h12 = torch.empty(2 * Fd, d, dtype=bf, device="cuda")

    def pair(i):
        tla.gemm(gt, hm, d, Fd, b, "sgd", m3, a_kmajor=False, b_kmajor=False, C2=h3, scale=c["alpha"],
                 seed=2 * i + 1)
        tla.gemm(dh12, xn, 2 * Fd, d, b, "sgd", m12, a_kmajor=False, b_kmajor=False, C2=h12, scale=c["alpha"],
                 seed=2 * i + 2)
    pair(0)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for i in range(reps):
        pair(i + 1)
    e1.record()
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) * 1e3 / (2 * reps)


def pmc_update_summary(c, dirs, workload):
    """Bytes per update launch from FETCH_SIZE and WRITE_SIZE runs of
    --update-replay and of --copy-probe (each counter scaled by copy bytes /
    copy counter), averaged over the dW3 and dW12 launches."""
    def read(d, name_part):
        f = os.path.join(d, "run_counter_collection.csv")
        with open(f) as fh:
            return [float(r["Counter_Value"]) * 1024 for r in csv.DictReader(fh) if name_part in r["Kernel_Name"]]
    fetch, write = read(dirs[0], "gemm_bf16_kernel"), read(dirs[1], "gemm_bf16_kernel")
    cf, cw = read(dirs[2], "copyBuffer"), read(dirs[3], "copyBuffer")
    copy_bytes = float(1 << 30)
    fs, ws = copy_bytes / (sum(cf) / len(cf)), copy_bytes / (sum(cw) / len(cw))
    assert len(fetch) == len(write) and len(fetch) % 2 == 0, (len(fetch), len(write))
    n = len(fetch)
    d, Fd = c["d_model"], c["dyn_ffn_hidden"]
    algo = 10.0 * 3 * d * Fd / 2   # per launch, averaged over dW3 and dW12
    out = dict(kernel="gemm_bf16_kernel (SGD epilogue)", workload=workload,
               source_sha=roof_source_hash(UPD_SOURCES), fetch_scale=round(fs, 4), write_scale=round(ws, 4),
               launches=n, fetch_bytes_per_launch=round(sum(fetch) / n), write_bytes_per_launch=round(sum(write) / n),
               traffic_bytes_per_launch=round((sum(fetch) * fs + sum(write) * ws) / n),
               dw3_traffic=round(fetch[0] * fs + write[0] * ws), dw12_traffic=round(fetch[1] * fs + write[1] * ws),
               algorithmic_bytes_per_launch=round(algo))
    print(json.dumps(out), flush=True)


def copy_probe():
    import torch
    n = 1 << 28  # 1 GiB of float32
    x = torch.ones(n, dtype=torch.float32, device="cuda")
    y = torch.empty_like(x)
    torch.cuda.synchronize()
    for _ in range(3):
        y.copy_(x)
    torch.cuda.synchronize()
    print(json.dumps(dict(copy_bytes_per_dispatch=n * 4, dispatches=3)), flush=True)


def algorithmic_flops(c: dict, T: int) -> float:
    """Matrix-product FLOPs of one prefill (recompute not counted; the causal
    window counted exactly)."""
    L, d, H, Hk, dh = c["n_layers"], c["d_model"], c["n_heads"], c["n_kv_heads"], c["head_dim"]
    F, Fd, V, k, b = c["ffn_hidden"], c["dyn_ffn_hidden"], c["vocab"], c["window"], c["minibatch"]
    Ld = c["n_dynamic"] or L - (3 * L) // 4
    Pa = d * H * dh + 2 * d * Hk * dh + H * dh * d
    Pm, Pmd = 3 * d * F, 3 * d * Fd
    kk = min(k, T)
    Wsum = kk * (kk + 1) / 2 + (T - kk) * k
    Ib = sum(min(b, T - a) * (min(b, T - a) + 1) / 2 for a in range(0, T, b))
    fwd = 2 * (L * (Pa + Pm) + Ld * Pmd + d * V) * T + L * 4 * H * dh * Wsum
    bwd = (2 * d * V + (Ld - 1) * (4 * Pmd + 2 * Pm + 2 * Pa) + 2 * Pmd + 2 * d * Fd) * T
    bwd += (Ld - 1) * (4 * H * dh * Wsum + 4 * H * dh * Ib)
    return float(fwd + bwd)


def _host_threads():
    try:
        from threadpoolctl import threadpool_info
        return max([x.get("num_threads", 0) for x in threadpool_info()] + [1])
    except Exception:
        return os.cpu_count()


def _oracle_weights(w):
    wn = {"embed": w["embed"].float().cpu().numpy(), "final_norm": w["final_norm"].float().cpu().numpy()}
    wn["lm_head"] = wn["embed"]
    wn["layers"] = [{k: v.float().cpu().numpy() for k, v in x.items()} for x in w["layers"]]
    wn["dyn"] = [{k: v.float().cpu().numpy() for k, v in x.items()} for x in w["dyn"]]
    return wn


def cpu_baseline(c, w, tok):
    """The oracle (float32 numpy) on one steady-state mini-batch of the same
    stream: positions [k, k + b) (the window then holds k earlier keys for
    every query) run forward through every block, cross-entropy, backward
    and the SGD step (oracle.ttt_e2e.minibatch_step), with the key/value
    store of positions [0, k) filled with random values (the cost does not
    depend on them). Tokens/s of that mini-batch is the oracle's rate in the
    steady state, which is where a long stream spends almost all its time."""
    import numpy as np
    from oracle import ttt_e2e as O
    cores = _host_threads()
    cfg = O.Cfg.from_dict(c)
    T = tok.numel()
    a = min(cfg.window, max(0, T - 2) // cfg.b * cfg.b)
    e = min(a + cfg.b, T - 1)
    wc = O._cast_weights(_oracle_weights(w), np.float32)
    dyn = [{k: np.array(b_[k]) for k in ("w1", "w2", "w3")} for b_ in wc["dyn"]]
    store = O.KVStore(cfg, e + 1, np.float32)
    rng = np.random.default_rng(0)
    for l in range(cfg.L):
        store.K[l][:a] = rng.standard_normal((a, cfg.Hk, cfg.dh), dtype=np.float32)
        store.V[l][:a] = rng.standard_normal((a, cfg.Hk, cfg.dh), dtype=np.float32)
    store.n = a
    t = tok[: e + 1].cpu().numpy().astype(np.int64)
    loss = np.zeros(e, dtype=np.float32)
    t0 = time.perf_counter()
    O.minibatch_step(cfg, wc, dyn, store, t, a, e, cfg.alpha, cfg.reduction, loss)
    dt = time.perf_counter() - t0
    assert np.all(np.isfinite(loss[a:e]))
    n = e - a
    return dict(value=round(n / dt, 2), unit="tokens/s", cores=int(cores), kind="oracle",
                sample=f"one steady-state mini-batch: positions {a}..{e - 1} of the same stream, each query "
                       f"seeing {'the full ' + str(cfg.window) + '-key window' if a >= cfg.window else 'every earlier key'} "
                       f"(store of the {a} earlier positions filled with random values), forward through all "
                       f"{cfg.L} blocks, cross-entropy, backward and the SGD step; {dt:.1f} s on the host",
                seconds=round(dt, 2))


def cpu_decode_baseline(c, w, p, nsteps=2):
    """The oracle's decode (float32 numpy) of nsteps tokens at position p of
    the same model: a full window of stored keys/values (random values: the
    cost does not depend on them) and the initial fast weights."""
    import numpy as np
    from oracle import ttt_e2e as O
    cores = _host_threads()
    cfg = O.Cfg.from_dict(c)
    wc = O._cast_weights(_oracle_weights(w), np.float32)
    store = O.KVStore(cfg, p + nsteps + 1, np.float32)
    rng = np.random.default_rng(0)
    lo = max(0, p - cfg.window)
    for l in range(cfg.L):
        store.K[l][lo:p] = rng.standard_normal((p - lo, cfg.Hk, cfg.dh), dtype=np.float32)
        store.V[l][lo:p] = rng.standard_normal((p - lo, cfg.Hk, cfg.dh), dtype=np.float32)
    store.n = p
    state = dict(cfg=cfg, weights=wc, store=store, dyn=[{k: np.array(b[k]) for k in ("w1", "w2", "w3")} for b in wc["dyn"]])
    t0 = time.perf_counter()
    for j in range(nsteps):
        z = O.decode_step(state, j % c["vocab"])
    dt = time.perf_counter() - t0
    assert np.all(np.isfinite(z))
    return dict(value=round(dt / nsteps * 1e3, 1), unit="ms/token", cores=int(cores), kind="oracle",
                sample=f"{nsteps} decode steps at position {p} (full {cfg.window}-key window); {dt:.1f} s on the host",
                seconds=round(dt, 2))


def e2_bench(args, tla, torch, synth):
    """E2-TTT chunk-end state over the whole sequence (16 heads x 32768
    tokens, D 128, chunks of 2048): e2ttt_chunk_scan timed with HIP events;
    HBM roofline on its algorithmic bytes; the oracle's closed form timed on
    the host."""
    import numpy as np
    e = synth.E2_CONFIG
    H, T, D, C = e["heads"], e["seq"], e["dim"], e["chunk"]
    x = synth.gen_e2(H, T, D, e["seed"], device="cuda")
    W0, M0 = x["W"].clone(), x["M"].clone()
    W, M = x["W"], x["M"]
    for _ in range(max(1, args.warmup)):
        W.copy_(W0)
        M.copy_(M0)
        tla.e2ttt_chunk_scan(x["k"], x["v"], x["eta"], x["beta"], x["gamma"], W, M, C)
    torch.cuda.synchronize()
    ts = []
    for _ in range(args.steps):
        W.copy_(W0)
        M.copy_(M0)
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        tla.e2ttt_chunk_scan(x["k"], x["v"], x["eta"], x["beta"], x["gamma"], W, M, C)
        b.record()
        torch.cuda.synchronize()
        ts.append(a.elapsed_time(b))
    ms = sorted(ts)[len(ts) // 2]
    nch = (T + C - 1) // C
    algo = 2 * H * T * D * 2 + 3 * H * T * 4 + nch * H * D * D * 4 * 2 * 2   # k, v; eta, beta, gamma; W, M per chunk
    gbs = algo / (ms * 1e-3) / 1e9
    flops = H * nch * 3 * 2 * C * D * D
    out = dict(metric="E2-TTT chunk-end state (16 heads x 32K tokens, D 128, C 2048), 1 MI355X",
               value=round(H * T / (ms * 1e-3), 1), unit="token-heads/s", n_gpus=1, steps=args.steps,
               warmup=args.warmup, ms_per_step=round(ms, 4), higher_is_better=True, scaling="weak",
               vs_baseline=None, dtype="bf16 inputs, fp32/fp64 scalars", data="synthetic",
               config=dict(workload=f"e2ttt chunk scan, H={H}, T={T}, D={D}, C={C}"),
               roofline=dict(bound="hbm", achieved=round(gbs, 1), peak=PEAK_HBM_GBS, unit="GB/s",
                             frac=round(gbs / PEAK_HBM_GBS, 4), traffic=None,
                             kernel="e2ttt_chunk_scan (scalar scan, one fused aggregation + update launch per chunk)",
                             algorithmic_bytes=algo, mfma_tflops=round(flops / (ms * 1e-3) / 1e12, 2)))
    # the chunk-wise baseline (LaCT's rule: one aggregation per chunk) on the
    # same inputs: the pages quote the exact kernel's throughput cost against it
    lts = []
    for i in range(max(1, args.warmup) + args.steps):
        W.copy_(W0)
        M.copy_(M0)
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        tla.lact_chunk_scan(x["k"], x["v"], x["eta"], x["beta"], W, M, C)
        b.record()
        torch.cuda.synchronize()
        if i >= max(1, args.warmup):
            lts.append(a.elapsed_time(b))
    lms = sorted(lts)[len(lts) // 2]
    # the token mixer's TTT path on its own workload (projections, SiLU +
    # L2 norm, input-dependent scalars, outputs and chunk-end state)
    mc = synth.E2_MIXER_CONFIG
    mx = synth.gen_e2_mixer(mc["heads"], mc["seq"], mc["dim"], mc["d_model"], mc["seed"], device="cuda")
    mW, mM = mx["W"].clone(), mx["M"].clone()
    mo = torch.empty(mc["seq"], mc["heads"] * mc["dim"], device="cuda")
    mts = []
    for i in range(max(1, args.warmup) + args.steps):
        mW.copy_(mx["W"])
        mM.copy_(mx["M"])
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        tla.e2ttt_mixer_forward(mx["x"], mx["wqkv"], mx["bias"], mc["eta_base"], mc["alpha_base"], mc["tau"], mW, mM,
                                mc["heads"], mc["chunk"], out=mo)
        b.record()
        torch.cuda.synchronize()
        if i >= max(1, args.warmup):
            mts.append(a.elapsed_time(b))
    mms = sorted(mts)[len(mts) // 2]
    proj_flops = 2.0 * mc["seq"] * mc["d_model"] * (3 * mc["heads"] * mc["dim"] + 3 * mc["heads"])
    out["mixer"] = dict(ms_per_step=round(mms, 4), value=round(mc["seq"] / (mms * 1e-3), 1), unit="tokens/s",
                        config=f"E2-TTT token mixer, TTT path: T={mc['seq']}, d_model={mc['d_model']}, "
                               f"H={mc['heads']} x {mc['dim']}, C={mc['chunk']}",
                        projection_gflop=round(proj_flops / 1e9, 1))
    # the same mixer with the SwiGLU fast-weight net
    sc = synth.E2_MLP_CONFIG
    sx = synth.gen_e2_mixer(sc["heads"], sc["seq"], sc["dim"], sc["d_model"], sc["seed"], device="cuda")
    s0 = synth.gen_e2_mlp_state(sc["heads"], sc["dim"], sc["hidden"], sc["seed"], device="cuda")
    sst = {k_: v_.clone() for k_, v_ in s0.items()}
    so = torch.empty(sc["seq"], sc["heads"] * sc["dim"], device="cuda")
    sts = []
    for i in range(max(1, args.warmup) + args.steps):
        for k_ in sst:
            sst[k_].copy_(s0[k_])
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        tla.e2ttt_mixer_swiglu_forward(sx["x"], sx["wqkv"], sx["bias"], sc["eta_base"], sc["alpha_base"], sc["tau"],
                                       sst, sc["heads"], sc["chunk"], out=so)
        b.record()
        torch.cuda.synchronize()
        if i >= max(1, args.warmup):
            sts.append(a.elapsed_time(b))
    sms = sorted(sts)[len(sts) // 2]
    # matrix-product FLOPs per token and head: forward of key and query
    # (2 x (2 Dh D + Dh D) x 2), backward through W3 twice (2 x Dh D x 2) and
    # four aggregations (2 x (Dh D + 2 Dh D) x 2)
    Dh_, D_ = sc["hidden"], sc["dim"]
    fw_flops = sc["seq"] * sc["heads"] * (12 * Dh_ * D_ + 4 * Dh_ * D_ + 12 * Dh_ * D_)
    out["swiglu_mixer"] = dict(ms_per_step=round(sms, 4), value=round(sc["seq"] / (sms * 1e-3), 1),
                               unit="tokens/s",
                               config=f"E2-TTT token mixer, SwiGLU fast-weight net: T={sc['seq']}, "
                                      f"d_model={sc['d_model']}, H={sc['heads']} x {D_}, hidden {Dh_}, "
                                      f"C={sc['chunk']}",
                               fast_weight_gflop=round(fw_flops / 1e9, 1),
                               fast_weight_tflops=round(fw_flops / (sms * 1e-3) / 1e12, 1))
    # the same mixer with the GELU fast-weight net
    gc = synth.E2_GELU_CONFIG
    gx = synth.gen_e2_mixer(gc["heads"], gc["seq"], gc["dim"], gc["d_model"], gc["seed"], device="cuda")
    g0 = synth.gen_e2_gelu_state(gc["heads"], gc["dim"], gc["hidden"], gc["seed"], device="cuda")
    gst = {k_: v_.clone() for k_, v_ in g0.items()}
    go = torch.empty(gc["seq"], gc["heads"] * gc["dim"], device="cuda")
    gts = []
    for i in range(max(1, args.warmup) + args.steps):
        for k_ in gst:
            gst[k_].copy_(g0[k_])
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        tla.e2ttt_mixer_gelu_forward(gx["x"], gx["wqkv"], gx["bias"], gc["eta_base"], gc["alpha_base"], gc["tau"],
                                     gst, gc["heads"], gc["chunk"], out=go)
        b.record()
        torch.cuda.synchronize()
        if i >= max(1, args.warmup):
            gts.append(a.elapsed_time(b))
    gms = sorted(gts)[len(gts) // 2]
    # matrix-product FLOPs per token and head: forward of key and query
    # (2 x (Dh D + D Dh) x 2), backward through W2 twice (2 x D Dh x 2) and
    # four aggregations (2 x (D Dh + Dh D) x 2)
    Dh_, D_ = gc["hidden"], gc["dim"]
    gf_flops = gc["seq"] * gc["heads"] * (8 * Dh_ * D_ + 4 * Dh_ * D_ + 8 * Dh_ * D_)
    out["gelu_mixer"] = dict(ms_per_step=round(gms, 4), value=round(gc["seq"] / (gms * 1e-3), 1),
                             unit="tokens/s",
                             config=f"E2-TTT token mixer, GELU fast-weight net: T={gc['seq']}, "
                                    f"d_model={gc['d_model']}, H={gc['heads']} x {D_}, hidden {Dh_}, "
                                    f"C={gc['chunk']}",
                             fast_weight_gflop=round(gf_flops / 1e9, 1),
                             fast_weight_tflops=round(gf_flops / (gms * 1e-3) / 1e12, 1))
    # the hybrid block: SWA beside the SwiGLU TTT path, gated
    hc = synth.E2_HYBRID_CONFIG
    hx = synth.gen_e2_mixer(hc["heads"], hc["seq"], hc["dim"], hc["d_model"], hc["seed"], device="cuda")
    hg = synth.gen_gate(hc["heads"], hc["dim"], hc["d_model"], hc["seed"], device="cuda")
    h0 = synth.gen_e2_mlp_state(hc["heads"], hc["dim"], hc["hidden"], hc["seed"], device="cuda")
    hst = {k_: v_.clone() for k_, v_ in h0.items()}
    ho = torch.empty(hc["seq"], hc["heads"] * hc["dim"], device="cuda")
    hts = []
    for i in range(max(1, args.warmup) + args.steps):
        for k_ in hst:
            hst[k_].copy_(h0[k_])
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        tla.e2ttt_hybrid_forward(hx["x"], hx["wqkv"], hx["bias"], hg["wgate"], hg["bgate"], hc["eta_base"],
                                 hc["alpha_base"], hc["tau"], hc["rope_theta"], hc["window"], hst, hc["heads"],
                                 hc["chunk"], out=ho)
        b.record()
        torch.cuda.synchronize()
        if i >= max(1, args.warmup):
            hts.append(a.elapsed_time(b))
    hms = sorted(hts)[len(hts) // 2]
    out["hybrid_block"] = dict(ms_per_step=round(hms, 4), value=round(hc["seq"] / (hms * 1e-3), 1), unit="tokens/s",
                               config=f"E2-TTT hybrid block (SWA window {hc['window']} beside the SwiGLU TTT path, "
                                      f"gated): T={hc['seq']}, d_model={hc['d_model']}, H={hc['heads']} x "
                                      f"{hc['dim']}, hidden {hc['hidden']}, C={hc['chunk']}")
    out["lact_baseline"] = dict(ms_per_step=round(lms, 4), value=round(H * T / (lms * 1e-3), 1),
                                unit="token-heads/s", e2_cost_vs_lact=round(ms / lms - 1.0, 4),
                                kernel="lact_chunk_scan (chunk-mean momentum, one aggregation per chunk)")
    if not args.no_cpu_baseline:
        from oracle import e2ttt as E
        xs = {k_: v_.double().cpu().numpy() for k_, v_ in x.items() if k_ in ("k", "v", "eta", "beta", "gamma")}
        t0 = time.perf_counter()
        E.e2_closed_form(xs["k"], xs["v"], xs["eta"], xs["beta"], xs["gamma"], W0.double().cpu().numpy(),
                         M0.double().cpu().numpy(), C)
        dt = time.perf_counter() - t0
        out["cpu_baseline"] = dict(value=round(H * T / dt, 1), unit="token-heads/s", cores=int(_host_threads()),
                                   kind="oracle", sample=f"the whole workload, float64 numpy; {dt:.1f} s on the host",
                                   seconds=round(dt, 2))
    else:
        out["cpu_baseline"] = None
    print(json.dumps(out), flush=True)


def attn_launches(c: dict, T: int):
    """(kind, n, pos0) of the distinct attention-forward launches of one step
    and the number of blocks that make each: the prefix covers blocks 0..s in
    slabs of up to 16384 positions, the loop blocks s+1..L-1 per mini-batch."""
    L = c["n_layers"]
    nd = c["n_dynamic"] or L - (3 * L) // 4
    s = L - nd
    slab = max(min(T + 1024, 16384), c["minibatch"])
    out = [("prefix", min(slab, T - p0), p0, s + 1) for p0 in range(0, T, slab)]
    out += [("loop", min(c["minibatch"], T - a0), a0, L - s - 1) for a0 in range(0, T, c["minibatch"])]
    return out


def attn_replay(c, T, tla, torch):
    """The attention forward launches of one step (attn_launches), each once,
    on random rings of the engine's capacity."""
    H, Hk, dh, k = c["n_heads"], c["n_kv_heads"], c["head_dim"], c["window"]
    slab = max(min(T + 1024, 16384), c["minibatch"])
    cap = 1 << (max(k + max(c["minibatch"], slab), 128) - 1).bit_length()
    bf = torch.bfloat16
    g = torch.Generator(device="cuda").manual_seed(0)
    K = torch.randn(Hk, cap, dh, device="cuda", generator=g).to(bf)
    V = torch.randn(Hk, cap, dh, device="cuda", generator=g).to(bf)
    sl = torch.arange(cap, device="cuda")
    perm = (sl & ~15) | (sl & 3) | ((sl & 4) << 1) | ((sl & 8) >> 1)  # the store's slot order
    VT = torch.empty(Hk, dh, cap, dtype=bf, device="cuda")
    VT[:, :, perm] = V.transpose(1, 2)
    q = torch.randn(slab, H, dh, device="cuda", generator=g).to(bf)
    o = torch.empty(slab, H, dh, dtype=bf, device="cuda")
    launches = attn_launches(c, T)
    for kind, n, p0, _ in launches:
        ws = tla.attn_fwd_workspace(n, H, dh, k, 0)   # the engine's key split for this shape
        work = torch.empty(max(ws // 4, 1), device="cuda")
        tla.attn_fwd(q[:n].contiguous() if n < slab else q, K, V, o, None, n, H, Hk, dh, cap, k, p0, vt=VT,
                     ksplit=0, work=work)
    torch.cuda.synchronize()
    print(json.dumps(dict(launches=len(launches))), flush=True)


def pmc_summary(c, T, dirs, workload):
    """Bytes per attention-forward launch of one step from four rocprofv3
    counter runs (FETCH_SIZE and WRITE_SIZE of --attn-replay and of
    --copy-probe), each counter scaled by copy bytes / copy counter."""
    def read(d, name_part):
        f = os.path.join(d, "run_counter_collection.csv")
        with open(f) as fh:
            return [float(r["Counter_Value"]) * 1024 for r in csv.DictReader(fh) if name_part in r["Kernel_Name"]]
    fetch, write = read(dirs[0], "attn_fwd2_kernel"), read(dirs[1], "attn_fwd2_kernel")
    cf, cw = read(dirs[2], "copyBuffer"), read(dirs[3], "copyBuffer")
    copy_bytes = float(1 << 30)
    fs, ws = copy_bytes / (sum(cf) / len(cf)), copy_bytes / (sum(cw) / len(cw))
    launches = attn_launches(c, T)
    assert len(fetch) == len(write) == len(launches), (len(fetch), len(write), len(launches))
    tot_n = sum(wt for *_, wt in launches)
    tf = sum(f * wt for f, (*_, wt) in zip(fetch, launches))
    tw = sum(x * wt for x, (*_, wt) in zip(write, launches))
    out = dict(kernel="attn_fwd2_kernel", workload=workload, seq=T, source_sha=roof_source_hash(),
               fetch_scale=round(fs, 4), write_scale=round(ws, 4), launches_per_step=tot_n,
               fetch_bytes_per_launch=round(tf / tot_n), write_bytes_per_launch=round(tw / tot_n),
               traffic_bytes_per_launch=round((tf * fs + tw * ws) / tot_n))
    print(json.dumps(out), flush=True)


def decode_bytes(c: dict, p: int) -> float:
    """HBM bytes one decode step must read at position p: every weight once
    (static weights and the dynamic MLPs' working copy in the storage dtype,
    lm_head) and the window's keys and values in every block."""
    L, d, H, Hk, dh = c["n_layers"], c["d_model"], c["n_heads"], c["n_kv_heads"], c["head_dim"]
    F, Fd, V, k = c["ffn_hidden"], c["dyn_ffn_hidden"], c["vocab"], c["window"]
    Ld = c["n_dynamic"] or L - (3 * L) // 4
    es = 2 if c["dtype"] == "bf16" else 4
    static = L * ((H + 2 * Hk) * dh * d + d * H * dh + 3 * F * d) * es + V * d * es
    dyn = Ld * 3 * Fd * d * es
    kv = L * min(p + 1, k) * Hk * dh * 2 * es
    return float(static + dyn + kv)


def decode_bench(args, c, w, tok, tla, torch):
    """Decode latency after prefills of 8K, 32K and 128K tokens: 256
    teacher-forced steps each, every step timed with HIP events."""
    ctxs = [x for x in (8192, 32768, 131072) if x + args.decode_steps <= tok.numel()]
    m = tla.TTT(c, w, max_seq=max(ctxs) + args.decode_steps + 1)
    # warm-up: the first decode step captures the launch graph
    m.prefill(tok[:ctxs[0]])
    m.decode_step(tok[ctxs[0]:ctxs[0] + 1])
    m.sync()
    res = {}
    for ctx in ctxs:
        m.reset()
        m.prefill(tok[:ctx])
        m.sync()
        ev = [torch.cuda.Event(enable_timing=True) for _ in range(args.decode_steps + 1)]
        logits = torch.empty(c["vocab"], dtype=torch.float32, device="cuda")
        ev[0].record()
        for j in range(args.decode_steps):
            m.decode_step(tok[ctx + j:ctx + j + 1], logits)
            ev[j + 1].record()
        torch.cuda.synchronize()
        m.sync()
        ts = sorted(ev[j].elapsed_time(ev[j + 1]) for j in range(args.decode_steps))
        p50, p99 = ts[len(ts) // 2], ts[min(len(ts) - 1, int(0.99 * len(ts)))]
        gbs = decode_bytes(c, ctx) / (p50 * 1e-3) / 1e9
        res[str(ctx)] = dict(p50_ms=round(p50, 3), p99_ms=round(p99, 3), hbm_gb_per_token=round(decode_bytes(c, ctx) / 1e9, 3),
                             achieved_gbs=round(gbs, 1))
        print(f"# decode after {ctx}: p50 {p50:.3f} ms  p99 {p99:.3f} ms  {gbs:.0f} GB/s", file=sys.stderr, flush=True)
    m.close()
    big, small = res[str(ctxs[-1])], res[str(ctxs[0])]
    out = dict(metric="TTT decode latency @3B-shape after a TTT prefill, 1 MI355X", value=big["p50_ms"],
               unit="ms/token (p50)", n_gpus=1, steps=args.decode_steps, higher_is_better=False,
               dtype="bf16" if c["dtype"] == "bf16" else "f32", data="synthetic",
               config=dict(workload=f"{args.workload}-shape decode, {args.decode_steps} teacher-forced steps after "
                                    f"prefills of {', '.join(str(x) for x in ctxs)} tokens", window=c["window"]),
               contexts=res, flat_ratio=round(big["p50_ms"] / small["p50_ms"], 3),
               roofline=dict(bound="hbm", achieved=big["achieved_gbs"], peak=PEAK_HBM_GBS, unit="GB/s",
                             frac=round(big["achieved_gbs"] / PEAK_HBM_GBS, 4), traffic=None,
                             kernel="whole decode step (GEMVs, window attention, lm_head)"))
    out["cpu_baseline"] = None if args.no_cpu_baseline else cpu_decode_baseline(c, w, ctxs[0])
    print(json.dumps(out), flush=True)


def decode_update_bench(args, c, w, tok, tla, torch):
    """Decode with test-time updates at the 3B shape: a prefill of 8192 + 1
    tokens, then decode steps with ttt_decode_step_update until one update
    (the b positions from 8192) has run and b more steps after it; every
    step timed with HIP events. Reports the p50 of the plain steps, the
    step that carried the update, and the cost per token amortised over a
    mini-batch of b decode steps."""
    b = c["minibatch"]
    T = 8192 + 1
    nsteps = 2 * b
    m = tla.TTT(c, w, max_seq=T + nsteps + 1)
    m.prefill(tok[:T])
    m.decode_step(tok[T:T + 1])   # captures the decode graph; position T
    m.reset()
    m.prefill(tok[:T])
    m.sync()
    logits = torch.empty(c["vocab"], dtype=torch.float32, device="cuda")
    loss = torch.empty(b, dtype=torch.float32, device="cuda")
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(nsteps + 1)]
    upd_at = []
    ev[0].record()
    for j in range(nsteps):
        _, l = m.decode_step_update(tok[T + j:T + j + 1], logits, loss)
        if l is not None:
            upd_at.append(j)
        ev[j + 1].record()
    torch.cuda.synchronize()
    m.sync()
    m.close()
    ts = [ev[j].elapsed_time(ev[j + 1]) for j in range(nsteps)]
    plain = sorted(t for j, t in enumerate(ts) if j not in upd_at)
    p50 = plain[len(plain) // 2]
    upd_ms = [ts[j] for j in upd_at]
    amort = (p50 * (b - 1) + (sum(upd_ms) / max(1, len(upd_ms)))) / b
    out = dict(metric="TTT decode with test-time updates @3B-shape, per-token latency amortised over a mini-batch",
               value=round(amort, 4), unit="ms/token", n_gpus=1, steps=nsteps, higher_is_better=False,
               dtype="bf16", data="synthetic",
               config=dict(workload=f"{args.workload}-shape decode with updates: prefill {T} tokens, then {nsteps} "
                                    f"decode steps, an update every {b}"),
               plain_step_p50_ms=round(p50, 3), update_steps=len(upd_at),
               update_step_ms=[round(x, 3) for x in upd_ms])
    print(json.dumps(out), flush=True)


def kb_sweep(args, tla, torch, synth):
    """Throughput of the 3B-shape prefill over the window k and the
    mini-batch b ([P2] 学会如何"持续学习": the ablation over k, b and the number
    of updated blocks): a 32768-token stream (the 128K stream's first 32K)
    for each (k, b) pair, one warm-up and two timed passes each."""
    T = args.seq or 32768
    rows = []
    for k in (4096, 8192, 16384):
        for b in (512, 1024, 2048):
            c = synth.config(args.workload, window=k, minibatch=b)
            w = synth.gen_weights(c, device="cuda")
            tok = synth.gen_tokens(c, n=T, device="cuda")
            m = tla.TTT(c, w, max_seq=T + 1024)
            loss = torch.empty(T - 1, dtype=torch.float32, device="cuda")
            m.reset()
            m.prefill(tok, loss)
            m.sync()
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            for _ in range(2):
                m.reset()
                m.prefill(tok, loss)
            e1.record()
            torch.cuda.synchronize()
            m.sync()
            ms = e0.elapsed_time(e1) / 2
            fl = algorithmic_flops(c, T)
            rows.append(dict(window=k, minibatch=b, ms=round(ms, 1), tokens_per_s=round(T / ms * 1e3, 1),
                             mfma_peak_frac=round(fl / (ms * 1e-3) / (PEAK_BF16_TFLOPS * 1e12), 4),
                             algorithmic_tflop=round(fl / 1e12, 1), mean_loss=round(float(loss.mean()), 4)))
            print(f"# k={k} b={b}: {ms:.1f} ms  {T / ms * 1e3:.0f} tok/s", file=sys.stderr, flush=True)
            m.close()
            del w, m
            torch.cuda.empty_cache()
    print(json.dumps(dict(metric="TTT prefill tokens/s over window k and mini-batch b, 3B shape, 1 MI355X",
                          config=dict(workload=f"{args.workload}-shape prefill, T={T}"), rows=rows)), flush=True)


def multi_seq(args, tla, torch, synth):
    """Throughput of the 3B-shape prefill with B independent sequences side
    by side (n_seq = B: the loop's products with frozen weights on B b rows,
    the fast-weight products batched): B streams of 32768 tokens each, one
    warm-up and two timed passes per B."""
    T = args.seq or 32768
    rows = []
    for B in (1, 2, 4, 8):
        c = synth.config(args.workload, n_seq=B)
        w = synth.gen_weights(c, device="cuda")
        tok = torch.stack([synth.gen_tokens(c, n=T, device="cuda", seed=c["seed"] + 100 * j) for j in range(B)])
        m = tla.TTT(c, w, max_seq=T + 1024)
        loss = torch.empty(B, T - 1, dtype=torch.float32, device="cuda")
        m.timing_enable((1 << 9) - 1)
        m.prefill(tok if B > 1 else tok[0], loss if B > 1 else loss[0])
        m.sync()
        classes = {x["kind"]: round(x["ms"], 1) for x in (m.timing_read(k) for k in range(9))}
        m.timing_enable(0)
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(2):
            m.reset()
            m.prefill(tok if B > 1 else tok[0], loss if B > 1 else loss[0])
        e1.record()
        torch.cuda.synchronize()
        m.sync()
        ms = e0.elapsed_time(e1) / 2
        fl = algorithmic_flops(c, T) * B
        rows.append(dict(n_seq=B, ms=round(ms, 1), tokens_per_s=round(B * T / ms * 1e3, 1),
                         mfma_peak_frac=round(fl / (ms * 1e-3) / (PEAK_BF16_TFLOPS * 1e12), 4),
                         algorithmic_tflop=round(fl / 1e12, 1), mean_loss=round(float(loss.mean()), 4),
                         warmup_class_ms=classes))
        print(f"# B={B}: {ms:.1f} ms  {B * T / ms * 1e3:.0f} tok/s", file=sys.stderr, flush=True)
        m.close()
        del w, m, tok, loss
        torch.cuda.empty_cache()
    print(json.dumps(dict(metric="TTT prefill tokens/s with B sequences side by side, 3B shape, 1 MI355X",
                          config=dict(workload=f"{args.workload}-shape prefill, T={T} per sequence, b=1024, "
                                               f"k=8192"), rows=rows)), flush=True)


def pmc_busy(c, T, d):
    """MFMA busy of the attention-forward launches of one step, from a rocprofv3
    --pmc SQ_VALU_MFMA_BUSY_CYCLES GRBM_GUI_ACTIVE SQ_BUSY_CYCLES SQ_INSTS_MFMA
    run of `bench.py --attn-replay`. SQ_VALU_MFMA_BUSY_CYCLES is summed over
    the chip's 1024 SIMDs; GRBM_GUI_ACTIVE over its 8 XCDs and SQ_BUSY_CYCLES
    over its 32 shader engines count the active cycles during each dispatch,
    so busy / (1024 x active per XCD) is the fraction of the kernel's time the
    matrix cores were busy, independent of the clock (both normalisations are
    printed as a cross-check). Launches are weighted as in --pmc-summary."""
    per = {}
    with open(os.path.join(d, "run_counter_collection.csv")) as fh:
        for r in csv.DictReader(fh):
            if "attn_fwd2_kernel" not in r["Kernel_Name"]:
                continue
            x = per.setdefault(int(r["Dispatch_Id"]), {})
            x[r["Counter_Name"]] = x.get(r["Counter_Name"], 0.0) + float(r["Counter_Value"])
    disp = [per[k] for k in sorted(per)]
    launches = attn_launches(c, T)
    assert len(disp) == len(launches), (len(disp), len(launches))
    def tot(name):
        return sum(wt * x.get(name, 0.0) for x, (*_, wt) in zip(disp, launches))
    busy, grbm, sq = tot("SQ_VALU_MFMA_BUSY_CYCLES"), tot("GRBM_GUI_ACTIVE"), tot("SQ_BUSY_CYCLES")
    print(json.dumps(dict(kernel="attn_fwd2_kernel", dispatches=len(disp), source_sha=roof_source_hash(),
                          mfma_busy_frac=round(busy / (1024 * grbm / 8), 4) if grbm else None,
                          mfma_busy_frac_by_se_cycles=round(busy / (1024 * sq / 32), 4) if sq else None)))


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=3)
    ap.add_argument("--warmup", type=int, default=1)
    ap.add_argument("--workload", default="3b", help="synth workload name (3b, 1b, 125m)")
    ap.add_argument("--seq", type=int, default=None, help="override the stream length")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--breakdown", action="store_true", help="print the per-class timing table")
    ap.add_argument("--copy-probe", action="store_true", help="1 GiB device copy for PMC scaling, then exit")
    ap.add_argument("--decode", action="store_true", help="measure decode latency instead of prefill throughput")
    ap.add_argument("--attn-replay", action="store_true", help="one step's attention-forward launches, then exit")
    ap.add_argument("--pmc-summary", nargs=4, metavar="DIR", help="bytes per attention launch from counter runs")
    ap.add_argument("--update-replay", action="store_true", help="two blocks' update launches, then exit")
    ap.add_argument("--pmc-update-summary", nargs=4, metavar="DIR",
                    help="bytes per update launch from counter runs of --update-replay and --copy-probe")
    ap.add_argument("--decode-steps", type=int, default=256)
    ap.add_argument("--sweep-kb", action="store_true", help="prefill throughput over window k and mini-batch b")
    ap.add_argument("--multi-seq", action="store_true",
                    help="prefill throughput with 1, 2, 4 and 8 sequences side by side")
    ap.add_argument("--decode-updates", action="store_true",
                    help="measure decode with test-time updates every mini-batch instead")
    ap.add_argument("--e2", action="store_true", help="measure the E2-TTT chunk-end kernel instead")
    ap.add_argument("--pmc-busy", metavar="DIR",
                    help="MFMA-busy fraction of the attention forward from a counter run of --attn-replay")
    args = ap.parse_args()

    if args.copy_probe:
        copy_probe()
        return
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py: the inner loop runs on one GPU only; --gpus N > 1 is not supported "
              "(one GPU's share of a sharded run is what this measures).", file=sys.stderr)
        sys.exit(2)

    import torch
    import synth
    import test_long_context_amd as tla

    if args.e2:
        e2_bench(args, tla, torch, synth)
        return
    if args.sweep_kb:
        kb_sweep(args, tla, torch, synth)
        return
    if args.multi_seq:
        multi_seq(args, tla, torch, synth)
        return
    c = synth.config(args.workload)
    T = args.seq or c["seq"]
    if args.pmc_summary:
        pmc_summary(c, T, args.pmc_summary, args.workload)
        return
    if args.pmc_update_summary:
        pmc_update_summary(c, args.pmc_update_summary, args.workload)
        return
    if args.update_replay:
        update_replay(c, tla, torch)
        return
    if args.pmc_busy:
        pmc_busy(c, T, args.pmc_busy)
        return
    if args.attn_replay:
        attn_replay(c, T, tla, torch)
        return
    torch.cuda.set_device(0)
    t_setup = time.perf_counter()
    w = synth.gen_weights(c, device="cuda")
    if args.decode_updates:
        tok = synth.gen_tokens(c, n=8193 + 2 * c["minibatch"] + 1, device="cuda")
        decode_update_bench(args, c, w, tok, tla, torch)
        return
    if args.decode:
        tok = synth.gen_tokens(c, n=T + args.decode_steps, device="cuda")
        decode_bench(args, c, w, tok, tla, torch)
        return
    tok = synth.gen_tokens(c, n=T, device="cuda")
    m = tla.TTT(c, w, max_seq=T + 1024)
    loss = torch.empty(T - 1, dtype=torch.float32, device="cuda")
    torch.cuda.synchronize()
    t_setup = time.perf_counter() - t_setup
    print(f"# setup {t_setup:.1f} s (weights generated on the GPU, context built)", file=sys.stderr, flush=True)

    # warm-up; the last warm-up step records every kernel class
    for i in range(max(1, args.warmup)):
        if i == max(1, args.warmup) - 1:
            m.timing_enable((1 << 9) - 1)
        m.reset()
        m.prefill(tok, loss)
        m.sync()
        print(f"# warm-up step {i} done", file=sys.stderr, flush=True)
    classes = [m.timing_read(k) for k in range(9)]
    if args.breakdown:
        tot = sum(x["ms"] for x in classes)
        for x in classes:
            eff = x["flops"] / (x["ms"] * 1e9) if x["ms"] > 0 and x["flops"] else 0.0
            bw = x["bytes"] / (x["ms"] * 1e6) if x["ms"] > 0 and x["bytes"] else 0.0
            print(f"# {x['kind']:12s} {x['ms']:9.2f} ms {100 * x['ms'] / tot:5.1f}%  launches {x['launches']:6d}"
                  f"  {eff:8.1f} TFLOP/s  {bw:8.1f} GB/s", file=sys.stderr)

    # timed steps: events around the launches of the update products (the
    # roofline kernel), the cross-entropy and the attention forward
    mask = 0
    for k in TIMED_CLASSES:
        mask |= 1 << KC[k]
    m.timing_enable(mask)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(args.steps):
        m.reset()
        m.prefill(tok, loss)
    e1.record()
    torch.cuda.synchronize()
    m.sync()
    ms = e0.elapsed_time(e1) / args.steps
    live = {k: m.timing_read(KC[k]) for k in TIMED_CLASSES}
    m.timing_enable(0)
    assert bool(torch.isfinite(loss).all()), "non-finite loss"
    mean_loss = float(loss.mean())

    flops = algorithmic_flops(c, T)
    tps = T / (ms / 1e3)
    frac = flops / (ms / 1e3) / (PEAK_BF16_TFLOPS * 1e12)

    def rate(x, what):
        """Average launch duration and the algorithmic rate per launch."""
        n = max(1, x["launches"])
        avg_s = x["ms"] / n * 1e-3
        if what == "bytes":
            return avg_s, x["bytes"] / n / avg_s / 1e9 if avg_s > 0 else 0.0
        return avg_s, x["flops"] / n / avg_s / 1e12 if avg_s > 0 else 0.0

    upd = live[ROOF_CLASS]
    u_avg, u_gbs = rate(upd, "bytes")
    nu = max(1, upd["launches"])
    utr = UPD_TRAFFIC.get((args.workload, roof_source_hash(UPD_SOURCES)))
    roof = dict(bound="hbm", achieved=round(u_gbs, 1), peak=PEAK_HBM_GBS, unit="GB/s",
                frac=round(u_gbs / PEAK_HBM_GBS, 4), traffic=None if utr is None else utr,
                kernel="fused dW = X^T dH product with the fp32 SGD update of the fast weights in its epilogue "
                       "(gemm_bf16_kernel, SGD epilogue)",
                algorithmic_bytes_per_launch=round(upd["bytes"] / nu),
                algorithmic_unit="10 bytes per fast-weight parameter: fp32 master read + write, bf16 working copy",
                launches_per_step=upd["launches"] // args.steps, avg_launch_us=round(u_avg * 1e6, 2),
                mfma_tflops=round(upd["flops"] / nu / u_avg / 1e12, 1) if u_avg > 0 else None,
                share_of_step=round(upd["ms"] / args.steps / ms, 4),
                traffic_unit="HBM bytes per launch (rocprofv3 FETCH_SIZE + WRITE_SIZE of --update-replay, "
                             "copy-scaled), averaged over a block's dW3 and dW12 launches",
                note="durations measured on the update's side streams, beside the main stream's kernels")
    if c["dtype"] == "bf16" and c["n_dynamic"] > 0:
        iso = update_isolated_us(c, tla, torch)
        iso_gbs = upd["bytes"] / nu / (iso * 1e-6) / 1e9
        roof.update(isolated_avg_launch_us=round(iso, 2), isolated_gbs=round(iso_gbs, 1),
                    isolated_frac=round(iso_gbs / PEAK_HBM_GBS, 4),
                    isolated_note="the same launches replayed alone on the GPU after the timed region")
    ce = live["ce"]
    c_avg, c_gbs = rate(ce, "bytes")
    attn = {k: sum(live[a][k] for a in ATTN_CLASSES) for k in ("ms", "launches", "flops", "bytes")}
    a_avg, a_tfs = rate(attn, "flops")
    src = roof_source_hash()
    tr = TRAFFIC.get((args.workload, T, src))
    kernels = dict(
        update=dict(bound="hbm", gbs=round(u_gbs, 1), frac=roof["frac"], avg_launch_us=roof["avg_launch_us"],
                    launches_per_step=roof["launches_per_step"]),
        cross_entropy=dict(bound="hbm", gbs=round(c_gbs, 1), frac=round(c_gbs / PEAK_HBM_GBS, 4),
                           avg_launch_us=round(c_avg * 1e6, 2), launches_per_step=ce["launches"] // args.steps,
                           algorithmic_unit="6 bytes per logit: fp32 logit read, bf16 gradient write"),
        attention_forward=dict(bound="mfma", tflops=round(a_tfs, 1), frac=round(a_tfs / PEAK_BF16_TFLOPS, 4),
                               avg_launch_us=round(a_avg * 1e6, 2),
                               launches_per_step=attn["launches"] // args.steps,
                               traffic=None if tr is None else tr["traffic_bytes_per_launch"],
                               mfma_busy_frac=MFMA_BUSY.get((args.workload, T, src)), source_sha=src))

    out = dict(metric=METRIC, value=round(tps, 1), unit="tokens/s", n_gpus=1, steps=args.steps,
               warmup=args.warmup, ms_per_step=round(ms, 2), higher_is_better=True, scaling="weak",
               vs_baseline=None, dtype="bf16" if c["dtype"] == "bf16" else "f32", data="synthetic",
               config=dict(workload=f"{args.workload}-shape TTT-E2E prefill, T={T}, b={c['minibatch']}, "
                                    f"k={c['window']}, alpha={c['alpha']}, Zipf(1.1) ids",
                           seq_len=T, minibatch=c["minibatch"], window=c["window"]),
               mfma_peak_frac=round(frac, 4), algorithmic_tflop=round(flops / 1e12, 1),
               ce_gbs=round(c_gbs, 1), update_gbs=round(u_gbs, 1),
               mean_loss=round(mean_loss, 4), roofline=roof, kernels=kernels,
               breakdown_warmup={x["kind"]: dict(ms=round(x["ms"], 2), launches=x["launches"],
                                                 tflops=round(x["flops"] / (x["ms"] * 1e9), 1) if x["ms"] > 0 and x["flops"] else None,
                                                 gbs=round(x["bytes"] / (x["ms"] * 1e6), 1) if x["ms"] > 0 and x["bytes"] else None)
                                 for x in classes})
    del m
    if not args.no_cpu_baseline:
        torch.cuda.synchronize()
        out["cpu_baseline"] = cpu_baseline(c, w, tok)
    else:
        out["cpu_baseline"] = None
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
