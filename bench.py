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
the dominant kernel -- the sliding-window attention forward (one kernel
symbol, launched by the hoisted prefix and by every mini-batch), timed with
HIP events on its launch stream during the timed steps -- and the CPU oracle
timed on a bounded sample of the same workload.

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
ROOF_CLASSES = ("attn_prefix", "attn_loop")   # the attention forward kernel
ROOF_SOURCES = ("test_long_context_amd/csrc/attn2.hip", "test_long_context_amd/csrc/common.hpp")

# HBM traffic of the attention forward from rocprofv3 --pmc FETCH_SIZE /
# WRITE_SIZE (--attn-replay, scaled by the --copy-probe counters; printed by
# --pmc-summary), keyed by (workload, T, source hash): valid only for the
# kernel source the counters were taken on.
TRAFFIC = {
    ("3b", 131072, "218a5e2b4cdd808d"): dict(fetch_bytes_per_launch=56619038, write_bytes_per_launch=60356339,
                                             fetch_scale=1.9999, write_scale=1.0,
                                             traffic_bytes_per_launch=173590785),
}


# MFMA busy of the same kernel (rocprofv3 SQ_VALU_MFMA_BUSY_CYCLES over the
# SIMDs x active cycles, --pmc-busy), keyed like TRAFFIC.
MFMA_BUSY = {
    ("3b", 131072, "218a5e2b4cdd808d"): 0.4277,
}


def roof_source_hash() -> str:
    h = hashlib.sha256()
    for f in ROOF_SOURCES:
        with open(os.path.join(ROOT, f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


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


def cpu_baseline(c, w, tok, ntok):
    """The oracle (float32 numpy) on the first mini-batch of the same stream."""
    import numpy as np
    from oracle import ttt_e2e as O
    cores = _host_threads()
    wn = _oracle_weights(w)
    t = tok[: ntok + 1].cpu().numpy()
    t0 = time.perf_counter()
    out = O.ttt_inner_loop(c, wn, t, dtype=np.float32)
    dt = time.perf_counter() - t0
    assert np.all(np.isfinite(out["loss"]))
    return dict(value=round(ntok / dt, 2), unit="tokens/s", cores=int(cores), kind="oracle",
                sample=f"mini-batch 0 of the same stream: {ntok} positions forward + 1 SGD step, "
                       f"plus the forward-only position {ntok}; {dt:.1f} s on the host",
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
    (static bf16, dynamic fp32 masters, lm_head) and the window's keys and
    values in every block."""
    L, d, H, Hk, dh = c["n_layers"], c["d_model"], c["n_heads"], c["n_kv_heads"], c["head_dim"]
    F, Fd, V, k = c["ffn_hidden"], c["dyn_ffn_hidden"], c["vocab"], c["window"]
    Ld = c["n_dynamic"] or L - (3 * L) // 4
    es = 2 if c["dtype"] == "bf16" else 4
    static = L * ((H + 2 * Hk) * dh * d + d * H * dh + 3 * F * d) * es + V * d * es
    dyn = Ld * 3 * Fd * d * 4
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
    ap.add_argument("--decode-steps", type=int, default=256)
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
    c = synth.config(args.workload)
    T = args.seq or c["seq"]
    if args.pmc_summary:
        pmc_summary(c, T, args.pmc_summary, args.workload)
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

    # timed steps: events only around the attention forward launches
    mask = 0
    for k in ROOF_CLASSES:
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
    parts = [m.timing_read(KC[k]) for k in ROOF_CLASSES]
    m.timing_enable(0)
    assert bool(torch.isfinite(loss).all()), "non-finite loss"
    mean_loss = float(loss.mean())

    flops = algorithmic_flops(c, T)
    tps = T / (ms / 1e3)
    frac = flops / (ms / 1e3) / (PEAK_BF16_TFLOPS * 1e12)
    r_ms = sum(x["ms"] for x in parts)
    r_fl = sum(x["flops"] for x in parts)
    r_n = sum(x["launches"] for x in parts)
    avg_s = r_ms / r_n * 1e-3
    ach = r_fl / r_n / avg_s / 1e12
    src = roof_source_hash()
    tr = TRAFFIC.get((args.workload, T, src))
    traffic = None if tr is None else tr["traffic_bytes_per_launch"]
    busy = MFMA_BUSY.get((args.workload, T, src))
    roof = dict(bound="mfma", achieved=round(ach, 1), peak=PEAK_BF16_TFLOPS, unit="TFLOP/s",
                frac=round(ach / PEAK_BF16_TFLOPS, 4), traffic=traffic,
                kernel=f"attn_fwd2_kernel (sliding-window attention forward, head_dim {c['head_dim']})",
                traffic_unit="bytes per launch (rocprofv3 FETCH_SIZE + WRITE_SIZE, copy-scaled)",
                launches_per_step=r_n // args.steps, avg_launch_us=round(avg_s * 1e6, 2),
                algorithmic_gflop_per_launch=round(r_fl / r_n / 1e9, 3),
                share_of_step=round(r_ms / args.steps / ms, 4), source_sha=src,
                mfma_busy_frac=busy)

    out = dict(metric=METRIC, value=round(tps, 1), unit="tokens/s", n_gpus=1, steps=args.steps,
               warmup=args.warmup, ms_per_step=round(ms, 2), higher_is_better=True, scaling="weak",
               vs_baseline=None, dtype="bf16" if c["dtype"] == "bf16" else "f32", data="synthetic",
               config=dict(workload=f"{args.workload}-shape TTT-E2E prefill, T={T}, b={c['minibatch']}, "
                                    f"k={c['window']}, alpha={c['alpha']}, Zipf(1.1) ids",
                           seq_len=T, minibatch=c["minibatch"], window=c["window"]),
               mfma_peak_frac=round(frac, 4), algorithmic_tflop=round(flops / 1e12, 1),
               mean_loss=round(mean_loss, 4), roofline=roof)
    del m
    if not args.no_cpu_baseline:
        torch.cuda.synchronize()
        out["cpu_baseline"] = cpu_baseline(c, w, tok, min(c["minibatch"], T - 1))
    else:
        out["cpu_baseline"] = None
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
