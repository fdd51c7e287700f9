#!/usr/bin/env python3
"""KLA prefill + decode benchmark on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W]

One timed step is one kla_fwd_chunked call over the layer-shaped workload
(8 sequences x 2048 tokens, 16 heads, dk = dv = 128, chunk 64, bf16 q/k/v,
fp32 gates, fp32 o and final state), inputs already resident in HBM.  The
headline value is prefill tokens/s.  The same JSON line also carries the
decode step (256 sequences x 16 heads, 128 steps, fp32 state updated in
place) as state GB/s, each kernel's roofline fraction from HIP events on the
launch stream, and the fp64 reference timed on the host cores.

Algorithmic work counted per token-head (d = 128, C = 64):
  prefill bytes  q,k,v bf16 3*256 + alpha,eta 2*4 + o fp32 512 = 1288 B,
                 plus the final state (d*d*4 B) once per (sequence, head)
  prefill flops  full 16x16-tile MFMA count of the chunk algorithm in its
                 W/U form: K K^T, Q K^T, T V, T Diag(g) K, M Delta: 2*C*d
                 each; Q S, W S, K^T Delta: 2*d*d each -> 10*C*d + 6*d*d =
                 180,224 (`mfma_frac`); the kernel's regrouped form forms no
                 W: 8*C*d + 6*d*d = 163,840 (`mfma_frac_regrouped`)
  packed         (`packed` object) the packed variable-length workload (64
                 sequences of 128..8192 tokens, cu_seqlens): bytes and flops
                 as the prefill over its token-heads
  decode bytes   the fp32 state read and written once: 2*d*d*4 per (seq, head)
  backward       (`backward` object) the gradients of the layer-shaped
                 prefill: reads q, k, v bf16, alpha, eta, d_o fp32, writes
                 dq, dk, dv, dalpha, deta fp32: 2832 B per token-head; full-
                 tile flops of the chunk form 20*C*d + 20*d*d = 491,520 per
                 token-head; priced against the bf16 MFMA peak (the dq/dk,
                 state-gradient and K S / Q S products run there with hi/lo
                 splits), with the fraction of the fp32 MFMA peak beside it
  gate_variants  the layer prefill with the direct step (Gated DeltaNet) and
                 without decay (DeltaNet), same kernel
  ccq            the curvature-conditioned read: layer prefill (query-
                 cleaning pass + one bf16 prefill reading both planes of the
                 cleaned query; algorithmic bytes as the prefill plus lambda
                 and the per-(sequence, head) sums) and the decode step
                 (state and running sums read and written once)
  per-channel decay (Kimi Delta Attention gate, `kda` object): the same
                 work with alpha fp32 [.., dk]: 1288 - 4 + 4*d = 1796 B per
                 token-head; with bf16 inputs its prefill's contractions run
                 on the bf16 MFMA (fp32 factors split hi/lo), so `mfma_frac`
                 is against the bf16 peak

Clock.  The GPU needs some tens of milliseconds of sustained work to reach
its steady clock.  Every leg first runs its own launch back to back for at
least --settle-ms of wall time (reported as `clock_settle_ms`), then the
--warmup counted warm-up launches, then its timed launches.

Oracle timings.  The fp64 oracle is timed on the host threads beside the
layer prefill (`cpu_baseline`) and beside the long-context, packed and
decode workloads (`oracle` inside those objects, one run each).
"""
import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0        # MI355X HBM3E
BF16_MFMA_PEAK_TF = 2500.0   # MI355X dense bf16 MFMA, TFLOP/s
FP32_MFMA_PEAK_TF = 157.3    # MI355X dense fp32 MFMA, TFLOP/s

PREFILL_KERNEL = "prefill_pc_kernel"  # the bf16 prefill kernel (producer/consumer waves)
DECODE_KERNEL = "decode_kernel"
KDA_KERNEL = "prefill_kda_bf_kernel"   # per-channel decay prefill (bf16 inputs)
BWD_KERNEL = "bwd_kernel"              # backward: the two-sweep kernel
BWD_FINISH = "bwd_finish_kernel"       # backward: the sum over column slices
BWD_STATES = "prefill_pc_kernel_states"  # backward (bf16): chunk-start states, no output
KERNEL_SOURCES = {PREFILL_KERNEL: "delta_rule_linear_amd/csrc/kla_prefill.hip",
                  DECODE_KERNEL: "delta_rule_linear_amd/csrc/kla_decode.hip",
                  KDA_KERNEL: "delta_rule_linear_amd/csrc/kla_kda.hip",
                  BWD_KERNEL: "delta_rule_linear_amd/csrc/kla_bwd.hip",
                  BWD_FINISH: "delta_rule_linear_amd/csrc/kla_bwd.hip",
                  BWD_STATES: "delta_rule_linear_amd/csrc/kla_prefill.hip"}
# mangled-name fragments of the instantiations the benchmark times (bf16
# inputs, d = 128; the decode one with the scalar decay)
# (prefill_pc_kernel<D, OUT, QLO>: the plain prefill is <128, true, false>)
KERNEL_MATCH = {PREFILL_KERNEL: "prefill_pc_kernelILi128ELb1ELb0E",
                DECODE_KERNEL: "decode_kernelIDF16bLi128ELb0E",
                KDA_KERNEL: "prefill_kda_bf_kernelILi128E",
                BWD_KERNEL: "bwd_kernelIDF16bLi128E",
                BWD_FINISH: "bwd_finish_kernelIDF16bLi128E",
                BWD_STATES: "prefill_pc_kernelILi128ELb0ELb0E"}
TRAFFIC_JSON = os.path.join(ROOT, "profiles", "hbm_traffic.json")


SHARED_HEADER = "delta_rule_linear_amd/csrc/kla_device.h"  # device helpers of the prefill kernels


def source_hash(kernel):
    """sha256 of the kernel's source file (followed by the shared device
    header for the prefill kernels, which include it, and by the unit's own
    extra build flags where it has any)."""
    import hashlib
    from delta_rule_linear_amd import build as kbuild
    h = hashlib.sha256()
    paths = [KERNEL_SOURCES[kernel]] + ([SHARED_HEADER] if kernel != DECODE_KERNEL else [])
    for p in paths:
        with open(os.path.join(ROOT, p), "rb") as f:
            h.update(f.read())
    extra = kbuild.EXTRA.get(os.path.basename(KERNEL_SOURCES[kernel]))
    if extra:
        h.update(" ".join(extra).encode())
    return h.hexdigest()


def measured_traffic(kernel):
    """HBM bytes per launch from the committed rocprofv3 counter summary, or
    None when the kernel source changed since the counters were taken."""
    try:
        with open(TRAFFIC_JSON) as f:
            rec = json.load(f)[kernel]
    except (OSError, KeyError, ValueError):
        return None
    if rec.get("source_sha256") != source_hash(kernel):
        return None
    return rec["bytes_per_launch"]


def ingest_counters(fetch_csv, write_csv, cal_fetch_csv, cal_write_csv):
    """Turn rocprofv3 FETCH_SIZE / WRITE_SIZE runs (KiB per dispatch) into
    bytes per launch, scaled by what the same counters read for a plain
    1 GiB device copy (bench.py --calibrate-copy), and record them with the
    kernel source hash in profiles/hbm_traffic.json (kernels absent from the
    runs keep their earlier records)."""
    import csv
    from collections import defaultdict

    def per_kernel(path, counter):
        acc = defaultdict(list)
        for r in csv.DictReader(open(path)):
            if r["Counter_Name"] == counter:
                acc[r["Kernel_Name"]].append(float(r["Counter_Value"]))
        return {k: sum(v) / len(v) for k, v in acc.items()}

    def copy_kib(path, counter):
        vals = [v for k, v in per_kernel(path, counter).items() if "copyBuffer" in k]
        return vals[0]

    gib_kib = float(1 << 20)  # the calibration copy reads and writes 1 GiB
    f_scale = gib_kib / copy_kib(cal_fetch_csv, "FETCH_SIZE")
    w_scale = gib_kib / copy_kib(cal_write_csv, "WRITE_SIZE")
    fetch = per_kernel(fetch_csv, "FETCH_SIZE")
    write = per_kernel(write_csv, "WRITE_SIZE")
    try:
        with open(TRAFFIC_JSON) as f:
            out = json.load(f)
    except (OSError, ValueError):
        out = {}
    for kernel in KERNEL_SOURCES:
        fk = [v for k, v in fetch.items() if KERNEL_MATCH[kernel] in k and
              (kernel != BWD_KERNEL or "finish" not in k)]
        wk = [v for k, v in write.items() if KERNEL_MATCH[kernel] in k and
              (kernel != BWD_KERNEL or "finish" not in k)]
        if not fk or not wk:
            continue
        rb, wb = fk[0] * f_scale * 1024, wk[0] * w_scale * 1024
        out[kernel] = {"source_sha256": source_hash(kernel), "fetch_kib_raw": fk[0],
                       "write_kib_raw": wk[0], "fetch_scale": round(f_scale, 5),
                       "write_scale": round(w_scale, 5), "read_bytes": round(rb),
                       "write_bytes": round(wb), "bytes_per_launch": round(rb + wb)}
    os.makedirs(os.path.dirname(TRAFFIC_JSON), exist_ok=True)
    with open(TRAFFIC_JSON, "w") as f:
        json.dump(out, f, indent=1)
        f.write("\n")
    print(json.dumps(out, indent=1))


def prefill_work(token_heads, n_seqs, H, d, C=64):
    """Algorithmic bytes and flops of one prefill launch over `token_heads`
    token-heads in n_seqs sequences.  Flops are full-tile counts: the W/U
    form of the chunk algorithm, 10Cd + 6d^2 per token-head (K K^T, Q K^T,
    T V, T Diag(g) K, M Delta at 2Cd each; Q S, W S, K^T Delta at 2d^2
    each), and this kernel's regrouped form, 8Cd + 6d^2 (no W)."""
    bytes_ = token_heads * (3 * d * 2 + 2 * 4 + d * 4) + n_seqs * H * d * d * 4
    flops = token_heads * (10 * C * d + 6 * d * d)
    flops_impl = token_heads * (8 * C * d + 6 * d * d)
    return bytes_, flops, flops_impl


def settle(fn, min_ms):
    """Run fn back to back for at least min_ms of wall time (synchronising
    every 16 launches), so the GPU reaches its steady clock before the
    counted warm-ups and the timed launches.  Returns the wall ms spent."""
    import torch
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    while True:
        for _ in range(16):
            fn()
        torch.cuda.synchronize()
        ms = (time.perf_counter() - t0) * 1e3
        if ms >= min_ms:
            return ms


def warm(fn, args):
    """The clock-settle phase, then args.warmup counted warm-up launches."""
    ms = settle(fn, args.settle_ms)
    for _ in range(args.warmup):
        fn()
    return ms


def time_launches(fn, n, stream):
    """Run fn n times back to back on `stream`, with one pair of HIP events
    around the whole run on that stream.  Returns (wall seconds for the n
    launches, event ms per launch).  One launch is one kernel, so the event
    figure is the kernel's average launch duration (the launches queue up
    faster than they run, so no host gaps fall between them)."""
    import torch
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    a.record(stream)
    for _ in range(n):
        fn()
    b.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    return wall, a.elapsed_time(b) / n


def bench_prefill(args, torch, kla, workloads):
    inp = workloads.prefill("layer")
    B, H, d = inp["n_seqs"], inp["H"], inp["d"]
    T = inp["lengths"][0]
    dev = "cuda:0"
    q = inp["q"].to(dev).view(B, T, H, d)
    k = inp["k"].to(dev).view(B, T, H, d)
    v = inp["v"].to(dev).view(B, T, H, d)
    a = inp["alpha"].to(dev).view(B, T, H)
    e = inp["eta"].to(dev).view(B, T, H)
    o = torch.empty((B, T, H, d), dtype=torch.float32, device=dev)
    S = torch.empty((B, H, d, d), dtype=torch.float32, device=dev)
    stream = torch.cuda.current_stream()

    def step():
        kla.kla_fwd_chunked(q, k, v, a, e, eps=inp["eps"], o=o, final_state=S)

    settle_ms = warm(step, args)
    wall, ev_ms = time_launches(step, args.steps, stream)
    nbytes, flops, flops_impl = prefill_work(B * T * H, B, H, d)
    return dict(inp=inp, tokens=B * T, wall=wall, ev_ms=ev_ms, bytes=nbytes, flops=flops,
                flops_impl=flops_impl, shape=(B, T, H, d), settle_ms=settle_ms)


def bench_decode(args, torch, kla, workloads):
    wl = workloads.decode(steps=args.decode_steps)
    dev = "cuda:0"
    N, H, d = wl["n_seqs"], wl["H"], wl["d"]
    state = wl["state"].to(dev)
    steps = [{n: st[n].to(dev) for n in ("q", "k", "v", "alpha", "eta")} for st in wl["steps"]]
    o = torch.empty((N, H, d), dtype=torch.float32, device=dev)
    stream = torch.cuda.current_stream()
    # settle and warm up on a scratch copy so the timed run starts from the drawn state
    scratch = state.clone()
    wi = iter(range(1 << 30))

    def on_scratch():
        st = steps[next(wi) % len(steps)]
        kla.kla_decode_step(st["q"], st["k"], st["v"], st["alpha"], st["eta"], scratch,
                            eps=wl["eps"], o=o)

    settle_ms = warm(on_scratch, args)
    del scratch
    it = iter(range(len(steps)))

    def one():
        st = steps[next(it) % len(steps)]
        kla.kla_decode_step(st["q"], st["k"], st["v"], st["alpha"], st["eta"], state,
                            eps=wl["eps"], o=o)

    wall, ev_ms = time_launches(one, len(steps), stream)
    state_bytes = 2 * N * H * d * d * 4
    # Successive steps on one 268 MB state let the GPU's 256 MB last-level
    # cache serve part of it.  The same step after a read sweep over 1 GiB
    # (which leaves none of the state cached): (sweep + step) - sweep.
    sweep = torch.ones(1 << 28, dtype=torch.float32, device=dev)
    red = torch.empty((), dtype=torch.float32, device=dev)
    n_sw, reps = 8, 5
    it = iter(range(2 * n_sw * (reps + 1)))
    both_fn = lambda: (torch.amax(sweep, dim=0, out=red), one())
    sweep_fn = lambda: torch.amax(sweep, dim=0, out=red)
    for _ in range(n_sw):  # warm-up: the reduction's first calls set up its workspace
        both_fn()
        sweep_fn()
    diffs = sorted(time_launches(both_fn, n_sw, stream)[1] - time_launches(sweep_fn, n_sw, stream)[1]
                   for _ in range(reps))
    del sweep
    return dict(N=N, H=H, d=d, steps=len(steps), wall=wall, ev_ms=ev_ms, state_bytes=state_bytes,
                swept_ms=diffs[reps // 2], settle_ms=settle_ms, wl=wl)


def bench_long(args, torch, kla, workloads, n_splits=3, launches=20):
    """Long-context prefill (2 sequences x 32768 tokens, 16 heads, d=128):
    one pass against the split-sequence path.  With 32 (sequence, head)
    pairs the one-pass kernel fills 64 of the 256 compute units; three
    segments fill all of them in the segment-map pass (32 x 2 x 4
    workgroups).  Each variant: 3 warm-up launches, then `launches` back to
    back between one event pair."""
    inp = workloads.prefill("long")
    B, H, d = inp["n_seqs"], inp["H"], inp["d"]
    T = inp["lengths"][0]
    dev = "cuda:0"
    q, k, v = (inp[n].to(dev).view(B, T, H, d) for n in ("q", "k", "v"))
    a, e = (inp[n].to(dev).view(B, T, H) for n in ("alpha", "eta"))
    o = torch.empty((B, T, H, d), dtype=torch.float32, device=dev)
    S = torch.empty((B, H, d, d), dtype=torch.float32, device=dev)
    ws = torch.empty(kla.kla_fwd_chunked_split_workspace_size(B, H, d, d, n_splits),
                     dtype=torch.uint8, device=dev)
    stream = torch.cuda.current_stream()

    def one():
        kla.kla_fwd_chunked(q, k, v, a, e, eps=inp["eps"], o=o, final_state=S)

    def split():
        kla.kla_fwd_chunked_split(q, k, v, a, e, eps=inp["eps"], n_splits=n_splits, o=o,
                                  final_state=S, workspace=ws)

    res, settled = {}, {}
    for name, fn in (("one_pass", one), ("split", split)):
        settled[name] = warm(fn, args)
        _, ev_ms = time_launches(fn, launches, stream)
        res[name] = ev_ms * 1e3
    tok = B * T
    nbytes, flops, _ = prefill_work(tok * H, B, H, d)
    best = min(res.values())
    gbs = nbytes / (best * 1e-6) / 1e9
    del q, k, v, a, e, o, S, ws
    out = {"workload": f"long-context KLA prefill: {B} sequences x {T} tokens, H={H}, "
                       f"dk=dv={d}, bf16 q/k/v (dense batch)",
           "n_splits": n_splits,
           "us_one_pass": round(res["one_pass"], 1), "us_split": round(res["split"], 1),
           "tokens_per_s_one_pass": round(tok / (res["one_pass"] * 1e-6), 1),
           "tokens_per_s_split": round(tok / (res["split"] * 1e-6), 1),
           "speedup": round(res["one_pass"] / res["split"], 3),
           "roofline_best": {"bound": "hbm", "achieved": round(gbs, 1), "peak": HBM_PEAK_GBS,
                             "unit": "GB/s", "frac": round(gbs / HBM_PEAK_GBS, 4),
                             "algorithmic_bytes_per_launch": nbytes,
                             "mfma_frac": round(flops / (best * 1e-6) / 1e12 / BF16_MFMA_PEAK_TF, 4)},
           "clock_settle_ms": {k2: round(v2, 1) for k2, v2 in settled.items()}}
    if not args.skip_cpu_baseline:
        out["oracle"] = time_oracle(inp, tok)
    return out


def bench_kda(args, torch, kla, workloads, launches=50):
    """Per-channel decay (one rate per key channel): the layer-shaped prefill
    with alpha [B, T, H, dk] and the decode workload with alpha [N, H, dk]."""
    inp = workloads.prefill("layer", channel_decay=True)
    B, H, d = inp["n_seqs"], inp["H"], inp["d"]
    T = inp["lengths"][0]
    dev = "cuda:0"
    q, k, v = (inp[n].to(dev).view(B, T, H, d) for n in ("q", "k", "v"))
    a = inp["alpha_ch"].to(dev).view(B, T, H, d)
    e = inp["eta"].to(dev).view(B, T, H)
    o = torch.empty((B, T, H, d), dtype=torch.float32, device=dev)
    S = torch.empty((B, H, d, d), dtype=torch.float32, device=dev)
    stream = torch.cuda.current_stream()

    def step():
        kla.kla_fwd_chunked_kda(q, k, v, a, e, eps=inp["eps"], o=o, final_state=S)

    settle_ms = warm(step, args)
    _, ev_ms = time_launches(step, launches, stream)
    th = B * T * H
    nbytes = th * (3 * d * 2 + 4 * d + 4 + d * 4) + B * H * d * d * 4
    flops = th * (10 * 64 * d + 6 * d * d)
    gbs = nbytes / (ev_ms * 1e-3) / 1e9
    tf = flops / (ev_ms * 1e-3) / 1e12
    del q, k, v, a, e, o, S, inp
    out = {"workload": f"per-channel decay prefill: {B} sequences x {T} tokens, H={H}, dk=dv={d}, "
                       f"bf16 q/k/v, fp32 alpha [.., dk], eta, o, final state",
           "prefill_us": round(ev_ms * 1e3, 2),
           "prefill_tokens_per_s": round(B * T / (ev_ms * 1e-3), 1),
           "roofline": {"bound": "hbm", "achieved": round(gbs, 1), "peak": HBM_PEAK_GBS,
                        "unit": "GB/s", "frac": round(gbs / HBM_PEAK_GBS, 4),
                        "traffic": measured_traffic(KDA_KERNEL), "kernel": KDA_KERNEL, "avg_launch_us": round(ev_ms * 1e3, 2),
                        "algorithmic_bytes_per_launch": nbytes,
                        "mfma_tflops": round(tf, 2),
                        "mfma_frac": round(tf / BF16_MFMA_PEAK_TF, 4),
                        "mfma_peak": BF16_MFMA_PEAK_TF,
                        "algorithmic_flops_per_launch": flops,
                        "flops_convention": "full-tile 10Cd+6d^2 = 180,224 per token-head"},
           "clock_settle_ms": round(settle_ms, 1)}
    if not args.skip_decode:
        wl = workloads.decode(steps=args.decode_steps, channel_decay=True)
        N = wl["n_seqs"]
        state = wl["state"].to(dev)
        steps = [{n: st[n].to(dev) for n in ("q", "k", "v", "alpha_ch", "eta")} for st in wl["steps"]]
        od = torch.empty((N, H, d), dtype=torch.float32, device=dev)
        scratch = state.clone()
        wi = iter(range(1 << 30))

        def on_scratch():
            st = steps[next(wi) % len(steps)]
            kla.kla_decode_step_kda(st["q"], st["k"], st["v"], st["alpha_ch"], st["eta"], scratch,
                                    eps=wl["eps"], o=od)

        warm(on_scratch, args)
        del scratch
        it = iter(range(len(steps)))

        def one():
            st = steps[next(it)]
            kla.kla_decode_step_kda(st["q"], st["k"], st["v"], st["alpha_ch"], st["eta"], state,
                                    eps=wl["eps"], o=od)

        _, dms = time_launches(one, len(steps), stream)
        dgbs = 2 * N * H * d * d * 4 / (dms * 1e-3) / 1e9
        out["decode_us_per_step"] = round(dms * 1e3, 2)
        out["decode_state_gbs"] = round(dgbs, 1)
        out["decode_frac"] = round(dgbs / HBM_PEAK_GBS, 4)
    return out


def bench_bwd(args, torch, kla, workloads, launches=10):
    """Backward of the layer-shaped prefill (kla_bwd_chunked): gradients of
    q, k, v, alpha, eta and the start state from seeded d_o and d_final.
    One call is three launches (the states-only prefill that writes the
    chunk-start states, the reverse-sweep kernel and the reduction over
    column slices); the events bracket whole calls."""
    inp = workloads.prefill("layer")
    B, H, d = inp["n_seqs"], inp["H"], inp["d"]
    T = inp["lengths"][0]
    dev = "cuda:0"
    g = workloads.grad_inputs(5, B * T, H, d, B)
    q, k, v = (inp[n].to(dev).view(B, T, H, d) for n in ("q", "k", "v"))
    a, e = (inp[n].to(dev).view(B, T, H) for n in ("alpha", "eta"))
    do = g["d_o"].to(dev).view(B, T, H, d)
    dfin = g["d_final"].to(dev)
    ws = torch.empty(kla.kla_bwd_chunked_workspace_size(B, B * T, H, d, d), dtype=torch.uint8,
                     device=dev)
    stream = torch.cuda.current_stream()

    def step():
        kla.kla_bwd_chunked(q, k, v, a, e, do, d_final=dfin, eps=inp["eps"], workspace=ws)

    settle_ms = warm(step, args)
    _, ev_ms = time_launches(step, launches, stream)
    th = B * T * H
    nbytes = th * (3 * d * 2 + 2 * 4 + d * 4 + 3 * d * 4 + 2 * 4) + 2 * B * H * d * d * 4
    flops = th * (20 * 64 * d + 20 * d * d)
    tf = flops / (ev_ms * 1e-3) / 1e12
    ws_bytes = ws.numel()
    parts = [measured_traffic(x) for x in (BWD_STATES, BWD_KERNEL, BWD_FINISH)]
    del q, k, v, a, e, do, dfin, ws, inp, g
    return {"workload": f"backward of the layer-shaped prefill: {B} sequences x {T} tokens, H={H}, "
                        f"dk=dv={d}, bf16 q/k/v, fp32 gates, d_o and d_final; gradients of q, k, "
                        f"v, alpha, eta and the start state (fp32)",
            "us_per_call": round(ev_ms * 1e3, 2),
            "tokens_per_s": round(B * T / (ev_ms * 1e-3), 1),
            "workspace_bytes": ws_bytes,
            # the dq/dk tiles, the state-gradient update and the K S / Q S
            # products run on the bf16 MFMA (fp32 factors split hi/lo), the
            # Gram planes on it exactly; the substitutions, W / Z planes and
            # Mq products stay on the fp32 MFMA.  Priced against both peaks.
            "roofline": {"bound": "mfma", "achieved": round(tf, 2), "peak": BF16_MFMA_PEAK_TF,
                         "unit": "TFLOP/s", "frac": round(tf / BF16_MFMA_PEAK_TF, 4),
                         "frac_of_fp32_mfma_peak": round(tf / FP32_MFMA_PEAK_TF, 4),
                         "traffic": None if None in parts else sum(parts),
                         "kernel": "prefill_pc_kernel<states> + bwd_kernel + bwd_finish_kernel "
                                   "(one call)",
                         "avg_launch_us": round(ev_ms * 1e3, 2),
                         "algorithmic_flops_per_launch": flops,
                         "algorithmic_bytes_per_launch": nbytes,
                         "hbm_gbs": round(nbytes / (ev_ms * 1e-3) / 1e9, 1)},
            "clock_settle_ms": round(settle_ms, 1)}


def bench_variants(args, torch, kla, workloads, launches=50):
    """The layer-shaped prefill with the other step-size rules on the same
    kernel: the direct step beta = eta (Gated DeltaNet) and the direct step
    without decay (DeltaNet)."""
    inp = workloads.prefill("layer")
    B, H, d = inp["n_seqs"], inp["H"], inp["d"]
    T = inp["lengths"][0]
    dev = "cuda:0"
    q, k, v = (inp[n].to(dev).view(B, T, H, d) for n in ("q", "k", "v"))
    # these step rules assume unit-norm keys (with |k| up to e^3 the direct
    # step beta = eta would make the recurrence diverge)
    kf = k.float()
    k = (kf / kf.norm(dim=-1, keepdim=True)).to(k.dtype).contiguous()
    a, e = (inp[n].to(dev).view(B, T, H) for n in ("alpha", "eta"))
    o = torch.empty((B, T, H, d), dtype=torch.float32, device=dev)
    S = torch.empty((B, H, d, d), dtype=torch.float32, device=dev)
    stream = torch.cuda.current_stream()
    out = {"workload": f"layer-shaped prefill ({B} x {T} tokens, H={H}, d={d}, bf16, unit-norm "
                       f"keys) with the direct step (Gated DeltaNet) and without decay (DeltaNet)"}
    for name, alpha in (("gated_deltanet", a), ("deltanet", None)):
        def step():
            kla.kla_fwd_chunked_ex(q, k, v, alpha, e, eps=inp["eps"], beta_mode="direct", o=o,
                                   final_state=S)
        warm(step, args)
        _, ms = time_launches(step, launches, stream)
        out[name + "_us"] = round(ms * 1e3, 2)
        out[name + "_tokens_per_s"] = round(B * T / (ms * 1e-3), 1)
    del q, k, kf, v, a, e, o, S, inp
    return out


def bench_ccq(args, torch, kla, workloads, launches=50):
    """The curvature-conditioned read: the layer-shaped prefill and the
    decode workload with o_t = S_t^T (q_t - lambda_t Sigma_t q_t).  One
    prefill call = the query-cleaning pass, the bf16 prefill on the cleaned
    query's hi and lo parts, and their sum; one decode step = the sums update
    with the cleaned query, then the decode kernel."""
    inp = workloads.prefill("layer")
    B, H, d = inp["n_seqs"], inp["H"], inp["d"]
    T = inp["lengths"][0]
    dev = "cuda:0"
    q, k, v = (inp[n].to(dev).view(B, T, H, d) for n in ("q", "k", "v"))
    a, e = (inp[n].to(dev).view(B, T, H) for n in ("alpha", "eta"))
    lam = workloads.ccq_gate(0, B * T, H).to(dev).view(B, T, H)
    o = torch.empty((B, T, H, d), dtype=torch.float32, device=dev)
    S = torch.empty((B, H, d, d), dtype=torch.float32, device=dev)
    rec = kla.kla_ccq_state_floats(d)
    cout = torch.empty((B, H, rec), dtype=torch.float32, device=dev)
    stream = torch.cuda.current_stream()

    def step():
        kla.kla_fwd_chunked_ccq(q, k, v, a, e, lam, eps=inp["eps"], o=o, final_state=S,
                                ccq_out=cout)

    settle_ms = warm(step, args)
    _, ms = time_launches(step, launches, stream)
    th = B * T * H
    nbytes = th * (3 * d * 2 + 3 * 4 + d * 4) + B * H * (d * d + rec) * 4
    gbs = nbytes / (ms * 1e-3) / 1e9
    del q, k, v, a, e, lam, o, S, cout, inp
    out = {"workload": f"curvature-conditioned read, layer-shaped prefill: {B} x {T} tokens, H={H}, "
                       f"d={d}, bf16 q/k/v, fp32 gates and lambda",
           "prefill_us": round(ms * 1e3, 2),
           "prefill_tokens_per_s": round(B * T / (ms * 1e-3), 1),
           "prefill_hbm_gbs": round(gbs, 1),
           "prefill_algorithmic_bytes": nbytes,
           "clock_settle_ms": round(settle_ms, 1)}
    if not args.skip_decode:
        wl = workloads.decode(steps=args.decode_steps)
        N = wl["n_seqs"]
        state = wl["state"].to(dev)
        sums = torch.zeros((N, H, rec), dtype=torch.float32, device=dev)
        steps = [{n: st[n].to(dev) for n in ("q", "k", "v", "alpha", "eta")} for st in wl["steps"]]
        lams = [workloads.ccq_gate(100 + i, N, H).to(dev) for i in range(len(steps))]
        od = torch.empty((N, H, d), dtype=torch.float32, device=dev)
        s_scr, c_scr = state.clone(), sums.clone()
        wi = iter(range(1 << 30))

        def on_scratch():
            i = next(wi) % len(steps)
            st = steps[i]
            kla.kla_decode_step_ccq(st["q"], st["k"], st["v"], st["alpha"], st["eta"], lams[i],
                                    s_scr, c_scr, eps=wl["eps"], o=od)

        warm(on_scratch, args)
        del s_scr, c_scr
        it = iter(range(len(steps)))

        def one():
            i = next(it)
            st = steps[i]
            kla.kla_decode_step_ccq(st["q"], st["k"], st["v"], st["alpha"], st["eta"], lams[i],
                                    state, sums, eps=wl["eps"], o=od)

        _, dms = time_launches(one, len(steps), stream)
        dbytes = 2 * N * H * (d * d + rec) * 4
        out["decode_us_per_step"] = round(dms * 1e3, 2)
        out["decode_gbs"] = round(dbytes / (dms * 1e-3) / 1e9, 1)
        out["decode_bytes_per_step"] = dbytes
    return out


def bench_packed(args, torch, kla, workloads, launches=20):
    """The packed variable-length prefill (64 sequences of 128..8192 tokens,
    16 heads, d = 128, 5% of keys x10) through cu_seqlens, one launch per
    call; bytes and flops as the prefill over its token-heads."""
    inp = workloads.prefill("packed")
    H, d, n = inp["H"], inp["d"], inp["n_seqs"]
    dev = "cuda:0"
    q, k, v, a, e = (inp[x].to(dev) for x in ("q", "k", "v", "alpha", "eta"))
    cu = inp["cu_seqlens"].to(dev)
    tok = q.shape[0]
    o = torch.empty((tok, H, d), dtype=torch.float32, device=dev)
    S = torch.empty((n, H, d, d), dtype=torch.float32, device=dev)
    stream = torch.cuda.current_stream()

    def step():
        kla.kla_fwd_chunked(q, k, v, a, e, cu_seqlens=cu, eps=inp["eps"], o=o, final_state=S)

    settle_ms = warm(step, args)
    _, ev_ms = time_launches(step, launches, stream)
    nbytes, flops, flops_impl = prefill_work(tok * H, n, H, d)
    us = ev_ms * 1e3
    gbs = nbytes / (us * 1e-6) / 1e9
    tf = flops / (us * 1e-6) / 1e12
    del q, k, v, a, e, cu, o, S
    lens = inp["lengths"]
    out = {"workload": f"packed variable-length KLA prefill: {n} sequences, lengths uniform in "
                       f"[128, 8192] (seeded: {min(lens)}..{max(lens)}, {tok} tokens), H={H}, "
                       f"dk=dv={d}, bf16 q/k/v, 5% of keys x10, cu_seqlens",
           "tokens": tok,
           "us_per_launch": round(us, 1),
           "tokens_per_s": round(tok / (us * 1e-6), 1),
           "roofline": {"bound": "hbm", "achieved": round(gbs, 1), "peak": HBM_PEAK_GBS,
                        "unit": "GB/s", "frac": round(gbs / HBM_PEAK_GBS, 4),
                        "kernel": PREFILL_KERNEL, "avg_launch_us": round(us, 1),
                        "algorithmic_bytes_per_launch": nbytes,
                        "mfma_tflops": round(tf, 2),
                        "mfma_frac": round(tf / BF16_MFMA_PEAK_TF, 4),
                        "mfma_frac_regrouped": round(flops_impl / (us * 1e-6) / 1e12
                                                     / BF16_MFMA_PEAK_TF, 4),
                        "algorithmic_flops_per_launch": flops},
           "clock_settle_ms": round(settle_ms, 1)}
    if not args.skip_cpu_baseline:
        out["oracle"] = time_oracle(inp, tok)
    return out


def time_oracle(inp, tokens):
    """One wall-clock run of the fp64 oracle over a whole prefill workload on
    the host threads (fp64 conversion of the inputs included)."""
    import numpy as np
    import oracle
    cu = (inp["cu_seqlens"].numpy().astype(np.int64) if inp["cu_seqlens"] is not None
          else np.concatenate([[0], np.cumsum(inp["lengths"])]).astype(np.int64))
    t0 = time.perf_counter()
    oracle.fwd(inp["q"], inp["k"], inp["v"], inp["alpha"], inp["eta"], cu_seqlens=cu,
               eps=float(np.float32(inp["eps"])))
    dt = time.perf_counter() - t0
    return {"seconds": round(dt, 3), "tokens_per_s": round(tokens / dt, 1),
            "threads": oracle.num_threads(), "kind": "oracle", "sample": "whole workload, one run"}


def time_oracle_decode(wl):
    """The fp64 oracle over all steps of the decode workload (every sequence
    and head), one run, from the drawn start state."""
    import numpy as np
    import oracle
    t0 = time.perf_counter()
    state = wl["state"].double().numpy()
    for st in wl["steps"]:
        _, state = oracle.decode_step(st["q"], st["k"], st["v"], st["alpha"], st["eta"], state,
                                      eps=float(np.float32(wl["eps"])))
    dt = time.perf_counter() - t0
    n = wl["n_seqs"] * len(wl["steps"])
    return {"seconds": round(dt, 3), "tokens_per_s": round(n / dt, 1),
            "us_per_step": round(dt * 1e6 / len(wl["steps"]), 1),
            "threads": oracle.num_threads(), "kind": "oracle",
            "sample": f"all {len(wl['steps'])} steps of {wl['n_seqs']} sequences x {wl['H']} heads, one run"}


def cpu_baseline(pre, oracle, runs=5):
    """fp64 reference on the host over the whole layer-shaped prefill, run
    `runs` times (about 2 s of wall time, some 30 s of CPU time on 16 host
    threads); the median run is reported."""
    import numpy as np
    inp = pre["inp"]
    B, T, H, d = pre["shape"]
    cu = np.arange(B + 1, dtype=np.int64) * T
    times = []
    for _ in range(runs):
        t0 = time.perf_counter()
        oracle.fwd(inp["q"], inp["k"], inp["v"], inp["alpha"], inp["eta"], cu_seqlens=cu,
                   eps=float(np.float32(inp["eps"])))
        times.append(time.perf_counter() - t0)
    dt = sorted(times)[runs // 2]
    return dict(value=B * T / dt, unit="tokens/s", cores=oracle.num_threads(), kind="oracle",
                sample=f"whole layer-shaped prefill ({B} seqs x {T} tokens x {H} heads, d={d}), "
                       f"median of {runs} runs ({', '.join(f'{x:.2f}' for x in times)} s wall, each "
                       f"including the fp64 conversion of the inputs)",
                seconds=round(dt, 3))


def calibrate_copy(torch):
    """A plain device copy of known size, for scaling HBM byte counters."""
    n = 1 << 28  # 256 Mi floats = 1 GiB read + 1 GiB written
    src = torch.ones(n, dtype=torch.float32, device="cuda:0")
    dst = torch.empty_like(src)
    for _ in range(3):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"calibration": "device copy", "bytes_read": 4 * n, "bytes_written": 4 * n,
                      "launches": 3}), flush=True)


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[1])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    # The GPU takes some tens of milliseconds of sustained work to reach its
    # steady clock: every leg first runs its launch for this long.
    ap.add_argument("--settle-ms", type=float, default=200.0)
    ap.add_argument("--decode-steps", type=int, default=128)
    ap.add_argument("--skip-decode", action="store_true")
    ap.add_argument("--skip-long", action="store_true",
                    help="skip the long-context one-pass vs split-sequence comparison")
    ap.add_argument("--skip-kda", action="store_true",
                    help="skip the per-channel decay prefill and decode")
    ap.add_argument("--skip-variants", action="store_true",
                    help="skip the direct-step (Gated DeltaNet, DeltaNet) prefills")
    ap.add_argument("--skip-ccq", action="store_true",
                    help="skip the curvature-conditioned read (prefill and decode)")
    ap.add_argument("--skip-bwd", action="store_true",
                    help="skip the backward of the layer-shaped prefill")
    ap.add_argument("--skip-packed", action="store_true",
                    help="skip the packed variable-length prefill")
    ap.add_argument("--skip-cpu-baseline", action="store_true")
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="only run a plain 1 GiB device copy (counter calibration)")
    ap.add_argument("--ingest-counters", nargs=4, metavar=("FETCH_CSV", "WRITE_CSV",
                                                           "CAL_FETCH_CSV", "CAL_WRITE_CSV"),
                    help="record rocprofv3 counter CSVs into profiles/hbm_traffic.json")
    args = ap.parse_args()
    if args.ingest_counters:
        ingest_counters(*args.ingest_counters)
        return

    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py: this build runs on one GPU only; the multi-GPU layout is a design "
              "(sequences and heads shard with no communication) and is not measured. "
              "Run with --gpus 1.", file=sys.stderr, flush=True)
        sys.exit(2)

    import torch
    if args.calibrate_copy:
        calibrate_copy(torch)
        return
    import workloads
    import delta_rule_linear_amd as kla

    pre = bench_prefill(args, torch, kla, workloads)
    ms_per_step = pre["wall"] * 1e3 / args.steps
    value = pre["tokens"] / (pre["wall"] / args.steps)
    ach_gbs = pre["bytes"] / (pre["ev_ms"] * 1e-3) / 1e9
    ach_tf = pre["flops"] / (pre["ev_ms"] * 1e-3) / 1e12
    ach_tf_impl = pre["flops_impl"] / (pre["ev_ms"] * 1e-3) / 1e12
    B, T, H, d = pre["shape"]
    out = {
        "metric": "KLA prefill tokens/s (H=16,d=128) + decode state GB/s, % of MI355X roofline",
        "value": round(value, 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": f"layer-shaped KLA prefill: {B} sequences x {T} tokens, H={H}, "
                               f"dk=dv={d}, chunk 64, bf16 q/k/v, fp32 alpha/eta/o/final state",
                   "tokens_per_step": pre["tokens"], "token_heads_per_step": B * T * H},
        "roofline": {"bound": "hbm", "achieved": round(ach_gbs, 1), "peak": HBM_PEAK_GBS,
                     "unit": "GB/s", "frac": round(ach_gbs / HBM_PEAK_GBS, 4),
                     "traffic": measured_traffic(PREFILL_KERNEL), "kernel": PREFILL_KERNEL, "avg_launch_us": round(pre["ev_ms"] * 1e3, 2),
                     "algorithmic_bytes_per_launch": pre["bytes"],
                     "mfma_tflops": round(ach_tf, 2),
                     "mfma_frac": round(ach_tf / BF16_MFMA_PEAK_TF, 4),
                     "algorithmic_flops_per_launch": pre["flops"],
                     "flops_convention": "full-tile 10Cd+6d^2 = 180,224 per token-head (W/U form)",
                     "mfma_frac_regrouped": round(ach_tf_impl / BF16_MFMA_PEAK_TF, 4),
                     "algorithmic_flops_regrouped": pre["flops_impl"]},
        "clock_settle_ms": round(pre["settle_ms"], 1),
    }
    if not args.skip_decode:
        dec = bench_decode(args, torch, kla, workloads)
        dgbs = dec["state_bytes"] / (dec["ev_ms"] * 1e-3) / 1e9
        out["decode"] = {
            "workload": f"decode step: {dec['N']} sequences x {dec['H']} heads, dk=dv={dec['d']}, "
                        f"bf16 q/k/v, fp32 state in place, {dec['steps']} successive steps",
            "us_per_step": round(dec["wall"] * 1e6 / dec["steps"], 2),
            "tokens_per_s": round(dec["N"] * dec["steps"] / dec["wall"], 1),
            "roofline": {"bound": "hbm", "achieved": round(dgbs, 1), "peak": HBM_PEAK_GBS,
                         "unit": "GB/s", "frac": round(dgbs / HBM_PEAK_GBS, 4),
                         "traffic": measured_traffic(DECODE_KERNEL), "kernel": DECODE_KERNEL, "avg_launch_us": round(dec["ev_ms"] * 1e3, 2),
                         "algorithmic_bytes_per_launch": dec["state_bytes"]},
            "us_per_step_after_cache_sweep": round(dec["swept_ms"] * 1e3, 2),
            "frac_after_cache_sweep": round(dec["state_bytes"] / (dec["swept_ms"] * 1e-3) / 1e9
                                            / HBM_PEAK_GBS, 4),
            "clock_settle_ms": round(dec["settle_ms"], 1),
        }
        if not args.skip_cpu_baseline:
            out["decode"]["oracle"] = time_oracle_decode(dec["wl"])
        del dec
    if not args.skip_packed:
        out["packed"] = bench_packed(args, torch, kla, workloads)
    if not args.skip_long:
        out["long_context"] = bench_long(args, torch, kla, workloads)
    if not args.skip_kda:
        out["kda"] = bench_kda(args, torch, kla, workloads)
    if not args.skip_variants:
        out["gate_variants"] = bench_variants(args, torch, kla, workloads)
    if not args.skip_ccq:
        out["ccq"] = bench_ccq(args, torch, kla, workloads)
    if not args.skip_bwd:
        out["backward"] = bench_bwd(args, torch, kla, workloads)
    if not args.skip_cpu_baseline:
        import oracle
        out["cpu_baseline"] = cpu_baseline(pre, oracle)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
