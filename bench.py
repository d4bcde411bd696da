"""Throughput of the MoE FFN-service layer on one MI355X.

One step = one forward of the whole layer (router + top-k, dispatch,
[quantise], gate/up GEMM + SwiGLU, down GEMM, shared expert, combine) over
one batch of seeded synthetic hidden states already resident in HBM.

Default workload: the prefill chunk with skewed routing, T = 16384 tokens in
two micro-batches of 8192 on two HIP streams, h = 7168, E = 256 routed
experts, top-8, SwiGLU intermediate 2048, one shared expert (2048), bf16
with fp32 accumulation, router logits N(0, 1) + log of a Zipf(1.2) share.
Prints one JSON line.  Extra fields: "roofline" of the dominant kernel and
"cpu_baseline" (the fp64 oracle on the host, on a bounded sample).

Roofline: weight-streaming layers (one micro-batch) time the gate/up launch
with HIP events on the forward's stream over the timed region, against the
algorithmic bytes of the touched experts; where gate/up and down run as one
launch (bf16 decode regime), that launch, against the bytes of both.  The two-micro-batch prefill layer
times its compute-bound gate/up launch (256-row tiles) with HIP events in a
serial pass after the timed region (micro-batches back to back on one
stream, so no other kernel shares the interval), against the unpadded flops
of the rows in those tiles.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "MoE-FFN layer tokens/s on 1 MI355X + % of HBM-BW / MFMA roofline"
HBM_PEAK_GBS = 8000.0
MFMA_PEAK_TFLOPS = {"bf16": 2500.0, "w8a8": 5000.0, "f32": 157.3}
DEFAULT_WORKLOAD = "prefill_skew_t16384"


def log(msg):
    print(msg, file=sys.stderr, flush=True)


def kernel_source_hash():
    """Hash of all kernel sources: a stored counter reading is only reported
    while the code it was taken on is unchanged."""
    h = hashlib.sha256()
    d = os.path.join(ROOT, "expert_side_attention_amd", "csrc")
    for f in sorted(os.listdir(d)):
        with open(os.path.join(d, f), "rb") as fh:
            h.update(f.encode())
            h.update(fh.read())
    return h.hexdigest()[:16]


def copy_calibration(mib):
    """A plain device-to-device copy of a known size (for scaling the HBM
    byte counters of a profiler run)."""
    import torch
    n = mib * 1024 * 1024
    a = torch.ones(n, dtype=torch.uint8, device="cuda:0")
    b = torch.empty_like(a)
    for _ in range(5):
        b.copy_(a)
    torch.cuda.synchronize()
    print(json.dumps({"copy_calibration_bytes": n, "launches": 5}), flush=True)


def work_model(s, counts):
    """Algorithmic bytes and flops of one forward, from the per-expert counts.

    Bytes: weights of the experts that received rows (+ E4M3 block scales),
    the router, the shared experts, the input and the output.  Intermediates
    (Z, Y) are the implementation's own traffic and are not counted."""
    wb = 1 if s.mode == "w8a8" else (4 if s.mode == "f32" else 2)
    ab = 4 if s.mode == "f32" else 2
    touched = int(sum(1 for c in counts if c > 0))
    scale_b = (4 / (128 * 128)) if s.mode == "w8a8" else 0.0
    per_gu = 2 * s.I * s.h * (wb + scale_b)
    per_dn = s.h * s.I * (wb + scale_b)
    sh_gu = s.S * 2 * s.Is * s.h * (wb + scale_b)
    sh_dn = s.S * s.h * s.Is * (wb + scale_b)
    io = 2 * s.T * s.h * ab
    router = s.E * s.h * ab
    gate_up_bytes = touched * per_gu + sh_gu + s.T * s.h * ab
    # gate/up and down in one launch: both GEMMs' weights and X
    ffn_bytes = gate_up_bytes + touched * per_dn + sh_dn
    flops = (2 * s.T * s.k * 3 * s.h * s.I + 2 * s.T * s.S * 3 * s.h * s.Is
             + 2 * s.T * s.h * s.E)
    gate_up_flops = 2 * s.T * s.k * 2 * s.h * s.I + 2 * s.T * s.S * 2 * s.h * s.Is
    return {
        "touched_experts": touched,
        "gate_up_bytes": gate_up_bytes,
        "ffn_bytes": ffn_bytes,
        "gate_up_flops": gate_up_flops,
        "forward_bytes": touched * (per_gu + per_dn) + sh_gu + sh_dn + io + router,
        "forward_flops": flops,
        "per_expert_gate_up_bytes": per_gu,
    }


def big_tile_rows(s, counts, T):
    """Rows the forward sends to the compute-bound kernel (256-row tiles) and
    the number of those tiles, per group (routed experts, then shared).

    The library's tile plan: bf16 batches averaging more than 112 rows per
    expert give every group of at least 129 rows its full 256-row tiles, plus
    one partial tile when the remainder exceeds 128 rows; the rest stays on
    the weight-streaming kernel.  The tile count is checked against the
    library's own (traced) count, so a change of plan cannot go unnoticed."""
    if s.mode != "bf16" or -(-T * s.k // s.E) <= 112:
        return [0] * (s.E + s.S), 0
    rows, tiles = [], 0
    for gc in list(counts) + [T] * s.S:
        nbig, rem = 0, gc
        if gc >= 129:
            nbig, rem = gc // 256, gc % 256
            if rem * 2 > 256:
                nbig, rem = nbig + 1, 0
        rows.append(gc - rem)
        tiles += nbig
    return rows, tiles


def work_model_microbatches(s, layers, xs):
    """Sum of the per-micro-batch models: each micro-batch streams the
    weights of the experts it touches.  Also the unpadded flops of the
    compute-bound gate/up launch, per launch."""
    import torch
    tot = None
    big_flops = []
    for li, xi in zip(layers, xs):
        _, tr = li.forward(xi, trace=True)
        torch.cuda.synchronize()
        counts = tr["counts"].cpu().tolist()
        sm = s.with_tokens(xi.shape[0])
        m = work_model(sm, counts)
        rows, tiles = big_tile_rows(sm, counts, xi.shape[0])
        lib_tiles = int(tr["num_tiles"][1].item())
        if tiles != lib_tiles:
            raise RuntimeError(f"tile plan mismatch: {tiles} compute-bound tiles predicted, "
                               f"the library made {lib_tiles}")
        big_flops.append(sum(2 * r * 2 * (s.I if g < s.E else s.Is) * s.h
                             for g, r in enumerate(rows)))
        if tot is None:
            tot = dict(m)
        else:
            for kk in ("gate_up_bytes", "ffn_bytes", "gate_up_flops", "forward_bytes",
                       "forward_flops"):
                tot[kk] += m[kk]
            tot["touched_experts"] = max(tot["touched_experts"], m["touched_experts"])
    tot["gate_up_big_flops"] = big_flops
    return tot


def cpu_baseline(syn, min_seconds=10.0, max_tokens=512):
    """The fp64 oracle on host cores.  Small layers: the whole batch, repeated
    for at least min_seconds.  Large layers: a bounded sample, the first
    tokens of the batch (routed the same way as in the full batch, since a
    token's routing does not depend on the others): at most max_tokens, and
    for W8A8 layers, whose oracle quantises every touched expert's weights
    on each pass (a few seconds per expert), no more tokens than touch 12
    experts.  Repeated until min_seconds.  The weights of the experts the
    sample touches are drawn into host memory before the clock starts."""
    import numpy as np
    from concurrent.futures import ThreadPoolExecutor
    from oracle import afd_oracle as O
    try:
        from threadpoolctl import threadpool_info
        blas_threads = max((i.get("num_threads", 1) for i in threadpool_info()), default=1)
    except Exception:  # pragma: no cover
        blas_threads = 1
    s = syn.shape
    cores = len(os.sched_getaffinity(0))
    n = s.T if s.T * s.h * s.E <= 256 * 4096 * 64 else min(s.T, max_tokens)
    x = syn.hidden()[:n]
    wr, b = syn.router_weight(), syn.router_bias()

    class Src:
        shape = s

        def router_weight(self):
            return wr

        def router_bias(self):
            return b

        def expert(self, e):
            return experts[e]

        def shared(self, j):
            return shared[j]

    # routing of the sample (untimed) tells which experts to draw
    ids = O.OracleFFN(Src()).route(x)[1]
    if s.mode == "w8a8" and n > 1:
        seen, n_ok = set(), 0
        for t in range(n):
            seen |= set(ids[t].tolist())
            if len(seen) > 12:
                break
            n_ok = t + 1
        n = max(1, n_ok)
        x, ids = x[:n], ids[:n]
    touched = sorted(set(np.unique(ids).tolist()))
    with ThreadPoolExecutor(max_workers=max(1, min(16, cores))) as ex:
        experts = dict(zip(touched, ex.map(syn.expert, touched)))
        shared = list(ex.map(syn.shared, range(s.S)))
    orc = O.OracleFFN(Src())
    tokens, t0 = 0, time.perf_counter()
    while True:
        orc.forward(x)
        tokens += n
        el = time.perf_counter() - t0
        log(f"[bench] oracle pass {tokens // n}: {el:.1f} s")
        if el >= min_seconds:
            break
    what = (f"full {s.name} batch of {n} tokens" if n == s.T else
            f"first {n} of the {s.T} tokens of {s.name} ({len(touched)} experts touched)")
    return {"value": tokens / el, "unit": "tokens/s", "cores": int(min(cores, blas_threads)),
            "kind": "oracle",
            "sample": f"{what}, {tokens // n} pass(es), {el:.1f} s; fp64 NumPy/OpenBLAS, "
                      f"weights drawn into host RAM before timing; host has {cores} cores"}


def pipeline(args):
    """Attention/FFN ping-pong of two decode micro-batches on one GPU, in the
    co-located, overlapped and CU-split placements."""
    import torch
    from afd_inputs import CONFIGS, SyntheticLayer
    from expert_side_attention_amd import afd_pipeline as AP
    from expert_side_attention_amd.workload import build_layer, hidden_tensor

    if not torch.cuda.is_available():
        raise SystemExit("bench.py needs a GPU")
    shape = CONFIGS[args.workload]
    if shape.micro_batches != 1 or shape.mode == "f32":
        raise SystemExit("--pipeline takes a bf16 or W8A8 decode workload")
    dev = "cuda:0"
    M = 2
    syn = SyntheticLayer(shape.with_tokens(M * shape.T), seed=args.seed)
    log(f"[bench] pipeline: building {shape.name} x {M} micro-batches on {dev}")
    ffn0 = build_layer(syn, dev, max_tokens=shape.T, split_gemms=args.split_gemms)
    ffns = [ffn0, ffn0.sibling()]
    x = hidden_tensor(syn, dev)
    xs = [x[m * shape.T:(m + 1) * shape.T].contiguous() for m in range(M)]
    attn = [AP.AttentionStub(shape.T, shape.h, args.pipeline_context, device=dev, seed=m + 1)
            for m in range(M)]
    res = AP.measure(ffns, xs, attn, layers=args.pipeline_layers, reps=max(5, args.steps // 5))
    res.pop("finals")
    def rounded(v):
        if isinstance(v, dict):
            return {k: rounded(w) for k, w in v.items()}
        return round(v, 5) if isinstance(v, float) else v

    out = {"pipeline": rounded(res),
           "config": {"workload": shape.name, "micro_batch_tokens": shape.T, "micro_batches": M,
                      "split_gemms": bool(args.split_gemms),
                      "attention_stub": {"context": args.pipeline_context, "heads": 16, "d": 512,
                                         "kv_bytes_per_micro_batch": attn[0].kv_bytes()}},
           "data": "synthetic"}
    print(json.dumps(out), flush=True)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", default=DEFAULT_WORKLOAD)
    ap.add_argument("--seed", type=int, default=0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--graph", action="store_true",
                    help="also time the forward captured in a HIP graph and replayed")
    ap.add_argument("--single-launch", action="store_true",
                    help="run forwards of at most 16 tokens of a tiny layer as one "
                         "cooperative launch (the layer's single_launch option)")
    ap.add_argument("--micro-batches", type=int, default=0, metavar="M",
                    help="M micro-batches of the workload's micro-batch size, one HIP stream "
                         "each (default: the workload's own count)")
    ap.add_argument("--split-gemms", action="store_true",
                    help="one launch per weight-streaming GEMM (the layer's split_gemms "
                         "option; by default a bf16 decode layer runs both in one launch)")
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="MIB",
                    help="only run a plain copy of MIB MiB (profiler calibration)")
    ap.add_argument("--pipeline", action="store_true",
                    help="only run the attention/FFN micro-pipeline (two micro-batches of a "
                         "decode workload and an attention stand-in) and print its line")
    ap.add_argument("--pipeline-context", type=int, default=4096, metavar="L",
                    help="KV positions per token of the attention stand-in")
    ap.add_argument("--pipeline-layers", type=int, default=20)
    args = ap.parse_args()
    if args.copy_calibration:
        copy_calibration(args.copy_calibration)
        return
    if args.pipeline:
        if args.gpus != 1:
            print("bench.py measures one GPU only.", file=sys.stderr)
            sys.exit(2)
        pipeline(args)
        return
    if args.gpus != 1:
        print(f"bench.py measures one GPU only: the layer runs on a single MI355X "
              f"(--gpus {args.gpus} is not supported).", file=sys.stderr)
        sys.exit(2)

    import torch
    from afd_inputs import CONFIGS, SyntheticLayer
    from expert_side_attention_amd.workload import build_layer, hidden_tensor

    if not torch.cuda.is_available():
        raise SystemExit("bench.py needs a GPU")
    shape = CONFIGS[args.workload]
    if args.micro_batches:
        if args.micro_batches < 1:
            raise SystemExit("--micro-batches must be at least 1")
        import dataclasses
        shape = dataclasses.replace(shape, T=shape.T // shape.micro_batches * args.micro_batches,
                                    micro_batches=args.micro_batches)
    syn = SyntheticLayer(shape, seed=args.seed)
    dev = "cuda:0"
    log(f"[bench] building {shape.name} on {dev}")
    nmb = shape.micro_batches
    mbT = shape.T // nmb
    layer = build_layer(syn, dev, max_tokens=mbT, single_launch=args.single_launch,
                        split_gemms=args.split_gemms)
    layers = [layer] + [layer.sibling() for _ in range(nmb - 1)]
    x = hidden_tensor(syn, dev)
    xs = [x[i * mbT:(i + 1) * mbT] for i in range(nmb)]
    outs = [torch.empty_like(xi) for xi in xs]
    # weights touched per micro-batch (each micro-batch streams its own)
    model = work_model_microbatches(shape, layers, xs)
    streams = ([torch.cuda.current_stream()] if nmb == 1
               else [torch.cuda.Stream() for _ in range(nmb)])

    def step():
        for li, xi, oi, st in zip(layers, xs, outs, streams):
            li.forward(xi, out=oi, stream=st)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    for li in layers:
        li.profile_read()  # reset

    # timed region: K steps; HIP events around the gate/up GEMM launches (or
    # the single launch of gate/up and down), recorded on the stream each
    # forward runs on
    for li in layers:
        li.profile_enable(["gate_up", "single", "ffn"])
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        step()
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    gu_ms = gu_n = one_ms = one_n = ffn_ms = ffn_n = 0
    for li in layers:
        prof = li.profile_read()
        li.profile_enable([])
        gu_ms += prof["gate_up"][0]
        gu_n += prof["gate_up"][1]
        one_ms += prof["single"][0]
        one_n += prof["single"][1]
        ffn_ms += prof["ffn"][0]
        ffn_n += prof["ffn"][1]
    ms_step = (t1 - t0) * 1e3 / args.steps
    gu_avg = gu_ms / max(gu_n, 1)
    # tiny layers run the whole forward as one launch
    one_avg = one_ms / one_n if one_n else None
    # bf16 decode-regime layers run gate/up and down as one launch
    ffn_avg = ffn_ms / ffn_n if ffn_n else None

    # two micro-batches: the dominant (compute-bound gate/up) launch timed in
    # a serial pass, so that no kernel of the other stream shares its
    # interval
    big_avg = None
    if nmb > 1:
        for li in layers:
            li.profile_enable(["gate_up_big"])
        torch.cuda.synchronize()
        for _ in range(args.steps):
            for li, xi, oi in zip(layers, xs, outs):
                li.forward(xi, out=oi)
        torch.cuda.synchronize()
        b_ms = b_n = 0
        for li in layers:
            prof = li.profile_read()
            li.profile_enable([])
            b_ms += prof["gate_up_big"][0]
            b_n += prof["gate_up_big"][1]
        big_avg = b_ms / max(b_n, 1)

    # untimed breakdown of all stages, one micro-batch at a time
    all_stages = ["router", "dispatch", "quant", "gate_up", "down", "combine", "gate_up_big",
                  "down_big", "single", "ffn"]
    stage_tot = {}
    for li in layers:
        li.profile_enable(all_stages)
    for _ in range(10):
        for li, xi, oi in zip(layers, xs, outs):
            li.forward(xi, out=oi)
    torch.cuda.synchronize()
    for li in layers:
        for kk, v in li.profile_read().items():
            if v[1]:
                a = stage_tot.setdefault(kk, [0.0, 0])
                a[0] += v[0]
                a[1] += v[1]
        li.profile_enable([])
    stages = {kk: round(v[0] / v[1], 4) for kk, v in stage_tot.items()}
    # serial time of one step (micro-batches back to back on one stream)
    torch.cuda.synchronize()
    ts0 = time.perf_counter()
    for _ in range(max(1, args.steps // 4)):
        for li, xi, oi in zip(layers, xs, outs):
            li.forward(xi, out=oi)
    torch.cuda.synchronize()
    ms_serial = (time.perf_counter() - ts0) * 1e3 / max(1, args.steps // 4)

    graph_ms = None
    if args.graph:
        # one step captured in a HIP graph (all micro-batches, each on its
        # own stream, forked from and joined into the capture stream)
        cap = torch.cuda.Stream()
        g = torch.cuda.CUDAGraph()
        torch.cuda.synchronize()
        with torch.cuda.graph(g, stream=cap):
            if nmb == 1:
                layers[0].forward(xs[0], out=outs[0], stream=cap)
            else:
                fork = torch.cuda.Event()
                fork.record(cap)
                for li, xi, oi, st in zip(layers, xs, outs, streams):
                    st.wait_event(fork)
                    li.forward(xi, out=oi, stream=st)
                    cap.wait_stream(st)
        for _ in range(args.warmup):
            g.replay()
        torch.cuda.synchronize()
        tg0 = time.perf_counter()
        for _ in range(args.steps):
            g.replay()
        torch.cuda.synchronize()
        graph_ms = (time.perf_counter() - tg0) * 1e3 / args.steps

    ai = model["forward_flops"] / model["forward_bytes"]
    ridge = MFMA_PEAK_TFLOPS[shape.mode] * 1e12 / (HBM_PEAK_GBS * 1e9)
    bound = "mfma" if ai > ridge else "hbm"
    gu_launch_bytes = model["gate_up_bytes"] / nmb
    kernel_name = "gate_up grouped GEMM + SwiGLU (weight streaming)"
    tfile = os.path.join(ROOT, "profiles", f"traffic_gate_up_{shape.name}.json")
    if one_avg is not None:
        # the single launch is the whole forward: its bytes are the forward's
        gu_launch_bytes, gu_avg = model["forward_bytes"], one_avg
        kernel_name = "single-launch forward (fused_small_kernel)"
    elif ffn_avg is not None:
        gu_launch_bytes, gu_avg = model["ffn_bytes"] / nmb, ffn_avg
        kernel_name = ("gate/up + SwiGLU and down grouped GEMMs, one launch "
                       "(weight streaming, stream_ffn_kernel)")
        tfile = os.path.join(ROOT, "profiles", f"traffic_ffn_{shape.name}.json")
    achieved = gu_launch_bytes / (gu_avg * 1e-3) / 1e9
    traffic = None
    if os.path.exists(tfile):
        with open(tfile) as f:
            t = json.load(f)
        if t.get("kernel_source_hash") == kernel_source_hash():
            traffic = t.get("hbm_bytes_per_launch")
    res_hash = kernel_source_hash()
    if bound == "hbm":
        roofline = {"bound": "hbm",
                    "kernel": kernel_name,
                    "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                    "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": traffic,
                    "avg_launch_ms": round(gu_avg, 5),
                    "algorithmic_bytes_per_launch": int(gu_launch_bytes),
                    "timed": "HIP events around each such launch in the timed region"}
    else:
        # compute-bound gate/up launch: unpadded flops of its rows, averaged
        # over the micro-batches' launches (one per micro-batch per step)
        flops = sum(model["gate_up_big_flops"]) / nmb
        avg = big_avg if big_avg is not None else gu_avg
        if flops <= 0:
            raise RuntimeError("compute-bound layer without compute-bound tiles")
        tf = flops / (avg * 1e-3) / 1e12
        peak = MFMA_PEAK_TFLOPS[shape.mode]
        roofline = {"bound": "mfma",
                    "kernel": "gate_up grouped GEMM + SwiGLU, 256-row tiles (prefill_gemm4_kernel<1>)",
                    "achieved": round(tf, 2), "peak": peak, "unit": "TFLOP/s",
                    "frac": round(tf / peak, 4), "traffic": traffic,
                    "avg_launch_ms": round(avg, 5),
                    "algorithmic_flops_per_launch": int(flops),
                    "timed": ("HIP events around each compute-bound gate/up launch, serial pass "
                              f"of {args.steps} steps after the timed region")}
    value = shape.T / (ms_step * 1e-3)
    fwd_gbs = model["forward_bytes"] / (ms_step * 1e-3) / 1e9
    res = {
        "metric": METRIC,
        "value": round(value, 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": shape.mode if shape.mode != "w8a8" else "fp8_e4m3",
        "data": "synthetic (seeded N(0,1) hidden states, N(0,0.02) weights; no trained weights)",
        "config": {"workload": shape.name, "T": shape.T, "h": shape.h, "E": shape.E,
                   "k": shape.k, "I": shape.I, "S": shape.S, "Is": shape.Is,
                   "mode": shape.mode, "seed": args.seed,
                   "single_launch": bool(args.single_launch),
                   "split_gemms": bool(args.split_gemms), "micro_batches": nmb},
        "roofline": roofline,
        "forward": {"hbm_gbs": round(fwd_gbs, 1), "hbm_frac": round(fwd_gbs / HBM_PEAK_GBS, 4),
                    "bytes": int(model["forward_bytes"]),
                    "tflops": round(model["forward_flops"] / (ms_step * 1e-3) / 1e12, 2),
                    "mfma_frac": round(model["forward_flops"] / (ms_step * 1e-3) / 1e12
                                       / MFMA_PEAK_TFLOPS[shape.mode], 4),
                    "touched_experts": model["touched_experts"],
                    "micro_batches": nmb, "ms_serial_one_stream": round(ms_serial, 5),
                    "ms_graph_replay": None if graph_ms is None else round(graph_ms, 5),
                    "stage_ms": stages},
        "cpu_baseline": None,
        "kernel_source_hash": res_hash,
    }
    if not args.no_cpu_baseline:
        log("[bench] timing the fp64 oracle on the host")
        res["cpu_baseline"] = cpu_baseline(syn)
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
