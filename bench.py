"""Benchmark of the fused MoE layer on one MI355X.

One step = one pass of the whole layer (router -> count/permute -> gated
grouped GEMM + SiLU-and-mul -> down grouped GEMM + unpermute -> top-k combine)
over one batch of synthetic tokens already resident in HBM, through the C ABI
(moe_forward).  Prints ONE JSON line: tokens/s for the whole job, the roofline
of the dominant kernel (the gated grouped GEMM, timed with HIP events on the
stream it runs on) and the CPU oracle's throughput on a bounded sample.

Default workload: the skewed bf16 prefill, M=16384 tokens, hidden 4096,
expert intermediate 1536, 128 experts, top-8 softmax over Zipf(1.2)-biased
logits -- the largest of the workloads, and the one whose grouped GEMMs are
bound by the matrix cores.  `--workload` selects the others.  Each run also
times hipGraph replay of the same step (`graph_ms_per_step`).
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

HBM_PEAK_GBS = 8000.0
MFMA_PEAK_TFLOPS = {"bf16": 2500.0, "fp8": 5000.0, "f32": 157.3}
DTYPE_NAME = {0: "f32", 1: "bf16", 2: "fp8"}
TRAFFIC_DIR = os.path.join(ROOT, "profiles")
GEMM_SOURCES = [os.path.join(ROOT, "combine_topk_softmax_amd", "csrc", f)
                for f in ("stream_gemm.hip", "grouped_gemm.hip", "mfma_gemm.hip", "moe_device.h")]


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="skewed_bf16")
    ap.add_argument("--cpu-sample-tokens", type=int, default=0,
                    help="tokens of the CPU-oracle sample (0: sized to ~15 s)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-graph", dest="graph", action="store_false",
                    help="skip timing hipGraph replay of the step (timed by default)")
    ap.add_argument("--weights", choices=["packed", "row_major"], default="packed",
                    help="expert weight layout (packed once before timing, as at model load)")
    ap.add_argument("--chunk-tokens", type=int, default=0,
                    help="run the experts step in chunks of this many tokens (Standard format; 0 = whole batch)")
    ap.add_argument("--activation", choices=["silu", "gelu"], default="silu",
                    help="gated activation of the experts (gelu_and_mul: exact GELU)")
    ap.add_argument("--router-weight-on-input", action="store_true",
                    help="top-1 routing with the router weight applied to the input before dispatch")
    ap.add_argument("--expert-shards", type=int, default=1,
                    help="run one expert-parallel shard of this many (expert_map: global expert g is local "
                         "to shard g %% N); routing stays global")
    ap.add_argument("--shard", type=int, default=0, help="which shard with --expert-shards")
    ap.add_argument("--dbo", action="store_true",
                    help="run the step as two microbatches (moe_forward_dbo: dispatch and combine on a second "
                         "stream beside the other microbatch's expert GEMMs)")
    ap.add_argument("--copy-calibration", type=float, default=0.0,
                    help="only run a plain device copy of this many GiB (counter calibration)")
    return ap.parse_args()


def kernel_source_hash() -> str:
    h = hashlib.sha256()
    for path in GEMM_SOURCES:
        with open(path, "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def gemm1_algorithmic(wl, counts):
    """Bytes and flops of one gated-GEMM launch: the w1 panels of experts that
    receive tokens, x read once, act written once; 2*rows*2I*K flops, rows the
    (token, pick) pairs routed to this GPU's experts (M*topk unsharded)."""
    import numpy as np
    eb_w = {0: 4, 1: 2, 2: 1}[wl.w_dtype]
    eb_a = 4 if wl.act_dtype == 0 else 2
    counts = np.asarray(counts)
    active = int((counts > 0).sum())
    rows = int(counts.sum())
    w_bytes = active * 2 * wl.I * wl.K * eb_w
    if wl.w_dtype == 2:
        w_bytes += active * (2 * wl.I // 128) * (wl.K // 128) * 4
    x_bytes = wl.M * wl.K * eb_a
    # act is written once: bf16 / fp32, or (fp8) e4m3 codes plus one fp32 scale per 128 columns
    act_bytes = rows * (wl.I + wl.I // 128 * 4 if wl.w_dtype == 2 else wl.I * eb_a)
    flops = 2 * rows * 2 * wl.I * wl.K
    return w_bytes + x_bytes + act_bytes, flops


def measured_traffic(workload: str):
    """HBM bytes per gated-GEMM launch from the committed rocprofv3 counter
    summary, if it was taken on the current kernel source."""
    path = os.path.join(TRAFFIC_DIR, f"gemm1_{workload}_traffic.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        t = json.load(f)
    if t.get("kernel_source_sha256") != kernel_source_hash():
        return None
    return t.get("hbm_bytes_per_launch")


def cpu_model() -> str:
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cpu_baseline(wl, d, sample_tokens: int):
    import oracle
    from workloads import sample_tokens as pick
    cores = int(os.environ.get("OMP_NUM_THREADS") or os.cpu_count() or 1)
    host = {k: (v.cpu() if hasattr(v, "cpu") else v) for k, v in d.items()}
    n = sample_tokens
    if n <= 0:
        # size the sample to roughly 15 s of oracle work: probes of 1 and 9
        # tokens split the call's fixed cost (the router over all tokens) from
        # the cost per sampled token
        t0 = time.perf_counter()
        oracle.moe_tokens(wl, host, [0])
        t1 = time.perf_counter()
        oracle.moe_tokens(wl, host, list(range(min(9, wl.M))))
        t9 = time.perf_counter() - t1
        per = max((t9 - (t1 - t0)) / max(min(9, wl.M) - 1, 1), 1e-4)
        fixed = max((t1 - t0) - per, 0.0)
        n = int(max(1, min(wl.M, (15.0 - fixed) / per)))
    toks = pick(wl.M, n, seed=7)
    t0 = time.perf_counter()
    oracle.moe_tokens(wl, host, toks)
    dt = time.perf_counter() - t0
    return {"value": len(toks) / dt, "unit": "tokens/s", "cores": cores, "kind": "oracle", "cpu": cpu_model(),
            "sample": f"{len(toks)} of {wl.M} tokens of {wl.name} (router over all {wl.M} tokens, "
                      f"then the expert MLPs and combine of the sampled tokens), float64 C, {dt:.1f} s"}


def copy_calibration(gib: float):
    import torch
    n = int(gib * (1 << 30))
    a = torch.empty(n, dtype=torch.uint8, device="cuda")
    b = torch.empty_like(a)
    a.fill_(1)
    torch.cuda.synchronize()
    for _ in range(3):
        b.copy_(a)
    torch.cuda.synchronize()
    print(json.dumps({"copy_bytes": n, "launches": 3}), flush=True)


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py: the fused MoE layer here runs on one GPU; --gpus {args.gpus} is not supported "
              f"(there is no multi-GPU expert-parallel path)", flush=True)
        sys.exit(2)
    import numpy as np
    import torch

    if args.copy_calibration > 0:
        copy_calibration(args.copy_calibration)
        return

    import combine_topk_softmax_amd as moe
    from workloads import WORKLOADS, make_inputs

    wl = WORKLOADS[args.workload]
    variant = {}
    if args.activation == "gelu":
        wl = wl.replace(activation=moe.ACTIVATION_GELU)
        variant["activation"] = "gelu"
    if args.router_weight_on_input:
        wl = wl.replace(topk=1, renormalize=False, router_weight_on_input=True)
        variant["router_weight_on_input"] = True
    torch.cuda.set_device(0)
    print(f"[bench] generating inputs for {wl.name}", file=sys.stderr, flush=True)
    d = make_inputs(wl, seed=0, device="cuda")
    if args.expert_shards > 1:
        # this GPU's share: global experts g with g % N == shard, local index g // N
        n, s = args.expert_shards, args.shard
        if not 0 <= s < n or wl.E % n:
            print("bench.py: --expert-shards needs 0 <= shard < N and N dividing E", flush=True)
            sys.exit(2)
        # the shard runs the routed experts only: a shared expert belongs to
        # each GPU's own tokens, not to an expert shard
        wl = wl.replace(shared_I=0)
        d.pop("w1s", None)
        d.pop("w2s", None)
        glob = torch.arange(s, wl.E, n, device="cuda")
        emap = torch.full((wl.E,), -1, dtype=torch.int32, device="cuda")
        emap[glob] = torch.arange(glob.numel(), dtype=torch.int32, device="cuda")
        for k in ("w1", "w2", "w1_scale", "w2_scale"):
            if d.get(k) is not None:
                d[k] = d[k][glob].contiguous()
        d["expert_map"] = emap
        variant["expert_shard"] = f"{s} of {n} ({glob.numel()} of {wl.E} experts)"
        wl = wl.replace(E=glob.numel(), global_E=wl.E)
    packed = args.weights == "packed" and wl.I % 128 == 0
    p = moe.make_problem(wl.E, wl.M, 2 * wl.I, wl.K, wl.topk, format=wl.format, act_dtype=wl.act_dtype,
                         w_dtype=wl.w_dtype, act_quant=wl.act_quant, scoring=wl.scoring,
                         renormalize=wl.renormalize, max_tokens_per_expert=wl.capacity, shared_N=2 * wl.shared_I,
                         weight_layout=moe.WEIGHTS_PACKED if packed else moe.WEIGHTS_ROW_MAJOR,
                         chunk_tokens=args.chunk_tokens, activation=wl.activation,
                         apply_router_weight_on_input=wl.router_weight_on_input, global_E=wl.global_E,
                         expert_map=d.get("expert_map"))
    pack_ms = None
    gw = {"w1": d["w1"], "w2": d["w2"]}
    if packed:
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        gw["w1"], gw["w2"] = moe.pack_weights(p, d["w1"], d["w2"])
        b.record()
        torch.cuda.synchronize()
        pack_ms = a.elapsed_time(b)
    ws = moe.empty_workspace(p)
    L = moe.workspace_layout(p)
    dbo = None
    if args.dbo:
        q = moe.dbo_microbatch_problem(p)
        dbo = ([moe.empty_workspace(q), moe.empty_workspace(q)], torch.cuda.Stream(), moe.DboEvents())
        variant["dbo"] = "two microbatches of %d and %d tokens" % ((wl.M + 1) // 2, wl.M // 2)
    odt = torch.float32 if wl.act_dtype == 0 else torch.bfloat16
    out = torch.empty(wl.M, wl.K, dtype=odt, device="cuda")
    shared = streams = None
    if wl.shared_I:
        shared = (d["w1s"], d["w2s"], torch.empty_like(out))
        streams = moe.SharedExpertStreams()
    stream = torch.cuda.current_stream()

    dbo_streams = (moe.SharedExpertStreams(), moe.SharedExpertStreams()) if (dbo and wl.shared_I) else None

    def step(events=None):
        if dbo:
            # no stage events inside the two-microbatch schedule: whole-step timing only
            moe.moe_forward_dbo(p, d["logits"], d["x"], gw["w1"], d.get("w1_scale"), gw["w2"], d.get("w2_scale"),
                                out, dbo[0], dbo[1], dbo[2], stream=stream, shared=shared, shared_streams=dbo_streams)
            return
        moe.moe_forward(p, d["logits"], d["x"], gw["w1"], d.get("w1_scale"), gw["w2"], d.get("w2_scale"), out, ws,
                        stream=stream, shared=shared, shared_streams=streams, events=events)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()

    # Timed region: K steps, each with stage events on the launch stream.
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(moe.NUM_STAGE_EVENTS)] for _ in range(args.steps)]
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    # torch creates its HIP events at their first record: do that here, so that
    # the timed steps do not create (and record twice) the stage events
    for e in [start, end] + [e for row in evs for e in row]:
        e.record(stream)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    start.record(stream)
    for k in range(args.steps):
        step(evs[k])
    end.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    total_ms = start.elapsed_time(end)
    ms_per_step = total_ms / args.steps
    stage_ms = np.array([[e[i].elapsed_time(e[i + 1]) for i in range(moe.NUM_STAGE_EVENTS - 1)] for e in evs])
    stage_avg = stage_ms.mean(axis=0)
    gemm1_ms = float(stage_avg[2])

    if dbo:
        # counts of the whole batch = the two microbatches' counts
        Lq = moe.workspace_layout(moe.dbo_microbatch_problem(p))
        counts = sum(w_[Lq.counts: Lq.counts + 4 * wl.E].view(torch.int32).cpu().numpy() for w_ in dbo[0][:2])
        stage_avg = np.full(moe.NUM_STAGE_EVENTS - 1, np.nan)
        gemm1_ms = float("nan")
    else:
        counts = ws[L.counts: L.counts + 4 * wl.E].view(torch.int32).cpu().numpy()
    local_pairs = wl.M * wl.topk * wl.E // wl.global_E if wl.global_E > wl.E else wl.M * wl.topk
    streaming = wl.w_dtype != 0 and local_pairs <= wl.E * (128 if wl.w_dtype == 2 else 256)
    g1_bytes, g1_flops = gemm1_algorithmic(wl, counts)
    achieved = g1_bytes / (gemm1_ms * 1e-3) / 1e9
    # the committed counter summaries cover the plain workloads only
    traffic = None if variant else measured_traffic(wl.name)
    rows = int(np.asarray(counts).sum())
    routed_flops = 2 * rows * 3 * wl.I * wl.K
    all_flops = routed_flops + wl.shared_flops()

    graph_ms = None
    if args.graph:
        g = torch.cuda.CUDAGraph()
        s = torch.cuda.Stream()
        s.wait_stream(stream)
        with torch.cuda.stream(s):
            with torch.cuda.graph(g, stream=s):
                if dbo:
                    moe.moe_forward_dbo(p, d["logits"], d["x"], gw["w1"], d.get("w1_scale"), gw["w2"],
                                        d.get("w2_scale"), out, dbo[0], dbo[1], dbo[2], shared=shared,
                                        shared_streams=dbo_streams)
                else:
                    moe.moe_forward(p, d["logits"], d["x"], gw["w1"], d.get("w1_scale"), gw["w2"],
                                    d.get("w2_scale"), out, ws, shared=shared, shared_streams=streams)
        torch.cuda.synchronize()
        for _ in range(args.warmup):
            g.replay()
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        a.record()
        for _ in range(args.steps):
            g.replay()
        b.record()
        torch.cuda.synchronize()
        graph_ms = a.elapsed_time(b) / args.steps

    cpu = None
    if not args.no_cpu_baseline:
        print("[bench] timing the CPU oracle on a sample", file=sys.stderr, flush=True)
        cpu = cpu_baseline(wl, d, args.cpu_sample_tokens)

    dtn = DTYPE_NAME[wl.w_dtype]
    # The gated GEMM is priced against whichever roof its arithmetic intensity
    # (algorithmic flops per algorithmic byte) puts it under.
    ridge = MFMA_PEAK_TFLOPS[dtn] * 1e12 / (HBM_PEAK_GBS * 1e9)
    roofline = {"kernel": "gated grouped GEMM (w1 + SiLU-and-mul), " + ("weight streaming" if streaming else "MFMA tiles"),
                "algorithmic_bytes_per_launch": g1_bytes, "algorithmic_flops_per_launch": g1_flops,
                "flops_per_byte": g1_flops / g1_bytes, "ridge_flops_per_byte": ridge, "avg_launch_ms": gemm1_ms}
    if g1_flops / g1_bytes > ridge:
        tflops = g1_flops / (gemm1_ms * 1e-3) / 1e12
        roofline = {"bound": "mfma", "achieved": tflops, "peak": MFMA_PEAK_TFLOPS[dtn], "unit": "TFLOP/s",
                    "frac": tflops / MFMA_PEAK_TFLOPS[dtn], "traffic": traffic, **roofline}
    else:
        roofline = {"bound": "hbm", "achieved": achieved, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                    "frac": achieved / HBM_PEAK_GBS, "traffic": traffic, **roofline}
    if args.chunk_tokens and args.chunk_tokens < wl.M:
        # the stage events mark the last chunk's kernels only: no per-launch roofline
        roofline = {"bound": None, "note": "chunked run: stage events cover the last chunk only"}
    if dbo:
        roofline = {"bound": None, "note": "two-microbatch run: no stage events, whole-step timing only"}
    result = {
        # value is the layer's tokens/s; the grouped GEMMs' TFLOP/s and roofline
        # fraction are in gemm_tflops and roofline
        "metric": "MoE layer tokens/s and grouped-GEMM TFLOP/s (% MFMA or HBM roofline), 1 GPU",
        "value": wl.M / (ms_per_step * 1e-3),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_per_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": dtn,
        "data": "synthetic (seeded; x ~ N(0,1), weights ~ N(0,0.02), logits per workload recipe)",
        "config": {"workload": wl.name, "tokens": wl.M, "hidden": wl.K, "intermediate": wl.I, "experts": wl.E,
                   "topk": wl.topk, "format": "batched_experts" if wl.format else "standard",
                   "shared_expert_intermediate": wl.shared_I or None,
                   "weight_layout": "packed (one-time reorder before timing)" if packed else "row_major",
                   "chunk_tokens": args.chunk_tokens or None, **variant,
                   "workspace_bytes": moe.workspace_size(p)},
        "weight_pack_ms": pack_ms,
        "roofline": roofline,
        "gemm_tflops": {"gated_gemm": g1_flops / (gemm1_ms * 1e-3) / 1e12,
                        "both_gemms": routed_flops / ((stage_avg[2] + stage_avg[3]) * 1e-3) / 1e12,
                        "peak": MFMA_PEAK_TFLOPS[dtn]},
        "layer_tflops": all_flops / (ms_per_step * 1e-3) / 1e12,
        "stage_ms": {"route": stage_avg[0], "prepare+plan": stage_avg[1], "gated_gemm": stage_avg[2],
                     "down_gemm": stage_avg[3], "combine": stage_avg[4]},
        "graph_ms_per_step": graph_ms,
        "cpu_baseline": cpu,
        "wall_s": wall,
    }
    def clean(v):
        # NaN (stages a two-microbatch run does not time) -> null
        if isinstance(v, dict):
            return {k: clean(x) for k, x in v.items()}
        if isinstance(v, float) and v != v:
            return None
        return v
    print(json.dumps(clean(result)), flush=True)


if __name__ == "__main__":
    main()
