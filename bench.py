#!/usr/bin/env python3
"""Benchmark of the weight-only-quantized MoE expert layer on one MI355X.

One step = one full layer forward (top-k gating, stable sort + permute, grouped GEMM 1 with
in-register dequantization and activation, grouped GEMM 2 with the gate weight, unpermute +
combine) over one batch of T synthetic tokens whose inputs already sit in HBM.

Default workload: the encoder MoE FFN of the MT model in "Who Says Elephants Can't Run"
(hidden 1024, FFN 4096, ReLU, 32 experts, top-1 Switch gating, softmax over all experts),
INT4 per-channel weights, T = 3840 tokens (96 sentences x 40 tokens), Zipf(1.1) skewed routing.

Prints one JSON line.  `roofline` describes the dominant kernel (the grouped GEMM launch with
the larger average duration), timed with HIP events on the stream the kernels run on, over
the timed region.  `cpu_baseline` times the CPU oracle on a bounded sample of the workload.
"""
import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "MoE-layer tokens/s + weight GB/s (or MFMA util) vs MI355X roofline, W4A16"
HBM_PEAK_GBS = 8000.0            # MI355X HBM3E
MFMA_F16_PEAK_TFLOPS = 2500.0    # MI355X dense fp16 MFMA
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic.json")
KERNEL_SOURCES = ("quantized_expert_layer_amd/csrc/gemm.hip",
                  "quantized_expert_layer_amd/csrc/common.hpp",
                  "quantized_expert_layer_amd/csrc/stream.hpp",
                  "quantized_expert_layer_amd/csrc/decode.hip",
                  "quantized_expert_layer_amd/csrc/route.hpp",
                  "quantized_expert_layer_amd/csrc/sort.hpp")


def kernel_source_hash():
    """Hash of the layer kernels' sources (GEMMs and the decode step) with comments and blank
    lines dropped, so that a traffic record stays valid across comment edits but not across any
    change to the code itself."""
    import re
    h = hashlib.sha256()
    for rel in KERNEL_SOURCES:
        with open(os.path.join(ROOT, rel), encoding="utf-8") as f:
            for line in f:
                line = re.sub(r"//.*", "", line).rstrip()
                if line:
                    h.update(line.encode() + b"\n")
    return h.hexdigest()[:16]


def parse():
    ap = argparse.ArgumentParser(description=__doc__.split("\n\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--config", default="mt_encoder")
    ap.add_argument("--T", type=int, default=0, help="tokens per step (default: config's first)")
    ap.add_argument("--wtype", default="int4")
    ap.add_argument("--active", type=int, default=0, help="restrict routing to experts [0, A)")
    ap.add_argument("--path", type=int, default=0, help="0 auto, 1 stream, 2 tile")
    ap.add_argument("--tile", type=int, default=0,
                    help="tile-path block tile: 0 auto, 1 64x256, 2 64x128, 3 128x128")
    ap.add_argument("--i2f", default="trick", choices=["trick", "native"],
                    help="int-to-float conversion of the codes in the tile GEMMs: the "
                         "exponent-of-1024 construction (default) or the conversion "
                         "instructions (the baseline it is measured against; MT encoder shape)")
    ap.add_argument("--rotate-gb", type=float, default=1.0,
                    help="cycle weight copies totalling at least this many GB (cold weights)")
    ap.add_argument("--no-fuse-rows", action="store_true",
                    help="copy x_perm and run the combine instead of reading and writing rows "
                         "through perm inside the GEMMs")
    ap.add_argument("--no-decode", action="store_true",
                    help="run a decode-sized step as the five separate calls instead of one "
                         "moe_decode_layer call")
    ap.add_argument("--finished", type=float, default=0.0,
                    help="batch pruning: this fraction of the sentences is finished (their tokens "
                         "take no expert); seeded, whole sentences of --sentence-len tokens")
    ap.add_argument("--sentence-len", type=int, default=40,
                    help="tokens per sentence for --finished (40: the MT workload's sentences)")
    ap.add_argument("--workload", default="layer", choices=["layer", "elb", "bf16"],
                    help="layer: the MoE layer step (default); elb: the expert lookahead buffer "
                         "of a speculative draft (--elb-layers layers, --elb-steps draft steps, "
                         "--T tokens per step, --elb-m experts per layer in the plan); bf16: "
                         "BF16 recovery from exponent / sign-mantissa bytes of one expert's "
                         "three matrices (--config's shape)")
    ap.add_argument("--elb-layers", type=int, default=24)
    ap.add_argument("--elb-steps", type=int, default=16)
    ap.add_argument("--elb-m", type=int, default=16)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-per-config", action="store_true",
                    help="skip the per-configuration block (graph step and dominant-kernel "
                         "roofline of the other layer shapes) of the default line")
    ap.add_argument("--cpu-budget-s", type=float, default=20.0)
    ap.add_argument("--no-shared-overlap", action="store_true",
                    help="capture the shared experts in series with the routed launches "
                         "(default: on a forked stream inside the graph)")
    ap.add_argument("--no-graph", action="store_true",
                    help="report the eager launches (one ctypes call per kernel) as the value "
                         "instead of the same steps replayed from captured HIP graphs")
    ap.add_argument("--calib-copy-mb", type=int, default=0,
                    help="run one device copy of this size before timing (counter calibration)")
    return ap.parse_args()


def attainable(q, torch, dev):
    """What plain code reaches on this device: a 1 GiB non-temporal read stream and a loop of
    independent MFMA 16x16x32 fp16 chains (the library's probe kernels), timed with HIP events."""
    cus = torch.cuda.get_device_properties(dev).multi_processor_count
    buf = torch.empty(1 << 30, dtype=torch.uint8, device=dev)
    sink = torch.empty(8 * cus, dtype=torch.int32, device=dev)
    out = torch.empty(2 * cus * 256, dtype=torch.float32, device=dev)
    iters = 4000

    def timed(fn, reps=10):
        for _ in range(2):
            fn()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        e0.record()
        for _ in range(reps):
            fn()
        e1.record()
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) * 1e-3 / reps

    t_read = timed(lambda: q.moe_probe_read(buf, 8 * cus, sink=sink))
    t_mfma = timed(lambda: q.moe_probe_mfma(iters, 2 * cus, out=out))
    flops = 2 * cus * 4 * iters * 16 * 16384.0
    del buf
    return {"hbm_read_GBps": (1 << 30) / t_read / 1e9, "mfma_f16_TFLOPs": flops / t_mfma / 1e12,
            "how": "library probes: 1 GiB read stream (4 x 16 B in flight per thread, "
                   f"{8 * cus} blocks); {2 * cus} blocks x 4 waves x {iters} x 16 independent "
                   "MFMA 16x16x32 fp16"}


def cpu_baseline(inp, budget_s):
    """Time the CPU oracle on a bounded sample of the workload's tokens."""
    import numpy as np

    import oracle
    try:
        from threadpoolctl import threadpool_info
        threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:
        threads = len(os.sched_getaffinity(0))
    T = inp.T
    n = min(T, 256)
    while True:
        toks = np.arange(n)
        t0 = time.perf_counter()
        oracle.moe_layer_tokens(inp, toks)
        dt = time.perf_counter() - t0
        if n >= T or dt * 2 > budget_s:
            break
        n = min(T, n * 4 if dt * 4 < budget_s else n * 2)
    return {"value": n / dt, "unit": "tokens/s", "cores": int(threads), "kind": "oracle",
            "sample": f"first {n} of {T} tokens of the same layer, fp64 NumPy oracle "
                      f"(dequantization of the experts those tokens use included), {dt:.2f} s"}


def bench_elb(args, q, torch, np, synth):
    """Expert lookahead buffer ("Specter" summary, Method steps, steps 2 and 3): device time of
    one draft step's count update over all layers, and of the planner's top-M snapshot."""
    import oracle
    cfg = synth.get_config(args.config)
    T = args.T or 1
    L, K, M = args.elb_layers, args.elb_steps, min(args.elb_m, cfg.E)
    dev = torch.device("cuda:0")
    inp = synth.make_inputs(cfg, K * L * T, with_weights=False)
    ids, _ = q.moe_route_topk(torch.from_numpy(inp.logits).to(dev), cfg.k, cfg.gate_mode)
    ids = ids.reshape(K, L, T, cfg.k).contiguous()
    steps = [ids[i].contiguous() for i in range(K)]
    counts = torch.zeros((L, cfg.E), dtype=torch.int32, device=dev)
    ex = torch.empty((L, M), dtype=torch.int32, device=dev)
    cn = torch.empty((L, M), dtype=torch.int32, device=dev)
    stream = torch.cuda.current_stream()

    def timed(fn, reps):
        for _ in range(args.warmup):
            fn()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        e0.record(stream)
        for r in range(reps):
            fn()
        e1.record(stream)
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) * 1e3 / reps

    acc_us = timed(lambda: q.moe_elb_accumulate(steps[0], cfg.E, counts), args.steps)
    top_us = timed(lambda: q.moe_elb_top_m(counts, M, experts=ex, top_counts=cn), args.steps)
    # working set per layer after k draft steps (experts with a nonzero count), checked
    # against the oracle's counts
    counts.zero_()
    want = np.zeros((L, cfg.E), dtype=np.int64)
    ids_h = ids.cpu().numpy()
    work = {}
    for i in range(K):
        q.moe_elb_accumulate(steps[i], cfg.E, counts)
        want = oracle.elb_accumulate(want, ids_h[i], cfg.E)
        if (i + 1) & i == 0 or i + 1 == K:
            work[i + 1] = float((want > 0).sum(axis=1).mean())
    if not np.array_equal(counts.cpu().numpy(), want):
        raise RuntimeError("ELB counts differ from the oracle")
    print(json.dumps({
        "metric": "expert lookahead buffer: device us per draft step (count update, all layers)",
        "value": acc_us, "unit": "us", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "higher_is_better": False, "vs_baseline": None, "dtype": "int32", "data": "synthetic",
        "top_m_us": top_us,
        "working_set_per_layer": work,
        "config": {"workload": f"elb_{cfg.name}_L{L}_K{K}_T{T}_M{M}", "layers": L,
                   "draft_steps": K, "tokens_per_step": T, "experts": cfg.E, "top_k": cfg.k,
                   "plan_m": M}}), flush=True)


def bench_bf16(args, q, torch, np, synth):
    """BF16 bit-field recombination ("ZipMoE" note): one expert's gate, up and down matrices
    (3 * d * I values) recovered from exponent and sign-mantissa bytes; HBM-bound."""
    import oracle
    cfg = synth.get_config(args.config)
    n = 3 * cfg.d * cfg.inter
    dev = torch.device("cuda:0")
    rng = np.random.default_rng(20261202)
    # expert-like values, bf16: N(0, 0.02^2)
    w = torch.from_numpy(rng.standard_normal(n, dtype=np.float32) * np.float32(0.02))
    bits = w.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    e_h, sm_h = oracle.bf16_decompose(bits)
    # enough copies to read past the 256 MB cache on every call
    n_copies = max(1, int(np.ceil(1e9 / (4.0 * n))))
    bufs = [(torch.from_numpy(e_h).to(dev), torch.from_numpy(sm_h).to(dev),
             torch.empty(n, dtype=torch.bfloat16, device=dev)) for _ in range(n_copies)]
    for b in bufs:
        q.moe_bf16_recombine(b[0], b[1], out=b[2])
    torch.cuda.synchronize()
    if not np.array_equal(bufs[0][2].view(torch.int16).cpu().numpy().view(np.uint16), bits):
        raise RuntimeError("BF16 recovery differs from the original bits")
    stream = torch.cuda.current_stream()
    for i in range(args.warmup):
        b = bufs[i % n_copies]
        q.moe_bf16_recombine(b[0], b[1], out=b[2])
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
           for _ in range(args.steps)]
    torch.cuda.synchronize()
    for i in range(args.steps):
        b = bufs[i % n_copies]
        evs[i][0].record(stream)
        q.moe_bf16_recombine(b[0], b[1], out=b[2])
        evs[i][1].record(stream)
    torch.cuda.synchronize()
    us = float(np.median([a.elapsed_time(z) for a, z in evs]) * 1e3)
    gbs = 4.0 * n / (us * 1e-6) / 1e9
    print(json.dumps({
        "metric": "BF16 recovery from bit fields: HBM GB/s (2 bytes read + 2 written per value)",
        "value": gbs, "unit": "GB/s", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "higher_is_better": True, "vs_baseline": None, "dtype": "u8->bf16", "data": "synthetic",
        "us_per_call": us,
        "roofline": {"bound": "hbm", "achieved": gbs, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": gbs / HBM_PEAK_GBS, "traffic": None},
        "config": {"workload": f"bf16_recombine_{cfg.name}_expert", "values": n,
                   "copies_rotated": n_copies}}), flush=True)


def measure_layer(args, q, torch, np, synth, cfg, T, wtype, active_n, steps, warmup, att):
    """One layer configuration: eager per-call times (HIP events on the launch stream), the
    dominant kernel's roofline, and the HIP-graph replayed step.  Returns (result, inputs)."""
    inp = synth.make_inputs(cfg, T, wtype=wtype, active=active_n)
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    layer = q.DeviceLayer.from_inputs(inp, device=dev, gemm_path=args.path, gemm_tile=args.tile,
                                      fuse_rows=not args.no_fuse_rows,
                                      decode=False if args.no_decode else None,
                                      gemm_i2f=q.I2FS[args.i2f])
    ws = layer.workspace(T)
    x = torch.from_numpy(inp.x).to(dev)
    logits = torch.from_numpy(inp.logits).to(dev)
    active = None
    if args.finished > 0:
        # whole sentences finish ("Who Says Elephants Can't Run", batch pruning), seeded
        n_sent = (T + args.sentence_len - 1) // args.sentence_len
        fin = np.random.default_rng(20261202 + T).random(n_sent) < args.finished
        running = ~np.repeat(fin, args.sentence_len)[:T]
        active = torch.from_numpy(running.astype(np.uint8)).to(dev)

    # weight rotation: enough copies that each step reads weights the caches do not hold (the
    # shared experts' too: every layer of a model has its own)
    own = (layer.w1, layer.w2) + (tuple(layer.shared) if layer.shared is not None else ())
    wbytes = sum(t.numel() for t in own)
    n_copies = max(1, int(np.ceil(args.rotate_gb * 1e9 / wbytes)))
    copies = [own] + [tuple(t.clone() for t in own) for _ in range(n_copies - 1)]
    plans = [layer.plan(ws, x, logits, weights=c, active=active) for c in copies]
    names = plans[0].names

    if args.calib_copy_mb:
        src = torch.empty(args.calib_copy_mb << 20, dtype=torch.uint8, device=dev)
        dst = torch.empty_like(src)
        dst.copy_(src)
        torch.cuda.synchronize()

    for i in range(warmup):
        plans[i % n_copies].run()
    torch.cuda.synchronize()

    K = steps
    n_ev = len(names) + 1
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(n_ev)] for _ in range(K)]
    stream = torch.cuda.current_stream()

    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(K):
        e = evs[i]
        plans[i % n_copies].run(marker=lambda j, e=e: e[j].record(stream))
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    ms_per_step = (t1 - t0) * 1e3 / K

    stage_us = {}
    for j, nm in enumerate(names):
        stage_us[nm] = float(np.mean([evs[i][j].elapsed_time(evs[i][j + 1]) for i in range(K)]) * 1e3)

    # algorithmic work of the two grouped GEMM launches (rows per expert from the routing)
    ids_h = ws.bufs["ids"].cpu().numpy().ravel()
    counts = np.bincount(ids_h[ids_h >= 0], minlength=cfg.E)
    n_active = int((counts > 0).sum())
    R = int(counts.sum())                       # routed rows (finished tokens route nowhere)
    per_expert_w1 = layer.w1.numel() // cfg.E + (0 if inp.scales1 is None else 2 * inp.scales1[0].size)
    per_expert_w2 = layer.w2.numel() // cfg.E + (0 if inp.scales2 is None else 2 * inp.scales2[0].size)
    g1 = {"flops": 2.0 * R * cfg.d * layer.n1, "bytes": n_active * per_expert_w1}
    g2 = {"flops": 2.0 * R * cfg.inter * cfg.d, "bytes": n_active * per_expert_w2}
    # the shared experts (fp16, every token): their weights once, over all T rows
    sh = {"flops": 0.0, "bytes": 0}
    if layer.shared is not None:
        sh = {"flops": 2.0 * T * cfg.d * 3 * layer.shared_inter,
              "bytes": int(sum(t.numel() for t in layer.shared))}
    if "decode" in stage_us:
        # one moe_decode_layer call (gating + sort, GEMM 1, GEMM 2 with the combine; with
        # shared experts, theirs inside the same launches): its events bracket all its
        # launches, so the unit is the whole call
        dom_name = "decode"
        dom = {"flops": g1["flops"] + g2["flops"], "bytes": g1["bytes"] + g2["bytes"]}
        if layer._shared_in_decode():
            dom = {"flops": dom["flops"] + sh["flops"], "bytes": dom["bytes"] + sh["bytes"]}
    else:
        dom_name, dom = max((("gemm1", g1), ("gemm2", g2)), key=lambda kv: stage_us[kv[0]])
    dom_us = stage_us[dom_name]
    t_hbm = dom["bytes"] / (HBM_PEAK_GBS * 1e9)
    t_mfma = dom["flops"] / (MFMA_F16_PEAK_TFLOPS * 1e12)
    if t_mfma >= t_hbm:
        achieved = dom["flops"] / (dom_us * 1e-6) / 1e12
        roof = {"bound": "mfma", "achieved": achieved, "peak": MFMA_F16_PEAK_TFLOPS,
                "unit": "TFLOP/s", "frac": achieved / MFMA_F16_PEAK_TFLOPS}
    else:
        achieved = dom["bytes"] / (dom_us * 1e-6) / 1e9
        roof = {"bound": "hbm", "achieved": achieved, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": achieved / HBM_PEAK_GBS}
    roof["kernel"] = dom_name
    roof["avg_us"] = dom_us
    traffic = None
    src_hash = kernel_source_hash()
    workload = f"{cfg.name}_{wtype}_T{T}" + (f"_A{active_n}" if active_n else "") + \
        (f"_fin{args.finished:g}" if args.finished else "") + \
        ("_i2fnative" if args.i2f == "native" else "")
    if os.path.exists(TRAFFIC_FILE):
        try:
            rec = json.load(open(TRAFFIC_FILE)).get(workload, {})
            if rec.get("kernel_source_hash") == src_hash and dom_name in rec:
                traffic = rec[dom_name].get("bytes_per_launch")
        except Exception:
            traffic = None
    roof["traffic"] = traffic
    roof["frac_of_attainable"] = roof["achieved"] / (att["hbm_read_GBps"] if roof["bound"] == "hbm"
                                                     else att["mfma_f16_TFLOPs"])

    graph_info = None
    if not args.no_graph:
        # one graph per weight copy, captured on a side stream; replays are checked against
        # the eager output of the same weights before they are timed
        gs = torch.cuda.Stream()
        gplans = [layer.plan(ws, x, logits, weights=c, stream=gs, active=active,
                             overlap_shared=not args.no_shared_overlap) for c in copies]
        graphs = []
        ref_out = None
        for gp in gplans:
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g, stream=gs):
                gp.run()
            graphs.append(g)
        torch.cuda.synchronize()
        plans[0].run()
        torch.cuda.synchronize()
        ref_out = ws.bufs["out"].clone()
        for _ in range(3):
            graphs[0].replay()
            torch.cuda.synchronize()
            if not torch.equal(ws.bufs["out"], ref_out):
                raise RuntimeError("graph replay differs from the eager layer output")
            plans[1 % n_copies].run()
            torch.cuda.synchronize()
        for i in range(warmup):
            graphs[i % n_copies].replay()
        torch.cuda.synchronize()
        tg0 = time.perf_counter()
        for i in range(K):
            graphs[i % n_copies].replay()
        torch.cuda.synchronize()
        tg1 = time.perf_counter()
        g_ms = (tg1 - tg0) * 1e3 / K
        graph_info = {"ms_per_step": g_ms, "tokens_per_s": T / (g_ms * 1e-3)}

    # The value is the graph replay when there is one: the same kernels on the same resident
    # buffers, without the per-call host overhead of the eager ctypes launches (which, for a
    # decode-sized layer, is as long as the GPU work itself).
    step_ms = graph_info["ms_per_step"] if graph_info is not None else ms_per_step
    layer_s = step_ms * 1e-3
    weight_bytes = g1["bytes"] + g2["bytes"] + sh["bytes"]
    flops = g1["flops"] + g2["flops"] + sh["flops"]
    result = {
        "metric": METRIC,
        "value": T / layer_s,
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": warmup,
        "ms_per_step": step_ms,
        "timing": "hip-graph replay" if graph_info is not None else "eager launches",
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "fp16",
        "data": "synthetic",
        "config": {"workload": workload, "d": cfg.d, "ffn": cfg.inter, "act": cfg.act,
                   "experts": cfg.E, "top_k": cfg.k, "tokens": T, "weights": wtype,
                   "group": cfg.group or "per-channel", "gate": cfg.gate_mode,
                   "active_experts": n_active, "max_rows_per_expert": int(counts.max()),
                   "finished_fraction": float(args.finished), "routed_rows": R,
                   "weight_copies_rotated": n_copies, "parallelism": "single-gpu"},
        "roofline": roof,
        "attainable": att,
        "layer": {"weight_GBps": weight_bytes / layer_s / 1e9,
                  "weight_frac_hbm": weight_bytes / layer_s / 1e9 / HBM_PEAK_GBS,
                  "mfma_TFLOPs": flops / layer_s / 1e12,
                  "mfma_frac": flops / layer_s / 1e12 / MFMA_F16_PEAK_TFLOPS,
                  "stage_us": stage_us, "kernel_source_hash": src_hash},
    }
    result["eager"] = {"ms_per_step": ms_per_step, "tokens_per_s": T / (ms_per_step * 1e-3)}
    if graph_info is not None:
        result["graph_replay"] = graph_info
    return result, inp


# The configurations of the pages' tables besides the headline (tokens per step as listed there):
# decode / verify steps and the mid-M and prefill layers of the fine-grained MoE shapes.
PER_CONFIG = (("qwen15_moe", 17), ("qwen15_moe", 544), ("dsv2_lite", 9), ("dsv2_lite", 288),
              ("phi35_moe", 1), ("phi35_moe", 17), ("phi35_moe", 8192))


def per_config(args, q, torch, np, synth, att):
    """Graph-replayed step and dominant-kernel roofline fraction of every other configuration
    (INT4 weights, their default routing), each timed like the headline on fewer steps."""
    out = {}
    for name, T in PER_CONFIG:
        cfg = synth.get_config(name)
        steps = 5 if T >= 4096 else 50
        res, _ = measure_layer(args, q, torch, np, synth, cfg, T, "int4", 0, steps, 5, att)
        roof = res["roofline"]
        out[res["config"]["workload"]] = {
            "ms_per_step": res["ms_per_step"], "timing": res["timing"],
            "tokens_per_s": res["value"], "steps": steps,
            "dominant": roof["kernel"], "dominant_us": roof["avg_us"], "bound": roof["bound"],
            "achieved": roof["achieved"], "unit": roof["unit"], "frac": roof["frac"],
            "traffic": roof["traffic"],
            "layer_weight_frac_hbm": res["layer"]["weight_frac_hbm"],
            "layer_mfma_frac": res["layer"]["mfma_frac"]}
        torch.cuda.synchronize()
        torch.cuda.empty_cache()
    return out


def main():
    args = parse()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py measures one GPU only: this layer build has no multi-GPU path "
              "(run with --gpus 1)", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    import quantized_expert_layer_amd as q
    import synth

    if args.workload in ("elb", "bf16"):
        torch.cuda.set_device(torch.device("cuda:0"))
        (bench_elb if args.workload == "elb" else bench_bf16)(args, q, torch, np, synth)
        return
    cfg = synth.get_config(args.config)
    T = args.T or cfg.T_list[0]
    att = attainable(q, torch, torch.device("cuda:0"))
    result, inp = measure_layer(args, q, torch, np, synth, cfg, T, args.wtype, args.active,
                                args.steps, args.warmup, att)
    if not args.no_per_config and args.config == "mt_encoder" and not args.T and not args.active \
            and args.wtype == "int4" and not args.finished and not args.path and not args.tile \
            and args.i2f == "trick" and not args.no_graph:
        result["per_config"] = per_config(args, q, torch, np, synth, att)
    if not args.no_cpu_baseline:
        result["cpu_baseline"] = cpu_baseline(inp, args.cpu_budget_s)
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
