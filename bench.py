"""Benchmark of the block-scaled FP8 GEMM on one MI355X.

One step = one launch of the GEMM (the whole path: host validation, operand
and scale fetch, MFMA partials, per-K-block promotion, bf16 epilogue) over one
batch of synthetic inputs already resident in HBM. The headline workload is
the decode-shaped dense GEMM M=8, N=4096, K=7168, which is bound by streaming
B from HBM; its metric is HBM GB/s of algorithmic bytes (A + sA + B + sB + D,
each counted once). The other workloads are timed the same way and reported
under "workloads", together with the 1x128 activation quantiser that
produces the GEMM's LHS (fp32 and bf16 token activations, 8192 x 7168;
HBM GB/s of algorithmic bytes: input + codes + scales), and the whole
contiguous MoE step (routing, quantisation into the padded layout, grouped
GEMM, rows back in token order) on the contiguous workload's shape.

Memory-bound workloads rotate over enough copies of their operands (> 2x the
256 MB last-level cache) that every launch reads its B from HBM.

Prints ONE JSON line on stdout.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, published
FP8_PEAK_TFLOPS = 5000.0       # MI355X dense FP8 MFMA, published (no sparsity)
ROTATE_BYTES = 600 * 2 ** 20   # > 2x the 256 MB last-level cache
HEADLINE = "decode_8x4096x7168"
METRIC = "FP8 GEMM TFLOP/s (and HBM GB/s at small M) + % of MI355X roofline, 1 GPU"
KERNEL_SOURCES = ["fp8_block_scaled_sa_amd/csrc/kernels.hpp", "fp8_block_scaled_sa_amd/csrc/dg_fp8.hip"]
# The quantiser's source is hashed on its own, so its counters stay valid
# while the GEMM kernels change, and the other way round.
QUANT_SOURCES = ["fp8_block_scaled_sa_amd/csrc/quant.hpp"]


def kernel_hash(sources=KERNEL_SOURCES) -> str:
    h = hashlib.sha256()
    for f in sources:
        with open(os.path.join(ROOT, f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def work(name, p):
    """Algorithmic flops and bytes (each tensor read or written once, real rows only)."""
    from synth import gen
    kind = gen.CONFIGS[name]["kind"]
    if kind == "dense":
        M, N, K = p.M, p.N, p.K
        flops = 2 * M * N * K
        byts = M * K + M * (K // 128) * 4 + N * K + (N // 128) * (K // 128) * 4 + M * N * 2
        return flops, byts, M
    if kind == "contiguous":
        N, K = p.N, p.K
        rows = int((p.ids >= 0).sum())
        used = int((p.counts > 0).sum())
        flops = 2 * rows * N * K
        byts = (p.M_total * K + p.M_total * (K // 128) * 4 + used * (N * K + (N // 128) * (K // 128) * 4)
                + rows * N * 2 + p.M_total * 4)
        return flops, byts, rows
    N, K = p.N, p.K
    rows = int(np.clip(p.masked_m, 0, p.M_max).sum())
    used = int((p.masked_m > 0).sum())
    flops = 2 * rows * N * K
    byts = (rows * K + rows * (K // 128) * 4 + used * (N * K + (N // 128) * (K // 128) * 4)
            + rows * N * 2 + p.G * 4)
    return flops, byts, rows


class Launcher:
    """Device copies of one workload and a closure that launches copy i."""

    def __init__(self, name, p, rotate):
        import torch
        from fp8_block_scaled_sa_amd import ops
        from synth import gen
        self.kind = gen.CONFIGS[name]["kind"]
        dev = torch.device("cuda:0")
        t = lambda x: torch.from_numpy(np.ascontiguousarray(x)).to(dev)  # noqa: E731
        self.copies = []
        if self.kind == "dense":
            one = p.a.nbytes + p.b.nbytes
            n = max(1, min(64, -(-ROTATE_BYTES // one))) if rotate else 1
            a, sa, b, sb = t(p.a), t(p.sa_t), t(p.b), t(p.sb)
            d = torch.empty((p.M, p.N), dtype=torch.bfloat16, device=dev)
            for i in range(n):
                c = (a, sa, b, sb) if i == 0 else (a.clone(), sa.clone(), b.clone(), sb.clone())
                self.copies.append(c)
            fa, fb = gen.CONFIGS[name].get("fmt", ("e4m3", "e4m3"))
            if (fa, fb) == ("e4m3", "e4m3"):
                self.fn = lambda c: ops.dg_fp8_gemm_nt(c[0], c[1].t(), c[2], c[3], d=d)
            else:
                self.fn = lambda c: ops.dg_fp8_gemm_nt_fmt(c[0], c[1].t(), c[2], c[3], fa, fb, d=d)
        elif self.kind == "contiguous":
            one = p.a.nbytes + p.b.nbytes
            n = max(1, min(8, -(-ROTATE_BYTES // one))) if rotate else 1
            base = (t(p.a), t(p.sa_t), t(p.b), t(p.sb), t(p.ids))
            d = torch.empty((p.M_total, p.N), dtype=torch.bfloat16, device=dev)
            for i in range(n):
                self.copies.append(base if i == 0 else tuple(x.clone() for x in base))
            if gen.CONFIGS[name].get("segments"):
                layout = t(gen.segment_layout(p.counts))
                self.fn = lambda c: ops.dg_fp8_grouped_gemm_contiguous_layout(c[0], c[1].t(), c[2], c[3], c[4],
                                                                              layout, d=d)
            else:
                self.fn = lambda c: ops.dg_fp8_grouped_gemm_contiguous(c[0], c[1].t(), c[2], c[3], c[4], d=d)
        else:
            one = p.a.nbytes + p.b.nbytes
            n = max(1, min(8, -(-ROTATE_BYTES // one))) if rotate else 1
            base = (t(p.a), t(p.sa_t), t(p.b), t(p.sb), t(p.masked_m))
            d = torch.empty((p.G, p.M_max, p.N), dtype=torch.bfloat16, device=dev)
            for i in range(n):
                self.copies.append(base if i == 0 else tuple(x.clone() for x in base))
            self.fn = lambda c: ops.dg_fp8_grouped_gemm_masked(c[0], c[1].transpose(1, 2), c[2], c[3], c[4], d=d)

    def __call__(self, i):
        self.fn(self.copies[i % len(self.copies)])


def time_workload(name, steps, warmup, rotate=True):
    """Warm up eagerly, then time exactly `steps` launches captured in one HIP
    graph (so host launch overhead is not measured), with HIP events on the
    stream the kernels run on around the replay. Eager per-launch events are
    kept as a cross-check."""
    import torch
    from synth import gen
    p = gen.make_config(name)
    flops, byts, rows = work(name, p)
    run = Launcher(name, p, rotate)
    for i in range(warmup):
        run(i)
    torch.cuda.synchronize()

    # eager cross-check: one event pair per launch
    cur = torch.cuda.current_stream()
    n_eager = min(steps, 50)
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(n_eager)]
    for i in range(n_eager):
        ev[i][0].record(cur)
        run(i)
        ev[i][1].record(cur)
    torch.cuda.synchronize()
    eager_us = [a.elapsed_time(b) * 1e3 for a, b in ev]

    # the timed region: `steps` launches in one graph
    graph = torch.cuda.CUDAGraph()
    cap = torch.cuda.Stream()
    cap.wait_stream(cur)
    with torch.cuda.stream(cap):    # one eager launch on the capture stream sets up its split-K workspace
        run(0)
    cap.synchronize()
    with torch.cuda.graph(graph, stream=cap):
        for i in range(steps):
            run(warmup + i)
    graph.replay()                  # untimed: first replay uploads the graph
    torch.cuda.synchronize()
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    start.record(cap)
    with torch.cuda.stream(cap):
        graph.replay()
    end.record(cap)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    avg_kernel_s = start.elapsed_time(end) / 1e3 / steps
    del graph
    return dict(p=p, flops=flops, bytes=byts, rows=rows, copies=len(run.copies),
                wall_s=wall, ms_per_step=wall / steps * 1e3,
                kernel_avg_us=avg_kernel_s * 1e6,
                eager_med_us=float(np.median(eager_us)), eager_min_us=float(np.min(eager_us)),
                tflops=flops / avg_kernel_s / 1e12, gbs=byts / avg_kernel_s / 1e9)


def time_quant(name, steps, warmup):
    """The 1x128 activation quantiser, timed like the GEMMs: eager warm-up, then
    `steps` launches in one graph between HIP events on the launch stream,
    rotating over enough input copies that every launch reads from HBM."""
    import torch
    from fp8_block_scaled_sa_amd import ops
    from synth import gen
    c = gen.QUANT_CONFIGS[name]
    M, K = c["M"], c["K"]
    x = torch.from_numpy(gen.make_activations(name))
    if c["dtype"] == "bf16":
        x = x.to(torch.bfloat16)
    x = x.cuda()
    n = max(1, min(8, -(-ROTATE_BYTES // (x.numel() * x.element_size()))))
    xs = [x] + [x.clone() for _ in range(n - 1)]
    q = torch.empty((M, K), dtype=torch.uint8, device="cuda")
    s = torch.empty((K // 128, M), dtype=torch.float32, device="cuda").t()
    run = lambda i: ops.dg_fp8_quantize_1x128(xs[i % n], q=q, s=s)  # noqa: E731
    for i in range(warmup):
        run(i)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    cap = torch.cuda.Stream()
    cap.wait_stream(torch.cuda.current_stream())
    with torch.cuda.graph(graph, stream=cap):
        for i in range(steps):
            run(i)
    graph.replay()
    torch.cuda.synchronize()
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    start.record(cap)
    with torch.cuda.stream(cap):
        graph.replay()
    end.record(cap)
    torch.cuda.synchronize()
    us = start.elapsed_time(end) * 1e3 / steps
    byts = M * K * x.element_size() + M * K + M * (K // 128) * 4
    del graph
    return {"kernel_avg_us": round(us, 2), "gbs": round(byts / us / 1e3, 1),
            "frac_hbm_peak": round(byts / us / 1e3 / HBM_PEAK_GBS, 4), "algorithmic_bytes": byts,
            "traffic": load_traffic(name, QUANT_SOURCES), "input_copies": n}


MOE_LAYER = "moe_layer_g8_t8192"


def time_moe_layer(steps, warmup):
    """The contiguous MoE step end to end on the contiguous workload's shape
    (8 experts, 8192 tokens, K 7168, N 4096, top-1 routing seed): routing ->
    bf16 activations quantised into the padded layout -> grouped GEMM over
    the layout's capacity on tiles that follow the experts' segments, written
    straight to token order. Whole step timed
    as one graph of `steps` repetitions; also the step with a separate
    un-permute, and each stage on its own."""
    import torch
    from fp8_block_scaled_sa_amd import ops
    from synth import gen
    c = gen.CONFIGS["moe_contiguous_g8_t8192"]
    G, T, N, K = c["G"], c["tokens"], c["N"], c["K"]
    x = torch.from_numpy(gen.normal_with_outliers(np.random.Generator(np.random.PCG64(921)), (T, K)))
    x = x.to(torch.bfloat16).cuda()
    e = np.random.Generator(np.random.PCG64(c["seeds"][2])).choice(G, T).astype(np.int32)
    ed = torch.from_numpy(e).cuda()
    b, sb = gen.make_grouped_rhs(G, N, K, c["seeds"][1])
    bd, sbd = torch.from_numpy(b).cuda(), torch.from_numpy(sb).cuda()
    del b
    n = max(1, min(4, -(-ROTATE_BYTES // (bd.numel() + x.numel() * 2))))
    xs = [x] + [x.clone() for _ in range(n - 1)]
    bs = [bd] + [bd.clone() for _ in range(n - 1)]
    M_cap = ops.dg_moe_contiguous_max_rows(T, G)
    row = torch.empty(T, dtype=torch.int32, device="cuda")
    ids = torch.empty(M_cap, dtype=torch.int32, device="cuda")
    tok = torch.empty(M_cap, dtype=torch.int32, device="cuda")
    layout = torch.empty(G + 1, dtype=torch.int32, device="cuda")
    q = torch.empty((M_cap, K), dtype=torch.uint8, device="cuda")
    s = torch.empty((K // 128, M_cap), dtype=torch.float32, device="cuda").t()
    d = torch.empty((M_cap, N), dtype=torch.bfloat16, device="cuda")
    out = torch.empty((T, N), dtype=torch.bfloat16, device="cuda")
    lib = ops._lib.load()

    def route(i):
        lib.dg_moe_route_contiguous(ed.data_ptr(), T, G, row.data_ptr(), ids.data_ptr(), tok.data_ptr(),
                                    layout.data_ptr(), M_cap, torch.cuda.current_stream().cuda_stream)

    def quant(i):
        ops.dg_fp8_quantize_1x128_gather(xs[i % n], tok, q=q, s=s)

    def gemm(i):
        ops.dg_fp8_grouped_gemm_contiguous(q, s, bs[i % n], sbd, ids, d=d)

    def unperm(i):
        ops.dg_moe_unpermute(d, row, out=out)

    def gemm_to_tokens(i):
        ops.dg_fp8_grouped_gemm_contiguous_to_tokens(q, s, bs[i % n], sbd, ids, tok, T, layout=layout, out=out)

    def step(i):  # the un-permute folded into the GEMM's epilogue
        route(i), quant(i), gemm_to_tokens(i)

    def step_unfused(i):
        route(i), quant(i), gemm(i), unperm(i)

    def graph_us(fn):
        graph = torch.cuda.CUDAGraph()
        cap = torch.cuda.Stream()
        cap.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(cap):    # warm-up on the capture stream also sets up its split-K workspace
            for i in range(warmup):
                fn(i)
        torch.cuda.synchronize()
        with torch.cuda.graph(graph, stream=cap):
            for i in range(steps):
                fn(i)
        graph.replay()
        torch.cuda.synchronize()
        a, z = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record(cap)
        with torch.cuda.stream(cap):
            graph.replay()
        z.record(cap)
        torch.cuda.synchronize()
        del graph
        return a.elapsed_time(z) * 1e3 / steps

    total = graph_us(step)
    unfused = graph_us(step_unfused)
    stages = {k: round(graph_us(f), 2) for k, f in (("route", route), ("quantize_gather", quant),
                                                    ("grouped_gemm_to_tokens", gemm_to_tokens),
                                                    ("grouped_gemm", gemm), ("unpermute", unperm))}
    flops = 2 * T * N * K
    return {"us_per_step": round(total, 2), "us_per_step_unfused": round(unfused, 2),
            "tflops": round(flops / total / 1e6, 1),
            "frac_fp8_peak": round(flops / total / 1e6 / FP8_PEAK_TFLOPS, 4), "stages_us": stages,
            "rows_used": int(layout[G].item()), "rows_capacity": M_cap, "operand_copies": n}


def cpu_baseline(name, p, byts, min_seconds=10.0):
    """The oracle, as it stands, on this host's cores: full passes over the
    workload, repeated until at least min_seconds of work have run (one pass if
    a single pass takes longer)."""
    import oracle
    threads = min(16, len(os.sched_getaffinity(0)))   # at most 16 host cores per GPU
    passes = 0
    t0 = time.perf_counter()
    while True:
        oracle.gemm_nt(p.a, p.sa_t.T, p.b, p.sb, threads=threads)
        passes += 1
        dt = time.perf_counter() - t0
        if dt >= min_seconds:
            break
    return {"value": round(passes * byts / dt / 1e9, 4), "unit": "GB/s", "cores": threads, "kind": "oracle",
            "sample": "the full %s problem (all %d outputs), %d passes in %.1f s" % (name, p.M * p.N, passes, dt)}


def load_traffic(workload, sources=KERNEL_SOURCES):
    """HBM bytes per launch from the committed FETCH_SIZE/WRITE_SIZE summary,
    or None when the kernel sources changed since the counters were taken."""
    path = os.path.join(ROOT, "profiles", "traffic.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        tr = json.load(f)
    ent = tr.get(workload)
    if not ent or ent.get("kernel_hash") != kernel_hash(sources):
        return None
    return ent.get("bytes_per_launch")


def workload_shape(kind, p):
    """Shape keys of a workload for the JSON config."""
    if kind == "dense":
        return {"M": p.M, "N": p.N, "K": p.K}
    if kind == "contiguous":
        return {"M_total": p.M_total, "N": p.N, "K": p.K, "G": p.G}
    return {"G": p.G, "M_max": p.M_max, "N": p.N, "K": p.K}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--workload", default=HEADLINE)
    ap.add_argument("--others", default="all",
                    help="comma-separated extra workloads to time, 'all' or 'none'")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: this build has no multi-GPU path "
              "(--gpus %d requested)" % args.gpus, file=sys.stderr)
        sys.exit(2)

    import torch
    from synth import gen
    assert torch.cuda.is_available(), "needs a GPU"

    head = time_workload(args.workload, args.steps, args.warmup)
    p = head["p"]
    traffic = load_traffic(args.workload)
    kind = gen.CONFIGS[args.workload]["kind"]
    small_m = kind == "dense" and p.M <= 64
    if small_m:
        value, unit = head["bytes"] / (head["ms_per_step"] / 1e3) / 1e9, "GB/s"
        roof = {"bound": "hbm", "achieved": round(head["gbs"], 2), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": round(head["gbs"] / HBM_PEAK_GBS, 4), "traffic": traffic}
    else:
        value, unit = head["flops"] / (head["ms_per_step"] / 1e3) / 1e12, "TFLOP/s"
        roof = {"bound": "mfma", "achieved": round(head["tflops"], 2), "peak": FP8_PEAK_TFLOPS,
                "unit": "TFLOP/s", "frac": round(head["tflops"] / FP8_PEAK_TFLOPS, 4), "traffic": traffic}
    roof["kernel_avg_us"] = round(head["kernel_avg_us"], 3)
    roof["eager_launch_med_us"] = round(head["eager_med_us"], 3)
    roof["algorithmic_bytes"] = head["bytes"]
    roof["algorithmic_flops"] = head["flops"]

    others = {}
    names = [] if args.others == "none" else (
        [n for n in list(gen.CONFIGS) + list(gen.QUANT_CONFIGS) + [MOE_LAYER] if n != args.workload]
        if args.others == "all" else args.others.split(","))
    for n in names:
        if n == MOE_LAYER:
            others[n] = time_moe_layer(max(10, args.steps // 10), max(3, args.warmup // 4))
            torch.cuda.empty_cache()
            continue
        if n in gen.QUANT_CONFIGS:
            # at least 50 timed launches: the graph's launch latency is spread over them
            others[n] = time_quant(n, max(50, args.steps // 4), max(3, args.warmup // 4))
            torch.cuda.empty_cache()
            continue
        r = time_workload(n, max(10, args.steps // 10), max(3, args.warmup // 4))
        others[n] = {"kernel_avg_us": round(r["kernel_avg_us"], 2), "eager_med_us": round(r["eager_med_us"], 2),
                     "tflops": round(r["tflops"], 2), "gbs": round(r["gbs"], 1),
                     "frac_fp8_peak": round(r["tflops"] / FP8_PEAK_TFLOPS, 4),
                     "frac_hbm_peak": round(r["gbs"] / HBM_PEAK_GBS, 4), "rows": r["rows"],
                     "operand_copies": r["copies"]}
        del r
        torch.cuda.empty_cache()

    cpu = None if args.no_cpu_baseline or kind != "dense" else cpu_baseline(args.workload, p, head["bytes"])

    line = {
        "metric": METRIC, "value": round(value, 3), "unit": unit, "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(head["ms_per_step"], 6),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "fp8_e4m3 (fp32 accumulate, bf16 out)", "data": "synthetic",
        "config": dict(workload_shape(kind, p), workload=args.workload, lhs_scale="1x128",
                       rhs_scale="128x128", operand_copies=head["copies"]),
        "tflops": round(head["tflops"], 3),
        "roofline": roof,
        "cpu_baseline": cpu,
        "workloads": others,
        "kernel_hash": kernel_hash(),
        "quant_kernel_hash": kernel_hash(QUANT_SOURCES),
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
