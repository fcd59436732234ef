"""Benchmark of the block-scaled FP8 GEMM on one MI355X.

One step = one call of the GEMM (the whole path: host validation, operand and
scale fetch, MFMA partials, per-K-block promotion, bf16 epilogue, and for the
grouped calls the device-side segment offsets and the split of the segment
tails over K) over one batch of synthetic inputs already resident in HBM.

The headline workload is the largest one, the contiguous MoE grouped GEMM
(8 experts, 8192 tokens routed top-1, N 4096, K 7168), called with the
workspace its query asks for; its metric is FP8 TFLOP/s of algorithmic flops
(real token rows only), against the 5.0 PFLOP/s dense FP8 MFMA peak. Every
other workload (the small dense, decode, 4096^3, prefill and masked MoE GEMMs,
the 1x128 activation quantiser and the whole MoE step) is reported under
"workloads", each with:

* timing: the mean over one graph of launches, and median / p10 / p90 over
  at least 100 launches (graphs of 10 launches, each replay timed with HIP
  events on the launch stream); every timed replay follows at least 0.2 s of
  untimed replays of the same graph, so the GPU runs at the clock it holds
  under that load;
* a roofline entry against its bound (MFMA for the large GEMMs, HBM for the
  decode and masked shapes and the quantiser) with the 60% target where one
  is set;
* a parity verdict: every output element of one launch against the oracle
  (bit-exact for the quantiser and for routing, the tolerance
  |d - ref| <= 8e-3 |ref| + 1e-3 max|ref| for the GEMMs);
* the oracle's time for the same whole problem on all host cores (and on one
  core for the two small workloads).

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
HEADLINE = "moe_contiguous_g8_t8192"
METRIC = "FP8 GEMM TFLOP/s (and HBM GB/s at small M) + % of MI355X roofline, 1 GPU"
KERNEL_SOURCES = ["fp8_block_scaled_sa_amd/csrc/kernels.hpp", "fp8_block_scaled_sa_amd/csrc/dg_fp8.hip",
                  "fp8_block_scaled_sa_amd/csrc/moe.hpp"]
# The quantiser's source is hashed on its own, so its counters stay valid
# while the GEMM kernels change, and the other way round.
QUANT_SOURCES = ["fp8_block_scaled_sa_amd/csrc/quant.hpp"]
# Roofline bound of each workload and the fraction of it the workload targets.
BOUNDS = {
    "dense_64x256x512": ("latency", None),
    "decode_8x4096x7168": ("hbm", 0.6),
    "square_4096": ("mfma", 0.6),
    "square_4096_e4m3xe5m2": ("mfma", None),
    "prefill_8192x7168x2048": ("mfma", 0.6),
    "moe_contiguous_g8_t8192": ("mfma", None),
    "moe_contiguous_g8_t8192_seg": ("mfma", None),
    "moe_masked_g32_m256": ("hbm", 0.6),
}
NO_BENCH_ORACLE = {"square_4096_e4m3xe5m2"}
CHUNK = 10          # launches per timed graph replay of the distribution
WARM_SECONDS = 0.2  # untimed graph replays before each timed one, at least this long
LAST_WARM_REPLAYS = 0  # untimed replays of the last graph_time call
MIN_LAUNCHES = 100  # launches timed per workload for the distribution, at least


def kernel_hash(sources=KERNEL_SOURCES) -> str:
    h = hashlib.sha256()
    for f in sources:
        with open(os.path.join(ROOT, f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def host_threads() -> int:
    return len(os.sched_getaffinity(0))


def cpu_model() -> str:
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


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
            self.d = torch.empty((p.M, p.N), dtype=torch.bfloat16, device=dev)
            d = self.d
            for i in range(n):
                c = (a, sa, b, sb) if i == 0 else (a.clone(), sa.clone(), b.clone(), sb.clone())
                self.copies.append(c)
            fa, fb = gen.CONFIGS[name].get("fmt", ("e4m3", "e4m3"))
            if (fa, fb) == ("e4m3", "e4m3"):
                ws = ops.workspace(ops.dg_fp8_gemm_nt_workspace_bytes(p.M, p.N, p.K))
                self.fn = lambda c: ops.dg_fp8_gemm_nt_ws(c[0], c[1].t(), c[2], c[3], ws, d=d)
            else:
                self.fn = lambda c: ops.dg_fp8_gemm_nt_fmt(c[0], c[1].t(), c[2], c[3], fa, fb, d=d)
        elif self.kind == "contiguous":
            one = p.a.nbytes + p.b.nbytes
            n = max(1, min(8, -(-ROTATE_BYTES // one))) if rotate else 1
            base = (t(p.a), t(p.sa_t), t(p.b), t(p.sb), t(p.ids))
            self.d = torch.empty((p.M_total, p.N), dtype=torch.bfloat16, device=dev)
            d = self.d
            for i in range(n):
                self.copies.append(base if i == 0 else tuple(x.clone() for x in base))
            # the caller's workspace: segment offsets derived on the device, tails split over K
            ws = ops.workspace(ops.dg_fp8_grouped_gemm_contiguous_workspace_bytes(p.M_total, p.N, p.K, p.G))
            layout = t(gen.segment_layout(p.counts)) if gen.CONFIGS[name].get("segments") else None
            self.fn = lambda c: ops.dg_fp8_grouped_gemm_contiguous_ws(c[0], c[1].t(), c[2], c[3], c[4], ws,
                                                                      layout=layout, d=d)
        else:
            one = p.a.nbytes + p.b.nbytes
            n = max(1, min(8, -(-ROTATE_BYTES // one))) if rotate else 1
            base = (t(p.a), t(p.sa_t), t(p.b), t(p.sb), t(p.masked_m))
            self.d = torch.empty((p.G, p.M_max, p.N), dtype=torch.bfloat16, device=dev)
            d = self.d
            for i in range(n):
                self.copies.append(base if i == 0 else tuple(x.clone() for x in base))
            self.fn = lambda c: ops.dg_fp8_grouped_gemm_masked(c[0], c[1].transpose(1, 2), c[2], c[3], c[4], d=d)

    def __call__(self, i):
        self.fn(self.copies[i % len(self.copies)])


def graph_time(fn, launches, warmup, replays=1):
    """Capture `launches` calls of fn(i) in one HIP graph on a side stream and
    replay it `replays` times, each replay between HIP events on that stream.
    Returns (µs per launch for each replay, wall seconds of the first replay)."""
    import torch
    cap = torch.cuda.Stream()
    cap.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(cap):
        for i in range(warmup):
            fn(i)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph, stream=cap):
        for i in range(launches):
            fn(warmup + i)
    # Untimed replays: the first uploads the graph; the rest run the GPU for
    # at least WARM_SECONDS so that the timed replays start at the clock it
    # holds under this load, not at the lower one it drops to while the host
    # checks the previous workload against the oracle.
    global LAST_WARM_REPLAYS
    LAST_WARM_REPLAYS = 0
    t_warm = time.perf_counter()
    while True:
        with torch.cuda.stream(cap):
            graph.replay()
        torch.cuda.synchronize()
        LAST_WARM_REPLAYS += 1
        if time.perf_counter() - t_warm >= WARM_SECONDS:
            break
    per_launch, wall = [], None
    for r in range(replays):
        start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        t0 = time.perf_counter()
        start.record(cap)
        with torch.cuda.stream(cap):
            graph.replay()
        end.record(cap)
        torch.cuda.synchronize()
        if wall is None:
            wall = time.perf_counter() - t0
        per_launch.append(start.elapsed_time(end) * 1e3 / launches)
    del graph
    return per_launch, wall


def distribution(fn, warmup):
    """Median / p10 / p90 µs per launch over >= MIN_LAUNCHES launches, as
    graph replays of CHUNK launches each (the per-replay mean is one sample)."""
    samples, _ = graph_time(fn, CHUNK, warmup, replays=-(-MIN_LAUNCHES // CHUNK) * 2)
    s = np.asarray(samples)
    return {"median": round(float(np.median(s)), 3), "p10": round(float(np.percentile(s, 10)), 3),
            "p90": round(float(np.percentile(s, 90)), 3), "min": round(float(s.min()), 3),
            "launches": len(samples) * CHUNK, "launches_per_sample": CHUNK}


def roofline(name, flops, byts, us):
    bound, target = BOUNDS.get(name, ("mfma", None))
    if bound == "mfma":
        ach, peak, unit = flops / us / 1e6, FP8_PEAK_TFLOPS, "TFLOP/s"
    else:   # hbm, and the latency-bound small GEMM (reported against HBM)
        ach, peak, unit = byts / us / 1e3, HBM_PEAK_GBS, "GB/s"
    r = {"bound": bound, "achieved": round(ach, 2), "peak": peak, "unit": unit, "frac": round(ach / peak, 4),
         "target_frac": target}
    if target is not None:
        r["meets_target"] = bool(ach / peak >= target)
    return r


def oracle_gemm(name, p, threads):
    """The oracle's whole output for a GEMM workload (bf16 bits, sentinel where
    nothing is produced) and its wall time."""
    import oracle
    from synth import gen
    from tests.check import SENTINEL
    kind = gen.CONFIGS[name]["kind"]
    t0 = time.perf_counter()
    if kind == "dense":
        fa, fb = gen.CONFIGS[name].get("fmt", ("e4m3", "e4m3"))
        if (fa, fb) == ("e4m3", "e4m3"):
            ref = oracle.gemm_nt(p.a, p.sa_t.T, p.b, p.sb, threads=threads)
        else:
            ref = oracle.gemm_nt_fmt(p.a, fa, p.sa_t.T, p.b, fb, p.sb, threads=threads)
    elif kind == "contiguous":
        ref = oracle.grouped_contiguous(p.a, p.sa_t.T, p.b, p.sb, p.ids,
                                        np.full((p.M_total, p.N), SENTINEL, np.uint16), threads=threads)
    else:
        ref = oracle.grouped_masked(p.a, p.sa_t, p.b, p.sb, p.masked_m,
                                    np.full((p.G, p.M_max, p.N), SENTINEL, np.uint16), threads=threads)
    return ref, time.perf_counter() - t0


def parity(got, ref):
    """Whole-output verdict: written elements = produced elements (routing,
    bit for bit through the sentinel), and every produced one in tolerance."""
    from tests.check import SENTINEL, tolerance_report
    produced = ref != SENTINEL
    routing = bool(np.array_equal(got == SENTINEL, ~produced))
    rep = tolerance_report(got[produced], ref[produced])
    n = max(rep["n"], 1)
    return {"ok": routing and rep["bad"] == 0, "routing_exact": routing, "elements": rep["n"],
            "out_of_tolerance": rep["bad"], "within_1ulp": round(rep["le1ulp"] / n, 6),
            "exact": round(rep["exact"] / n, 6), "max_err_over_tol": round(rep["max_err_over_tol"], 4)}


DISTRIBUTION = True


def bench_gemm(name, steps, warmup, check, threads):
    """One GEMM workload: graph-timed mean over `steps` launches, the launch
    distribution, roofline, parity and the oracle's time on the same problem."""
    import torch
    from synth import gen
    from tests.check import SENTINEL
    from tests.gpu_util import bits
    p = gen.make_config(name)
    flops, byts, rows = work(name, p)
    run = Launcher(name, p, rotate=True)
    for i in range(warmup):
        run(i)
    torch.cuda.synchronize()
    per, wall = graph_time(run, steps, 0)
    warm_replays = LAST_WARM_REPLAYS
    mean_us = per[0]
    dist = distribution(run, 2) if DISTRIBUTION else None
    r = {"kernel_avg_us": round(mean_us, 3), "wall_ms_per_step": round(wall / steps * 1e3, 6),
         "us": dist, "tflops": round(flops / mean_us / 1e6, 2), "gbs": round(byts / mean_us / 1e3, 1),
         "algorithmic_flops": flops, "algorithmic_bytes": byts, "rows": rows, "operand_copies": len(run.copies),
         "warm_replays": warm_replays,
         "roofline": roofline(name, flops, byts, mean_us), "traffic": load_traffic(name)}
    # The e5m2 oracle sums each block exactly in 128-bit integers, ~50x slower
    # than the e4m3 one: the whole 4096^3 problem takes minutes, so that
    # variant's whole-output parity lives in the test suite only.
    if check and name in NO_BENCH_ORACLE:
        r["parity"] = "not checked here: tests/test_gpu_parity.py compares every element"
    elif check:
        run.d.view(torch.int16).fill_(SENTINEL)
        run(0)
        torch.cuda.synchronize()
        got = bits(run.d)
        ref, secs = oracle_gemm(name, p, threads)
        r["parity"] = parity(got, ref)
        r["oracle"] = {"seconds": round(secs, 3), "threads": threads, "gflops": round(flops / secs / 1e9, 2)}
        if name in ("dense_64x256x512", "decode_8x4096x7168"):
            reps = 5 if name == "dense_64x256x512" else 1
            t0 = time.perf_counter()
            for _ in range(reps):
                oracle_gemm(name, p, 1)
            r["oracle"]["seconds_1thread"] = round((time.perf_counter() - t0) / reps, 4)
    del run
    torch.cuda.empty_cache()
    return r, p


def time_quant(name, steps, warmup, check, threads):
    """The 1x128 activation quantiser, timed like the GEMMs, rotating over
    enough input copies that every launch reads from HBM; parity is bit-exact
    codes and scales against the oracle's quantiser."""
    import torch
    from fp8_block_scaled_sa_amd import ops
    from synth import gen
    c = gen.QUANT_CONFIGS[name]
    M, K = c["M"], c["K"]
    x = torch.from_numpy(gen.make_activations(name))
    if c["dtype"] == "bf16":
        x = x.to(torch.bfloat16)
    xc = x.cuda()
    n = max(1, min(8, -(-ROTATE_BYTES // (xc.numel() * xc.element_size()))))
    xs = [xc] + [xc.clone() for _ in range(n - 1)]
    q = torch.empty((M, K), dtype=torch.uint8, device="cuda")
    s = torch.empty((K // 128, M), dtype=torch.float32, device="cuda").t()
    run = lambda i: ops.dg_fp8_quantize_1x128(xs[i % n], q=q, s=s)  # noqa: E731
    per, _ = graph_time(run, steps, warmup)
    us = per[0]
    byts = M * K * xc.element_size() + M * K + M * (K // 128) * 4
    r = {"kernel_avg_us": round(us, 2), "us": distribution(run, 2) if DISTRIBUTION else None,
         "gbs": round(byts / us / 1e3, 1),
         "roofline": {"bound": "hbm", "achieved": round(byts / us / 1e3, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                      "frac": round(byts / us / 1e3 / HBM_PEAK_GBS, 4), "target_frac": None},
         "algorithmic_bytes": byts, "traffic": load_traffic(name, QUANT_SOURCES), "input_copies": n}
    if check:
        import oracle
        run(0)
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        rq, rs = oracle.quantize_1x128(x, threads=threads)
        secs = time.perf_counter() - t0
        ok_q = bool(np.array_equal(q.cpu().numpy(), rq))
        ok_s = bool(np.array_equal(s.cpu().numpy(), rs))
        r["parity"] = {"ok": ok_q and ok_s, "codes_bit_exact": ok_q, "scales_bit_exact": ok_s, "elements": M * K}
        r["oracle"] = {"seconds": round(secs, 3), "threads": threads}
    del xs
    torch.cuda.empty_cache()
    return r


MOE_LAYER = "moe_layer_g8_t8192"


def time_moe_layer(steps, warmup):
    """The contiguous MoE step end to end on the contiguous workload's shape
    (8 experts, 8192 tokens, K 7168, N 4096, top-1 routing seed): routing ->
    bf16 activations quantised into the padded layout -> grouped GEMM over
    the layout's capacity on tiles that follow the experts' segments (tails
    split over K in the caller's workspace), written straight to token order.
    Whole step timed as one graph of `steps` repetitions; also the step with
    a separate un-permute, and each stage on its own."""
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
    ws = ops.workspace(ops.dg_fp8_grouped_gemm_contiguous_workspace_bytes(M_cap, N, K, G))
    lib = ops._lib.load()

    def route(i):
        lib.dg_moe_route_contiguous(ed.data_ptr(), T, G, row.data_ptr(), ids.data_ptr(), tok.data_ptr(),
                                    layout.data_ptr(), M_cap, torch.cuda.current_stream().cuda_stream)

    def quant(i):
        ops.dg_fp8_quantize_1x128_gather(xs[i % n], tok, q=q, s=s)

    def gemm(i):
        ops.dg_fp8_grouped_gemm_contiguous_ws(q, s, bs[i % n], sbd, ids, ws, d=d)

    def unperm(i):
        ops.dg_moe_unpermute(d, row, out=out)

    def gemm_to_tokens(i):
        ops.dg_fp8_grouped_gemm_contiguous_ws(q, s, bs[i % n], sbd, ids, ws, token_of_row=tok, T=T, layout=layout,
                                              d=out)

    def step(i):  # the un-permute folded into the GEMM's epilogue
        route(i), quant(i), gemm_to_tokens(i)

    def step_unfused(i):
        route(i), quant(i), gemm(i), unperm(i)

    total = graph_time(step, steps, warmup)[0][0]
    unfused = graph_time(step_unfused, steps, warmup)[0][0]
    stages = {k: round(graph_time(f, steps, warmup)[0][0], 2)
              for k, f in (("route", route), ("quantize_gather", quant), ("grouped_gemm_to_tokens", gemm_to_tokens),
                           ("grouped_gemm", gemm), ("unpermute", unperm))}
    flops = 2 * T * N * K
    r = {"us_per_step": round(total, 2), "us_per_step_unfused": round(unfused, 2),
         "us": distribution(step, 2) if DISTRIBUTION else None,
         "tflops": round(flops / total / 1e6, 1), "stages_us": stages,
         "roofline": {"bound": "mfma", "achieved": round(flops / total / 1e6, 1), "peak": FP8_PEAK_TFLOPS,
                      "unit": "TFLOP/s", "frac": round(flops / total / 1e6 / FP8_PEAK_TFLOPS, 4), "target_frac": None},
         "rows_used": int(layout[G].item()), "rows_capacity": M_cap, "operand_copies": n,
         "parity": "not checked here (tests/test_gpu_moe.py and tests/test_gpu_graph.py check the step)"}
    del xs, bs
    torch.cuda.empty_cache()
    return r


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
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", default=HEADLINE)
    ap.add_argument("--others", default="all",
                    help="comma-separated extra workloads to time, 'all' or 'none'")
    ap.add_argument("--no-cpu-baseline", action="store_true",
                    help="skip the oracle (parity verdicts and CPU timings), e.g. under a profiler")
    ap.add_argument("--no-distribution", action="store_true",
                    help="skip the per-launch timing distribution (fewer launches under a profiler)")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: this build has no multi-GPU path "
              "(--gpus %d requested)" % args.gpus, file=sys.stderr)
        sys.exit(2)

    import torch
    from synth import gen
    assert torch.cuda.is_available(), "needs a GPU"
    check = not args.no_cpu_baseline
    threads = host_threads()
    global DISTRIBUTION
    DISTRIBUTION = not args.no_distribution

    head, p = bench_gemm(args.workload, args.steps, args.warmup, check, threads)
    kind = gen.CONFIGS[args.workload]["kind"]
    roof = dict(head["roofline"])
    roof["traffic"] = head["traffic"]
    roof["kernel_avg_us"] = head["kernel_avg_us"]
    roof["algorithmic_flops"] = head["algorithmic_flops"]
    roof["algorithmic_bytes"] = head["algorithmic_bytes"]
    roof["timed"] = "the whole call: every kernel it launches, graph-replayed on the launch stream"
    wall_s = head["wall_ms_per_step"] / 1e3
    if roof["unit"] == "TFLOP/s":
        value, unit = head["algorithmic_flops"] / wall_s / 1e12, "TFLOP/s"
    else:
        value, unit = head["algorithmic_bytes"] / wall_s / 1e9, "GB/s"

    cpu = None
    if check:
        o = head["oracle"]
        per_unit = head["algorithmic_flops"] / 1e12 if unit == "TFLOP/s" else head["algorithmic_bytes"] / 1e9
        cpu = {"value": round(per_unit / o["seconds"], 6), "unit": unit, "cores": threads, "kind": "oracle",
               "sample": "the whole %s problem (every output element, fp64 block sums), one pass of %.1f s on %d "
                         "threads of %s" % (args.workload, o["seconds"], threads, cpu_model())}

    others = {}
    names = [] if args.others == "none" else (
        [n for n in list(gen.CONFIGS) + list(gen.QUANT_CONFIGS) + [MOE_LAYER] if n != args.workload]
        if args.others == "all" else args.others.split(","))
    side_steps = max(MIN_LAUNCHES, args.steps)
    for n in names:
        if n == MOE_LAYER:
            others[n] = time_moe_layer(max(20, args.steps // 5), 3)
        elif n in gen.QUANT_CONFIGS:
            others[n] = time_quant(n, side_steps, 3, check, threads)
        else:
            others[n], _ = bench_gemm(n, side_steps, 3, check, threads)
        torch.cuda.empty_cache()

    line = {
        "metric": METRIC, "value": round(value, 3), "unit": unit, "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(head["wall_ms_per_step"], 6),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "fp8_e4m3 (fp32 accumulate, bf16 out)", "data": "synthetic",
        "config": dict(workload_shape(kind, p), workload=args.workload, lhs_scale="1x128",
                       rhs_scale="128x128", operand_copies=head["operand_copies"]),
        "tflops": head["tflops"],
        "us": head["us"],
        "warm_replays": head["warm_replays"],
        "roofline": roof,
        "cpu_baseline": cpu,
        "parity": head.get("parity"),
        "host": {"threads": threads, "cpu": cpu_model()},
        "workloads": others,
        "kernel_hash": kernel_hash(),
        "quant_kernel_hash": kernel_hash(QUANT_SOURCES),
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
