"""Benchmark of the MXFP8 o_proj chain on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--config decode|tiny|prefill|long]

One step = one pass of the chain over one batch of synthetic tokens:
mxfp8_quantize (BF16 x -> MXFP8), grouped_fp8_einsum (wo_a, MXFP8 epilogue
writing z), fp8_gemm_nt (wo_b on (z, sf), BF16 out), replayed from a HIP graph.
Inputs are resident in HBM before the timed region.  Every step uses the next of
R rotating copies of the inputs, weights and outputs (together >= 600 MB, more
than the 256 MB Infinity Cache), so each step reads its weights cold, as the
layers of a model do.

Printed: one JSON line.  `value` is chain TFLOP/s at the configuration's token
count; `ms_per_step` its time per call: the median of three timed rounds (after
an untimed clock ramp), the arms interleaved within each round, with the spread
of the rounds reported beside it.  Besides the headline arm ("chain") it
reports the arm that hands the einsum BF16 x ("x_fused": the library quantizes it
in the load path of the split-K decode kernel, otherwise into the workspace
first) and the unfused arm ("unfused": BF16 z re-quantized by a separate
launch, the arrangement the fused epilogue replaces), per-kernel durations from
HIP events on the launch stream, the dominant kernel's roofline fraction, and the
CPU oracle timed on this host's cores.  Per-kernel durations come from graphs of
one kernel each, replayed back to back, so they compare with a profiler's kernel
trace of the same command.  By default the line also carries the chain over 20
token counts from 1 to 32768 ("sweep": x drawn on the device, N(0, 1) with 0.1%
of the entries x100 as in the decode / prefill / long configurations; each
point the median of three rounds, and at 4096 and 32768 tokens also the
per-kernel times and the roofline of the dominant kernel, "rooflines"), the standalone quantizer on the
quantize-sweep rows ("quant_sweep") and the RMS-normalizing producer on the same
rows ("producer_sweep"); --no-sweep --no-quant-sweep --no-producer-sweep leaves
them out (profiling runs do, so that their kernel traces hold the configuration's
launches only).
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

METRIC = "o_proj chain µs/call + TFLOP/s (% HBM/FP8-MFMA roofline) at M=1..32768"
HBM_PEAK_GBS = 8000.0
FP8_PEAK_TFLOPS = 5000.0
ROTATE_BYTES = 600 << 20
RAMP_S = 0.3          # untimed load before each timed arm (clock ramp-up)
# token counts of the chain sweep: decode (1-256), 384, and prefill (512-32768)
DEFAULT_SWEEP = "1,2,4,8,16,32,64,128,192,256,384,512,768,1024,2048,4096,8192,16384,24576,32768"
KERNEL_SOURCES = ["gemm_tiled.hip", "gemm_tiled.hpp", "gemm_tiled_kernel.hpp", "gemm_tiled_inst.hip", "gemm_skinny.hip",
                  "gemm_common.hpp", "quantize.hip", "mx_device.hpp"]
KERNEL_NAMES = {"quantize": "mxfp8_quantize", "einsum": "grouped_fp8_einsum", "gemm": "fp8_gemm_nt"}


def kernel_source_hash() -> str:
    h = hashlib.sha256()
    for f in KERNEL_SOURCES:
        with open(os.path.join(ROOT, "mxfp8_activation_quantization_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def chain_bytes(M, G, K, N, P):
    """Algorithmic HBM bytes of each launch of the chain (every operand read once, every result written once)."""
    wa = G * N * K + G * N * (K // 128) * 4
    wb = P * G * N + P * (G * N // 128) * 4
    x_mx = M * (G * K + (G * K // 128) * 4)
    z_mx = M * (G * N + (G * N // 128) * 4)
    return {
        "quantize": M * G * K * 2 + x_mx,                  # BF16 x in, MXFP8 x out
        "einsum": x_mx + wa + z_mx,                        # MXFP8 x in, MXFP8 z out
        "gemm": z_mx + wb + M * P * 2,                     # MXFP8 z in, BF16 out
    }


def chain_flops(M, G, K, N, P):
    return {"quantize": 0, "einsum": 2 * M * G * K * N, "gemm": 2 * M * G * N * P}


def threads_used() -> int:
    try:
        from threadpoolctl import threadpool_info
        n = [i.get("num_threads", 0) for i in threadpool_info() if i.get("user_api") == "blas"]
        if n:
            return max(n)
    except Exception:
        pass
    return len(os.sched_getaffinity(0))


def cpu_baseline(cfg_name, inp, budget_s=12.0):
    """The oracle chain, as it stands, on a bounded sample of the same workload."""
    from oracle import chain_ref as cr

    w = cr.quantize_weights(inp["wo_a"], inp["wo_b"])
    x = inp["x"]
    rows = min(x.shape[0], 64)
    sample = x[:rows]
    G, N, K = w[0].shape
    P = w[2].shape[0]
    flop = 2 * rows * (G * K * N + G * N * P)
    reps, t0 = 0, time.perf_counter()
    while True:
        cr.o_proj_chain(sample, *w)
        reps += 1
        el = time.perf_counter() - t0
        if el >= budget_s:
            break
    tflops = flop * reps / el / 1e12
    cpu = ""
    try:
        with open("/proc/cpuinfo") as f:
            cpu = next((l.split(":", 1)[1].strip() for l in f if l.startswith("model name")), "")
    except OSError:
        pass
    return {"value": tflops, "unit": "TFLOP/s", "cores": threads_used(), "kind": "oracle",
            "sample": f"{cfg_name}: first {rows} token rows, whole chain incl. weight dequantization, "
                      f"{reps} repetitions in {el:.1f} s ({el / reps * 1e6:.0f} us/call)",
            "host_cpu": cpu, "host_threads_visible": len(os.sched_getaffinity(0)),
            "scalar_quantize": scalar_quantize_timing()}


def cpu_long(block=1024):
    """The oracle chain over all 32768 rows of the long configuration, in row blocks (the float64 x of every
    row at once would take 8.6 GB), timed once; the input generation is outside the timed span."""
    import synth_inputs as si
    from oracle import chain_ref as cr

    cfg = si.CHAIN_CONFIGS["long"]
    inp = si.chain_inputs(cfg.shape, cfg.seed, cfg.outlier_rate)
    t0 = time.perf_counter()
    w = cr.quantize_weights(inp["wo_a"], inp["wo_b"])
    t_w = time.perf_counter() - t0
    x = inp["x"]
    M = x.shape[0]
    t0 = time.perf_counter()
    for r0 in range(0, M, block):
        cr.o_proj_chain(x[r0:r0 + block], *w)
        if (r0 + block) % 4096 == 0:
            print(f"[bench] oracle long: {r0 + block} of {M} rows, {time.perf_counter() - t0:.1f} s", file=sys.stderr,
                  flush=True)
    el = time.perf_counter() - t0
    flop = cfg.shape.flop
    return {"value": flop / el / 1e12, "unit": "TFLOP/s", "cores": threads_used(), "kind": "oracle",
            "sample": f"long: all {M} rows in blocks of {block}, timed once: {el:.1f} s "
                      f"(+ {t_w:.1f} s to quantize the weights)", "seconds": el}


def scalar_quantize_timing():
    """The oracle's scalar (pure-Python, exact-rational) quantizer, one thread, labelled "scalar": the tiny
    configuration's x and the quantize-sweep rows at M = 1 and 7 (larger M take minutes)."""
    import synth_inputs as si
    from oracle import mxfp8_ref as mx

    cases = {}
    tiny = si.CHAIN_CONFIGS["tiny"]
    inputs = {"tiny x [4, 512]": si.chain_inputs(tiny.shape, tiny.seed, tiny.outlier_rate)["x"]}
    for M in (1, 7):
        inputs[f"quantize sweep [{M}, 7168]"] = si.quant_sweep_input(M)
    for name, x in inputs.items():
        t0 = time.perf_counter()
        mx.quantize_scalar(x)
        el = time.perf_counter() - t0
        cases[name] = {"us_per_call": el * 1e6, "ns_per_element": el * 1e9 / x.size}
    return {"kind": "scalar", "threads": 1, "cases": cases}


def copy_calibration(torch, mib):
    """A plain device copy of known size: what FETCH_SIZE / WRITE_SIZE read for it calibrates them."""
    n = mib << 20
    src = torch.empty(n, dtype=torch.uint8, device="cuda").fill_(1)
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    for _ in range(5):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"copy_bytes_read": n, "copy_bytes_written": n, "repeats": 5}), flush=True)


def time_arm_graphs(torch, graphs, stream, steps, warmup):
    """Average µs per replay of a list of captured graphs, replayed round-robin on `stream`
    (HIP events on that stream)."""
    with torch.cuda.stream(stream):
        for i in range(warmup):
            graphs[i % len(graphs)].replay()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    with torch.cuda.stream(stream):
        e0.record(stream)
        for i in range(steps):
            graphs[i % len(graphs)].replay()
        e1.record(stream)
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) / steps * 1e3


def median_rounds(torch, graphs_by_arm, stream, reps, rounds=3, ramp_s=RAMP_S, calls_per_replay=1):
    """µs per call of each arm: an untimed clock ramp (all arms replayed for ramp_s seconds), then `rounds`
    rounds in which every arm's graph is replayed `reps` times and timed with HIP events on `stream`, the
    arms interleaved within a round.  Returns {arm: {"us": median, "rounds": [...], "spread": max - min}}."""
    t_ramp = time.perf_counter()
    while time.perf_counter() - t_ramp < ramp_s:
        with torch.cuda.stream(stream):
            for g in graphs_by_arm.values():
                g.replay()
        torch.cuda.synchronize()
    res = {a: [] for a in graphs_by_arm}
    for _ in range(rounds):
        for arm, g in graphs_by_arm.items():
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            with torch.cuda.stream(stream):
                e0.record(stream)
                for _ in range(reps):
                    g.replay()
                e1.record(stream)
            torch.cuda.synchronize()
            res[arm].append(e0.elapsed_time(e1) * 1e3 / (reps * calls_per_replay))
    return {a: {"us": float(np.median(v)), "rounds": v, "spread": max(v) - min(v)} for a, v in res.items()}


def recorded_traffic(workload, kind):
    """HBM bytes per launch of `kind` from profiles/traffic_<workload>.json (rocprofv3 FETCH_SIZE +
    WRITE_SIZE, scaled by a device copy), or None when absent or taken on other kernel sources."""
    path = os.path.join(ROOT, "profiles", f"traffic_{workload}.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        tr = json.load(f)
    if tr.get("kernel_source_hash") != kernel_source_hash():
        return None
    return tr.get(kind, {}).get("hbm_bytes_per_launch")


def roofline_block(kind, M, G, K, N, P, t_us, traffic=None):
    """Roofline of one launch (the einsum or the GEMM) at M tokens from its average duration."""
    flops = chain_flops(M, G, K, N, P)[kind]
    nbytes = chain_bytes(M, G, K, N, P)[kind]
    if flops / nbytes < FP8_PEAK_TFLOPS / HBM_PEAK_GBS * 1e3:
        ach = nbytes / (t_us * 1e-6) / 1e9
        return {"bound": "hbm", "achieved": ach, "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": ach / HBM_PEAK_GBS,
                "traffic": traffic, "kernel": KERNEL_NAMES[kind], "algorithmic_bytes_per_launch": nbytes,
                "avg_launch_us": t_us}
    ach = flops / (t_us * 1e-6) / 1e12
    return {"bound": "mfma", "achieved": ach, "peak": FP8_PEAK_TFLOPS, "unit": "TFLOP/s",
            "frac": ach / FP8_PEAK_TFLOPS, "traffic": traffic, "kernel": KERNEL_NAMES[kind],
            "algorithmic_flop_per_launch": flops, "avg_launch_us": t_us}


def sweep_x(torch, M, G, K):
    """BF16 [M, G*K] on the device: N(0, 1) with round(0.001 * numel) entries (positions drawn with
    replacement) multiplied by 100 before the BF16 rounding, seeded per token count."""
    gen = torch.Generator(device="cuda")
    gen.manual_seed(20260100 + M)
    x = torch.randn((M, G * K), generator=gen, device="cuda", dtype=torch.float32)
    n_out = int(round(0.001 * x.numel()))
    if n_out:
        pos = torch.randint(0, x.numel(), (n_out,), generator=gen, device="cuda")
        x.view(-1)[pos] *= 100.0
    return x.to(torch.bfloat16)


def sweep(torch, L, Ms, dims, w, stream, args, kernel_ms=(4096, 32768)):
    """µs/call of the chain, x_fused and unfused arms over token counts, weights rotated as in the headline
    run; `fusion_saving_us` = unfused - chain (what the MXFP8 epilogue saves against a separate requantize)."""
    G, K, N, P = dims
    out = []
    for M in Ms:
        x = sweep_x(torch, M, G, K)
        set_bytes = x.numel() * 2 + w["wa_q"].numel() + w["wb_q"].numel()
        R = int(min(8, max(1, -(-ROTATE_BYTES // set_bytes))))
        sets = [{"x": x if r == 0 else x.clone(),
                 "wa_q": w["wa_q"].clone(), "wa_sf": w["wa_sf"].clone(),
                 "wb_q": w["wb_q"].clone(), "wb_sf": w["wb_sf"].clone()} for r in range(R)]
        graphs = {}
        for arm in ("chain", "x_fused", "unfused"):
            # one graph with the chain once per rotating set, in a row (as consecutive layers)
            g = torch.cuda.CUDAGraph()
            with torch.cuda.stream(stream):
                for s in sets:
                    L.o_proj_chain(s["x"], s["wa_q"], s["wa_sf"], s["wb_q"], s["wb_sf"], mode=arm, stream=stream)
                stream.synchronize()
                with torch.cuda.graph(g, stream=stream):
                    for s in sets:
                        L.o_proj_chain(s["x"], s["wa_q"], s["wa_sf"], s["wb_q"], s["wb_sf"], mode=arm,
                                       stream=stream)
            graphs[arm] = g
        steps = max(6, min(args.steps, int(2e5 // max(1, M))))
        reps = max(2, -(-steps // R))
        timed = median_rounds(torch, graphs, stream, reps, ramp_s=0.1, calls_per_replay=R)
        del graphs
        res = {"M": M}
        for arm in ("chain", "x_fused", "unfused"):
            res[f"{arm}_us"] = timed[arm]["us"]
            res[f"{arm}_spread_us"] = timed[arm]["spread"]
        flop = sum(chain_flops(M, G, K, N, P).values())
        nb = chain_bytes(M, G, K, N, P)
        us = res["chain_us"]
        res["tflops"] = flop / (us * 1e-6) / 1e12
        res["hbm_frac"] = sum(nb.values()) / (us * 1e-6) / 1e9 / HBM_PEAK_GBS
        res["mfma_frac"] = res["tflops"] / FP8_PEAK_TFLOPS
        res["fusion_saving_us"] = res["unfused_us"] - us
        if M in kernel_ms:
            res["kernels_avg_us"] = kernel_times(torch, L, sets, M, stream, args)
            # traffic: the counters of the configuration with this token count (the prefill and long
            # configurations; same shapes and outlier rate, other seeds)
            wl = {4096: "prefill", 32768: "long"}.get(M)
            res["roofline"] = {k: roofline_block(k, M, G, K, N, P, res["kernels_avg_us"][KERNEL_NAMES[k]],
                                                 recorded_traffic(wl, k) if wl else None)
                               for k in ("einsum", "gemm")}
        print(f"[bench] sweep M={M}: chain {us:.2f} us (spread {res['chain_spread_us']:.2f}), x_fused "
              f"{res['x_fused_us']:.2f} us, unfused {res['unfused_us']:.2f} us, {res['tflops']:.1f} TFLOP/s",
              file=sys.stderr, flush=True)
        out.append(res)
        del sets, x
        torch.cuda.empty_cache()
    return out


def kernel_times(torch, L, sets, M, stream, args):
    """Average µs per launch of each kernel of the chain at M tokens: one graph per kernel holding that launch
    at least 16 times over the rotating sets, timed as the median of three rounds."""
    G, N, K = sets[0]["wa_q"].shape
    P = sets[0]["wb_q"].shape[0]
    dev = sets[0]["x"].device
    inter = {"x_q": torch.empty((M, G * K), dtype=torch.uint8, device=dev),
             "x_sf": torch.empty((M, G * K // 128), dtype=torch.int32, device=dev),
             "z_q": torch.empty((M, G * N), dtype=torch.uint8, device=dev),
             "z_sf": torch.empty((M, G * N // 128), dtype=torch.int32, device=dev),
             "out": torch.empty((M, P), dtype=torch.bfloat16, device=dev)}

    def one(kind, s):
        if kind == "quantize":
            L.mxfp8_quantize(s["x"], q=inter["x_q"], sf=inter["x_sf"], stream=stream)
        elif kind == "einsum":
            L.grouped_fp8_einsum(inter["x_q"], inter["x_sf"], s["wa_q"], s["wa_sf"], out="mxfp8", z_q=inter["z_q"],
                                 z_sf=inter["z_sf"], stream=stream)
        else:
            L.fp8_gemm_nt(inter["z_q"], inter["z_sf"], s["wb_q"], s["wb_sf"], d=inter["out"], stream=stream)

    R = len(sets)
    reps = max(1, -(-16 // R))
    graphs = {}
    for kind in ("quantize", "einsum", "gemm"):
        g = torch.cuda.CUDAGraph()
        with torch.cuda.stream(stream):
            for s in sets:
                one(kind, s)
            stream.synchronize()
            with torch.cuda.graph(g, stream=stream):
                for _ in range(reps):
                    for s in sets:
                        one(kind, s)
        torch.cuda.synchronize()
        graphs[kind] = g
    n = max(2, min(args.steps, 200) // (reps * R))
    timed = median_rounds(torch, graphs, stream, n, ramp_s=0.1, calls_per_replay=reps * R)
    return {KERNEL_NAMES[k]: v["us"] for k, v in timed.items()}


def quant_sweep(torch, L, si, stream, args):
    """Standalone mxfp8_quantize over the quantize-sweep rows (BF16 [M, 7168] -> E4M3 + packed scales):
    µs/launch from a graph of at least 16 launches over rotating inputs, and the HBM roofline fraction
    of its 3.03125 bytes per element."""
    out = []
    K = si.QUANT_SWEEP_K
    for M in si.QUANT_SWEEP_M:
        x0 = torch.from_numpy(np.ascontiguousarray(si.quant_sweep_input(M)).view(np.int16)).view(
            torch.bfloat16).to("cuda")
        R = int(min(8, max(1, -(-ROTATE_BYTES // (x0.numel() * 3)))))
        xs = [x0 if r == 0 else x0.clone() for r in range(R)]
        qs = [torch.empty((M, K), dtype=torch.uint8, device="cuda") for _ in range(R)]
        sfs = [torch.empty((M, K // 128), dtype=torch.int32, device="cuda") for _ in range(R)]
        reps = max(1, -(-16 // R))
        g = torch.cuda.CUDAGraph()
        with torch.cuda.stream(stream):
            for r in range(R):
                L.mxfp8_quantize(xs[r], q=qs[r], sf=sfs[r], stream=stream)
            stream.synchronize()
            with torch.cuda.graph(g, stream=stream):
                for _ in range(reps):
                    for r in range(R):
                        L.mxfp8_quantize(xs[r], q=qs[r], sf=sfs[r], stream=stream)
        torch.cuda.synchronize()
        n = max(2, min(args.steps, 200) // (reps * R))
        us = time_arm_graphs(torch, [g], stream, n, 1) / (reps * R)
        nbytes = M * K * (2 + 1) + M * (K // 32)
        out.append({"M": M, "K": K, "us_per_launch": us, "hbm_frac": nbytes / (us * 1e-6) / 1e9 / HBM_PEAK_GBS})
        print(f"[bench] quantize sweep M={M}: {us:.2f} us/launch", file=sys.stderr, flush=True)
        del g, xs, qs, sfs, x0
        torch.cuda.empty_cache()
    return out


def producer_sweep(torch, L, si, stream, args):
    """The RMS-normalizing MXFP8 producer (mxfp8_rmsnorm_quantize) over the quantize-sweep rows
    (BF16 [M, 7168]), with and without its BF16 output, next to the unfused pair it replaces (the producer
    writing BF16 y only, then a standalone mxfp8_quantize of y) and the standalone quantize alone.  µs/launch from graphs of >= 16 launches over rotating
    inputs; HBM roofline fraction of the algorithmic bytes (x read once, codes + scales written, the BF16 y
    when written; gamma is 14 KB, read from cache)."""
    out = []
    K = si.QUANT_SWEEP_K
    g = torch.from_numpy(si.rmsnorm_gamma(K).view(np.int16)).view(torch.bfloat16).to("cuda")
    for M in si.QUANT_SWEEP_M:
        x0 = torch.from_numpy(np.ascontiguousarray(si.quant_sweep_input(M)).view(np.int16)).view(
            torch.bfloat16).to("cuda")
        R = int(min(8, max(1, -(-ROTATE_BYTES // (x0.numel() * 5)))))
        xs = [x0 if r == 0 else x0.clone() for r in range(R)]
        ys = [torch.empty((M, K), dtype=torch.bfloat16, device="cuda") for _ in range(R)]
        qs = [torch.empty((M, K), dtype=torch.uint8, device="cuda") for _ in range(R)]
        sfs = [torch.empty((M, K // 128), dtype=torch.int32, device="cuda") for _ in range(R)]
        reps = max(1, -(-16 // R))
        arms = {
            "fused": lambda r: L.mxfp8_rmsnorm_quantize(xs[r], g, 1e-6, q=qs[r], sf=sfs[r], stream=stream),
            "fused_bf16_out": lambda r: L.mxfp8_rmsnorm_quantize(xs[r], g, 1e-6, y=ys[r], q=qs[r], sf=sfs[r],
                                                                  stream=stream),
            "quantize_only": lambda r: L.mxfp8_quantize(xs[r], q=qs[r], sf=sfs[r], stream=stream),
            # the arrangement the fusion replaces: the producer writes BF16 y, a standalone quantize reads it
            "unfused": lambda r: (L.mxfp8_rmsnorm_quantize(xs[r], g, 1e-6, mxfp8_out=False, y=ys[r], stream=stream),
                                  L.mxfp8_quantize(ys[r], q=qs[r], sf=sfs[r], stream=stream)),
        }
        res = {"M": M, "K": K}
        for name, fn in arms.items():
            gr = torch.cuda.CUDAGraph()
            with torch.cuda.stream(stream):
                for r in range(R):
                    fn(r)
                stream.synchronize()
                with torch.cuda.graph(gr, stream=stream):
                    for _ in range(reps):
                        for r in range(R):
                            fn(r)
            torch.cuda.synchronize()
            n = max(2, min(args.steps, 200) // (reps * R))
            us = time_arm_graphs(torch, [gr], stream, n, 1) / (reps * R)
            nbytes = M * K * 2 + M * K + M * (K // 32) + (M * K * 2 if name == "fused_bf16_out" else 0) + (
                M * K * 4 if name == "unfused" else 0)                 # unfused: BF16 y written and read back
            res[f"{name}_us"] = us
            res[f"{name}_hbm_frac"] = nbytes / (us * 1e-6) / 1e9 / HBM_PEAK_GBS
            del gr
        res["fusion_saving_us"] = res["unfused_us"] - res["fused_bf16_out_us"]
        print(f"[bench] producer sweep M={M}: fused {res['fused_us']:.2f} us, with BF16 out "
              f"{res['fused_bf16_out_us']:.2f} us, unfused {res['unfused_us']:.2f} us, quantize alone "
              f"{res['quantize_only_us']:.2f} us", file=sys.stderr, flush=True)
        out.append(res)
        del xs, ys, qs, sfs, x0
        torch.cuda.empty_cache()
    return out


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--config", default="decode")
    ap.add_argument("--tokens", type=int, default=None,
                    help="run the configuration's shapes, seed and outlier rate at this many tokens instead (the "
                         "workload is then named CONFIG_M<tokens>, e.g. for kernel traces and counters)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--arms", default="chain,x_fused,unfused")
    ap.add_argument("--sweep", default=DEFAULT_SWEEP,
                    help="comma-separated token counts: also time the chain, x_fused and unfused arms at each "
                         "(decode-config weights, x drawn on the device) and report them under 'sweep' "
                         "('' for none)")
    ap.add_argument("--no-sweep", dest="sweep", action="store_const", const="",
                    help="leave the chain sweep out (same as --sweep '')")
    ap.add_argument("--quant-sweep", action=argparse.BooleanOptionalAction, default=True,
                    help="also time the standalone quantizer on the quantize-sweep rows (M x 7168)")
    ap.add_argument("--producer-sweep", action=argparse.BooleanOptionalAction, default=True,
                    help="also time the RMS-normalizing MXFP8 producer on the quantize-sweep rows (M x 7168), "
                         "next to the standalone quantizer it replaces")
    ap.add_argument("--cpu-long", action="store_true",
                    help="also time the oracle chain once on all 32768 rows of the long configuration, in blocks "
                         "of 1024 rows (several minutes of CPU work; off by default)")
    ap.add_argument("--copy-mib", type=int, default=0,
                    help="only run a device-to-device copy of this many MiB 5 times (HBM counter calibration)")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only (asked for --gpus {args.gpus}); the chain shards by token rows "
              f"with no exchange, so N GPUs run N independent copies of this measurement.", file=sys.stderr)
        sys.exit(2)

    import torch

    if args.copy_mib:
        copy_calibration(torch, args.copy_mib)
        return

    import synth_inputs as si
    import mxfp8_activation_quantization_amd as L

    L.device_check()
    cfg = si.CHAIN_CONFIGS[args.config]
    S = cfg.shape
    wname = args.config
    if args.tokens is not None:
        if args.tokens < 1:
            raise SystemExit("--tokens must be at least 1")
        S = si.ChainShape(args.tokens, S.G, S.K, S.N, S.P)
        wname = f"{args.config}_M{args.tokens}"
    M, G, K, N, P = S.M, S.G, S.K, S.N, S.P
    dev = torch.device("cuda", 0)
    print(f"[bench] config {wname}: M={M} G={G} K={K} N={N} P={P}; generating inputs", file=sys.stderr,
          flush=True)
    inp = si.chain_inputs(S, cfg.seed, cfg.outlier_rate)

    def to_dev(bits):
        return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).to(dev)

    x0 = to_dev(inp["x"])
    wa_q0, wa_sf0 = L.quantize_weight(to_dev(inp["wo_a"]))
    wb_q0, wb_sf0 = L.quantize_weight(to_dev(inp["wo_b"]))
    set_bytes = x0.numel() * 2 + wa_q0.numel() + wb_q0.numel()
    R = int(min(8, max(1, -(-ROTATE_BYTES // set_bytes))))

    # Inputs and weights rotate over R sets (as consecutive layers: each layer's weights are cold);
    # the intermediates (x_q, z, output) are one set of buffers that every layer reuses, as a
    # model's activation buffers are -- and as the x_fused and unfused arms get them from the
    # allocator inside the captured graph.
    inter = {
        "x_q": torch.empty((M, G * K), dtype=torch.uint8, device=dev),
        "x_sf": torch.empty((M, G * K // 128), dtype=torch.int32, device=dev),
        "z_q": torch.empty((M, G * N), dtype=torch.uint8, device=dev),
        "z_sf": torch.empty((M, G * N // 128), dtype=torch.int32, device=dev),
        "out": torch.empty((M, P), dtype=torch.bfloat16, device=dev),
    }
    sets = []
    for r in range(R):
        s = {
            "x": x0 if r == 0 else x0.clone(),
            "wa_q": wa_q0 if r == 0 else wa_q0.clone(), "wa_sf": wa_sf0 if r == 0 else wa_sf0.clone(),
            "wb_q": wb_q0 if r == 0 else wb_q0.clone(), "wb_sf": wb_sf0 if r == 0 else wb_sf0.clone(),
            **inter,
        }
        sets.append(s)
    torch.cuda.synchronize()

    stream = torch.cuda.Stream()

    def launch_chain(s, ev=None):
        """The headline chain into preallocated buffers; optional events around each launch."""
        if ev is not None:
            ev[0].record(stream)
        L.mxfp8_quantize(s["x"], q=s["x_q"], sf=s["x_sf"], stream=stream)
        if ev is not None:
            ev[1].record(stream)
        L.grouped_fp8_einsum(s["x_q"], s["x_sf"], s["wa_q"], s["wa_sf"], out="mxfp8", z_q=s["z_q"], z_sf=s["z_sf"],
                             stream=stream)
        if ev is not None:
            ev[2].record(stream)
        L.fp8_gemm_nt(s["z_q"], s["z_sf"], s["wb_q"], s["wb_sf"], d=s["out"], stream=stream)
        if ev is not None:
            ev[3].record(stream)

    def launch_arm(arm, s):
        if arm == "chain":
            launch_chain(s)
        else:
            L.o_proj_chain(s["x"], s["wa_q"], s["wa_sf"], s["wb_q"], s["wb_sf"], mode=arm, stream=stream)

    def capture(arm):
        """One graph holding the chain once per rotating set, in a row (as consecutive layers)."""
        g = torch.cuda.CUDAGraph()
        with torch.cuda.stream(stream):
            for s in sets:
                launch_arm(arm, s)                      # warm: allocations of intermediate buffers
            stream.synchronize()
            with torch.cuda.graph(g, stream=stream):
                for s in sets:
                    launch_arm(arm, s)
        torch.cuda.synchronize()
        return g

    # The arms, each one graph of R chains, timed as the median of three rounds after a clock ramp (after the
    # idle host-side set-up the device's clocks take milliseconds of load to ramp up: the first arm timed
    # after a short warm-up read 10-15% slow), the arms interleaved within each round.
    arms = [a for a in args.arms.split(",") if a]
    graphs = {arm: capture(arm) for arm in arms}
    n_warm = max(1, -(-args.warmup // R))
    with torch.cuda.stream(stream):
        for g in graphs.values():
            for _ in range(n_warm):
                g.replay()
    torch.cuda.synchronize()
    timed = median_rounds(torch, graphs, stream, max(1, -(-args.steps // R)), calls_per_replay=R)
    del graphs
    results = {}
    for arm in arms:
        results[arm] = {"us_per_call": timed[arm]["us"], "rounds_us": timed[arm]["rounds"],
                        "spread_us": timed[arm]["spread"]}
        print(f"[bench] arm {arm}: {timed[arm]['us']:.2f} us/call (graph replay, median of "
              f"{len(timed[arm]['rounds'])} rounds, spread {timed[arm]['spread']:.2f})", file=sys.stderr,
              flush=True)

    # Per-kernel durations: each launch of the headline chain captured alone in one
    # graph, at least 16 times in a row over the rotating sets (inputs stay cold), and
    # the graph replayed and timed with HIP events on the launch stream -- the kernel's
    # own duration plus the small gap between graph nodes, comparable with a
    # profiler's kernel trace (one launch per graph would time the host's submission).
    t_k = {k: v for k, v in zip(("quantize", "einsum", "gemm"),
                                kernel_times(torch, L, sets, M, stream, args).values())}

    flops = chain_flops(M, G, K, N, P)
    nbytes = chain_bytes(M, G, K, N, P)
    total_flop = sum(flops.values())
    head = results.get("chain", next(iter(results.values())))
    us = head["us_per_call"]
    value = total_flop / (us * 1e-6) / 1e12

    dom = max(("einsum", "gemm"), key=lambda k: t_k[k])
    roof = roofline_block(dom, M, G, K, N, P, t_k[dom], recorded_traffic(wname, dom))

    line = {
        "metric": METRIC, "value": value, "unit": "TFLOP/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": us / 1e3, "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "mxfp8 (e4m3 x e4m3, fp32 accumulate)", "data": "synthetic",
        "config": {"workload": f"{wname}: o_proj chain (mxfp8_quantize -> grouped_fp8_einsum with MXFP8 "
                               f"epilogue -> fp8_gemm_nt), M={M} tokens, wo_a {G}x{K}->{N}, wo_b {G * N}->{P}",
                   "M": M, "G": G, "K": K, "N": N, "P": P, "seed": cfg.seed,
                   "x": "BF16 N(0,1)" + (f", {cfg.outlier_rate:g} of entries x100" if cfg.outlier_rate else ""),
                   "weights": "MXFP8 of BF16 N(0,0.02)", "rotating_sets": R, "timing": "HIP graph replay"},
        "us_per_call": us,
        "arms_us_per_call": {a: r["us_per_call"] for a, r in results.items()},
        "arms_rounds_us": {a: r["rounds_us"] for a, r in results.items()},
        "fusion_saving_us": (results["unfused"]["us_per_call"] - us) if "unfused" in results else None,
        "kernels_avg_us": {KERNEL_NAMES[k]: v for k, v in t_k.items()},
        "hbm_roofline_frac_chain": sum(nbytes.values()) / (us * 1e-6) / 1e9 / HBM_PEAK_GBS,
        "mfma_roofline_frac_chain": value / FP8_PEAK_TFLOPS,
        "roofline": roof,
        "kernel_source_hash": kernel_source_hash(),
    }
    if args.sweep:
        line["sweep"] = sweep(torch, L, [int(v) for v in args.sweep.split(",") if v], (G, K, N, P),
                              sets[0], stream, args)
        # the dominant kernel's roofline at the prefill (4096) and long (32768) token counts as well
        line["rooflines"] = {"decode": roof}
        for pt in line["sweep"]:
            if "roofline" in pt:
                name = {4096: "prefill", 32768: "long"}.get(pt["M"], f"M={pt['M']}")
                line["rooflines"][name] = max(pt["roofline"].values(), key=lambda r: r["avg_launch_us"])
    if args.quant_sweep:
        line["quant_sweep"] = quant_sweep(torch, L, si, stream, args)
    if args.producer_sweep:
        line["producer_sweep"] = producer_sweep(torch, L, si, stream, args)
    if not args.no_cpu_baseline and args.tokens is None:
        print("[bench] timing the CPU oracle", file=sys.stderr, flush=True)
        line["cpu_baseline"] = cpu_baseline(args.config, inp)
    if args.cpu_long:
        print("[bench] timing the CPU oracle on every row of the long configuration", file=sys.stderr, flush=True)
        line["cpu_long"] = cpu_long()
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
