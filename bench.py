"""Benchmark of the ternary weight-only linear layer on one MI355X.

Default workload (the headline metric): a Llama-3-8B decode pass at M = 1 -
32 layers x 7 ternary projections (q, k, v, o, gate, up, down), 1.66 GB of
packed codes resident in HBM, distinct seeded weights per layer, so every
step streams all weights from HBM (the set is 6.5x the 256 MB MALL).  One
step = one such pass (224 GEMV launches).  ``value`` is packed-weight bytes
per second over the timed steps.

Secondary (reported in the same line): the prefill GEMM at M = 4096 on the
Llama-3-8B MLP shapes (14336 x 4096 and 4096 x 14336) in fp16 and bf16,
TFLOP/s = 2MNK / time.

The ``cpu_baseline`` leg times the oracle (fp64 dequant + fp64 matmul) on
the host on a bounded sample of the same workload.

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--graph]
"""

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0        # MI355X HBM3E, published
MFMA_PEAK_TFLOPS = 2500.0    # MI355X dense fp16 / bf16 matrix peak, published


def log(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--layers", type=int, default=32)
    ap.add_argument("--graph", action="store_true", help="replay each step from a captured HIP graph")
    ap.add_argument("--fused", action="store_true", help="q,k,v and gate,up as one call each (N stacked)")
    ap.add_argument("--no-prefill", action="store_true")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--only", default="", help="profiling helper: 'decode' or 'prefill'")
    return ap.parse_args()


def ternary_bytes(M, N, K):
    """Algorithmic bytes of one ternary call: codes + scales + A + C."""
    return N * ((K + 3) // 4) + 2 * N + 2 * M * K + 2 * M * N


def layer_shapes(fused):
    """Projections of one Llama-3-8B layer; fused = q,k,v and gate,up stacked along N
    (one call each, as a serving stack lays them out)."""
    import synth
    if not fused:
        return list(synth.LLAMA3_8B.items())
    s = synth.LLAMA3_8B
    return [("qkv", (s["q"][0] + s["k"][0] + s["v"][0], 4096)), ("o", s["o"]),
            ("gate_up", (2 * s["gate"][0], 4096)), ("down", s["down"])]


def build_decode(layers, dev, fused=False):
    import torch
    import bit_weight_only_tq_amd as tq
    import synth
    mats = []
    t0 = time.time()
    for layer in range(layers):
        for name, (N, K) in layer_shapes(fused):
            W = synth.weights_device(N, K, synth.seed_for("bench8b", layer, name), dev)
            codes, scale = tq.tq_pack(W)
            del W
            mats.append((name, N, K, codes, scale))
    torch.cuda.synchronize()
    log(f"packed {len(mats)} matrices in {time.time() - t0:.1f} s")
    return mats


def decode_step_fn(mats, xs, outs):
    import bit_weight_only_tq_amd as tq

    def step():
        for i, (name, N, K, codes, scale) in enumerate(mats):
            tq.tq_gemm(xs[K], codes, scale, out=outs[i])
    return step


def time_region(fn, steps, stream):
    import torch
    start = torch.cuda.Event(enable_timing=True)
    end = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    start.record(stream)
    for _ in range(steps):
        fn()
    end.record(stream)
    end.synchronize()
    return start.elapsed_time(end) / 1e3  # seconds


def per_launch_durations(mats, xs, outs, stream, reps=3):
    """Average device time of each GEMV launch, from HIP events recorded on
    the launch stream around every launch of `reps` full steps."""
    import torch
    import bit_weight_only_tq_amd as tq
    tot_t, tot_b, n = 0.0, 0, 0
    pairs = []
    for _ in range(reps):
        for i, (name, N, K, codes, scale) in enumerate(mats):
            e0 = torch.cuda.Event(enable_timing=True)
            e1 = torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            tq.tq_gemm(xs[K], codes, scale, out=outs[i])
            e1.record(stream)
            pairs.append((e0, e1, ternary_bytes(1, N, K)))
    torch.cuda.synchronize()
    for e0, e1, b in pairs:
        tot_t += e0.elapsed_time(e1) / 1e3
        tot_b += b
        n += 1
    return tot_t / n, tot_b / n, n


def bench_prefill(dev, iters=5):
    import torch
    import bit_weight_only_tq_amd as tq
    import synth
    res = {}
    M = 4096
    flops_tot, t_tot = 0.0, 0.0
    for (N, K) in [(14336, 4096), (4096, 14336)]:
        W = synth.weights_device(N, K, synth.seed_for("benchpf", N, K), dev)
        codes, scale = tq.tq_pack(W)
        del W
        for dt in ("f16", "bf16"):
            A = synth.activations_device(M, K, synth.seed_for("benchpfa", N, K, dt), dt, dev)
            C = torch.empty((M, N), dtype=A.dtype, device=dev)
            for _ in range(2):
                tq.tq_gemm(A, codes, scale, out=C)
            s = torch.cuda.current_stream()
            t = time_region(lambda: tq.tq_gemm(A, codes, scale, out=C), iters, s) / iters
            tf = 2.0 * M * N * K / t / 1e12
            res[f"{N}x{K}_{dt}"] = {"ms": round(t * 1e3, 4), "tflops": round(tf, 1)}
            if dt == "f16":
                flops_tot += 2.0 * M * N * K
                t_tot += t
            del A, C
    res["fp16_tflops_M4096"] = round(flops_tot / t_tot / 1e12, 1)
    res["frac_of_peak"] = round(flops_tot / t_tot / 1e12 / MFMA_PEAK_TFLOPS, 4)
    return res


def cpu_baseline():
    """The oracle, untuned, on one Llama-3-8B layer (7 projections) at M = 1:
    fp64 unpack + dequant of the packed codes, then the fp64 product."""
    import numpy as np
    import oracle.gemm as OG
    import oracle.ternary as OT
    import synth
    rng_seed = 7
    total_bytes, total_t = 0, 0.0
    for name, (N, K) in synth.LLAMA3_8B.items():
        W = synth.weights(N, K, synth.seed_for("cpu", name))
        codes, sb = OT.ternary_pack(W)
        a = synth.activations(1, K, rng_seed).double().numpy()
        t0 = time.perf_counter()
        wdq = OT.ternary_dequant(codes, sb, K)
        out, mag = OG.gemm_ref64(a, wdq)
        total_t += time.perf_counter() - t0
        total_bytes += codes.nbytes
        del W, wdq
    threads = None
    try:
        import threadpoolctl
        info = threadpoolctl.threadpool_info()
        threads = max((i.get("num_threads", 1) for i in info), default=1)
    except Exception:
        pass
    return {
        "value": round(total_bytes / total_t / 1e9, 3),
        "unit": "GB/s",
        "cores": threads or 1,
        "kind": "oracle",
        "sample": "one Llama-3-8B layer (q,k,v,o,gate,up,down; 52 MiB packed) at M=1, "
                  f"fp64 dequant + fp64 matmul, {total_t:.1f} s; host has {os.cpu_count()} CPUs",
    }


def main():
    args = parse()
    if args.gpus != 1:
        print(json.dumps({"error": "this build runs on exactly one GPU; --gpus must be 1"}))
        sys.exit(2)
    import torch
    import bit_weight_only_tq_amd as tq
    tq.load()
    if not torch.cuda.is_available():
        print(json.dumps({"error": "no GPU visible"}))
        sys.exit(1)
    dev = torch.device("cuda", 0)
    stream = torch.cuda.current_stream()

    out = {}
    if args.only in ("", "decode"):
        import synth
        mats = build_decode(args.layers, dev, args.fused)
        xs = {K: synth.activations_device(1, K, synth.seed_for("benchx", K), "f16", dev)
              for K in {m[2] for m in mats}}
        outs = [torch.empty((1, m[1]), dtype=torch.float16, device=dev) for m in mats]
        step = decode_step_fn(mats, xs, outs)
        packed = sum(m[3].numel() for m in mats)
        alg = sum(ternary_bytes(1, m[1], m[2]) for m in mats)
        if args.graph:
            g = torch.cuda.CUDAGraph()
            s2 = torch.cuda.Stream()
            s2.wait_stream(stream)
            with torch.cuda.stream(s2):
                step()
            stream.wait_stream(s2)
            torch.cuda.synchronize()
            with torch.cuda.graph(g):
                step()
            run = g.replay
        else:
            run = step
        for _ in range(args.warmup):
            run()
        torch.cuda.synchronize()
        log(f"timing {args.steps} steps")
        t = time_region(run, args.steps, stream)
        ms = t / args.steps * 1e3
        value = packed * args.steps / t / 1e9
        avg_dur, avg_bytes, nl = per_launch_durations(mats, xs, outs, stream)
        achieved = avg_bytes / avg_dur / 1e9
        out.update({
            "metric": "HBM GB/s (% peak) ternary GEMV at M=1; fp16-MFMA TFLOP/s at M=4096",
            "value": round(value, 1),
            "unit": "GB/s",
            "n_gpus": 1,
            "steps": args.steps,
            "warmup": args.warmup,
            "ms_per_step": round(ms, 4),
            "higher_is_better": True,
            "scaling": "weak",
            "vs_baseline": None,
            "dtype": "f16",
            "data": "synthetic (seeded N(0,0.02) weights ternarized on device, N(0,1) activations)",
            "config": {
                "workload": "Llama-3-8B decode, M=1: 32 layers x {q,k,v,o,gate,up,down} ternary GEMV",
                "layers": args.layers, "M": 1, "launches_per_step": len(mats),
                "packed_bytes_per_step": packed, "algorithmic_bytes_per_step": alg,
                "graph": bool(args.graph), "fused_qkv_gate_up": bool(args.fused),
                "hbm_frac": round(value / HBM_PEAK_GBS, 4),
            },
            "roofline": {
                "bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": None,
                "kernel": "ternary_gemv_mfma_kernel", "avg_launch_us": round(avg_dur * 1e6, 3),
                "avg_alg_bytes_per_launch": round(avg_bytes), "launches_timed": nl,
            },
        })
        del mats, xs, outs
        torch.cuda.empty_cache()
    if args.only in ("", "prefill") and not args.no_prefill:
        log("prefill GEMM M=4096")
        out["secondary"] = {"metric": "fp16-MFMA TFLOP/s at M=4096 (ternary prefill GEMM)",
                            **bench_prefill(dev)}
    if not args.no_cpu_baseline and args.only == "":
        log("cpu baseline (oracle)")
        out["cpu_baseline"] = cpu_baseline()
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
