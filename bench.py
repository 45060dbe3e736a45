"""Benchmark of the ternary weight-only linear layer on one MI355X.

Headline workload (``value``): Llama-3-8B decode at M = 1.  One step is one
pass over the linear layers of all 32 decoder layers, laid out as a serving
stack lays them out - q, k, v stacked along N into one call (6144 x 4096),
o (4096 x 4096), gate and up stacked into one call (28672 x 4096), down
(4096 x 14336) - 128 ternary GEMV launches, replayed from a HIP graph.  The
1.74 GB of packed codes (distinct seeded weights per layer) are resident in
HBM, 6.8x the 256 MB last-level cache, so every step streams them from HBM.
``value`` = packed-weight bytes per second over the timed steps.

Also reported in the same JSON line:
  * ``roofline``: algorithmic bytes (codes + scales + activations + outputs)
    per GEMV launch over the average launch time, both measured with HIP
    events around the timed region on the launch stream; HBM peak 8 TB/s.
    ``traffic`` is filled from rocprofv3 FETCH_SIZE / WRITE_SIZE runs (see
    profiles/) when given with --traffic-json.
  * ``decode_unfused``: the same pass with q, k, v, gate, up as separate
    calls (224 launches).
  * ``decode_70b``: Llama-3-70B decode at M = 1 - 80 layers x {qkv
    (10240 x 8192), o (8192 x 8192), gate_up (57344 x 8192), down
    (8192 x 28672)}, 320 launches per step over 17.1 GB of resident packed
    codes (one seeded layer packed on the device, copied to 80 layers).
  * ``secondary``: the prefill GEMM at M = 4096 on the MLP shapes
    (14336 x 4096, 4096 x 14336), fp16 and bf16, TFLOP/s = 2MNK / time.
  * ``w4a16_decode``: the Llama-3-8B decode step of the headline with
    W4A16 weights (group 128) at M = 1, 4 and 16, GB/s of packed codes +
    group scales.
  * ``medium_m``: the medium-M path (K split across workgroups) on one
    Llama-3-70B layer's four shapes at M = 32 and 64, eight resident copies
    rotated so that every call streams its codes from HBM.
  * ``cpu_baseline``: the CPU oracle (fp64 dequant + fp64 product), untuned,
    timed on the host on a bounded sample of the same workload.

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--mode MODE]
  --mode full (default) | decode | decodem | decode70b | w4 | medium | prefill | attrib | calib
  (plain copy of known size, for scaling hardware byte counters)
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
METRIC = "HBM GB/s (% peak) ternary GEMV at M=1; fp16-MFMA TFLOP/s at M=4096"


def log(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--layers", type=int, default=32)
    ap.add_argument("--mode", default="full",
                    choices=["full", "decode", "decodem", "decode70b", "w4", "w4act", "medium", "w4medium", "prefill", "w4prefill",
                             "attrib", "calib"])
    ap.add_argument("--no-graph", action="store_true", help="launch eagerly instead of replaying a HIP graph")
    ap.add_argument("--unfused", action="store_true", help="decode mode: q,k,v,gate,up as separate calls")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=10.0, help="lower bound on the CPU sample's run time")
    ap.add_argument("--settle", type=float, default=0.3,
                    help="seconds of untimed calls before each prefill line (counter passes use less: "
                         "every call is a profiled dispatch)")
    ap.add_argument("--traffic-json", default=os.path.join(ROOT, "profiles", "ternary_gemv_traffic.json"))
    return ap.parse_args()


def ternary_bytes(M, N, K):
    """Algorithmic bytes of one ternary call: codes + scales + A + C."""
    return N * ((K + 3) // 4) + 2 * N + 2 * M * K + 2 * M * N


def layer_shapes(fused, model="8b"):
    """Projections of one decoder layer (name, (N, K)); fused stacks q,k,v and gate,up along N."""
    import synth
    s = synth.LLAMA3_8B if model == "8b" else synth.LLAMA3_70B
    if not fused:
        return list(s.items())
    hidden = s["q"][1]
    return [("qkv", (s["q"][0] + s["k"][0] + s["v"][0], hidden)), ("o", s["o"]),
            ("gate_up", (s["gate"][0] + s["up"][0], hidden)), ("down", s["down"])]


def build_decode(layers, dev, fused, model="8b"):
    """Packed matrices of `layers` decoder layers, distinct seeded weights per
    layer and projection (drawn on the device, ternarized there)."""
    import torch
    import bit_weight_only_tq_amd as tq
    import synth
    mats = []
    t0 = time.time()
    for layer in range(layers):
        for name, (N, K) in layer_shapes(fused, model):
            W = synth.weights_device(N, K, synth.seed_for("bench" + model, layer, name), dev)
            codes, scale = tq.tq_pack(W)
            del W
            mats.append((name, N, K, codes, scale))
    torch.cuda.synchronize()
    log(f"packed {len(mats)} matrices in {time.time() - t0:.1f} s")
    return mats


SAMPLE_ROWS = 32      # weight rows per sampled matrix whose outputs the oracle re-computes
SAMPLE_M = 4          # activation rows sampled when M is larger


def sample_rows(n, k, seed):
    import numpy as np
    return np.sort(np.random.default_rng(seed).choice(n, size=min(k, n), replace=False))


def ternary_sample(line, A, C, codes, scale, seed):
    """Copy to the host what the oracle needs to re-compute a few outputs of a
    timed call: sampled weight rows (codes, scale bits), sampled activation
    rows, and the GPU outputs at those (row, column) pairs."""
    import numpy as np
    import torch
    N, K = codes.shape[0], A.shape[1]
    rows = sample_rows(N, SAMPLE_ROWS, seed)
    ms = sample_rows(A.shape[0], SAMPLE_M, seed + 1)
    ri = torch.from_numpy(rows).to(codes.device)
    mi = torch.from_numpy(ms).to(codes.device)
    return {"line": line, "kind": "ternary", "K": K, "dtype": "bf16" if A.dtype == torch.bfloat16 else "f16",
            "codes": codes.index_select(0, ri).cpu().numpy(),
            "scale": scale.index_select(0, ri).cpu().view(torch.int16).numpy().view(np.uint16),
            "A": A.index_select(0, mi).double().cpu().numpy(),
            "C": C.index_select(0, mi).index_select(1, ri).double().cpu().numpy()}


def w4_sample(line, A, C, q, sc, seed, zeros=None, perm=None):
    import numpy as np
    import torch
    N, K = q.shape[0], A.shape[1]
    rows = sample_rows(N, SAMPLE_ROWS, seed)
    ms = sample_rows(A.shape[0], SAMPLE_M, seed + 1)
    ri = torch.from_numpy(rows).to(q.device)
    mi = torch.from_numpy(ms).to(q.device)
    d = {"line": line, "kind": "w4", "K": K, "dtype": "bf16" if A.dtype == torch.bfloat16 else "f16",
         "q": q.index_select(0, ri).cpu().numpy(),
         "scale": sc.index_select(0, ri).cpu().view(torch.int16).numpy().view(np.uint16),
         "A": A.index_select(0, mi).double().cpu().numpy(),
         "C": C.index_select(0, mi).index_select(1, ri).double().cpu().numpy()}
    if zeros is not None or perm is not None:
        d["kind"] = "w4a"
        d["zeros"] = zeros.index_select(0, ri).cpu().numpy()
        d["perm"] = None if perm is None else perm.cpu().numpy()
    return d


def time_region(fn, steps, stream, per_step=None):
    """Seconds for `steps` calls of fn, from HIP events on `stream`.  With a
    list as `per_step`, an event is also recorded after every call and the
    per-call milliseconds are appended to it (the total is unchanged: it is
    still read from the first and last event)."""
    import torch
    start = torch.cuda.Event(enable_timing=True)
    end = torch.cuda.Event(enable_timing=True)
    marks = [torch.cuda.Event(enable_timing=True) for _ in range(steps - 1)] if per_step is not None else []
    torch.cuda.synchronize()
    start.record(stream)
    for i in range(steps):
        fn()
        if per_step is not None and i < steps - 1:
            marks[i].record(stream)
    end.record(stream)
    end.synchronize()
    if per_step is not None:
        edges = [start] + marks + [end]
        per_step.extend(a.elapsed_time(b) for a, b in zip(edges[:-1], edges[1:]))
    return start.elapsed_time(end) / 1e3


SETTLE_SECONDS = [0.3]  # set from --settle


def settle(fn, seconds=None):
    """Untimed calls of fn for at least `seconds` of wall clock, ending with a
    synchronize.  The part raises its shader clock only after some tens of
    milliseconds of sustained load: a compute-bound line timed straight after
    idle host work (packing, the previous line's checks) would catch the
    ramp and report less than the sustained rate a serving loop sees."""
    import torch
    seconds = SETTLE_SECONDS[0] if seconds is None else seconds
    t0 = time.perf_counter()
    while True:
        for _ in range(4):
            fn()
        torch.cuda.synchronize()
        if time.perf_counter() - t0 >= seconds:
            return


def percentiles(ms):
    """p10 / p50 / p90 of a list of per-step milliseconds."""
    v = sorted(ms)
    pick = lambda f: v[min(len(v) - 1, int(round(f * (len(v) - 1))))]  # noqa: E731
    return {"p10": round(pick(0.1), 4), "p50": round(pick(0.5), 4), "p90": round(pick(0.9), 4)}


def run_decode(args, dev, fused, graph, model="8b", layers=None, steps=None, M=1, dt="f16", line=None, samples=None,
               mats=None):
    import torch
    import bit_weight_only_tq_amd as tq
    import synth
    stream = torch.cuda.current_stream()
    layers = args.layers if layers is None else layers
    steps = args.steps if steps is None else steps
    own = mats is None
    if own:
        mats = build_decode(layers, dev, fused, model)
    xs = {K: synth.activations_device(M, K, synth.seed_for("benchx", K, M), dt, dev) for K in {m[2] for m in mats}}
    odt = torch.float16 if dt == "f16" else torch.bfloat16
    outs = [torch.empty((M, m[1]), dtype=odt, device=dev) for m in mats]
    # one workspace for every call of the step (they run in stream order), its
    # arrival counters zeroed once, as a serving loop would hold it
    ws = tq.new_workspace(max(tq.tq_gemm_workspace_bytes(M, m[1], m[2], dt) for m in mats), dev)

    def step():
        for i, (name, N, K, codes, scale) in enumerate(mats):
            tq.tq_gemm(xs[K], codes, scale, out=outs[i], workspace=ws)

    run = step
    if graph:
        g = torch.cuda.CUDAGraph()
        side = torch.cuda.Stream()
        side.wait_stream(stream)
        with torch.cuda.stream(side):
            step()
        stream.wait_stream(side)
        torch.cuda.synchronize()
        with torch.cuda.graph(g):
            step()
        run = g.replay
    for _ in range(args.warmup):
        run()
    torch.cuda.synchronize()
    step_ms = []
    t = time_region(run, steps, stream, per_step=step_ms)
    torch.cuda.synchronize()
    if samples is not None:  # the first and the last layer's outputs of the timed steps
        nl = len(layer_shapes(fused, model))
        for i in list(range(nl)) + list(range(len(mats) - nl, len(mats))):
            name, N, K, codes, scale = mats[i]
            samples.append(ternary_sample(line, xs[K], outs[i], codes, scale, synth.seed_for("bs", line, i)))
    packed = sum(m[3].numel() for m in mats)
    alg = sum(ternary_bytes(M, m[1], m[2]) for m in mats)
    res = {
        "launches": len(mats), "seconds": t, "packed_bytes": packed, "alg_bytes": alg,
        "ms_per_step": t / steps * 1e3, "packed_gbs": packed * steps / t / 1e9,
        "alg_gbs": alg * steps / t / 1e9,
        "avg_launch_us": t / steps / len(mats) * 1e6, "alg_bytes_per_launch": alg / len(mats),
        "step_ms": percentiles(step_ms),
    }
    if own:
        del mats
    del xs, outs
    if graph:
        del g
    torch.cuda.empty_cache()
    return res


def w4_bytes(M, N, K):
    """Algorithmic bytes of one W4A16 call: codes + group scales + A + C."""
    return N * K // 2 + 2 * N * (K // 128) + 2 * M * K + 2 * M * N


def w4_act_bytes(M, N, K):
    """Algorithmic bytes of one W4A16 call with zero points and activation
    order: codes + group scales + zero points + A + the gathered A (written
    once, read once) + C."""
    return w4_bytes(M, N, K) + N * (K // 128) + 4 * M * K


def run_w4_decode(args, dev, Ms=(1, 4, 16), act_order=False, dt="f16", samples=None):
    """Llama-3-8B decode step with W4A16 weights, fused layout, graph replay;
    act_order: zero points and activation-order groups (gather + kernel)."""
    import torch
    import bit_weight_only_tq_amd as tq
    import synth
    stream = torch.cuda.current_stream()
    mats = []
    for layer in range(args.layers):
        for name, (N, K) in layer_shapes(True):
            W = synth.weights_device(N, K, synth.seed_for("benchw4", layer, name), dev)
            if act_order:
                gi = torch.from_numpy(synth.group_index(K, synth.seed_for("benchw4g", layer, name))).to(dev)
                q, sc, zp, perm = tq.w4a16_pack_asym(W, gi)
            else:
                (q, sc), zp, perm = tq.w4a16_pack(W), None, None
            del W
            mats.append((N, K, q, sc, zp, perm))
    torch.cuda.synchronize()
    packed = sum(m[2].numel() * 4 + m[3].numel() * 2 + (m[4].numel() if act_order else 0) for m in mats)
    what = "W4A16 with zero points and activation order" if act_order else "W4A16"
    what += ", bf16 activations" if dt == "bf16" else ""
    res = {"metric": f"HBM GB/s {what} GEMV, Llama-3-8B decode (32 layers, fused qkv / gate_up)",
           "unit": "GB/s", "packed_bytes_per_step": packed, "launches_per_step": len(mats)}
    for M in Ms:
        xs = {K: synth.activations_device(M, K, synth.seed_for("benchw4x", K, M), dt, dev) for K in {m[1] for m in mats}}
        odt = torch.float16 if dt == "f16" else torch.bfloat16
        outs = [torch.empty((M, m[0]), dtype=odt, device=dev) for m in mats]
        # one workspace for every call (they run in order on one stream), its
        # arrival counters zeroed once
        if act_order:
            nb = max(tq.w4a16_gemm_asym_workspace_bytes(M, m[0], m[1], dt, with_perm=True) for m in mats)
        else:
            nb = max(tq.w4a16_gemm_workspace_bytes(M, m[0], m[1], dt) for m in mats)
        ws = tq.new_workspace(nb, dev)

        def step():
            for i, (N, K, q, sc, zp, perm) in enumerate(mats):
                if act_order:
                    tq.w4a16_gemm(xs[K], q, sc, out=outs[i], zeros=zp, perm=perm, workspace=ws)
                else:
                    tq.w4a16_gemm(xs[K], q, sc, out=outs[i], workspace=ws)

        g = torch.cuda.CUDAGraph()
        side = torch.cuda.Stream()
        side.wait_stream(stream)
        with torch.cuda.stream(side):
            step()
        stream.wait_stream(side)
        torch.cuda.synchronize()
        with torch.cuda.graph(g):
            step()
        for _ in range(args.warmup):
            g.replay()
        t = time_region(g.replay, args.steps, stream)
        torch.cuda.synchronize()
        if samples is not None:
            line = f"w4{'_act' if act_order else ''}_{dt}_M{M}"
            for i in (0, 1, 2, 3, len(mats) - 4, len(mats) - 3, len(mats) - 2, len(mats) - 1):
                N, K, q, sc, zp, perm = mats[i]
                samples.append(w4_sample(line, xs[K], outs[i], q, sc, synth.seed_for("bsw", line, i), zp, perm))
        alg = sum((w4_act_bytes if act_order else w4_bytes)(M, m[0], m[1]) for m in mats)
        res[f"M{M}"] = {"value": round(packed * args.steps / t / 1e9, 1),
                        "frac_of_peak": round(packed * args.steps / t / 1e9 / HBM_PEAK_GBS, 4),
                        "ms_per_step": round(t / args.steps * 1e3, 4),
                        "avg_launch_us": round(t / args.steps / len(mats) * 1e6, 3),
                        "alg_gbs": round(alg * args.steps / t / 1e9, 1)}
        del g, xs, outs, ws
    del mats
    torch.cuda.empty_cache()
    return res


def run_w4_medium(dev, copies=4, iters=16, samples=None):
    """W4A16 at medium M on one Llama-3-70B layer, M = 32 and 64 (the
    matrix-core GEMM's 64-row tiles with split K), and the decode kernels
    over 16-row blocks beside it for comparison."""
    import torch
    import bit_weight_only_tq_amd as tq
    import synth
    stream = torch.cuda.current_stream()
    res = {"metric": "W4A16 medium-M path, one Llama-3-70B layer", "unit": "us per call",
           "kernel": "w4p::gemm_kernel<T, ASYM, 64> + mm::splitk_reduce_kernel"}
    ws = tq.new_workspace(64 << 20, dev)
    for name, (N, K) in layer_shapes(True, "70b"):
        W = synth.weights_device(N, K, synth.seed_for("benchw4m", name), dev)
        q, s = tq.w4a16_pack(W)
        del W
        reps = [(q, s)] + [(q.clone(), s.clone()) for _ in range(copies - 1)]
        for M in (32, 64):
            A = synth.activations_device(M, K, synth.seed_for("benchw4ma", N, K, M), "f16", dev)
            C = torch.empty((M, N), dtype=torch.float16, device=dev)
            entry = {}
            for path in ("gemm", "gemv"):
                calls = [lambda qq=qq, ss=ss: tq.w4a16_gemm(A, qq, ss, out=C, workspace=ws, path=path)
                         for qq, ss in reps]
                for c in calls:
                    c()
                t = time_region(lambda: [c() for c in calls], iters, stream) / (iters * copies)
                torch.cuda.synchronize()
                if path == "gemm":
                    if samples is not None:  # C holds the last copy's output
                        samples.append(w4_sample(f"w4_medium_M{M}", A, C, reps[-1][0], reps[-1][1],
                                                 synth.seed_for("bw4m", name, M)))
                    flops = 2.0 * M * N * K
                    alg = w4_bytes(M, N, K)
                    roof_s = max(alg / (HBM_PEAK_GBS * 1e9), flops / (MFMA_PEAK_TFLOPS * 1e12))
                    entry.update({"us": round(t * 1e6, 2), "tflops": round(flops / t / 1e12, 1),
                                  "packed_gbs": round(q.numel() * 4 / t / 1e9, 1), "roof_us": round(roof_s * 1e6, 2),
                                  "frac_of_roof": round(roof_s / t, 4)})
                else:
                    entry["row_blocks_us"] = round(t * 1e6, 2)
            res[f"{name}_{N}x{K}_M{M}"] = entry
            del A, C
        del reps, q, s
    torch.cuda.empty_cache()
    return res


def run_medium(dev, copies=8, iters=16, samples=None):
    """Medium-M path on one Llama-3-70B layer at M = 32, 64 (split K)."""
    import torch
    import bit_weight_only_tq_amd as tq
    import synth
    stream = torch.cuda.current_stream()
    res = {"metric": "ternary medium-M path (K split across workgroups), one Llama-3-70B layer",
           "kernel": "mm3::tile_kernel (fp16, K % 256 == 0) + mm::splitk_reduce_kernel; "
                     "mm3::pair_activations_kernel first where N K >= 200 * 2^20"}
    for name, (N, K) in layer_shapes(True, "70b"):
        W = synth.weights_device(N, K, synth.seed_for("benchmm", name), dev)
        codes, scale = tq.tq_pack(W)
        del W
        reps = [(codes, scale)] + [(codes.clone(), scale.clone()) for _ in range(copies - 1)]
        for M in (32, 64):
            A = synth.activations_device(M, K, synth.seed_for("benchmma", N, K, M), "f16", dev)
            C = torch.empty((M, N), dtype=torch.float16, device=dev)
            nbytes = tq.tq_gemm_workspace_bytes(M, N, K)
            # the library pairs the activations once per call into the
            # workspace (after the split partials) when N K >= 200 * 2^20
            pair_b = M * K * 2 if K % 256 == 0 and N * K >= (200 << 20) else 0
            ws = tq.new_workspace(nbytes, dev)
            calls = [lambda c=c, s_=s_: tq.tq_gemm(A, c, s_, out=C, workspace=ws) for c, s_ in reps]
            for c in calls:
                c()
            t = time_region(lambda: [c() for c in calls], iters, stream) / (iters * copies)
            torch.cuda.synchronize()
            if samples is not None:  # C holds the last copy's output
                samples.append(ternary_sample(f"medium_M{M}", A, C, reps[-1][0], reps[-1][1],
                                              synth.seed_for("bsm", name, M)))
            flops = 2.0 * M * N * K
            alg = ternary_bytes(M, N, K)
            roof_s = max(alg / (HBM_PEAK_GBS * 1e9), flops / (MFMA_PEAK_TFLOPS * 1e12))  # min(BW * I, peak)
            res[f"{name}_{N}x{K}_M{M}"] = {"us": round(t * 1e6, 2), "tflops": round(flops / t / 1e12, 1),
                                           "packed_gbs": round(codes.numel() / t / 1e9, 1),
                                           "roof_us": round(roof_s * 1e6, 2), "frac_of_roof": round(roof_s / t, 4),
                                           "splits": max(1, (nbytes - tq.TQ_WORKSPACE_FLAG_BYTES - pair_b) // (4 * M * N)),
                                           "paired_activations": pair_b > 0}
            del A, C, ws
        del reps, codes, scale
    torch.cuda.empty_cache()
    return res


def run_decode_m(args, dev, graph, Ms=(4, 16), dt="f16", samples=None, ceiling_ms=None):
    """Llama-3-8B ternary decode step (32 layers, fused qkv / gate_up) at
    several activation rows M."""
    res = {"metric": f"HBM GB/s ternary GEMV, Llama-3-8B decode (32 layers, fused qkv / gate_up), {dt} activations",
           "unit": "GB/s"}
    for M in Ms:
        d = run_decode(args, dev, True, graph, M=M, dt=dt, line=f"decode_{dt}_M{M}", samples=samples)
        res[f"M{M}"] = {"value": round(d["packed_gbs"], 1), "frac_of_peak": round(d["packed_gbs"] / HBM_PEAK_GBS, 4),
                        "ms_per_step": round(d["ms_per_step"], 4), "step_ms_percentiles": d["step_ms"],
                        "avg_launch_us": round(d["avg_launch_us"], 3), "alg_gbs": round(d["alg_gbs"], 1)}
        if ceiling_ms:
            res[f"M{M}"]["frac_of_ceiling"] = round(ceiling_ms / d["ms_per_step"], 4)
    return res


def capture(fn, stream):
    """fn's launches recorded into a HIP graph (warmed up once on a side
    stream first); returns the graph's replay."""
    import torch
    g = torch.cuda.CUDAGraph()
    side = torch.cuda.Stream()
    side.wait_stream(stream)
    with torch.cuda.stream(side):
        fn()
    stream.wait_stream(side)
    torch.cuda.synchronize()
    with torch.cuda.graph(g):
        fn()
    return g


def run_ceiling(dev, sizes, reps=2):
    """Measured HBM read ceiling: for each byte count, a plain streaming read
    of that many bytes per launch (tq_diag_stream_read), back-to-back in a
    graph over copies cycled through >= 2 GiB (8x the 256 MB last-level
    cache), with the workgroup count swept; the fastest launch time is the
    ceiling any kernel reading that many bytes per launch can reach here.
    Returns {bytes: us per launch}."""
    import torch
    import bit_weight_only_tq_amd as tq
    stream = torch.cuda.current_stream()
    cus = torch.cuda.get_device_properties(dev).multi_processor_count
    out = {}
    for nb in sorted(set(sizes)):
        copies = max(2, -(-(2 << 30) // nb))
        buf = torch.empty((copies * nb,), dtype=torch.uint8, device=dev)
        views = [buf[i * nb:(i + 1) * nb] for i in range(copies)]
        sink = torch.empty((16 * cus,), dtype=torch.int32, device=dev)
        best = float("inf")
        for blocks in (cus, 2 * cus, 4 * cus, 8 * cus, 16 * cus):
            if blocks > nb // 16:
                continue
            g = capture(lambda: [tq.tq_diag_stream_read(v, blocks, sink) for v in views], stream)
            g.replay()
            best = min(best, time_region(g.replay, reps, stream) / (reps * copies))
            del g
        out[nb] = best * 1e6
        del views, buf, sink
        torch.cuda.empty_cache()
    return out


def ceiling_step_ms(shapes_per_step, ceil_us):
    """Ceiling time of a decode step: the read ceiling of each launch's code bytes, summed."""
    return sum(ceil_us[N * K // 4] for (N, K) in shapes_per_step) / 1e3


def run_attrib(dev, ceil_us, reps=8):
    """Where an M = 1 decode call's time goes (Llama-3-8B fused shapes), from
    real runs of the decode kernel and its measurement variants
    (tq_diag_gemv), each a graph of back-to-back calls:
      hbm_us      variant 0, the kernel tq_gemm runs, codes streamed from
                  HBM (copies cycled over >= 2 GiB);
      cached_us   variant 1, every workgroup reads the first 16 rows' codes,
                  so they come from the cache: HBM time removed;
      unpack_us   variant 2, as 1 without the matrix-core multiply;
      floor_us    a launch of the plain streaming read over 16 KiB.
    Split: launch_us = floor; unpack_us - floor = loads from cache +
    activation prep + unpack + reduction; mac_us = cached - unpack;
    hbm_exposed_us = hbm - cached; read_ceiling_us = the plain read of the
    same bytes."""
    import torch
    import bit_weight_only_tq_amd as tq
    import synth
    stream = torch.cuda.current_stream()
    res = {"metric": "decode GEMV time split, Llama-3-8B shapes, M=1 (us per call)",
           "kernel": "ternary_gemv_m1_kernel and its measurement variants"}
    small = torch.empty((16 << 10,), dtype=torch.uint8, device=dev)
    sink = torch.empty((64,), dtype=torch.int32, device=dev)
    g = capture(lambda: [tq.tq_diag_stream_read(small, 64, sink) for _ in range(64)], stream)
    g.replay()
    floor = time_region(g.replay, reps, stream) / (reps * 64) * 1e6
    res["launch_floor_us"] = round(floor, 2)
    del g
    for name, (N, K) in layer_shapes(True):
        W = synth.weights_device(N, K, synth.seed_for("attr", N, K), dev)
        codes, scale = tq.tq_pack(W)
        del W
        nb = codes.numel()
        copies = max(2, -(-(2 << 30) // nb))
        buf = torch.empty((copies * nb,), dtype=torch.uint8, device=dev)
        views = [buf[i * nb:(i + 1) * nb].view(N, K // 4) for i in range(copies)]
        for v in views:
            v.copy_(codes)
        x = synth.activations_device(1, K, synth.seed_for("attrx", K), "f16", dev)
        out = torch.empty((1, N), dtype=torch.float16, device=dev)
        g_hbm = capture(lambda: [tq.tq_diag_gemv(x, v, scale, 0, out=out) for v in views], stream)
        g_hbm.replay()
        t_hbm = time_region(g_hbm.replay, 2, stream) / (2 * copies) * 1e6
        del g_hbm
        tv = {}
        for var in (1, 2):
            gv = capture(lambda: [tq.tq_diag_gemv(x, views[0], scale, var, out=out) for _ in range(64)], stream)
            gv.replay()
            tv[var] = time_region(gv.replay, reps, stream) / (reps * 64) * 1e6
            del gv
        res[f"{name}_{N}x{K}"] = {
            "hbm_us": round(t_hbm, 2), "cached_us": round(tv[1], 2), "unpack_only_us": round(tv[2], 2),
            "read_ceiling_us": round(ceil_us[nb], 2), "hbm_gbs": round(nb / t_hbm / 1e3, 1),
            "split_us": {"launch": round(floor, 2), "loads_prep_unpack_reduce": round(tv[2] - floor, 2),
                         "mac": round(tv[1] - tv[2], 2), "hbm_exposed": round(t_hbm - tv[1], 2)},
        }
        del views, buf, codes, scale
        torch.cuda.empty_cache()
    return res


def run_decode_70b(args, dev, samples=None, ceiling=None):
    """Llama-3-70B decode over 80 resident layers (17.1 GB of packed codes,
    distinct seeded weights per layer and projection) at M = 1, 32 and 64:
    the decode kernel at M = 1, the medium-M path above 16 rows."""
    import torch
    import synth
    mats = build_decode(synth.LLAMA3_70B_LAYERS, dev, True, "70b")
    res = {"metric": "HBM GB/s ternary GEMV at M=1, Llama-3-70B decode (80 layers resident)",
           "unit": "GB/s",
           "workload": "80 layers x {qkv (10240x8192), o (8192x8192), gate_up (57344x8192), down (8192x28672)}, "
                       "distinct seeded weights per layer and projection"}
    for M in (1, 32, 64):
        d = run_decode(args, dev, True, not args.no_graph, model="70b", layers=synth.LLAMA3_70B_LAYERS,
                       steps=max(2, args.steps // 2) if M == 1 else 3, M=M, line=f"decode70b_M{M}",
                       samples=samples, mats=mats)
        e = {"value": round(d["packed_gbs"], 1), "frac_of_peak": round(d["packed_gbs"] / HBM_PEAK_GBS, 4),
             "ms_per_step": round(d["ms_per_step"], 4), "step_ms_percentiles": d["step_ms"],
             "avg_launch_us": round(d["avg_launch_us"], 3), "launches_per_step": d["launches"],
             "packed_bytes_per_step": d["packed_bytes"],
             "tflops": round(2.0 * M * d["packed_bytes"] * 4 / (d["ms_per_step"] * 1e-3) / 1e12, 1)}
        if ceiling:
            e["frac_of_ceiling"] = round(ceiling / d["ms_per_step"], 4)
        if M == 1:
            res.update(e)
        else:
            res[f"M{M}"] = e
    del mats
    torch.cuda.empty_cache()
    return res


def run_prefill(dev, iters=10, samples=None):
    """Ternary prefill GEMM on the Llama-3-8B MLP shapes: M = 4096 in fp16 (the
    metric) and bf16, and bf16 at M = 2048 and 8192.  Beside it, as context only,
    the same products with dense fp16/bf16 weights through torch's F.linear
    (the vendor GEMM library), timed in the same process on the same inputs."""
    import torch
    import bit_weight_only_tq_amd as tq
    import synth
    res = {}
    flops_f16, t_f16 = 0.0, 0.0
    stream = torch.cuda.current_stream()
    points = [(4096, "f16"), (4096, "bf16"), (2048, "bf16"), (8192, "bf16")]
    for (N, K) in [(14336, 4096), (4096, 14336)]:
        W = synth.weights_device(N, K, synth.seed_for("benchpf", N, K), dev)
        codes, scale = tq.tq_pack(W)
        for M, dt in points:
            A = synth.activations_device(M, K, synth.seed_for("benchpfa", N, K, dt), dt, dev)
            C = torch.empty((M, N), dtype=A.dtype, device=dev)
            nbytes = tq.tq_gemm_workspace_bytes(M, N, K, dt)
            ws = tq.new_workspace(nbytes, dev)
            settle(lambda: tq.tq_gemm(A, codes, scale, out=C, workspace=ws))
            t = time_region(lambda: tq.tq_gemm(A, codes, scale, out=C, workspace=ws), iters, stream) / iters
            torch.cuda.synchronize()
            if samples is not None:
                samples.append(ternary_sample(f"prefill_{dt}_M{M}", A, C, codes, scale,
                                              synth.seed_for("bsp", N, K, M, dt)))
            entry = {"ms": round(t * 1e3, 4), "tflops": round(2.0 * M * N * K / t / 1e12, 1),
                     "splits": (nbytes - tq.TQ_WORKSPACE_FLAG_BYTES) // (4 * M * N) if nbytes else 1}
            if M == 4096:
                Wd = W.to(A.dtype)
                settle(lambda: torch.nn.functional.linear(A, Wd))
                td = time_region(lambda: torch.nn.functional.linear(A, Wd), iters, stream) / iters
                entry["dense_ref_tflops"] = round(2.0 * M * N * K / td / 1e12, 1)
                del Wd
            res[f"{N}x{K}_M{M}_{dt}"] = entry
            if M == 4096 and dt == "f16":
                flops_f16 += 2.0 * M * N * K
                t_f16 += t
            del A, C, ws
        del W, codes, scale
    tf = flops_f16 / t_f16 / 1e12
    return {"metric": "fp16-MFMA TFLOP/s at M=4096 (ternary prefill GEMM, Llama-3-8B MLP shapes)",
            "value": round(tf, 1), "unit": "TFLOP/s", "peak": MFMA_PEAK_TFLOPS,
            "frac_of_peak": round(tf / MFMA_PEAK_TFLOPS, 4), "kernel": "v3::gemm_kernel",
            "dense_ref": "torch.nn.functional.linear with dense weights of the same shape and dtype (context only)",
            **res}


def run_w4_prefill(dev, iters=10, samples=None):
    """W4A16 prefill GEMM on the Llama-3-8B MLP shapes: M = 2048 and 4096,
    fp16 and bf16 activations, symmetric format; zero points with
    activation order at M = 4096 fp16.  TFLOP/s = 2MNK / time."""
    import torch
    import bit_weight_only_tq_amd as tq
    import synth
    res = {"metric": "W4A16 prefill GEMM TFLOP/s (Llama-3-8B MLP shapes)", "unit": "TFLOP/s",
           "peak": MFMA_PEAK_TFLOPS, "kernel": "w4p::gemm_kernel"}
    stream = torch.cuda.current_stream()
    for (N, K) in [(14336, 4096), (4096, 14336)]:
        W = synth.weights_device(N, K, synth.seed_for("benchw4pf", N, K), dev)
        q, sc = tq.w4a16_pack(W)
        gi = torch.from_numpy(synth.group_index(K, synth.seed_for("benchw4pfg", K))).to(dev)
        qa, sca, za, pa = tq.w4a16_pack_asym(W, gi)
        del W
        for M, dt, act in [(2048, "f16", False), (4096, "f16", False), (2048, "bf16", False), (4096, "bf16", False),
                           (4096, "f16", True)]:
            A = synth.activations_device(M, K, synth.seed_for("benchw4pfa", N, K, dt), dt, dev)
            C = torch.empty((M, N), dtype=A.dtype, device=dev)
            if act:
                nb = tq.w4a16_gemm_asym_workspace_bytes(M, N, K, dt, with_perm=True)
                ws = tq.new_workspace(nb, dev)
                call = lambda: tq.w4a16_gemm(A, qa, sca, zeros=za, perm=pa, out=C, workspace=ws)  # noqa: E731
            else:
                call = lambda: tq.w4a16_gemm(A, q, sc, out=C, workspace=None)  # noqa: E731
            settle(call)
            t = time_region(call, iters, stream) / iters
            torch.cuda.synchronize()
            if samples is not None:
                if act:
                    samples.append(w4_sample(f"w4_prefill_act_{dt}_M{M}", A, C, qa, sca, synth.seed_for("bsw4p", N, M),
                                             za, pa))
                else:
                    samples.append(w4_sample(f"w4_prefill_{dt}_M{M}", A, C, q, sc, synth.seed_for("bsw4p", N, M, dt)))
            tf = 2.0 * M * N * K / t / 1e12
            res[f"{N}x{K}_M{M}_{dt}{'_zp_act' if act else ''}"] = {"ms": round(t * 1e3, 4), "tflops": round(tf, 1),
                                                                  "frac_of_peak": round(tf / MFMA_PEAK_TFLOPS, 4)}
            del A, C
        del q, sc, qa, sca, za, pa
    torch.cuda.empty_cache()
    return res


def run_calib(dev, nbytes=1 << 30, iters=5):
    """A plain device copy of known size, for scaling FETCH_SIZE / WRITE_SIZE."""
    import torch
    src = torch.empty(nbytes // 2, dtype=torch.float16, device=dev).fill_(1.0)
    dst = torch.empty_like(src)
    stream = torch.cuda.current_stream()
    dst.copy_(src)
    t = time_region(lambda: dst.copy_(src), iters, stream) / iters
    return {"calib_copy_bytes": nbytes, "copy_ms": round(t * 1e3, 4), "copy_read_gbs": round(nbytes / t / 1e9, 1)}


def cpu_info():
    """Host cores, affinity, CPU model and the BLAS library numpy uses."""
    info = {"os_cpu_count": os.cpu_count(), "affinity_cpus": len(os.sched_getaffinity(0)), "cpu_model": None,
            "blas": None}
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    info["cpu_model"] = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    try:
        import threadpoolctl
        pools = [p for p in threadpoolctl.threadpool_info() if p.get("user_api") == "blas"]
        if pools:
            info["blas"] = {"library": pools[0].get("internal_api"), "threads": pools[0].get("num_threads")}
    except Exception:
        pass
    return info


def check_samples(samples):
    """The oracle's verdict on sampled outputs of the timed GPU calls (part of
    the CPU leg): fp64 dequant of the sampled weight rows, fp64 product with
    the sampled activation rows, tolerance 2e-3 * sum|a w| + 1e-3 per output."""
    import oracle.check as OC
    import oracle.gemm as OG
    import oracle.ternary as OT
    import oracle.w4 as OW
    import oracle.w4asym as OA
    lines = {}
    for smp in samples:
        K = smp["K"]
        if smp["kind"] == "ternary":
            wdq = OT.ternary_dequant(smp["codes"], smp["scale"], K)
        elif smp["kind"] == "w4":
            wdq = OW.w4_dequant(smp["q"], smp["scale"], K)
        else:
            wdq = OA.w4a_dequant(smp["q"], smp["scale"], smp["zeros"], K, smp["perm"])
        out, mag = OG.gemm_ref64(smp["A"], wdq)
        ok, st = OC.tolerance_ok(smp["C"], out, mag, out_dtype=smp["dtype"])
        e = lines.setdefault(smp["line"], {"outputs": 0, "ok": True, "max_ratio_to_bound": 0.0})
        e["outputs"] += int(smp["C"].size)
        e["ok"] = e["ok"] and ok
        e["max_ratio_to_bound"] = round(max(e["max_ratio_to_bound"], st["max_ratio_to_bound"]), 4)
    return {"ok": all(e["ok"] for e in lines.values()) if lines else None,
            "sample": f"per timed matrix sampled: {SAMPLE_ROWS} weight rows x up to {SAMPLE_M} activation rows "
                      "(first and last layer of each decode step, every medium-M / prefill call)",
            "lines": lines}


def cpu_baseline(min_seconds, samples):
    """The oracle, untuned, on the host, beside the GPU run:
      * parity: the oracle's fp64 product for the sampled outputs of every
        timed line (weight rows and activation rows drawn per matrix; the
        GPU outputs are those of the timed steps), each judged against
        2e-3 * sum|a w| + 1e-3 - the vectorized tier (fp64 dequant + BLAS);
      * value: the vectorized tier on one Llama-3-8B layer's 7 projections
        at M = 1, repeated for at least `min_seconds`, as packed GB/s;
      * the pure-loop tier on the 256 x 256 case and on 64 weight rows of
        each Llama-3-8B shape, extrapolated to the full M = 1 step;
      * the oracle's ternary pack of one 1024 x 4096 matrix (the CPU
        counterpart of tq_pack), per matrix and per fp32 byte."""
    import oracle.gemm as OG
    import oracle.ternary as OT
    import synth
    parity = check_samples(samples)
    # vectorized tier on one Llama-3-8B layer at M = 1
    layer = []
    for name, (N, K) in layer_shapes(False):
        W = synth.weights(N, K, synth.seed_for("cpu", name))
        codes, sb = OT.ternary_pack(W)
        layer.append((K, codes, sb, synth.activations(1, K, synth.seed_for("cpux", K)).double().numpy()))
        del W
    total_bytes, total_t, reps = 0, 0.0, 0
    while total_t < min_seconds:
        for K, codes, sb, a in layer:
            t0 = time.perf_counter()
            wdq = OT.ternary_dequant(codes, sb, K)
            OG.gemm_ref64(a, wdq)
            total_t += time.perf_counter() - t0
            total_bytes += codes.nbytes
            del wdq
        reps += 1
    # loop tier: the 256 x 256 case, and 64 rows of each fused 8B shape
    W0, A0 = synth.smallest_case()
    c0, s0 = OT.ternary_pack(W0)
    t0 = time.perf_counter()
    OG.gemm_ref64_loop(A0.double().numpy().tolist(), OT.ternary_dequant_loop(c0.tolist(), s0.tolist(), 256))
    t_loop0 = time.perf_counter() - t0
    step_loop_s = 0.0
    for name, (N, K) in layer_shapes(True):
        W = synth.weights(64, K, synth.seed_for("cpuloop", name))
        c, sb = OT.ternary_pack(W)
        a = synth.activations(1, K, synth.seed_for("cpuloopx", K)).double().numpy().tolist()
        t0 = time.perf_counter()
        OG.gemm_ref64_loop(a, OT.ternary_dequant_loop(c.tolist(), sb.tolist(), K))
        step_loop_s += (time.perf_counter() - t0) * (N / 64) * synth.LLAMA3_8B_LAYERS
    # the oracle's pack of one matrix
    Wp = synth.weights(1024, 4096, synth.seed_for("cpupack"))
    t0 = time.perf_counter()
    OT.ternary_pack(Wp)
    t_pack = time.perf_counter() - t0
    info = cpu_info()
    threads = (info["blas"] or {}).get("threads") or 1
    return {
        "value": round(total_bytes / total_t / 1e9, 4), "unit": "GB/s", "cores": threads, "kind": "oracle",
        "sample": f"vectorized tier (fp64 dequant + BLAS fp64 product): {reps} passes over one Llama-3-8B layer's "
                  f"7 projections (52 MiB packed) at M=1, {total_t:.1f} s of CPU work",
        "loop_tier": {"smallest_case_s": round(t_loop0, 3),
                      "llama3_8b_step_s_extrapolated": round(step_loop_s, 1),
                      "how": "pure-Python loops on 64 weight rows of each fused shape at M=1, scaled by "
                             "N/64 x 32 layers (extrapolated)"},
        "pack": {"matrix": "1024x4096", "s": round(t_pack, 3),
                 "fp32_gbs": round(1024 * 4096 * 4 / t_pack / 1e9, 3)},
        "host": info,
    }, parity


def kernel_digest(source, spans, headers=()):
    """sha256 of the parts of `source` that decide one kernel's HBM traffic
    and of the headers it includes, so that edits elsewhere in the file do
    not invalidate a measurement of it.  Each span (first, last) runs from
    the definition of `first` (with its template line) to the lone closing
    brace that ends the definition of `last`."""
    import hashlib
    lines = open(os.path.join(ROOT, source)).read().split("\n")
    h = hashlib.sha256()
    for first, last in spans:
        start = next(i for i, ln in enumerate(lines) if f" {first}(" in ln and not ln.rstrip().endswith(";"))
        if start > 0 and lines[start - 1].startswith("template"):
            start -= 1
        at = next(i for i in range(start, len(lines)) if f" {last}(" in lines[i])
        end = next(i for i in range(at, len(lines)) if lines[i] == "}")
        h.update("\n".join(lines[start:end + 1]).encode())
    for hdr in headers:
        h.update(open(os.path.join(ROOT, hdr), "rb").read())
    return h.hexdigest()


# The M = 1 ternary decode kernel: its device helpers and body, and the plan
# and launch code that fix its grid.
TRAFFIC_KERNEL = ("bit_weight_only_tq_amd/csrc/gemv.hip",
                  (("sm_mma", "ternary_gemv_m1_kernel"), ("gemv_m1_plan", "launch_gemv_m1_plan")),
                  ("bit_weight_only_tq_amd/csrc/tq_device.h",))


def load_traffic(path):
    """HBM bytes per GEMV launch from the committed counter summary, or None
    when it is missing or was measured on a different kernel definition."""
    try:
        with open(path) as f:
            tj = json.load(f)
        if kernel_digest(*TRAFFIC_KERNEL) != tj["kernel_digest"]:
            return None
        return tj["hbm_bytes_per_launch"]
    except (OSError, KeyError, ValueError, StopIteration):
        return None


def main():
    args = parse()
    SETTLE_SECONDS[0] = args.settle
    if args.gpus != 1:
        print(json.dumps({"error": "the benchmark runs on exactly one GPU (no multi-GPU path); --gpus must be 1"}), flush=True)
        sys.exit(2)
    import torch
    import bit_weight_only_tq_amd as tq
    tq.load()
    if not torch.cuda.is_available():
        print(json.dumps({"error": "no GPU visible"}), flush=True)
        sys.exit(1)
    dev = torch.device("cuda", 0)

    if args.mode == "calib":
        print(json.dumps(run_calib(dev)), flush=True)
        return
    if args.mode == "prefill":
        print(json.dumps({"secondary": run_prefill(dev)}), flush=True)
        return
    if args.mode == "attrib":
        ceil = run_ceiling(dev, [N * K // 4 for _, (N, K) in layer_shapes(True)])
        print(json.dumps({"attribution": run_attrib(dev, ceil)}), flush=True)
        return
    if args.mode == "decodem":
        print(json.dumps({"decode_m": run_decode_m(args, dev, not args.no_graph),
                          "decode_bf16": run_decode_m(args, dev, not args.no_graph, Ms=(1, 2, 16), dt="bf16")}), flush=True)
        return
    if args.mode == "decode70b":
        print(json.dumps({"decode_70b": run_decode_70b(args, dev)}), flush=True)
        return
    if args.mode == "w4":
        print(json.dumps({"w4a16_decode": run_w4_decode(args, dev),
                          "w4a16_decode_bf16": run_w4_decode(args, dev, Ms=(1, 4, 16), dt="bf16")}), flush=True)
        return
    if args.mode == "w4act":
        print(json.dumps({"w4a16_act_decode": run_w4_decode(args, dev, act_order=True)}), flush=True)
        return
    if args.mode == "medium":
        print(json.dumps({"medium_m": run_medium(dev)}), flush=True)
        return
    if args.mode == "w4prefill":
        print(json.dumps({"w4a16_prefill": run_w4_prefill(dev)}), flush=True)
        return
    if args.mode == "w4medium":
        print(json.dumps({"w4a16_medium_m": run_w4_medium(dev)}), flush=True)
        return

    graph = not args.no_graph
    fused = not args.unfused
    full = args.mode == "full"
    samples = [] if full and not args.no_cpu_baseline else None
    shapes8 = [s_ for _, s_ in layer_shapes(fused)]
    shapes70 = [s_ for _, s_ in layer_shapes(True, "70b")]
    ceil = None
    if full:
        log("measured read ceiling per launch size")
        sizes = [N * K // 4 for N, K in shapes8 + shapes70] + [N * K // 2 for N, K in shapes8]
        ceil = run_ceiling(dev, sizes)
    log(f"decode: {args.layers} layers, fused={fused}, graph={graph}")
    d = run_decode(args, dev, fused, graph, line="value", samples=samples)
    traffic = load_traffic(args.traffic_json)
    achieved = d["alg_bytes_per_launch"] / (d["avg_launch_us"] * 1e-6) / 1e9
    out = {
        "metric": METRIC,
        "value": round(d["packed_gbs"], 1),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(d["ms_per_step"], 4),
        "step_ms_percentiles": d["step_ms"],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f16",
        "data": "synthetic: seeded N(0,0.02) fp32 weights ternarized on device, N(0,1) fp16 activations",
        "config": {
            "workload": "Llama-3-8B decode, M=1: 32 layers x {qkv (6144x4096), o (4096x4096), "
                        "gate_up (28672x4096), down (4096x14336)} ternary GEMV",
            "M": 1, "layers": args.layers, "launches_per_step": d["launches"],
            "packed_bytes_per_step": d["packed_bytes"], "algorithmic_bytes_per_step": d["alg_bytes"],
            "graph_replay": graph, "fused_qkv_gate_up": fused,
            "hbm_frac_packed": round(d["packed_gbs"] / HBM_PEAK_GBS, 4),
        },
        "roofline": {
            "bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
            "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": traffic,
            "kernel": "ternary_gemv_m1_kernel", "avg_launch_us": round(d["avg_launch_us"], 3),
            "alg_bytes_per_launch": round(d["alg_bytes_per_launch"]),
        },
    }
    if full:
        ceil8 = ceiling_step_ms(shapes8, ceil) * args.layers
        out["roofline"]["ceiling"] = {
            "what": "plain streaming read of each launch's code bytes (tq_diag_stream_read), best workgroup "
                    "count, back-to-back in a graph over >= 2 GiB; summed over the step's launches",
            "step_ms": round(ceil8, 4), "gbs": round(d["packed_bytes"] / (ceil8 * 1e-3) / 1e9, 1),
            "frac": round(ceil8 / d["ms_per_step"], 4),
            "per_launch_us": {f"{N}x{K}": round(ceil[N * K // 4], 2) for N, K in shapes8 + shapes70},
        }
        if fused:
            log("decode, unfused projections")
            u = run_decode(args, dev, False, graph)
            out["decode_unfused"] = {"value": round(u["packed_gbs"], 1), "unit": "GB/s",
                                     "ms_per_step": round(u["ms_per_step"], 4), "launches_per_step": u["launches"],
                                     "avg_launch_us": round(u["avg_launch_us"], 3)}
        log("decode, M = 4 and 16")
        out["decode_m"] = run_decode_m(args, dev, graph, samples=samples, ceiling_ms=ceil8)
        log("decode, bf16 activations, M = 1, 2 and 16")
        out["decode_bf16"] = run_decode_m(args, dev, graph, Ms=(1, 2, 16), dt="bf16", samples=samples,
                                          ceiling_ms=ceil8)
        log("decode time split")
        out["attribution"] = run_attrib(dev, ceil)
        log("decode, Llama-3-70B, 80 layers, M = 1, 32, 64")
        out["decode_70b"] = run_decode_70b(args, dev, samples=samples,
                                           ceiling=ceiling_step_ms(shapes70, ceil) * 80)
        log("W4A16 decode")
        out["w4a16_decode"] = run_w4_decode(args, dev, samples=samples)
        w4ceil = sum(ceil[N * K // 2] for N, K in shapes8) / 1e3 * args.layers
        for key in ("M1", "M4", "M16"):
            out["w4a16_decode"][key]["frac_of_ceiling"] = round(w4ceil / out["w4a16_decode"][key]["ms_per_step"], 4)
        log("W4A16 decode, bf16 activations")
        out["w4a16_decode_bf16"] = run_w4_decode(args, dev, Ms=(1, 4, 16), dt="bf16", samples=samples)
        log("W4A16 decode, zero points and activation order")
        out["w4a16_act_decode"] = run_w4_decode(args, dev, act_order=True, samples=samples)
        log("medium M")
        out["medium_m"] = run_medium(dev, samples=samples)
        log("W4A16 medium M")
        out["w4a16_medium_m"] = run_w4_medium(dev, samples=samples)
        log("prefill GEMM M=4096")
        out["secondary"] = run_prefill(dev, samples=samples)
        log("W4A16 prefill GEMM")
        out["w4a16_prefill"] = run_w4_prefill(dev, samples=samples)
        if not args.no_cpu_baseline:
            log("cpu baseline (oracle) and parity of the sampled outputs")
            out["cpu_baseline"], out["parity"] = cpu_baseline(args.cpu_seconds, samples)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
