"""The apply calls allocate nothing and never synchronize, so they can be
captured in a HIP graph; every replay must equal the eager result."""
import pytest

import synth
from gpu_common import log, require_gpu

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("fmt,M,N,K", [
    ("ternary", 1, 4096, 4096), ("ternary", 16, 1024, 4096),
    ("ternary", 2, 1024, 4096), ("ternary", 4, 4096, 14336),  # small-M kernel, two and four rows held
    ("ternary", 512, 1024, 4096), ("ternary", 2048, 14336, 4096),  # large M: split K summed in the kernel; one pass
    ("ternary", 40, 1024, 4096), ("ternary", 200, 2048, 1024),  # medium path: split K, reduction kernel
    ("w4a16", 4, 1024, 4096), ("w4a16", 16, 4096, 14336),  # W4: one pass; split K summed in the kernel
    ("w4a16_act", 1, 4096, 4096), ("w4a16_act", 16, 4096, 14336),  # zero points + column order: gather first
])
def test_graph_replay_matches_eager(fmt, M, N, K):
    import torch
    import bit_weight_only_tq_amd as tq
    dev = require_gpu()
    log(f"graph {fmt} M={M} N={N} K={K}")
    W = torch.from_numpy(synth.weights(N, K, synth.seed_for("g", fmt, N, K))).to(dev)
    if fmt == "ternary":
        wq, sc = tq.tq_pack(W)
        fn = lambda a, out: tq.tq_gemm(a, wq, sc, out=out)  # noqa: E731
    elif fmt == "w4a16":
        wq, sc = tq.w4a16_pack(W)
        fn = lambda a, out: tq.w4a16_gemm(a, wq, sc, out=out)  # noqa: E731
    else:
        gi = torch.from_numpy(synth.group_index(K, synth.seed_for("gg", K))).to(dev)
        wq, sc, zp, perm = tq.w4a16_pack_asym(W, gi)
        fn = lambda a, out: tq.w4a16_gemm(a, wq, sc, out=out, zeros=zp, perm=perm)  # noqa: E731
    A = synth.activations(M, K, synth.seed_for("ga", M), "f16").to(dev)
    eager = fn(A, None)
    torch.cuda.synchronize()
    out = torch.empty_like(eager)
    g = torch.cuda.CUDAGraph()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        fn(A, out)  # warm-up outside the graph
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    with torch.cuda.graph(g):
        fn(A, out)
    for i in range(4):
        out.fill_(0)
        junk = torch.randn(1000, device=dev).sum()  # unrelated eager work between replays
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out.view(torch.int16), eager.view(torch.int16)), f"replay {i}"
        del junk


@pytest.mark.parametrize("fmt,M,N,K", [
    ("ternary", 16, 4096, 14336),   # streaming decode kernel, K split 7 ways, summed in the kernel
    ("ternary", 512, 1024, 4096),   # prefill GEMM, K split, summed in the kernel
    ("ternary", 40, 1024, 4096),    # medium path, K split, reduction kernel (counters untouched)
    ("w4a16", 16, 4096, 14336),     # W4A16 streaming kernel, K split, summed in the kernel
])
def test_graph_replay_shared_workspace(fmt, M, N, K):
    """One caller workspace, counters zeroed once before capture: the split
    kernels must leave their arrival counters at zero after every replay, so
    that each replay (no zeroing in the graph) still equals the eager call."""
    import torch
    import bit_weight_only_tq_amd as tq
    dev = require_gpu()
    log(f"graph shared workspace {fmt} M={M} N={N} K={K}")
    W = torch.from_numpy(synth.weights(N, K, synth.seed_for("gw", fmt, N, K))).to(dev)
    if fmt == "ternary":
        wq, sc = tq.tq_pack(W)
        nbytes = tq.tq_gemm_workspace_bytes(M, N, K, "f16")
        fn = lambda a, out, ws: tq.tq_gemm(a, wq, sc, out=out, workspace=ws)  # noqa: E731
    else:
        wq, sc = tq.w4a16_pack(W)
        nbytes = tq.w4a16_gemm_workspace_bytes(M, N, K, "f16")
        fn = lambda a, out, ws: tq.w4a16_gemm(a, wq, sc, out=out, workspace=ws)  # noqa: E731
    assert nbytes > tq.TQ_WORKSPACE_FLAG_BYTES, "the case must split K"
    A = synth.activations(M, K, synth.seed_for("gwa", M), "f16").to(dev)
    eager = fn(A, None, "auto")
    ws = tq.new_workspace(nbytes, dev)
    out = torch.empty_like(eager)
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        fn(A, out, ws)  # warm-up outside the graph
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    assert torch.equal(out.view(torch.int16), eager.view(torch.int16))
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        fn(A, out, ws)
    for i in range(4):
        out.fill_(0)
        junk = torch.randn(1000, device=dev).sum()  # unrelated eager work between replays
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out.view(torch.int16), eager.view(torch.int16)), f"replay {i}"
        assert int(ws[:tq.TQ_WORKSPACE_FLAG_BYTES].count_nonzero()) == 0, f"counters after replay {i}"
        del junk
