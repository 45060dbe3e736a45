"""GPU checks of the split-K workspace protocol.  The streaming decode kernels
and the prefill GEMM complete a split in the kernel: the last split
workgroup of each output tile to finish sums the fp32 partials, counted by
per-tile arrival counters at the front of the workspace; the medium-M tiles
and the W4A16 GEMM leave the sum to a second kernel and never touch the
counters.

For every kernel family that splits K (streaming decode kernels, medium-M
tiles, prefill GEMM, W4A16 GEMM, activation-order W4A16 through the gather):
outputs within the tolerance of the oracle on sampled columns, the counters
back at zero after every call, repeated calls bit-identical (the sum order
is fixed whichever split finishes last), and garbage in the partial area
before the first call harmless (every partial is rewritten).
"""
import numpy as np
import pytest

import oracle.ternary as OT
import oracle.w4 as OW
import oracle.w4asym as OA
import synth
from gpu_common import check_close, log, require_gpu

pytestmark = pytest.mark.gpu

# (label, format, M, N, K, dtype, forced path)
CASES = [
    ("ternary decode stream", "ternary", 16, 4096, 14336, "f16", "gemv"),
    ("ternary decode stream bf16", "ternary", 9, 4100, 14336, "bf16", "gemv"),
    ("ternary medium", "ternary", 32, 8192, 8192, "bf16", "stream_mfma"),
    ("ternary medium paired", "ternary", 64, 8192, 28672, "f16", "stream_mfma"),
    ("ternary prefill", "ternary", 2048, 4096, 14336, "f16", "gemm"),
    ("ternary prefill ragged", "ternary", 300, 1000, 4096, "bf16", "gemm"),
    ("w4 decode stream", "w4", 16, 4096, 14336, "f16", "auto"),
    ("w4 gemm 64-row tiles", "w4", 40, 4096, 14336, "bf16", "auto"),
    ("w4 gemm 256-row tiles", "w4", 256, 4096, 14336, "f16", "auto"),
    ("w4 act order stream", "w4act", 8, 4096, 14336, "f16", "auto"),
]


def _flag_bytes():
    import bit_weight_only_tq_amd as tq
    return tq.TQ_WORKSPACE_FLAG_BYTES


@pytest.mark.parametrize("case", CASES, ids=[c[0] for c in CASES])
def test_counters_left_zero_and_results_repeat(case):
    import torch
    import bit_weight_only_tq_amd as tq
    dev = require_gpu()
    label, fmt, M, N, K, dt, path = case
    F = _flag_bytes()
    W = synth.weights_device(N, K, synth.seed_for("spc", fmt, N, K), dev)
    cols = np.sort(np.random.default_rng(N + K + 9).choice(N, min(N, 128), replace=False))
    idx = torch.from_numpy(cols).to(dev)
    Wc = W.index_select(0, idx).cpu().numpy()
    if fmt == "ternary":
        codes, scale = tq.tq_pack(W)
        rc, rs = OT.ternary_pack(Wc)
        wdq = OT.ternary_dequant(rc, rs, K)
        nbytes = tq.tq_gemm_workspace_bytes(M, N, K, dt, path=path)
        call = lambda A, ws: tq.tq_gemm(A, codes, scale, path=path, workspace=ws)  # noqa: E731
    elif fmt == "w4":
        q, s = tq.w4a16_pack(W)
        rq, rs = OW.w4_pack(Wc)
        wdq = OW.w4_dequant(rq, rs, K)
        nbytes = tq.w4a16_gemm_workspace_bytes(M, N, K, dt)
        call = lambda A, ws: tq.w4a16_gemm(A, q, s, workspace=ws)  # noqa: E731
    else:
        g = synth.group_index(K, synth.seed_for("spcg", K))
        q, s, z, perm = tq.w4a16_pack_asym(W, torch.from_numpy(g).to(dev))
        rq, rs, rz, rp = OA.w4a_pack(Wc, g)
        wdq = OA.w4a_dequant(rq, rs, rz, K, rp)
        nbytes = tq.w4a16_gemm_asym_workspace_bytes(M, N, K, dt, with_perm=True)
        call = lambda A, ws: tq.w4a16_gemm(A, q, s, zeros=z, perm=perm, workspace=ws)  # noqa: E731
    del W
    log(f"split counters {label} M={M} N={N} K={K} {dt} workspace={nbytes}")
    assert nbytes > F, "the case must split K"
    A = synth.activations(M, K, synth.seed_for("spca", fmt, M, K, dt), dt)
    Ad = A.to(dev)
    ws = tq.new_workspace(nbytes, dev)
    ws[F:].fill_(0xFF)  # partials of an earlier user: the call must rewrite them all
    C0 = call(Ad, ws)
    check_close(C0.index_select(1, idx), A, wdq, label=f"{label} first call")
    assert int(ws[:F].count_nonzero()) == 0, "arrival counters not left at zero"
    for _ in range(4):
        C = call(Ad, ws)
        assert torch.equal(C0.view(torch.int16), C.view(torch.int16))
    assert int(ws[:F].count_nonzero()) == 0


def test_counters_shared_by_back_to_back_shapes():
    """One workspace for a sequence of split calls of different shapes and
    kernel families in stream order (each leaves the counters zero for the
    next), checked against calls that each get a fresh workspace."""
    import torch
    import bit_weight_only_tq_amd as tq
    dev = require_gpu()
    F = _flag_bytes()
    shapes = [(16, 4096, 14336, "gemv"), (32, 8192, 8192, "stream_mfma"), (9, 4100, 14336, "gemv"),
              (300, 1000, 4096, "gemm"), (64, 1024, 8192, "stream_mfma")]
    mats = {}
    for M, N, K, path in shapes:
        if (N, K) not in mats:
            mats[(N, K)] = tq.tq_pack(synth.weights_device(N, K, synth.seed_for("spcs", N, K), dev))
    need = max(tq.tq_gemm_workspace_bytes(M, N, K, "f16", path=p) for M, N, K, p in shapes)
    shared = tq.new_workspace(need, dev)
    log(f"split counters shared workspace {need} bytes over {len(shapes)} shapes")
    for rep in range(2):
        for M, N, K, path in shapes:
            codes, scale = mats[(N, K)]
            A = synth.activations(M, K, synth.seed_for("spcsa", M, K), "f16").to(dev)
            C = tq.tq_gemm(A, codes, scale, path=path, workspace=shared)
            ref = tq.tq_gemm(A, codes, scale, path=path, workspace="auto")
            assert torch.equal(C.view(torch.int16), ref.view(torch.int16)), (rep, M, N, K, path)
    assert int(shared[:F].count_nonzero()) == 0
