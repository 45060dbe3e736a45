"""The measurement entry points run on the GPU and stay in bounds.

tq_diag_gemv variant 0 is the M = 1 decode kernel tq_gemm runs, so its
output equals tq_gemm's bit for bit; variants 1 and 2 (codes from the cache,
with and without the multiply) complete and leave the output buffer's
neighbours untouched; tq_diag_stream_read completes for several workgroup
counts and writes nothing past its sink.
"""
import numpy as np
import pytest

import synth
from gpu_common import bits16, log, require_gpu

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("N,K", [(4096, 4096), (6144, 4096), (4096, 14336), (28672, 4096)])
def test_diag_gemv_variants(N, K):
    import torch
    import bit_weight_only_tq_amd as tq
    dev = require_gpu()
    log(f"diag gemv N={N} K={K}")
    W = synth.weights_device(N, K, synth.seed_for("diag", N, K), dev)
    codes, scale = tq.tq_pack(W)
    x = synth.activations_device(1, K, synth.seed_for("diagx", K), "f16", dev)
    ref = tq.tq_gemm(x, codes, scale)
    buf = torch.full((3, N), -5.0, dtype=torch.float16, device=dev)
    out = tq.tq_diag_gemv(x, codes, scale, 0, out=buf[1:2])
    torch.cuda.synchronize()
    np.testing.assert_array_equal(bits16(out), bits16(ref))
    for var in (1, 2):
        tq.tq_diag_gemv(x, codes, scale, var, out=buf[1:2])
    torch.cuda.synchronize()
    assert bool((buf[0] == -5.0).all()) and bool((buf[2] == -5.0).all())
    with pytest.raises(tq.TQError, match="TQ_ERR_PATH"):
        tq.tq_diag_gemv(synth.activations_device(2, K, 1, "f16", dev), codes, scale, 0)


@pytest.mark.parametrize("nbytes", [16 << 10, 4 << 20, 28 << 20])
def test_diag_stream_read(nbytes):
    import torch
    import bit_weight_only_tq_amd as tq
    dev = require_gpu()
    log(f"diag stream read {nbytes} bytes")
    src = torch.zeros((nbytes,), dtype=torch.uint8, device=dev)
    cus = torch.cuda.get_device_properties(dev).multi_processor_count
    sink = torch.full((16 * cus + 8,), 7, dtype=torch.int32, device=dev)
    for blocks in (1, cus, 4 * cus, 16 * cus):
        if blocks <= nbytes // 16:
            tq.tq_diag_stream_read(src, blocks, sink=sink[:blocks])
    torch.cuda.synchronize()
    assert bool((sink == 7).all())  # all-zero data never matches the improbable fold
