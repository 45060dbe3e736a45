"""GPU parity: pack and unpack match the oracle bit for bit (through the C ABI)."""
import numpy as np
import pytest

import oracle.ternary as OT
import oracle.w4 as OW
import synth
from gpu_common import bits16, log, require_gpu

pytestmark = pytest.mark.gpu


def _special_rows(K):
    """Rows that stress the pack rule: zeros, a threshold tie, tiny and huge
    magnitudes, signed zeros, a single nonzero."""
    rows = [np.zeros(K)]
    tie = np.array([7, 11, 11, 11] * (K // 4) + [11] * (K % 4), dtype=np.float64) * 2.0 ** -9
    rows.append(tie)
    rows.append(np.linspace(-1, 1, K) * 1e-9)          # scale underflows to +0
    rows.append(np.full(K, 60000.0) * np.where(np.arange(K) % 3 == 0, -1, 1))
    one = np.zeros(K)
    one[K // 2] = -0.5
    rows.append(one)
    rows.append(np.where(np.arange(K) % 2 == 0, -0.0, 0.0))
    return np.array(rows, dtype=np.float32)


@pytest.mark.parametrize("N,K", [
    (256, 256), (1, 64), (63, 100), (65, 257), (130, 3), (7, 1), (64, 4096), (33, 1000),
    (4096, 4096), (1024, 4096), (14336, 4096), (4096, 14336),
])
def test_ternary_pack_parity(N, K):
    import torch
    import bit_weight_only_tq_amd as tq
    dev = require_gpu()
    log(f"tq_pack N={N} K={K}")
    W = synth.smallest_case()[0] if (N, K) == (256, 256) else synth.weights(N, K, synth.seed_for("pack", N, K))
    if N >= 8:
        sp = _special_rows(K)
        W[:len(sp)] = sp
    codes, scale = tq.tq_pack(torch.from_numpy(W).to(dev))
    torch.cuda.synchronize()
    rc, rs = OT.ternary_pack(W)
    assert tq.TernaryLayout(N, K).codes_shape == tuple(codes.shape)
    np.testing.assert_array_equal(codes.cpu().numpy(), rc)
    np.testing.assert_array_equal(bits16(scale), rs)
    # unpack back through the library: exact t and t * scale
    t, wdq = tq.tq_unpack(codes, scale, K)
    np.testing.assert_array_equal(t.cpu().numpy(), OT.ternary_unpack(rc, K))
    np.testing.assert_array_equal(bits16(wdq), OT.ternary_dequant_f16_bits(rc, rs, K))


def test_ternary_pack_errors():
    import torch
    import bit_weight_only_tq_amd as tq
    dev = require_gpu()
    log("tq_pack errors")
    W = torch.full((70, 128), 0.1, dtype=torch.float32, device=dev)
    W[33, 17] = float("nan")
    with pytest.raises(tq.TQError) as e:
        tq.tq_pack(W)
    assert e.value.name == "TQ_ERR_NONFINITE"
    W[33, 17] = float("-inf")
    with pytest.raises(tq.TQError) as e:
        tq.tq_pack(W)
    assert e.value.name == "TQ_ERR_NONFINITE"
    W[33, 17] = 70000.0
    W[33, :] = 70000.0
    with pytest.raises(tq.TQError) as e:
        tq.tq_pack(W)
    assert e.value.name == "TQ_ERR_RANGE"


def test_ternary_unpack_bad_code():
    import torch
    import bit_weight_only_tq_amd as tq
    dev = require_gpu()
    log("tq_unpack bad code")
    codes = torch.full((5, 16), 0x55, dtype=torch.uint8, device=dev)
    scale = torch.ones(5, dtype=torch.float16, device=dev)
    t, _ = tq.tq_unpack(codes, scale, 64)
    assert int(t.abs().sum()) == 0
    codes[3, 7] = 0b01110101  # field 3 of byte 7 is 0b01, field 2 is 0b11
    with pytest.raises(tq.TQError) as e:
        tq.tq_unpack(codes, scale, 64)
    assert e.value.name == "TQ_ERR_BAD_CODE"
    # a 0b11 in a padding field (columns >= K) is not examined
    codes2 = torch.full((2, 2), 0x55, dtype=torch.uint8, device=dev)
    codes2[1, 1] = 0b11010101  # field 3 of byte 1 = column 7
    tq.tq_unpack(codes2, scale[:2], 7)


@pytest.mark.parametrize("N,K", [
    (3, 128), (5, 384), (64, 1024), (4096, 4096), (1024, 4096), (14336, 4096), (4096, 14336),
])
def test_w4_pack_parity(N, K):
    import torch
    import bit_weight_only_tq_amd as tq
    dev = require_gpu()
    log(f"w4a16_pack N={N} K={K}")
    W = synth.weights(N, K, synth.seed_for("w4pack", N, K))
    if N >= 3:
        W[0, :128] = 0.0                                                # zero group
        W[1, :3] = np.array([-9.8, 9.8, 2.5]) * 2.0 ** -24              # subnormal scale, clamp
        W[1, 3:128] = 0.0
        s16 = np.float64(np.float16(0.0234375))
        W[2, :128] = ((np.arange(128) % 14 - 7 + 0.5) * s16).astype(np.float32)   # exact ties
        W[2, 127] = np.float32(7 * s16)
    q, s = tq.w4a16_pack(torch.from_numpy(W).to(dev))
    torch.cuda.synchronize()
    rq, rs = OW.w4_pack(W)
    assert tq.W4Layout(N, K).qweight_shape == tuple(q.shape)
    np.testing.assert_array_equal(q.cpu().numpy(), rq)
    np.testing.assert_array_equal(bits16(s), rs)
    qo, wdq = tq.w4a16_unpack(q, s, K)
    np.testing.assert_array_equal(qo.cpu().numpy(), OW.w4_unpack(rq, K))
    np.testing.assert_array_equal(bits16(wdq), OW.w4_dequant_f16_bits(rq, rs, K))


def test_w4_pack_errors():
    import torch
    import bit_weight_only_tq_amd as tq
    dev = require_gpu()
    log("w4a16_pack errors")
    W = torch.zeros((4, 256), dtype=torch.float32, device=dev)
    W[2, 5] = float("nan")
    with pytest.raises(tq.TQError) as e:
        tq.w4a16_pack(W)
    assert e.value.name == "TQ_ERR_NONFINITE"
    W[2, 5] = 5e5
    with pytest.raises(tq.TQError) as e:
        tq.w4a16_pack(W)
    assert e.value.name == "TQ_ERR_RANGE"
