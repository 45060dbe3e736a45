"""The Python binding rejects mismatched tensors before any library call.

The C ABI takes bare pointers and cannot check buffer sizes, so the binding
checks shapes and dtypes against the packed layouts (codes [N, ceil(K/4)]
uint8, scale [N] fp16; qweight [N, K/8] int32, scales and zeros [N, K/128];
bias [N] and out [M, N] in the activation dtype).  These run on CPU tensors:
every check fires before the device check, which is what a well-formed CPU
tensor then trips.  No GPU is touched.
"""
import pytest
import torch

import bit_weight_only_tq_amd as tq


def _ternary(M=2, N=64, K=256, dt=torch.float16):
    A = torch.zeros((M, K), dtype=dt)
    codes = torch.zeros((N, K // 4), dtype=torch.uint8)
    scale = torch.zeros((N,), dtype=torch.float16)
    return A, codes, scale


def _w4(M=2, N=64, K=256, dt=torch.float16):
    A = torch.zeros((M, K), dtype=dt)
    q = torch.zeros((N, K // 8), dtype=torch.int32)
    s = torch.zeros((N, K // 128), dtype=torch.float16)
    return A, q, s


def test_tq_gemm_well_formed_cpu_tensors_reach_device_check():
    A, codes, scale = _ternary()
    with pytest.raises(ValueError, match="device tensors"):
        tq.tq_gemm(A, codes, scale)


@pytest.mark.parametrize("bad", ["codes_cols", "codes_dtype", "scale_len", "scale_dtype", "A_1d", "A_dtype",
                                 "bias_len", "bias_dtype", "out_shape", "out_dtype"])
def test_tq_gemm_rejects(bad):
    A, codes, scale = _ternary()
    bias, out = None, None
    if bad == "codes_cols":
        codes = torch.zeros((64, 65), dtype=torch.uint8)
    elif bad == "codes_dtype":
        codes = torch.zeros((64, 64), dtype=torch.int8)
    elif bad == "scale_len":
        scale = torch.zeros((63,), dtype=torch.float16)
    elif bad == "scale_dtype":
        scale = torch.zeros((64,), dtype=torch.float32)
    elif bad == "A_1d":
        A = torch.zeros((256,), dtype=torch.float16)
    elif bad == "A_dtype":
        A = torch.zeros((2, 256), dtype=torch.float32)
    elif bad == "bias_len":
        bias = torch.zeros((65,), dtype=torch.float16)
    elif bad == "bias_dtype":
        bias = torch.zeros((64,), dtype=torch.bfloat16)
    elif bad == "out_shape":
        out = torch.zeros((2, 63), dtype=torch.float16)
    elif bad == "out_dtype":
        out = torch.zeros((2, 64), dtype=torch.bfloat16)
    with pytest.raises((ValueError, TypeError)) as ei:
        tq.tq_gemm(A, codes, scale, bias=bias, out=out)
    assert "device tensors" not in str(ei.value)


@pytest.mark.parametrize("bad", ["q_cols", "q_dtype", "scales_shape", "zeros_shape", "zeros_dtype", "perm_len",
                                 "K_not_group", "out_dtype"])
def test_w4a16_gemm_rejects(bad):
    A, q, s = _w4()
    zeros, perm, out = None, None, None
    if bad == "q_cols":
        q = torch.zeros((64, 31), dtype=torch.int32)
    elif bad == "q_dtype":
        q = torch.zeros((64, 32), dtype=torch.int64)
    elif bad == "scales_shape":
        s = torch.zeros((64, 3), dtype=torch.float16)
    elif bad == "zeros_shape":
        zeros = torch.zeros((64, 3), dtype=torch.uint8)
    elif bad == "zeros_dtype":
        zeros = torch.zeros((64, 2), dtype=torch.int32)
    elif bad == "perm_len":
        perm = torch.zeros((255,), dtype=torch.int32)
    elif bad == "K_not_group":
        A = torch.zeros((2, 192), dtype=torch.float16)
        q = torch.zeros((64, 24), dtype=torch.int32)
    elif bad == "out_dtype":
        out = torch.zeros((2, 64), dtype=torch.bfloat16)
    with pytest.raises((ValueError, TypeError)) as ei:
        tq.w4a16_gemm(A, q, s, zeros=zeros, perm=perm, out=out)
    assert "device tensors" not in str(ei.value)


def test_unpack_rejects_mismatched_scale():
    codes = torch.zeros((64, 64), dtype=torch.uint8)
    with pytest.raises(ValueError, match="scale"):
        tq.tq_unpack(codes, torch.zeros((32,), dtype=torch.float16), 256)
    q = torch.zeros((64, 32), dtype=torch.int32)
    with pytest.raises(ValueError, match="scales"):
        tq.w4a16_unpack(q, torch.zeros((64, 1), dtype=torch.float16), 256)
