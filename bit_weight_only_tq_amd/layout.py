"""Packed weight layouts: shapes, dtypes, strides and validation.

Ternary (page "Ternary quantized models in vLLM ...", sections 2.1, 3.1, 3.2):
a checkpoint holds the packed codes (uint8, four 2-bit codes per byte) and a
fp16 scale per output row; a packed row is ceil(K/4) bytes (4096 -> 1024;
section 3.3 shows what floor instead of ceil breaks).

W4A16 (page "Model quantization - vLLM runtime quantization architecture",
section 5): eight int4 codes per int32 along K (packed factor 8), weight
[d_out, d_in/8], group scales [d_out, d_in/128], symmetric with zero point 8.

These classes only describe and check tensors; they do no arithmetic.
"""

from dataclasses import dataclass


@dataclass(frozen=True)
class TernaryLayout:
    N: int  # output features (weight rows)
    K: int  # input features

    packed_factor = 4          # codes per byte
    bits = 2
    code_of = {-1: 0b00, 0: 0b01, 1: 0b10}

    def __post_init__(self):
        if self.N <= 0 or self.K <= 0:
            raise ValueError(f"TernaryLayout needs N, K > 0, got {self.N}, {self.K}")

    @property
    def row_bytes(self) -> int:
        return -(-self.K // self.packed_factor)

    @property
    def codes_shape(self):
        return (self.N, self.row_bytes)

    @property
    def scale_shape(self):
        return (self.N,)

    @property
    def packed_bytes(self) -> int:
        return self.N * self.row_bytes

    @property
    def gemm_ok(self) -> bool:
        """The apply kernels need whole 16-byte chunks per row (K % 64 == 0)."""
        return self.K % 64 == 0

    def validate(self, codes, scale):
        import torch
        if codes.dtype != torch.uint8 or tuple(codes.shape) != self.codes_shape:
            raise ValueError(f"codes must be uint8 {self.codes_shape}, got {codes.dtype} {tuple(codes.shape)}")
        if scale.dtype != torch.float16 or tuple(scale.shape) != self.scale_shape:
            raise ValueError(f"scale must be float16 {self.scale_shape}, got {scale.dtype} {tuple(scale.shape)}")
        if not (codes.is_contiguous() and scale.is_contiguous()):
            raise ValueError("packed tensors must be contiguous")
        if codes.device != scale.device:
            raise ValueError("codes and scale must live on the same device")


@dataclass(frozen=True)
class W4Layout:
    N: int
    K: int
    group: int = 128

    packed_factor = 8          # int4 codes per int32
    bits = 4
    zero_point = 8

    def __post_init__(self):
        if self.N <= 0 or self.K <= 0:
            raise ValueError(f"W4Layout needs N, K > 0, got {self.N}, {self.K}")
        if self.group != 128:
            raise ValueError("W4A16 group size must be 128")
        if self.K % self.group:
            raise ValueError(f"K={self.K} must be a multiple of the group size {self.group}")

    @property
    def qweight_shape(self):
        return (self.N, self.K // self.packed_factor)

    @property
    def scales_shape(self):
        return (self.N, self.K // self.group)

    @property
    def packed_bytes(self) -> int:
        return self.N * self.K // 2

    @property
    def scale_bytes(self) -> int:
        return 2 * self.N * (self.K // self.group)

    def validate(self, qweight, scales):
        import torch
        if qweight.dtype != torch.int32 or tuple(qweight.shape) != self.qweight_shape:
            raise ValueError(f"qweight must be int32 {self.qweight_shape}, got {qweight.dtype} {tuple(qweight.shape)}")
        if scales.dtype != torch.float16 or tuple(scales.shape) != self.scales_shape:
            raise ValueError(f"scales must be float16 {self.scales_shape}, got {scales.dtype} {tuple(scales.shape)}")
        if not (qweight.is_contiguous() and scales.is_contiguous()):
            raise ValueError("packed tensors must be contiguous")
