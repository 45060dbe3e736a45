"""fp64 reference for the quantized linear layer (test infrastructure only).

The layer computes C[m, n] = sum_k A[m, k] * Wdq[n, k] (+ bias[n]), where Wdq
is the dequantized weight ([P1] section 2.3: the layer is handed the packed
weight, its fp16 scale and an optional bias; [P1] section 4: each output is a
dot product of an activation row with a weight row).  Its plain definition is
the matrix product with the dequantized weights, so the oracle is exactly
that product in fp64: numpy's BLAS matmul in the vectorized tier, a plain
Python loop in the loop tier.

It also returns mag[m, n] = sum_k |A[m, k] * Wdq[n, k]| (+ |bias[n]|), the
quantity the per-element tolerance is stated in.
"""

import numpy as np


def gemm_ref64(A64, wdq64, bias64=None):
    """A64 fp64 [M, K], wdq64 fp64 [N, K] -> (out fp64 [M, N], mag fp64 [M, N])."""
    A64 = np.asarray(A64, dtype=np.float64)
    wdq64 = np.asarray(wdq64, dtype=np.float64)
    if A64.ndim != 2 or wdq64.ndim != 2 or A64.shape[1] != wdq64.shape[1]:
        raise ValueError(f"shape mismatch {A64.shape} x {wdq64.shape}")
    out = A64 @ wdq64.T
    mag = np.abs(A64) @ np.abs(wdq64).T
    if bias64 is not None:
        b = np.asarray(bias64, dtype=np.float64)
        out = out + b[None, :]
        mag = mag + np.abs(b)[None, :]
    return out, mag


def gemm_ref64_loop(A, wdq, bias=None):
    """Pure-Python loop tier of ``gemm_ref64`` for tiny inputs."""
    M, K = len(A), len(A[0])
    N = len(wdq)
    out = [[0.0] * N for _ in range(M)]
    mag = [[0.0] * N for _ in range(M)]
    for m in range(M):
        for n in range(N):
            s = 0.0
            g = 0.0
            for k in range(K):
                p = float(A[m][k]) * float(wdq[n][k])
                s += p
                g += abs(p)
            if bias is not None:
                s += float(bias[n])
                g += abs(float(bias[n]))
            out[m][n] = s
            mag[m][n] = g
    return out, mag
