"""Seeded synthetic inputs shared by the tests, the bench and the smoke check.

This module only draws random weights and activations and names the workload
shapes.  It holds none of the quantization arithmetic: it neither packs nor
unpacks, and both the HIP path and the oracle take its outputs as plain
inputs.

Recipe
------
* Weights: fp32 W[N, K] ~ N(0, 0.02^2) (sigma = 0.02 is the standard
  deviation), drawn with ``numpy.random.default_rng(seed).normal`` on the host
  or, for workloads too large to draw on the host in reasonable time, with a
  seeded ``torch.Generator`` on the device (``weights_device``; a sample of
  rows is copied back for checking).
* Activations: A[M, K] ~ N(0, 1), drawn in fp64 with
  ``default_rng(seed).standard_normal`` then rounded to fp16 by numpy, or to
  bf16 by torch from the fp32 value.
* Activation-order groups (``group_index``): a seeded random permutation
  ranks the input columns and group g takes ranks 128g .. 128g + 127.
* Seeds: the smallest case (256 x 256, M = 1) uses seed 0 for both, weights
  drawn first.  Every other tensor gets ``seed_for(*names)``, a CRC-32 of its
  name, so a weight matrix is shared by every M it is used with.

Shapes are the linear layers of Llama-3-8B (hidden 4096, intermediate 14336,
8 KV heads of 128) and Llama-3-70B (hidden 8192, intermediate 28672, 8 KV
heads of 128), stored as (N = out features, K = in features).
"""

import zlib

import numpy as np

SIGMA = 0.02

# (N, K) per projection, in layer order
LLAMA3_8B = {
    "q": (4096, 4096),
    "k": (1024, 4096),
    "v": (1024, 4096),
    "o": (4096, 4096),
    "gate": (14336, 4096),
    "up": (14336, 4096),
    "down": (4096, 14336),
}
LLAMA3_8B_LAYERS = 32

LLAMA3_70B = {
    "q": (8192, 8192),
    "k": (1024, 8192),
    "v": (1024, 8192),
    "o": (8192, 8192),
    "gate": (28672, 8192),
    "up": (28672, 8192),
    "down": (8192, 28672),
}
LLAMA3_70B_LAYERS = 80

# the four distinct Llama-3-8B shapes (q/o, k/v, gate/up, down)
SHAPES_8B = [(4096, 4096), (1024, 4096), (14336, 4096), (4096, 14336)]


def seed_for(*names) -> int:
    """Deterministic 32-bit seed from a tensor's name parts."""
    return zlib.crc32("/".join(str(n) for n in names).encode())


def weights(N: int, K: int, seed: int, sigma: float = SIGMA) -> np.ndarray:
    """fp32 [N, K] ~ N(0, sigma^2) on the host."""
    rng = np.random.default_rng(seed)
    return rng.normal(0.0, sigma, (N, K)).astype(np.float32)


def activations(M: int, K: int, seed: int, dtype: str = "f16"):
    """torch CPU tensor [M, K] ~ N(0, 1) in fp16 or bf16."""
    import torch

    a = np.random.default_rng(seed).standard_normal((M, K))
    return _to_torch(a, dtype)


def _to_torch(a64: np.ndarray, dtype: str):
    import torch

    if dtype == "f16":
        return torch.from_numpy(a64.astype(np.float16))
    if dtype == "bf16":
        return torch.from_numpy(a64.astype(np.float32)).to(torch.bfloat16)
    raise ValueError(f"unknown activation dtype {dtype!r}")


def smallest_case():
    """The 256 x 256 case at M = 1: seed 0, weights drawn first, then A (fp16)."""
    rng = np.random.default_rng(0)
    W = rng.normal(0.0, SIGMA, (256, 256)).astype(np.float32)
    a = rng.standard_normal((1, 256))
    return W, _to_torch(a, "f16")


def group_index(K: int, seed: int, group: int = 128) -> np.ndarray:
    """Activation-order group of each input column, int32 [K]: the columns
    take a seeded random rank (a stand-in for an ordering by importance) and
    consecutive ranks form the groups, so every group holds ``group``
    columns scattered over the row."""
    rank = np.random.default_rng(seed).permutation(K)
    return (rank // group).astype(np.int32)


def weights_device(N: int, K: int, seed: int, device, sigma: float = SIGMA):
    """fp32 [N, K] ~ N(0, sigma^2) drawn on ``device`` with a seeded torch generator."""
    import torch

    g = torch.Generator(device=device)
    g.manual_seed(seed)
    w = torch.randn((N, K), generator=g, device=device, dtype=torch.float32)
    return w.mul_(sigma)


def activations_device(M: int, K: int, seed: int, dtype: str, device):
    """[M, K] ~ N(0, 1) drawn on ``device`` (fp32, then rounded by torch)."""
    import torch

    g = torch.Generator(device=device)
    g.manual_seed(seed)
    a = torch.randn((M, K), generator=g, device=device, dtype=torch.float32)
    return a.to(torch.float16 if dtype == "f16" else torch.bfloat16)


# ---------------------------------------------------------------- edge cases
#
# Inputs that stress the accumulation rather than the pack rule: weight rows
# with very few nonzero values and scales across the binary16 range, next to
# dense rows, and activations with outliers or of tiny magnitude.

EDGE_SCALES = (1.0, 0.5, 3.0e-3, 6.0e4, 1.0e-4, 7.3, 1.5e3, 0.02)
ACT_REGIMES = ("dense", "outlier", "tiny")


def sparse_ternary_weights(N: int, K: int, seed: int) -> np.ndarray:
    """fp32 [N, K] whose rows cycle through: all zero; one kept entry (+s or
    -s); 2 .. 8 kept entries of random sign; dense N(0, 0.02); dense with a
    large spread (N(0, 2e4)).  A row of k entries of magnitude s and zeros
    elsewhere keeps exactly those k entries (s > 0.7 k s / K) with scale s;
    s cycles through EDGE_SCALES."""
    rng = np.random.default_rng(seed)
    W = np.zeros((N, K), dtype=np.float32)
    kinds = 12
    for n in range(N):
        kind = n % kinds
        s = EDGE_SCALES[(n // kinds) % len(EDGE_SCALES)]
        if kind == 0:
            continue
        if kind in (1, 2):
            W[n, rng.integers(K)] = s if kind == 1 else -s
        elif kind <= 9:
            k = kind - 1  # 2 .. 8 entries
            cols = rng.choice(K, size=k, replace=False)
            W[n, cols] = np.where(rng.integers(2, size=k) == 0, -s, s)
        elif kind == 10:
            W[n] = rng.normal(0.0, SIGMA, K)
        else:
            W[n] = rng.normal(0.0, 2.0e4, K)
    return W


def sparse_w4_weights(N: int, K: int, seed: int) -> np.ndarray:
    """fp32 [N, K] with 128-column groups of these kinds, cycling over rows
    and groups: all zero; one nonzero value (magnitudes from EDGE_SCALES); one
    large value among values 1e-3 times smaller (which quantize to zero);
    dense N(0, 0.02); dense N(0, 0.02) shifted by a per-group offset (zero
    points spread over 0 .. 15 in the asymmetric format)."""
    rng = np.random.default_rng(seed)
    G = K // 128
    W = np.zeros((N, K), dtype=np.float32)
    for n in range(N):
        for g in range(G):
            kind = (n + 3 * g) % 5
            s = EDGE_SCALES[(n + g) % len(EDGE_SCALES)]
            blk = W[n, 128 * g:128 * (g + 1)]
            if kind == 1:
                blk[rng.integers(128)] = s * (1 if rng.integers(2) else -1)
            elif kind == 2:
                blk[:] = rng.normal(0.0, 1.0e-3 * s, 128)
                blk[rng.integers(128)] = s
            elif kind == 3:
                blk[:] = rng.normal(0.0, SIGMA, 128)
            elif kind == 4:
                blk[:] = rng.normal(0.0, SIGMA, 128) + rng.uniform(-0.03, 0.03)
    return W


def activations_regime(M: int, K: int, seed: int, regime: str, dtype: str = "f16"):
    """torch CPU tensor [M, K]: "dense" N(0, 1); "outlier" N(0, 1) with eight
    entries per row replaced by +-U(200, 1000); "tiny" N(0, 1) * 2^-12 (a
    few values fall into the binary16 subnormal range)."""
    rng = np.random.default_rng(seed)
    a = rng.standard_normal((M, K))
    if regime == "outlier":
        for m in range(M):
            cols = rng.choice(K, size=min(8, K), replace=False)
            a[m, cols] = rng.uniform(200.0, 1000.0, len(cols)) * np.where(rng.integers(2, size=len(cols)) == 0, -1, 1)
    elif regime == "tiny":
        a = a * 2.0 ** -12
    elif regime != "dense":
        raise ValueError(f"unknown activation regime {regime!r}")
    return _to_torch(a, dtype)
