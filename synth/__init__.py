"""Seeded synthetic operands for the FP8 linear layer.

Shared by the tests, the bench and the oracle's callers.  This module holds
only random-number generation and bf16 rounding of the drawn values; none of
the method's arithmetic (amax, scaling, encoding, GEMMs) lives here.

Every tensor is drawn on the CPU with ``torch.Generator('cpu')`` seeded as
stated, as fp32 ``randn * sigma`` (optionally with a Bernoulli outlier mask
scaled by ``outlier_factor``) and rounded to bf16 by torch's
round-to-nearest-even conversion.  Operands are drawn in the order X, W, dY
from one generator per workload, so the same seed gives the same bytes on any
host.  The workloads mirror the synthetic normal operands of the isolated
linear timings in "Native FP8 MLP reconstruction" (X ~ N(0,1), W ~ N(0,0.02),
dY ~ N(0,1e-3)); their shapes are those of the configurations below.
"""
import hashlib

import torch

# name -> (N, K, M, sigma_x, sigma_w, sigma_dy, outlier_frac, scaling)
WORKLOADS = {
    "linear_512x512_n1024": (1024, 512, 512, 1.0, 0.02, 1e-3, 0.0, "tensor"),
    "linear_512x2048_n131072": (131072, 512, 2048, 1.0, 0.02, 1e-3, 0.0, "tensor"),
    "linear_2048x512_n131072": (131072, 2048, 512, 1.0, 0.02, 1e-3, 0.0, "tensor"),
    "linear_512x8192_n131072_block": (131072, 512, 8192, 1.0, 1.0, 1.0, 0.01, "block"),
    "linear_8192x8192_n16384": (16384, 8192, 8192, 1.0, 1.0, 1.0, 0.0, "tensor"),
    "linear_8192x8192_n16384_block": (16384, 8192, 8192, 1.0, 1.0, 1.0, 0.0, "block"),
    "linear_512x8192_n262144": (262144, 512, 8192, 1.0, 1.0, 1.0, 0.0, "tensor"),
    "linear_512x8192_n262144_block": (262144, 512, 8192, 1.0, 1.0, 1.0, 0.0, "block"),
}


def normal_bf16(shape, sigma, gen, outlier_frac=0.0, outlier_factor=100.0, device="cpu"):
    """fp32 N(0, sigma^2) draws rounded to bf16; with outlier_frac > 0 a
    Bernoulli(outlier_frac) mask drawn next from the same generator selects
    entries multiplied by outlier_factor before the bf16 rounding."""
    x = torch.randn(shape, generator=gen, dtype=torch.float32, device=device)
    if sigma != 1.0:
        x.mul_(sigma)
    if outlier_frac > 0.0:
        mask = torch.rand(shape, generator=gen, dtype=torch.float32, device=device) < outlier_frac
        x[mask] *= outlier_factor
    return x.to(torch.bfloat16)


def operands(N, K, M, seed=0, sigma_x=1.0, sigma_w=0.02, sigma_dy=1e-3, outlier_frac=0.0):
    """X [N, K], W [M, K], dY [N, M] as CPU bf16 tensors, drawn in that order."""
    g = torch.Generator(device="cpu")
    g.manual_seed(seed)
    x = normal_bf16((N, K), sigma_x, g, outlier_frac)
    w = normal_bf16((M, K), sigma_w, g, outlier_frac)
    dy = normal_bf16((N, M), sigma_dy, g, outlier_frac)
    return x, w, dy


def workload(name, seed=0, n_override=None):
    N, K, M, sx, sw, sdy, frac, scaling = WORKLOADS[name]
    if n_override is not None:
        N = n_override
    x, w, dy = operands(N, K, M, seed, sx, sw, sdy, frac)
    return {"x": x, "w": w, "dy": dy, "N": N, "K": K, "M": M, "scaling": scaling}


def bits(t):
    """bf16 tensor -> numpy uint16 bit patterns (CPU copy)."""
    return t.detach().cpu().contiguous().view(torch.int16).numpy().view("uint16")


def sha256(t):
    return hashlib.sha256(bits(t).tobytes()).hexdigest()


def operands_on_device(N, K, M, seed=0, sigma_x=1.0, sigma_w=0.02, sigma_dy=1e-3, device="cuda",
                       outlier_frac=0.0):
    """Same distributions as ``operands`` drawn with a seeded device generator
    (for large runs where CPU drawing would dominate); drawn in the order
    X, W, dY."""
    g = torch.Generator(device=device)
    g.manual_seed(seed)
    x = normal_bf16((N, K), sigma_x, g, outlier_frac, device=device)
    w = normal_bf16((M, K), sigma_w, g, outlier_frac, device=device)
    dy = normal_bf16((N, M), sigma_dy, g, outlier_frac, device=device)
    return x, w, dy


def workload_on_device(name, seed=0, device="cuda"):
    """A named workload drawn with the seeded device generator."""
    N, K, M, sx, sw, sdy, frac, scaling = WORKLOADS[name]
    x, w, dy = operands_on_device(N, K, M, seed, sx, sw, sdy, device, frac)
    return {"x": x, "w": w, "dy": dy, "N": N, "K": K, "M": M, "scaling": scaling}
