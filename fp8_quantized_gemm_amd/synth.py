"""Seeded synthetic inputs for the block-scaled MLP GEMM workloads.

This module holds only random-number recipes and shapes; none of the method's
arithmetic.  Both the HIP path's tests/benchmark and the CPU oracle's tests
draw their inputs here.

Workloads (synthetic stand-ins for the MaxText Llama runs measured in the
NVFP4 pretraining post, section "Performance results": sequence 8,192,
per-device batch 4, Llama 3 8B and Llama 3.1 405B MLPs with SwiGLU):

* tiny:   A [256, 256], W [256, 256]
* mx:     A, B [4096, 4096]
* 8b:     X [32768, 4096], W_gu [28672, 4096], H [32768, 14336],
          W_down [4096, 14336], dY_gu [32768, 28672], dY_down [32768, 4096]
* 405b:   X [8192, 16384], W_gu [106496, 16384], H [8192, 53248],
          W_down [16384, 53248], dY_gu [8192, 106496], dY_down [8192, 16384]

Value recipe: z = randn(shape) * sigma in float32; an independent
Bernoulli(1e-3) mask scales its entries by 50 (outliers); x = z.to(bfloat16)
(round to nearest even).  Activations: sigma 1 with outliers.  Weights:
sigma 0.02 (8B) / 0.01 (405B), no outliers.  8B gradients: sigma 1e-3, no
outliers; 405B gradients: sigma 1 with outliers.  The H operand is its own
draw (not silu(gate) * up of the forward pass).
"""

import torch

OUTLIER_P = 1e-3
OUTLIER_X = 50.0


def bf16_tensor(shape, seed, sigma=1.0, outliers=True, device="cpu"):
    """Seeded BF16 tensor: N(0, sigma^2), optional 0.1% outliers x50."""
    g = torch.Generator(device=device)
    g.manual_seed(int(seed))
    z = torch.randn(shape, generator=g, device=device, dtype=torch.float32)
    z.mul_(sigma)
    if outliers:
        mask = torch.rand(shape, generator=g, device=device, dtype=torch.float32) < OUTLIER_P
        z = torch.where(mask, z * OUTLIER_X, z)
    return z.to(torch.bfloat16)


def rht_sign_mask(seed):
    """Seeded 16-bit sign mask for the Hadamard transform (drawn on the CPU)."""
    g = torch.Generator(device="cpu")
    g.manual_seed(int(seed))
    return int(torch.randint(0, 1 << 16, (1,), generator=g).item())


# name -> (shape, seed, sigma, outliers)
WORKLOADS = {
    "tiny": {
        "A": ((256, 256), 101, 1.0, True),
        "W": ((256, 256), 102, 1.0, True),
    },
    "mx": {
        "A": ((4096, 4096), 201, 1.0, True),
        "B": ((4096, 4096), 202, 1.0, True),
    },
    "8b": {
        "X": ((32768, 4096), 301, 1.0, True),
        "W_gu": ((28672, 4096), 302, 0.02, False),
        "H": ((32768, 14336), 303, 1.0, True),
        "W_down": ((4096, 14336), 304, 0.02, False),
        "dY_gu": ((32768, 28672), 401, 1e-3, False),
        "dY_down": ((32768, 4096), 402, 1e-3, False),
    },
    "405b": {
        "X": ((8192, 16384), 501, 1.0, True),
        "W_gu": ((106496, 16384), 502, 0.01, False),
        "H": ((8192, 53248), 503, 1.0, True),
        "W_down": ((16384, 53248), 504, 0.01, False),
        "dY_gu": ((8192, 106496), 505, 1.0, True),
        "dY_down": ((8192, 16384), 506, 1.0, True),
    },
}

# stochastic-rounding seeds and Hadamard sign seeds per workload
SR_SEED = {"tiny": 1001, "mx": 1002, "8b": 1004, "405b": 1005}
RHT_SEED = {"tiny": 2001, "mx": 2002, "8b": 2004, "405b": 2005}


def workload_tensor(workload, name, device="cpu"):
    shape, seed, sigma, outl = WORKLOADS[workload][name]
    return bf16_tensor(shape, seed, sigma, outl, device)
