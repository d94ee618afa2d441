"""Shared helpers for the GPU parity tests."""

import os
import sys

import numpy as np
import pytest
import torch

import fp8_quantized_gemm_amd as bsq

HAVE_GPU = torch.cuda.is_available()

gpu = [pytest.mark.gpu,
       pytest.mark.skipif(not HAVE_GPU, reason="needs an MI355X GPU"),
       pytest.mark.skipif(not os.path.exists(bsq.LIB_PATH), reason="libbsq.so not built")]


def announce(*what):
    """Name the case on stdout before a GPU step (survives a lost box)."""
    print("[gpu case]", *what, flush=True)
    sys.stdout.flush()


def bits(t):
    """BF16 tensor (any device) -> numpy uint16 bit patterns."""
    return t.detach().contiguous().cpu().view(torch.int16).numpy().view(np.uint16)


def u8(t):
    return t.detach().contiguous().cpu().numpy()


def f32(t):
    return t.detach().float().cpu().numpy()


def from_bits(b, device="cuda"):
    """numpy uint16 BF16 bits -> BF16 tensor on device."""
    return torch.from_numpy(np.ascontiguousarray(b).view(np.int16)).view(torch.bfloat16).to(device)


def assert_bytes_equal(got, want, what):
    got = np.asarray(got)
    want = np.asarray(want)
    assert got.shape == want.shape, (what, got.shape, want.shape)
    if not np.array_equal(got, want):
        bad = np.argwhere(got != want)
        i = tuple(bad[0])
        raise AssertionError(f"{what}: {len(bad)} of {got.size} bytes differ; first at {i}: "
                             f"got {got[i]:#04x} want {want[i]:#04x}")
