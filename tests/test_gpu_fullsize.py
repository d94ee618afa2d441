"""Full-size parity on sampled outputs, in the configuration bench.py times.

Workloads: the Llama-3-8B MLP layer (32,768 tokens, hidden 4096, FFN 14336)
and the Llama-3.1-405B MLP layer (8,192 tokens, hidden 16384, FFN 53248),
one GPU's share.  Every tensor is quantized on the GPU exactly as in the
benchmark step (activations row RNE + column RNE/RHT, weights 16x16, output
gradients row SR + column SR/RHT) and every GEMM runs at full size.

The oracle computes each per-tensor amax over the whole tensor itself (plain,
and of the RHT view for the column outputs), quantizes sampled rows and
columns with their global indices (so the stochastic-rounding stream is the
same), and recomputes sampled GEMM outputs in FP64 from its own quantization
of the sampled operand rows.  Nothing it consumes comes from the GPU path.
Each test stays well under a minute of host work.
"""

import zlib

import numpy as np
import pytest
import torch

import fp8_quantized_gemm_amd as bsq
from fp8_quantized_gemm_amd import synth
from oracle import gemm as G
from oracle import quantize as Q

from _gpu import announce, assert_bytes_equal, f32, gpu, u8

pytestmark = gpu

RNE, SR = "rne", "sr"
# tensor -> (rounding, RHT on the column output, block rows)
PLAN = {"X": (RNE, True, 1), "W_gu": (RNE, False, 16), "H": (RNE, True, 1),
        "W_down": (RNE, False, 16), "dY_gu": (SR, True, 1), "dY_down": (SR, True, 1)}

_cache = {}


def _dev(workload, name):
    key = ("dev", workload, name)
    if key not in _cache:
        if any(k[1] != workload for k in _cache):      # one workload resident at a time
            _cache.clear()
            torch.cuda.empty_cache()
        _cache[key] = synth.workload_tensor(workload, name, "cuda")
    return _cache[key]


def _seed(*parts):
    return zlib.crc32(repr(parts).encode())


def _host_bits(workload, name):
    key = ("host", workload, name)
    if key not in _cache:
        x = _dev(workload, name)
        _cache[key] = x.cpu().view(torch.int16).numpy().view(np.uint16)
    return _cache[key]


def _amax(workload, name, rht):
    """Oracle per-tensor amax over the whole tensor (chunked over rows)."""
    key = ("amax", workload, name, rht)
    if key not in _cache:
        x = _host_bits(workload, name)
        if rht:
            a = Q.tensor_amax_rht_cols(x, synth.rht_sign_mask(synth.RHT_SEED[workload]))
        else:
            a = np.float32(0.0)
            for r0 in range(0, x.shape[0], 4096):
                a = max(a, Q.tensor_amax(Q.as_f32(x[r0:r0 + 4096])))
        _cache[key] = np.float32(a)
    return _cache[key]


def _gpu_quant(workload, name):
    key = ("q", workload, name)
    if key not in _cache:
        rnd, rht, br = PLAN[name]
        x = _dev(workload, name)
        _cache[key] = bsq.quantize_transpose(
            x, "nvfp4", br, rnd, synth.SR_SEED[workload], 0, rht_col=rht,
            rht_signs=synth.rht_sign_mask(synth.RHT_SEED[workload]))
        torch.cuda.synchronize()
    return _cache[key]


def _tiles(idx):
    """Expand indices to their whole 16-element tiles (sorted, unique)."""
    t = np.unique(np.asarray(idx) // 16)
    return (t[:, None] * 16 + np.arange(16)[None, :]).ravel()


def _oracle_rows(workload, name, orient, idx):
    """Oracle NVFP4 quantization of rows `idx` of orientation `orient` ('row' =
    x, 'col' = x^T) of a workload tensor, as the benchmark configures it.
    Returns (codes, scales) for exactly those rows."""
    rnd, rht, br = PLAN[name]
    x = _host_bits(workload, name)
    idx = np.asarray(idx)
    rows = _tiles(idx) if br == 16 else np.unique(idx)
    if orient == "row":
        data = x[rows]
        amax = _amax(workload, name, False)
        use_rht = False
    else:
        data = np.ascontiguousarray(x[:, rows].T)
        amax = _amax(workload, name, rht)
        use_rht = rht
    codes, scales, _ = Q.nvfp4_quantize(
        data, br, rnd, synth.SR_SEED[workload], 0, stream=0 if orient == "row" else 1,
        rht=use_rht, rht_signs=synth.rht_sign_mask(synth.RHT_SEED[workload]), amax=amax,
        row_ids=rows)
    pos = {r: i for i, r in enumerate(rows)}
    sel = np.array([pos[r] for r in idx])
    return codes[sel], scales[sel]


def _rows_from_gpu(t, idx):
    return u8(t[torch.as_tensor(np.asarray(idx), device=t.device)])


def _check_quant(workload, name):
    announce("full-size quantize", workload, name, synth.WORKLOADS[workload][name][0])
    rnd, rht, br = PLAN[name]
    out = _gpu_quant(workload, name)
    R, C = synth.WORKLOADS[workload][name][0]
    assert f32(out["row_amax"])[0] == _amax(workload, name, False)
    assert f32(out["col_amax"])[0] == _amax(workload, name, rht)
    rng = np.random.default_rng(_seed(workload, name))
    ridx = np.sort(rng.choice(R, 24, replace=False))
    cidx = np.sort(rng.choice(C, 24, replace=False))
    ridx[0], cidx[0] = R - 1, C - 1                 # the ragged ends of each orientation
    oc, os_ = _oracle_rows(workload, name, "row", ridx)
    assert_bytes_equal(_rows_from_gpu(out["row_codes"], ridx), oc, f"{name} row codes")
    assert_bytes_equal(_rows_from_gpu(out["row_scales"], ridx), os_, f"{name} row scales")
    oc, os_ = _oracle_rows(workload, name, "col", cidx)
    assert_bytes_equal(_rows_from_gpu(out["col_codes"], cidx), oc, f"{name} col codes")
    assert_bytes_equal(_rows_from_gpu(out["col_scales"], cidx), os_, f"{name} col scales")


# (name, A tensor, A orientation, B tensor, B orientation)
GEMMS = [("FPROP_gu", "X", "row", "W_gu", "row"), ("FPROP_down", "H", "row", "W_down", "row"),
         ("DGRAD_down", "dY_down", "row", "W_down", "col"), ("WGRAD_down", "dY_down", "col", "H", "col"),
         ("DGRAD_gu", "dY_gu", "row", "W_gu", "col"), ("WGRAD_gu", "dY_gu", "col", "X", "col")]


def _shape(workload, name, orient):
    R, C = synth.WORKLOADS[workload][name][0]
    return (R, C) if orient == "row" else (C, R)


def _check_gemm(workload, gname, an, ao, bn, bo):
    M, K = _shape(workload, an, ao)
    N, K2 = _shape(workload, bn, bo)
    assert K == K2
    announce("full-size gemm", workload, gname, (M, N, K))
    qa, qb = _gpu_quant(workload, an), _gpu_quant(workload, bn)
    C = bsq.bs_gemm("nvfp4", qa[ao + "_codes"], qa[ao + "_scales"], qb[bo + "_codes"],
                    qb[bo + "_scales"], qa[ao + "_amax"], qb[bo + "_amax"])
    torch.cuda.synchronize()
    rng = np.random.default_rng(_seed(workload, gname))
    mi = np.sort(rng.choice(M, 12, replace=False))
    ni = np.sort(rng.choice(N, 12, replace=False))
    mi[0], ni[0] = M - 1, N - 1
    ac, as_ = _oracle_rows(workload, an, ao, mi)
    bc, bs = _oracle_rows(workload, bn, bo, ni)
    a_amax = _amax(workload, an, PLAN[an][1] if ao == "col" else False)
    b_amax = _amax(workload, bn, PLAN[bn][1] if bo == "col" else False)
    ref = G.gemm_nvfp4(ac, as_, a_amax, bc, bs, b_amax)
    got = C[torch.as_tensor(mi, device="cuda")][:, torch.as_tensor(ni, device="cuda")]
    rep = G.tolerance_report(got.float().cpu().numpy().astype(np.float64), ref)
    print(gname, workload, rep)
    assert rep["passed"], rep
    del C


# 8B first (quantizers, then GEMMs on the same resident tensors), then 405B.

@pytest.mark.parametrize("name", list(PLAN))
def test_quantize_8b_sampled(name):
    _check_quant("8b", name)


@pytest.mark.parametrize("g", GEMMS, ids=[g[0] for g in GEMMS])
def test_gemm_8b_sampled(g):
    _check_gemm("8b", *g)


@pytest.mark.parametrize("name", list(PLAN))
def test_quantize_405b_sampled(name):
    _check_quant("405b", name)


@pytest.mark.parametrize("g", GEMMS, ids=[g[0] for g in GEMMS])
def test_gemm_405b_sampled(g):
    _check_gemm("405b", *g)
