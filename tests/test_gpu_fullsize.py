"""Full-size parity, in the configuration bench.py times.

Workloads: the Llama-3-8B MLP layer (32,768 tokens, hidden 4096, FFN 14336)
and the Llama-3.1-405B MLP layer (8,192 tokens, hidden 16384, FFN 53248),
one GPU's share.  Every tensor is quantized on the GPU exactly as in the
benchmark step (activations row RNE + column RNE/RHT, weights 16x16, output
gradients row SR + column SR/RHT) and every GEMM runs at full size.

The oracle computes each per-tensor amax over the whole tensor itself (plain,
and of the RHT view for the column outputs), quantizes the operand rows it
needs with their global indices (so the stochastic-rounding stream is the
same), and recomputes GEMM outputs in FP64 from its own quantization.
Nothing it consumes comes from the GPU path.

Quantizers: sampled rows and columns of both orientations, bit for bit.
GEMMs (each of the six, at both sizes), against the oracle:
* one output row from every 256-row tile of M times one output column from
  every 256-column tile of N (every output tile of the kernels is checked;
  the ragged last row and column included);
* 8 whole output rows (the oracle quantizes all of B);
* 8 whole output columns (the oracle quantizes all of A), except where A is
  the SwiGLU-input gradient dY_gu (DGRAD_gu, WGRAD_gu): the oracle's
  stochastic rounding of its 0.9G elements takes minutes of host time, so
  those two GEMMs rely on the tile grid, the whole rows and the repeat;
* a second launch whose whole output must be bitwise identical.
The pre-expanded-B route (nvfp4_expand + bs_gemm_nvfp4_bx) that the step
uses for FPROP_down and DGRAD_down at 8B gets the same checks, called as
bench.py calls it.  Host work runs in a thread pool (NumPy releases the GIL).
"""

import os
import zlib
from concurrent.futures import ThreadPoolExecutor

import numpy as np
import pytest
import torch

import fp8_quantized_gemm_amd as bsq
from fp8_quantized_gemm_amd import synth
from oracle import gemm as G
from oracle import quantize as Q

from _gpu import announce, assert_bytes_equal, f32, gpu, u8

try:
    from threadpoolctl import threadpool_limits
except ImportError:                      # BLAS threads then stay as configured
    threadpool_limits = None

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
        signs = synth.rht_sign_mask(synth.RHT_SEED[workload])
        step = 2048                      # whole 16-row RHT chunks per work item

        def part(r0):
            if rht:
                return Q.tensor_amax_rht_cols(x[r0:r0 + step], signs)
            return Q.tensor_amax(Q.as_f32(x[r0:r0 + step]))

        _cache[key] = np.float32(max(_pool_map(part, range(0, x.shape[0], step))))
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
NO_FULL_COLS = {"dY_gu"}                 # A operands too large for the oracle's SR at full size
WORKERS = max(1, min(16, os.cpu_count() or 1))


def _chunk(n):
    """Operand rows per oracle work item: a multiple of 16 (whole 16x16
    tiles), at most 1024, and at least four items per worker when n allows."""
    c = -(-n // (4 * WORKERS))
    return int(min(1024, max(16, -(-c // 16) * 16)))


def _shape(workload, name, orient):
    R, C = synth.WORKLOADS[workload][name][0]
    return (R, C) if orient == "row" else (C, R)


def _side_amax(workload, name, orient):
    return _amax(workload, name, PLAN[name][1] if orient == "col" else False)


def _tile_grid(n, rng, tile=256):
    """One index from every `tile`-sized tile of [0, n); the last is n - 1."""
    t = (n + tile - 1) // tile
    idx = np.minimum(np.arange(t) * tile + rng.integers(0, tile, t), n - 1)
    idx[-1] = n - 1
    return idx


def _pool_map(fn, items):
    def run():
        with ThreadPoolExecutor(WORKERS) as ex:
            return list(ex.map(fn, items))
    if threadpool_limits is None:
        return run()
    with threadpool_limits(1):
        return run()


def _ref_rows(workload, an, ao, mi, bn, bo):
    """FP64 oracle of whole output rows mi: every row of B, in chunks of rows."""
    ac, as_ = _oracle_rows(workload, an, ao, mi)
    aa, ba = _side_amax(workload, an, ao), _side_amax(workload, bn, bo)
    N = _shape(workload, bn, bo)[0]
    out = np.empty((len(mi), N))
    ch = _chunk(N)

    def work(n0):
        n = np.arange(n0, min(n0 + ch, N))
        bc, bs = _oracle_rows(workload, bn, bo, n)
        out[:, n0:n0 + len(n)] = G.gemm_nvfp4(ac, as_, aa, bc, bs, ba)

    _pool_map(work, range(0, N, ch))
    return out


def _ref_cols(workload, an, ao, bn, bo, ni):
    """FP64 oracle of whole output columns ni: every row of A, in chunks of rows."""
    bc, bs = _oracle_rows(workload, bn, bo, ni)
    aa, ba = _side_amax(workload, an, ao), _side_amax(workload, bn, bo)
    M = _shape(workload, an, ao)[0]
    out = np.empty((M, len(ni)))
    ch = _chunk(M)

    def work(m0):
        m = np.arange(m0, min(m0 + ch, M))
        ac, as_ = _oracle_rows(workload, an, ao, m)
        out[m0:m0 + len(m), :] = G.gemm_nvfp4(ac, as_, aa, bc, bs, ba)

    _pool_map(work, range(0, M, ch))
    return out


def _compare(what, got, ref):
    rep = G.tolerance_report(got.float().cpu().numpy().astype(np.float64), ref)
    print(what, rep, flush=True)
    assert rep["passed"], (what, rep)


def _run_gemm(workload, an, ao, bn, bo, bx):
    """The GEMM as bench.py launches it: bs_gemm, or with bx the weight
    orientation expanded once (nvfp4_expand) and bs_gemm_nvfp4_bx."""
    qa, qb = _gpu_quant(workload, an), _gpu_quant(workload, bn)
    if not bx:
        return lambda: bsq.bs_gemm("nvfp4", qa[ao + "_codes"], qa[ao + "_scales"], qb[bo + "_codes"],
                                   qb[bo + "_scales"], qa[ao + "_amax"], qb[bo + "_amax"])
    wx = bsq.nvfp4_expand(qb[bo + "_codes"], qb[bo + "_scales"])
    return lambda: bsq.bs_gemm_nvfp4_bx(qa[ao + "_codes"], qa[ao + "_scales"], qa[ao + "_amax"], wx,
                                        qb[bo + "_amax"])


def _check_gemm(workload, gname, an, ao, bn, bo, bx=False):
    M, K = _shape(workload, an, ao)
    N, K2 = _shape(workload, bn, bo)
    assert K == K2
    announce("full-size gemm", workload, gname, (M, N, K), "bx" if bx else "")
    launch = _run_gemm(workload, an, ao, bn, bo, bx)
    C = launch()
    torch.cuda.synchronize()
    C2 = launch()
    torch.cuda.synchronize()
    assert torch.equal(C.view(torch.int16), C2.view(torch.int16)), "second launch differs"
    del C2
    rng = np.random.default_rng(_seed(workload, gname))
    dev = lambda i: torch.as_tensor(i, device="cuda")
    # every output tile
    mi, ni = _tile_grid(M, rng), _tile_grid(N, rng)
    ac, as_ = _oracle_rows(workload, an, ao, mi)
    bc, bs = _oracle_rows(workload, bn, bo, ni)
    ref = G.gemm_nvfp4(ac, as_, _side_amax(workload, an, ao), bc, bs, _side_amax(workload, bn, bo))
    _compare(f"{gname} {workload} tile grid {len(mi)}x{len(ni)}", C[dev(mi)][:, dev(ni)], ref)
    # whole rows
    rows = np.sort(rng.choice(M, 8, replace=False))
    rows[-1] = M - 1
    _compare(f"{gname} {workload} 8 full rows", C[dev(rows)], _ref_rows(workload, an, ao, rows, bn, bo))
    # whole columns
    if an not in NO_FULL_COLS:
        cols = np.sort(rng.choice(N, 8, replace=False))
        cols[-1] = N - 1
        _compare(f"{gname} {workload} 8 full columns", C[:, dev(cols)],
                 _ref_cols(workload, an, ao, bn, bo, cols))
    del C


# 8B first (quantizers, then GEMMs on the same resident tensors), then 405B.

@pytest.mark.parametrize("name", list(PLAN))
def test_quantize_8b_sampled(name):
    _check_quant("8b", name)


@pytest.mark.parametrize("g", GEMMS, ids=[g[0] for g in GEMMS])
def test_gemm_8b_sampled(g):
    _check_gemm("8b", *g)


@pytest.mark.parametrize("g", [g for g in GEMMS if g[0] in ("FPROP_down", "DGRAD_down")],
                         ids=["FPROP_down", "DGRAD_down"])
def test_gemm_8b_pre_expanded_weight(g):
    """The route the 8B step takes for the two GEMMs whose B is W_down."""
    _check_gemm("8b", *g, bx=True)


@pytest.mark.parametrize("name", list(PLAN))
def test_quantize_405b_sampled(name):
    _check_quant("405b", name)


@pytest.mark.parametrize("g", GEMMS, ids=[g[0] for g in GEMMS])
def test_gemm_405b_sampled(g):
    _check_gemm("405b", *g)
