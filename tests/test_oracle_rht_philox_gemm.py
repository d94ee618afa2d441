"""Pins for the oracle's RHT, Philox and GEMM (CPU only).

* RHT: the butterfly equals scipy.linalg.hadamard(16) (Sylvester order) times
  the sign diagonal, / 4 (exactly on small-integer inputs, within float32
  rounding otherwise); R is orthogonal in float64; norms are preserved; the
  WGRAD identity (R dY)^T (R X) = dY^T X holds.
* Philox4x32-10: equals rocRAND's installed Philox4x32-10 engine (an
  independent implementation) on random keys and counters.
* GEMM: exact Fraction arithmetic from the codes on 16x16x32 equals the FP64
  oracle; a planted mistake (transposed operand, dropped scale) fails the
  tolerance rule.
"""

import os
import shutil
import subprocess
import tempfile
from fractions import Fraction

import numpy as np
import pytest
import scipy.linalg
import torch

from oracle import formats as F
from oracle import gemm as G
from oracle import philox as P
from oracle import quantize as Q
from oracle import rht as R
from fp8_quantized_gemm_amd import synth

HERE = os.path.dirname(os.path.abspath(__file__))


def _D(signs):
    return np.array([-1.0 if (signs >> i) & 1 else 1.0 for i in range(16)])


# ---------------------------------------------------------------- RHT

def test_rht_matches_scipy_hadamard_exact_on_integers():
    rng = np.random.default_rng(0)
    H = scipy.linalg.hadamard(16).astype(np.float64)
    for signs in (0, 0xFFFF, 0x1234, 0xA5C3):
        x = rng.integers(-64, 64, (50, 16)).astype(np.float32)
        got = R.rht16(x, signs).astype(np.float64)
        want = (x.astype(np.float64) * _D(signs)) @ H.T / 4.0
        assert np.array_equal(got, want)


def test_rht_matches_scipy_within_float32():
    rng = np.random.default_rng(1)
    H = scipy.linalg.hadamard(16).astype(np.float64)
    x = rng.standard_normal((1000, 16)).astype(np.float32)
    got = R.rht16(x, 0x5A5A).astype(np.float64)
    want = (x.astype(np.float64) * _D(0x5A5A)) @ H.T / 4.0
    assert np.max(np.abs(got - want)) <= 4 * 2.0 ** -24 * np.max(np.abs(x)) * 4


def test_rht_orthogonal_and_norm():
    for signs in (0, 0x8001, 0xBEEF):
        Rm = R.rht_matrix_f64(signs)
        assert np.array_equal(Rm @ Rm.T, np.eye(16))
    x = np.random.default_rng(2).standard_normal((500, 16)).astype(np.float32)
    y = R.rht16(x, 0xBEEF).astype(np.float64)
    n0 = np.linalg.norm(x.astype(np.float64), axis=1)
    assert np.allclose(np.linalg.norm(y, axis=1), n0, rtol=1e-6)
    # R^T (R x) = x
    back = y @ R.rht_matrix_f64(0xBEEF)
    assert np.allclose(back, x, atol=1e-6)


def test_rht_wgrad_identity():
    rng = np.random.default_rng(3)
    T, N, K = 64, 24, 40
    dY = rng.standard_normal((T, N))
    X = rng.standard_normal((T, K))
    Rm = R.rht_matrix_f64(0x1F2E)
    Rb = np.kron(np.eye(T // 16), Rm)            # block-diagonal along tokens
    lhs = (Rb @ dY).T @ (Rb @ X)
    rhs = dY.T @ X
    assert np.max(np.abs(lhs - rhs)) <= 1e-12 * np.sqrt(np.mean(rhs ** 2))


def test_rht_along_rows_chunking():
    x = np.arange(64, dtype=np.float32).reshape(2, 32)
    y = R.rht_along_rows(x, 3)
    assert np.array_equal(y[1, 16:], R.rht16(x[1, 16:], 3))


# ---------------------------------------------------------------- Philox

def _build_rocrand_helper():
    hipcc = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    if not os.path.exists(hipcc) or not os.path.exists("/opt/rocm/include/rocrand/rocrand_kernel.h"):
        return None
    out = os.path.join(tempfile.mkdtemp(), "rocrand_philox_words")
    src = os.path.join(HERE, "helpers", "rocrand_philox_words.cpp")
    r = subprocess.run([hipcc, "--offload-arch=gfx950", "-x", "hip", "--cuda-host-only", "-O1",
                        src, "-o", out], capture_output=True, text=True, cwd=tempfile.gettempdir())
    return out if r.returncode == 0 else None


def test_philox_matches_rocrand_engine():
    exe = _build_rocrand_helper()
    if exe is None:
        pytest.skip("rocRAND headers / hipcc not available: Philox cross-check skipped")
    rng = np.random.default_rng(4)
    # rocRAND takes counter words 0..1 as a number-of-draws offset (4 per call) in 64 bits,
    # so word 1 stays below 2**30 here; words 0, 2, 3 and the key span their full range.
    rows = [(0, 0, 0, 0, 0), (2 ** 64 - 1, 2 ** 32 - 1, 2 ** 30 - 1, 2 ** 32 - 1, 2 ** 32 - 1)]
    for _ in range(200):
        c = [int(v) for v in rng.integers(0, 2 ** 32, 4)]
        c[1] >>= 2
        rows.append((int(rng.integers(0, 2 ** 63)) * 2 + int(rng.integers(0, 2)),) + tuple(c))
    inp = "\n".join(" ".join(str(v) for v in r) for r in rows) + "\n"
    out = subprocess.run([exe], input=inp, capture_output=True, text=True, check=True).stdout
    ref = np.array([[int(v) for v in line.split()] for line in out.strip().split("\n")], dtype=np.uint64)
    for row, want in zip(rows, ref):
        seed = row[0]
        got = P.philox4x32_10(row[1:], (seed & 0xFFFFFFFF, seed >> 32))
        assert [int(g) for g in got] == [int(w) for w in want]


def test_sr_stream_map_words():
    # element idx takes 16-bit half (idx & 7) of the Philox call at counter idx >> 3
    idx = np.arange(64, dtype=np.uint64) + np.uint64(2 ** 35)
    r = P.sr_random16(idx, seed=0x123456789, offset=5, stream=1)
    for k in (0, 7, 8, 63):
        g = int(idx[k]) >> 3
        w = P.philox4x32_10((g & 0xFFFFFFFF, g >> 32, 5, 1), (0x23456789, 0x1))
        want = (int(w[(int(idx[k]) & 7) >> 1]) >> (16 * (int(idx[k]) & 1))) & 0xFFFF
        assert int(r[k]) == want
    u = P.sr_random16(np.arange(200000, dtype=np.uint64), 1, 0, 0).astype(np.float64)
    assert abs(u.mean() / 65535 - 0.5) < 0.005


def test_sr_decisions_follow_an_independent_philox():
    """End to end through the oracle's SR quantizer: MXFP4 blocks [4, 0.25 x 31]
    have block exponent 0, so every 0.25 sits exactly halfway between E2M1
    magnitudes 0 and 0.5 and rounds up iff its 16-bit word is below 2^15.
    The expected decisions come from rocRAND's installed Philox4x32-10 engine
    (not the oracle's generator): element idx of a rowwise output uses the
    16-bit half (idx & 1) of word (idx & 7) >> 1 of the call at counter
    (idx >> 3, offset, stream)."""
    exe = _build_rocrand_helper()
    if exe is None:
        pytest.skip("rocRAND headers / hipcc not available: SR cross-check skipped")
    R, C, seed, offset = 6, 64, 0xA5A5123456, 7
    x = np.full((R, C), 0.25, dtype=np.float32)
    x[:, ::32] = 4.0
    codes, scales = Q.mx_quantize(x, "mxfp4", "sr", seed, offset)
    assert np.all(scales == 127)
    got = F.unpack_e2m1(codes).reshape(R, C)
    groups = R * C // 8
    inp = "".join(f"{seed} {g} 0 {offset} 0\n" for g in range(groups))
    out = subprocess.run([exe], input=inp, capture_output=True, text=True, check=True).stdout
    words = np.array([[int(v) for v in ln.split()] for ln in out.strip().split("\n")], dtype=np.uint64)
    idx = np.arange(R * C)
    w = words[idx >> 3, (idx & 7) >> 1]
    r16 = (w >> (16 * (idx & 1)).astype(np.uint64)) & np.uint64(0xFFFF)
    want = np.where(r16 < 0x8000, 1, 0).reshape(R, C)          # E2M1 code 1 = 0.5
    want[:, ::32] = 6                                          # 4.0 is on the grid
    assert np.array_equal(got, want)
    # row-major global index: the same values as one row give the same codes,
    # the column stream (1) gives different ones
    flat, _ = Q.mx_quantize(x.reshape(1, R * C), "mxfp4", "sr", seed, offset)
    assert np.array_equal(flat.reshape(codes.shape), codes)
    other, _ = Q.mx_quantize(x, "mxfp4", "sr", seed, offset, stream=1)
    assert not np.array_equal(other, codes)


# ---------------------------------------------------------------- GEMM

E2M1_TAB = [Fraction(v) for v in ("0", "1/2", "1", "3/2", "2", "3", "4", "6")]


def _e2m1_frac(code):
    v = E2M1_TAB[code & 7]
    return -v if code & 8 else v


def _e4m3_frac(code):
    e, m = (code >> 3) & 15, code & 7
    v = Fraction(m, 8) * Fraction(2) ** -6 if e == 0 else Fraction(8 + m, 8) * Fraction(2) ** (e - 7)
    return -v if code & 0x80 else v


def _unpack(byte_row):
    out = []
    for b in byte_row:
        out += [int(b) & 15, int(b) >> 4]
    return out


def test_gemm_nvfp4_brute_force_fractions():
    a = synth.bf16_tensor((16, 32), 21).view(torch.int16).numpy().view(np.uint16)
    b = synth.bf16_tensor((16, 32), 22, sigma=0.02, outliers=False).view(torch.int16).numpy().view(np.uint16)
    ac, as_, aa = Q.nvfp4_quantize(a, 1)
    bc, bs, ba = Q.nvfp4_quantize(b, 16)
    C = G.gemm_nvfp4(ac, as_, aa, bc, bs, ba)
    sa = Fraction(float(Q.nvfp4_scale_dec(aa)))
    sb = Fraction(float(Q.nvfp4_scale_dec(ba)))
    for m in range(16):
        ra = _unpack(ac[m])
        for n in range(16):
            rb = _unpack(bc[n])
            acc = Fraction(0)
            for k in range(32):
                acc += (_e2m1_frac(ra[k]) * _e4m3_frac(int(as_[m, k // 16]))
                        * _e2m1_frac(rb[k]) * _e4m3_frac(int(bs[n, k // 16])))
            ref = float(acc * sa * sb)
            assert abs(C[m, n] - ref) <= 1e-15 * max(abs(ref), 1e-300)


def test_gemm_mx_brute_force_fractions():
    a = synth.bf16_tensor((16, 32), 23).view(torch.int16).numpy().view(np.uint16)
    b = synth.bf16_tensor((16, 32), 24).view(torch.int16).numpy().view(np.uint16)
    for fmt in ("mxfp4", "mxfp8"):
        ac, as_ = Q.mx_quantize(a, fmt)
        bc, bs = Q.mx_quantize(b, fmt)
        C = G.gemm_mx(ac, as_, bc, bs, fmt)
        for m in range(16):
            ra = _unpack(ac[m]) if fmt == "mxfp4" else [int(v) for v in ac[m]]
            for n in range(16):
                rb = _unpack(bc[n]) if fmt == "mxfp4" else [int(v) for v in bc[n]]
                dec = _e2m1_frac if fmt == "mxfp4" else _e4m3_frac
                acc = sum(dec(ra[k]) * dec(rb[k]) for k in range(32))
                acc *= Fraction(2) ** (int(as_[m, 0]) - 127) * Fraction(2) ** (int(bs[n, 0]) - 127)
                assert abs(C[m, n] - float(acc)) <= 1e-15 * max(abs(float(acc)), 1e-300)


def test_gemm_matches_blas_at_scale():
    a = synth.bf16_tensor((96, 256), 25).view(torch.int16).numpy().view(np.uint16)
    b = synth.bf16_tensor((80, 256), 26).view(torch.int16).numpy().view(np.uint16)
    ac, as_, aa = Q.nvfp4_quantize(a, 1)
    bc, bs, ba = Q.nvfp4_quantize(b, 1)
    C = G.gemm_nvfp4(ac, as_, aa, bc, bs, ba)
    A = G.dequant_nvfp4(ac, as_)
    B = G.dequant_nvfp4(bc, bs)
    ref = np.einsum("mk,nk->mn", A, B) * G.nvfp4_alpha(aa, ba)
    assert np.max(np.abs(C - ref)) <= 1e-12 * np.sqrt(np.mean(ref ** 2))


def test_tolerance_rule_accepts_bf16_rounding_and_rejects_planted_mistakes():
    a = synth.bf16_tensor((128, 512), 27).view(torch.int16).numpy().view(np.uint16)
    b = synth.bf16_tensor((96, 512), 28).view(torch.int16).numpy().view(np.uint16)
    ac, as_, aa = Q.nvfp4_quantize(a, 1)
    bc, bs, ba = Q.nvfp4_quantize(b, 1)
    C = G.gemm_nvfp4(ac, as_, aa, bc, bs, ba)
    good = torch.from_numpy(C).to(torch.bfloat16).double().numpy()
    assert G.tolerance_report(good, C)["passed"]
    # torch rounds float64 -> bfloat16 through float32 (double rounding), so a few differ
    assert G.tolerance_report(good, C)["frac_equal_rne"] > 0.999
    exact = F.f64_to_bf16_rne(C)
    assert G.tolerance_report(exact, C)["frac_equal_rne"] == 1.0
    # a dropped block scale on one operand block
    bs_bad = bs.copy()
    bs_bad[:, 3] = bs_bad[:, 4]
    bad = G.gemm_nvfp4(ac, as_, aa, bc, bs_bad, ba)
    assert not G.tolerance_report(bad, C)["passed"]
    # swapped nibble order
    swapped = ((bc >> 4) | (bc << 4)).astype(np.uint8)
    bad = G.gemm_nvfp4(ac, as_, aa, swapped, bs, ba)
    assert not G.tolerance_report(bad, C)["passed"]
    # a dropped per-tensor scale
    assert not G.tolerance_report(C / G.nvfp4_alpha(aa, ba) * 1.01 * G.nvfp4_alpha(aa, ba) * 1.03, C)["passed"]


def test_rht_vectorized_equals_scalar_butterfly():
    rng = np.random.default_rng(11)
    x = (rng.standard_normal((40, 16)) * 10.0 ** rng.uniform(-3, 3, (40, 1))).astype(np.float32)
    for signs in (0, 0x8421, 0xFFFF):
        v = R.rht16(x, signs)
        for r in range(40):
            assert np.array_equal(v[r], R.rht16_scalar(x[r], signs))
