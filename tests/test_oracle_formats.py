"""Pins for the oracle's element/scale formats (CPU only).

E2M1 is pinned by a brute-force nearest-value search written independently
of the oracle's decision table; E4M3 by torch's float8_e4m3fn CPU cast (a
library routine, RNE, non-saturating below 464); E8M0 by torch's
float8_e8m0fnu; stochastic rounding by its statistics (unbiasedness over 1e5
draws, small values not crushed, grid points fixed).
"""

from fractions import Fraction

import numpy as np
import pytest
import torch

from oracle import formats as F

GRID = [0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0]   # OCP MX E2M1 magnitudes


def brute_e2m1_rne(v):
    """Nearest grid magnitude by exhaustive search; ties to the even code; saturate."""
    a = abs(Fraction(float(v)))
    best = None
    for code, g in enumerate(GRID):
        d = abs(a - Fraction(g))
        if best is None or d < best[0] or (d == best[0] and code % 2 == 0):
            best = (d, code)
    code = best[1]
    if a > 6:
        code = 7
    sign = 8 if np.signbit(np.float32(v)) else 0
    return code | sign


def test_e2m1_decode_value_set():
    vals = F.e2m1_decode(np.arange(16, dtype=np.uint8))
    assert list(vals[:8]) == GRID
    assert list(-vals[8:]) == GRID
    assert np.signbit(vals[8])          # code 0x8 is -0


def test_e2m1_rne_brute_force_sweep():
    rng = np.random.default_rng(0)
    mids = np.array([0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0], dtype=np.float32)
    pts = [mids, np.nextafter(mids, np.float32(0)), np.nextafter(mids, np.float32(10)),
           np.array(GRID, dtype=np.float32),
           rng.uniform(0, 8, 4000).astype(np.float32),
           rng.uniform(0, 0.3, 500).astype(np.float32),
           np.array([6.0001, 7.0, 1e30, 0.0, 1e-30], dtype=np.float32)]
    v = np.concatenate(pts)
    v = np.concatenate([v, -v])
    got = F.e2m1_encode_rne(v)
    want = np.array([brute_e2m1_rne(x) for x in v], dtype=np.uint8)
    assert np.array_equal(got, want)


def test_e2m1_rne_ties_and_saturation():
    v = np.array([0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0, 6.0, 6.5, 100.0, np.inf], dtype=np.float32)
    assert list(F.e2m1_encode_rne(v)) == [0, 2, 2, 4, 4, 6, 6, 7, 7, 7, 7]
    assert list(F.e2m1_encode_rne(-v)) == [8, 10, 10, 12, 12, 14, 14, 15, 15, 15, 15]
    assert F.e2m1_encode_rne(np.array([-0.0], dtype=np.float32))[0] == 0x8


def test_pack_low_nibble_is_even_index():
    packed = F.pack_e2m1(np.array([1, 7, 0xF, 0x2], dtype=np.uint8))
    assert list(packed) == [0x71, 0x2F]
    assert list(F.unpack_e2m1(packed)) == [1, 7, 0xF, 0x2]


def test_e4m3_decode_matches_torch():
    codes = np.arange(256, dtype=np.uint8)
    ours = F.e4m3_decode(codes)
    ref = torch.from_numpy(codes.copy()).view(torch.float8_e4m3fn).float().numpy()
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(ours), nan)
    assert np.array_equal(ours[~nan], ref[~nan])
    assert F.e4m3_decode(np.array([0x7E], dtype=np.uint8))[0] == 448.0
    assert F.e4m3_decode(np.array([0x01], dtype=np.uint8))[0] == 2.0 ** -9


def _e4m3_sweep():
    rng = np.random.default_rng(1)
    allv = F.e4m3_decode(np.arange(0x7F, dtype=np.uint8)).astype(np.float64)
    mids = (allv[1:] + allv[:-1]) / 2
    mids32 = mids.astype(np.float32)
    bf = (np.arange(0, 0x43E1, dtype=np.uint32) << 16).view(np.float32)    # all BF16 in [0, 448]
    s = np.concatenate([allv.astype(np.float32), mids32,
                        np.nextafter(mids32, np.float32(0)), np.nextafter(mids32, np.float32(1e9)),
                        bf, rng.uniform(0, 448, 20000).astype(np.float32),
                        (2.0 ** rng.uniform(-40, 8.8, 20000)).astype(np.float32)])
    return s[s <= 448]


def test_e4m3_encode_matches_torch_rne():
    s = _e4m3_sweep()
    ours = F.e4m3_encode_rne(s)
    ref = torch.from_numpy(s.copy()).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(ours, ref)
    ours_n = F.e4m3_encode_rne(-s)
    ref_n = torch.from_numpy(-s).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(ours_n, ref_n)


def test_e4m3_saturation():
    s = np.array([448.0, 449.0, 463.9, 464.0, 1000.0, 1e30, np.inf], dtype=np.float32)
    assert list(F.e4m3_encode_rne(s)) == [0x7E] * 7
    assert list(F.e4m3_encode_rne(-s)) == [0xFE] * 7


def test_e8m0_decode_matches_torch():
    codes = np.arange(255, dtype=np.uint8)
    ours = F.e8m0_decode(codes)
    ref = torch.from_numpy(codes.copy()).view(torch.float8_e8m0fnu).double().numpy()
    assert np.array_equal(ours, ref)


def test_floor_log2():
    a = np.array([1.0, 1.5, 2.0, 0.75, 2.0 ** -130, 3.0e38], dtype=np.float32)
    assert list(F.floor_log2(a)) == [0, 0, 1, -1, -130, 127]


# ---------------------------------------------------------------- stochastic rounding

def test_sr_unbiased_1e5():
    rng = np.random.default_rng(7)
    for v in [0.1, 0.3, 0.75, 1.2, 2.9, 5.5]:
        r = rng.integers(0, 1 << 16, 100000, dtype=np.uint32)
        codes = F.e2m1_encode_sr(np.full(r.shape, v, dtype=np.float32), r)
        deq = F.e2m1_decode(codes).astype(np.float64)
        lo = max(g for g in GRID if g <= v)
        hi = min(g for g in GRID if g > v)
        assert set(np.unique(deq)) <= {lo, hi}
        p = (v - lo) / (hi - lo)
        sigma = (hi - lo) * np.sqrt(p * (1 - p) / r.size)
        assert abs(deq.mean() - v) <= 5 * sigma + (hi - lo) * 2.0 ** -16


def test_sr_small_values_not_crushed():
    r = np.random.default_rng(8).integers(0, 1 << 16, 100000, dtype=np.uint32)
    v = np.float32(2.0 ** -12)                         # frac = 2**-11 of the 0 -> 0.5 gap
    codes = F.e2m1_encode_sr(np.full(r.shape, v, dtype=np.float32), r)
    ups = int(np.sum(codes == 1))
    assert 20 <= ups <= 90                              # expectation 48.8
    assert set(np.unique(codes)) <= {0, 1}


def test_sr_threshold_rule_exact():
    # with r enumerating all 2**16 values, the count of round-ups equals floor(frac * 2**16)
    r = np.arange(1 << 16, dtype=np.uint32)
    for v in [0.1, 0.3, 1.2, 2.9, 5.5, 0.5 + 2.0 ** -20]:
        codes = F.e2m1_encode_sr(np.full(r.shape, v, dtype=np.float32), r)
        lo = max(g for g in GRID if g <= v)
        hi = min(g for g in GRID if g > v)
        frac = (Fraction(float(np.float32(v))) - Fraction(lo)) / Fraction(hi - lo)
        expect = int(frac * 65536)
        assert int(np.sum(F.e2m1_decode(codes) == hi)) == expect


def test_sr_grid_points_fixed_and_saturation():
    r = np.random.default_rng(9).integers(0, 1 << 16, 1000, dtype=np.uint32)
    for code, g in enumerate(GRID):
        c = F.e2m1_encode_sr(np.full(r.shape, g, dtype=np.float32), r)
        assert np.all(c == code)
        c = F.e2m1_encode_sr(np.full(r.shape, -g, dtype=np.float32), r)
        assert np.all(c == (code | 8))
    for v in [6.0, 6.5, 1e30]:
        assert np.all(F.e2m1_encode_sr(np.full(r.shape, v, dtype=np.float32), r) == 7)


def test_f64_to_bf16_rne_matches_torch_for_float32_values():
    rng = np.random.default_rng(3)
    x = (rng.standard_normal(10000) * 10.0 ** rng.uniform(-30, 30, 10000)).astype(np.float32)
    ours = F.f64_to_bf16_rne(x.astype(np.float64))
    ref = torch.from_numpy(x).to(torch.bfloat16).double().numpy()
    assert np.array_equal(ours, ref)
