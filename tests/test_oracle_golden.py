"""The oracle reproduces its stored small cases byte for byte.

tests/golden/oracle_cases.json was written by tests/golden/make_oracle_cases.py
from the oracle itself; a change to the oracle's arithmetic that alters any of
these bytes fails here until the file is regenerated deliberately."""

import numpy as np
import pytest

from oracle import gemm as G
from oracle import mlp as MLP
from oracle import quantize as Q

import golden_cases as GC

CASES = GC.load()


@pytest.mark.parametrize("case", CASES, ids=GC.ids(CASES))
def test_oracle_matches_stored_case(case):
    if case["kind"] == "quantize_transpose":
        R, C = case["shape"]
        x = GC.u16(case["x"], (R, C))
        a = case["args"]
        d = Q.quantize_transpose(x, a["fmt"], a["block_rows"], a["rnd"], a.get("seed", 0),
                                 a.get("offset", 0), a.get("rht_col", False), a.get("rht_signs", 0))
        shapes = GC.qt_shapes(R, C, a["fmt"])
        for k, shp in shapes.items():
            np.testing.assert_array_equal(d[k], GC.u8(case["out"][k], shp), err_msg=k)
        for k in ("row_amax", "col_amax"):
            if k in case["out"]:
                assert np.float32(d[k]).tobytes() == np.float32(GC.f32(case["out"][k])).tobytes(), k
    elif case["kind"] == "mx_quantize":
        R, C = case["shape"]
        fmt = case["args"]["fmt"]
        c, s = Q.mx_quantize(GC.u16(case["x"], (R, C)), fmt)
        np.testing.assert_array_equal(c, GC.u8(case["out"]["codes"], c.shape))
        np.testing.assert_array_equal(s, GC.u8(case["out"]["scales"], (R, C // 32)))
    elif case["kind"] == "fp8_quantize_transpose":
        R, C = case["shape"]
        d = Q.fp8_quantize_transpose(GC.u16(case["x"], (R, C)))
        np.testing.assert_array_equal(d["row_codes"], GC.u8(case["out"]["row_codes"], (R, C)))
        np.testing.assert_array_equal(d["col_codes"], GC.u8(case["out"]["col_codes"], (C, R)))
        assert np.float32(d["amax"]).tobytes() == np.float32(GC.f32(case["out"]["amax"])).tobytes()
    elif case["kind"] in ("swiglu", "swiglu_backward"):
        T, F = case["shape"]
        y = GC.u16(case["y"], (T, 2 * F))
        if case["kind"] == "swiglu":
            out, key = MLP.swiglu(y), "h"
        else:
            out, key = MLP.swiglu_backward(y, GC.u16(case["dh"], (T, F))), "dy"
        np.testing.assert_array_equal(out, GC.u16(case["out"][key], out.shape))
        q = Q.quantize_transpose(out, "nvfp4", 1, "rne", rht_col=True, rht_signs=case["rht_signs"])
        assert np.float32(q["row_amax"]) == GC.f32(case["out"]["amax_row"])
        assert np.float32(q["col_amax"]) == GC.f32(case["out"]["amax_col"])
    elif case["kind"] == "master_update":
        wn, wb, wa = MLP.master_update(GC.f32s(case["w"]), GC.u16(case["g"], (case["n"],)),
                                       GC.f32(case["lr"]))
        np.testing.assert_array_equal(wn.view(np.uint32), GC.f32s(case["out"]["w"]).view(np.uint32))
        np.testing.assert_array_equal(wb, GC.u16(case["out"]["w_bf16"], (case["n"],)))
        assert wa == GC.f32(case["out"]["amax"])
    else:
        M, N, K, fmt = case["M"], case["N"], case["K"], case["fmt"]
        w = 1 if fmt == "mxfp8" else 2
        b = 16 if fmt == "nvfp4" else 32
        ac, as_ = GC.u8(case["a_codes"], (M, K // w)), GC.u8(case["a_scales"], (M, K // b))
        bc, bs = GC.u8(case["b_codes"], (N, K // w)), GC.u8(case["b_scales"], (N, K // b))
        if fmt == "nvfp4":
            c = G.gemm_nvfp4(ac, as_, GC.f32(case["a_amax"]), bc, bs, GC.f32(case["b_amax"]))
        else:
            c = G.gemm_mx(ac, as_, bc, bs, fmt)
        want = np.array([float(v) for v in case["c_ref"]]).reshape(M, N)
        # FP64 products summed by BLAS: the order (and so the last bits) may
        # differ between hosts
        rms = float(np.sqrt(np.mean(want ** 2)))
        np.testing.assert_allclose(c, want, rtol=0, atol=1e-12 * rms)
