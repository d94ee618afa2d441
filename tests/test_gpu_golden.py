"""The HIP path on the stored small cases of tests/golden/oracle_cases.json:
quantizer bytes and amax bit for bit, GEMMs within the tolerance rule.  The
expected values were written by the CPU oracle; nothing is recomputed here."""

import numpy as np
import pytest
import torch

import fp8_quantized_gemm_amd as bsq
from oracle import gemm as G

import golden_cases as GC
from _gpu import announce, from_bits, gpu

pytestmark = gpu

CASES = GC.load()


def _dev(a):
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


@pytest.mark.parametrize("case", CASES, ids=GC.ids(CASES))
def test_gpu_matches_stored_case(case):
    announce("golden", case["name"])
    if case["kind"] == "quantize_transpose":
        R, C = case["shape"]
        a = case["args"]
        d = bsq.quantize_transpose(from_bits(GC.u16(case["x"], (R, C))), a["fmt"], a["block_rows"],
                                   a["rnd"], a.get("seed", 0), a.get("offset", 0),
                                   a.get("rht_col", False), a.get("rht_signs", 0))
        torch.cuda.synchronize()
        for k, shp in GC.qt_shapes(R, C, a["fmt"]).items():
            np.testing.assert_array_equal(d[k].cpu().numpy(), GC.u8(case["out"][k], shp), err_msg=k)
        for k in ("row_amax", "col_amax"):
            if k in case["out"]:
                got = np.float32(d[k].cpu().numpy().reshape(-1)[0])
                assert got.tobytes() == np.float32(GC.f32(case["out"][k])).tobytes(), k
    elif case["kind"] == "mx_quantize":
        R, C = case["shape"]
        fmt = case["args"]["fmt"]
        c, s = bsq.mx_quantize(from_bits(GC.u16(case["x"], (R, C))), fmt)
        torch.cuda.synchronize()
        c, s = c.cpu().numpy(), s.cpu().numpy()
        np.testing.assert_array_equal(c, GC.u8(case["out"]["codes"], c.shape))
        np.testing.assert_array_equal(s, GC.u8(case["out"]["scales"], (R, C // 32)))
    else:
        M, N, K, fmt = case["M"], case["N"], case["K"], case["fmt"]
        w = 1 if fmt == "mxfp8" else 2
        b = 16 if fmt == "nvfp4" else 32
        ac, as_ = _dev(GC.u8(case["a_codes"], (M, K // w))), _dev(GC.u8(case["a_scales"], (M, K // b)))
        bc, bs = _dev(GC.u8(case["b_codes"], (N, K // w))), _dev(GC.u8(case["b_scales"], (N, K // b)))
        if fmt == "nvfp4":
            aa = _dev(np.array([GC.f32(case["a_amax"])], dtype=np.float32))
            ba = _dev(np.array([GC.f32(case["b_amax"])], dtype=np.float32))
            c = bsq.bs_gemm(fmt, ac, as_, bc, bs, aa, ba)
        else:
            c = bsq.bs_gemm(fmt, ac, as_, bc, bs, K=K)
        torch.cuda.synchronize()
        want = np.array([float(v) for v in case["c_ref"]]).reshape(M, N)
        rep = G.tolerance_report(c.float().cpu().numpy().astype(np.float64), want)
        print(case["name"], rep)
        assert rep["passed"], rep
