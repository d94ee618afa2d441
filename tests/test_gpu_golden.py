"""The HIP path on the stored small cases of tests/golden/oracle_cases.json:
quantizer bytes, amaxes and the master-weight update bit for bit, GEMMs
within the tolerance rule, SwiGLU outputs within one BF16 ulp (their amaxes
bit for bit when the outputs match, else within one ulp).  The expected
values were written by the CPU oracle; nothing is recomputed here."""

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
    elif case["kind"] == "fp8_quantize_transpose":
        R, C = case["shape"]
        d = bsq.fp8_quantize_transpose(from_bits(GC.u16(case["x"], (R, C))))
        torch.cuda.synchronize()
        np.testing.assert_array_equal(d["row_codes"].cpu().numpy(), GC.u8(case["out"]["row_codes"], (R, C)))
        np.testing.assert_array_equal(d["col_codes"].cpu().numpy(), GC.u8(case["out"]["col_codes"], (C, R)))
        assert d["amax"].cpu().numpy()[0] == GC.f32(case["out"]["amax"])
    elif case["kind"] in ("swiglu", "swiglu_backward"):
        T, F = case["shape"]
        y = from_bits(GC.u16(case["y"], (T, 2 * F)))
        if case["kind"] == "swiglu":
            d, key, want = bsq.swiglu(y, rht_col=True, rht_signs=case["rht_signs"]), "h", (T, F)
        else:
            dh = from_bits(GC.u16(case["dh"], (T, F)))
            d, key, want = bsq.swiglu_backward(y, dh, rht_col=True, rht_signs=case["rht_signs"]), "d_y_gu", (T, 2 * F)
        torch.cuda.synchronize()
        got = d[key].contiguous().cpu().view(torch.int16).numpy().view(np.uint16)
        ref = GC.u16(case["out"]["h" if key == "h" else "dy"], want)
        k = lambda b: np.where(b & 0x8000, -(b.astype(np.int32) & 0x7FFF), b.astype(np.int32) & 0x7FFF)
        assert np.abs(k(got) - k(ref)).max() <= 1
        ar, ac = d["amax_row"].cpu().numpy()[0], d["amax_col"].cpu().numpy()[0]
        rr, rc = GC.f32(case["out"]["amax_row"]), GC.f32(case["out"]["amax_col"])
        if np.array_equal(got, ref):
            assert (ar, ac) == (rr, rc)
        else:
            assert abs(ar - rr) <= rr * 2.0 ** -7 and abs(ac - rc) <= rc * 2.0 ** -7
    elif case["kind"] == "master_update":
        w = _dev(GC.f32s(case["w"]))
        d = bsq.master_weight_update(w, from_bits(GC.u16(case["g"], (case["n"],))), float(GC.f32(case["lr"])))
        torch.cuda.synchronize()
        np.testing.assert_array_equal(w.cpu().numpy().view(np.uint32), GC.f32s(case["out"]["w"]).view(np.uint32))
        np.testing.assert_array_equal(d["w_bf16"].cpu().view(torch.int16).numpy().view(np.uint16),
                                      GC.u16(case["out"]["w_bf16"], (case["n"],)))
        assert d["amax"].cpu().numpy()[0] == GC.f32(case["out"]["amax"])
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
