"""Writes oracle_cases.json: small seeded cases with the CPU oracle's outputs.

The source pages print no worked numeric example, so the stored outputs here
come from the oracle alone (this script imports only `oracle/` and the seeded
input recipes).  They pin the oracle against later drift (a change to its
arithmetic must regenerate this file and say why) and give the GPU tests
fixed expected bytes that need no oracle run.

Run from the repository root:  python tests/golden/make_oracle_cases.py
"""

import json
import os
import sys

import numpy as np

ROOT = os.path.dirname(os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
sys.path.insert(0, ROOT)

from fp8_quantized_gemm_amd import synth  # noqa: E402  (seeded input recipes only)
from oracle import gemm as G  # noqa: E402
from oracle import mlp as MLP  # noqa: E402
from oracle import quantize as Q  # noqa: E402

OUT = os.path.join(os.path.dirname(os.path.abspath(__file__)), "oracle_cases.json")


def bits(shape, seed, sigma=1.0, outliers=True):
    t = synth.bf16_tensor(shape, seed, sigma, outliers, device="cpu")
    return t.contiguous().view(__import__("torch").int16).numpy().view(np.uint16)


def hexa(a):
    return np.ascontiguousarray(a).tobytes().hex()


def f32hex(x):
    return np.float32(x).tobytes().hex()


def qt_record(d):
    rec = {}
    for side in ("row", "col"):
        rec[f"{side}_codes"] = hexa(d[f"{side}_codes"])
        rec[f"{side}_scales"] = hexa(d[f"{side}_scales"])
        if d[f"{side}_amax"] is not None:
            rec[f"{side}_amax"] = f32hex(d[f"{side}_amax"])
    return rec


def main():
    cases = []

    # NVFP4 1x16 RNE, both orientations (activation-like, with outliers)
    x = bits((32, 64), 9101)
    cases.append(dict(name="nvfp4_1x16_rne", kind="quantize_transpose", shape=[32, 64],
                      x=hexa(x), args=dict(fmt="nvfp4", block_rows=1, rnd="rne"),
                      out=qt_record(Q.quantize_transpose(x, "nvfp4", 1, "rne"))))

    # NVFP4 16x16 2D (weight-like)
    w = bits((48, 32), 9102, sigma=0.02, outliers=False)
    cases.append(dict(name="nvfp4_16x16_rne", kind="quantize_transpose", shape=[48, 32],
                      x=hexa(w), args=dict(fmt="nvfp4", block_rows=16, rnd="rne"),
                      out=qt_record(Q.quantize_transpose(w, "nvfp4", 16, "rne"))))

    # NVFP4 gradient: stochastic rounding both sides, RHT on the column side
    dy = bits((32, 48), 9103, sigma=1e-3, outliers=False)
    sr = dict(fmt="nvfp4", block_rows=1, rnd="sr", seed=0x1234567890ABCDEF, offset=7,
              rht_col=True, rht_signs=0xB3C5)
    cases.append(dict(name="nvfp4_sr_rht", kind="quantize_transpose", shape=[32, 48],
                      x=hexa(dy), args=sr,
                      out=qt_record(Q.quantize_transpose(dy, sr["fmt"], sr["block_rows"], sr["rnd"],
                                                         sr["seed"], sr["offset"], sr["rht_col"],
                                                         sr["rht_signs"]))))

    # MX rowwise
    for fmt in ("mxfp4", "mxfp8"):
        m = bits((16, 96), 9104 if fmt == "mxfp4" else 9105)
        c, s = Q.mx_quantize(m, fmt)
        cases.append(dict(name=f"{fmt}_rne", kind="mx_quantize", shape=[16, 96], x=hexa(m),
                          args=dict(fmt=fmt), out=dict(codes=hexa(c), scales=hexa(s))))

    # NVFP4 GEMM (A 1x16 activations, B 16x16 weights), K = 128
    a = bits((32, 128), 9106)
    b = bits((48, 128), 9107, sigma=0.02, outliers=False)
    ac, as_, aa = Q.nvfp4_quantize(a, 1)
    bc, bs, ba = Q.nvfp4_quantize(b, 16)
    c_ref = G.gemm_nvfp4(ac, as_, aa, bc, bs, ba)
    cases.append(dict(name="gemm_nvfp4", kind="gemm", fmt="nvfp4", M=32, N=48, K=128,
                      a_codes=hexa(ac), a_scales=hexa(as_), a_amax=f32hex(aa),
                      b_codes=hexa(bc), b_scales=hexa(bs), b_amax=f32hex(ba),
                      c_ref=[repr(float(v)) for v in c_ref.ravel()]))

    # MXFP8 GEMM, K = 512 (one scale period)
    a = bits((32, 512), 9108)
    b = bits((16, 512), 9109)
    ac, as_ = Q.mx_quantize(a, "mxfp8")
    bc, bs = Q.mx_quantize(b, "mxfp8")
    c_ref = G.gemm_mx(ac, as_, bc, bs, "mxfp8")
    cases.append(dict(name="gemm_mxfp8", kind="gemm", fmt="mxfp8", M=32, N=16, K=512,
                      a_codes=hexa(ac), a_scales=hexa(as_), b_codes=hexa(bc), b_scales=hexa(bs),
                      c_ref=[repr(float(v)) for v in c_ref.ravel()]))

    # per-tensor FP8 baseline, both orientations
    x8 = bits((32, 48), 9114)
    d8 = Q.fp8_quantize_transpose(x8)
    cases.append(dict(name="fp8_qt", kind="fp8_quantize_transpose", shape=[32, 48], x=hexa(x8),
                      out=dict(row_codes=hexa(d8["row_codes"]), col_codes=hexa(d8["col_codes"]),
                               amax=f32hex(d8["amax"]))))

    # SwiGLU forward and backward (F = 32) with the amaxes of their outputs
    # (plain, and column RHT under the sign mask below)
    signs = 0xB3C5
    y = bits((16, 64), 9110, sigma=2.0)
    h = MLP.swiglu(y)
    qh = Q.quantize_transpose(h, "nvfp4", 1, "rne", rht_col=True, rht_signs=signs)
    cases.append(dict(name="swiglu_fwd", kind="swiglu", shape=[16, 32], y=hexa(y), rht_signs=signs,
                      out=dict(h=hexa(h), amax_row=f32hex(qh["row_amax"]),
                               amax_col=f32hex(qh["col_amax"]))))
    dh = bits((16, 32), 9111, sigma=1e-3, outliers=False)
    dy = MLP.swiglu_backward(y, dh)
    qd = Q.quantize_transpose(dy, "nvfp4", 1, "rne", rht_col=True, rht_signs=signs)
    cases.append(dict(name="swiglu_bwd", kind="swiglu_backward", shape=[16, 32], y=hexa(y),
                      dh=hexa(dh), rht_signs=signs,
                      out=dict(dy=hexa(dy), amax_row=f32hex(qd["row_amax"]),
                               amax_col=f32hex(qd["col_amax"]))))

    # FP32 master-weight update with its BF16 copy and amax
    w = (np.random.default_rng(9112).standard_normal(256) * 0.02).astype(np.float32)
    g = bits((256,), 9113, sigma=1e-2, outliers=False)
    lr = np.float32(1e-3)
    wn, wb, wa = MLP.master_update(w, g, lr)
    cases.append(dict(name="master_update", kind="master_update", n=256, lr=f32hex(lr), w=hexa(w),
                      g=hexa(g), out=dict(w=hexa(wn), w_bf16=hexa(wb), amax=f32hex(wa))))

    with open(OUT, "w") as f:
        json.dump({"generator": "tests/golden/make_oracle_cases.py", "cases": cases}, f, indent=1)
    print(f"wrote {OUT}: {len(cases)} cases")


if __name__ == "__main__":
    main()
