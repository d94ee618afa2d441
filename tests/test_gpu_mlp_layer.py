"""GPU parity of the master-weight update and of a whole MLP-layer step.

* master_weight_update bit for bit against the oracle (FP32 master, BF16
  copy, amax), ragged sizes, two calls in a row, the full 8B W_gu size
  (sampled elements; amax against the whole copy).
* MLPLayer (forward, backward, update, chained through the C ABI) against the
  same chain run by the oracle from the same seeded inputs, for two steps.
  The two chains agree bit for bit except where an FP32-accumulated GEMM
  output or an FP32 SwiGLU value rounds to the other BF16 neighbour (about
  1e-4 of the elements), which can move an element's E2M1 code in a later
  quantizer.  Bar: each GEMM output meets the single-GEMM rule
  (max(|err| - ulp/2) <= 1e-2 rms) on at least 99.9% of its elements and its
  relative Frobenius difference from the BF16-rounded reference is below 1e-3; the change the updates made
  to each FP32 master agrees with the oracle's to 1e-2 (relative Frobenius).
"""

import numpy as np
import pytest
import torch

import fp8_quantized_gemm_amd as bsq
from fp8_quantized_gemm_amd import synth
from fp8_quantized_gemm_amd.mlp import MLPLayer
from oracle import formats as F
from oracle import gemm as G
from oracle import mlp as M
from oracle import quantize as Q

from _gpu import announce, assert_bytes_equal, bits, f32, gpu

pytestmark = gpu


def _grad(shape, seed, device="cuda"):
    """BF16 gradient-like values over a wide exponent range."""
    g = torch.Generator(device="cpu")
    g.manual_seed(seed)
    z = torch.randn(shape, generator=g) * 10.0 ** torch.randint(-7, 1, shape, generator=g).float()
    return z.to(torch.bfloat16).to(device)


@pytest.mark.parametrize("n,lr", [(8, 1e-3), (4104, 3e-4), (1 << 20, 2.0 ** -7), (65536, 0.0),
                                  (262144, 0.1)])
def test_master_update(n, lr):
    announce("master update", n, lr)
    g = torch.Generator(device="cpu")
    g.manual_seed(9000 + n)
    w = (torch.randn(n, generator=g) * 0.02).cuda()
    w0 = w.cpu().numpy().copy()
    gr = _grad((n,), 9100 + n)
    d = bsq.master_weight_update(w, gr, lr)
    torch.cuda.synchronize()
    w_ref, b_ref, a_ref = M.master_update(w0, bits(gr), np.float32(lr))
    assert_bytes_equal(w.cpu().numpy().view(np.uint32), w_ref.view(np.uint32), "w32")
    assert_bytes_equal(bits(d["w_bf16"]), b_ref, "w_bf16")
    assert f32(d["amax"])[0] == a_ref


def test_master_update_twice_and_without_amax():
    announce("master update twice")
    n = 1 << 16
    w = (torch.randn(n, generator=torch.Generator().manual_seed(9201)) * 0.02).cuda()
    w0 = w.cpu().numpy().copy()
    g1, g2 = _grad((n,), 9202), _grad((n // 2,), 9203)
    d1 = bsq.master_weight_update(w, g1, 1e-3)
    half = w[: n // 2]
    d2 = bsq.master_weight_update(half, g2, 1e-3, amax=False)
    torch.cuda.synchronize()
    r1, b1, a1 = M.master_update(w0, bits(g1), np.float32(1e-3))
    r2, b2, _ = M.master_update(r1[: n // 2], bits(g2), np.float32(1e-3))
    assert f32(d1["amax"])[0] == a1 and d2["amax"] is None
    assert_bytes_equal(w.cpu().numpy()[: n // 2].view(np.uint32), r2.view(np.uint32), "w32 twice")
    assert_bytes_equal(w.cpu().numpy()[n // 2:].view(np.uint32), r1[n // 2:].view(np.uint32), "w32 tail")
    assert_bytes_equal(bits(d2["w_bf16"]), b2, "copy twice")


@pytest.mark.parametrize("shape,sigma", [((28672, 4096), 0.02), ((106496, 16384), 0.01)], ids=["8b", "405b"])
def test_master_update_w_gu_full_size(shape, sigma):
    """W_gu of the 8B MLP (28672 x 4096 = 117.4M elements) and of the 405B MLP
    (106496 x 16384 = 1.74G elements): every 4099th element against the
    oracle; the amax against the whole BF16 copy."""
    announce("master update W_gu", shape)
    w = synth.bf16_tensor(shape, 9301, sigma, False, device="cuda").float()
    idx = torch.arange(0, w.numel(), 4099, device="cuda")
    w0 = w.view(-1)[idx].cpu().numpy()
    gr = synth.bf16_tensor(shape, 9302, 1e-3, False, device="cuda")
    d = bsq.master_weight_update(w, gr, 3e-4)
    torch.cuda.synchronize()
    r, b, _ = M.master_update(w0, bits(gr.view(-1)[idx]), np.float32(3e-4))
    assert_bytes_equal(w.view(-1)[idx].cpu().numpy().view(np.uint32), r.view(np.uint32), "w32 sampled")
    assert_bytes_equal(bits(d["w_bf16"].view(-1)[idx]), b, "copy sampled")
    assert f32(d["amax"])[0] == d["w_bf16"].float().abs().max().item()


# ---------------------------------------------------------------- the layer chain

def _bf(c):
    return M.f64_to_bf16_bits(c)


def _gemm(qa, sa, qb, sb):
    return G.gemm_nvfp4(qa[sa + "_codes"], qa[sa + "_scales"], qa[sa + "_amax"],
                        qb[sb + "_codes"], qb[sb + "_scales"], qb[sb + "_amax"])


def oracle_layer(x, w_gu, w_down, dy, rht, signs, seed, lr, steps):
    """The MLPLayer data flow run by the oracle (BF16 bits and FP32 masters)."""
    w_gu, w_down = w_gu.copy(), w_down.copy()
    _, wgu_b, _ = M.master_update(w_gu, np.zeros(w_gu.shape, np.uint16), np.float32(0.0))
    _, wd_b, _ = M.master_update(w_down, np.zeros(w_down.shape, np.uint16), np.float32(0.0))
    out = {}
    for it in range(steps):
        qx = Q.quantize_transpose(x, "nvfp4", 1, "rne", rht_col=rht, rht_signs=signs)
        qwg = Q.quantize_transpose(wgu_b, "nvfp4", 16, "rne")
        y_gu = _bf(_gemm(qx, "row", qwg, "row"))
        h = M.swiglu(y_gu)
        qh = Q.quantize_transpose(h, "nvfp4", 1, "rne", rht_col=rht, rht_signs=signs)
        qwd = Q.quantize_transpose(wd_b, "nvfp4", 16, "rne")
        y_down = _gemm(qh, "row", qwd, "row")
        qdy = Q.quantize_transpose(dy, "nvfp4", 1, "sr", seed, 2 * it, rht, signs)
        dh = _bf(_gemm(qdy, "row", qwd, "col"))
        dw_down = _gemm(qdy, "col", qh, "col")
        dy_gu = M.swiglu_backward(y_gu, dh)
        qdg = Q.quantize_transpose(dy_gu, "nvfp4", 1, "sr", seed, 2 * it + 1, rht, signs)
        dx = _gemm(qdg, "row", qwg, "col")
        dw_gu = _gemm(qdg, "col", qx, "col")
        out = dict(Y_down=y_down, dX=dx, dW_down=dw_down, dW_gu=dw_gu)
        w_gu, wgu_b, _ = M.master_update(w_gu, _bf(dw_gu), np.float32(lr))
        w_down, wd_b, _ = M.master_update(w_down, _bf(dw_down), np.float32(lr))
    out["W_gu"], out["W_down"] = w_gu, w_down
    return out


def _chain_check(got, ref, what):
    rep = G.tolerance_report(got, ref)
    rms = rep["rms"]
    err = np.abs(got - ref) - 0.5 * G.ulp_bf16(np.maximum(np.abs(got), np.abs(ref)))
    ok_frac = float(np.mean(err <= 1e-2 * rms))
    # against the BF16 rounding of the reference: the divergence of the chains,
    # not the output's own rounding (about 2^-9 / sqrt(3) relative)
    frob = float(np.linalg.norm(got - F.bf16_bits_to_f32(_bf(ref)).astype(np.float64)) / np.linalg.norm(ref))
    print(what, f"ok fraction {ok_frac:.6f}, rel frobenius {frob:.2e}, bf16-equal {rep['frac_equal_rne']:.6f}")
    assert ok_frac >= 0.999 and frob <= 1e-3, (what, ok_frac, frob)
    return frob


@pytest.mark.parametrize("rht", [True, False])
def test_mlp_layer_two_steps_against_oracle(rht):
    announce("mlp layer chain", rht)
    T, Hd, F = 256, 256, 512
    signs, seed, lr = 0x6A5D, 0xC0FFEE, 1e-2
    x = synth.bf16_tensor((T, Hd), 9401, 1.0, True, device="cuda")
    dy = synth.bf16_tensor((T, Hd), 9402, 1e-3, False, device="cuda")
    w_gu = (torch.randn((2 * F, Hd), generator=torch.Generator().manual_seed(9403)) * 0.02)
    w_down = (torch.randn((Hd, F), generator=torch.Generator().manual_seed(9404)) * 0.02)
    layer = MLPLayer(w_gu.cuda(), w_down.cuda(), T, rht=rht, rht_signs=signs, sr_seed=seed, lr=lr)
    for _ in range(2):
        y, dx = layer.step(x, dy)
    torch.cuda.synchronize()
    ref = oracle_layer(bits(x), w_gu.numpy(), w_down.numpy(), bits(dy), rht, signs, seed, lr, 2)
    fr = {}
    for name, t in (("Y_down", y), ("dX", dx), ("dW_gu", layer.grad["W_gu"]),
                    ("dW_down", layer.grad["W_down"])):
        fr[name] = _chain_check(t.double().cpu().numpy(), ref[name], name)
    for name, w0 in (("W_gu", w_gu), ("W_down", w_down)):
        # the change the two updates made to the FP32 master, GPU against oracle
        d_gpu = layer.w32[name].double().cpu().numpy() - w0.double().numpy()
        d_ref = ref[name].astype(np.float64) - w0.double().numpy()
        rel = np.linalg.norm(d_gpu - d_ref) / np.linalg.norm(d_ref)
        print(name, "update relative difference", rel)
        assert rel <= 1e-2, (name, rel)
