"""Benchmark: block-scaled GEMM TFLOP/s including quantize on Llama MLP shapes.

One step = the whole hot path of one transformer-MLP layer on one GPU's share
(8B: 32,768 tokens, hidden 4096, FFN 14336, gate+up fused):
  FPROP   quantize_transpose X (row RNE, col RNE+RHT), W_gu (16x16 2D),
          GEMM Y_gu = X . W_gu^T; quantize_transpose H (row, col RHT),
          W_down (2D); GEMM Y_down = H . W_down^T
  DGRAD / WGRAD
          quantize_transpose dY_down (row SR, col SR+RHT); GEMM dH = dY_down . W_down;
          GEMM dW_down = dY_down^T . H;
          quantize_transpose dY_gu (row SR, col SR+RHT); GEMM dX = dY_gu . W_gu;
          GEMM dW_gu = dY_gu^T . X
value = sum(2 M N K) / step time, with BF16 inputs already resident in HBM;
the step time is the median over the timed steps (HIP events on the launch
stream), with a 1 GiB scratch read between steps so that no step starts
with its inputs in the 256 MB MALL.

Also reported, each in its own field:
  rht_off / rht_on       the same step with the RHT setting flipped;
  rht_wgrad_error        WGRAD_down error with and without the RHT against an
                         FP64 product (8B only);
  fp8_baseline           the same step with the per-tensor FP8 baseline the
                         NVFP4 post compares against (E4M3 under 448 / amax,
                         FP8 matrix path) and the NVFP4 step's speed relative
                         to it, also against the vendor's FP8 GEMM
                         (hipBLASLt via torch._scaled_mm) on the same codes;
  vendor_fp16_gemm       for scale: the vendor's FP16 GEMM (hipBLASLt via
                         torch.mm) on the six GEMMs with both operands
                         pre-expanded to the FP16 values the NVFP4 GEMM forms
                         in its tiles (expansion not timed);
  workload_405b          the Llama-3.1-405B MLP layer step (8,192 tokens,
                         hidden 16384, FFN 53248), same method;
  tiny_fprop_256         the 256^3 NVFP4 FPROP (quantize + GEMM);
  swiglu_fused_quantize  the SwiGLU forward and backward around the H and
                         dY_gu quantizers, with and without their fused amaxes;
  mlp_layer_step         the whole chained MLP-layer training step with SwiGLU
                         and the FP32 master-weight update;
  mx_square_4096         the MX square workload (4096^3, MXFP8 and MXFP4:
                         mx_quantize of both operands + GEMM), with its
                         roofline fraction;
  nvfp4_route_ceilings   inner-loop ceilings of the two exact NVFP4 GEMM routes.

Prints one JSON line.  Usage: python bench.py [--steps K] [--warmup W] [--no-rht]
[--workload 8b|405b] [--no-cpu-baseline] [--no-mx] [--no-fp8] [--no-vendor-fp16] [--no-swiglu]
[--no-route-ceiling] [--no-405b] [--no-tiny] [--no-bx].
"""

import argparse
import ctypes
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

import torch  # noqa: E402

import fp8_quantized_gemm_amd as bsq  # noqa: E402
from fp8_quantized_gemm_amd import synth  # noqa: E402

PEAK_FP16_TFLOPS = 2516.6      # MI355X dense FP16 MFMA (the NVFP4 GEMM's matrix path; BF16 is the same)
PEAK_FP8_TFLOPS = 5033.2       # dense FP8 MFMA (MXFP8 GEMM)
PEAK_FP4_TFLOPS = 10066.3      # dense FP4 MFMA (MXFP4 GEMM)
PEAK_HBM_GBS = 8000.0

NV, MXF4, MXF8, FP8 = 0, 1, 2, 3
RNE, SR = 0, 1


def P(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


FLUSH_BYTES = 1 << 30


class Flusher:
    """Reads a 1 GiB scratch buffer between timed repetitions, so that no
    repetition finds its inputs in the 256 MB MALL or the L2s left warm by
    the previous one (the per-tensor amax passes would otherwise be
    flattered).  A read, not a write: the lines it leaves behind are clean,
    so the next repetition's first kernel does not share HBM with the
    write-back of the flush itself (the previous repetition's dirty lines are
    written back during the flush)."""

    def __init__(self, device):
        self.buf = torch.ones(FLUSH_BYTES // 4, dtype=torch.int32, device=device)

    def __call__(self):
        torch.sum(self.buf, dtype=torch.int64)


def progress(msg):
    """One line on stderr as each part of the run finishes."""
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def median(v):
    v = sorted(v)
    n = len(v)
    return v[n // 2] if n % 2 else 0.5 * (v[n // 2 - 1] + v[n // 2])


def timed_reps(run, reps, flush):
    """reps repetitions of run(events), each after a flush and bracketed by
    HIP events on the launch stream.  Returns (per-repetition ms, events)."""
    ev, marks = {}, []
    for _ in range(reps):
        flush()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        run(ev)
        e1.record()
        marks.append((e0, e1))
    torch.cuda.synchronize()
    return [a.elapsed_time(b) for a, b in marks], ev


def per_call_median(ev):
    """name -> median ms over the repetitions of that call."""
    return {k: median([a.elapsed_time(b) for a, b in v]) for k, v in ev.items()}


class Step:
    """Preallocated buffers and the launch sequence of one MLP-layer step."""

    def __init__(self, workload, rht, device, bx=True):
        self.dev = device
        self.lib = bsq.lib()
        self.stream = ctypes.c_void_p(torch.cuda.current_stream(device).cuda_stream)
        self.rht = 1 if rht else 0
        self.signs = synth.rht_sign_mask(synth.RHT_SEED[workload])
        self.seed = synth.SR_SEED[workload]
        t = {k: synth.workload_tensor(workload, k, device) for k in synth.WORKLOADS[workload]}
        self.t = t
        T, Hd = t["X"].shape
        F2 = t["W_gu"].shape[0]
        F = t["W_down"].shape[1]
        self.dims = dict(tokens=T, hidden=Hd, ffn=F)
        u8 = lambda *s: torch.empty(s, dtype=torch.uint8, device=device)
        f32 = lambda: torch.empty(1, dtype=torch.float32, device=device)
        bf = lambda *s: torch.empty(s, dtype=torch.bfloat16, device=device)
        q = {}
        for name, (R, C) in (("X", (T, Hd)), ("W_gu", (F2, Hd)), ("H", (T, F)),
                             ("W_down", (Hd, F)), ("dY_gu", (T, F2)), ("dY_down", (T, Hd))):
            q[name] = dict(rc=u8(R, C // 2), rs=u8(R, C // 16), ra=f32(),
                           cc=u8(C, R // 2), cs=u8(C, R // 16), ca=f32())
        self.q = q
        self.out = dict(Y_gu=bf(T, F2), Y_down=bf(T, Hd), dH=bf(T, F), dW_down=bf(Hd, F),
                        dX=bf(T, Hd), dW_gu=bf(F2, Hd))
        # (name, A operand, B operand, M, N, K)
        self.gemms = [
            ("FPROP_gu", ("X", "r"), ("W_gu", "r"), T, F2, Hd),
            ("FPROP_down", ("H", "r"), ("W_down", "r"), T, Hd, F),
            ("DGRAD_down", ("dY_down", "r"), ("W_down", "c"), T, F, Hd),
            ("WGRAD_down", ("dY_down", "c"), ("H", "c"), Hd, F, T),
            ("DGRAD_gu", ("dY_gu", "r"), ("W_gu", "c"), T, Hd, F2),
            ("WGRAD_gu", ("dY_gu", "c"), ("X", "c"), F2, Hd, T),
        ]
        # GEMMs whose B operand is expanded to FP16 once (nvfp4_expand right
        # after its quantization) and fed to bs_gemm_nvfp4_bx
        self.bx = {g[0]: bx and bsq.bx_pays(g[4], g[5]) for g in self.gemms}
        self.xb = {}
        for g in self.gemms:
            if self.bx[g[0]]:
                self.xb[g[2]] = torch.empty((g[4], g[5]), dtype=torch.float16, device=device)
        self.flops = sum(2.0 * M * N * K for _, _, _, M, N, K in self.gemms)
        self.gemm_flops = {g[0]: 2.0 * g[3] * g[4] * g[5] for g in self.gemms}
        self.gemm_out = dict(FPROP_gu="Y_gu", FPROP_down="Y_down", DGRAD_down="dH",
                             WGRAD_down="dW_down", DGRAD_gu="dX", WGRAD_gu="dW_gu")
        # quantizer input bytes (BF16) + algorithmic output bytes per call
        self.quant_bytes = {}
        for name, x in t.items():
            n = x.numel()
            # amax pass reads x, encode pass reads x and writes 2 x (codes + scales)
            self.quant_bytes[name] = 2 * n + 2 * n + 2 * (n // 2 + n // 16)

    def quant(self, name, rnd, rht_col, block_rows=1):
        x, b = self.t[name], self.q[name]
        R, C = x.shape
        st = self.lib.quantize_transpose(P(x), R, C, NV, block_rows, rnd, self.seed, 0,
                                         rht_col, self.signs, P(b["rc"]), P(b["rs"]), P(b["ra"]),
                                         P(b["cc"]), P(b["cs"]), P(b["ca"]), self.stream)
        assert st == 0, (name, bsq.status_string(st))

    def expand(self, name):
        """FP16 expansions of tensor `name`'s quantized orientations that a GEMM
        takes pre-expanded."""
        for (bn, bo), out in self.xb.items():
            if bn != name:
                continue
            b = self.q[bn]
            R, C = out.shape
            st = self.lib.nvfp4_expand(P(b[bo + "c"]), P(b[bo + "s"]), R, C, P(out), self.stream)
            assert st == 0, (name, bsq.status_string(st))

    def gemm(self, g):
        name, (an, ao), (bn, bo), M, N, K = g
        a, b = self.q[an], self.q[bn]
        c = self.out[self.gemm_out[name]]
        if self.bx[name]:
            st = self.lib.bs_gemm_nvfp4_bx(M, N, K, P(a[ao + "c"]), P(a[ao + "s"]), P(a[ao + "a"]),
                                           P(self.xb[(bn, bo)]), P(b[bo + "a"]), P(c), N, self.stream)
        else:
            st = self.lib.bs_gemm(NV, M, N, K, P(a[ao + "c"]), P(a[ao + "s"]), P(a[ao + "a"]),
                                  P(b[bo + "c"]), P(b[bo + "s"]), P(b[bo + "a"]), P(c), N, self.stream)
        assert st == 0, (name, bsq.status_string(st))

    def run(self, events=None):
        """One step.  events: optional dict name -> list of (start, end) to record GEMM/quant times."""
        def timed(name, fn):
            if events is None:
                fn()
                return
            s, e = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            s.record()
            fn()
            e.record()
            events.setdefault(name, []).append((s, e))
        G = {g[0]: g for g in self.gemms}
        expanded = {bn for bn, _ in self.xb}

        def q(name, rnd, rht, block_rows=1):
            timed("q_" + name, lambda: self.quant(name, rnd, rht, block_rows))
            if name in expanded:
                timed("x_" + name, lambda: self.expand(name))
        q("X", RNE, self.rht)
        q("W_gu", RNE, 0, 16)
        timed("FPROP_gu", lambda: self.gemm(G["FPROP_gu"]))
        q("H", RNE, self.rht)
        q("W_down", RNE, 0, 16)
        timed("FPROP_down", lambda: self.gemm(G["FPROP_down"]))
        q("dY_down", SR, self.rht)
        timed("DGRAD_down", lambda: self.gemm(G["DGRAD_down"]))
        timed("WGRAD_down", lambda: self.gemm(G["WGRAD_down"]))
        q("dY_gu", SR, self.rht)
        timed("DGRAD_gu", lambda: self.gemm(G["DGRAD_gu"]))
        timed("WGRAD_gu", lambda: self.gemm(G["WGRAD_gu"]))


class Fp8Step:
    """The same MLP-layer step with the per-tensor FP8 baseline the NVFP4 post
    compares against (section "Performance results"): every tensor quantized
    by fp8_quantize_transpose (E4M3 codes of x and x^T under 448 / amax), the
    six GEMMs on the FP8 matrix path.  Shares the BF16 inputs of `step`."""

    def __init__(self, step):
        self.step = step
        self.vendor = False
        dev = step.dev
        u8 = lambda *s_: torch.empty(s_, dtype=torch.uint8, device=dev)
        self.q = {}
        for name, x in step.t.items():
            R, C = x.shape
            self.q[name] = dict(rc=u8(R, C), cc=u8(C, R),
                                ra=torch.empty(1, dtype=torch.float32, device=dev))

    def quant(self, name):
        x, b, st = self.step.t[name], self.q[name], self.step
        R, C = x.shape
        r = st.lib.fp8_quantize_transpose(P(x), R, C, P(b["rc"]), P(b["cc"]), P(b["ra"]), st.stream)
        assert r == 0, (name, bsq.status_string(r))

    def gemm(self, g):
        name, (an, ao), (bn, bo), M, N, K = g
        st = self.step
        a, b = self.q[an], self.q[bn]
        c = st.out[st.gemm_out[name]]
        if self.vendor:
            # the same FP8 codes and decode scales through the vendor GEMM
            # (hipBLASLt behind torch._scaled_mm), for comparison only
            f8 = torch.float8_e4m3fn
            torch._scaled_mm(a[ao + "c"].view(f8), b[bo + "c"].view(f8).t(), scale_a=self.sdec[an],
                             scale_b=self.sdec[bn], out_dtype=torch.bfloat16, out=c)
            return
        r = st.lib.bs_gemm(FP8, M, N, K, P(a[ao + "c"]), None, P(a["ra"]), P(b[bo + "c"]), None,
                           P(b["ra"]), P(c), N, st.stream)
        assert r == 0, (name, bsq.status_string(r))

    def vendor_scales(self):
        """Decode scales 1 / (448 / amax) of the quantized tensors, as the
        vendor GEMM takes them (device float32 scalars)."""
        self.sdec = {n: (1.0 / (448.0 / b["ra"][0])).reshape(()) for n, b in self.q.items()}

    def run(self, events=None):
        G = {g[0]: g for g in self.step.gemms}
        order = ["q:X", "q:W_gu", "FPROP_gu", "q:H", "q:W_down", "FPROP_down", "q:dY_down",
                 "DGRAD_down", "WGRAD_down", "q:dY_gu", "DGRAD_gu", "WGRAD_gu"]
        for item in order:
            fn = (lambda n=item[2:]: self.quant(n)) if item.startswith("q:") else (lambda n=item: self.gemm(G[n]))
            if events is None:
                fn()
                continue
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            fn()
            e1.record()
            events.setdefault(item, []).append((e0, e1))


def rht_wgrad_error(step):
    """Accuracy side of the recipe's RHT (WGRAD inputs only): relative
    Frobenius error of the NVFP4 WGRAD_down output dW = dY_down^T . H against
    the FP64 product of the same BF16 inputs, with the column RHT on and off
    (dY_down: SR; H: RNE, N(0,1) with 0.1% x50 outliers)."""
    g = {x[0]: x for x in step.gemms}["WGRAD_down"]
    dY, Hm = step.t["dY_down"], step.t["H"]
    ref = dY.double().t() @ Hm.double()
    nref = float(torch.linalg.norm(ref))
    out = {}
    saved = step.rht
    for flag, key in ((1, "rht_on"), (0, "rht_off")):
        step.rht = flag
        step.quant("dY_down", SR, flag)
        step.quant("H", RNE, flag)
        step.gemm(g)
        torch.cuda.synchronize()
        c = step.out[step.gemm_out["WGRAD_down"]].double()
        out[key] = float(torch.linalg.norm(c - ref)) / nref
    step.rht = saved
    del ref
    out["error_ratio_on_over_off"] = out["rht_on"] / out["rht_off"]
    return {k: round(v, 6) for k, v in out.items()}


def fp8_baseline(step, steps, warmup, nvfp4_ms, flush):
    """Times Fp8Step like the NVFP4 step (median over repetitions, flushed
    between them); reports its rate and the NVFP4 step's speed relative to
    it (the pages' metric: NVFP4 over FP8 step throughput).  The same step
    with the vendor's per-tensor FP8 GEMM (hipBLASLt through torch._scaled_mm)
    on the same codes gives a second denominator: the fastest FP8 GEMM this
    card has, with this library's FP8 quantizers."""
    f = Fp8Step(step)
    for _ in range(max(1, warmup)):
        flush()
        f.run()
    ms_list, ev = timed_reps(f.run, steps, flush)
    ms = median(ms_list)
    per = per_call_median(ev)
    gemm_ms = sum(per[g[0]] for g in step.gemms)
    quant_ms = sum(v for k, v in per.items() if k.startswith("q:"))
    out = {"format": "per-tensor FP8 (E4M3, s = 448/amax) on the FP8 MFMA",
           "ms_per_step": round(ms, 4),
           "value": round(step.flops / (ms * 1e-3) / 1e12, 2),
           "gemm_tflops": round(step.flops / (gemm_ms * 1e-3) / 1e12, 1),
           "gemm_frac_of_fp8_peak": round(step.flops / (gemm_ms * 1e-3) / 1e12 / PEAK_FP8_TFLOPS, 4),
           "quant_ms": round(quant_ms, 4),
           "nvfp4_speedup_over_fp8": round(ms / nvfp4_ms, 4)}
    try:
        f.vendor = True
        f.vendor_scales()
        for _ in range(max(1, warmup)):
            flush()
            f.run()
        vms_list, vev = timed_reps(f.run, steps, flush)
        vms = median(vms_list)
        vper = per_call_median(vev)
        vgemm = sum(vper[g[0]] for g in step.gemms)
        out["vendor_fp8_gemm"] = {
            "gemm": "hipBLASLt per-tensor FP8 (torch._scaled_mm) on the same E4M3 codes and scales",
            "ms_per_step": round(vms, 4),
            "gemm_ms": round(vgemm, 4),
            "gemm_tflops": round(step.flops / (vgemm * 1e-3) / 1e12, 1),
            "gemm_frac_of_fp8_peak": round(step.flops / (vgemm * 1e-3) / 1e12 / PEAK_FP8_TFLOPS, 4),
            "nvfp4_speedup_over_fp8": round(vms / nvfp4_ms, 4)}
    except (RuntimeError, AttributeError, TypeError) as e:     # no FP8 GEMM in this torch build
        out["vendor_fp8_gemm"] = {"error": str(e)[:200]}
    f.vendor = False
    del f
    return out


def vendor_fp16_gemm(step, nvfp4_gemm_ms, flush, reps=5):
    """For scale: the vendor's FP16 GEMM (hipBLASLt through torch.mm) on the
    step's six GEMMs with both operands pre-expanded to the same FP16 values
    the NVFP4 GEMM forms in its tiles (nvfp4_expand of the step's codes and
    scales), FP32 accumulation.  Pure GEMM time, flushed medians; the
    expansion is not timed.  One GEMM's operands are held at a time."""
    tot = 0.0
    per = {}
    for name, (an, ao), (bn, bo), M, N, K in step.gemms:
        a, b = step.q[an], step.q[bn]
        A16 = bsq.nvfp4_expand(a[ao + "c"], a[ao + "s"])
        B16 = bsq.nvfp4_expand(b[bo + "c"], b[bo + "s"])
        C16 = torch.empty((M, N), dtype=torch.float16, device=step.dev)
        run = lambda ev: torch.mm(A16, B16.t(), out=C16)
        for _ in range(2):
            run(None)
        ms_list, _ = timed_reps(run, reps, flush)
        per[name] = median(ms_list)
        tot += per[name]
        del A16, B16, C16
        torch.cuda.empty_cache()
    tf = step.flops / (tot * 1e-3) / 1e12
    return {"gemm": "hipBLASLt FP16 GEMM (torch.mm) on both operands pre-expanded to FP16 (nvfp4_expand), "
                    "the values the NVFP4 GEMM forms in its tiles; expansion not timed",
            "gemm_ms": round(tot, 4), "gemm_tflops": round(tf, 1),
            "gemm_frac_of_fp16_peak": round(tf / PEAK_FP16_TFLOPS, 4),
            "per_gemm_tflops": {k: round(step.gemm_flops[k] / (v * 1e-3) / 1e12, 1) for k, v in per.items()},
            "nvfp4_gemm_over_vendor_fp16": round(tot / nvfp4_gemm_ms, 4)}


def swiglu_fused(step, reps=10):
    """The producer-side fusion around the H and dY_gu quantizers: SwiGLU
    forward of the step's Y_gu (FPROP_gu output) and backward with its dH
    (DGRAD_down output), each followed by the NVFP4 quantize_transpose of its
    output; unfused = SwiGLU alone, then quantize_transpose with its own amax
    pass; fused = SwiGLU that also emits both amaxes, then
    quantize_transpose_amax.  Median of `reps` timings per route (HIP events
    on the launch stream); the SwiGLU kernels' own rate against the HBM peak
    (algorithmic bytes: forward 6 B, backward 10 B per element of H)."""
    lib, s, dev = step.lib, step.stream, step.dev
    Y, dH = step.out["Y_gu"], step.out["dH"]
    T, F2 = Y.shape
    F = F2 // 2
    H = torch.empty((T, F), dtype=torch.bfloat16, device=dev)
    dY = torch.empty((T, F2), dtype=torch.bfloat16, device=dev)
    am = [torch.empty(1, dtype=torch.float32, device=dev) for _ in range(2)]
    qh, qd = step.q["H"], step.q["dY_gu"]
    rht, signs, seed = step.rht, step.signs, step.seed

    def ok(st):
        assert st == 0, bsq.status_string(st)

    def fwd(amax):
        ok(lib.swiglu_amax(P(Y), T, F, rht, signs, P(H), P(am[0]) if amax else None,
                           P(am[1]) if amax else None, s))

    def bwd(amax):
        ok(lib.swiglu_backward_amax(P(Y), P(dH), T, F, rht, signs, P(dY), P(am[0]) if amax else None,
                                    P(am[1]) if amax else None, s))

    def qt(x, b, rnd):
        R, C = x.shape
        ok(lib.quantize_transpose(P(x), R, C, NV, 1, rnd, seed, 0, rht, signs, P(b["rc"]), P(b["rs"]),
                                  P(b["ra"]), P(b["cc"]), P(b["cs"]), P(b["ca"]), s))

    def qta(x, b, rnd):
        R, C = x.shape
        ok(lib.quantize_transpose_amax(P(x), R, C, 1, rnd, seed, 0, rht, signs, P(am[0]), P(am[1]),
                                       P(b["rc"]), P(b["rs"]), P(b["cc"]), P(b["cs"]), s))

    routes = {
        "fwd_unfused": lambda: (fwd(False), qt(H, qh, RNE)),
        "fwd_fused": lambda: (fwd(True), qta(H, qh, RNE)),
        "bwd_unfused": lambda: (bwd(False), qt(dY, qd, SR)),
        "bwd_fused": lambda: (bwd(True), qta(dY, qd, SR)),
        "swiglu_fwd_amax": lambda: fwd(True),
        "swiglu_bwd_amax": lambda: bwd(True),
    }
    res = {}
    for name, fn in routes.items():
        for _ in range(2):
            fn()
        ts = []
        for _ in range(reps):
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            fn()
            e1.record()
            ts.append((e0, e1))
        torch.cuda.synchronize()
        v = sorted(a.elapsed_time(b) for a, b in ts)
        res[name] = v[len(v) // 2]
    n = T * F
    out = {"shape": {"tokens": T, "ffn": F}, "rht_col": bool(rht)}
    for k in ("fwd", "bwd"):
        out[k] = {"unfused_ms": round(res[k + "_unfused"], 4), "fused_ms": round(res[k + "_fused"], 4),
                  "speedup": round(res[k + "_unfused"] / res[k + "_fused"], 4)}
    for k, b in (("swiglu_fwd_amax", 6 * n), ("swiglu_bwd_amax", 10 * n)):
        gbs = b / (res[k] * 1e-3) / 1e9
        out[k] = {"ms": round(res[k], 4), "gbs": round(gbs, 1), "frac_of_hbm_peak": round(gbs / PEAK_HBM_GBS, 4)}
    del H, dY
    return out


def mlp_layer_step(step, steps, warmup, rel_update=1e-4):
    """The whole MLP-layer training step chained through the C ABI
    (fp8_quantized_gemm_amd.mlp.MLPLayer): quantizers, the six GEMMs, the
    SwiGLU forward and backward with their fused amaxes, encode-only
    quantizers of H and dY_gu and of the weights (amax from the update), and
    the FP32 master-weight update of W_gu and W_down.  Same shapes and inputs
    as the plain step (X, dY_down; W masters from the BF16 weights).  The
    learning rate is set from one untimed step so that an update moves each
    master weight by about rel_update of its norm: the same inputs every step
    with a fixed large rate would drive the weights, and then every operand,
    to overflow within a few steps (the 405B gradients are N(0,1))."""
    from fp8_quantized_gemm_amd.mlp import MLPLayer
    t = step.t
    layer = MLPLayer(t["W_gu"].float(), t["W_down"].float(), step.dims["tokens"], rht=bool(step.rht),
                     rht_signs=step.signs, sr_seed=step.seed, lr=0.0)
    x, dy = t["X"], t["dY_down"]
    layer.step(x, dy)
    torch.cuda.synchronize()
    layer.lr = rel_update * min(float(layer.w32[k].norm() / layer.grad[k].float().norm())
                                for k in ("W_gu", "W_down"))
    for _ in range(max(1, warmup)):
        layer.step(x, dy)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(steps):
        layer.step(x, dy)
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / steps
    finite = all(bool(torch.isfinite(v).all()) for v in (layer.act["Y_down"], layer.act["dX"],
                                                          layer.w32["W_gu"], layer.w32["W_down"]))
    out = {"ms_per_step": round(ms, 4), "value": round(layer.flops / (ms * 1e-3) / 1e12, 2),
           "unit": "TFLOP/s (the six GEMMs' 2MNK over the whole layer step)",
           "lr": layer.lr, "outputs_finite": finite,
           "includes": "quantizers, 6 NVFP4 GEMMs, SwiGLU fwd/bwd with fused amaxes, "
                       "FP32 master-weight update of W_gu and W_down"}
    del layer
    return out


def route_ceilings(device, iters=4000, blocks=1024):
    """Inner-loop ceilings of the exact NVFP4 GEMM routes (operands in
    registers, no memory): route (a), a per-16-K MFMA on unscaled E2M1 values
    plus the VALU rescale acc += sA * sB * P, on the FP16 32x32x16 MFMA and on
    the scaled FP4 32x32x64 MFMA (one 16-block per instruction); route (b)'s
    FP16 MFMAs accumulating directly; and the scaled FP4 MFMA accumulating
    directly over all 64 K positions (the MXFP4 instruction's own ceiling);
    route (b) on the 16x16x32 FP16 MFMA the GEMM uses, alone and with one
    expansion pair (two VALU operations) per MFMA as in the GEMM's loop.
    Useful flops only (a 16-block per route-(a) instruction).  Two timed
    launches each (HIP events on the launch stream), the second reported."""
    path = os.path.join(ROOT, "fp8_quantized_gemm_amd", "libbsq_ceiling.so")
    L = ctypes.CDLL(path)
    L.bsq_route_ceiling.argtypes = [ctypes.c_int, ctypes.c_void_p, ctypes.c_int, ctypes.c_int, ctypes.c_void_p]
    L.bsq_route_ceiling.restype = ctypes.c_int
    stream = ctypes.c_void_p(torch.cuda.current_stream(device).cuda_stream)
    sink = torch.zeros(blocks * 512, dtype=torch.float32, device=device)
    flops16 = blocks * 8 * iters * 8 * 2.0 * 32 * 32 * 16
    out = {}
    for mode, key, kmul, peak in ((1, "route_b_fp16_mfma_only", 1, PEAK_FP16_TFLOPS),
                                  (0, "route_a_fp16_mfma_plus_valu_rescale", 1, PEAK_FP16_TFLOPS),
                                  (2, "route_a_scaled_fp4_mfma_plus_valu_rescale", 1, PEAK_FP16_TFLOPS),
                                  (3, "mxfp4_scaled_mfma_only", 4, PEAK_FP4_TFLOPS),
                                  (4, "route_b_fp16_16x16x32_mfma_only", 0.5, PEAK_FP16_TFLOPS),
                                  (5, "route_b_fp16_16x16x32_mfma_plus_expansion_pair", 0.5, PEAK_FP16_TFLOPS)):
        for _ in range(2):
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            st = L.bsq_route_ceiling(mode, P(sink), iters, blocks, stream)
            e1.record()
            assert st == 0, st
            torch.cuda.synchronize()
        ms = e0.elapsed_time(e1)
        tf = flops16 * kmul / (ms * 1e-3) / 1e12
        out[key] = {"ms": round(ms, 3), "tflops": round(tf, 1), "frac_of_peak": round(tf / peak, 4),
                    "peak_tflops": peak}
    out["note"] = ("MFMA loops with operands in registers; route (a) counts the 16-block's flops "
                   "(the scaled FP4 instruction runs 64 K positions, 48 of them zero); the "
                   "complete route (b) GEMM (roofline.achieved) includes all memory traffic and "
                   "the expansion, whose instruction mix the 16x16x32 plus-expansion loop has")
    return out


def mx_square(device, reps=20):
    """The MX workload (4096 x 4096 x 4096, A and B N(0,1) with outliers):
    rowwise mx_quantize of both operands, then the block-scaled GEMM, for MXFP8
    and MXFP4.  Median of `reps` timed repetitions of each call (HIP events on
    the launch stream)."""
    lib = bsq.lib()
    stream = ctypes.c_void_p(torch.cuda.current_stream(device).cuda_stream)
    A = synth.workload_tensor("mx", "A", device)
    B = synth.workload_tensor("mx", "B", device)
    M, K = A.shape
    N = B.shape[0]
    out = {}
    for fmt, fcode, peak in (("mxfp8", MXF8, PEAK_FP8_TFLOPS), ("mxfp4", MXF4, PEAK_FP4_TFLOPS)):
        cw = K if fmt == "mxfp8" else K // 2
        ac = torch.empty((M, cw), dtype=torch.uint8, device=device)
        bc = torch.empty((N, cw), dtype=torch.uint8, device=device)
        as_ = torch.empty((M, K // 32), dtype=torch.uint8, device=device)
        bs = torch.empty((N, K // 32), dtype=torch.uint8, device=device)
        C = torch.empty((M, N), dtype=torch.bfloat16, device=device)

        def quant():
            for x, c_, s_ in ((A, ac, as_), (B, bc, bs)):
                st = lib.mx_quantize(P(x), x.shape[0], K, fcode, RNE, 0, 0, P(c_), P(s_), stream)
                assert st == 0, bsq.status_string(st)

        def gemm():
            st = lib.bs_gemm(fcode, M, N, K, P(ac), P(as_), None, P(bc), P(bs), None, P(C), N, stream)
            assert st == 0, bsq.status_string(st)

        def median_ms(fn):
            for _ in range(3):
                fn()
            ts = []
            for _ in range(reps):
                e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                e0.record()
                fn()
                e1.record()
                ts.append((e0, e1))
            torch.cuda.synchronize()
            v = sorted(a.elapsed_time(b) for a, b in ts)
            return v[len(v) // 2]

        q_ms, g_ms = median_ms(quant), median_ms(gemm)
        tf = 2.0 * M * N * K / (g_ms * 1e-3) / 1e12
        qbytes = 2 * (M + N) * K + (M + N) * (cw + K // 32)
        out[fmt] = {"gemm_ms": round(g_ms, 4), "gemm_tflops": round(tf, 1),
                    "gemm_frac_of_peak": round(tf / peak, 4), "peak_tflops": peak,
                    "quant_ms": round(q_ms, 4), "quant_gbs": round(qbytes / (q_ms * 1e-3) / 1e9, 1),
                    "tflops_incl_quant": round(2.0 * M * N * K / ((g_ms + q_ms) * 1e-3) / 1e12, 1)}
    return out


def gemm_traffic(workload):
    """HBM bytes per NVFP4 GEMM call (all its dispatches) from the committed rocprofv3 FETCH_SIZE /
    WRITE_SIZE summary of this workload, or None when the kernel sources have
    changed since those counters were taken (the summary stores their SHA-256)."""
    import hashlib
    path = os.path.join(ROOT, "profiles", f"nvfp4_gemm_{workload}_traffic.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        rec = json.load(f)
    h = hashlib.sha256()
    for src in rec["sources"]:
        with open(os.path.join(ROOT, src), "rb") as f:
            h.update(f.read())
    return rec["bytes_per_launch"] if h.hexdigest() == rec["sources_sha256"] else None


def cpu_baseline(workload, rht):
    """The oracle on a bounded slice of the same workload (about 10-25 s of host
    work): FPROP_gu for the first TOK tokens and the first NOUT output features (quantize X rows 1x16 RNE,
    W_gu rows 16x16 RNE, FP64 GEMM), with the per-tensor amax of both full
    tensors.  Reports TFLOP/s of that slice."""
    import numpy as np
    from oracle import gemm as G
    from oracle import quantize as Q
    try:
        from threadpoolctl import threadpool_info
        blas_threads = max([i.get("num_threads", 1) for i in threadpool_info()] + [1])
    except Exception:
        blas_threads = os.cpu_count() or 1
    TOK, NOUT = 24576, 28672                  # about 10-25 s with 16 host cores
    X = synth.workload_tensor(workload, "X", "cpu")
    W = synth.workload_tensor(workload, "W_gu", "cpu")
    bits = lambda t: t.contiguous().view(torch.int16).numpy().view(np.uint16)
    xb, wb = bits(X), bits(W)
    t0 = time.perf_counter()
    ax = Q.tensor_amax(Q.as_f32(xb))
    aw = Q.tensor_amax(Q.as_f32(wb))
    xc, xs, _ = Q.nvfp4_quantize(xb[:TOK], 1, amax=ax)
    wc, ws, _ = Q.nvfp4_quantize(wb[:NOUT], 16, amax=aw)
    C = G.gemm_nvfp4(xc, xs, ax, wc, ws, aw)
    dt = time.perf_counter() - t0
    K = xb.shape[1]
    flops = 2.0 * TOK * NOUT * K
    assert C.shape == (TOK, NOUT)
    return {"value": flops / dt / 1e12, "unit": "TFLOP/s", "cores": int(max(1, blas_threads)),
            "kind": "oracle",
            "sample": (f"FPROP_gu slice: {TOK} tokens x {NOUT} outputs x K={K} "
                       f"(X rows 1x16 RNE, W_gu rows 16x16 RNE, full-tensor amax of X and W_gu, "
                       f"FP64 GEMM) in {dt:.2f} s; quantizers single-threaded NumPy, GEMM BLAS")}


def tiny_fprop(device, reps=50):
    """The tiny NVFP4 FPROP (256 x 256 x 256: A 1x16 RNE, W 16x16 RNE, no
    RHT), timed for the record: nvfp4_quantize of both operands and the GEMM.
    Launch-bound at this size.  Median over `reps` repetitions."""
    lib = bsq.lib()
    stream = ctypes.c_void_p(torch.cuda.current_stream(device).cuda_stream)
    A = synth.workload_tensor("tiny", "A", device)
    W = synth.workload_tensor("tiny", "W", device)
    M, K = A.shape
    N = W.shape[0]
    u8 = lambda *s_: torch.empty(s_, dtype=torch.uint8, device=device)
    f32 = lambda: torch.empty(1, dtype=torch.float32, device=device)
    ac, as_, aa, wc, ws, wa = u8(M, K // 2), u8(M, K // 16), f32(), u8(N, K // 2), u8(N, K // 16), f32()
    C = torch.empty((M, N), dtype=torch.bfloat16, device=device)

    def quant():
        for x, c, sc, am, br in ((A, ac, as_, aa, 1), (W, wc, ws, wa, 16)):
            st = lib.nvfp4_quantize(P(x), x.shape[0], K, br, RNE, 0, 0, 0, 0, None, P(c), P(sc), P(am), stream)
            assert st == 0, bsq.status_string(st)

    def gemm():
        st = lib.bs_gemm(NV, M, N, K, P(ac), P(as_), P(aa), P(wc), P(ws), P(wa), P(C), N, stream)
        assert st == 0, bsq.status_string(st)

    def med(fn):
        for _ in range(5):
            fn()
        ts = []
        for _ in range(reps):
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            fn()
            e1.record()
            ts.append((e0, e1))
        torch.cuda.synchronize()
        return median([a.elapsed_time(b) for a, b in ts])

    q_ms, g_ms = med(quant), med(gemm)
    fl = 2.0 * M * N * K
    return {"shape": [M, N, K], "quant_ms": round(q_ms, 5), "gemm_ms": round(g_ms, 5),
            "gemm_tflops": round(fl / (g_ms * 1e-3) / 1e12, 2),
            "tflops_incl_quant": round(fl / ((q_ms + g_ms) * 1e-3) / 1e12, 2),
            "note": "launch-bound (one 256x256 output tile); timed for the record"}


def run_step_bench(workload, rht, device, steps, warmup, flush, bx=True):
    """Warm up, then time `steps` flushed repetitions of one MLP-layer step.
    Returns (step, per-step ms list, per-call median ms, wall seconds)."""
    step = Step(workload, rht, device, bx=bx)
    torch.cuda.synchronize()
    for _ in range(warmup):
        flush()
        step.run()
    torch.cuda.synchronize()
    wall0 = time.perf_counter()
    ms_list, ev = timed_reps(step.run, steps, flush)
    wall = time.perf_counter() - wall0
    return step, ms_list, per_call_median(ev), wall


def step_summary(step, ms, per):
    gemm_names = [g[0] for g in step.gemms]
    gemm_ms = sum(per[n] for n in gemm_names)
    gemm_tflops = step.flops / (gemm_ms * 1e-3) / 1e12
    breakdown = {}
    for n in gemm_names:
        breakdown[n] = {"ms": round(per[n], 4),
                        "tflops": round(step.gemm_flops[n] / (per[n] * 1e-3) / 1e12, 1)}
    for n in ("X", "W_gu", "H", "W_down", "dY_down", "dY_gu"):
        k = "q_" + n
        breakdown[k] = {"ms": round(per[k], 4),
                        "gbs": round(step.quant_bytes[n] / (per[k] * 1e-3) / 1e9, 1)}
        if "x_" + n in per:   # FP16 expansions: 0.5625 B read + 2 B written per element
            nel = sum(o.numel() for (bn, _), o in step.xb.items() if bn == n)
            breakdown["x_" + n] = {"ms": round(per["x_" + n], 4),
                                   "gbs": round(2.5625 * nel / (per["x_" + n] * 1e-3) / 1e9, 1)}
    return gemm_ms, gemm_tflops, breakdown


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default="8b", choices=["8b", "405b"])
    ap.add_argument("--no-rht", action="store_true")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-mx", action="store_true", help="skip the MX square-GEMM lines")
    ap.add_argument("--no-fp8", action="store_true", help="skip the per-tensor FP8 baseline step")
    ap.add_argument("--no-vendor-fp16", action="store_true",
                    help="skip the vendor FP16 GEMM on pre-expanded operands (for scale)")
    ap.add_argument("--no-swiglu", action="store_true", help="skip the fused SwiGLU + quantize lines")
    ap.add_argument("--no-bx", action="store_true",
                    help="expand every B operand inside the GEMM (no pre-expanded weights)")
    ap.add_argument("--no-route-ceiling", action="store_true",
                    help="skip the inner-loop ceilings of the two NVFP4 GEMM routes")
    ap.add_argument("--no-405b", action="store_true",
                    help="skip the Llama-3.1-405B layer summary of the default (8B) run")
    ap.add_argument("--no-tiny", action="store_true", help="skip the 256^3 FPROP record")
    ap.add_argument("--only", choices=["route-ceilings", "mx-square"],
                    help="run one auxiliary leg alone and print its JSON (for counter profiles)")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (got --gpus {args.gpus}); the multi-GPU path "
              f"is a design note, not built", file=sys.stderr)
        sys.exit(2)

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    if args.only:
        leg = {"route-ceilings": route_ceilings, "mx-square": mx_square}[args.only]
        print(json.dumps({args.only: leg(dev)}))
        return
    flush = Flusher(dev)
    step, ms_list, per, wall = run_step_bench(args.workload, not args.no_rht, dev, args.steps,
                                              args.warmup, flush, bx=not args.no_bx)
    ms = median(ms_list)
    progress(f"{args.workload} step: {ms:.3f} ms")

    # the same step with RHT off on the WGRAD operands (only the quantizers change)
    step.rht = 1 - step.rht
    for _ in range(max(1, args.warmup)):
        flush()
        step.run()
    other_list, _ = timed_reps(step.run, args.steps, flush)
    step.rht = 1 - step.rht
    ms_other = median(other_list)

    gemm_ms, gemm_tflops, breakdown = step_summary(step, ms, per)
    value = step.flops / (ms * 1e-3) / 1e12
    out = {
        "metric": "block-scaled GEMM TFLOP/s incl. quantize, Llama-3-8B MLP shapes; % MFMA peak",
        "value": round(value, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "nvfp4 (e2m1 x e4m3 blocks) -> exact fp16 expansion, fp16 mfma, fp32 accumulate, bf16 out",
        "data": ("synthetic (seeded N(0,1)+0.1% x50 outliers activations, N(0,0.02^2) weights, "
                 "N(0,1e-3^2) gradients)" if args.workload == "8b" else
                 "synthetic (seeded N(0,1)+0.1% x50 outliers activations and gradients, N(0,0.01^2) weights)"),
        "config": {"workload": f"llama3-{args.workload} MLP layer FPROP+DGRAD+WGRAD, one GPU share",
                   "tokens": step.dims["tokens"], "hidden": step.dims["hidden"],
                   "ffn": step.dims["ffn"], "rht": not args.no_rht,
                   "step_tflop": round(step.flops / 1e12, 3),
                   "pct_of_fp16_mfma_peak": round(100 * value / PEAK_FP16_TFLOPS, 2)},
        "timing": (f"median of {args.steps} steps (HIP events on the launch stream), a 1 GiB "
                   f"scratch read between steps; mean {sum(ms_list) / len(ms_list):.4f} ms"),
        "roofline": {"bound": "mfma", "kernel": ("NVFP4 GEMM, 6 calls per step: k_gemm_nvfp4_rx (a last wave of "
                                                 "tiles filling at most half the CUs split over K + join)" +
                                                 "".join(f"; k_gemm_nvfp4_px for {n}" for n, v in step.bx.items() if v)),
                     "achieved": round(gemm_tflops, 1), "peak": PEAK_FP16_TFLOPS,
                     "unit": "TFLOP/s", "frac": round(gemm_tflops / PEAK_FP16_TFLOPS, 4),
                     "traffic": gemm_traffic(args.workload),
                     "traffic_unit": "HBM bytes per GEMM call (rocprofv3 FETCH_SIZE x2 + WRITE_SIZE)"},
        "breakdown": breakdown,
        ("rht_off" if not args.no_rht else "rht_on"): {
            "ms_per_step": round(ms_other, 4),
            "value": round(step.flops / (ms_other * 1e-3) / 1e12, 2)},
        "wall_s": round(wall, 3),
    }
    progress("step with the other RHT setting done")
    if not args.no_fp8:
        out["fp8_baseline"] = fp8_baseline(step, args.steps, args.warmup, ms, flush)
        progress("FP8 baseline done")
    if not args.no_vendor_fp16:
        out["vendor_fp16_gemm"] = vendor_fp16_gemm(step, step.flops / (gemm_tflops * 1e12) * 1e3, flush)
        progress("vendor FP16 GEMM done")
    if not args.no_swiglu:
        out["swiglu_fused_quantize"] = swiglu_fused(step)
        out["mlp_layer_step"] = mlp_layer_step(step, args.steps, args.warmup)
        progress("SwiGLU and MLP-layer step done")
    if args.workload == "8b":
        out["rht_wgrad_error"] = rht_wgrad_error(step)
        progress("RHT error done")
    del step
    torch.cuda.empty_cache()
    if args.workload == "8b" and not args.no_405b:
        s405, l405, p405, _ = run_step_bench("405b", not args.no_rht, dev, max(3, args.steps // 4),
                                             max(1, args.warmup // 2), flush, bx=not args.no_bx)
        m405 = median(l405)
        g_ms, g_tf, bd = step_summary(s405, m405, p405)
        out["workload_405b"] = {
            "workload": "llama3.1-405b MLP layer FPROP+DGRAD+WGRAD, one GPU share",
            "tokens": s405.dims["tokens"], "hidden": s405.dims["hidden"], "ffn": s405.dims["ffn"],
            "rht": not args.no_rht, "steps": len(l405), "step_tflop": round(s405.flops / 1e12, 3),
            "ms_per_step": round(m405, 4), "value": round(s405.flops / (m405 * 1e-3) / 1e12, 2),
            "gemm_ms": round(g_ms, 4), "gemm_tflops": round(g_tf, 1),
            "gemm_frac_of_fp16_peak": round(g_tf / PEAK_FP16_TFLOPS, 4), "breakdown": bd}
        del s405
        torch.cuda.empty_cache()
        progress("405b step done")
    if not args.no_tiny:
        out["tiny_fprop_256"] = tiny_fprop(dev)
    if not args.no_mx:
        out["mx_square_4096"] = mx_square(dev)
        progress("MX 4096^3 done")
    if not args.no_route_ceiling:
        out["nvfp4_route_ceilings"] = route_ceilings(dev)
        progress("route ceilings done")
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(args.workload, not args.no_rht)
        progress("CPU baseline done")
    print(json.dumps(out))


if __name__ == "__main__":
    main()
