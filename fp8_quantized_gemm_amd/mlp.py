"""One transformer-MLP layer's NVFP4 training step, driven through the C ABI.

Every step is a libbsq call on the current stream; this module only holds the
preallocated buffers and the launch order.  Data flow (NVFP4 pretraining post:
the data-flow paragraph after Figure 1 and the recipe's ingredients; the
SwiGLU MLP of the Llama models in "Performance results"):

  forward   q(X): rows RNE, columns RNE + RHT (amax pass + encode)
            q(W_gu), q(W_down): 16x16 tiles, under the amax the last update
              of the master weight produced (encode only); a weight orientation
              whose FP16 copy stays cache-resident is expanded once
              (nvfp4_expand) and its GEMMs take it pre-expanded
            Y_gu = X . W_gu^T;  H = SwiGLU(Y_gu), emitting H's amaxes
            q(H): rows RNE, columns RNE + RHT (encode only)
            Y_down = H . W_down^T
  backward  q(dY_down): rows SR, columns SR + RHT (amax pass + encode)
            dH = dY_down . W_down;  dW_down = dY_down^T . H
            dY_gu = SwiGLU backward (Y_gu, dH), emitting dY_gu's amaxes
            q(dY_gu): rows SR, columns SR + RHT (encode only)
            dX = dY_gu . W_gu;  dW_gu = dY_gu^T . X
  update    W <- W - lr * dW on the FP32 masters, writing the BF16 copies
            and their amaxes for the next step

Stochastic rounding uses counter word `offset` = 2 * step (dY_down) and
2 * step + 1 (dY_gu), so successive steps draw fresh bits.
"""

import ctypes

import torch

from . import bx_pays, lib as _lib, status_string

NV, RNE, SR = 0, 0, 1


def _p(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


class MLPLayer:
    """Buffers and launch sequence of one MLP layer (gate/up fused, SwiGLU).

    w_gu: FP32 master [2F, hidden]; w_down: FP32 master [hidden, F] (both
    copied).  tokens % 16 == 0, hidden % 16 == 0, F % 16 == 0."""

    def __init__(self, w_gu, w_down, tokens, rht=True, rht_signs=0, sr_seed=0, lr=1e-4):
        if not (w_gu.is_cuda and w_down.is_cuda and w_gu.device == w_down.device):
            raise ValueError("the master weights must be CUDA tensors on one device")
        dev = w_gu.device
        self.lib = _lib()
        self.dev = dev
        F2, Hd = w_gu.shape
        F = F2 // 2
        assert w_down.shape == (Hd, F) and F2 == 2 * F
        T = tokens
        self.T, self.Hd, self.F = T, Hd, F
        self.rht, self.signs, self.seed, self.lr = (1 if rht else 0), int(rht_signs) & 0xFFFF, int(sr_seed), float(lr)
        self.it = 0
        bf = lambda *s: torch.empty(s, dtype=torch.bfloat16, device=dev)
        u8 = lambda *s: torch.empty(s, dtype=torch.uint8, device=dev)
        f32 = lambda: torch.empty(1, dtype=torch.float32, device=dev)
        self.w32 = {"W_gu": w_gu.detach().float().contiguous().clone(),
                    "W_down": w_down.detach().float().contiguous().clone()}
        self.wbf = {k: bf(*v.shape) for k, v in self.w32.items()}
        self.wamax = {k: f32() for k in self.w32}
        self.q = {}
        for name, (R, C) in (("X", (T, Hd)), ("W_gu", (F2, Hd)), ("H", (T, F)), ("W_down", (Hd, F)),
                             ("dY_down", (T, Hd)), ("dY_gu", (T, F2))):
            self.q[name] = dict(rc=u8(R, C // 2), rs=u8(R, C // 16), ra=f32(),
                                cc=u8(C, R // 2), cs=u8(C, R // 16), ca=f32())
        # a weight's 16x16 quantization runs under the amax its last update
        # produced; both orientations share it, and the GEMMs read it from here
        for k in self.w32:
            self.q[k]["ra"] = self.q[k]["ca"] = self.wamax[k]
        self.act = dict(Y_gu=bf(T, F2), H=bf(T, F), Y_down=bf(T, Hd), dH=bf(T, F),
                        dY_gu=bf(T, F2), dX=bf(T, Hd))
        self.grad = {"W_gu": bf(F2, Hd), "W_down": bf(Hd, F)}
        # B operands taken pre-expanded to FP16 (see bx_pays): (tensor, side) -> buffer
        self.xb = {}
        for name, b, side, N, K in (("FPROP_gu", "W_gu", "r", F2, Hd), ("FPROP_down", "W_down", "r", Hd, F),
                                    ("DGRAD_down", "W_down", "c", F, Hd), ("DGRAD_gu", "W_gu", "c", Hd, F2)):
            if bx_pays(N, K):
                self.xb[(b, side)] = torch.empty((N, K), dtype=torch.float16, device=dev)
        self.flops = 2.0 * 3 * (T * F2 * Hd + T * Hd * F)
        # the BF16 working copies and their amaxes: an update with a zero gradient
        for k in self.w32:
            self.grad[k].zero_()
            self._update(k, 0.0)

    # -- single launches -------------------------------------------------------------
    def _stream(self):
        return ctypes.c_void_p(torch.cuda.current_stream(self.dev).cuda_stream)

    def _ok(self, what, st):
        if st != 0:
            raise RuntimeError(f"{what}: {status_string(st)}")

    def _quant(self, name, x, rnd, rht, offset):
        b, (R, C) = self.q[name], x.shape
        self._ok("quantize_transpose " + name, self.lib.quantize_transpose(
            _p(x), R, C, NV, 1, rnd, self.seed, offset, rht, self.signs, _p(b["rc"]), _p(b["rs"]),
            _p(b["ra"]), _p(b["cc"]), _p(b["cs"]), _p(b["ca"]), self._stream()))

    def _quant_amax(self, name, x, block_rows, rnd, rht, offset, amax_row, amax_col):
        b, (R, C) = self.q[name], x.shape
        self._ok("quantize_transpose_amax " + name, self.lib.quantize_transpose_amax(
            _p(x), R, C, block_rows, rnd, self.seed, offset, rht, self.signs, _p(amax_row),
            _p(amax_col), _p(b["rc"]), _p(b["rs"]), _p(b["cc"]), _p(b["cs"]), self._stream()))

    def _expand(self, name):
        for (b, side), out in self.xb.items():
            if b == name:
                q, (R, C) = self.q[b], out.shape
                self._ok("nvfp4_expand " + b, self.lib.nvfp4_expand(
                    _p(q[side + "c"]), _p(q[side + "s"]), R, C, _p(out), self._stream()))

    def _gemm(self, what, a, ao, b, bo, c, M, N, K):
        qa, qb = self.q[a], self.q[b]
        if (b, bo) in self.xb:
            self._ok("bs_gemm_nvfp4_bx " + what, self.lib.bs_gemm_nvfp4_bx(
                M, N, K, _p(qa[ao + "c"]), _p(qa[ao + "s"]), _p(qa[ao + "a"]), _p(self.xb[(b, bo)]),
                _p(qb[bo + "a"]), _p(c), N, self._stream()))
            return
        self._ok("bs_gemm " + what, self.lib.bs_gemm(
            NV, M, N, K, _p(qa[ao + "c"]), _p(qa[ao + "s"]), _p(qa[ao + "a"]), _p(qb[bo + "c"]),
            _p(qb[bo + "s"]), _p(qb[bo + "a"]), _p(c), N, self._stream()))

    def _update(self, name, lr):
        w = self.w32[name]
        self._ok("master_weight_update " + name, self.lib.master_weight_update(
            _p(w), _p(self.grad[name]), w.numel(), ctypes.c_float(lr), _p(self.wbf[name]),
            _p(self.wamax[name]), self._stream()))

    # -- the step --------------------------------------------------------------------
    def forward(self, x):
        T, Hd, F = self.T, self.Hd, self.F
        if not (x.shape == (T, Hd) and x.dtype == torch.bfloat16 and x.is_contiguous()
                and x.device == self.dev):
            raise ValueError(f"x must be a contiguous bfloat16 [{T}, {Hd}] tensor on {self.dev}")
        self._quant("X", x, RNE, self.rht, 0)
        wa = self.wamax["W_gu"]
        self._quant_amax("W_gu", self.wbf["W_gu"], 16, RNE, 0, 0, wa, wa)
        self._expand("W_gu")
        self._gemm("FPROP_gu", "X", "r", "W_gu", "r", self.act["Y_gu"], T, 2 * F, Hd)
        H, qh = self.act["H"], self.q["H"]
        self._ok("swiglu_amax", self.lib.swiglu_amax(
            _p(self.act["Y_gu"]), T, F, self.rht, self.signs, _p(H), _p(qh["ra"]), _p(qh["ca"]),
            self._stream()))
        self._quant_amax("H", H, 1, RNE, self.rht, 0, qh["ra"], qh["ca"])
        wa = self.wamax["W_down"]
        self._quant_amax("W_down", self.wbf["W_down"], 16, RNE, 0, 0, wa, wa)
        self._expand("W_down")
        self._gemm("FPROP_down", "H", "r", "W_down", "r", self.act["Y_down"], T, Hd, F)
        return self.act["Y_down"]

    def backward(self, dy_down):
        T, Hd, F = self.T, self.Hd, self.F
        if not (dy_down.shape == (T, Hd) and dy_down.dtype == torch.bfloat16 and dy_down.is_contiguous()
                and dy_down.device == self.dev):
            raise ValueError(f"dy_down must be a contiguous bfloat16 [{T}, {Hd}] tensor on {self.dev}")
        off = 2 * self.it
        self._quant("dY_down", dy_down, SR, self.rht, off)
        self._gemm("DGRAD_down", "dY_down", "r", "W_down", "c", self.act["dH"], T, F, Hd)
        self._gemm("WGRAD_down", "dY_down", "c", "H", "c", self.grad["W_down"], Hd, F, T)
        dY, qd = self.act["dY_gu"], self.q["dY_gu"]
        self._ok("swiglu_backward_amax", self.lib.swiglu_backward_amax(
            _p(self.act["Y_gu"]), _p(self.act["dH"]), T, F, self.rht, self.signs, _p(dY),
            _p(qd["ra"]), _p(qd["ca"]), self._stream()))
        self._quant_amax("dY_gu", dY, 1, SR, self.rht, off + 1, qd["ra"], qd["ca"])
        self._gemm("DGRAD_gu", "dY_gu", "r", "W_gu", "c", self.act["dX"], T, Hd, 2 * F)
        self._gemm("WGRAD_gu", "dY_gu", "c", "X", "c", self.grad["W_gu"], 2 * F, Hd, T)
        return self.act["dX"]

    def update(self):
        for k in ("W_gu", "W_down"):
            self._update(k, self.lr)
        self.it += 1

    def step(self, x, dy_down):
        """Forward, backward and the master-weight update; returns (Y_down, dX)."""
        y = self.forward(x)
        dx = self.backward(dy_down)
        self.update()
        return y, dx
