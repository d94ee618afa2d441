"""C-ABI checks that need no GPU: libbsq.so loads, exports exactly the entry
points include/bsq.h declares, and rejects invalid arguments before touching
the device (argument validation returns without any HIP call)."""

import ctypes
import os
import re

import pytest

import fp8_quantized_gemm_amd as bsq

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "bsq.h")

pytestmark = pytest.mark.skipif(not os.path.exists(bsq.LIB_PATH),
                                reason="libbsq.so not built (run __graft_entry__.build())")


def declared_functions():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return set(re.findall(r"^\s*(?:const\s+)?\w+\s*\*?\s*(\w+)\s*\(", src, flags=re.M))


def test_header_declares_the_entry_points():
    assert declared_functions() == set(bsq.ABI_SYMBOLS)


def test_library_exports_every_declared_symbol():
    L = ctypes.CDLL(bsq.LIB_PATH)
    for name in declared_functions():
        assert hasattr(L, name), name


def test_status_strings():
    for st, word in ((0, "BSQ_OK"), (1, "EINVAL"), (2, "EUNSUPPORTED"), (3, "EHIP")):
        assert word in bsq.status_string(st)
    assert "UNKNOWN" in bsq.status_string(99)


FAKE = 0x100000   # a 16-byte aligned non-null address that is never dereferenced


def _nv(**kw):
    a = dict(x=FAKE, rows=32, cols=32, block_rows=1, rnd=0, seed=0, offset=0, rht=0, signs=0,
             amax_in=None, codes=FAKE, scales=FAKE, amax_out=FAKE)
    a.update(kw)
    return bsq.lib().nvfp4_quantize(a["x"], a["rows"], a["cols"], a["block_rows"], a["rnd"],
                                    a["seed"], a["offset"], a["rht"], a["signs"], a["amax_in"],
                                    a["codes"], a["scales"], a["amax_out"], None)


def test_nvfp4_quantize_argument_errors():
    assert _nv(cols=24) == bsq.BSQ_EINVAL                 # cols % 16
    assert _nv(rows=-1) == bsq.BSQ_EINVAL
    assert _nv(block_rows=4) == bsq.BSQ_EINVAL
    assert _nv(block_rows=16, rows=24) == bsq.BSQ_EINVAL  # 2D needs rows % 16
    assert _nv(amax_out=None) == bsq.BSQ_EINVAL           # no amax source
    assert _nv(x=None) == bsq.BSQ_EINVAL
    assert _nv(codes=FAKE + 4) == bsq.BSQ_EINVAL          # misaligned
    assert _nv(rnd=7) == bsq.BSQ_EINVAL
    assert _nv(block_rows=16, rnd=1) == bsq.BSQ_EUNSUPPORTED
    assert _nv(block_rows=16, rht=1) == bsq.BSQ_EUNSUPPORTED


def _mx(fmt=1, rows=32, cols=64, rnd=0, x=FAKE, codes=FAKE, scales=FAKE):
    return bsq.lib().mx_quantize(x, rows, cols, fmt, rnd, 0, 0, codes, scales, None)


def test_mx_quantize_argument_errors():
    assert _mx(cols=48) == bsq.BSQ_EINVAL
    assert _mx(fmt=0) == bsq.BSQ_EUNSUPPORTED
    assert _mx(fmt=5) == bsq.BSQ_EINVAL
    assert _mx(fmt=2, rnd=1) == bsq.BSQ_EUNSUPPORTED
    assert _mx(scales=None) == bsq.BSQ_EINVAL
    assert _mx(rows=0) == bsq.BSQ_OK                      # empty: nothing to launch


def _qt(fmt=0, rows=32, cols=32, block_rows=1, rnd=0, rht=0, row=True, col=True, x=FAKE):
    r = FAKE if row else None
    c = FAKE if col else None
    return bsq.lib().quantize_transpose(x, rows, cols, fmt, block_rows, rnd, 0, 0, rht, 0,
                                        r, r, r, c, c, c, None)


def test_quantize_transpose_argument_errors():
    assert _qt(rows=24) == bsq.BSQ_EINVAL                 # rows % 16
    assert _qt(fmt=1, rows=48) == bsq.BSQ_EINVAL          # MX needs rows % 32
    assert _qt(row=False, col=False) == bsq.BSQ_EINVAL
    assert _qt(fmt=1, rht=1) == bsq.BSQ_EUNSUPPORTED
    assert _qt(fmt=1, block_rows=16) == bsq.BSQ_EUNSUPPORTED
    assert _qt(fmt=2, rnd=1) == bsq.BSQ_EUNSUPPORTED
    assert _qt(block_rows=16, rnd=1) == bsq.BSQ_EUNSUPPORTED
    assert _qt(block_rows=16, rht=1) == bsq.BSQ_EUNSUPPORTED
    assert _qt(x=None) == bsq.BSQ_EINVAL
    assert _qt(cols=1 << 26, rht=1) == bsq.BSQ_EINVAL     # column RHT amax addressing limit
    L = bsq.lib()
    # partial triple: codes given, scales missing
    assert L.quantize_transpose(FAKE, 32, 32, 0, 1, 0, 0, 0, 0, 0, FAKE, None, FAKE,
                                None, None, None, None) == bsq.BSQ_EINVAL


def _fp8(rows=32, cols=32, x=FAKE, row=FAKE, col=FAKE, amax=FAKE):
    return bsq.lib().fp8_quantize_transpose(x, rows, cols, row, col, amax, None)


def test_fp8_quantize_transpose_argument_errors():
    assert _fp8(rows=24) == bsq.BSQ_EINVAL                # rows % 16
    assert _fp8(cols=40) == bsq.BSQ_EINVAL                # cols % 16
    assert _fp8(row=None, col=None) == bsq.BSQ_EINVAL     # no output
    assert _fp8(amax=None) == bsq.BSQ_EINVAL              # amax is required
    assert _fp8(amax=FAKE + 2) == bsq.BSQ_EINVAL          # misaligned amax
    assert _fp8(x=None) == bsq.BSQ_EINVAL
    assert _fp8(row=FAKE + 8) == bsq.BSQ_EINVAL           # misaligned codes
    assert _mx(fmt=3) == bsq.BSQ_EUNSUPPORTED             # not an MX format
    assert _qt(fmt=3) == bsq.BSQ_EUNSUPPORTED             # per-tensor FP8 has its own entry point


def _qta(rows=32, cols=32, block_rows=1, rnd=0, rht=0, ar=FAKE, ac=FAKE, cr=FAKE, sr=FAKE,
         cc=FAKE, sc=FAKE, x=FAKE):
    return bsq.lib().quantize_transpose_amax(x, rows, cols, block_rows, rnd, 0, 0, rht, 0, ar, ac,
                                             cr, sr, cc, sc, None)


def test_quantize_transpose_amax_argument_errors():
    assert _qta(rows=24) == bsq.BSQ_EINVAL                # rows % 16
    assert _qta(cols=8) == bsq.BSQ_EINVAL                 # cols % 16
    assert _qta(block_rows=2) == bsq.BSQ_EINVAL
    assert _qta(rnd=5) == bsq.BSQ_EINVAL
    assert _qta(cr=None, sr=None, cc=None, sc=None) == bsq.BSQ_EINVAL   # no output
    assert _qta(ar=None) == bsq.BSQ_EINVAL                # row outputs need amax_row
    assert _qta(ac=None) == bsq.BSQ_EINVAL                # col outputs need amax_col
    assert _qta(sr=None) == bsq.BSQ_EINVAL                # half of the row pair
    assert _qta(ac=FAKE + 2) == bsq.BSQ_EINVAL            # misaligned amax
    assert _qta(cc=FAKE + 8) == bsq.BSQ_EINVAL            # misaligned codes
    assert _qta(x=None) == bsq.BSQ_EINVAL
    assert _qta(block_rows=16, rnd=1) == bsq.BSQ_EUNSUPPORTED
    assert _qta(block_rows=16, rht=1) == bsq.BSQ_EUNSUPPORTED
    assert _qta(rows=0) == bsq.BSQ_OK                     # empty: nothing to launch
    # 16x16 tiles encode both sides under one amax: the same pointer for both
    assert _qta(block_rows=16, ac=FAKE + 0x1000) == bsq.BSQ_EINVAL


def _sw(rows=32, f=32, y=FAKE, h=FAKE + 0x100000, ar=None, ac=None, rht=0):
    return bsq.lib().swiglu_amax(y, rows, f, rht, 0, h, ar, ac, None)


def _swb(rows=32, f=32, y=FAKE, d=FAKE + 0x100000, out=FAKE + 0x200000, ar=None, ac=None):
    return bsq.lib().swiglu_backward_amax(y, d, rows, f, 0, 0, out, ar, ac, None)


def test_swiglu_argument_errors():
    assert _sw(rows=24) == bsq.BSQ_EINVAL                 # rows % 16
    assert _sw(f=40) == bsq.BSQ_EINVAL                    # f % 16
    assert _sw(f=1 << 25) == bsq.BSQ_EINVAL               # 16 rows of y per buffer resource
    assert _sw(y=None) == bsq.BSQ_EINVAL
    assert _sw(h=None) == bsq.BSQ_EINVAL
    assert _sw(h=FAKE + 8) == bsq.BSQ_EINVAL              # misaligned
    assert _sw(h=FAKE + 32 * 32 * 2) == bsq.BSQ_EINVAL    # h overlaps the up half of y
    assert _sw(ar=FAKE + 2) == bsq.BSQ_EINVAL             # misaligned amax
    assert _sw(rows=0) == bsq.BSQ_OK and _sw(f=0) == bsq.BSQ_OK
    assert _swb(d=None) == bsq.BSQ_EINVAL
    assert _swb(d=FAKE + 8) == bsq.BSQ_EINVAL
    assert _swb(out=FAKE + 0x100000 + 16) == bsq.BSQ_EINVAL   # out overlaps d_h
    assert _swb(out=FAKE) == bsq.BSQ_EINVAL               # out overlaps y
    assert _swb(rows=16, f=24) == bsq.BSQ_EINVAL
    assert _swb(rows=0, d=None) == bsq.BSQ_OK


def test_master_weight_update_argument_errors():
    L = bsq.lib()
    u = lambda n=64, w=FAKE, g=FAKE + 0x100000, wb=FAKE + 0x200000, a=None: L.master_weight_update(
        w, g, n, 0.1, wb, a, None)
    assert u(n=12) == bsq.BSQ_EINVAL                      # n % 8
    assert u(n=-8) == bsq.BSQ_EINVAL
    assert u(w=None) == bsq.BSQ_EINVAL and u(g=None) == bsq.BSQ_EINVAL and u(wb=None) == bsq.BSQ_EINVAL
    assert u(g=FAKE + 8) == bsq.BSQ_EINVAL                # misaligned
    assert u(wb=FAKE + 64) == bsq.BSQ_EINVAL              # copy overlaps w32
    assert u(a=FAKE + 2) == bsq.BSQ_EINVAL                # misaligned amax
    assert u(n=0) == bsq.BSQ_OK


def test_expand_and_gemm_bx_argument_errors():
    L = bsq.lib()
    assert L.nvfp4_expand(FAKE, FAKE, 16, 24, FAKE, None) == bsq.BSQ_EINVAL       # cols % 16
    assert L.nvfp4_expand(FAKE + 4, FAKE, 16, 32, FAKE, None) == bsq.BSQ_EINVAL   # codes 8-byte aligned
    assert L.nvfp4_expand(FAKE, FAKE, 16, 32, FAKE + 8, None) == bsq.BSQ_EINVAL   # out 16-byte aligned
    assert L.nvfp4_expand(None, FAKE, 16, 32, FAKE, None) == bsq.BSQ_EINVAL
    assert L.nvfp4_expand(None, None, 0, 32, None, None) == bsq.BSQ_OK
    g = lambda M=64, N=64, K=256, a=FAKE, bx=FAKE, amax=FAKE, c=FAKE, ldc=64: L.bs_gemm_nvfp4_bx(
        M, N, K, a, FAKE, amax, bx, amax, c, ldc, None)
    assert g(K=96) == bsq.BSQ_EUNSUPPORTED                 # K % 128
    assert g(bx=FAKE + 8) == bsq.BSQ_EUNSUPPORTED          # B not 16-byte aligned
    assert g(a=None) == bsq.BSQ_EINVAL and g(bx=None) == bsq.BSQ_EINVAL and g(amax=None) == bsq.BSQ_EINVAL
    assert g(ldc=32) == bsq.BSQ_EINVAL
    assert g(M=0) == bsq.BSQ_OK


@pytest.mark.parametrize("entry", ["bs_gemm", "bs_gemm_noalloc"])
def test_bs_gemm_argument_errors(entry):
    L = bsq.lib()
    fn = getattr(L, entry)
    g = lambda fmt=0, M=16, N=16, K=32, ldc=16, a=FAKE, amax=FAKE, c=FAKE: fn(
        fmt, M, N, K, a, FAKE, amax, FAKE, FAKE, amax, c, ldc, None)
    assert g(K=24) == bsq.BSQ_EINVAL                      # NVFP4 K % 16
    assert g(fmt=1, K=48) == bsq.BSQ_EINVAL               # MX K % 32
    assert g(ldc=8) == bsq.BSQ_EINVAL                     # ldc < N
    assert g(a=None) == bsq.BSQ_EINVAL
    assert g(amax=None) == bsq.BSQ_EINVAL                 # NVFP4 needs both amax
    assert g(c=None) == bsq.BSQ_EINVAL
    assert g(fmt=9) == bsq.BSQ_EINVAL
    assert g(M=0) == bsq.BSQ_OK and g(N=0) == bsq.BSQ_OK  # empty output: nothing to launch
    # per-tensor FP8: scales may be NULL, both amaxes are required
    f = lambda K=64, amax=FAKE, sc=None: fn(3, 16, 16, K, FAKE, sc, amax, FAKE, sc, amax,
                                            FAKE, 16, None)
    assert f(K=48) == bsq.BSQ_EINVAL                      # K % 32
    assert f(amax=None) == bsq.BSQ_EINVAL
    assert fn(1, 16, 16, 64, FAKE, None, None, FAKE, None, None, FAKE, 16, None) == bsq.BSQ_EINVAL


def test_ceiling_library_loads_and_checks_arguments():
    """The route-ceiling measurement kernels live in their own library."""
    path = os.path.join(os.path.dirname(bsq.LIB_PATH), "libbsq_ceiling.so")
    L = ctypes.CDLL(path)
    L.bsq_route_ceiling.argtypes = [ctypes.c_int, ctypes.c_void_p, ctypes.c_int, ctypes.c_int, ctypes.c_void_p]
    L.bsq_route_ceiling.restype = ctypes.c_int
    assert L.bsq_route_ceiling(6, FAKE, 1, 1, None) == -1        # no such mode
    assert L.bsq_route_ceiling(0, None, 1, 1, None) == -1        # no sink
    assert L.bsq_route_ceiling(1, FAKE, 1, 0, None) == -1        # no workgroups
    assert not hasattr(bsq.lib(), "bsq_route_ceiling")           # not part of the product ABI


def test_binding_raises_without_library(monkeypatch):
    monkeypatch.setattr(bsq, "_lib", None)
    monkeypatch.setattr(bsq, "LIB_PATH", "/nonexistent/libbsq.so")
    with pytest.raises(RuntimeError):
        bsq.lib()


def test_binding_rejects_host_tensors():
    """Host tensors never reach the library (it would dereference their
    addresses on the GPU)."""
    import torch
    cpu = torch.zeros(16, 8, dtype=torch.uint8)
    with pytest.raises(ValueError):
        bsq.bs_gemm("nvfp4", cpu, cpu, cpu, cpu, K=16)
    with pytest.raises(ValueError):
        bsq.nvfp4_expand(cpu, cpu)
    with pytest.raises(ValueError):
        bsq.quantize_transpose(torch.zeros(16, 16, dtype=torch.bfloat16))
    from fp8_quantized_gemm_amd.mlp import MLPLayer
    with pytest.raises(ValueError):
        MLPLayer(torch.zeros(32, 16), torch.zeros(16, 16), 16)


def test_binding_checks_operand_shapes_before_any_launch():
    """Wrong operand widths, dtypes or output shapes raise ValueError in the
    binding (the C ABI sees raw pointers and cannot check buffer sizes); the
    checks run before the device check, so host tensors exercise them."""
    import torch
    u8 = lambda *s: torch.zeros(s, dtype=torch.uint8)
    f32 = torch.zeros(1, dtype=torch.float32)
    M, N, K = 32, 48, 64
    a, sa, b, sb = u8(M, K // 2), u8(M, K // 16), u8(N, K // 2), u8(N, K // 16)
    with pytest.raises(ValueError, match="B codes"):          # K wider than B's codes
        bsq.bs_gemm("nvfp4", a, sa, u8(N, K // 4), sb, f32, f32, K=K)
    with pytest.raises(ValueError, match="A codes"):          # explicit K beyond the codes
        bsq.bs_gemm("nvfp4", a, sa, b, sb, f32, f32, K=2 * K)
    with pytest.raises(ValueError, match="A scales"):         # scales narrower than K / 16
        bsq.bs_gemm("nvfp4", a, u8(M, K // 32), b, sb, f32, f32)
    with pytest.raises(ValueError, match="B scales"):         # MX scales are per 32
        bsq.bs_gemm("mxfp4", a, u8(M, K // 32), b, sb)
    with pytest.raises(ValueError, match="codes must be"):    # codes of the wrong dtype
        bsq.bs_gemm("nvfp4", a.float(), sa, b, sb, f32, f32, K=K)
    with pytest.raises(ValueError, match="amax"):             # NVFP4 needs both amaxes
        bsq.bs_gemm("nvfp4", a, sa, b, sb, f32, None)
    with pytest.raises(ValueError, match="amax"):             # amax of the wrong dtype
        bsq.bs_gemm("nvfp4", a, sa, b, sb, f32, torch.zeros(1, dtype=torch.float64))
    with pytest.raises(ValueError, match="out"):              # out with fewer rows than M
        bsq.bs_gemm("nvfp4", a, sa, b, sb, f32, f32, out=torch.zeros(M - 1, N, dtype=torch.bfloat16))
    with pytest.raises(ValueError, match="out"):              # out not bf16
        bsq.bs_gemm("nvfp4", a, sa, b, sb, f32, f32, out=torch.zeros(M, N, dtype=torch.float16))
    with pytest.raises(ValueError, match="A codes"):          # fp8 codes: one byte per element
        bsq.bs_gemm("fp8", a, None, u8(N, K), None, f32, f32, K=K)
    with pytest.raises(ValueError, match="unknown format"):
        bsq.bs_gemm("nvfp8", a, sa, b, sb, f32, f32)
    with pytest.raises(ValueError, match="expand scales"):
        bsq.nvfp4_expand(b, u8(N, K // 32))
    with pytest.raises(ValueError, match="out"):              # expansion output is fp16 [N, K]
        bsq.nvfp4_expand(b, sb, out=torch.zeros(N, K, dtype=torch.bfloat16))
    bx = torch.zeros(N, K, dtype=torch.float16)
    with pytest.raises(ValueError, match="b_x"):
        bsq.bs_gemm_nvfp4_bx(a, sa, f32, bx.bfloat16(), f32)
    with pytest.raises(ValueError, match="A codes"):          # A narrower than B's K
        bsq.bs_gemm_nvfp4_bx(u8(M, K // 4), sa, f32, bx, f32)
    with pytest.raises(ValueError, match="out"):
        bsq.bs_gemm_nvfp4_bx(a, sa, f32, bx, f32, out=torch.zeros(M, N + 1, dtype=torch.bfloat16))
    with pytest.raises(ValueError, match="CUDA"):             # right shapes, host memory
        bsq.bs_gemm("nvfp4", a, sa, b, sb, f32, f32)


def test_element_counts_beyond_2_48_are_rejected():
    """rows * cols (n, M * K, N * K, M * ldc) above 2^48 returns BSQ_EINVAL before
    any size-dependent arithmetic can overflow."""
    L, big = bsq.lib(), 1 << 40
    assert _nv(rows=big, cols=1 << 16) == bsq.BSQ_EINVAL
    assert _mx(rows=big, cols=1 << 16) == bsq.BSQ_EINVAL
    assert _qt(rows=big, cols=1 << 16) == bsq.BSQ_EINVAL
    assert _qt(fmt=1, rows=big, cols=1 << 16) == bsq.BSQ_EINVAL
    assert _fp8(rows=big, cols=1 << 16) == bsq.BSQ_EINVAL
    assert _qta(rows=big, cols=1 << 16) == bsq.BSQ_EINVAL
    assert _sw(rows=big, f=1 << 10) == bsq.BSQ_EINVAL
    assert L.master_weight_update(FAKE, FAKE + 0x100000, 1 << 49, ctypes.c_float(0.1),
                                  FAKE + 0x200000, None, None) == bsq.BSQ_EINVAL
    assert L.nvfp4_expand(FAKE, FAKE, big, 1 << 16, FAKE, None) == bsq.BSQ_EINVAL
    for M, N, K, ldc in ((1 << 20, 16, 1 << 29, 16), (16, 1 << 20, 1 << 29, 1 << 20),
                         (1 << 20, 16, 256, 1 << 29)):
        assert L.bs_gemm(0, M, N, K, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, ldc, None) == bsq.BSQ_EINVAL
        assert L.bs_gemm(1, M, N, K, FAKE, FAKE, None, FAKE, FAKE, None, FAKE, ldc, None) == bsq.BSQ_EINVAL
        assert L.bs_gemm_nvfp4_bx(M, N, K, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, ldc, None) == bsq.BSQ_EINVAL
