"""Static checks of the gfx950 assembly of the GEMMs whose MFMAs are inline
assembly: the register-expansion NVFP4 GEMM and the four-wave MX GEMM.

Their MFMAs are inline assembly (so that every accumulator tile keeps fixed
registers), and the compiler's hazard recognizer does not see their operand
timing.  The kernel's correctness then rests on the code the compiler emits
around them, which these checks read from a fresh `hipcc -S` of the source:

* no scratch (spill) instruction touches an accumulator register: a spill
  right after an MFMA reads its result before the MFMA has written it;
* an accumulator read (v_accvgpr_read) comes at least 18 wait states after
  the MFMA that last wrote that register (an 8-pass MFMA result needs 11);
* an accumulator write (v_accvgpr_write) comes at least 4 wait states before
  an MFMA that reads it as the C operand (2 are required);
* a VALU write of an A or B fragment register comes at least 2 wait states
  before the MFMA that reads it.

Wait states are counted as issued instructions between the two, an s_nop N
counting N + 1.  The checker itself is pinned on small synthetic listings.
No GPU is needed; the test is skipped without hipcc.

The quantizer's stochastic FP4 packs are inline assembly too, for the same
reason (the byte of the destination word they write is kept fixed, the other
bytes tied through).  gfx950 needs one wait state between such a
byte-selected result and the next VALU instruction that reads the register
(the compiler inserts exactly one after its own builtin); the fifth rule
checks that every function of the quantizer source keeps it."""

import os
import re
import shutil
import subprocess
import tempfile

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "fp8_quantized_gemm_amd", "csrc")

_RANGE = re.compile(r"^([va])\[(\d+):(\d+)\]$")
_ONE = re.compile(r"^([va])(\d+)$")


def _regs(tok):
    """('v'|'a', register numbers) of an operand token, or None."""
    tok = tok.strip()
    m = _RANGE.match(tok)
    if m:
        return m.group(1), set(range(int(m.group(2)), int(m.group(3)) + 1))
    m = _ONE.match(tok)
    if m:
        return m.group(1), {int(m.group(2))}
    return None


def _instructions(lines):
    """(mnemonic, [operands]) of the instruction lines of one function."""
    out = []
    for line in lines:
        t = line.split(";")[0].strip()
        if not t or t.startswith(".") or t.endswith(":"):
            continue
        parts = t.split(None, 1)
        ops = [o.strip() for o in parts[1].split(",")] if len(parts) > 1 else []
        out.append((parts[0], ops))
    return out


def _weight(ins):
    mn, ops = ins
    if mn == "s_nop":
        return int(ops[0], 0) + 1
    return 1


def _overlap(a, b):
    return a is not None and b is not None and a[0] == b[0] and a[1] & b[1]


def hazards(lines, acc_read_ws=18, acc_write_ws=4, frag_ws=2):
    """Violations (index, text) of the four rules in one function's listing."""
    ins = _instructions(lines)
    bad = []
    for i, (mn, ops) in enumerate(ins):
        if mn.startswith("scratch_") and any(r and r[0] == "a" for r in map(_regs, ops)):
            bad.append((i, f"accumulator spill: {mn} {', '.join(ops)}"))
        if mn == "v_accvgpr_read_b32":
            src = _regs(ops[1])
            ws = 0
            for j in range(i - 1, -1, -1):
                pm, pops = ins[j]
                if pm.startswith("v_mfma") and _overlap(_regs(pops[0]), src):
                    bad.append((i, f"{mn} {ops[1]} {ws} wait states after {pm} {pops[0]}"))
                    break
                ws += _weight(ins[j])
                if ws >= acc_read_ws:
                    break
        if mn.startswith("v_mfma"):
            srcab = [_regs(ops[1]), _regs(ops[2])]
            srcc = _regs(ops[3])
            ws = 0
            for j in range(i - 1, -1, -1):
                pm, pops = ins[j]
                dst = _regs(pops[0]) if pops else None
                if pm == "v_accvgpr_write_b32" and _overlap(dst, srcc) and ws < acc_write_ws:
                    bad.append((i, f"{mn} reads {ops[3]} {ws} wait states after {pm} {pops[0]}"))
                if (pm.startswith("v_") and not pm.startswith("v_mfma") and not pm.startswith("v_accvgpr")
                        and any(_overlap(dst, s) for s in srcab) and ws < frag_ws):
                    bad.append((i, f"{mn} reads {ops[1]}/{ops[2]} {ws} wait states after {pm} {pops[0]}"))
                ws += _weight(ins[j])
                if ws >= max(acc_write_ws, frag_ws):
                    break
    return bad


_SR_PACK = re.compile(r"^v_cvt_scalef32_sr_pk_fp4_f32\s+(v\d+),.*op_sel:\[(\d),(\d),(\d),(\d)\]")


def _source_regs(tok):
    """Register operand of a source token, modifiers (neg, abs, sdwa and
    op_sel suffixes) stripped."""
    tok = tok.strip().split()[0] if tok.strip() else tok
    return _regs(tok.lstrip("-|").rstrip("|"))


def sr_pack_hazards(lines, ws_needed=1):
    """Violations (index, text) of the fifth rule: a VALU instruction reads
    the destination of a byte-selected stochastic FP4 pack (op_sel naming
    byte 1, 2 or 3) fewer than ws_needed wait states after it."""
    text = []
    for line in lines:
        t = line.split(";")[0].strip()
        if t and not t.startswith(".") and not t.endswith(":"):
            text.append(t)
    ins = _instructions(lines)
    bad = []
    for i, t in enumerate(text):
        m = _SR_PACK.match(t)
        if not m or (m.group(4) == "0" and m.group(5) == "0"):
            continue
        dst = _regs(m.group(1))
        ws = 0
        for j in range(i + 1, len(ins)):
            mn, ops = ins[j]
            if ws >= ws_needed:
                break
            if mn.startswith("v_"):
                # a later byte-selected pack also reads its own destination
                srcs = ops if _SR_PACK.match(text[j]) else ops[1:]
                if any(_overlap(_source_regs(o), dst) for o in srcs):
                    bad.append((j, f"{mn} reads {m.group(1)} {ws} wait states after a byte-selected SR pack"))
            ws += _weight(ins[j])
    return bad


def _functions(asm, name_part):
    """{symbol: body lines} of the functions whose symbol contains name_part."""
    funcs, cur = {}, None
    for line in asm.splitlines():
        m = re.match(r"^(_Z\w+):", line)
        if m:
            cur = m.group(1) if name_part in m.group(1) else None
            if cur:
                funcs[cur] = []
            continue
        if cur and line.strip().startswith(".Lfunc_end"):
            cur = None
            continue
        if cur:
            funcs[cur].append(line)
    return funcs


# ------------------------------------------------------------------ checker pins

def test_checker_flags_accumulator_spill():
    lines = ["\tv_mfma_f32_16x16x32_f16 a[4:7], v[0:3], v[4:7], a[4:7]",
             "\tscratch_store_dwordx4 off, a[4:7], off"]
    assert any("spill" in t for _, t in hazards(lines))


def test_checker_flags_early_accumulator_read():
    lines = ["\tv_mfma_f32_16x16x32_f16 a[4:7], v[0:3], v[4:7], a[4:7]", "\ts_nop 7",
             "\tv_accvgpr_read_b32 v9, a6"]
    assert len(hazards(lines)) == 1
    ok = lines[:2] + ["\ts_nop 7", "\ts_nop 7"] + lines[2:]
    assert hazards(ok) == []


def test_checker_flags_late_accumulator_init():
    lines = ["\tv_accvgpr_write_b32 a5, 0", "\tv_mov_b32 v40, v41",
             "\tv_mfma_f32_16x16x32_f16 a[4:7], v[0:3], v[8:11], a[4:7]"]
    assert len(hazards(lines)) == 1
    assert hazards(["\tv_accvgpr_write_b32 a5, 0", "\ts_nop 4"] + lines[2:]) == []


def test_checker_flags_fragment_written_just_before_mfma():
    lines = ["\tv_pk_mul_f16 v3, v20, v21", "\tv_mfma_f32_16x16x32_f16 a[4:7], v[0:3], v[8:11], a[4:7]"]
    assert len(hazards(lines)) == 1
    spaced = [lines[0], "\tv_mfma_f32_16x16x32_f16 a[8:11], v[12:15], v[8:11], a[8:11]", "\ts_nop 0", lines[1]]
    assert hazards(spaced) == []
    # a write of a register the MFMA does not read is no hazard
    assert hazards(["\tv_pk_mul_f16 v30, v20, v21", lines[1]]) == []


def test_checker_flags_sr_pack_read_without_wait_state():
    pack = "\tv_cvt_scalef32_sr_pk_fp4_f32 v5, v[0:1], v2, 1.0 op_sel:[0,0,1,0]"
    read = "\tv_and_b32_e32 v6, 0xf0f0f0f, v5"
    assert len(sr_pack_hazards([pack, read])) == 1
    assert sr_pack_hazards([pack, "\ts_nop 0", read]) == []
    # another instruction in between is the wait state
    assert sr_pack_hazards([pack, "\tv_lshlrev_b32_e32 v9, 16, v8", read]) == []
    # the next pack into the same word reads it (tied bytes)
    tied = "\tv_cvt_scalef32_sr_pk_fp4_f32 v5, v[10:11], v3, 1.0 op_sel:[0,0,0,1]"
    assert len(sr_pack_hazards([pack, tied])) == 1
    # byte 0 needs no wait state, and a write of another register is no hazard
    byte0 = "\tv_cvt_scalef32_sr_pk_fp4_f32 v5, v[0:1], v2, 1.0"
    assert sr_pack_hazards([byte0, read]) == []
    assert sr_pack_hazards([pack, "\tv_and_b32_e32 v6, 0xf0f0f0f, v7"]) == []
    # source modifiers and sdwa suffixes do not hide a read
    assert len(sr_pack_hazards([pack, "\tv_lshlrev_b32_sdwa v1, v2, v5 dst_sel:DWORD src1_sel:BYTE_1"])) == 1


# ------------------------------------------------------------------ the kernel

def _compile(src):
    hipcc = os.environ.get("HIPCC") or shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    if not os.path.exists(hipcc):
        pytest.skip("hipcc not available")
    from fp8_quantized_gemm_amd import _build
    with tempfile.TemporaryDirectory() as d:
        out = os.path.join(d, "k.s")
        cmd = [hipcc] + _build.FLAGS + ["-x", "hip", "--cuda-device-only", "-S", os.path.join(CSRC, src),
                                        "-o", out]
        r = subprocess.run(cmd, capture_output=True, text=True)
        assert r.returncode == 0, r.stderr[-2000:]
        return open(out).read()


@pytest.fixture(scope="module")
def rx_asm():
    return _compile("bsq_gemm_nvfp4_rx.hip")


@pytest.fixture(scope="module")
def mx_asm():
    return _compile("bsq_gemm_mx_rx.hip")


def test_rx_kernels_present(rx_asm):
    funcs = _functions(rx_asm, "k_gemm_nvfp4_rx")
    names = " ".join(funcs)
    assert "ILb0E" in names and "ILb1E" in names, names      # full-tile and split instantiations
    for body in funcs.values():
        assert len(_instructions(body)) > 0


def _check_kernels(funcs, skip=()):
    report = []
    for name, body in funcs.items():
        if any(k in name for k in skip):
            continue
        n_mfma = sum(1 for mn, _ in _instructions(body) if mn.startswith("v_mfma"))
        assert n_mfma > 0, name
        report += [f"{name}: {t}" for _, t in hazards(body)]
    assert report == [], "\n".join(report[:20])


def test_rx_mfma_operand_timing(rx_asm):
    _check_kernels(_functions(rx_asm, "k_gemm_nvfp4_rx"), skip=("join",))


def test_mx_mfma_operand_timing(mx_asm):
    funcs = _functions(mx_asm, "k_gemm_mx_rx")
    assert len(funcs) == 3, list(funcs)                       # MXFP4, MXFP8, per-tensor FP8
    _check_kernels(funcs)


@pytest.fixture(scope="module")
def quant_asm():
    return _compile("bsq_quantize.hip")


def test_sr_pack_wait_states(quant_asm):
    funcs = _functions(quant_asm, "bsq")
    packs, report = 0, []
    for name, body in funcs.items():
        packs += sum(1 for line in body if "v_cvt_scalef32_sr_pk_fp4_f32" in line and "op_sel" in line)
        report += [f"{name}: {t}" for _, t in sr_pack_hazards(body)]
    assert packs > 0, "no byte-selected SR pack found"
    assert report == [], "\n".join(report[:20])
