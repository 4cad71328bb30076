"""Static checks of the gfx950 assembly of the kernels whose MFMAs and LDS fragment reads are
inline asm (k_lm_head_w4, k_gemm_w4).

The compiler takes an asm statement's outputs as written when the statement issues, and it does
not know that an asm MFMA's accumulators arrive many cycles later.  So it may
  (1) copy, spill or otherwise touch a register that an asm ds_read_b128 is still filling
      (before the s_waitcnt lgkmcnt(0) that names it), or
  (2) read an accumulator (a copy, a spill, the epilogue) before the wait states the MFMA
      result needs.
Both give wrong values on some runs and right ones on others, so they are checked here on the
assembly itself: the device code is compiled exactly as the library build does, each kernel's
body is scanned in layout order, and every instruction is checked against the registers of
pending fragment reads and of MFMAs issued within the last 48 issue slots (s_nop N counts
N + 1; every other instruction one).  No GPU is needed.
"""
import os
import re
import shutil
import subprocess

import pytest

from block_diffusion_sparse_amd import build as B

CSRC = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))),
                    "block_diffusion_sparse_amd", "csrc")
MFMA_WAIT_SLOTS = 48


_CACHE = {}


def _assembly(src, tmp_path_factory):
    if src in _CACHE:
        return _CACHE[src]
    hipcc = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    if not os.path.exists(hipcc):
        pytest.skip("hipcc not available")
    out = os.path.join(str(tmp_path_factory.mktemp("isa")), os.path.basename(src) + ".s")
    flags = [f for f in B.HIPCC_FLAGS if f != "-fPIC"]
    res = subprocess.run([hipcc, *flags, "--cuda-device-only", "-S", "-o", out,
                          os.path.join(CSRC, src)], capture_output=True, text=True)
    assert res.returncode == 0, res.stderr[-2000:]
    _CACHE[src] = open(out).read()
    return _CACHE[src]


def _kernel_body(asm, mangled_prefix):
    m = re.search(r"^(" + re.escape(mangled_prefix) + r"\S*):", asm, re.M)
    assert m, f"kernel {mangled_prefix} not found"
    end = asm.index(".Lfunc_end", m.start())
    return asm[m.start():end].split("\n")


def _regs(text):
    out = set()
    for kind, a, b in re.findall(r"\b([va])\[(\d+):(\d+)\]", text):
        out |= {f"{kind}{i}" for i in range(int(a), int(b) + 1)}
    for kind, a in re.findall(r"\b([va])(\d+)\b", text):
        out.add(f"{kind}{a}")
    return out


def scan(lines):
    """Findings of (1) and (2) over one kernel body, plus the block labels reached with
    fragment reads pending (a loop back edge that carries them to the loop's first wait)."""
    pending = {}       # register -> line of the ds_read_b128 filling it
    recent = []        # [registers written by an MFMA, issue slots left]
    touched, early, labels, scratch = [], [], [], 0
    for n, raw in enumerate(lines, 1):
        text = raw.split(";")[0].strip()
        if not text or text.startswith("."):
            if text.startswith(".LBB") and pending:
                labels.append(n)
            continue
        if text.endswith(":"):
            continue
        op = text.split()[0]
        args = text[len(op):]
        if op.startswith("scratch_"):
            scratch += 1
        if op == "s_waitcnt":
            if "lgkmcnt(0)" in args:
                pending = {}
            continue
        used = _regs(args)
        if op == "ds_read_b128":
            dst, src = args.split(",", 1)
            hit = _regs(src) & set(pending)
            if hit:
                touched.append((n, text))
            for r in _regs(dst):
                pending[r] = n
            slots = 1
        else:
            if used & set(pending):
                touched.append((n, text))
            slots = int(args.strip()) + 1 if op == "s_nop" else 1
        if op.startswith("v_mfma"):
            recent.append([_regs(args.split(",")[0]), MFMA_WAIT_SLOTS])
        else:
            for regs, _ in recent:
                if used & regs:
                    early.append((n, text))
                    break
        for item in recent:
            item[1] -= slots
        recent = [item for item in recent if item[1] > 0]
    return touched, early, labels, scratch


def test_scanner_flags_planted_hazards():
    """The scanner itself: a copy of a register still being filled, an accumulator read right
    after its MFMA, and the same sequences made safe by the waits."""
    bad = [
        "ds_read_b128 v[10:13], v2 offset:0",
        "v_mov_b64_e32 v[20:21], v[10:11]",
        "s_waitcnt lgkmcnt(0)",
        "v_mfma_f32_16x16x32_bf16 a[0:3], v[10:13], v[14:17], a[0:3]",
        "s_nop 3",
        "v_accvgpr_read_b32 v30, a2",
    ]
    touched, early, _, _ = scan(bad)
    assert [n for n, _ in touched] == [2]
    assert [n for n, _ in early] == [6]
    good = [
        "ds_read_b128 v[10:13], v2 offset:0",
        "s_waitcnt lgkmcnt(0)",
        "v_mov_b64_e32 v[20:21], v[10:11]",
        "v_mfma_f32_16x16x32_bf16 a[0:3], v[10:13], v[14:17], a[0:3]",
        "s_nop 15", "s_nop 15", "s_nop 15",
        "v_accvgpr_read_b32 v30, a2",
    ]
    touched, early, _, _ = scan(good)
    assert not touched and not early


def test_lm_head_kernel_has_no_fragment_or_accumulator_hazards(tmp_path_factory):
    lines = _kernel_body(_assembly("decode.hip", tmp_path_factory), "_ZN5epoch12k_lm_head_w4")
    touched, early, labels, scratch = scan(lines)
    assert not touched, touched[:5]
    assert not early, early[:5]
    # every step waits for its own fragment reads, so none is pending where code paths meet
    assert not labels, labels[:5]
    assert scratch == 0


@pytest.mark.parametrize("gateup", [True, False])
def test_dense_tile_kernel_has_no_fragment_or_accumulator_hazards(tmp_path_factory, gateup):
    asm = _assembly("experts.hip", tmp_path_factory)
    lines = _kernel_body(asm, "_ZN5epoch9k_gemm_w4ILb%dELb0EE" % int(gateup))
    touched, early, labels, scratch = scan(lines)
    assert not touched, touched[:5]
    assert not early, early[:5]
    # every chunk step waits for its fragment reads before the loop's back edge
    assert not labels, labels[:5]
    assert scratch == 0
