"""Device code checks that need no GPU: the gfx950 assembly the compiler
writes for the MFMA kernels, read for hazards that the compiler cannot see.

The direct memory-to-LDS loads are written as inline assembly (so the
compiler does not wait for them before every LDS read).  The compiler's
hazard checks do not look inside an asm statement, so the statement itself
has to provide the wait states its operands need: 5 when a vector
instruction (a v_readlane restoring a spilled SGPR, say) has just written
the base address SGPRs or M0.  Without them the load read a stale base.
"""
import os
import re
import subprocess

import pytest

from expert_routing_quantized_amd import build as B

CSRC = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))),
                    "expert_routing_quantized_amd", "csrc")


@pytest.fixture(scope="module")
def mfma_asm(tmp_path_factory):
    out = tmp_path_factory.mktemp("asm") / "mfma.s"
    flags = [f for f in B.COMMON if f not in ("-shared", "-fPIC")]
    subprocess.run([B.hipcc()] + flags + ["--cuda-device-only", "-S", os.path.join(CSRC, "mfma.hip"),
                                          "-o", str(out)], check=True, capture_output=True)
    return out.read_text().splitlines()


def instructions(lines):
    """(index, text) of the instruction lines (no labels, directives or comments)."""
    out = []
    for i, l in enumerate(lines):
        t = l.split(";")[0].strip()
        if not t or t.endswith(":") or t.startswith("."):
            continue
        out.append((i, t))
    return out


def test_direct_lds_loads_follow_five_wait_states(mfma_asm):
    ins = instructions(mfma_asm)
    loads = [k for k, (_, t) in enumerate(ins) if t.startswith("global_load_lds_dwordx4")]
    assert loads, "no direct-to-LDS loads in the MFMA kernels"
    for k in loads:
        prev = ins[k - 1][1]
        m = re.match(r"s_nop\s+(\d+)", prev)
        assert m and int(m.group(1)) >= 4, f"line {ins[k][0] + 1}: '{prev}' before '{ins[k][1]}'"


def test_big_tile_router_kernel_does_not_spill(mfma_asm):
    text = "\n".join(mfma_asm)
    for name in ("router_gemm_big_kernelIfE", "router_gemm_big_kernelIdE"):
        start = text.index("_ZN3moe22" + name)
        info = text[text.index("; Kernel info", start):]
        scratch = int(re.search(r"; ScratchSize: (\d+)", info).group(1))
        assert scratch == 0, f"{name}: {scratch} bytes of scratch"


# Every inline-asm memory instruction of the library whose address or M0
# comes from scalar registers: the direct-to-LDS loads above and the scalar
# loads that fetch a kernel's argument lines at its start.  A vector
# instruction that writes one of those SGPRs (v_readlane / v_readfirstlane
# restoring a spill, a v_cmp writing a mask) must be at least 5 wait states
# earlier (s_nop N counts N + 1), whatever the compiler put around the asm.
ASM_SOURCES = ("mfma.hip", "experts.hip", "screen_window.hip")
SGPR = re.compile(r"^s(\d+)$|^s\[(\d+):(\d+)\]$")


def _sgprs(tok):
    m = SGPR.match(tok.strip())
    if not m:
        return set()
    if m.group(1) is not None:
        return {int(m.group(1))}
    return set(range(int(m.group(2)), int(m.group(3)) + 1))


@pytest.fixture(scope="module")
def library_asm(tmp_path_factory):
    d = tmp_path_factory.mktemp("asm_all")
    flags = [f for f in B.COMMON if f not in ("-shared", "-fPIC")]
    out = {}
    for src in ASM_SOURCES:
        path = d / (src + ".s")
        subprocess.run([B.hipcc()] + flags + ["--cuda-device-only", "-S", os.path.join(CSRC, src), "-o", str(path)],
                       check=True, capture_output=True)
        out[src] = path.read_text().splitlines()
    return out


def _asm_memory_ops(lines):
    """(line index, instruction) of the memory instructions inside inline-asm blocks."""
    ops, inside = [], False
    for i, l in enumerate(lines):
        t = l.split(";")[0].strip()
        if ";;#ASMSTART" in l:
            inside = True
        elif ";;#ASMEND" in l:
            inside = False
        elif inside and re.match(r"(global_|buffer_|s_load|s_buffer_load|flat_)", t):
            ops.append((i, t))
    return ops


def test_inline_asm_memory_ops_have_scalar_operand_wait_states(library_asm):
    checked = 0
    for src, lines in library_asm.items():
        for i, t in _asm_memory_ops(lines):
            ops = [o.strip() for o in t.split(None, 1)[1].split(",")] if " " in t else []
            if t.startswith(("s_load", "s_buffer_load")):
                ops = ops[1:]                              # the destination is not read
            regs = set()
            for o in ops:
                regs |= _sgprs(o)
            if t.startswith("global_load_lds"):
                regs.add("m0")
            assert regs, f"{src}:{i + 1}: no scalar operand found in '{t}'"
            states = 0
            j = i - 1
            while j >= 0 and states < 5:
                p = lines[j].split(";")[0].strip()
                j -= 1
                if not p or p.endswith(":") or p.startswith("."):
                    continue
                m = re.match(r"s_nop\s+(\d+)", p)
                if m:
                    states += int(m.group(1)) + 1
                    continue
                if p.startswith("v_"):
                    dst = p.split(None, 1)[1].split(",")[0] if " " in p else ""
                    hit = _sgprs(dst) & regs or (dst.strip() == "m0" and "m0" in regs)
                    assert not hit, f"{src}:{i + 1}: '{p}' writes an operand of '{t}' {states} wait states before it"
                states += 1
            checked += 1
    assert checked >= 8, f"only {checked} inline-asm memory instructions found"
