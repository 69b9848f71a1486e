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
