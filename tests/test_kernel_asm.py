"""Static checks of the generated gfx950 assembly (CPU; needs hipcc).

The inter-chunk kernel's bf16 path loads the next chunk's U tiles with inline
assembly global loads that the compiler does not track, and makes them usable
only after the step's explicit s_waitcnt (see kda_prefill.hip).  That is
sound only if the compiler never reads, copies or spills those registers
between the load and the wait.  Nothing in the source language can promise
that, so these tests read the assembly the build produces and fail if a
toolchain or register-pressure change ever breaks it:
  * every bf16 inter_kernel variant uses no scratch (no spills);
  * between each untracked load and the end of the step (the empty "settle"
    asm statements that mark the registers written), no instruction names a
    register the load writes;
  * an explicit counted wait (s_waitcnt vmcnt) lies between the last
    untracked load and the settle statements.
"""
import os
import re
import subprocess

import pytest

from gated_delta_rule_21_amd import build as B

SRC = os.path.join(B.CSRC, "kda_prefill.hip")


@pytest.fixture(scope="module")
def asm(tmp_path_factory):
    out = str(tmp_path_factory.mktemp("asm") / "kda_prefill.s")
    cmd = [B.HIPCC, *B.FLAGS, "--cuda-device-only", "-S", SRC, "-o", out]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr
    return open(out).read()


def kernels(asm_text, pattern):
    """{symbol: body} of every kernel whose symbol matches `pattern`."""
    out = {}
    for m in re.finditer(r"^(%s\w*):" % pattern, asm_text, flags=re.M):
        name = m.group(1)
        end = asm_text.find(".Lfunc_end", m.end())
        out[name] = asm_text[m.end():end]
    return out


def vregs(operand):
    """VGPR numbers named by an operand like v7 or v[10:13]."""
    m = re.fullmatch(r"v(\d+)", operand)
    if m:
        return {int(m.group(1))}
    m = re.fullmatch(r"v\[(\d+):(\d+)\]", operand)
    if m:
        return set(range(int(m.group(1)), int(m.group(2)) + 1))
    return set()


def named_vregs(line):
    regs = set()
    for tok in re.findall(r"v\[\d+:\d+\]|\bv\d+\b", line):
        regs |= vregs(tok)
    return regs


BF16_INTER = r"_ZN3kda12inter_kernelILi(32|64|128)ELb0ELi[012]E"


def untracked(lines):
    """Line indices of the untracked loads: a global load inside an inline-asm block."""
    return [i for i in range(1, len(lines) - 1)
            if re.search(r"global_load_dwordx[24] ", lines[i]) and "ASMSTART" in lines[i - 1]]


def test_bf16_inter_kernels_found(asm):
    # output, transition and gated-output modes at d = 32, 64, 128
    assert len(kernels(asm, BF16_INTER)) == 9


def test_bf16_inter_kernels_use_no_scratch(asm):
    for name in kernels(asm, BF16_INTER):
        m = re.search(r"\.set %s\.private_seg_size, (\d+)" % re.escape(name), asm)
        assert m is not None, name
        assert int(m.group(1)) == 0, (name, "spills to scratch")


def test_untracked_loads_are_untouched_until_the_wait(asm):
    for name, body in kernels(asm, BF16_INTER).items():
        lines = body.splitlines()
        loads = untracked(lines)
        # four U tiles per step; the gated mode also loads two pieces of g
        gate = "ELi2EE" in name
        assert len(loads) == (6 if gate else 4), (name, len(loads))
        # the settle statements: the first run of empty asm blocks after the loads
        settle = None
        for i in range(loads[-1], len(lines) - 1):
            if "ASMSTART" in lines[i] and "ASMEND" in lines[i + 1]:
                settle = i
                break
        assert settle is not None, name
        dest = set()
        for i in loads:
            dest |= vregs(lines[i].split()[1].rstrip(","))
        assert len(dest) == (16 if gate else 8), (name, dest)
        for i in range(loads[0], settle):
            if i in loads:
                continue
            hit = named_vregs(lines[i]) & dest
            assert not hit, (name, "line %d touches an untracked load's register before the wait" % i,
                             lines[i].strip())
        waits = [l for l in lines[loads[-1]:settle] if re.search(r"s_waitcnt vmcnt\(\d+\)", l)]
        assert waits, (name, "no explicit vmcnt wait before the settle statements")
