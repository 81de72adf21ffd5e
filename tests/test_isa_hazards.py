"""The LDS-direct loads (global_load_lds_*) are written in inline assembly,
which the compiler's hazard recognizer does not inspect.  The CDNA ISA wants
5 wait states between a VALU instruction that writes an SGPR (v_readfirstlane,
v_readlane restoring a spilled SGPR, v_cmp with an SGPR destination) and a
VMEM instruction that reads it, and 1 between an SALU write of M0 and an
LDS-DMA load.  Without them the load can take the SGPR's previous value as
its base address.  This test compiles every kernel source to gfx950 assembly
and checks each LDS-direct load's base SGPRs and M0 against the instructions
in front of it.
"""
import os
import re
import shutil
import subprocess
from concurrent.futures import ThreadPoolExecutor

import pytest

CSRC = os.path.join(os.path.dirname(__file__), "..", "sparse_long_context_piattn_amd", "csrc")
HIPCC = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
SOURCES = ["fwd_split.hip", "fwd_resid.hip", "decode.hip", "bwd_band.hip", "proj.hip"]

pytestmark = pytest.mark.skipif(not os.path.exists(HIPCC), reason="needs hipcc")


def _sregs(tok):
    m = re.match(r"s\[(\d+):(\d+)\]$", tok)
    if m:
        return set(range(int(m.group(1)), int(m.group(2)) + 1))
    m = re.match(r"s(\d+)$", tok)
    return {int(m.group(1))} if m else set()


def _wait_states(instr):
    """Wait states an instruction provides (s_nop N gives N + 1)."""
    m = re.match(r"s_nop\s+(\w+)", instr)
    return int(m.group(1), 0) + 1 if m else 1


def scan(asm_text):
    """[(kernel, problem, instruction)] for the LDS-direct loads in asm_text."""
    problems, fn, ins = [], None, []
    for raw in asm_text.splitlines():
        line = raw.split(";")[0].strip()
        m = re.match(r"^(_Z\w+):", raw.strip())
        if m:
            fn = m.group(1)
            continue
        if not line or line.startswith(".") or line.endswith(":"):
            continue
        ins.append((fn, line))
    for i, (fn, line) in enumerate(ins):
        if not line.startswith("global_load_lds"):
            continue
        base = _sregs(line.split(None, 1)[1].split(",")[1].split()[0])   # "s[2:3]" before any cache bits
        waited = 0
        for j in range(i - 1, max(-1, i - 8), -1):
            prev = ins[j][1]
            if prev.startswith("v_"):
                dst = prev.split(None, 1)[1].split(",")[0].strip()
                if _sregs(dst) & base and waited < 5:
                    problems.append((fn, "VALU-written base SGPR after %d wait states" % waited, line))
                    break
            if prev.startswith(("s_", "v_")) and re.match(r"s_\w+\s+m0,", prev) and waited < 1:
                problems.append((fn, "M0 written by the previous instruction", line))
            waited += _wait_states(prev)
            if waited >= 5:
                break
    return problems


def _compile(src, tmp):
    out = os.path.join(tmp, src + ".s")
    cmd = [HIPCC, "--offload-arch=gfx950", "-O3", "-std=c++17", "-Xclang", "-target-feature", "-Xclang",
           "-packed-fp32-ops", "--cuda-device-only", "-S", os.path.join(CSRC, src), "-o", out]
    subprocess.run(cmd, check=True, capture_output=True)
    with open(out) as f:
        return f.read()


def test_scanner_flags_a_short_distance():
    bad = "\n".join(["_Zk:", "v_readfirstlane_b32 s2, v8", "s_cselect_b32 m0, s8, -1",
                     "global_load_lds_dwordx4 v7, s[2:3]"])
    kinds = {p[1].split(" after")[0] for p in scan(bad)}
    assert "VALU-written base SGPR" in kinds and "M0 written by the previous instruction" in kinds
    good = "\n".join(["_Zk:", "v_readfirstlane_b32 s2, v8", "s_cselect_b32 m0, s8, -1", "s_nop 4",
                      "global_load_lds_dwordx4 v7, s[2:3]"])
    assert scan(good) == []
    bad_sc1 = "\n".join(["_Zk:", "v_readfirstlane_b32 s3, v8", "global_load_lds_dwordx4 v7, s[2:3] sc1"])
    assert scan(bad_sc1)


def test_lds_direct_loads_have_their_wait_states(tmp_path):
    with ThreadPoolExecutor(max_workers=4) as ex:
        texts = list(ex.map(lambda s: _compile(s, str(tmp_path)), SOURCES))
    n_loads = sum(t.count("global_load_lds") for t in texts)
    assert n_loads > 100
    problems = [p for t in texts for p in scan(t)]
    assert problems == [], problems[:5]
