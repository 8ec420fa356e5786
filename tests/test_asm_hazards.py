"""The saddr direct-to-LDS loads are inline asm, so the compiler's hazard
recognizer does not protect them: a vector memory instruction that reads an
SGPR written by a VALU instruction (for instance v_readlane reloading a
spilled base address) needs 5 wait states in between on gfx9, or it reads a
stale address.  This compiles the kernels that use the saddr form to gfx950
assembly and checks every such load (host only; needs hipcc)."""
import os
import re
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "state_space_sequence_02_amd", "csrc")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")


def _sgprs(tok):
    m = re.match(r"s\[(\d+):(\d+)\]$", tok)
    if m:
        return set(range(int(m.group(1)), int(m.group(2)) + 1))
    m = re.match(r"s(\d+)$", tok)
    return {int(m.group(1))} if m else set()


def _hazards(asm):
    """(load, writer, wait states) for every saddr LDS load whose base SGPRs a
    VALU instruction wrote fewer than 5 wait states before it."""
    ins = []
    for line in asm.splitlines():
        line = line.split(";")[0].strip()
        if line and not line.endswith(":") and not line.startswith("."):
            ins.append(line)
    out = []
    for k, line in enumerate(ins):
        if not line.startswith("global_load_lds"):
            continue
        ops = [o.strip() for o in line.split(None, 1)[1].split(",")]
        base = _sgprs(ops[1]) if len(ops) > 1 else set()
        if not base:
            continue
        ws = 0
        for j in range(k - 1, max(-1, k - 16), -1):
            if ws >= 5:
                break
            p = ins[j]
            op = p.split()[0]
            if op == "s_nop":
                ws += int(p.split()[1], 0) + 1
                continue
            if op.startswith("v_") and " " in p:
                dst = p.split(None, 1)[1].split(",")[0].strip()
                if _sgprs(dst) & base:
                    out.append((line, p, ws))
            ws += 1
    return out


def test_hazard_scan_finds_a_planted_case():
    asm = "v_readlane_b32 s6, v10, 0\nv_readlane_b32 s7, v10, 1\nglobal_load_lds_dwordx4 v2, s[6:7]\n"
    assert len(_hazards(asm)) == 2
    ok = "v_readlane_b32 s6, v10, 0\nv_readlane_b32 s7, v10, 1\ns_nop 4\nglobal_load_lds_dwordx4 v2, s[6:7]\n"
    assert _hazards(ok) == []


@pytest.mark.skipif(shutil.which(HIPCC) is None and not os.path.exists(HIPCC),
                    reason="hipcc not available")
def test_saddr_lds_loads_have_their_wait_states(tmp_path):
    srcs = [f for f in sorted(os.listdir(CSRC)) if f.endswith(".hip")
            and "global_load_lds_dwordx4 %0, %1" in open(os.path.join(CSRC, f)).read()]
    assert srcs, "no source uses the saddr form"
    for f in srcs:
        out = tmp_path / (f + ".s")
        subprocess.run([HIPCC, "--offload-arch=gfx950", "-O3", "-std=c++17", "-Xclang",
                        "-target-feature", "-Xclang", "-packed-fp32-ops",
                        f"-I{os.path.join(ROOT, 'include')}", f"-I{CSRC}", "--cuda-device-only",
                        "-S", os.path.join(CSRC, f), "-o", str(out)],
                       check=True, capture_output=True)
        asm = out.read_text()
        assert "global_load_lds_dwordx4" in asm
        bad = _hazards(asm)
        assert not bad, (f, bad[:4])
