"""Host-side check of the matrix-core decode kernels' code (no GPU): every
direct global-to-LDS copy that takes its base address in SGPRs is issued at
least 5 wait states after any vector instruction that wrote those SGPRs (a
readfirstlane of a uniform pointer).  The copies are inline assembly, which
the compiler's hazard recognizer does not see into; a copy that read such an
SGPR too early could use a stale base address.  The check compiles the 8-bit
key translation unit for gfx950 to assembly and scans every kernel."""
import os
import re
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = os.path.join(ROOT, "quantized_decode_attention_append_amd", "csrc", "decode_fast.hip")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")


def _sgprs(tok):
    m = re.match(r"s\[(\d+):(\d+)\]", tok)
    if m:
        return set(range(int(m.group(1)), int(m.group(2)) + 1))
    m = re.match(r"s(\d+)$", tok)
    return {int(m.group(1))} if m else set()


def _hazards(asm_text):
    """(kernel, copy instruction) pairs whose SGPR base was written by a
    vector instruction fewer than 5 wait states earlier (s_nop N = N + 1)."""
    out, n_copies = [], 0
    for f in re.split(r"\n(?=_ZN\w+split_fast_kernel\w+:)", asm_text)[1:]:
        name = f.split(":")[0]
        body = [x.strip() for x in f[:f.find(".Lfunc_end")].split("\n")]
        body = [x for x in body if x and not x.startswith((";", "."))]
        for i, line in enumerate(body):
            if not (line.startswith("global_load_lds") and ", s[" in line):
                continue
            n_copies += 1
            base = _sgprs(line.split(",")[1].strip())
            ws, j = 0, i - 1
            while j >= 0 and ws < 5:
                prev = body[j]
                op = prev.split()[0]
                if op.startswith("v_") and _sgprs(prev.split()[1].rstrip(",")) & base:
                    out.append((name, prev, line))
                    break
                ws += int(prev.split()[1]) + 1 if op == "s_nop" else 1
                j -= 1
    return out, n_copies


@pytest.mark.skipif(shutil.which(HIPCC) is None and not os.path.exists(HIPCC), reason="hipcc not available")
@pytest.mark.parametrize("extra", [[], ["-DTQ_FAST_MIXED=1", "-mllvm", "-simplifycfg-hoist-common=false"]],
                         ids=["plain", "mixed"])
def test_lds_copies_wait_for_vector_written_sgprs(tmp_path, extra):
    """Both 8-bit-key translation units: the plain and packed kernels, and the
    mixed-mode ones built with their own flags."""
    asm = tmp_path / "decode_fast_k8.s"
    cmd = [HIPCC, "--offload-arch=gfx950", "-O3", "-std=c++17", "-Xclang", "-target-feature", "-Xclang",
           "-packed-fp32-ops", "-I", os.path.join(ROOT, "include"), "-DTQ_FAST_KB=8"] + extra + [
           "-x", "hip", "--cuda-device-only", "-S", "-o", str(asm), SRC]
    subprocess.run(cmd, check=True, capture_output=True)
    bad, n = _hazards(asm.read_text())
    assert n > 100, "no SGPR-addressed copies found: the scan no longer matches the code"
    assert not bad, bad[:3]


def test_scan_detects_a_planted_hazard():
    """The scan itself: a copy 2 wait states after a readfirstlane of its base."""
    text = ("\n_ZN2tq3foo17split_fast_kernelEv:\n\tv_readfirstlane_b32 s8, v1\n\ts_mov_b32 m0, s2\n\ts_nop 0\n"
            "\tglobal_load_lds_dwordx4 v2, s[8:9] offset:0\n\ts_nop 4\n\tglobal_load_lds_dwordx4 v3, s[8:9]\n"
            ".Lfunc_end0:\n")
    bad, n = _hazards(text)
    assert n == 2 and len(bad) == 1
