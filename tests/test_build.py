"""Properties of the generated gfx950 code that the kernels' correctness
rests on, checked on the CPU by compiling the sources (hipcc cross-compiles
without a GPU)."""
import os
import re
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "bit_weight_quantized_amd", "csrc")


@pytest.mark.slow
def test_lds_copy_asm_owns_m0(tmp_path):
    """The global -> LDS copies of the GEMM kernels are inline asm that load
    m0 themselves; the compiler does not preserve m0 across them, so no
    compiler-generated instruction in that file may use m0."""
    from bit_weight_quantized_amd import build
    hipcc = build.HIPCC
    if not (os.path.exists(hipcc) or shutil.which(hipcc)):
        pytest.skip("hipcc not available")
    out = tmp_path / "gemm.s"
    cmd = [hipcc, *[f for f in build.COMMON if f not in ("-fPIC", "-Wall")], "-x", "hip",
           "--cuda-device-only", "-S", os.path.join(CSRC, "qmm_gemm.hip"), "-o", str(out)]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-2000:]
    inside, blocks, copies, bad, pending = False, 0, 0, [], None
    for line in out.read_text().splitlines():
        code = line.split(";")[0].strip()
        if "ASMSTART" in line:
            inside, blocks, pending = True, blocks + 1, "start"
            continue
        if inside and pending == "load":
            copies += 1
        if "ASMEND" in line:
            inside = False
            continue
        if not code:
            continue
        if inside:
            # inside a copy: m0 is written first, then the LDS-destination load;
            # any other asm block (the fp16 weight conversion) leaves m0 alone
            if pending == "start":
                pending = "load" if code.startswith("s_mov_b32 m0,") else "other"
                if pending == "other":
                    assert not re.search(r"\bm0\b", code) and " lds" not in code, line
            elif pending == "load":
                assert re.match(r"buffer_load_dword(x4)?\b.*\blds$", code), line
                pending = None
            elif pending == "other":
                assert not re.search(r"\bm0\b", code), line
        elif re.search(r"\bm0\b", code):
            bad.append(line)
    assert copies > 0, "no LDS copies found: the check would be vacuous"
    assert not bad, bad[:10]
