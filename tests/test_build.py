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


def device_asm(tmp_path, src):
    """The gfx950 assembly hipcc writes for one kernel source."""
    from bit_weight_quantized_amd import build
    hipcc = build.HIPCC
    if not (os.path.exists(hipcc) or shutil.which(hipcc)):
        pytest.skip("hipcc not available")
    out = tmp_path / (src + ".s")
    cmd = [hipcc, *[f for f in build.COMMON if f not in ("-fPIC", "-Wall")], "-x", "hip",
           "--cuda-device-only", "-S", os.path.join(CSRC, src), "-o", str(out)]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-2000:]
    return out


@pytest.mark.slow
@pytest.mark.parametrize("src", ["qmm_gemm.hip", "qmm_mrow.hip"])
def test_lds_copy_asm_owns_m0(tmp_path, src):
    """The global -> LDS copies of the GEMM and multi-row kernels are inline
    asm that load m0 themselves; the compiler does not preserve m0 across
    them, so no compiler-generated instruction in those files may use m0."""
    out = device_asm(tmp_path, src)
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


def _vgprs(op):
    m = re.fullmatch(r"v\[(\d+):(\d+)\]", op)
    if m:
        return set(range(int(m.group(1)), int(m.group(2)) + 1))
    m = re.fullmatch(r"v(\d+)", op)
    return {int(m.group(1))} if m else set()


@pytest.mark.slow
@pytest.mark.parametrize("src", ["qmm_gemm.hip", "qmm_skinny.hip", "qmm_mrow.hip"])
def test_inline_asm_results_reach_mfma_after_two_wait_states(tmp_path, src):
    """The compiler inserts the wait states a VALU result needs before an
    MFMA reads it only for instructions it generated: a VGPR written by an
    inline-asm block is invisible to its hazard check.  A product-of-codes
    operand read one instruction after the asm that built it gave wrong sums
    in a multi-row kernel build.  So every MFMA source register written by
    inline asm must be at least two wait states old (instructions issued in
    between, s_nop N counting N + 1), scanning each function in order."""
    out = device_asm(tmp_path, src)
    inside, clock, asm_def, bad, mfmas = False, 0, {}, [], 0
    for line in out.read_text().splitlines():
        code = line.split(";")[0].strip()
        if "ASMSTART" in line:
            inside = True
            continue
        if "ASMEND" in line:
            inside = False
            continue
        if not code or code.startswith(".") or code.endswith(":"):
            if code.endswith(":") and not code.startswith(".L"):
                asm_def = {}   # a new function
            continue
        ops = [o for o in re.split(r"[\s,]+", code) if o]
        clock += int(ops[1]) + 1 if ops[0] == "s_nop" and len(ops) > 1 and ops[1].isdigit() else 1
        if ops[0].startswith("v_mfma"):
            mfmas += 1
            for op in ops[2:5]:
                for r in _vgprs(op):
                    if r in asm_def and clock - asm_def[r] - 1 < 2:
                        bad.append(line.strip())
        if len(ops) > 1 and ops[0].startswith("v_"):
            for r in _vgprs(ops[1]):
                if inside:
                    asm_def[r] = clock
                else:
                    asm_def.pop(r, None)
    assert mfmas > 0, "no MFMAs found: the check would be vacuous"
    assert not bad, bad[:10]
