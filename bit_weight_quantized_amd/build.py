"""Compile the HIP sources into in-tree shared libraries for gfx950.

    python -m bit_weight_quantized_amd.build          # libqmm.so and synth's libsynth.so

hipcc cross-compiles without a GPU.  Objects go to _build/ (not committed);
each library lands next to the Python code that loads it.
"""
from __future__ import annotations

import os
import shutil
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
PKG = os.path.join(ROOT, "bit_weight_quantized_amd")
CSRC = os.path.join(PKG, "csrc")
BUILD = os.path.join(ROOT, "_build")
ARCH = os.environ.get("QMM_OFFLOAD_ARCH", "gfx950")

HIPCC = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"

# packed-fp32 instructions are kept out of every kernel (they are generated
# from ordinary float code otherwise); the host pass warns that it does not
# know the feature, which is harmless.
COMMON = ["-O3", "-fPIC", "-std=c++17", f"--offload-arch={ARCH}", "-Wall",
          "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
          "-ffp-contract=off"]

LIBS = {
    "qmm": dict(sources=["qmm_pack.hip", "qmm_gemv.hip", "qmm_gemm.hip", "qmm_stream.hip", "qmm_route.hip", "qmm_combine.hip", "qmm_gemv_i8.hip", "qmm_skinny.hip", "qmm_mrow.hip", "qmm_noalloc.hip", "qmm_api.cpp"],
                srcdir=CSRC, out=os.path.join(PKG, "libqmm.so")),
    "synth": dict(sources=["synth_gen.hip"], srcdir=os.path.join(ROOT, "synth", "csrc"),
                  out=os.path.join(ROOT, "synth", "libsynth.so")),
}


def _compile(src: str, obj: str) -> None:
    lang = ["-x", "hip"] if src.endswith(".hip") else []
    cmd = [HIPCC, *COMMON, *lang, "-c", src, "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    noise = "is not a recognized feature for this target"
    err = "\n".join(l for l in (r.stderr or "").splitlines() if noise not in l)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{err}")
    if err.strip():
        sys.stderr.write(err + "\n")


def build(names=("qmm", "synth"), jobs: int = 4) -> dict:
    os.makedirs(BUILD, exist_ok=True)
    out = {}
    for name in names:
        spec = LIBS[name]
        srcs = [os.path.join(spec["srcdir"], s) for s in spec["sources"]]
        objs = [os.path.join(BUILD, f"{name}_{os.path.basename(s)}.o") for s in srcs]
        with ThreadPoolExecutor(max_workers=jobs) as ex:
            list(ex.map(lambda p: _compile(*p), zip(srcs, objs)))
        tmp = spec["out"] + ".tmp"
        cmd = [HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp]
        r = subprocess.run(cmd, capture_output=True, text=True)
        if r.returncode != 0:
            raise RuntimeError(f"link failed for {name}:\n{r.stderr}")
        os.replace(tmp, spec["out"])
        out[name] = spec["out"]
    return out


if __name__ == "__main__":
    for k, v in build().items():
        print(k, v)
