"""Build libqlora.so (HIP for gfx950) in-tree.

    python -m bit_nf4_quantized_double_amd.build

Compiles every source under csrc/ with hipcc and links one shared library
next to this file.  Always recompiles (no staleness tracking).
"""

from __future__ import annotations

import os
import shutil
import subprocess
import sys
import tempfile
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(PKG, "csrc")
LIB = os.path.join(PKG, "libqlora.so")
# The same sources with every raw global access range checked (skipped and
# counted when outside its buffer; qlora_debug_oob_count reads the count).
LIB_CHECKED = os.path.join(PKG, "libqlora_checked.so")
SOURCES = ["nf4_table.cpp", "codec.hip", "gemm.hip", "skinny.hip", "lora.hip", "adapter.hip", "merge.hip", "abi.hip"]

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"
FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC",
    # no packed fp32 instructions (v_pk_*_f32) anywhere in device code
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    # IEEE fp32 division / sqrt (the quantizer's x = w / absmax must be exact)
    "-fhip-fp32-correctly-rounded-divide-sqrt",
    "-Wall", "-Wno-unused-function",
]
# The codec and the merge produce bit-exact results: no multiply-add is fused
# behind the source's back there (the few fused ones are written explicitly).
# Elsewhere products accumulate on the matrix cores and contraction is free.
CONTRACT = {"codec.hip": "-ffp-contract=off", "merge.hip": "-ffp-contract=off"}


def _compile(src: str, obj: str, checked: bool = False) -> None:
    cmd = [HIPCC, *FLAGS, CONTRACT.get(src, "-ffp-contract=fast")]
    if checked:
        cmd.append("-DQLORA_BOUNDS_CHECK")
    if src.endswith(".cpp"):
        cmd += ["-x", "hip"]
    cmd += ["-c", os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{r.stdout}\n{r.stderr}")
    noise = [ln for ln in r.stderr.splitlines() if "packed-fp32-ops" not in ln and ln.strip()]
    if noise:
        sys.stderr.write(f"[{src}]\n" + "\n".join(noise) + "\n")


def build(verbose: bool = True) -> str:
    """Build libqlora.so and its bounds-checked twin libqlora_checked.so."""
    if not shutil.which(HIPCC) and not os.path.exists(HIPCC):
        raise RuntimeError("hipcc not found; cannot build libqlora.so")
    with tempfile.TemporaryDirectory(prefix="qlora_build_") as tmp:
        jobs = []
        for checked, lib in ((False, LIB), (True, LIB_CHECKED)):
            tag = "c_" if checked else ""
            objs = [os.path.join(tmp, tag + s.rsplit(".", 1)[0] + ".o") for s in SOURCES]
            jobs.append((lib, objs, [(s, o, checked) for s, o in zip(SOURCES, objs)]))
        with ThreadPoolExecutor(max_workers=8) as ex:
            list(ex.map(lambda t: _compile(*t), [t for _, _, ts in jobs for t in ts]))
        for lib, objs, _ in jobs:
            out_tmp = lib + ".tmp"
            cmd = [HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", out_tmp, *objs]
            r = subprocess.run(cmd, capture_output=True, text=True)
            if r.returncode != 0:
                raise RuntimeError(f"link failed:\n{r.stdout}\n{r.stderr}")
            os.replace(out_tmp, lib)
            if verbose:
                print(f"built {lib}")
    return LIB


if __name__ == "__main__":
    build()
