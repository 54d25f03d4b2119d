"""Build ``libverify_attn.so`` (the C-ABI library) in-tree with hipcc for gfx950.

``python -m speculative_decoding_attention_amd.build`` or ``build()`` compiles
every source under ``csrc/`` and links them into the package directory.
"""
from __future__ import annotations

import os
import shutil
import subprocess
import sys
import tempfile

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB_NAME = "libverify_attn.so"
LIB_PATH = os.path.join(PKG, LIB_NAME)
ARCH = "gfx950"

# -packed-fp32-ops: keep the compiler from emitting packed fp32 VALU forms.
# kernarg preload: the leading kernel arguments of every kernel (up to 13
# SGPRs: the pointers and sizes the first memory round needs) arrive in SGPRs
# at wave launch.
COMMON = ["-O3", "-std=c++17", "-fPIC", "-fvisibility=hidden", "-Wall",
          "-I", INCLUDE, "-I", CSRC]
DEVICE = ["-x", "hip", "--offload-arch=" + ARCH,
          "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
          "-mllvm", "-amdgpu-kernarg-preload-count=10"]

SOURCES = ["va_kernels.hip", "va_aux.hip", "va_noalloc.hip", "va_plan.cpp", "va_api.cpp",
           "va_aux_api.cpp"]


def hipcc() -> str:
    for cand in (shutil.which("hipcc"), "/opt/rocm/bin/hipcc"):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found")


def build(verbose: bool = False, jobs: int = 4) -> str:
    cc = hipcc()
    tmp = tempfile.mkdtemp(prefix="va_build_")
    objs, procs = [], []
    try:
        for src in SOURCES:
            path = os.path.join(CSRC, src)
            obj = os.path.join(tmp, src + ".o")
            cmd = [cc] + COMMON + (DEVICE if src.endswith(".hip") else ["-x", "hip", "--offload-arch=" + ARCH])
            cmd += ["-c", path, "-o", obj]
            if verbose:
                print(" ".join(cmd), flush=True)
            procs.append((src, subprocess.Popen(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT)))
            objs.append(obj)
        failed = []
        for src, pr in procs:
            out, _ = pr.communicate()
            text = out.decode(errors="replace")
            # hipcc's host pass does not know the device feature flag: harmless
            lines = [l for l in text.splitlines() if "not a recognized feature" not in l]
            if lines and (verbose or pr.returncode != 0):
                print("\n".join(lines), file=sys.stderr)
            if pr.returncode != 0:
                failed.append(src)
        if failed:
            raise RuntimeError("hipcc failed for: " + ", ".join(failed))
        out_tmp = LIB_PATH + ".tmp%d" % os.getpid()
        cmd = [cc, "-shared", "-fPIC", "--offload-arch=" + ARCH, "-o", out_tmp] + objs
        subprocess.run(cmd, check=True)
        os.replace(out_tmp, LIB_PATH)
    finally:
        shutil.rmtree(tmp, ignore_errors=True)
    return LIB_PATH


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
