"""Builds librelpos.so in-tree with hipcc for gfx950 (python -m relative_position_bias_relpos_amd.build)."""

import concurrent.futures
import os
import shutil
import subprocess
import sys
import tempfile

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(HERE, "librelpos.so")
SOURCES = ["relpos_api.hip", "relpos_build.hip", "relpos_attn_fwd.hip", "relpos_attn16.hip",
           "relpos_attn12.hip"]

# Packed-fp32 VALU forms are kept out of the generated code on purpose.
HIP_FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    # MFMA accumulators in ordinary VGPRs (no AGPR copies around each MFMA)
    "-mllvm", "-amdgpu-mfma-vgpr-form",
    "-Wno-unused-command-line-argument",
    # the 12-wave kernel's LDS-direct load helper clobbers M0 on purpose
    "-Wno-inline-asm",
]


def _hipcc():
    exe = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    if not os.path.exists(exe):
        raise RuntimeError("hipcc not found; librelpos needs ROCm's hipcc")
    return exe


def build(verbose=False):
    """Compile every HIP source and link librelpos.so next to this file."""
    hipcc = _hipcc()
    with tempfile.TemporaryDirectory(prefix="relpos_build_") as tmp:
        objs = [os.path.join(tmp, s.replace(".hip", ".o")) for s in SOURCES]

        def compile_one(pair):
            src, obj = pair
            cmd = [hipcc, *HIP_FLAGS, "-I", INCLUDE, "-c", os.path.join(CSRC, src), "-o", obj]
            r = subprocess.run(cmd, capture_output=True, text=True)
            if r.returncode != 0:
                raise RuntimeError(f"hipcc failed on {src}:\n{r.stderr}")
            if verbose and r.stderr.strip():
                print(r.stderr, file=sys.stderr)

        with concurrent.futures.ThreadPoolExecutor(len(SOURCES)) as ex:
            list(ex.map(compile_one, zip(SOURCES, objs)))
        out_tmp = os.path.join(tmp, "librelpos.so")
        cmd = [hipcc, "--offload-arch=gfx950", "-shared", "-fPIC", *objs, "-o", out_tmp]
        r = subprocess.run(cmd, capture_output=True, text=True)
        if r.returncode != 0:
            raise RuntimeError(f"link failed:\n{r.stderr}")
        shutil.copyfile(out_tmp, LIB + ".tmp")
        os.replace(LIB + ".tmp", LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
