"""Build libdta.so -- the gfx950 HIP kernels and their C ABI -- in-tree.

    python -m diffusion_transformer_attention_flash_amd.build

Every source under csrc/ is compiled by hipcc for gfx950 only, with packed
fp32 VALU forms disabled, then linked into one shared library next to this
file. Always recompiles (a few seconds per source).
"""

import os
import shutil
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
BUILD_DIR = os.path.join(HERE, "_build")
LIB_PATH = os.path.join(HERE, "libdta.so")

SOURCES = ["attn_fwd.hip", "attn_fwd_fp8.hip", "merge.hip", "reduce.hip", "layout.hip"]

HIPCC_FLAGS = [
    "--offload-arch=gfx950",
    "-O3",
    "-std=c++17",
    "-fPIC",
    "-Wall",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
]


def _hipcc():
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (ROCm is required to build libdta.so)")


def _run(cmd):
    r = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    if r.returncode != 0:
        raise RuntimeError("build step failed:\n%s\n%s" % (" ".join(cmd), r.stdout))
    return r.stdout


# The same library with a workgroup barrier at every point where the attention
# kernels reuse LDS between phases (DTA_DEBUG_BARRIERS): its outputs must be
# bit-identical to libdta.so's, which the GPU tests check.
DEBUG_LIB_PATH = os.path.join(HERE, "libdta_debug.so")


def build(verbose=False, jobs=4, lib_path=LIB_PATH, build_dir=BUILD_DIR, extra_flags=(),
          link_flags=()):
    """Compile every csrc/*.hip source and link a shared library (libdta.so
    by default); returns its path."""
    hipcc = _hipcc()
    os.makedirs(build_dir, exist_ok=True)
    objs = []
    cmds = []
    for src in SOURCES:
        obj = os.path.join(build_dir, src.replace(".hip", ".o"))
        objs.append(obj)
        cmds.append([hipcc, *HIPCC_FLAGS, *extra_flags, "-c", os.path.join(CSRC, src), "-o", obj])
    with ThreadPoolExecutor(max_workers=max(1, int(jobs))) as ex:
        outs = list(ex.map(_run, cmds))
    tmp = lib_path + ".tmp"
    outs.append(_run([hipcc, "--offload-arch=gfx950", "-shared", "-fPIC", *link_flags, *objs,
                      "-o", tmp]))
    os.replace(tmp, lib_path)
    if verbose:
        for o in outs:
            if o.strip():
                print(o)
    return lib_path


def build_debug_barriers(verbose=False, jobs=4):
    """libdta_debug.so: DTA_DEBUG_BARRIERS builds of the same sources."""
    return build(verbose, jobs, DEBUG_LIB_PATH, os.path.join(HERE, "_build_debug"),
                 ("-DDTA_DEBUG_BARRIERS",))


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
    print(build_debug_barriers(verbose="-v" in sys.argv))
