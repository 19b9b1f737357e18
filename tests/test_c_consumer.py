"""include/dta.h is a C header and libdta.so a C library: a C11 program
built with gcc against them links, and every argument check it calls returns
its documented status before any HIP call (runs without a GPU). The same
holds for the library built by the package's CMakeLists.txt."""

import ctypes
import os
import shutil
import subprocess

import pytest

from diffusion_transformer_attention_flash_amd import _lib

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
PKG = os.path.dirname(_lib.LIB_PATH)

C_SOURCE = r"""
#include "dta.h"
#include <stdio.h>
#include <string.h>

static int fails = 0;
#define CHECK(x) do { if (!(x)) { printf("FAIL %s\n", #x); ++fails; } } while (0)

int main(void) {
    void *g = (void *)0x10000;              /* aligned, never dereferenced */
    void *odd = (void *)0x10008;            /* 8-byte aligned only */
    float *gf = (float *)g;
    hipStream_t s = (hipStream_t)0;
    int lens[2] = {3, 4}, zero[2] = {0, 0};
    /* every call below fails its argument checks, so none reaches HIP */
    CHECK(dta_ws_bytes() >= 16384);
    CHECK(strlen(dta_status_str(DTA_EINVAL)) > 0);
    CHECK(attn_fwd(NULL, g, g, g, gf, 1, 1, 1, 1, 128, 0.1f, s) == DTA_EINVAL);
    CHECK(attn_fwd(g, g, g, g, gf, 1, 1, 1, 0, 128, 0.1f, s) == DTA_EINVAL);
    CHECK(attn_fwd(g, g, g, g, gf, 1, 1, 1, 1, 96, 0.1f, s) == DTA_EUNSUPPORTED);
    CHECK(attn_fwd(odd, g, g, g, gf, 1, 1, 1, 1, 128, 0.1f, s) == DTA_EALIGN);
    CHECK(attn_fwd_accum(g, g, g, g, NULL, 1, 1, 1, 1, 128, 0.1f, s) == DTA_EINVAL);
    CHECK(attn_merge(g, gf, 0, g, gf, 1, 1, 1, 128, s) == DTA_EINVAL);
    CHECK(attn_merge_into(g, gf, g, NULL, 1, 1, 1, 128, s) == DTA_EINVAL);
    CHECK(residual_diff(g, g, 0, gf, g, s) == DTA_EINVAL);
    CHECK(residual_diff(g, g, 8, gf, NULL, s) == DTA_EINVAL);
    CHECK(residual_diff_noalloc(g, g, (int64_t)1 << 62, gf, s) == DTA_EINVAL);
    CHECK(fbcache_step(g, g, 8, 0.1f, g, g, 0, gf, (int *)g, g, s) == DTA_EINVAL);
    CHECK(fp8_quant_per_tensor(g, 0, g, gf, g, s) == DTA_EINVAL);
    CHECK(attn_fwd_fp8(g, g, g, NULL, g, gf, 1, 1, 1, 1, 128, 0.1f, s) == DTA_EINVAL);
    CHECK(fp8_quant_rows_pow2(g, 1, 7, g, g, s) == DTA_EINVAL);
    CHECK(fp8_quant_rows_pow2(odd, 1, 8, g, g, s) == DTA_EALIGN);
    CHECK(seq_concat(g, g, 0, lens, lens, 1, 1, 128, s) == DTA_EINVAL);
    CHECK(seq_concat(g, g, 2, lens, zero, 1, 1, 128, s) == DTA_EINVAL);   /* padded < lens */
    printf(fails ? "FAILED %d\n" : "ok\n", fails);
    return fails != 0;
}
"""


def _consumer(tmp_path, lib_dir):
    """Builds the C program against dta.h and lib_dir/libdta.so and runs it."""
    gcc = shutil.which("gcc")
    if gcc is None:
        pytest.skip("gcc not available")
    src = tmp_path / "consumer.c"
    src.write_text(C_SOURCE)
    exe = tmp_path / "consumer"
    build = subprocess.run(
        [gcc, "-std=c11", "-Wall", "-Werror", "-D__HIP_PLATFORM_AMD__",
         "-I", os.path.join(ROOT, "include"), "-I", "/opt/rocm/include", str(src),
         "-L", lib_dir, "-ldta", "-Wl,-rpath," + lib_dir, "-o", str(exe)],
        capture_output=True, text=True)
    assert build.returncode == 0, build.stderr
    run = subprocess.run([str(exe)], capture_output=True, text=True, timeout=60)
    assert run.returncode == 0 and run.stdout.strip() == "ok", run.stdout + run.stderr


def test_a_c_program_builds_against_the_header_and_library(tmp_path):
    if not os.path.exists(_lib.LIB_PATH):
        pytest.fail("libdta.so is not built")
    _consumer(tmp_path, PKG)


def test_the_cmake_build_gives_the_same_c_library(tmp_path):
    """The package's CMakeLists.txt builds libdta.so for gfx950 with the same
    device flags as build.py; it exports every function include/dta.h
    declares, and the C program above runs against it."""
    cmake, ninja = shutil.which("cmake"), shutil.which("ninja")
    if cmake is None or ninja is None:
        pytest.skip("cmake or ninja not available")
    bdir = tmp_path / "build"
    cfg = subprocess.run([cmake, "-S", os.path.join(ROOT, "diffusion_transformer_attention_flash_amd"),
                          "-B", str(bdir), "-G", "Ninja"], capture_output=True, text=True)
    assert cfg.returncode == 0, cfg.stdout + cfg.stderr
    flags = (bdir / "build.ninja").read_text()
    assert "--offload-arch=gfx950" in flags and "--offload-arch=gfx9" not in flags.replace(
        "--offload-arch=gfx950", "")
    assert "-Xclang -target-feature -Xclang -packed-fp32-ops" in flags
    bld = subprocess.run([cmake, "--build", str(bdir), "-j", "6"], capture_output=True, text=True)
    assert bld.returncode == 0, bld.stdout[-4000:] + bld.stderr[-4000:]
    so = bdir / "libdta.so"
    lib = ctypes.CDLL(str(so))
    for name in _lib.SIGNATURES:
        assert hasattr(lib, name), name
    lib.dta_ws_bytes.restype = ctypes.c_size_t
    assert lib.dta_ws_bytes() == _lib.lib().dta_ws_bytes()
    _consumer(tmp_path, str(bdir))
