"""The C ABI's argument validation under AddressSanitizer (host code only,
no GPU): libdta is rebuilt with the sanitizer on its host side and
tests/test_abi.py runs against it in a child process with the sanitizer
runtime preloaded. Any out-of-bounds access or use-after-free in the
validation paths fails this test."""

import glob
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _asan_runtime():
    hits = sorted(glob.glob("/opt/rocm/llvm/lib/clang/*/lib/linux/libclang_rt.asan-x86_64.so"))
    return hits[-1] if hits else None


def test_abi_validation_under_host_asan(tmp_path):
    rt = _asan_runtime()
    if rt is None:
        pytest.skip("no clang AddressSanitizer runtime in this ROCm image")
    sys.path.insert(0, ROOT)
    from diffusion_transformer_attention_flash_amd import build
    lib = str(tmp_path / "libdta_asan.so")
    host_asan = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fno-omit-frame-pointer"]
    build.build(lib_path=lib, build_dir=str(tmp_path / "obj"), extra_flags=["-g"] + host_asan,
                link_flags=["-Xarch_host", "-fsanitize=address", "-shared-libasan"])
    code = ("import sys; sys.path.insert(0, %r); "
            "from diffusion_transformer_attention_flash_amd import _lib; _lib.LIB_PATH = %r; "
            "import pytest; sys.exit(pytest.main(['%s', '-q', '-m', 'not gpu', "
            "'-p', 'no:cacheprovider']))" % (ROOT, lib, os.path.join(ROOT, "tests", "test_abi.py")))
    env = dict(os.environ)
    env["LD_PRELOAD"] = " ".join(x for x in (rt, os.environ.get("LD_PRELOAD", "")) if x)
    env["ASAN_OPTIONS"] = "detect_leaks=0:abort_on_error=1"
    r = subprocess.run([sys.executable, "-c", code], capture_output=True, text=True,
                       timeout=600, cwd=ROOT, env=env)
    out = r.stdout + r.stderr
    assert "ERROR: AddressSanitizer" not in out, out[-4000:]
    assert r.returncode == 0 and "passed" in r.stdout, out[-4000:]
