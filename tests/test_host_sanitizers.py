"""The library's host code under AddressSanitizer and UndefinedBehaviorSanitizer,
on the CPU: the C ABI layer (argument checks with fake device pointers, so nothing
is launched; the host repack and MXFP4 -> NVFP4 conversion on exact-size heap
buffers) compiled with host-only sanitizers and driven by a small C program
(host_sanitize/driver.c). Device code is built without them. Needs hipcc and the
kernel objects of the last in-tree build (_build/)."""
import glob
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HIPCC = "/opt/rocm/bin/hipcc"
CLANG = "/opt/rocm/llvm/bin/clang"
OBJS = [o for o in glob.glob(os.path.join(ROOT, "_build", "*.o")) if not o.endswith("moeq_api.o")]


@pytest.mark.skipif(not (os.path.exists(HIPCC) and os.path.exists(CLANG) and OBJS),
                    reason="hipcc or the built kernel objects are missing")
def test_host_code_is_clean_under_asan_and_ubsan(tmp_path):
    inc = ["-I", os.path.join(ROOT, "include"), "-I", os.path.join(ROOT, "bit_quantized_moe_dequant_amd", "csrc")]
    api = str(tmp_path / "moeq_api.o")
    san = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
           "-Xarch_host", "-fno-omit-frame-pointer"]
    subprocess.run([HIPCC, "--offload-arch=gfx950", "-O1", "-g", "-std=c++17", "-fPIC", *san, *inc, "-c",
                    os.path.join(ROOT, "bit_quantized_moe_dequant_amd", "csrc", "moeq_api.hip"), "-o", api],
                   check=True, capture_output=True)
    drv = str(tmp_path / "driver.o")
    subprocess.run([CLANG, "-c", "-g", "-fsanitize=address,undefined", "-fno-omit-frame-pointer", *inc,
                    os.path.join(ROOT, "tests", "host_sanitize", "driver.c"), "-o", drv],
                   check=True, capture_output=True)
    exe = str(tmp_path / "driver")
    subprocess.run([HIPCC, "--offload-arch=gfx950", "-fsanitize=address", "-fsanitize=undefined", "-fno-gpu-sanitize",
                    drv, api, *OBJS, "-o", exe], check=True, capture_output=True)
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1", UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1")
    r = subprocess.run([exe], capture_output=True, text=True, env=env, timeout=300, cwd=str(tmp_path))
    assert r.returncode == 0, r.stdout + r.stderr
    assert "ok (0 failures)" in r.stdout
