"""The C ABI's host code under AddressSanitizer and UndefinedBehaviorSanitizer
(CPU only).  capi.hip is compiled for the host alone, with the kernel
launchers replaced by recording stand-ins (tests/host_check/), and a driver
exercises validation, sequence ordering, launch parameters and the split-KV
workspace layout on full and invalid batches."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "chunked_prefill_sparse_amd", "csrc")
HC = os.path.join(ROOT, "tests", "host_check")
ROCM = os.environ.get("ROCM_PATH", "/opt/rocm")
HIPCC = os.path.join(ROCM, "bin", "hipcc")
CLANG = os.path.join(ROCM, "lib", "llvm", "bin", "clang++")
SAN = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
       "-Xarch_host", "-fno-sanitize-recover=undefined"]


def _run(cmd, **kw):
    r = subprocess.run(cmd, capture_output=True, text=True, timeout=300, **kw)
    assert r.returncode == 0, f"{' '.join(cmd)}\n{r.stdout}\n{r.stderr[-4000:]}"
    return r


@pytest.mark.skipif(not (os.path.exists(HIPCC) and os.path.exists(CLANG)),
                    reason="ROCm compilers not found")
def test_capi_host_code_under_sanitizers(tmp_path):
    out = str(tmp_path)
    common = ["-x", "hip", "--cuda-host-only", "--offload-arch=gfx950", "-std=c++17", "-O1", "-g",
              "-fno-omit-frame-pointer", "-I", os.path.join(ROOT, "include"), "-I", CSRC,
              "-I", HC] + SAN
    objs = []
    for src in (os.path.join(CSRC, "capi.hip"), os.path.join(HC, "launch_stubs.cpp"),
                os.path.join(HC, "driver.cpp")):
        obj = os.path.join(out, os.path.splitext(os.path.basename(src))[0] + "_host.o")
        _run([HIPCC] + common + ["-c", src, "-o", obj])
        objs.append(obj)
    exe = os.path.join(out, "host_check")
    _run([CLANG, "-fsanitize=address,undefined"] + objs +
         ["-L", os.path.join(ROCM, "lib"), "-lamdhip64", "-Wl,-rpath," + os.path.join(ROCM, "lib"),
          "-o", exe])
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=0:abort_on_error=0",
               UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1")
    r = subprocess.run([exe], capture_output=True, text=True, timeout=120, env=env)
    assert r.returncode == 0 and "host check OK" in r.stdout, r.stdout + r.stderr[-4000:]
