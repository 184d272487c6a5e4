"""The library's host code under AddressSanitizer and UndefinedBehaviorSanitizer (CPU only).

Every source of libvc is compiled host-only (no device code) with both sanitizers and linked
into tests/native/host_sanitize.cpp, which drives the page allocator and the Admit scheduler
with random operation sequences against simple models, and the attention calls' validation and
launch planning (up to 1024 requests, random splits) up to the point where a device would be
needed.  Any sanitizer report fails the run.  The oracle is Python and numpy, which these
sanitizers do not cover.
"""
import concurrent.futures as cf
import glob
import os
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CLANG = "/opt/rocm/lib/llvm/bin/clang++"
SAN = ["-fsanitize=address", "-fsanitize=undefined", "-fno-sanitize-recover=all"]


def _run(cmd):
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, f"{' '.join(cmd)}\n{r.stderr[-3000:]}"


@pytest.mark.timeout(900)
def test_host_code_under_asan_and_ubsan(tmp_path):
    if not os.path.exists(CLANG):
        pytest.skip("ROCm clang is not installed")
    inc = ["-I", os.path.join(ROOT, "include"), "-I", "/opt/rocm/include"]
    # the sanitizers instrument the host side only (each flag behind -Xarch_host; device code is
    # compiled as usual and never launched here)
    host_san = [f for x in SAN for f in ("-Xarch_host", x)]
    host_hip = ["-x", "hip", "--offload-arch=gfx950", "-fno-gpu-sanitize", "-O1", "-g", "-std=c++17", "-fPIC",
                "-fno-omit-frame-pointer", "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
                *host_san, *inc]
    srcs = sorted(glob.glob(os.path.join(ROOT, "lossless_kv_cache_vc_amd", "csrc", "*.hip")))
    objs = [str(tmp_path / (os.path.basename(s) + ".o")) for s in srcs]
    with cf.ThreadPoolExecutor(max_workers=4) as ex:
        list(ex.map(_run, [[CLANG, *host_hip, "-c", s, "-o", o] for s, o in zip(srcs, objs)]))
    drv = str(tmp_path / "host_sanitize.o")
    _run([CLANG, "-O1", "-g", "-std=c++17", "-fno-omit-frame-pointer", *SAN, *inc, "-c",
          os.path.join(ROOT, "tests", "native", "host_sanitize.cpp"), "-o", drv])
    exe = str(tmp_path / "host_sanitize")
    _run([CLANG, *SAN, drv, *objs, "-L/opt/rocm/lib", "-Wl,-rpath,/opt/rocm/lib", "-lamdhip64", "-o", exe])
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=0", UBSAN_OPTIONS="print_stacktrace=1")
    r = subprocess.run([exe], capture_output=True, text=True, env=env, timeout=600)
    out = r.stdout + r.stderr
    assert r.returncode == 0, out[-4000:]
    assert "runtime error" not in out and "AddressSanitizer" not in out, out[-4000:]
    assert "host sanitize checks passed" in out
