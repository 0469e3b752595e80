"""The C ABI's host code under AddressSanitizer and UndefinedBehaviorSanitizer.

salr_api.cpp (argument validation, size arithmetic, workspace layouts) is
compiled with both sanitizers for the host (device code is not
instrumented), linked with the library's other objects into the driver
tests/host_sanitize_driver.c, and run on the CPU: every status code the
driver expects must come back, with no sanitizer report.  No GPU is needed:
none of the driver's calls reaches the device."""

import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
PKG = os.path.join(ROOT, "sparse_rank_linear_amd")
BUILD = os.path.join(PKG, "_build")
SAN = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
       "-Xarch_host", "-fno-sanitize-recover=all", "-Xarch_host", "-fno-omit-frame-pointer"]


def _tool(name, *cands):
    for c in cands:
        if c and os.path.exists(c):
            return c
    return shutil.which(name)


def test_abi_host_code_under_asan_ubsan(tmp_path):
    hipcc = _tool("hipcc", os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc")
    cc = _tool("gcc", "/usr/bin/gcc")
    if not hipcc or not cc:
        pytest.skip("hipcc and gcc are needed")
    objs = sorted(os.path.join(BUILD, f) for f in os.listdir(BUILD)) if os.path.isdir(BUILD) else []
    objs = [o for o in objs if o.endswith(".o") and not o.endswith("salr_api.cpp.o")]
    if not objs:
        pytest.skip("library objects not built (python -m sparse_rank_linear_amd.build)")
    inc = ["-I", os.path.join(ROOT, "include"), "-I", os.path.join(PKG, "csrc")]
    api_o, drv_o, exe = tmp_path / "api.o", tmp_path / "drv.o", tmp_path / "drv"
    run = lambda cmd: subprocess.run(cmd, capture_output=True, text=True, timeout=600)
    r = run([hipcc, "-O1", "-g", "-std=c++17", "-fPIC", *inc, *SAN, "-c",
             os.path.join(PKG, "csrc", "salr_api.cpp"), "-o", str(api_o)])
    assert r.returncode == 0, r.stderr[-3000:]
    r = run([cc, "-O1", "-g", *inc, "-fsanitize=address,undefined", "-fno-sanitize-recover=all", "-c",
             os.path.join(ROOT, "tests", "host_sanitize_driver.c"), "-o", str(drv_o)])
    assert r.returncode == 0, r.stderr[-3000:]
    r = run([hipcc, "--offload-arch=gfx950", *SAN[:4], "-o", str(exe), str(drv_o), str(api_o), *objs])
    assert r.returncode == 0, r.stderr[-3000:]
    syms = run(["nm", str(exe)])
    assert "__asan_init" in syms.stdout and "__ubsan_handle" in syms.stdout  # the sanitizers are linked in
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=0:abort_on_error=0", UBSAN_OPTIONS="print_stacktrace=1",
               HIP_VISIBLE_DEVICES="")
    r = subprocess.run([str(exe)], capture_output=True, text=True, timeout=300, env=env)
    assert "AddressSanitizer" not in r.stderr and "runtime error" not in r.stderr, r.stderr[-3000:]
    assert r.returncode == 0 and r.stdout.strip() == "ok", (r.stdout, r.stderr[-3000:])
