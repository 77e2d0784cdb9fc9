"""The library's host code under AddressSanitizer and UndefinedBehaviorSanitizer
(no GPU needed).

api.hip (argument validation, planning, the C ABI) is compiled with both
sanitizers on its host side (`-Xarch_host -fsanitize=...`; the device code is
built as usual) and linked with the other objects of the regular build into
a separate library; tests/host/host_checks.cpp, built with the same
sanitizers, drives every rejection path of the C ABI through it, including
shapes near the int64 limits.  Any sanitizer report fails the run.  Nothing
here touches a device: every call is rejected before the device query or
before any work is enqueued.
"""
import os
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "deformable_convolution_amd", "csrc")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
CLANG = "/opt/rocm/llvm/bin/clang++"
SAN_HOST = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined", "-Xarch_host",
            "-fno-sanitize-recover=undefined", "-Xarch_host", "-fno-omit-frame-pointer"]


def _run(cmd, **kw):
    r = subprocess.run(cmd, capture_output=True, text=True, **kw)
    assert r.returncode == 0, "%s\n%s%s" % (" ".join(cmd), r.stdout[-3000:], r.stderr[-3000:])
    return r


@pytest.fixture(scope="module")
def driver(tmp_path_factory):
    if not (os.path.exists(HIPCC) and os.path.exists(CLANG)):
        pytest.skip("hipcc / clang not available")
    d = str(tmp_path_factory.mktemp("san"))
    objdir = os.path.join(CSRC, "_build")
    others = [os.path.join(objdir, f.replace(".hip", ".o")) for f in
              ("k_direct.hip", "k_backward.hip", "k_packed.hip", "k_dc2d.hip", "k_mfma.hip", "k_mfma_f32.hip",
               "k_mfma_f32_mask.hip", "k_mfma_bf16.hip", "k_mfma_bf16_mask.hip")]
    if not all(os.path.exists(o) for o in others):
        from deformable_convolution_amd.csrc import build
        build.build()
    api = os.path.join(d, "api_san.o")
    _run([HIPCC, "--offload-arch=gfx950", "-O1", "-g", "-std=c++17", "-fPIC", "-Xclang", "-target-feature",
          "-Xclang", "-packed-fp32-ops", *SAN_HOST, "-I", os.path.join(ROOT, "include"), "-c",
          os.path.join(CSRC, "api.hip"), "-o", api])
    lib = os.path.join(d, "libdc1d_san.so")
    # linked by the host compiler (the objects already carry their device code)
    _run([CLANG, "-shared", "-fPIC", "-fsanitize=address,undefined", "-shared-libsan", "-o", lib, api, *others,
          "-L/opt/rocm/lib", "-lamdhip64", "-Wl,-rpath,/opt/rocm/lib"])
    rt = os.path.dirname(subprocess.run(["/opt/rocm/llvm/bin/clang", "-print-file-name=libclang_rt.asan-x86_64.so"],
                                        capture_output=True, text=True).stdout.strip())
    exe = os.path.join(d, "host_checks")
    _run([CLANG, "-O1", "-g", "-fsanitize=address,undefined", "-fno-sanitize-recover=undefined", "-shared-libsan",
          "-I", os.path.join(ROOT, "include"), os.path.join(ROOT, "tests", "host", "host_checks.cpp"), "-o", exe,
          "-L", d, "-ldc1d_san", "-Wl,-rpath," + d, "-Wl,-rpath," + rt])
    return exe


def test_host_validation_is_sanitizer_clean(driver):
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=0:abort_on_error=0",
               UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1",
               HIP_VISIBLE_DEVICES="", ROCR_VISIBLE_DEVICES="")
    r = subprocess.run([driver], capture_output=True, text=True, timeout=300, env=env)
    out = r.stdout + r.stderr
    assert "ERROR: AddressSanitizer" not in out and "runtime error" not in out, out[-4000:]
    assert r.returncode == 0, out[-4000:]
    assert "host checks: 0 failure(s)" in out
