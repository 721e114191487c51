"""Host code of the C ABI under AddressSanitizer and UndefinedBehaviorSanitizer.

Builds a copy of librk.so whose host code (api.cpp: argument validation,
workspace layout, launch set-up) is instrumented — the device objects are
the regular ones — and a C++ driver (tests/abi_host_check.cpp) with the same
instrumentation that exercises every validation path.  No GPU is involved:
each call returns before any HIP call.  Any sanitizer report, or a status
other than the expected one, fails the test.
"""

import os
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
PKG = os.path.join(ROOT, "masked_attention_amd")
BUILD = os.path.join(PKG, "_build")
DEVICE_OBJS = ["plan.hip.o", "rope.hip.o", "attn_ref.hip.o", "attn_mfma.hip.o",
               "attn_combine.hip.o", "attn_bwd_ref.hip.o", "attn_bwd_mfma.hip.o",
               "gather_sum.hip.o", "attn_pointwise_ref.hip.o", "attn_pointwise_mfma.hip.o",
               "norm_bwd.hip.o"]
HIPCC = "/opt/rocm/bin/hipcc"


def _run(cmd, **kw):
    r = subprocess.run(cmd, capture_output=True, text=True, **kw)
    assert r.returncode == 0, f"{' '.join(cmd)}\n{r.stdout}\n{r.stderr}"
    return r


@pytest.mark.skipif(not os.path.exists(HIPCC) or not os.path.exists("/opt/rocm/llvm/bin/clang++"),
                    reason="needs ROCm's hipcc and clang++")
def test_abi_host_paths_under_asan_ubsan(tmp_path):
    objs = [os.path.join(BUILD, o) for o in DEVICE_OBJS]
    if not all(os.path.exists(o) for o in objs):
        pytest.skip("device objects not built (run __graft_entry__.build() first)")
    host_objs = []
    for src in ("api.cpp", "layout.cpp"):
        o = str(tmp_path / (src + ".asan.o"))
        # host pass instrumented, device pass unchanged
        _run([HIPCC, "-O1", "-g", "-std=c++17", "-fPIC", "-I", os.path.join(ROOT, "include"),
              "--offload-arch=gfx950", "-Xclang", "-target-feature", "-Xclang",
              "-packed-fp32-ops", "-Xarch_host", "-fsanitize=address", "-Xarch_host",
              "-fsanitize=undefined", "-Xarch_host", "-fno-sanitize-recover=all", "-Xarch_host",
              "-fno-omit-frame-pointer", "-x", "hip", "-c", os.path.join(PKG, "csrc", src),
              "-o", o])
        host_objs.append(o)
    clang = "/opt/rocm/llvm/bin/clang++"
    # directory of the shared sanitizer runtimes that -shared-libsan links to
    rt = os.path.dirname(subprocess.run([clang, "--print-file-name=libclang_rt.asan-x86_64.so"],
                                        capture_output=True, text=True).stdout.strip())
    rpath = [f"-Wl,-rpath,{rt}", "-Wl,-rpath,/opt/rocm/lib", f"-Wl,-rpath,{tmp_path}"]
    lib = str(tmp_path / "librk_asan.so")
    _run([clang, "-shared", "-o", lib, *host_objs, *objs, "-L/opt/rocm/lib", "-lamdhip64",
          "-fsanitize=address,undefined", "-shared-libsan", *rpath])
    exe = str(tmp_path / "abi_host_check")
    _run([clang, "-O1", "-g", "-std=c++17", "-fsanitize=address,undefined",
          "-fno-sanitize-recover=all", "-shared-libsan", "-I", os.path.join(ROOT, "include"),
          os.path.join(ROOT, "tests", "abi_host_check.cpp"), "-o", exe, lib, *rpath])
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=0:abort_on_error=0",
               UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1")
    r = subprocess.run([exe], capture_output=True, text=True, env=env, timeout=120)
    assert r.returncode == 0, r.stdout + r.stderr
    assert "abi host checks passed" in r.stdout
    assert "ERROR: AddressSanitizer" not in r.stderr
    assert "runtime error" not in r.stderr
    # and the instrumentation is live: a planted overflow in the driver is caught
    r = subprocess.run([exe, "--self-test"], capture_output=True, text=True, env=env, timeout=120)
    assert r.returncode != 0 and "heap-buffer-overflow" in r.stderr
