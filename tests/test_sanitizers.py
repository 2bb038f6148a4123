"""Sanitizer builds of the host code (CPU only; nothing runs on a GPU).

1. The fp64 oracle (plain C) built with AddressSanitizer and UndefinedBehaviorSanitizer,
   running the oracle pin tests (forward, block options, MIMO projections, gains and biases,
   gradients) in a child process with the ASan runtime preloaded.
2. The library's host dispatch layer (m3_api.cpp) built with ASan and UBSan on the host side
   only (its device part is the static scratch array), linked against stub launchers that
   check every parameter block and workspace carve-out instead of launching
   (tests/sanitize/stub_launchers.cpp), and driven over a seeded sweep of shapes, options,
   strides, projections and argument errors (tests/sanitize/host_driver.cpp).

Both stop at the first sanitizer report (-fno-sanitize-recover=all).
"""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SAN = ["-fsanitize=address,undefined", "-fno-sanitize-recover=all", "-fno-omit-frame-pointer"]


def _have(tool):
    return shutil.which(tool) is not None


def _gcc_runtime(name):
    out = subprocess.run(["gcc", f"-print-file-name={name}"], capture_output=True, text=True).stdout.strip()
    return out if os.path.isabs(out) and os.path.exists(out) else None


def _clean(log):
    return "AddressSanitizer" not in log and "runtime error:" not in log and "LeakSanitizer" not in log


@pytest.mark.skipif(not _have("gcc"), reason="gcc not available")
def test_oracle_pins_under_asan_ubsan(tmp_path):
    asan = _gcc_runtime("libasan.so")
    if asan is None:
        pytest.skip("libasan not available")
    lib = str(tmp_path / "m3_oracle_san.so")
    srcs = [os.path.join(ROOT, "oracle", f) for f in ("m3_oracle.c", "m3_oracle_bwd.c")]
    subprocess.check_call(["gcc", "-O1", "-g", "-std=c11", "-fPIC", "-shared", "-pthread", "-fno-fast-math", *SAN,
                           *srcs, "-o", lib, "-lm"])
    env = dict(os.environ, M3_ORACLE_LIB=lib, LD_PRELOAD=asan, ASAN_OPTIONS="detect_leaks=0",
               UBSAN_OPTIONS="print_stacktrace=1")
    pins = ["tests/test_oracle_pins.py", "tests/test_oracle_pins_block.py", "tests/test_oracle_pins_mimo_proj.py",
            "tests/test_oracle_pins_gain_bias.py", "tests/test_oracle_bwd_pins.py"]
    r = subprocess.run(["python", "-m", "pytest", "-q", "-x", "-p", "no:cacheprovider", "-m", "not gpu", *pins],
                       cwd=ROOT, env=env, capture_output=True, text=True, timeout=900)
    log = r.stdout + r.stderr
    assert r.returncode == 0 and _clean(log), log[-4000:]


@pytest.mark.skipif(not (_have("hipcc") and _have("g++")), reason="hipcc / g++ not available")
def test_host_dispatch_under_asan_ubsan(tmp_path):
    csrc = os.path.join(ROOT, "mamba_selective_scan_amd", "csrc")
    inc = os.path.join(ROOT, "include")
    san = os.path.join(ROOT, "tests", "sanitize")
    rocm = os.environ.get("ROCM_PATH", "/opt/rocm")
    api, stub, drv, exe = (str(tmp_path / n) for n in ("api.o", "stub.o", "drv.o", "m3_host_san"))
    host_san = []
    for flag in SAN:  # host side only: each flag behind -Xarch_host
        host_san += ["-Xarch_host", flag]
    subprocess.check_call(["hipcc", "-x", "hip", "--offload-arch=gfx950", "-O1", "-g", "-std=c++17", "-fPIC",
                           "-I", inc, *host_san, "-c", os.path.join(csrc, "m3_api.cpp"), "-o", api],
                          stderr=subprocess.DEVNULL)
    subprocess.check_call(["g++", "-std=c++17", "-O1", "-g", *SAN, "-D__HIP_PLATFORM_AMD__", "-I",
                           os.path.join(rocm, "include"), "-I", csrc, "-c", os.path.join(san, "stub_launchers.cpp"),
                           "-o", stub])
    subprocess.check_call(["g++", "-std=c++17", "-O1", "-g", *SAN, "-I", inc, "-c",
                           os.path.join(san, "host_driver.cpp"), "-o", drv])
    subprocess.check_call(["g++", *SAN, api, stub, drv, "-L", os.path.join(rocm, "lib"),
                           "-Wl,-rpath," + os.path.join(rocm, "lib"), "-lamdhip64", "-o", exe])
    r = subprocess.run([exe], capture_output=True, text=True, timeout=600,
                       env=dict(os.environ, ASAN_OPTIONS="detect_leaks=0"))
    log = r.stdout + r.stderr
    assert r.returncode == 0 and _clean(log), log[-4000:]
    assert "stub failures 0, unexpected 0" in log
