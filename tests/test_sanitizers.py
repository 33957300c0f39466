"""CPU sanitizer builds: the fp64 oracle under AddressSanitizer + UndefinedBehaviorSanitizer
and, separately, ThreadSanitizer (it splits (sequence, head) pairs over threads); and the
library's host-side argument checks (kda_api.hip, the segmented prefill's sizing in
kda_scan.hip) under AddressSanitizer + UndefinedBehaviorSanitizer, compiled with the
sanitizers on the host side only and linked with stand-ins for the two kernel units'
launchers, which the refused calls never reach.  The drivers are tests/csrc/*.c; every
build goes to a temporary directory.  No GPU is used."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "tests", "csrc")
LIB_CSRC = os.path.join(ROOT, "gated_delta_rule_kda_amd", "csrc")
ROCM = os.environ.get("ROCM_PATH", "/opt/rocm")
HIPCC = os.path.join(ROCM, "bin", "hipcc")
CLANG = os.path.join(ROCM, "llvm", "bin", "clang")
CLANGXX = os.path.join(ROCM, "llvm", "bin", "clang++")
SAN_ENV = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=0",
               UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1", TSAN_OPTIONS="halt_on_error=1")


def _run(cmd, **kw):
    r = subprocess.run(cmd, capture_output=True, text=True, timeout=300, **kw)
    assert r.returncode == 0, f"{' '.join(cmd)}\n{r.stdout}\n{r.stderr}"
    return r


def _instrumented(binary, marker):
    nm = shutil.which("nm")
    if nm is None:
        return True
    syms = subprocess.run([nm, binary], capture_output=True, text=True).stdout
    return marker in syms


@pytest.mark.skipif(shutil.which("gcc") is None, reason="gcc not found")
def test_oracle_under_asan_ubsan(tmp_path):
    exe = str(tmp_path / "oracle_asan")
    _run(["gcc", "-O1", "-g", "-fsanitize=address,undefined", "-fno-sanitize-recover=all",
          "-fno-omit-frame-pointer", os.path.join(CSRC, "oracle_sanitize.c"),
          os.path.join(ROOT, "oracle", "kda_oracle.c"), "-o", exe, "-lm", "-lpthread"])
    assert _instrumented(exe, "__asan_init") and _instrumented(exe, "__ubsan_handle")
    r = _run([exe], env=SAN_ENV)
    assert "oracle checks passed" in r.stdout


@pytest.mark.skipif(shutil.which("gcc") is None, reason="gcc not found")
def test_oracle_under_tsan(tmp_path):
    exe = str(tmp_path / "oracle_tsan")
    _run(["gcc", "-O1", "-g", "-fsanitize=thread", os.path.join(CSRC, "oracle_sanitize.c"),
          os.path.join(ROOT, "oracle", "kda_oracle.c"), "-o", exe, "-lm", "-lpthread"])
    assert _instrumented(exe, "__tsan_init")
    r = subprocess.run([exe], capture_output=True, text=True, timeout=300, env=SAN_ENV)
    if r.returncode != 0 and "unexpected memory mapping" in r.stderr:
        pytest.skip("ThreadSanitizer cannot map its shadow memory on this kernel")
    assert r.returncode == 0, r.stderr
    assert "WARNING: ThreadSanitizer" not in r.stderr
    assert "oracle checks passed" in r.stdout


@pytest.mark.skipif(not (os.path.exists(HIPCC) and os.path.exists(CLANGXX)), reason="ROCm toolchain not found")
def test_library_host_checks_under_asan_ubsan(tmp_path):
    # hipcc builds the device side as usual and instruments only the host side (each
    # sanitizer flag behind -Xarch_host)
    host_san = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
                "-Xarch_host", "-fno-sanitize-recover=all", "-Xarch_host", "-fno-omit-frame-pointer"]
    objs = []
    for src in (os.path.join(LIB_CSRC, "kda_api.hip"), os.path.join(LIB_CSRC, "kda_scan.hip"),
                os.path.join(CSRC, "launch_stubs.hip")):
        obj = str(tmp_path / (os.path.basename(src) + ".o"))
        _run([HIPCC, "-O1", "-g", "-std=c++17", "-fPIC", "--offload-arch=gfx950", "-Xclang", "-target-feature",
              "-Xclang", "-packed-fp32-ops", *host_san, "-I", os.path.join(ROOT, "include"), "-I", LIB_CSRC,
              "-c", src, "-o", obj])
        objs.append(obj)
    drv = str(tmp_path / "abi_sanitize.o")
    _run([CLANG, "-O1", "-g", "-fsanitize=address,undefined", "-fno-sanitize-recover=all",
          "-I", os.path.join(ROOT, "include"), "-c", os.path.join(CSRC, "abi_sanitize.c"), "-o", drv])
    exe = str(tmp_path / "abi_asan")
    _run([CLANGXX, "-fsanitize=address,undefined", "-o", exe, drv, *objs, "-L", os.path.join(ROCM, "lib"),
          "-lamdhip64", f"-Wl,-rpath,{os.path.join(ROCM, 'lib')}"])
    assert _instrumented(exe, "__asan_init")
    r = _run([exe], env=SAN_ENV)
    assert "abi checks passed" in r.stdout
