"""The host layer of libfd (argument checks, workspace sizes, split
planner) built with AddressSanitizer and UndefinedBehaviorSanitizer on the
host side only, with the kernel launchers replaced by stand-ins that report
an error, then driven from C: the C ABI program of test_c_abi.py and a
deterministic stress of the planner and workspace functions. CPU only."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "decode_attention_09_amd", "csrc")
HIPCC = "/opt/rocm/bin/hipcc"
CLANG = "/opt/rocm/llvm/bin/clang"
ROCM_LIB = "/opt/rocm/lib"

# Sanitizers instrument host code only: each -fsanitize sits behind -Xarch_host.
HOST_SAN = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
            "-Xarch_host", "-fno-sanitize-recover=undefined",
            "-Xarch_host", "-fno-omit-frame-pointer"]


@pytest.fixture(scope="module")
def san_lib(tmp_path_factory):
    if not (os.path.exists(HIPCC) and os.path.exists(CLANG)):
        pytest.skip("ROCm clang toolchain not available")
    d = tmp_path_factory.mktemp("san")
    flags = ["--offload-arch=gfx950", "-O1", "-g", "-std=c++17", "-fPIC",
             "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
             "-I", os.path.join(ROOT, "include"), "-I", CSRC, *HOST_SAN]
    objs = []
    for src in (os.path.join(CSRC, "fd_api.hip"), os.path.join(ROOT, "tests", "c", "launch_stubs.hip")):
        obj = str(d / (os.path.basename(src) + ".o"))
        r = subprocess.run([HIPCC, *flags, "-c", src, "-o", obj], capture_output=True, text=True)
        assert r.returncode == 0, r.stderr
        objs.append(obj)
    lib = str(d / "libfd_san.so")
    r = subprocess.run([HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", "-o", lib, *objs],
                       capture_output=True, text=True)
    assert r.returncode == 0, r.stderr
    return d


def _run_c(san_dir, source, name):
    exe = str(san_dir / name)
    cmd = [CLANG, "-std=c99", "-O1", "-g", "-Wall", "-Wextra", "-Werror",
           "-fsanitize=address,undefined", "-fno-sanitize-recover=undefined",
           "-I", os.path.join(ROOT, "include"), source, "-o", exe,
           "-L", str(san_dir), "-lfd_san", f"-Wl,-rpath,{san_dir}",
           "-L", ROCM_LIB, f"-Wl,-rpath,{ROCM_LIB}", "-lm"]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr
    env = dict(os.environ)
    # the HIP runtime is not instrumented and keeps allocations until exit
    env["ASAN_OPTIONS"] = "detect_leaks=0:abort_on_error=0"
    env["UBSAN_OPTIONS"] = "print_stacktrace=1"
    r = subprocess.run([exe], capture_output=True, text=True, env=env, timeout=120)
    assert r.returncode == 0, r.stdout + r.stderr
    assert "ERROR: AddressSanitizer" not in r.stderr
    assert "runtime error" not in r.stderr
    return r.stdout


def test_library_is_instrumented(san_lib):
    r = subprocess.run(["nm", "-D", str(san_lib / "libfd_san.so")], capture_output=True, text=True)
    if r.returncode != 0 or shutil.which("nm") is None:
        pytest.skip("nm not available")
    assert "__asan" in r.stdout


def test_c_abi_program_under_sanitizers(san_lib):
    out = _run_c(san_lib, os.path.join(ROOT, "tests", "c", "abi_check.c"), "abi_san")
    lines = dict(line.split(" ", 1) for line in out.strip().splitlines())
    assert lines["plan_empty"] == "3" and lines["null_args"] == "1"


def test_host_stress_under_sanitizers(san_lib):
    out = _run_c(san_lib, os.path.join(ROOT, "tests", "c", "host_stress.c"), "stress_san")
    assert out.startswith("stress ok ")
    assert int(out.split()[2]) > 10000
