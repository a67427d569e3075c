"""The C ABI from C (CPU only): include/fd.h compiles as strict C99, a C
program links against libfd.so and the host-only entry points return what
the header documents."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
PKG = os.path.join(ROOT, "decode_attention_09_amd")


@pytest.fixture(scope="module")
def c_program(tmp_path_factory):
    cc = shutil.which("gcc") or shutil.which("cc")
    if cc is None:
        pytest.skip("no C compiler")
    if not os.path.exists(os.path.join(PKG, "libfd.so")):
        pytest.fail("libfd.so must be built before the tests")
    exe = str(tmp_path_factory.mktemp("cabi") / "abi_check")
    cmd = [cc, "-std=c99", "-Wall", "-Wextra", "-Werror", "-pedantic",
           "-I", os.path.join(ROOT, "include"), os.path.join(ROOT, "tests", "c", "abi_check.c"),
           "-o", exe, "-L", PKG, "-lfd", f"-Wl,-rpath,{PKG}", "-lm"]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr
    return exe


def test_c_program(c_program):
    env = dict(os.environ)
    rocm_lib = "/opt/rocm/lib"
    env["LD_LIBRARY_PATH"] = rocm_lib + (":" + env["LD_LIBRARY_PATH"]
                                         if env.get("LD_LIBRARY_PATH") else "")
    r = subprocess.run([c_program], capture_output=True, text=True, env=env, timeout=60)
    assert r.returncode == 0, r.stderr
    out = dict(line.split(" ", 1) for line in r.stdout.strip().splitlines())
    st, ns = out["plan"].split()
    assert st == "0" and 1 <= int(ns) <= 16
    assert out["plan_empty"] == "3"
    assert out["plan_sched"] == "0 3 8"   # FD_OK, FD_SCHED_STEAL, 8 slots
    rows = 2 * 8 * 4
    # control block: claim counter 256 B, arrival counters padded to 256 B,
    # 4096 share words of the steal schedule
    steal = 4096 * 8
    assert int(out["ws"]) == ((rows * 128 * 4 + 255) // 256 * 256 + (rows * 4 + 255) // 256 * 256
                              + 256 + 256 + steal)
    assert int(out["ws_unnorm"]) == ((rows * 128 * 4 + 255) // 256 * 256
                                     + (rows * 4 + 255) // 256 * 256 + rows * 4)
    assert out["ws_bad"] == "0"
    # (batch, heads, num_splits, dim): 128 splits at dim 64, then 64 splits at dim 128
    a, b = (int(x) for x in out["ws_order"].split())
    assert a == 128 * 64 * 4 + 512 + 512 + steal and b == 64 * 128 * 4 + 256 + 512 + steal
    assert a != b
    a, b = (int(x) for x in out["ws_unnorm_order"].split())
    assert a == 128 * 64 * 4 + 2 * 128 * 4 and b == 64 * 128 * 4 + 256 + 64 * 4
    assert out["null_args"] == "1"
    assert out["bad_dim"] == "2"
    assert out["nan_scale"] == "1"
    assert out["combine_null"] == "1"
    assert "empty" in out["status"]
    assert out["path"] == "0 1 -1"
    assert out["sched"] == "0 2 -1"
    assert out["combine"] == "0 1 -1"
