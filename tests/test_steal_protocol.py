"""The steal schedule's share-word protocol (decode_attention_09_amd/csrc/
fd_steal.h, the functions the matrix-core kernel applies with atomics),
driven on the host through 200,000 random interleavings of an owner's
claims and up to eight thieves' takes, stale loads included
(tests/c/steal_protocol.hip): every chunk must end in exactly one run, the
owner's run must be a prefix, takes must be ranges behind it in slot order,
and the steal count the owner reads with its last claim must equal the
takes. Built with hipcc for the host only (no device code), with the
host-side AddressSanitizer and UndefinedBehaviorSanitizer. CPU only."""
import os
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HIPCC = "/opt/rocm/bin/hipcc"
HOST_SAN = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
            "-Xarch_host", "-fno-sanitize-recover=undefined"]


def test_share_word_protocol(tmp_path):
    if not os.path.exists(HIPCC):
        pytest.skip("hipcc not available")
    exe = str(tmp_path / "steal_protocol")
    cmd = [HIPCC, "--offload-host-only", "-O1", "-g", "-std=c++17",
           "-I", os.path.join(ROOT, "decode_attention_09_amd", "csrc"), *HOST_SAN,
           os.path.join(ROOT, "tests", "c", "steal_protocol.hip"), "-o", exe]
    r = subprocess.run(cmd, capture_output=True, text=True, cwd=str(tmp_path))
    assert r.returncode == 0, r.stderr
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=0", UBSAN_OPTIONS="print_stacktrace=1")
    r = subprocess.run([exe], capture_output=True, text=True, env=env, timeout=300)
    assert r.returncode == 0, r.stdout + r.stderr
    assert r.stdout.startswith("steal protocol ok 200000 cases"), r.stdout
    assert "runtime error" not in r.stderr
    takes = int(r.stdout.split()[5])
    assert takes > 100000   # the interleavings do exercise takes
