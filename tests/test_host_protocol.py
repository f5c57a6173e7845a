"""The host side of the task mailbox (pk_ring.h) against a CPU thread playing the
device, built with ThreadSanitizer and with AddressSanitizer (CPU only)."""

import os
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = os.path.join(ROOT, "tests", "hostproto", "fake_device.cpp")
INC = [f"-I{os.path.join(ROOT, 'include')}", "-I/opt/rocm/include"]


@pytest.mark.parametrize("san", ["thread", "address,undefined", "none"])
def test_mailbox_protocol_against_fake_device(san, tmp_path):
    exe = str(tmp_path / f"fake_device_{san.replace(',', '_')}")
    flags = ["-std=c++17", "-O1", "-g", "-pthread", *INC]
    if san != "none":
        flags += [f"-fsanitize={san}", "-fno-omit-frame-pointer"]
    subprocess.check_call(["g++", *flags, SRC, "-o", exe])
    env = dict(os.environ, TSAN_OPTIONS="halt_on_error=1", ASAN_OPTIONS="detect_leaks=1")
    out = subprocess.run([exe], capture_output=True, text=True, timeout=120, env=env)
    assert out.returncode == 0, out.stdout + out.stderr
    assert "all checks passed" in out.stdout
