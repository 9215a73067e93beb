"""The host API under AddressSanitizer and UBSan, on the CPU.

smla_api.hip (argument checks, planning, workspace layout, launch marshalling, the
allocation-free entry point's scratch lookup) is compiled for the host alone with ASan and
UBSan, every UB check fatal, and linked with stand-ins for the kernel launchers and the HIP
runtime calls (tests/host_check/).  Two child processes load it with the ASan runtime
preloaded: one runs the C-ABI tests of test_abi_host.py against it, the other the launch
checks of tests/host_check/launch_checks.py.  No GPU and no HIP runtime is involved."""

from __future__ import annotations

import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, os.path.join(ROOT, "tests", "host_check"))


@pytest.fixture(scope="module")
def hostcheck():
    try:
        import hostcheck_build as hc
        hc.asan_runtime()
        path = hc.build()
    except FileNotFoundError as e:
        pytest.skip(f"sanitizer toolchain not available: {e}")
    return hc, path


def _child(hc, args, extra_env=None, timeout=600):
    env = hc.runtime_env()
    env.update(extra_env or {})
    res = subprocess.run([sys.executable, *args], cwd=ROOT, env=env, capture_output=True, text=True,
                         timeout=timeout)
    out = res.stdout + res.stderr
    assert "AddressSanitizer" not in out, out[-4000:]
    assert "runtime error" not in out, out[-4000:]
    assert res.returncode == 0, out[-4000:]
    return out


def test_abi_tests_pass_under_asan_and_ubsan(hostcheck):
    hc, path = hostcheck
    out = _child(hc, ["-m", "pytest", "-q", "-p", "no:cacheprovider", "-m", "not gpu",
                      os.path.join("tests", "test_abi_host.py")],
                 {"SMLA_HOST_CHECK_LIB": path})
    assert " passed" in out and "skipped" not in out, out[-2000:]


def test_launch_marshalling_under_asan_and_ubsan(hostcheck):
    hc, path = hostcheck
    out = _child(hc, [os.path.join("tests", "host_check", "launch_checks.py"), path])
    assert "all launch checks passed" in out
