"""The host side of the library (pack, SVD, layouts, argument checks of
every entry point) built with AddressSanitizer and UndefinedBehaviorSanitizer
(host code only) and run through the host ABI tests (CPU only)."""
import pytest


def test_host_abi_under_asan_and_ubsan():
    from tests import host_sanitize as h
    h.build()
    r = h.run_tests(["-s", "tests/test_lib_host.py"])
    tail = (r.stdout[-1500:] + "\n" + r.stderr[-4000:])
    assert r.returncode == 0, f"sanitized host tests failed (exit {r.returncode}):\n{tail}"
    assert " passed" in r.stdout and " failed" not in r.stdout
