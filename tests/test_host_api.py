"""The C ABI's host-side argument handling, built with AddressSanitizer and
UndefinedBehaviorSanitizer against stand-in launchers (CPU only; see
tests/c_abi/host_api_test.cpp)."""
import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))


def test_host_api_under_sanitizers():
    d = os.path.join(HERE, "c_abi")
    subprocess.run(["make", "-s", "-C", d, "host_api_test"], check=True)
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=0:verify_asan_link_order=0",
               UBSAN_OPTIONS="print_stacktrace=1")
    r = subprocess.run([os.path.join(d, "host_api_test")], capture_output=True, text=True,
                       env=env, timeout=120)
    print(r.stdout, r.stderr)
    assert r.returncode == 0, r.stderr
    assert "checks passed" in r.stdout
