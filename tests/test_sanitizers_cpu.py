"""The host part of the library under AddressSanitizer and
UndefinedBehaviorSanitizer (CPU only): the C ABI tests run against a build
whose eta_host.cpp is instrumented, with the ASan runtime preloaded; any
invalid access or undefined behaviour in argument validation, workspace
layout or statistics read-back fails them."""
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_abi_tests_pass_under_host_sanitizers():
    from learned_threshold_block_amd import sanitized_build as SB  # CPU-only helper, imported here

    lib = SB.build_sanitized()
    undefined = subprocess.run(["nm", "-D", "--undefined-only", lib], capture_output=True, text=True).stdout
    assert "__asan_report_load" in undefined, "the host code is not instrumented"
    env = dict(os.environ, LD_PRELOAD=SB.asan_runtime(), ASAN_OPTIONS="detect_leaks=0:abort_on_error=1",
               ETA_LIBRARY=lib)
    r = subprocess.run([sys.executable, "-m", "pytest", os.path.join(ROOT, "tests", "test_abi_cpu.py"), "-q",
                        "-p", "no:cacheprovider"], env=env, capture_output=True, text=True, timeout=900, cwd=ROOT)
    out = r.stdout + r.stderr
    assert r.returncode == 0, out[-4000:]
    assert "AddressSanitizer" not in out and "runtime error" not in out, out[-4000:]
