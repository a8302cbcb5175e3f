"""The C ABI's host code under AddressSanitizer: build liblla_asan.so (host code
instrumented, device code unchanged) and run the CPU ABI tests against it in a child
process with the ASan runtime preloaded. Argument validation, split planning and the
pointer arithmetic of every entry point run there (fake device pointers never reach a
GPU: each call is rejected, or sized, on the host)."""

import os
import subprocess
import sys

from latent_decode_attention_lla_amd import build

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_abi_tests_pass_under_host_asan():
    lib = build.build(asan=True)
    syms = subprocess.run(["nm", "-D", lib], capture_output=True, text=True).stdout
    assert "__asan_report" in syms  # the host code really is instrumented
    env = dict(os.environ)
    env.update(LD_PRELOAD=build.asan_runtime(), ASAN_OPTIONS="detect_leaks=0:abort_on_error=1",
               LLA_LIBRARY=lib)
    probe = subprocess.run([sys.executable, "-c",
                            "from latent_decode_attention_lla_amd import lla; print(lla.LIB_PATH)"],
                           cwd=ROOT, env=env, capture_output=True, text=True)
    assert probe.returncode == 0 and probe.stdout.strip() == lib, probe.stderr[-2000:]
    r = subprocess.run([sys.executable, "-m", "pytest", "-q", "-m", "not gpu", "-p", "no:cacheprovider",
                        "tests/test_abi.py", "tests/test_zz_no_alloc.py"],
                       cwd=ROOT, env=env, capture_output=True, text=True, timeout=600)
    out = r.stdout + r.stderr
    assert "AddressSanitizer" not in out, out[-4000:]
    assert r.returncode == 0, out[-4000:]
