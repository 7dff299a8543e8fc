"""The C ABI's CPU tests (tests/test_abi.py, tests/test_binding_checks.py) re-run against a build
whose host code carries AddressSanitizer and UndefinedBehaviorSanitizer checks: argument
validation, overlap and alignment checks, sizing arithmetic and the alpha fit then run with every
memory access and every signed overflow, shift, enum load and conversion checked.  Any report
ends the run (no recovery).  The GPU code objects are the ordinary ones and are not launched."""
from __future__ import annotations

import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_abi_tests_pass_under_asan_and_ubsan():
    import sanitized_build as sb  # only imported here: the build step is CPU-only

    lib = sb.build_sanitized()
    env = dict(os.environ)
    env.update({
        "LD_PRELOAD": sb.asan_runtime(),
        "ASAN_OPTIONS": "detect_leaks=0:abort_on_error=1:halt_on_error=1",
        "UBSAN_OPTIONS": "halt_on_error=1:print_stacktrace=1",
        "QUEST_LIBRARY": lib,
    })
    # the child really runs the sanitized library, with the ASan runtime in the process
    probe = ("import quantization_aware_amd as qa; qa.load_library(); maps = open('/proc/self/maps').read(); "
             "print('san' if 'libquest_san.so' in maps and 'libclang_rt.asan' in maps else 'plain')")
    res = subprocess.run([sys.executable, "-c", probe], cwd=ROOT, env=env, capture_output=True, text=True,
                         timeout=300)
    assert res.stdout.strip() == "san", res.stdout + res.stderr
    res = subprocess.run([sys.executable, "-m", "pytest", "-q", "-x", "-m", "not gpu", "-p", "no:cacheprovider",
                          os.path.join(ROOT, "tests", "test_abi.py"),
                          os.path.join(ROOT, "tests", "test_binding_checks.py")],
                         cwd=ROOT, env=env, capture_output=True, text=True, timeout=900)
    out = res.stdout + res.stderr
    assert "Sanitizer" not in out and "runtime error:" not in out, out[-4000:]
    assert res.returncode == 0, out[-4000:]
