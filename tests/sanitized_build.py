"""A build of libquest whose host code runs under AddressSanitizer and UndefinedBehaviorSanitizer.

The host side of the library (argument validation, the overlap and alignment
checks, the alpha fit, sizing helpers, launch routing) is compiled with the
two sanitizers; the GPU code objects are the ordinary ones.  The sanitizers
apply to the host pass only: each -fsanitize flag is preceded by -Xarch_host.
The result is linked from the ordinary build's other objects into
quantization_aware_amd/_build/san/libquest_san.so and is loaded by a Python
process started with the ASan runtime preloaded.
"""
from __future__ import annotations

import os
import subprocess

from quantization_aware_amd import build

HOST_SOURCES = ["quest_api.hip", "quest_launch.hip"]
SAN_DIR = os.path.join(build.BUILD_DIR, "san")
SAN_LIB = os.path.join(SAN_DIR, "libquest_san.so")
SAN_FLAGS = "-Xarch_host -fsanitize=address -Xarch_host -fsanitize=undefined -Xarch_host -fno-sanitize-recover=all -Xarch_host -fno-omit-frame-pointer -g".split()


def asan_runtime() -> str:
    """Path of the ASan runtime of hipcc's clang, to be preloaded into the process that loads the library."""
    out = subprocess.run([build.hipcc_path(), "-print-file-name=libclang_rt.asan-x86_64.so"], capture_output=True,
                         text=True, check=True).stdout.strip()
    if not os.path.isabs(out) or not os.path.exists(out):
        raise RuntimeError(f"ASan runtime not found (hipcc printed {out!r})")
    return out


def build_sanitized() -> str:
    """Compile the host-code sources with the sanitizers, link with the ordinary objects, return the path."""
    os.makedirs(SAN_DIR, exist_ok=True)
    objs = []
    for src in build.SOURCES:
        normal = os.path.join(build.BUILD_DIR, os.path.splitext(src)[0] + ".o")
        if src in HOST_SOURCES:
            obj = os.path.join(SAN_DIR, os.path.splitext(src)[0] + ".o")
            cmd = build.compile_command(src, obj)
            cmd[1:1] = SAN_FLAGS
            build._run(cmd, False)
            objs.append(obj)
        else:
            if not os.path.exists(normal):
                build._run(build.compile_command(src, normal), False)
            objs.append(normal)
    tmp = SAN_LIB + ".tmp"
    build._run(build.link_command(objs, tmp), False)
    os.replace(tmp, SAN_LIB)
    return SAN_LIB
