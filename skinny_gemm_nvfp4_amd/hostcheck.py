"""A copy of libnvfp4.so with AddressSanitizer and UndefinedBehaviorSanitizer in its host code
(argument validation, plan choice, launch set-up), for runs of the host checks on a machine with
no GPU. Every sanitizer flag goes to hipcc's host pass only. The device code of this copy is
compiled without optimisation because it never runs: a process that loads the copy must have no
GPU visible, and it needs the clang ASan runtime first in line (LD_PRELOAD=asan_runtime()).
Only the host sanitizer test uses this module.
"""
import os
import subprocess

from . import build as _build

COMPILE = ["-Xarch_device", "-O0",
           "-Xarch_host", "-O1", "-Xarch_host", "-g",
           "-Xarch_host", "-fno-omit-frame-pointer",
           "-Xarch_host", "-fsanitize=address",
           "-Xarch_host", "-fsanitize=undefined",
           "-Xarch_host", "-fno-sanitize-recover=undefined"]
LINK = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
        "-Xarch_host", "-shared-libsan"]


def build_checked(out: str, verbose: bool = False) -> str:
    obj_dir = os.path.join(os.path.dirname(os.path.abspath(out)), "checked_objs")
    return _build._build(out, _build.compile_flags() + COMPILE, LINK, obj_dir, verbose)


def asan_runtime() -> str:
    """The clang AddressSanitizer runtime that build_checked links against, or ''."""
    res = subprocess.run([_build.hipcc(), "-print-file-name=libclang_rt.asan-x86_64.so"],
                         capture_output=True, text=True)
    path = res.stdout.strip()
    return path if res.returncode == 0 and os.path.isabs(path) and os.path.exists(path) else ""
