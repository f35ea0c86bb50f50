"""A checked copy of the CPU oracle (test infrastructure): gcc with AddressSanitizer and
UndefinedBehaviorSanitizer. A process that loads it needs gcc's ASan runtime first in line
(LD_PRELOAD=asan_runtime()). Only the host sanitizer test uses this module.
"""
import os
import subprocess

from . import build as _build

FLAGS = ("-g", "-fno-omit-frame-pointer", "-fsanitize=address,undefined",
         "-fno-sanitize-recover=undefined")


def build_checked(out: str, verbose: bool = False) -> str:
    return _build.build(verbose=verbose, extra_flags=FLAGS, out=out)


def asan_runtime() -> str:
    """gcc's AddressSanitizer runtime, or '' if gcc has none."""
    res = subprocess.run(["gcc", "-print-file-name=libasan.so"], capture_output=True, text=True)
    path = res.stdout.strip()
    return path if res.returncode == 0 and os.path.isabs(path) and os.path.exists(path) else ""
