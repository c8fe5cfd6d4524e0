"""Host-sanitizer build of libtq for CPU tests.

The host C++ sources (argument checks, parameter construction, dispatch)
are compiled with AddressSanitizer and UndefinedBehaviorSanitizer for the
host only; the device objects come from the ordinary build (``_build.py``)
unchanged.  The result is linked into ``_build/sanitize/libtq.so`` against
the shared sanitizer runtime, which a Python process must preload
(``runtime()``); the package loads the library named by ``TQ_LIBRARY``.
"""
import glob
import os
import subprocess

from . import _build

OUT = os.path.join(_build.ROOT, "_build", "sanitize")
LIB = os.path.join(OUT, "libtq.so")
# each sanitizer flag applies to the host pass only
SAN = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined"]
HOST = ["-O1", "-g", "-fPIC", "-std=c++17", "-fno-omit-frame-pointer", "-I", os.path.join(_build.ROOT, "include")]


def runtime():
    """Path of clang's shared ASan runtime (UBSan included), or None."""
    root = os.path.dirname(os.path.dirname(os.path.realpath(_build.hipcc())))
    hits = sorted(glob.glob(os.path.join(root, "lib", "llvm", "lib", "clang", "*", "lib", "linux",
                                         "libclang_rt.asan-x86_64.so")))
    return hits[-1] if hits else None


def build():
    """Compile the host sources with the sanitizers and link them with the
    ordinary device objects (built first).  Returns the library path."""
    _build.build()
    os.makedirs(OUT, exist_ok=True)
    objs = []
    for src in _build.sources():
        if src.endswith(".hip"):
            objs.append(os.path.join(_build.OBJDIR, os.path.basename(src) + ".o"))
            continue
        obj = os.path.join(OUT, os.path.basename(src) + ".o")
        cmd = [_build.hipcc()] + HOST + SAN + ["-c", src, "-o", obj]
        res = subprocess.run(cmd, capture_output=True, text=True)
        if res.returncode != 0:
            raise RuntimeError(f"compile failed: {' '.join(cmd)}\n{res.stdout}\n{res.stderr}")
        objs.append(obj)
    cmd = ([_build.hipcc(), "-shared", "-fPIC", f"--offload-arch={_build.ARCH}"] + SAN + ["-shared-libsan", "-o", LIB]
           + objs + ["-lpthread"])
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"link failed: {' '.join(cmd)}\n{res.stdout}\n{res.stderr}")
    return LIB
