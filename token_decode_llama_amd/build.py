"""Builds liblmdecode.so (gfx950) in-tree with hipcc."""
from __future__ import annotations

import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
LIB_PATH = os.path.join(HERE, "liblmdecode.so")

SOURCES = ["lm_kernels.hip", "lm_runtime.cpp"]

HIPCC_FLAGS = [
    "--offload-arch=gfx950",
    "-O3",
    "-std=c++17",
    "-fPIC",
    "-shared",
    # packed fp32 ops stay off: the compiler must not form v_pk_*_f32
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall",
    "-Wno-unused-function",
]


def hipcc() -> str:
    for p in ("/opt/rocm/bin/hipcc", "hipcc"):
        if os.path.sep not in p or os.path.exists(p):
            return p
    return "hipcc"


def build(verbose: bool = False, out: str = LIB_PATH, defines=()) -> str:
    """Compiles every source to an object in parallel, then links the library.
    defines: extra -D flags (compile-time tuning knobs), for experiments."""
    from concurrent.futures import ThreadPoolExecutor
    import tempfile
    flags = [f for f in HIPCC_FLAGS if f != "-shared"] + [f"-D{d}" for d in defines]
    with tempfile.TemporaryDirectory(prefix="lmdecode_build_") as tmpdir:
        objs = [os.path.join(tmpdir, s + ".o") for s in SOURCES]
        cmds = [[hipcc(), *flags, "-c", "-o", o, os.path.join(CSRC, s)] for s, o in zip(SOURCES, objs)]
        if verbose:
            for c in cmds:
                print(" ".join(c), flush=True)
        with ThreadPoolExecutor(max_workers=len(cmds)) as ex:
            results = list(ex.map(lambda c: subprocess.run(c, capture_output=True, text=True), cmds))
        for res in results:
            if res.returncode != 0:
                raise RuntimeError("hipcc failed:\n" + res.stdout + res.stderr)
        tmp = out + ".tmp"
        link = [hipcc(), "--offload-arch=gfx950", "-shared", "-fPIC", "-o", tmp, *objs]
        res = subprocess.run(link, capture_output=True, text=True)
        if res.returncode != 0:
            raise RuntimeError("link failed:\n" + res.stdout + res.stderr)
    os.replace(tmp, out)
    return out


if __name__ == "__main__":
    print(build(verbose=True))
