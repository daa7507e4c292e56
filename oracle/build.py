"""Build the CPU oracle library (plain C, gcc, OpenMP over tokens).

The oracle is test infrastructure: only the tests, the smoke check and the
benchmark's CPU-baseline leg load it.
"""
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "moe_oracle.c")
LIB = os.path.join(HERE, "liboracle.so")


def build(verbose: bool = False, src: str = SRC, lib: str = LIB) -> str:
    """Compile ``src`` (both accumulation types) into the shared library ``lib``."""
    here = os.path.dirname(lib)
    objs = []
    for tag, defs in (("f64", []), ("f32", ["-DORACLE_ACC=float", "-DORACLE_SUFFIX=f32"])):
        obj = os.path.join(here, f"_oracle_{tag}.o")
        cmd = ["gcc", "-std=c11", "-O2", "-fopenmp", "-fPIC", "-Wall", "-Wextra",
               "-c", src, "-o", obj] + defs
        if verbose:
            print(" ".join(cmd), file=sys.stderr)
        subprocess.run(cmd, check=True)
        objs.append(obj)
    tmp = lib + ".tmp"
    subprocess.run(["gcc", "-shared", "-fopenmp", "-o", tmp] + objs + ["-lm"], check=True)
    os.replace(tmp, lib)
    for o in objs:
        os.remove(o)
    return lib


def ensure_built() -> str:
    if not os.path.exists(LIB) or os.path.getmtime(LIB) < os.path.getmtime(SRC):
        build()
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
