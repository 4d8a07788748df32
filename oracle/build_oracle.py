"""Compile the float64 CPU oracle (test infrastructure only) into liboracle.so.

Plain gcc, -O2 with OpenMP; no -ffast-math, so libm exp/log and IEEE float64
arithmetic are used exactly as written.
"""
import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "oracle_attn.c")
LIB = os.path.join(HERE, "liboracle.so")


def build(verbose: bool = False, sanitize_dir: str = None) -> str:
    """Build liboracle.so; with sanitize_dir, build instead a copy with
    AddressSanitizer and UndefinedBehaviorSanitizer into that folder (for the
    CPU sanitizer tests; load it with gcc's libasan preloaded)."""
    out = LIB
    extra = []
    if sanitize_dir:
        os.makedirs(sanitize_dir, exist_ok=True)
        out = os.path.join(sanitize_dir, "liboracle_asan.so")
        extra = ["-g", "-fsanitize=address,undefined", "-fno-sanitize-recover=undefined",
                 "-fno-omit-frame-pointer"]
    cmd = ["gcc", "-O2", "-fopenmp", "-fPIC", "-shared", "-std=c99",
           "-Wall", "-Wextra", *extra, "-o", out + ".tmp", SRC, "-lm"]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(out + ".tmp", out)
    return out


if __name__ == "__main__":
    print(build(verbose=True))
