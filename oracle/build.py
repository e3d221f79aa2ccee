"""Builds the CPU oracle shared library (test infrastructure only).

Plain gcc, no fast-math (which would flush denormals) and no FMA contraction,
so every fp32 step is one correctly rounded IEEE operation.
"""
import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "sq_oracle.c")
LIB = os.path.join(HERE, "liboracle.so")


def build(verbose: bool = False) -> str:
    cmd = ["gcc", "-std=c99", "-O2", "-fopenmp", "-ffp-contract=off", "-fno-fast-math",
           "-fPIC", "-shared", "-Wall", "-Wextra", "-o", LIB + ".tmp", SRC, "-lm"]
    if verbose:
        print(" ".join(cmd))
    subprocess.run(cmd, check=True)
    os.replace(LIB + ".tmp", LIB)
    return LIB


def build_sanitized(out_dir: str) -> str:
    """The oracle with AddressSanitizer and UndefinedBehaviorSanitizer (any report is
    fatal); load it with gcc's libasan preloaded (asan_runtime())."""
    os.makedirs(out_dir, exist_ok=True)
    lib = os.path.join(out_dir, "liboracle_sanitized.so")
    cmd = ["gcc", "-std=c99", "-O1", "-g", "-fno-omit-frame-pointer", "-fsanitize=address,undefined",
           "-fno-sanitize-recover=undefined", "-fopenmp", "-ffp-contract=off", "-fno-fast-math",
           "-fPIC", "-shared", "-o", lib, SRC, "-lm"]
    subprocess.run(cmd, check=True)
    return lib


def asan_runtime() -> str:
    return subprocess.run(["gcc", "-print-file-name=libasan.so"], capture_output=True, text=True,
                          check=True).stdout.strip()


if __name__ == "__main__":
    print(build(verbose=True))
