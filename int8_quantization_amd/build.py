"""Builds libsq.so (gfx950) in-tree with hipcc.

Flags:
  --offload-arch=gfx950          CDNA4 only
  -ffp-contract=off              no FMA contraction: the dequant epilogue keeps
                                 its three separate fp32 roundings
  -packed-fp32-ops disabled      hipcc must not form v_pk_{add,mul,fma}_f32
IEEE fp32 division and denormals stay on (HIP's defaults); no fast-math.
"""
import concurrent.futures as cf
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
BUILD = os.path.join(os.path.dirname(HERE), "_build")
LIB = os.path.join(HERE, "libsq.so")
SOURCES = ["sq_api.hip", "quant.hip", "quant_stream.hip", "gemm.hip", "gemv.hip", "outlier.hip", "lnquant.hip",
           "static.hip", "kvcache.hip"]
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

FLAGS = [
    "--offload-arch=gfx950", "-O3", "-fPIC", "-std=c++17", "-ffp-contract=off",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-function", "-Wno-unused-variable",
]


def _compile(src: str) -> str:
    obj = os.path.join(BUILD, src.replace(".hip", ".o"))
    cmd = [HIPCC, *FLAGS, "-c", os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    out = "\n".join(l for l in (r.stdout + r.stderr).splitlines()
                    if "packed-fp32-ops" not in l)   # host pass does not know the feature
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{out}")
    if out.strip():
        sys.stderr.write(out + "\n")
    return obj


def device_asm(src: str) -> str:
    """gfx950 assembly of one source, with the library's flags (for ISA checks)."""
    cmd = [HIPCC, *FLAGS, "--cuda-device-only", "-S", "-o", "-", os.path.join(CSRC, src)]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc -S failed for {src}:\n{r.stderr}")
    return r.stdout


def build(verbose: bool = False) -> str:
    os.makedirs(BUILD, exist_ok=True)
    jobs = min(len(SOURCES), max(1, (os.cpu_count() or 4)))
    with cf.ThreadPoolExecutor(jobs) as ex:
        objs = list(ex.map(_compile, SOURCES))
    cmd = [HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", "-o", LIB + ".tmp", *objs]
    subprocess.run(cmd, check=True)
    os.replace(LIB + ".tmp", LIB)
    if verbose:
        print(LIB)
    return LIB


def build_host_sanitized(out_dir: str) -> str:
    """The same library with AddressSanitizer and UndefinedBehaviorSanitizer on its host
    code only (argument validation, dispatch); the gfx950 device code is built as usual.
    Load it with clang's ASan runtime preloaded (host_asan_runtime())."""
    os.makedirs(out_dir, exist_ok=True)
    san = ["-O1", "-g", "-Xarch_host", "-fsanitize=address,undefined", "-Xarch_host", "-fno-omit-frame-pointer"]
    flags = [f for f in FLAGS if f != "-O3"] + san

    def one(src):
        obj = os.path.join(out_dir, src.replace(".hip", ".o"))
        r = subprocess.run([HIPCC, *flags, "-c", os.path.join(CSRC, src), "-o", obj], capture_output=True, text=True)
        if r.returncode != 0:
            raise RuntimeError(f"hipcc failed for {src}:\n{r.stderr}")
        return obj

    with cf.ThreadPoolExecutor(min(len(SOURCES), max(1, os.cpu_count() or 4))) as ex:
        objs = list(ex.map(one, SOURCES))
    lib = os.path.join(out_dir, "libsq_host_sanitized.so")
    subprocess.run([HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", "-shared-libasan",
                    "-Xarch_host", "-fsanitize=address,undefined", "-o", lib, *objs], check=True)
    return lib


def host_asan_runtime() -> str:
    """clang's shared ASan runtime (it carries the UBSan handlers too)."""
    import glob
    found = sorted(glob.glob(os.path.join(os.path.dirname(os.path.dirname(HIPCC)), "llvm", "lib", "clang", "*",
                                          "lib", "linux", "libclang_rt.asan-x86_64.so")))
    if not found:
        raise FileNotFoundError("libclang_rt.asan-x86_64.so not found under the ROCm LLVM")
    return found[-1]


if __name__ == "__main__":
    build(verbose=True)
