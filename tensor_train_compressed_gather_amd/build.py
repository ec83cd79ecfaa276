"""Build libtt_emb.so (HIP for gfx950) in-tree with hipcc."""

from __future__ import annotations

import concurrent.futures as cf
import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
BUILD = os.path.join(HERE, "_build")
LIB = os.path.join(HERE, "libtt_emb.so")
SOURCES = ["api.hip", "group.hip", "forward.hip", "backward.hip", "kcores.hip", "misc.hip", "peak.hip"]
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
FLAGS = [
    "-O3", "--offload-arch=gfx950", "-fPIC", "-std=c++17",
    # packed fp32 instructions stay disabled (hipcc still emits plain fp32 FMAs)
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-I", os.path.join(ROOT, "include"),
]


def _compile(src: str) -> str:
    obj = os.path.join(BUILD, os.path.splitext(src)[0] + ".o")
    cmd = [HIPCC, *FLAGS, "-c", os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{r.stderr[-6000:]}")
    return obj


def build(verbose: bool = True) -> str:
    """Compile every HIP source and link the shared library (always rebuilds)."""
    os.makedirs(BUILD, exist_ok=True)
    with cf.ThreadPoolExecutor(max_workers=min(len(SOURCES), os.cpu_count() or 4)) as ex:
        objs = list(ex.map(_compile, SOURCES))
    tmp = LIB + f".tmp{os.getpid()}"
    cmd = [HIPCC, "-shared", "-fPIC", "--offload-arch=gfx950", "-o", tmp, *objs]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stderr[-4000:]}")
    os.replace(tmp, LIB)
    if verbose:
        print(f"built {LIB}")
    return LIB


# The host-side code of the C ABI (argument checks, the workspace plan, launch
# sequencing) built with AddressSanitizer and UndefinedBehaviorSanitizer for a
# CPU check; the sanitizers apply to the host pass only (-Xarch_host), the
# device code is the ordinary build's.
SAN_HOST = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
            "-Xarch_host", "-fno-sanitize-recover=all", "-Xarch_host", "-fno-omit-frame-pointer"]


def asan_runtime() -> str:
    """The clang AddressSanitizer runtime the host-sanitizer build links to
    (to be preloaded into a Python process that loads that build)."""
    import glob

    hits = sorted(glob.glob(os.path.join(os.path.dirname(os.path.dirname(HIPCC)), "llvm", "lib", "clang", "*",
                                         "lib", "linux", "libclang_rt.asan-x86_64.so")))
    if not hits:
        raise FileNotFoundError("libclang_rt.asan-x86_64.so not found under the ROCm LLVM")
    return hits[-1]


def build_host_sanitized(path: str) -> str:
    """libtt_emb.so with api.hip's host code under ASan + UBSan, written to path."""
    if not all(os.path.exists(os.path.join(BUILD, os.path.splitext(f)[0] + ".o")) for f in SOURCES):
        build(verbose=False)
    obj = path + ".api.o"
    cmd = [HIPCC, *FLAGS, "-O1", "-g", *SAN_HOST, "-c", os.path.join(CSRC, "api.hip"), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc (sanitized api.hip) failed:\n{r.stderr[-4000:]}")
    objs = [obj] + [os.path.join(BUILD, os.path.splitext(f)[0] + ".o") for f in SOURCES if f != "api.hip"]
    cmd = [HIPCC, "-shared", "-fPIC", "--offload-arch=gfx950", *SAN_HOST[:4], "-shared-libsan", "-o", path, *objs]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link (sanitized) failed:\n{r.stderr[-4000:]}")
    return path


if __name__ == "__main__":
    build()
