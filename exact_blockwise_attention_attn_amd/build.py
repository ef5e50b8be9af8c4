"""Build libattn.so (HIP for gfx950) in-tree with hipcc.

    python -m exact_blockwise_attention_attn_amd.build [--verbose] [--host-asan]

Every source is compiled to an object under ``_build/`` in parallel, then
linked into ``exact_blockwise_attention_attn_amd/libattn.so`` (replaced
atomically).  Packed fp32 VALU instructions are disabled for all device code.

``--host-asan`` instead builds ``_build/libattn_host_asan.so``, with the host
code of the C ABI (argument validation, table building) under AddressSanitizer
and the device code unchanged.  The host tests run against it with

    ATTN_LIBRARY=<that path> LD_PRELOAD=<hipcc -print-file-name=libclang_rt.asan-x86_64.so> \
        ASAN_OPTIONS=detect_leaks=0 python -m pytest tests/test_abi_host.py
"""

from __future__ import annotations

import argparse
import concurrent.futures as cf
import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
BUILD_DIR = os.path.join(PKG, "_build")
LIB_PATH = os.path.join(PKG, "libattn.so")
HOST_ASAN_LIB_PATH = os.path.join(BUILD_DIR, "libattn_host_asan.so")
# A plain C program that drives the library through its C ABI (examples/c_forward.c).
C_EXAMPLE_SRC = os.path.join(PKG, "examples", "c_forward.c")
C_EXAMPLE_PATH = os.path.join(PKG, "bin", "c_forward")
ROCM = os.environ.get("ROCM_PATH", "/opt/rocm")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"

SOURCES = [
    "abi.hip",
    "fwd_bf16.hip",
    "fwd_f32.hip",
    "merge.hip",
    "bwd_bf16.hip",
    "bwd_f32.hip",
    "decode.hip",
    "check.hip",
]

COMMON_FLAGS = [
    f"--offload-arch={ARCH}",
    "-O3",
    "-std=c++17",
    "-fPIC",
    "-fvisibility=hidden",
    "-I", os.path.join(ROOT, "include"),
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
]


# Host-only AddressSanitizer for the C ABI's host code (each sanitizer flag
# applies to the host pass only, never to device code).
HOST_ASAN_FLAGS = "-Xarch_host -fsanitize=address -Xarch_host -fno-omit-frame-pointer".split()


def _compile(src: str, verbose: bool, extra=(), out_dir: str = BUILD_DIR) -> str:
    obj = os.path.join(out_dir, os.path.splitext(src)[0] + ".o")
    cmd = [HIPCC, *COMMON_FLAGS, *extra, "-c", os.path.join(CSRC, src), "-o", obj]
    if verbose:
        cmd += ["-Rpass-analysis=kernel-resource-usage"]
    res = subprocess.run(cmd, capture_output=True, text=True)
    # The host pass does not know the packed-fp32 target feature; that warning is expected.
    noise = "'-packed-fp32-ops' is not a recognized feature"
    msgs = "\n".join(l for l in (res.stdout + res.stderr).splitlines() if noise not in l)
    if res.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{msgs}")
    if verbose and msgs.strip():
        print(f"--- {src}\n{msgs}", file=sys.stderr)
    return obj


def build(verbose: bool = False, jobs: int | None = None) -> str:
    """Compile and link libattn.so; returns its path.  Raises on any compiler error."""
    os.makedirs(BUILD_DIR, exist_ok=True)
    jobs = jobs or min(len(SOURCES), os.cpu_count() or 4, 16)
    with cf.ThreadPoolExecutor(jobs) as ex:
        objs = list(ex.map(lambda s: _compile(s, verbose), SOURCES))
    tmp = LIB_PATH + ".tmp"
    cmd = [HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"link failed:\n{res.stdout}\n{res.stderr}")
    os.replace(tmp, LIB_PATH)
    build_c_example()
    return LIB_PATH


def build_c_example() -> str:
    """Compile examples/c_forward.c with the system C compiler against include/attn.h, the HIP runtime
    and the in-tree libattn.so (found next to the binary's directory at run time)."""
    os.makedirs(os.path.dirname(C_EXAMPLE_PATH), exist_ok=True)
    cmd = ["gcc", "-std=c11", "-O2", "-Wall", "-Wextra", "-Werror", "-D__HIP_PLATFORM_AMD__",
           "-I", os.path.join(ROCM, "include"), "-I", os.path.join(ROOT, "include"), C_EXAMPLE_SRC,
           "-o", C_EXAMPLE_PATH, "-L", PKG, "-lattn", "-L", os.path.join(ROCM, "lib"), "-lamdhip64",
           "-Wl,-rpath,$ORIGIN/..", "-Wl,-rpath," + os.path.join(ROCM, "lib")]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"C example build failed:\n{res.stdout}\n{res.stderr}")
    return C_EXAMPLE_PATH


def build_host_asan(jobs: int | None = None) -> str:
    """Build _build/libattn_host_asan.so: abi.hip's host code under AddressSanitizer, every
    other object as in build().  Returns its path."""
    out_dir = os.path.join(BUILD_DIR, "host_asan")
    os.makedirs(out_dir, exist_ok=True)
    jobs = jobs or min(len(SOURCES), os.cpu_count() or 4, 16)
    with cf.ThreadPoolExecutor(jobs) as ex:
        objs = list(ex.map(lambda s: _compile(s, False, HOST_ASAN_FLAGS if s == "abi.hip" else (), out_dir),
                           SOURCES))
    cmd = [HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-shared-libasan", *HOST_ASAN_FLAGS[:2], *objs,
           "-o", HOST_ASAN_LIB_PATH]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"link failed:\n{res.stdout}\n{res.stderr}")
    return HOST_ASAN_LIB_PATH


def resource_usage(sources=None) -> dict:
    """Per-kernel register, scratch and LDS use as the compiler reports it.

    Compiles each source (default: all) to a throw-away object with the
    library's flags plus -Rpass-analysis=kernel-resource-usage and returns
    {mangled kernel name: {"VGPRs": .., "AGPRs": .., "ScratchSize": .., "VGPRs Spill": ..,
    "SGPRs Spill": .., "Occupancy": .., "LDS Size": ..}}.  The in-tree library is
    not touched.
    """
    import re
    import tempfile

    out = {}
    with tempfile.TemporaryDirectory() as tmp:
        def one(src):
            obj = os.path.join(tmp, os.path.splitext(src)[0] + ".o")
            cmd = [HIPCC, *COMMON_FLAGS, "-Rpass-analysis=kernel-resource-usage", "-c", os.path.join(CSRC, src),
                   "-o", obj]
            res = subprocess.run(cmd, capture_output=True, text=True)
            if res.returncode != 0:
                raise RuntimeError(f"hipcc failed for {src}:\n{res.stderr[-4000:]}")
            return res.stdout + res.stderr

        with cf.ThreadPoolExecutor(min(16, os.cpu_count() or 4)) as ex:
            texts = list(ex.map(one, sources or SOURCES))
    for text in texts:
        cur = None
        for line in text.splitlines():
            m = re.search(r"remark: Function Name: (\S+)", line)
            if m:
                cur = out.setdefault(m.group(1), {})
                continue
            m = re.search(r"remark: ([A-Za-z ]+?)(?: \[[^\]]*\])?: (\d+)", line)
            if m and cur is not None:
                cur[m.group(1).strip()] = int(m.group(2))
    return out


def main() -> None:
    ap = argparse.ArgumentParser(description=__doc__)
    ap.add_argument("--verbose", action="store_true", help="print kernel register/LDS usage")
    ap.add_argument("--host-asan", action="store_true", help="build the host-AddressSanitizer library instead")
    args = ap.parse_args()
    print(build_host_asan() if args.host_asan else build(verbose=args.verbose))


if __name__ == "__main__":
    main()
