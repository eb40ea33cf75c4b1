"""Build libdecode_attn.so in-tree with hipcc for gfx950.

    python -m decode_attention_paged_gqa_amd.build [--checked | --asan]

Every source under csrc/ is compiled to an object in parallel, then linked
into ``decode_attention_paged_gqa_amd/libdecode_attn.so``.  With --checked
the same sources are built with -DDA_CHECKED into libdecode_attn_checked.so,
whose kernels also record violations of the device-data contract
(decode_attn_checks).  With --asan the host code (argument validation,
dispatch, the host-only entry points) is built with AddressSanitizer into
libdecode_attn_asan.so; the GPU code is compiled as usual, unsanitised.  A
process using it must load the sanitizer runtime first (an executable linked
with -fsanitize=address, or LD_PRELOAD of asan_runtime()).  Always rebuilds.
"""
from __future__ import annotations

import os
import shutil
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD = os.path.join(PKG, "_build")
LIB = os.path.join(PKG, "libdecode_attn.so")
CHECKED_LIB = os.path.join(PKG, "libdecode_attn_checked.so")
ASAN_LIB = os.path.join(PKG, "libdecode_attn_asan.so")
# host-side AddressSanitizer: every -fsanitize flag applies to host code only
ASAN_FLAGS = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fno-omit-frame-pointer"]
ARCH = "gfx950"


def hipcc() -> str:
    for c in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if c and os.path.exists(c):
            return c
    raise RuntimeError("hipcc not found")


COMMON_FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC",
    # keep the compiler from forming packed fp32 (v_pk_*_f32) instructions
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-I", INCLUDE, "-I", CSRC,
    "-Wno-unused-command-line-argument",
]


def sources():
    return sorted(os.path.join(CSRC, f) for f in os.listdir(CSRC)
                  if f.endswith((".hip", ".cpp")))


def _compile(src: str, extra, build_dir: str) -> str:
    obj = os.path.join(build_dir, os.path.basename(src) + ".o")
    cmd = [hipcc()] + COMMON_FLAGS + list(extra) + ["-c", src, "-o", obj]
    if src.endswith(".cpp"):
        cmd[1:1] = ["-x", "hip"]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{r.stderr[-6000:]}")
    return obj


def asan_runtime() -> str:
    """The clang AddressSanitizer runtime that goes with hipcc's compiler."""
    llvm = os.path.join(os.path.dirname(os.path.realpath(hipcc())), "..", "llvm")
    for root in (os.path.join(llvm, "lib", "clang"), "/opt/rocm/llvm/lib/clang"):
        if os.path.isdir(root):
            for ver in sorted(os.listdir(root), reverse=True):
                p = os.path.join(root, ver, "lib", "linux", "libclang_rt.asan-x86_64.so")
                if os.path.exists(p):
                    return os.path.realpath(p)
    raise RuntimeError("clang AddressSanitizer runtime not found")


def build(extra_flags=(), verbose=True, jobs=None, checked=False, asan=False) -> str:
    if checked and asan:
        raise ValueError("one variant at a time")
    lib = CHECKED_LIB if checked else ASAN_LIB if asan else LIB
    build_dir = BUILD + ("_checked" if checked else "_asan" if asan else "")
    extra = list(extra_flags) + (["-DDA_CHECKED"] if checked else []) + (ASAN_FLAGS if asan else [])
    os.makedirs(build_dir, exist_ok=True)
    srcs = sources()
    jobs = jobs or min(len(srcs), max(1, min(8, os.cpu_count() or 1)))
    with ThreadPoolExecutor(max_workers=jobs) as ex:
        objs = list(ex.map(lambda s: _compile(s, extra, build_dir), srcs))
    tmp = lib + ".tmp"
    cmd = [hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp] + objs
    if asan:  # sanitizer symbols resolve against the runtime the process loaded first
        cmd += ["-Xarch_host", "-fsanitize=address", "-shared-libsan"]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stderr[-4000:]}")
    os.replace(tmp, lib)
    if verbose:
        print(f"built {lib} from {len(srcs)} sources", flush=True)
    return lib


if __name__ == "__main__":
    args = sys.argv[1:]
    build([a for a in args if a not in ("--checked", "--asan")], checked="--checked" in args,
          asan="--asan" in args)
