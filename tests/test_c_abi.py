"""The C ABI from C: tests/c/abi_host.c includes include/decode_attn.h as a
C99 translation unit (-Wall -Wextra -Werror), links the built library and
calls its host-only entry points and argument checks (no GPU needed)."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
PKG = os.path.join(ROOT, "decode_attention_paged_gqa_amd")
LIB = os.path.join(PKG, "libdecode_attn.so")


@pytest.mark.skipif(shutil.which("gcc") is None, reason="no C compiler")
def test_c99_caller_builds_links_and_runs(tmp_path):
    if not os.path.exists(LIB):
        pytest.fail("libdecode_attn.so is not built (run __graft_entry__.build())")
    exe = str(tmp_path / "abi_host")
    rocm_lib = "/opt/rocm/lib"
    cmd = ["gcc", "-std=c99", "-Wall", "-Wextra", "-Werror", "-I", os.path.join(ROOT, "include"),
           os.path.join(ROOT, "tests", "c", "abi_host.c"), "-o", exe, "-L", PKG, "-ldecode_attn",
           f"-Wl,-rpath,{PKG}", f"-Wl,-rpath-link,{rocm_lib}", f"-Wl,-rpath,{rocm_lib}"]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr
    r = subprocess.run([exe], capture_output=True, text=True, timeout=120)
    assert r.returncode == 0 and r.stdout.strip() == "ok", r.stdout + r.stderr
