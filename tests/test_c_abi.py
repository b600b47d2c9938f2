"""include/ring_attn.h is a C ABI: a C99 program (tests/c_abi_check.c), built
with gcc -std=c99 -pedantic -Werror against the header and linked to
libringattn.so, runs the host-only calls and the device calls' argument checks
(which return before any device work, so no GPU is needed)."""
import os
import shutil
import subprocess

import pytest

from ring_attention_attn_amd import binding as B

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.mark.skipif(shutil.which("gcc") is None, reason="no gcc")
@pytest.mark.skipif(not os.path.exists(B.LIB_PATH), reason="libringattn.so not built")
def test_header_is_a_c_abi(tmp_path):
    libdir = os.path.dirname(B.LIB_PATH)
    exe = str(tmp_path / "c_abi_check")
    rocm_lib = os.path.join(os.environ.get("ROCM_PATH", "/opt/rocm"), "lib")
    cmd = ["gcc", "-std=c99", "-Wall", "-Wextra", "-Werror", "-pedantic",
           "-I", os.path.join(ROOT, "include"), os.path.join(ROOT, "tests", "c_abi_check.c"),
           "-L", libdir, "-lringattn", f"-Wl,-rpath,{libdir}", f"-Wl,-rpath,{rocm_lib}",
           f"-Wl,-rpath-link,{rocm_lib}", "-o", exe]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stdout + r.stderr
    r = subprocess.run([exe], capture_output=True, text=True, timeout=120)
    assert r.returncode == 0 and r.stdout.strip() == "ok", r.stdout + r.stderr
