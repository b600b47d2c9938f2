"""The library's host code under AddressSanitizer (opt-in: RA_HOST_ASAN=1;
it rebuilds the library, about a minute). The HIP sources are compiled with
-fsanitize=address on the host side only (-Xarch_host; device code is not
instrumented), and the C99 checker (tests/c_abi_check.c) and the ABI tests
(tests/test_abi.py: argument checks, index maps, chunk marshalling) run
against that build with the sanitizer's runtime preloaded. No GPU is used."""
import glob
import os
import subprocess
import sys
import tempfile

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
ROCM = os.environ.get("ROCM_PATH", "/opt/rocm")

pytestmark = pytest.mark.skipif(os.environ.get("RA_HOST_ASAN") != "1",
                                reason="opt-in: set RA_HOST_ASAN=1")


def test_host_code_under_asan(tmp_path):
    sys.path.insert(0, ROOT)
    from ring_attention_attn_amd import build as b
    objs_dir = tempfile.mkdtemp(prefix="ra_asan_", dir=str(tmp_path))
    objs = [b._compile(s, False, objs_dir, ("-Xarch_host", "-fsanitize=address",
                                            "-Xarch_host", "-fno-omit-frame-pointer"))
            for s in b.sources()]
    lib = str(tmp_path / "libringattn.so")
    r = subprocess.run([b.HIPCC, f"--offload-arch={b.ARCH}", "-shared", "-fPIC", "-o", lib] + objs +
                       ["-Xarch_host", "-fsanitize=address", "-shared-libasan"],
                       capture_output=True, text=True)
    assert r.returncode == 0, r.stderr
    rt = glob.glob(os.path.join(ROCM, "llvm/lib/clang/*/lib/linux/libclang_rt.asan-x86_64.so"))
    assert rt, "ASan runtime not found"
    env = dict(os.environ, LD_PRELOAD=rt[0], ASAN_OPTIONS="detect_leaks=0")
    # the C99 checker, built with the same compiler's sanitizer runtime
    exe = str(tmp_path / "c_abi_check")
    r = subprocess.run([os.path.join(ROCM, "llvm/bin/clang"), "-std=c99", "-Wall", "-Werror",
                        "-fsanitize=address", "-shared-libasan", "-I", os.path.join(ROOT, "include"),
                        os.path.join(ROOT, "tests", "c_abi_check.c"), lib,
                        f"-Wl,-rpath,{os.path.join(ROCM, 'lib')}", "-o", exe],
                       capture_output=True, text=True)
    assert r.returncode == 0, r.stderr
    r = subprocess.run([exe], capture_output=True, text=True, env=env, timeout=300)
    assert r.returncode == 0 and r.stdout.strip() == "ok", r.stdout + r.stderr
    # the ABI tests through the Python binding, against the instrumented library
    code = ("import sys; sys.path.insert(0, %r)\n"
            "import ring_attention_attn_amd.binding as B\n"
            "B.LIB_PATH = %r\n"
            "import pytest\n"
            "sys.exit(pytest.main(['-q', '-p', 'no:cacheprovider', %r]))\n"
            % (ROOT, lib, os.path.join(ROOT, "tests", "test_abi.py")))
    r = subprocess.run([sys.executable, "-c", code], capture_output=True, text=True, env=env,
                       cwd=ROOT, timeout=600)
    assert r.returncode == 0 and "ERROR: AddressSanitizer" not in r.stderr, r.stdout + r.stderr
