"""Build libringattn.so (HIP, gfx950) in-tree with hipcc.

    python -m ring_attention_attn_amd.build [--verbose]

Every call recompiles all sources (no staleness heuristics): object files go to
``_build/`` at the repository root, the shared library next to this file.
"""
import concurrent.futures as cf
import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
OUT = os.path.join(PKG, "libringattn.so")
BUILD = os.path.join(ROOT, "_build")

HIPCC = os.environ.get("HIPCC", shutil.which("hipcc") or "/opt/rocm/bin/hipcc")
ARCH = "gfx950"
CFLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-fPIC", "-std=c++17", "-Wall",
    "-munsafe-fp-atomics",
    # keep MFMA accumulators in VGPRs (the AGPR form made the dK/dV kernel copy
    # its accumulators every iteration)
    "-mllvm", "-amdgpu-mfma-vgpr-form=1",
    # packed fp32 VALU ops are disabled for all device code
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-I", os.path.join(ROOT, "include"),
]


def sources(src_dir=CSRC):
    return sorted(os.path.join(src_dir, f) for f in os.listdir(src_dir) if f.endswith(".hip"))


def _compile(src, verbose, build_dir, extra, drop=()):
    obj = os.path.join(build_dir, os.path.basename(src)[:-4] + ".o")
    flags = list(CFLAGS)
    for d in drop:  # drop a flag and its argument list entry, e.g. ("-mllvm", "-amdgpu-...")
        for i in range(len(flags) - len(d) + 1):
            if tuple(flags[i:i + len(d)]) == tuple(d):
                del flags[i:i + len(d)]
                break
    cmd = [HIPCC] + flags + list(extra) + ["-c", src, "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    noise = "is not a recognized feature for this target"
    msgs = "\n".join(l for l in (r.stdout + r.stderr).splitlines() if noise not in l)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{msgs}")
    if verbose and msgs.strip():
        print(msgs)
    return obj


def build(verbose=False, out=OUT, src_dir=CSRC, build_dir=BUILD, extra_flags=(), drop_flags=()):
    """Compile every source in ``src_dir`` and link ``out``. ``extra_flags`` are
    appended to each compile (e.g. -D tile settings); ``drop_flags`` lists flag
    sequences removed from the defaults."""
    os.makedirs(build_dir, exist_ok=True)
    srcs = sources(src_dir)
    with cf.ThreadPoolExecutor(max_workers=min(8, len(srcs))) as ex:
        objs = list(ex.map(lambda s: _compile(s, verbose, build_dir, extra_flags, drop_flags),
                           srcs))
    tmp = out + ".tmp"
    # -z defs: an unresolved symbol (e.g. a kernel launch stub) fails the build
    cmd = [HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-Wl,-z,defs", "-o", tmp] + objs
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("link failed:\n" + r.stdout + r.stderr)
    os.replace(tmp, out)
    return out


if __name__ == "__main__":
    print(build(verbose="--verbose" in sys.argv))
