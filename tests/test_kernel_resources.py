"""Resource budget of every gfx950 kernel, read from the assembler metadata of
the library's own sources compiled with the library's flags (no GPU needed):
no kernel spills registers to scratch memory, none uses scratch at all, and
each fits one CU's LDS (160 KiB). The step kernels are tuned at one
workgroup of 512 threads per CU, two waves per SIMD: a spill or an LDS
overflow would either slow them by a large factor or fail at launch."""
import os
import re
import shutil
import subprocess

import pytest

from ring_attention_attn_amd import build as B

LDS_PER_CU = 160 * 1024


def _device_asm(src, tmp_path):
    out = tmp_path / (os.path.basename(src) + ".s")
    cmd = [B.HIPCC] + list(B.CFLAGS) + ["--cuda-device-only", "-S", src, "-o", str(out)]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-2000:]
    return out.read_text()


def _kernels(asm):
    """(name, metadata dict) for each kernel in the AMDGPU metadata block."""
    meta = asm[asm.index("amdhsa.kernels:"):]
    out = []
    for block in re.split(r"\n  - ", meta)[1:]:
        name = re.search(r"\.name:\s+(\S+)", block)
        vals = dict(re.findall(r"\.(\w+):\s+(\d+)\s*$", block, re.M))
        if name:
            out.append((name.group(1), {k: int(v) for k, v in vals.items()}))
    return out


@pytest.mark.skipif(shutil.which(B.HIPCC) is None and not os.path.exists(B.HIPCC),
                    reason="hipcc not available")
@pytest.mark.parametrize("src", B.sources(), ids=os.path.basename)
def test_kernel_resources(src, tmp_path):
    text = open(src).read()
    ks = _kernels(_device_asm(src, tmp_path))
    if "__global__" not in text:
        assert not ks
        return
    assert ks, "no kernel metadata found"
    for k in ("fwd_mfma_kernel", "bwd_dq_kernel", "bwd_dkv_kernel"):  # the parser sees them
        if f"void {k}(" in text:
            assert any(k in name for name, _ in ks), k
    for name, m in ks:
        assert m.get("vgpr_spill_count", 0) == 0, (name, m)
        assert m.get("sgpr_spill_count", 0) == 0, (name, m)
        assert m.get("private_segment_fixed_size", 0) == 0, (name, m)
        assert m.get("group_segment_fixed_size", 0) <= LDS_PER_CU, (name, m)
        # 512 unified registers per SIMD lane: the 512-thread step kernels run
        # two waves per SIMD, so each wave may hold at most 256
        if m.get("max_flat_workgroup_size", 0) >= 512:
            assert m.get("vgpr_count", 0) + m.get("agpr_count", 0) <= 256, (name, m)
