"""Resource checks on the compiled grouped-GEMM kernels (CPU only: hipcc emits
the gfx950 assembly here).

The GEMM's LDS-DMA pipeline waits on the vector-memory counter with counts
that assume the kernel issues no vector-memory operations other than its own
operand loads.  Register spills to scratch are such operations (scratch
stores, which may complete out of order with the loads), so every k_gemm
instantiation must compile without scratch.
"""
import os
import re
import subprocess
import tempfile

import pytest

from block_scaled_precision_token_amd import build

HIPCC = build.HIPCC


def _kernel_meta(asm: str):
    """{kernel name: {field: int}} from the AMDGPU metadata block."""
    meta = {}
    cur = None
    for line in asm.splitlines():
        m = re.match(r"\s+\.name:\s+(\S+)", line)
        if m:
            cur = m.group(1)
            meta[cur] = {}
            continue
        m = re.match(r"\s+\.(private_segment_fixed_size|vgpr_spill_count|sgpr_spill_count|vgpr_count):\s+(\d+)",
                     line)
        if m and cur:
            meta[cur][m.group(1)] = int(m.group(2))
    return meta


@pytest.mark.skipif(not os.path.exists(HIPCC), reason="hipcc not available")
def test_gemm_kernels_use_no_scratch():
    src = os.path.join(build.CSRC, "bsp_gemm.hip")
    with tempfile.TemporaryDirectory() as td:
        out = os.path.join(td, "gemm.s")
        cmd = [HIPCC, *build.COMMON, *build.DEVICE, "--cuda-device-only", "-S", src, "-o", out]
        res = subprocess.run(cmd, capture_output=True, text=True)
        assert res.returncode == 0, res.stderr[-2000:]
        with open(out) as f:
            asm = f.read()
    meta = _kernel_meta(asm)
    gemm = {k: v for k, v in meta.items() if "k_gemm" in k}
    assert len(gemm) >= 8, sorted(meta)
    for name, m in gemm.items():
        assert m.get("private_segment_fixed_size", 0) == 0, (name, m)
        assert m.get("vgpr_spill_count", 0) == 0, (name, m)
    assert "scratch_" not in asm
