"""Build-time guards on the generated gfx950 code (no GPU needed).

The product kernels keep 256 int32/fp32 accumulators per lane in registers;
if the compiler ever demotes them to scratch memory (for instance when an
epilogue path grows enough to stop the unrolling that keeps their indices
constant), the kernels still compute the right result but run several times
slower. The code-object metadata shows it as a large private segment.
"""

import os
import re
import subprocess


ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = os.path.join(ROOT, "int8_quantized_matmul_amd", "csrc", "gemm_kernels.hip")


def _kernel_metadata():
    from int8_quantized_matmul_amd import build
    flags = [f for f in build.HIP_FLAGS if f != "-fPIC"]
    out = subprocess.run([build._hipcc(), *flags, "--cuda-device-only", "-S", "-o", "-", SRC],
                         capture_output=True, text=True, check=True).stdout
    meta = {}
    for block in re.split(r"\n\s+- \.", out):
        name = re.search(r"\.name:\s+(\S+)", block)
        priv = re.search(r"\.private_segment_fixed_size:\s+(\d+)", block)
        if name and priv:
            meta[name.group(1)] = int(priv.group(1))
    return meta


def test_product_kernels_keep_accumulators_in_registers():
    meta = _kernel_metadata()
    gemm = {k: v for k, v in meta.items() if "k_gemm_prefill" in k or "k_gemm_decode" in k}
    assert len(gemm) >= 5, sorted(meta)
    big = {k: v for k, v in gemm.items() if v > 128}
    assert not big, f"kernels with scratch-resident arrays: {big}"
