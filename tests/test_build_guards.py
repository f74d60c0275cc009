"""Build-time guards on the generated gfx950 code (no GPU needed).

The product kernels keep 256 int32/fp32 accumulators per lane in registers;
if the compiler ever demotes them to scratch memory (for instance when an
epilogue path grows enough to stop the unrolling that keeps their indices
constant), the kernels still compute the right result but run several times
slower. The code-object metadata shows it as a large private segment.

Buffer loads and stores take their resource descriptor in scalar registers.
When the compiler cannot prove a descriptor uniform across the wavefront
(for instance when it is built from a wavefront index held in a vector
register), it wraps each such access in a loop over the distinct
descriptors: read one lane's descriptor, compare it with every lane's
(a 64-bit scalar/vector compare), run the access for the matching lanes,
repeat. The result is still right, but every access pays the loop.
"""

import functools

import os
import re
import subprocess


ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "int8_quantized_matmul_amd", "csrc")
SRC = os.path.join(CSRC, "gemm_kernels.hip")


@functools.lru_cache(maxsize=None)
def _assembly(src):
    from int8_quantized_matmul_amd import build
    flags = [f for f in build.HIP_FLAGS if f not in ("-fPIC", "-Werror")]   # hipcc adds an unused --hip-link to -S
    return subprocess.run([build._hipcc(), *flags, "--cuda-device-only", "-S", "-o", "-", src],
                          capture_output=True, text=True, check=True).stdout


def _kernel_bodies(src):
    out = _assembly(src)
    starts = [(m.start(), m.group(1)) for m in re.finditer(r"^(_Z\S+):", out, re.M)]
    bodies = {}
    for i, (pos, name) in enumerate(starts):
        end = starts[i + 1][0] if i + 1 < len(starts) else len(out)
        bodies[name] = out[pos:end].split(".Lfunc_end")[0]
    return bodies


def _kernel_metadata():
    out = _assembly(SRC)
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


# A 64-bit compare of a scalar register pair with a vector register pair: the
# test at the head of a loop over distinct buffer descriptors.
_DESCRIPTOR_LOOP = re.compile(r"v_cmp_eq_u64_e(?:32|64)\s+\S+,\s*s\[\d+:\d+\],\s*v\[\d+:\d+\]")


def test_hot_kernels_use_uniform_buffer_descriptors():
    checked = {}
    for src, pats in (("gemm_kernels.hip", ("k_gemm_prefill", "k_gemm_decode")),
                      ("quant_kernels.hip", ("k_quant_rows", "k_detect", "k_small_")),
                      ("variant_kernels.hip", ("k_quant_rows_zp",))):
        for name, body in _kernel_bodies(os.path.join(CSRC, src)).items():
            if any(p in name for p in pats):
                checked[name] = len(_DESCRIPTOR_LOOP.findall(body))
    assert len(checked) >= 20, sorted(checked)
    looped = {k: v for k, v in checked.items() if v}
    assert not looped, f"kernels with per-access descriptor loops: {looped}"
