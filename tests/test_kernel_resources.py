"""Register budgets of the streaming kernels, checked on the compiled gfx950 code.

The GEMV and GEMM kernels are sized so that their operand rings live in
registers at the occupancy each launch assumes (the launch bounds' second
value is waves per SIMD).  A kernel that spills to scratch still computes
the right values but streams at a fraction of the rate, which no parity
test notices; this compiles the device code (no GPU needed) and reads the
kernel descriptors instead.
"""
from __future__ import annotations

import os
import re
import shutil
import subprocess
from concurrent.futures import ThreadPoolExecutor

import pytest

from weight_only_quantization_quantize_amd import build as woq_build

HIPCC = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
pytestmark = pytest.mark.skipif(not os.path.exists(HIPCC), reason="hipcc not available")

# source file -> kernel name prefix (mangled) whose every instance must not spill
FILES = {
    "gemv.hip": "gemv_kernel",
    "gemm_mid.hip": "gemm_mid_kernel",
    "gemm_regb.hip": "gemm_regb_kernel",
    "quantize_pack.hip": "quantize_pack",
}


def _descriptors(src: str, tmp: str) -> dict[str, dict[str, int]]:
    out = os.path.join(tmp, os.path.basename(src) + ".s")
    cmd = [HIPCC, "-x", "hip", *woq_build.COMMON_FLAGS, "--cuda-device-only", "-S", src, "-o", out]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-2000:]
    text = open(out).read()
    kernels = {}
    for m in re.finditer(r"\.amdhsa_kernel (\S+)\n(.*?)\.end_amdhsa_kernel", text, re.S):
        fields = dict(re.findall(r"\.amdhsa_(\w+) (-?\d+)", m.group(2)))
        kernels[m.group(1)] = {k: int(v) for k, v in fields.items()}
    return kernels


@pytest.fixture(scope="module")
def descriptors(tmp_path_factory):
    tmp = str(tmp_path_factory.mktemp("asm"))
    srcs = [os.path.join(woq_build.CSRC, f) for f in FILES]
    with ThreadPoolExecutor(max_workers=len(srcs)) as ex:
        results = list(ex.map(lambda s: _descriptors(s, tmp), srcs))
    return dict(zip(FILES, results))


@pytest.mark.parametrize("src", sorted(FILES))
def test_streaming_kernels_do_not_spill(descriptors, src):
    kernels = {k: v for k, v in descriptors[src].items() if FILES[src] in k}
    assert kernels, f"no {FILES[src]} instance found in {src}"
    spilling = {k: v["private_segment_fixed_size"] for k, v in kernels.items() if v["private_segment_fixed_size"]}
    assert not spilling, spilling


def test_mid_m_two_workgroup_instances_fit_128_vgprs(descriptors):
    # Template argument 4 of gemm_mid_kernel is the ring depth: 3 is the
    # instance launched with two 8-wave workgroups per compute unit.
    ring3 = {k: v for k, v in descriptors["gemm_mid.hip"].items() if re.search(r"ELi[012]ELi3ELb[01]E", k)}
    assert ring3
    for name, d in ring3.items():
        assert d["next_free_vgpr"] <= 128, (name, d["next_free_vgpr"])
