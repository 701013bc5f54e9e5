"""Compile-time resource checks of the gfx950 kernels (no GPU needed).

The attention kernels are written to run one 8-wavefront workgroup per
compute unit without private (scratch) memory: a spill or a helper left as a
real call (which puts the kernel arguments on the scratch stack) slows every
launch, and a register count above 256 would not fit two wavefronts per SIMD.
This compiles the kernel source with the resource-usage remarks of the AMDGPU
backend and checks those figures.
"""
import os
import re
import shutil
import subprocess

import pytest

from sparse_layer_reuse_amd import build as B

SRC = os.path.join(B.CSRC, "hylra_kernels.hip")


def resource_report(tmp_path, src=SRC):
    try:
        hipcc = B.hipcc()
    except RuntimeError:
        pytest.skip("hipcc not available")
    if shutil.which(hipcc) is None and not os.path.exists(hipcc):
        pytest.skip("hipcc not available")
    cmd = [hipcc, "--offload-arch=" + B.ARCH, "-O3", "-std=c++17", "-fPIC", "-c",
           "-I" + os.path.join(B.ROOT, "include"), *B.DEVICE_FLAGS,
           "-Rpass-analysis=kernel-resource-usage", src, "-o", str(tmp_path / "k.o")]
    res = subprocess.run(cmd, capture_output=True, text=True, timeout=B.COMPILE_TIMEOUT_S)
    assert res.returncode == 0, res.stderr[-2000:]
    kernels, cur = {}, None
    for line in res.stderr.splitlines():
        m = re.search(r"Function Name: (\S+)", line)
        if m:
            cur = kernels.setdefault(m.group(1), {})
            continue
        m = re.search(r"(VGPRs|AGPRs|ScratchSize \[bytes/lane\]|LDS Size \[bytes/block\]|"
                      r"Occupancy \[waves/SIMD\]): (\d+)", line)
        if m and cur is not None:
            cur[m.group(1).split()[0]] = int(m.group(2))
    return kernels


def test_attention_kernels_fit_without_scratch(tmp_path):
    kernels = resource_report(tmp_path)
    attn = {k: v for k, v in kernels.items() if "attn_split" in k}
    # bf16 / f32, d 64 / 128, four modes (full, scored, sparse, staged), and the
    # two-level merge of bf16 d 128 in the two full modes
    assert len(attn) == 18, sorted(kernels)
    for name, r in attn.items():
        assert r["ScratchSize"] == 0, (name, r)
        assert r["LDS"] <= 160 * 1024, (name, r)
        assert r["VGPRs"] + r.get("AGPRs", 0) <= 256, (name, r)
        assert r["Occupancy"] >= 2, (name, r)
    topk = [v for k, v in kernels.items() if "score_topk" in k]
    assert topk and topk[0]["ScratchSize"] == 0


def test_gather_kernel_has_no_scratch(tmp_path):
    kernels = resource_report(tmp_path, os.path.join(B.CSRC, "hylra_offload.hip"))
    gather = [v for k, v in kernels.items() if "gather_blocks" in k]
    assert len(gather) == 1, sorted(kernels)
    assert gather[0]["ScratchSize"] == 0, gather[0]
