"""The compiler's resource report for every kernel of librc.so (written by the
build): no vector-register spills, no scratch arrays, and the occupancy the
attention kernels' 512-thread workgroups are laid out for.

A kernel whose accumulators the compiler moves to scratch memory computes the
same values, so no parity test notices; only its time does (an attention
kernel whose output accumulators went to scratch ran three times slower).
These checks catch that at build time, without a GPU.
"""
import json
import os

import pytest

from autoregressive_video_diffusion_ring_amd import build as rc_build

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HOT = "_ZN2rc12_GLOBAL__N_115attn_fp8_kernelILi128ELb0ELb0EEEvNS0_6F8ArgsE"  # attn_fp8_kernel<128, false, false>


def _report():
    path = rc_build.RESOURCES
    if not os.path.exists(path):
        pytest.skip("no kernel resource report: run the build first")
    newest_src = max(os.path.getmtime(os.path.join(rc_build.CSRC, s)) for s in rc_build.SOURCES)
    assert os.path.getmtime(path) >= newest_src, "kernel resource report older than the sources: build again"
    with open(path) as f:
        return json.load(f)


def test_parser_reads_hipcc_remarks():
    text = "\n".join([
        "a.hip:3:1: remark: Function Name: _Z1kv [-Rpass-analysis=kernel-resource-usage]",
        "    3 | __global__ void k() {}",
        "      | ^",
        "a.hip:3:1: remark:     VGPRs: 12 [-Rpass-analysis=kernel-resource-usage]",
        "a.hip:3:1: remark:     ScratchSize [bytes/lane]: 16 [-Rpass-analysis=kernel-resource-usage]",
        "a.hip:3:1: remark:     Dynamic Stack: False [-Rpass-analysis=kernel-resource-usage]",
        "a.hip:3:1: remark:     Occupancy [waves/SIMD]: 8 [-Rpass-analysis=kernel-resource-usage]",
        "a.hip:9:1: remark: Function Name: _Z2k2v [-Rpass-analysis=kernel-resource-usage]",
        "a.hip:9:1: remark:     VGPRs Spill: 3 [-Rpass-analysis=kernel-resource-usage]",
    ])
    assert rc_build.parse_resource_remarks(text) == {
        "_Z1kv": {"VGPRs": 12, "ScratchSize": 16, "Dynamic Stack": "False", "Occupancy": 8},
        "_Z2k2v": {"VGPRs Spill": 3},
    }


def test_every_kernel_is_reported():
    rep = _report()
    for name in ("attn_fp8_kernel", "chunk_attn_kernel", "cache_write_fp8_kernel", "rerotate_kernel",
                 "qkv_proj_kernel", "key_mass_kernel"):
        assert any(name in k for k in rep), name
    for k, v in rep.items():
        for field in ("VGPRs", "VGPRs Spill", "ScratchSize", "Occupancy", "LDS Size"):
            assert field in v, (k, field)


def test_no_vector_spills_or_scratch_arrays():
    rep = _report()
    for k, v in rep.items():
        assert v["VGPRs Spill"] == 0, (k, v)
        assert v["Dynamic Stack"] == "False", (k, v)
        # scalar-register spill slots only (a few words); an array in scratch is far larger
        assert v["ScratchSize"] <= 16, (k, v)
        assert v["LDS Size"] <= 160 * 1024, (k, v)


def test_attention_kernels_fit_two_waves_per_simd():
    # 512-thread workgroups: two waves on each of a compute unit's four SIMDs
    rep = _report()
    attn = {k: v for k, v in rep.items() if "attn_fp8_kernel" in k or "chunk_attn_kernel" in k}
    assert len(attn) >= 8
    for k, v in attn.items():
        assert v["Occupancy"] >= 2 and v["VGPRs"] + v.get("AGPRs", 0) <= 256, (k, v)


def test_streaming_attention_kernel_uses_no_scratch():
    v = _report()[HOT]
    assert v["ScratchSize"] == 0 and v["VGPRs Spill"] == 0, v
