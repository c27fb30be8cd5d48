"""The compiler's resource report of every kernel in librescomp.so (written by
the build, lib/kernel_resources.json): no kernel spills to scratch memory, and
the streaming kernels keep enough waves resident to cover HBM latency."""
import json
import os

import pytest

from activation_residual_compression_amd import build as hipbuild


@pytest.fixture(scope="module")
def kernels():
    if not os.path.exists(hipbuild.RESOURCES):
        pytest.fail("%s is missing: run __graft_entry__.build()" % hipbuild.RESOURCES)
    with open(hipbuild.RESOURCES) as f:
        data = json.load(f)
    assert data["arch"] == "gfx950"
    return data["kernels"]


def test_every_kernel_reported(kernels):
    names = " ".join(kernels)
    for k in ("q_compress_kernel", "q_decompress_kernel", "nm_compress_kernel", "nm_decompress_kernel",
              "lr_rq_kernel", "lr_rtp_kernel", "lr_chol_kernel", "lr_solve_kernel", "lr_recon_kernel",
              "lr_int4_kernel", "bs_score_kernel", "bs_select_kernel", "bs_pack_kernel", "bs_unpack_kernel"):
        assert k in names, k


def test_no_kernel_spills(kernels):
    bad = {k: v for k, v in kernels.items() if v.get("scratch_bytes", 0) or v.get("vgpr_spill", 0)}
    assert not bad, bad


def test_streaming_kernels_occupancy(kernels):
    for name, v in kernels.items():
        if any(s in name for s in ("q_compress_kernel", "q_decompress_kernel", "nm_compress_kernel",
                                   "nm_decompress_kernel", "bs_score_kernel")):
            assert v["occupancy"] >= 4, (name, v)


def test_parser_reads_compiler_remarks():
    text = ("x.hip:1:1: remark: Function Name: _Z1kv [-Rpass-analysis=kernel-resource-usage]\n"
            "x.hip:1:1: remark:     VGPRs: 12 [-Rpass-analysis=kernel-resource-usage]\n"
            "x.hip:1:1: remark:     ScratchSize [bytes/lane]: 16 [-Rpass-analysis=kernel-resource-usage]\n"
            "x.hip:1:1: remark:     Occupancy [waves/SIMD]: 8 [-Rpass-analysis=kernel-resource-usage]\n")
    assert hipbuild.parse_resource_report(text) == {"_Z1kv": {"vgprs": 12, "scratch_bytes": 16, "occupancy": 8}}
