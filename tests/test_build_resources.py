"""The compiler's per-kernel resource report (kept by the build).

Every kernel is designed to run without register spills or scratch memory:
a spill puts scratch traffic inside the tile loops.  The build keeps hipcc's
kernel-resource-usage remarks as ``_build/resource_usage.json``; these
tests read that report (CPU only, no kernel runs) so that a source change
which makes the compiler spill fails here, before any GPU run.
"""
import glob
import json
import os

import pytest

from exact_io_aware_58_amd import build

SAMPLE = """\
x.hip:49:1: remark: Function Name: _ZN2fa14merge16_kernelINS_4BF16ELi64EEEvPtPfPKtPKfm [-Rpass-analysis=kernel-resource-usage]
x.hip:49:1: remark:     TotalSGPRs: 36 [-Rpass-analysis=kernel-resource-usage]
x.hip:49:1: remark:     VGPRs: 31 [-Rpass-analysis=kernel-resource-usage]
x.hip:49:1: remark:     AGPRs: 0 [-Rpass-analysis=kernel-resource-usage]
x.hip:49:1: remark:     ScratchSize [bytes/lane]: 16 [-Rpass-analysis=kernel-resource-usage]
x.hip:49:1: remark:     Dynamic Stack: False [-Rpass-analysis=kernel-resource-usage]
x.hip:49:1: remark:     Occupancy [waves/SIMD]: 8 [-Rpass-analysis=kernel-resource-usage]
x.hip:49:1: remark:     SGPRs Spill: 0 [-Rpass-analysis=kernel-resource-usage]
x.hip:49:1: remark:     VGPRs Spill: 4 [-Rpass-analysis=kernel-resource-usage]
x.hip:49:1: remark:     LDS Size [bytes/block]: 1024 [-Rpass-analysis=kernel-resource-usage]
x.hip:60:1: remark: Function Name: other [-Rpass-analysis=kernel-resource-usage]
x.hip:60:1: remark:     VGPRs: 7 [-Rpass-analysis=kernel-resource-usage]
"""

FAMILIES = ["fwd16_kernel", "fwd16pp_kernel", "fwd32_kernel", "bwd_delta_kernel",
            "bwd_dkdv_kernel", "bwd_dq_kernel", "bwd_dkdv_dq_kernel", "merge16_kernel",
            "merge32_kernel"]


def test_parser_reads_the_remarks():
    u = build.parse_resource_remarks(SAMPLE)
    k = "_ZN2fa14merge16_kernelINS_4BF16ELi64EEEvPtPfPKtPKfm"
    assert set(u) == {k, "other"}
    assert u[k] == {"sgprs": 36, "vgprs": 31, "agprs": 0, "scratch_bytes": 16,
                    "occupancy": 8, "sgpr_spill": 0, "vgpr_spill": 4, "lds_bytes": 1024}
    assert u["other"] == {"vgprs": 7}


def _report():
    if not os.path.exists(build.REPORT):
        pytest.skip("no build report: run __graft_entry__.build() first")
    newest = max(os.path.getmtime(p) for p in glob.glob(os.path.join(build.CSRC, "*")))
    if newest > os.path.getmtime(build.REPORT):
        pytest.skip("sources changed after the last build: rebuild first")
    with open(build.REPORT) as fh:
        return json.load(fh)


def _family(symbol):
    for fam in sorted(FAMILIES, key=len, reverse=True):
        if fam in symbol:
            return fam
    return None


def test_every_kernel_family_is_built():
    u = _report()
    assert {_family(k) for k in u} >= set(FAMILIES)


def test_no_kernel_spills_vector_registers_or_uses_scratch():
    u = _report()
    bad = {k: v for k, v in u.items() if v.get("vgpr_spill", 0) or v.get("scratch_bytes", 0)}
    assert not bad, f"kernels with VGPR spills or scratch: {sorted(bad)}"


def test_matrix_kernels_fit_their_occupancy_and_lds():
    """The 16-bit tile kernels are built for two waves per SIMD (their
    launch bounds); the one exception is the masked D = 128 dK/dV kernel,
    which holds K, V and the dK/dV accumulators of 32 rows x 128 and runs
    one wave per SIMD.  Every workgroup's LDS fits the 160 KiB of a CU."""
    u = _report()
    for k, v in u.items():
        fam = _family(k)
        assert v.get("lds_bytes", 0) <= 160 * 1024, k
        if fam in ("fwd16_kernel", "fwd16pp_kernel", "bwd_dq_kernel", "bwd_dkdv_dq_kernel"):
            assert v["occupancy"] >= 2, (k, v)
        if fam == "bwd_dkdv_kernel":
            one_wave = "Li128ELb1E" in k  # D = 128, causal
            assert v["occupancy"] >= (1 if one_wave else 2), (k, v)
