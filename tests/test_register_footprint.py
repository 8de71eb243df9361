"""Register footprints that let the ring's block pass run beside a ring step.

A ring step (every one but the last) runs while the next K/V block is copied
on a side stream. The copy runs on the compute units, so it can only make
progress during the step if one of its waves fits on a SIMD next to the two
step waves: the d = 128 step kernels must stay within 248 VGPRs (no AGPRs, no
scratch), and the pass kernel within 16 (512 registers per SIMD lane). The
kernels are compiled for gfx950 with the library's own flags and the
footprints read from the compiler's resource report. The backward kernels
hold their LDS operands a few products ahead in registers; they must still fit
two waves per SIMD without spilling.
"""

import os
import re
import subprocess

import pytest

from context_attention_ra_amd import build

CSRC = build.CSRC


def resource_report(source):
    flags = [f for f in build.HIPCC_FLAGS if f not in ("-shared", "-fPIC")]
    cmd = [build.hipcc(), *flags, "--cuda-device-only", "-c", "-Rpass-analysis=kernel-resource-usage",
           "-I", build.INCLUDE, "-I", CSRC, os.path.join(CSRC, source), "-o", os.devnull]
    res = subprocess.run(cmd, capture_output=True, text=True)
    assert res.returncode == 0, res.stderr[-3000:]
    out, cur = {}, None
    for line in res.stderr.splitlines():
        m = re.search(r"Function Name: (\S+)", line)
        if m:
            cur = m.group(1)
            out[cur] = {}
            continue
        m = re.search(r"remark: +(VGPRs|AGPRs|ScratchSize \[bytes/lane\]|Occupancy \[waves/SIMD\]): (\d+)", line)
        if m and cur:
            out[cur][m.group(1)] = int(m.group(2))
    return out


@pytest.fixture(scope="module")
def hipcc_available():
    try:
        build.hipcc()
    except RuntimeError:
        pytest.skip("hipcc not found")


def test_non_final_step_kernels_leave_a_copy_wave_room(hipcc_available):
    rep = resource_report("step_mfma.hip")
    # step_mfma_kernel<128, causal, kStep>
    steps = {k: v for k, v in rep.items() if re.search(r"step_mfma_kernelILi128ELb[01]ELi0E", k)}
    assert len(steps) == 2, sorted(rep)
    for name, r in steps.items():
        assert r["VGPRs"] <= 248, (name, r)
        assert r["AGPRs"] == 0, (name, r)
        assert r["ScratchSize [bytes/lane]"] == 0, (name, r)
        assert r["Occupancy [waves/SIMD]"] >= 2, (name, r)


def test_pass_kernel_fits_beside_a_step(hipcc_available):
    rep = resource_report("rows.hip")
    pas = [v for k, v in rep.items() if "kv_pass_kernel" in k]
    assert len(pas) == 1, sorted(rep)
    r = pas[0]
    assert r["VGPRs"] + r["AGPRs"] <= 16, r
    assert r["ScratchSize [bytes/lane]"] == 0, r
    # two step waves of 248 and one pass wave fill at most the 512 registers of a SIMD lane
    assert 2 * 248 + 16 <= 512


def test_backward_kernels_fit_two_waves_per_simd_without_spills(hipcc_available):
    rep = resource_report("bwd_mfma.hip")
    kern = {k: v for k, v in rep.items() if "bwd_dq_kernel" in k or "bwd_dkdv_kernel" in k}
    assert len(kern) == 8, sorted(rep)  # dQ and dK/dV, d = 64 and 128, causal or not
    for name, r in kern.items():
        assert r["ScratchSize [bytes/lane]"] == 0, (name, r)
        assert r["Occupancy [waves/SIMD]"] >= 2, (name, r)
