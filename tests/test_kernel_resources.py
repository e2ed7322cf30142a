"""Register and scratch budget of the hot kernels (CPU: hipcc cross-compiles for
gfx950 and reports each kernel's resource usage).  The streaming passes rely on
occupancy to hide memory latency, so a change that pushes a hot kernel past its
register budget, or into scratch (register spills to memory), fails here
before it can cost bandwidth on the GPU."""
import os
import re
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "draft_token_verification_08_amd", "csrc")
SRCS = [os.path.join(CSRC, "sv_kernels.hip"), os.path.join(CSRC, "sv_lmhead.hip")]
HIPCC = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"

# mangled kernel name -> minimum waves per SIMD
BUDGET = {
    "_ZN2sv7k_statsILi1ELi1ELb1EEEvNS_11StatsParamsE": 8,   # greedy, bf16, aligned
    "_ZN2sv12k_stats_treeILi1ELb1EEEvNS_11StatsParamsE": 8,  # greedy tree verification, bf16, aligned
    "_ZN2sv7k_statsILi1ELi0ELb1EEEvNS_11StatsParamsE": 7,   # sampling, bf16, aligned
    # sampling with no drafts (the draw inside), bf16: no-draft launches run about
    # 1024 workgroups, which 6 waves per SIMD keep resident
    "_ZN2sv12k_stats_drawILi1ELb1EEEvNS_11StatsParamsE": 6,
    "_ZN2sv6k_drawILi1EEEvNS_10DrawParamsE": 5,             # draw pass, bf16, aligned
    # sampling tree verification, bf16, aligned: statistics pass and round kernel
    "_ZN2sv19k_stats_tree_sampleILi1ELb1EEEvNS_11StatsParamsE": 6,
    # tree round: its deciding workgroup also forms the pending child's ratio in binary64
    # from the residual's plan (98 registers: 4 waves per SIMD; 1.5% of the tree step)
    "_ZN2sv12k_tree_roundILi1ELb1EEEvNS_11RoundParamsE": 4,
    "_ZN2sv5k_mtpILb1EEEvNS_9MtpParamsE": 8,               # MTP copy, aligned
    # logit projection (256 x 256 tiles, 8 waves, one workgroup per CU): two
    # waves per SIMD; the accumulators alone take 128 registers
    "_ZN2sv12_GLOBAL__N_18k_lmheadILi2ELi4ELb1EEEvNS_8LmParamsEi": 2,
}


@pytest.fixture(scope="module")
def usage(tmp_path_factory):
    if not os.path.exists(HIPCC):
        pytest.skip("hipcc not available")
    text = ""
    for i, src in enumerate(SRCS):
        out = tmp_path_factory.mktemp("ru") / f"k{i}.o"
        cmd = [HIPCC, "--offload-arch=gfx950", "-O3", "-std=c++17", "-ffp-contract=off", "-Xclang",
               "-target-feature", "-Xclang", "-packed-fp32-ops", "-I" + os.path.join(ROOT, "include"),
               "-I" + CSRC, "-x", "hip", "--cuda-device-only", "-c", src, "-o", str(out),
               "-Rpass-analysis=kernel-resource-usage"]
        text += subprocess.run(cmd, capture_output=True, text=True, check=True).stderr
    kernels = {}
    cur = None
    for line in text.splitlines():
        m = re.search(r"Function Name: (\S+)", line)
        if m:
            cur = kernels.setdefault(m.group(1), {})
            continue
        for key, pat in (("scratch", r"ScratchSize \[bytes/lane\]: (\d+)"), ("occ", r"Occupancy \[waves/SIMD\]: (\d+)"),
                         ("vgpr", r"VGPRs: (\d+)")):
            m = re.search(pat, line)
            if m and cur is not None:
                cur[key] = int(m.group(1))
    return kernels


def test_every_kernel_is_reported(usage):
    for k in BUDGET:
        assert k in usage, sorted(usage)


def test_no_kernel_spills(usage):
    spilled = {k: v["scratch"] for k, v in usage.items() if v.get("scratch", 0) != 0}
    assert not spilled, spilled


@pytest.mark.parametrize("kernel,min_occ", sorted(BUDGET.items()))
def test_hot_kernel_occupancy(usage, kernel, min_occ):
    assert usage[kernel]["occ"] >= min_occ, usage[kernel]
