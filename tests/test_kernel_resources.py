"""Register budget of the hot kernels, checked at compile time (no GPU).

The assignment and decode kernels are sized so that nothing spills to
scratch memory: a spill would turn register traffic into memory traffic on
the MFMA loop or the decode chain. hipcc's resource report for gfx950 must
show 0 bytes of scratch per lane for every instantiation of these kernels,
and the assignment's 8-wave workgroups must fit two waves per SIMD.
"""
import os
import re
import shutil
import subprocess

import pytest

from sparse_decode_attention_ckv_amd import build as B

# kernel-name substring -> source file
CHECKED = {
    "k_assign_bf16": "cluster.hip",
    "k_sel_attn_bf16": "decode.hip",
    "k_sel_score": "select.hip",
    "k_sel_cut": "select.hip",
    "k_attn_partial_bf16": "attn.hip",
    "k_attn_combine": "attn.hip",
    "k_sel_attn_f32": "decode.hip",
    "k_attn_partial_f32": "attn.hip",
}


def _report(src):
    cmd = [B.HIPCC, *[f for f in B.FLAGS if f != "-fPIC"], "--cuda-device-only", "-c",
           os.path.join(B.CSRC, src), "-o", os.devnull, "-Rpass-analysis=kernel-resource-usage"]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-2000:]
    kernels, cur = {}, None
    for line in r.stderr.splitlines():
        m = re.search(r"Function Name: (\S+)", line)
        if m:
            cur = m.group(1)
            kernels[cur] = {}
            continue
        m = re.search(r"remark:\s+([A-Za-z /\[\]]+?):\s+(\d+)", line)
        if m and cur:
            kernels[cur][m.group(1).strip()] = int(m.group(2))
    return kernels


@pytest.mark.skipif(not os.path.exists(B.HIPCC) and shutil.which("hipcc") is None,
                    reason="hipcc not available")
def test_hot_kernels_do_not_spill():
    reports = {}
    for src in sorted(set(CHECKED.values())):
        reports.update(_report(src))
    for name, src in CHECKED.items():
        inst = {k: v for k, v in reports.items() if name in k}
        assert inst, f"{name} not found in the resource report of {src}"
        for k, v in inst.items():
            assert v.get("ScratchSize [bytes/lane]") == 0, (k, v)
    for k, v in reports.items():
        if "k_assign_bf16" in k:
            assert v.get("VGPRs", 999) <= 256 and v.get("Occupancy [waves/SIMD]", 0) >= 2, (k, v)
