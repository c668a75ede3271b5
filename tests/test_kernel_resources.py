"""Compiled resources of the HIP kernels, without a GPU.

Every kernel is compiled for gfx950 with the library's own flags and the compiler's
per-kernel resource report is read: no kernel may spill to scratch memory, and the kernels
of the two streaming passes must fit their waves per SIMD in the 512 registers (VGPRs +
AGPRs) of a SIMD lane and a workgroup in the CU's 160 KB of LDS: the forward runs 512
threads (two waves per SIMD, 256 registers each), the score pass 256 threads (one wave per
SIMD, up to 512). A change that breaks one of these still computes the right values, so
the parity tests would not notice.
"""
import glob
import os
import re
import subprocess

import pytest

from kv_cache_eviction_kvscore_amd import build as kbuild

SOURCES = sorted(glob.glob(os.path.join(kbuild.CSRC, "*.hip")))


def resources(src):
    cmd = [kbuild.HIPCC] + kbuild.CFLAGS + kbuild.EXTRA.get(os.path.basename(src), []) + [
        "--cuda-device-only", "-c", src, "-o", os.devnull, "-Rpass-analysis=kernel-resource-usage"]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-2000:]
    out, cur = {}, None
    for line in r.stderr.splitlines():
        m = re.search(r"Function Name: (\S+)", line)
        if m:
            cur = m.group(1)
            out[cur] = {}
            continue
        m = re.search(r"remark: ([A-Za-z ]+?)(?: \[[^\]]*\])?: (\d+)", line)
        if m and cur:
            out[cur][m.group(1).strip()] = int(m.group(2))
    assert out, "no resource report"
    return out


@pytest.mark.parametrize("src", SOURCES, ids=[os.path.basename(s) for s in SOURCES])
def test_no_kernel_spills(src):
    for fn, r in resources(src).items():
        assert r.get("ScratchSize", 0) == 0, (fn, r)


# kernel name fragment -> (source, registers a wave may use)
STREAMING = {"fwd_partial_kernel": ("attn_fwd.hip", 256), "score_kernel": ("score.hip", 512)}


@pytest.mark.parametrize("kernel", sorted(STREAMING))
def test_streaming_kernels_fit_their_waves_per_simd(kernel):
    name, regs = STREAMING[kernel]
    rep = resources(os.path.join(kbuild.CSRC, name))
    main = {fn: r for fn, r in rep.items() if kernel in fn}
    assert main
    for fn, r in main.items():
        assert r["VGPRs"] + r.get("AGPRs", 0) <= regs, (fn, r)
        assert r["LDS Size"] <= 160 * 1024, (fn, r)
