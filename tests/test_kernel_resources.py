"""Register, LDS and scratch budgets of the HIP kernels, read from the gfx950 assembly that
hipcc writes for each source (CPU only: a cross-compile, nothing runs on a GPU).

The occupancy the forward and backward kernels are designed for rests on these numbers:
the 128-row forward work-group (Dh = 64) fits four to a CU only with at most 128 VGPRs and
at most 40,960 bytes of LDS (the CU allocates LDS in 1,280-byte steps), and the backward
kernels fit three waves per SIMD only with at most 168 VGPRs.  No hot kernel may spill to
scratch memory."""
import concurrent.futures as cf
import os
import re
import shutil
import subprocess
import tempfile

import pytest

from positional_prior_bias_amd import build as B

pytestmark = pytest.mark.skipif(shutil.which("hipcc") is None and not os.path.exists("/opt/rocm/bin/hipcc"),
                                reason="hipcc is needed to read the kernels' resources")


def _asm(src, out):
    cmd = [B._hipcc(), *[f for f in B.CXXFLAGS if f != "-fPIC"], "--cuda-device-only", "-S", src, "-o", out]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr
    return out


@pytest.fixture(scope="module")
def kernels():
    res = {}
    with tempfile.TemporaryDirectory() as td:
        srcs = B.sources()
        with cf.ThreadPoolExecutor(max_workers=min(4, len(srcs))) as ex:
            outs = list(ex.map(lambda s: _asm(s, os.path.join(td, os.path.basename(s) + ".s")), srcs))
        for out in outs:
            name = None
            for line in open(out):
                m = re.match(r"\s*\.amdhsa_kernel\s+(\S+)", line)
                if m:
                    name, cur = m.group(1), {}
                    continue
                if name is None:
                    continue
                m = re.match(r"\s*\.amdhsa_(next_free_vgpr|group_segment_fixed_size|private_segment_fixed_size)\s+(\d+)", line)
                if m:
                    cur[m.group(1)] = int(m.group(2))
                if ".end_amdhsa_kernel" in line:
                    res[name] = cur
                    name = None
    return res


def _find(kernels, *parts):
    found = {k: v for k, v in kernels.items() if all(p in k for p in parts)}
    assert found, parts
    return found


def test_no_kernel_spills(kernels):
    assert kernels
    spills = {k: v["private_segment_fixed_size"] for k, v in kernels.items() if v["private_segment_fixed_size"]}
    assert not spills, spills


def test_short_sequence_forward_fits_four_per_cu(kernels):
    # fwd_bf16_kernel<64, causal, 1> and <64, non-causal, 1>
    for k, v in _find(kernels, "fwd_bf16_kernelILi64E", "ELi1E").items():
        assert v["next_free_vgpr"] <= 128, (k, v)
        assert v["group_segment_fixed_size"] <= 4 * 1280 * 8, (k, v)   # 40,960 B


def test_backward_fits_three_waves_per_simd(kernels):
    for k, v in _find(kernels, "bwd_", "ILi64E").items():
        assert v["next_free_vgpr"] <= 168, (k, v)
