"""Host-side logic of the Python binding (no GPU): flag composition, the per-head
parameter helpers, and the arithmetic that turns a skipping plan into a work fraction."""
import numpy as np
import pytest
import torch

import positional_prior_bias_amd as bam
from positional_prior_bias_amd import workloads as wl


def test_flag_composition():
    f = bam._flags
    assert f(True, True) == bam.BAM_CAUSAL | bam.BAM_SSMAX
    assert f(False, False, prior_ref=True) == bam.BAM_PRIOR_REF
    assert f(True, False, prior="ref") == bam.BAM_CAUSAL | bam.BAM_PRIOR_REF
    assert f(True, False, prior="sandwich") == bam.BAM_CAUSAL | bam.BAM_PRIOR_SANDWICH
    assert f(True, False, prior="alpha") == bam.BAM_CAUSAL
    with pytest.raises(bam.BamError):
        f(True, False, prior_ref=True, prior="sandwich")
    with pytest.raises(bam.BamError):
        f(True, False, prior="rope")


def test_flag_values_match_the_header():
    hdr = open(bam.__file__.replace("positional_prior_bias_amd/__init__.py", "include/bam.h")).read()
    for name in ("BAM_CAUSAL", "BAM_SSMAX", "BAM_TABLE_READY", "BAM_PRIOR_REF", "BAM_PRIOR_SANDWICH",
                 "BAM_SKIP_FAR"):
        line = next(l for l in hdr.splitlines() if l.startswith(f"#define {name} "))
        assert int(line.split()[2].rstrip("u")) == getattr(bam, name), name


def test_parameter_helpers():
    """ALiBi slopes 2^(-8 (h + 1) / H) (H = 4: 1/4, 1/16, 1/64, 1/256, as the NNX page
    prints); Sandwich ratios 8 (h + 1) / H; both equal the seeded-input module's values."""
    assert np.allclose(bam.alibi_slopes(4).numpy(), [0.25, 1 / 16, 1 / 64, 1 / 256], rtol=0, atol=0)
    for H in (4, 12):
        assert np.array_equal(bam.alibi_slopes(H).numpy(), wl.alibi_slopes(H).astype(np.float32))
    assert np.allclose(bam.sandwich_ratios(12).numpy(), 8 * np.arange(1, 13) / 12, rtol=1e-7)


@pytest.mark.parametrize("T,Dh", [(512, 64), (1024, 64), (1025, 64), (2100, 64), (700, 128), (300, 32)])
def test_skipped_fraction_arithmetic(T, Dh):
    """fwd_skipped_fraction reads the plan at the offset the library reports and divides by
    the causal tile count of each query block."""
    B, H = 2, 3
    flags = bam.BAM_CAUSAL | bam.BAM_SKIP_FAR
    off, cnt = bam.bam_fwd_skip_plan_offset(B, H, T, Dh, flags)
    rows = 128 if (Dh == 128 or (Dh == 64 and T <= 1024)) else 256   # include/bam.h
    nqb = (T + rows - 1) // rows
    assert cnt == nqb * B * H
    assert bam.bam_fwd_workspace_size(B, H, T, Dh, flags) >= off + 4 * cnt
    ws = torch.zeros(bam.bam_fwd_workspace_size(B, H, T, Dh, flags), dtype=torch.uint8)
    rng = np.random.default_rng(T)
    tiles = np.array([(min((qb + 1) * rows, T) + 63) // 64 for qb in range(nqb)])
    plan = np.concatenate([rng.integers(0, (qb * rows) // 64 + 1, B * H) for qb in range(nqb)]).astype(np.int32)
    ws[off:off + 4 * cnt] = torch.from_numpy(plan.view(np.uint8))
    expect = plan.sum() / (tiles.sum() * B * H)
    assert abs(bam.fwd_skipped_fraction(ws, B, H, T, Dh, flags) - expect) < 1e-12
