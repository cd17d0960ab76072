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


# ---------------------------------------------------------------------------------------
# Argument validation: every mismatch the kernels would turn into an out-of-bounds access
# is refused by the binding before anything is launched.  These run on CPU tensors: the
# shape / dtype checks come before the device check, so the message names the mismatch.
# ---------------------------------------------------------------------------------------

def _t(*shape, dtype=torch.bfloat16):
    return torch.zeros(shape, dtype=dtype)


def _f32(n):
    return torch.ones(n, dtype=torch.float32)


def _raises(match, fn, *a, **k):
    with pytest.raises(bam.BamError, match=match):
        fn(*a, **k)


def test_fwd_argument_checks():
    B, H, T, Dh = 2, 3, 16, 64
    q, k, v = _t(B, H, T, Dh), _t(B, H, T, Dh), _t(B, H, T, Dh)
    p = dict(alpha=_f32(H), beta=_f32(H), mu=_f32(H), s=_f32(H))
    _raises("k has shape", bam.bam_attn_fwd, q, _t(B, H, T + 1, Dh), v, **p)
    _raises("v has dtype", bam.bam_attn_fwd, q, k, _t(B, H, T, Dh, dtype=torch.float32), **p)
    _raises("alpha has shape", bam.bam_attn_fwd, q, k, v, **{**p, "alpha": _f32(H + 1)})
    _raises("beta has dtype", bam.bam_attn_fwd, q, k, v, **{**p, "beta": torch.ones(H, dtype=torch.float64)})
    _raises("mu has shape", bam.bam_attn_fwd, q, k, v, **{**p, "mu": _f32(1)})
    _raises("s is required", bam.bam_attn_fwd, q, k, v, **{**p, "s": None})
    _raises("s has shape", bam.bam_attn_fwd, q, k, v, **{**p, "s": _f32(2 * H)})
    _raises("o has shape", bam.bam_attn_fwd, q, k, v, **p, o=_t(B, H, T, Dh // 2))
    _raises("o has dtype", bam.bam_attn_fwd, q, k, v, **p, o=_t(B, H, T, Dh, dtype=torch.float16))
    _raises("lse has shape", bam.bam_attn_fwd, q, k, v, **p, lse=_t(B, H, T - 1, dtype=torch.float32))
    _raises("lse has dtype", bam.bam_attn_fwd, q, k, v, **p, lse=_t(B, H, T))
    _raises("q must be a 4-D", bam.bam_attn_fwd, _t(B, H, T), k, v, **p)
    _raises("workspace too small", bam.bam_attn_fwd, q, k, v, **p, workspace=_t(8, dtype=torch.uint8))
    # metadata right: the remaining objection is the device
    _raises("device tensor", bam.bam_attn_fwd, q, k, v, **p)


def test_decode_argument_checks():
    B, H, L, Dh = 2, 3, 128, 64
    kc, vc, q = _t(B, H, L, Dh), _t(B, H, L, Dh), _t(B, H, Dh)
    kv = torch.full((B,), L, dtype=torch.int32)
    p = dict(alpha=_f32(H), beta=_f32(H), mu=_f32(H), s=_f32(H))
    _raises("v_cache has shape", bam.bam_attn_decode, q, kc, _t(B, H, L - 64, Dh), kv, **p)
    _raises("q has shape", bam.bam_attn_decode, _t(B, H, 2 * Dh), kc, vc, kv, **p)
    _raises("q has dtype", bam.bam_attn_decode, _t(B, H, Dh, dtype=torch.float32), kc, vc, kv, **p)
    _raises("kv_len has shape", bam.bam_attn_decode, q, kc, vc, torch.full((B - 1,), L, dtype=torch.int32), **p)
    _raises("kv_len has dtype", bam.bam_attn_decode, q, kc, vc, kv.long(), **p)
    _raises("o has shape", bam.bam_attn_decode, q, kc, vc, kv, **p, o=_t(B, H, Dh, 1))
    _raises("lse has shape", bam.bam_attn_decode, q, kc, vc, kv, **p, lse=_t(B * H, dtype=torch.float32))
    _raises("alpha has shape", bam.bam_attn_decode, q, kc, vc, kv, **{**p, "alpha": _f32(B)})
    _raises("device tensor", bam.bam_attn_decode, q, kc, vc, kv, **p)


def test_paged_decode_argument_checks():
    P, H, ps, Dh, B, nb = 6, 3, 64, 64, 2, 3
    kp, vp, q = _t(P, H, ps, Dh), _t(P, H, ps, Dh), _t(B, H, Dh)
    bt = torch.zeros((B, nb), dtype=torch.int32)
    kv = torch.full((B,), nb * ps, dtype=torch.int32)
    p = dict(alpha=_f32(H), beta=_f32(H), mu=_f32(H), s=_f32(H))
    _raises("v_pages has shape", bam.bam_attn_decode_paged, q, kp, _t(P - 1, H, ps, Dh), bt, kv, **p)
    _raises("block_table has dtype", bam.bam_attn_decode_paged, q, kp, vp, bt.long(), kv, **p)
    _raises("block_table must be a 2-D", bam.bam_attn_decode_paged, q, kp, vp, bt.view(-1), kv, **p)
    _raises("q has shape", bam.bam_attn_decode_paged, _t(B + 1, H, Dh), kp, vp, bt, kv, **p)
    _raises("kv_len has shape", bam.bam_attn_decode_paged, q, kp, vp, bt, kv[:1], **p)
    _raises("device tensor", bam.bam_attn_decode_paged, q, kp, vp, bt, kv, **p)


def test_bwd_argument_checks():
    B, H, T, Dh = 2, 3, 16, 64
    q = _t(B, H, T, Dh)
    o, lse, do = _t(B, H, T, Dh, dtype=torch.float32), _t(B, H, T, dtype=torch.float32), _t(B, H, T, Dh)
    p = dict(alpha=_f32(H), beta=_f32(H), mu=_f32(H), s=_f32(H))
    _raises("dout has shape", bam.bam_attn_bwd, q, q, q, o, lse, _t(B, H, T, Dh + 8), **p)
    _raises("dout has dtype", bam.bam_attn_bwd, q, q, q, o, lse, do.float(), **p)
    _raises("o has shape", bam.bam_attn_bwd, q, q, q, o[:, :, :-1], lse, do, **p)
    _raises("lse has shape", bam.bam_attn_bwd, q, q, q, o, lse[:, :, :-1], do, **p)
    _raises("lse has dtype", bam.bam_attn_bwd, q, q, q, o, lse.to(torch.bfloat16), do, **p)
    _raises("k has shape", bam.bam_attn_bwd_ex, q, _t(B, H, T, 32), q, o, lse, do, **p)
    _raises("v has dtype", bam.bam_attn_bwd, q, q, q.float(), o, lse, do, **p)
    _raises("s has shape", bam.bam_attn_bwd, q, q, q, o, lse, do, **{**p, "s": _f32(1)})
    _raises("device tensor", bam.bam_attn_bwd, q, q, q, o, lse, do, **p)


def test_prior_table_argument_checks():
    _raises("beta has shape", bam.bam_prior_table, _f32(4), _f32(3), None, 0, 8)
    _raises("mu has dtype", bam.bam_prior_table_ex, _f32(4), _f32(4), torch.zeros(4, dtype=torch.int32), 0, 8)
    _raises("alpha must be a 1-D", bam.bam_prior_table, _f32(4).view(2, 2), _f32(4), None, 0, 8)
