"""GPU tests of prior-aware key skipping (BAM_SKIP_FAR, causal bf16 forward).

A skipped key's weight is below 2^-150 of its row's largest (include/bam.h), so:
* the skipped call matches the full call to float32 precision: |dO| <= 1e-6 and
  |dlse| <= 1e-6 on float32 outputs (in practice the two agree bit for bit);
* both match the fp64 oracle at the bf16 tolerances (|O| 1e-2, lse 1e-3);
* the plan actually skips on local heads (ALiBi-like beta = 1 heads at T = 2100), never on
  inverted (beta < 0) or NoPE heads, and does not drop a far key whose content score
  outweighs the prior (the |q| max|k| term of the bound);
* at the 32k length-extrapolation workload, skipped and full calls agree on every output.
"""
import numpy as np
import pytest

import oracle
from gpu_util import within
from gpu_util import BF16_LSE_ABS, BF16_O_ABS, dev, host, max_abs, torch_mod
from positional_prior_bias_amd import workloads as wl

pytestmark = pytest.mark.gpu

SKIP_EXACT = 1e-6


def _bam():
    import positional_prior_bias_amd as bam
    return bam


def _run(q, k, v, alpha, beta, mu, s, ssmax, skip, prior=None):
    """Forward with float32 outputs; returns (o, lse, skipped fraction or None)."""
    torch = torch_mod()
    bam = _bam()
    B, H, T, Dh = q.shape
    flags = bam.BAM_CAUSAL | (bam.BAM_SSMAX if ssmax else 0) | (bam.BAM_SKIP_FAR if skip else 0)
    if prior == "sandwich":
        flags |= bam.BAM_PRIOR_SANDWICH
    ws = torch.empty(bam.bam_fwd_workspace_size(B, H, T, Dh, flags), dtype=torch.uint8, device="cuda")
    o, lse = bam.bam_attn_fwd(q, k, v, alpha, beta, mu, s, causal=True, ssmax=ssmax, o_dtype=torch.float32,
                              workspace=ws, skip_far=skip, prior=prior)
    torch.cuda.synchronize()
    frac = bam.fwd_skipped_fraction(ws, B, H, T, Dh, flags) if skip else None
    return host(o), host(lse), frac


def _rows(w, rows, ssmax=True):
    """Oracle O [B, H, R, Dh] and lse [B, H, R] of the given query rows."""
    B, H = w.q.shape[:2]
    O = np.empty((B, H, len(rows), w.q.shape[3]))
    L = np.empty((B, H, len(rows)))
    for b in range(B):
        for h in range(H):
            O[b, h], L[b, h] = oracle.attn_fwd_rows(w.q[b, h], w.k[b, h], w.v[b, h], rows, w.alpha[h], w.beta[h],
                                                    w.mu[h], w.s[h], causal=True, ssmax=ssmax)
    return O, L


def _case(w, ssmax=True, prior=None):
    q, k, v = (dev(x, "bf16") for x in (w.q, w.k, w.v))
    a, b, m, s = dev(w.alpha), dev(w.beta), dev(w.mu), dev(w.s)
    o1, l1, _ = _run(q, k, v, a, b, m, s, ssmax, False, prior)
    o2, l2, frac = _run(q, k, v, a, b, m, s, ssmax, True, prior)
    print(f"skipped fraction {frac:.3f}  |dO| {max_abs(o1, o2):.2e}  |dlse| {max_abs(l1, l2):.2e}")
    within(max_abs(o1, o2), SKIP_EXACT, "max_abs(o1, o2)")
    within(max_abs(l1, l2), SKIP_EXACT, "max_abs(l1, l2)")
    return o2, l2, frac


@pytest.mark.parametrize("T,Dh,ssmax", [(2100, 64, True), (1000, 64, True), (1500, 32, True), (1100, 128, True),
                                        (2100, 64, False)])
def test_skip_local_heads(T, Dh, ssmax):
    """Local heads (beta = 1 and 0.8, alpha = 1 .. 8) skip most tiles; results unchanged."""
    H = 4
    w = wl.random_case(1600 + T + Dh, 1, H, T, Dh, "bf16", wl.CAUSAL | (wl.SSMAX if ssmax else 0))
    w.alpha = np.array([1.0, 2.0, 4.0, 8.0], np.float32)
    w.beta = np.array([1.0, 1.0, 0.8, 1.0], np.float32)
    w.mu = np.zeros(H, np.float32)
    w.s = np.full(H, 0.45, np.float32)
    o, lse, frac = _case(w, ssmax)
    assert frac > 0.3
    O, L = oracle.attn_fwd(w.q, w.k, w.v, w.alpha, w.beta, w.mu, w.s, causal=True, ssmax=ssmax)
    within(max_abs(o, O), BF16_O_ABS, "max_abs(o, O)")
    within(max_abs(lse, L), BF16_LSE_ABS, "max_abs(lse, L)")


def test_skip_never_on_inverted_or_nope_heads():
    H, T = 4, 1300
    w = wl.random_case(1700, 1, H, T, 64, "bf16", wl.CAUSAL | wl.SSMAX)
    w.alpha = np.array([2.0, 0.5, np.inf, 3.0], np.float32)
    w.beta = np.array([-0.5, -0.2, 1.0, -0.8], np.float32)
    w.mu = np.full(H, -0.5, np.float32)
    w.s = np.full(H, 0.45, np.float32)
    _, _, frac = _case(w)
    assert frac == 0.0


def test_skip_keeps_a_far_key_that_outweighs_the_prior():
    """Query 1999 and a key at position 3 aligned with it, |k| = 60: its content score
    (~60 |q| / 8) beats the ALiBi penalty of 1996 / 64 = 31, so it must survive; the
    max|k| term of the bound keeps its tile (and every tile of that head)."""
    H, T, Dh = 2, 2048, 64
    w = wl.random_case(1800, 1, H, T, Dh, "bf16", wl.CAUSAL | wl.SSMAX)
    w.alpha = np.array([64.0, 64.0], np.float32)
    w.beta = np.ones(H, np.float32)
    w.mu = np.zeros(H, np.float32)
    w.s = np.full(H, 0.45, np.float32)
    qi = w.q[0, 0, 1999]
    w.k[0, 0, 3] = wl.bf16_round((60.0 * qi / np.linalg.norm(qi)).astype(np.float32))
    w.v[0, 0, 3] = 7.0
    o, lse, frac = _case(w)
    O, L = _rows(w, np.array([1999, 2047]))
    within(max_abs(o[:, :, [1999, 2047]], O), BF16_O_ABS, "max_abs(o[:, :, [1999, 2047]], O)")
    within(max_abs(lse[:, :, [1999, 2047]], L), BF16_LSE_ABS, "max_abs(lse[:, :, [1999, 2047]], L)")
    assert o[0, 0, 1999, 0] > 6.0        # the planted key dominates row 1999


def test_skip_with_reference_and_sandwich_priors():
    """The plan works from the table, so any prior kind is covered: the reference form with
    the pages' linspace(0, 1) theta_beta and the Sandwich bias."""
    H, T = 4, 1600
    w = wl.ref_case(1900, 1, H, T, 64, "bf16", wl.CAUSAL | wl.SSMAX, theta_alpha_range=(0.0, 1.0),
                    theta_beta_range=(0.6, 1.0))
    q, k, v = (dev(x, "bf16") for x in (w.q, w.k, w.v))
    a, b, m, s = dev(w.alpha), dev(w.beta), dev(w.mu), dev(w.s)
    torch = torch_mod()
    bam = _bam()
    flags = bam.BAM_CAUSAL | bam.BAM_SSMAX | bam.BAM_SKIP_FAR | bam.BAM_PRIOR_REF
    ws = torch.empty(bam.bam_fwd_workspace_size(1, H, T, 64, flags), dtype=torch.uint8, device="cuda")
    o1, l1 = bam.bam_attn_fwd(q, k, v, a, b, m, s, o_dtype=torch.float32, prior_ref=True)
    o2, l2 = bam.bam_attn_fwd(q, k, v, a, b, m, s, o_dtype=torch.float32, prior_ref=True, skip_far=True,
                              workspace=ws)
    torch.cuda.synchronize()
    assert bam.fwd_skipped_fraction(ws, 1, H, T, 64, flags) > 0.2
    within(max_abs(host(o1), host(o2)), SKIP_EXACT, "skipping against full O")
    within(max_abs(host(l1), host(l2)), SKIP_EXACT, "skipping against full lse")
    O, L = oracle.attn_fwd(w.q, w.k, w.v, w.alpha, w.beta, w.mu, w.s, causal=True, ssmax=True, param="ref")
    within(max_abs(host(o2), O), BF16_O_ABS, "O")
    within(max_abs(host(l2), L), BF16_LSE_ABS, "lse")

    ws_ = wl.sandwich_case(1901, 1, 3, 700, 64, "bf16")
    _case(ws_, prior="sandwich")


def test_skip_rejections():
    torch = torch_mod()
    bam = _bam()
    x = torch.zeros((1, 1, 64, 32), dtype=torch.float32, device="cuda")
    one = torch.ones(1, dtype=torch.float32, device="cuda")
    with pytest.raises(bam.BamError):
        bam.bam_attn_fwd(x, x, x, one, one, None, None, ssmax=False, skip_far=True)    # fp32 path
    xb = x.to(torch.bfloat16)
    with pytest.raises(bam.BamError):
        bam.bam_attn_fwd(xb, xb, xb, one, one, None, None, causal=False, ssmax=False, skip_far=True)
    with pytest.raises(bam.BamError):
        bam.bam_fwd_skip_plan_offset(1, 1, 64, 64, bam.BAM_CAUSAL)


def test_skip_length_extrapolation_32k():
    """The 32k workload (six heavy-tailed, six inverted heads): skipped and full calls agree
    on every output; sampled rows against the oracle."""
    torch = torch_mod()
    bam = _bam()
    w = wl.long_prefill()
    q, k, v = (dev(x, "bf16") for x in (w.q, w.k, w.v))
    a, b, m, s = dev(w.alpha), dev(w.beta), dev(w.mu), dev(w.s)
    B, H, T, Dh = w.q.shape
    o1, l1, _ = _run(q, k, v, a, b, m, s, True, False)
    o2, l2, frac = _run(q, k, v, a, b, m, s, True, True)
    print(f"32k skipped fraction {frac:.3f}")
    assert frac > 0.05
    within(max_abs(o1, o2), SKIP_EXACT, "T = 32768 skipping against full O")
    within(max_abs(l1, l2), SKIP_EXACT, "T = 32768 skipping against full lse")
    rows = np.array([0, 1, 4095, 20000, T - 1])
    O, L = _rows(w, rows)
    within(max_abs(o2[:, :, rows], O), BF16_O_ABS, "max_abs(o2[:, :, rows], O)")
    within(max_abs(l2[:, :, rows], L), BF16_LSE_ABS, "max_abs(l2[:, :, rows], L)")
