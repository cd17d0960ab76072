"""GPU tests of prior-aware skipping in the backward (BAM_SKIP_FAR with bam_attn_bwd_ex).

Every term the skipping backward leaves out has a weight that is zero in float32, so its
dZ is zero and so is everything it would add (include/bam.h): dQ, dK, dV and the per-head
dalpha, dbeta, dmu, ds must equal those of the full backward bit for bit.  The skipping
call is also checked against the fp64 oracle at the backward's tolerances, and the plan
must actually leave work out on local heads (measured with the forward's plan, which at
T <= 1024 and Dh = 64 uses the same 128-query blocks).
"""
import numpy as np
import pytest

import oracle
from gpu_util import within
from gpu_util import dev, host, max_abs, torch_mod
from positional_prior_bias_amd import workloads as wl

pytestmark = pytest.mark.gpu


def _bam():
    import positional_prior_bias_amd as bam
    return bam


def _local(seed, T, Dh, ssmax=True, H=4, ref=False):
    """Local heads (ALiBi-like decay) that skip most key tiles."""
    if ref:
        return wl.ref_case(seed, 1, H, T, Dh, "bf16", wl.CAUSAL | (wl.SSMAX if ssmax else 0),
                           theta_alpha_range=(0.0, 1.0), theta_beta_range=(0.6, 1.0), with_grad=True)
    w = wl.random_case(seed, 1, H, T, Dh, "bf16", wl.CAUSAL | (wl.SSMAX if ssmax else 0), with_grad=True)
    w.alpha = np.array([1.0, 2.0, 4.0, 8.0][:H], np.float32)
    w.beta = np.array([1.0, 1.0, 0.8, 1.0][:H], np.float32)
    w.mu = np.array([0.0, 0.0, 0.0, 0.25][:H], np.float32)
    w.s = np.full(H, 0.45, np.float32)
    return w


def _both(w, ref=False, ssmax=True):
    """(full, skipping) backward results, float32 gradients, with the offset gradient."""
    torch = torch_mod()
    bam = _bam()
    q, k, v, do = (dev(x, "bf16") for x in (w.q, w.k, w.v, w.do))
    a, b, m, s = dev(w.alpha), dev(w.beta), dev(w.mu), dev(w.s)
    o, lse = bam.bam_attn_fwd(q, k, v, a, b, m, s, causal=True, ssmax=ssmax, o_dtype=torch.float32, prior_ref=ref)
    full = bam.bam_attn_bwd_ex(q, k, v, o, lse, do, a, b, m, s, causal=True, ssmax=ssmax,
                               grad_dtype=torch.float32, prior_ref=ref)
    skip = bam.bam_attn_bwd_ex(q, k, v, o, lse, do, a, b, m, s, causal=True, ssmax=ssmax,
                               grad_dtype=torch.float32, prior_ref=ref, skip_far=True)
    torch.cuda.synchronize()
    return [host(x) for x in full], [host(x) for x in skip]


def _same_bits(full, skip):
    for name, x, y in zip(("dq", "dk", "dv", "dalpha", "dbeta", "dmu", "ds"), full, skip):
        same = np.array_equal(x.view(np.uint32), y.view(np.uint32))
        print(f"{name}: same bits {same}, max |d| {max_abs(x, y):.2e}")
        assert same, name


def _fwd_skipped_fraction(w, ssmax=True, ref=False):
    torch = torch_mod()
    bam = _bam()
    B, H, T, Dh = w.q.shape
    flags = bam.BAM_CAUSAL | (bam.BAM_SSMAX if ssmax else 0) | bam.BAM_SKIP_FAR | (bam.BAM_PRIOR_REF if ref else 0)
    ws = torch.empty(bam.bam_fwd_workspace_size(B, H, T, Dh, flags), dtype=torch.uint8, device="cuda")
    q, k, v = (dev(x, "bf16") for x in (w.q, w.k, w.v))
    bam.bam_attn_fwd(q, k, v, dev(w.alpha), dev(w.beta), dev(w.mu), dev(w.s), causal=True, ssmax=ssmax,
                     workspace=ws, skip_far=True, prior_ref=ref)
    torch.cuda.synchronize()
    return bam.fwd_skipped_fraction(ws, B, H, T, Dh, flags)


@pytest.mark.parametrize("T,Dh,ssmax", [(1000, 64, True), (2100, 64, True), (1500, 32, True), (2100, 64, False),
                                        (500, 64, True)])
def test_bwd_skip_same_bits(T, Dh, ssmax):
    """Local heads: the skipping backward equals the full one bit for bit (T = 500 runs the
    kernels' own bias strips, the longer ones the table)."""
    w = _local(2000 + T + Dh, T, Dh, ssmax)
    full, skip = _both(w, ssmax=ssmax)
    _same_bits(full, skip)
    if T <= 1024 and Dh == 64:   # fewer far tiles at T = 500
        assert _fwd_skipped_fraction(w, ssmax) > (0.3 if T >= 1000 else 0.15)


def test_bwd_skip_reference_prior_same_bits():
    w = _local(2300, 1600, 64, ref=True)
    full, skip = _both(w, ref=True)
    _same_bits(full, skip)


def test_bwd_skip_never_on_inverted_heads():
    """Inverted (beta < 0) and NoPE heads keep every tile; the result is still the full one."""
    H, T = 4, 1100
    w = wl.random_case(2400, 1, H, T, 64, "bf16", wl.CAUSAL | wl.SSMAX, with_grad=True)
    w.alpha = np.array([2.0, 0.5, np.inf, 3.0], np.float32)
    w.beta = np.array([-0.5, -0.2, 1.0, -0.8], np.float32)
    w.mu = np.full(H, -0.5, np.float32)
    w.s = np.full(H, 0.45, np.float32)
    full, skip = _both(w)
    _same_bits(full, skip)
    assert _fwd_skipped_fraction(w) == 0.0


def test_bwd_skip_against_oracle():
    """The skipping backward against the fp64 oracle (tolerances of test_parity_bwd)."""
    w = _local(2500, 700, 64)
    _, got = _both(w)
    ref = oracle.attn_bwd(w.q, w.k, w.v, w.do, w.alpha, w.beta, w.mu, w.s, causal=True, ssmax=True)
    for name, x in zip(("dq", "dk", "dv"), got[:3]):
        r = ref[name]
        within(max_abs(x, r), 1e-2 * max(1.0, float(np.max(np.abs(r)))), name)
    for name, x, A in zip(("dalpha", "dbeta", "dmu", "ds"), (got[3], got[4], got[5], got[6]),
                          ("A_alpha", "A_beta", "A_mu", "A_s")):
        err = np.abs(x - ref[name])
        tol = 1e-3 * ref[A] + 1e-6
        h = int(np.argmax(err / tol))
        within(err[h], tol[h], f"{name} (worst head {h})")
