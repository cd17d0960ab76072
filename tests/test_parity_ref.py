"""GPU parity of the reference parameterisation (BAM_PRIOR_REF) and of the offset
gradient (bam_attn_bwd_ex) against the fp64 oracle ("Bayesian Attention Mechanism"
README, "Implementation Details": -e^theta_alpha (|(j - i) - mu| + eps)^theta_beta,
mu = e^theta_mu - e^-theta_mu, eps = 1e-5).

Tolerances as in the other parity tests: table entries within 2e-6 relative to the
largest entry of their row (float32 rounding of float64 values); forward bf16 path
|O| 1e-2, lse 1e-3; fp32 path normwise relative 1e-5; backward dQ/dK/dV 1e-2 of the
largest entry, per-head parameter gradients 1e-3 of that head's sum of |terms| + 1e-6."""
import math

import numpy as np
import pytest

import oracle
from gpu_util import within
from gpu_util import BF16_LSE_ABS, BF16_O_ABS, F32_REL, dev, host, max_abs, normwise_rel, params, torch_mod
from positional_prior_bias_amd import workloads as wl

pytestmark = pytest.mark.gpu


def _bam():
    import positional_prior_bias_amd as bam
    return bam


@pytest.mark.parametrize("ref", [False, True])
def test_prior_table_ex(ref):
    """Bias and the three parameter derivatives of the table against the oracle."""
    H, d0, n = 6, -700, 1401
    rng = np.random.default_rng(42 + ref)
    if ref:
        p1, p2, p3 = rng.uniform(-2, 0.5, H), rng.uniform(-0.5, 1.5, H), rng.uniform(-0.6, 0.6, H)
        fns = (oracle.prior_bias_ref, oracle.prior_bias_ref_dtheta_alpha, oracle.prior_bias_ref_dtheta_beta,
               oracle.prior_bias_ref_dtheta_mu)
    else:
        p1, p2, p3 = np.exp(rng.uniform(0, 6, H)), rng.uniform(0.1, 2.0, H), rng.uniform(-3.3, 3.3, H) + 0.25
        fns = (oracle.prior_bias, oracle.prior_bias_dalpha, oracle.prior_bias_dbeta, oracle.prior_bias_dmu)
    p1, p2, p3 = (x.astype(np.float32) for x in (p1, p2, p3))
    got = _bam().bam_prior_table_ex(dev(p1), dev(p2), dev(p3), d0, n, prior_ref=ref)
    torch_mod().cuda.synchronize()
    d = np.arange(d0, d0 + n)
    for k, (f, g) in enumerate(zip(fns, got)):
        g = host(g)
        for h in range(H):
            r = f(d, float(p1[h]), float(p2[h]), float(p3[h]))
            tol = 2e-6 * max(1.0, float(np.max(np.abs(r))))
            within(max_abs(g[h], r), tol, f"table {k} head {h}")


def _fwd(w, o_dtype=None):
    p = params(w)
    ty = "bf16" if w.dtype == "bf16" else "f32"
    q, k, v = (dev(x, ty) for x in (w.q, w.k, w.v))
    torch = torch_mod()
    o, lse = _bam().bam_attn_fwd(q, k, v, p["alpha"], p["beta"], p["mu"], p["s"], causal=w.causal, ssmax=w.ssmax,
                                 o_dtype=o_dtype if o_dtype is not None else torch.float32,
                                 prior_ref=True)
    torch.cuda.synchronize()
    return host(o), host(lse)


@pytest.mark.parametrize("T,Dh,causal,ssmax", [(37, 64, True, True), (300, 64, True, True), (513, 64, False, True),
                                              (700, 32, True, False), (2100, 64, True, True), (200, 128, True, True)])
def test_fwd_ref_bf16(T, Dh, causal, ssmax):
    B = 1 if T > 1000 else 2
    w = wl.ref_case(900 + T, B, 3, T, Dh, "bf16", wl.CAUSAL * causal | wl.SSMAX * ssmax)
    o, lse = _fwd(w)
    O, L = oracle.attn_fwd(w.q, w.k, w.v, w.alpha, w.beta, w.mu, w.s, causal=causal, ssmax=ssmax, param="ref")
    within(max_abs(o, O), BF16_O_ABS, "max_abs(o, O)")
    within(max_abs(lse, L), BF16_LSE_ABS, "max_abs(lse, L)")


@pytest.mark.parametrize("T,Dh,causal,ssmax", [(63, 32, True, True), (200, 64, False, True), (130, 64, True, False)])
def test_fwd_ref_f32(T, Dh, causal, ssmax):
    w = wl.ref_case(950 + T, 1, 4, T, Dh, "f32", wl.CAUSAL * causal | wl.SSMAX * ssmax)
    o, lse = _fwd(w)
    O, L = oracle.attn_fwd(w.q, w.k, w.v, w.alpha, w.beta, w.mu, w.s, causal=causal, ssmax=ssmax, param="ref")
    within(normwise_rel(o, O), F32_REL, "normwise_rel(o, O)")
    within(normwise_rel(lse, L), F32_REL, "normwise_rel(lse, L)")


def test_decode_ref():
    torch = torch_mod()
    B, H, L, Dh = 3, 4, 3000, 64
    w = wl.ref_case(77, B, H, L, Dh, "bf16")
    kv_len = np.array([3000, 1, 1777], np.int32)
    rng = np.random.default_rng(5)
    q = wl.bf16_round(rng.standard_normal((B, H, Dh)).astype(np.float32))
    p = params(w)
    o, lse = _bam().bam_attn_decode(dev(q, "bf16"), dev(w.k, "bf16"), dev(w.v, "bf16"), torch.from_numpy(kv_len).cuda(),
                                    p["alpha"], p["beta"], p["mu"], p["s"], ssmax=True, o_dtype=torch.float32,
                                    prior_ref=True)
    torch.cuda.synchronize()
    O, Lse = oracle.attn_decode(q, w.k, w.v, kv_len, w.alpha, w.beta, w.mu, w.s, ssmax=True, param="ref")
    within(max_abs(host(o), O), BF16_O_ABS, "max_abs(host(o), O)")
    within(max_abs(host(lse), Lse), BF16_LSE_ABS, "max_abs(host(lse), Lse)")


def _check_bwd(w, ref):
    torch = torch_mod()
    p = params(w)
    q, k, v, do = (dev(x, "bf16") for x in (w.q, w.k, w.v, w.do))
    o, lse = _bam().bam_attn_fwd(q, k, v, p["alpha"], p["beta"], p["mu"], p["s"], causal=w.causal, ssmax=w.ssmax,
                                 o_dtype=torch.float32, prior_ref=ref)
    g = _bam().bam_attn_bwd_ex(q, k, v, o, lse, do, p["alpha"], p["beta"], p["mu"], p["s"], causal=w.causal,
                               ssmax=w.ssmax, grad_dtype=torch.float32, prior_ref=ref)
    torch.cuda.synchronize()
    got = [host(x) for x in g]
    R = oracle.attn_bwd(w.q, w.k, w.v, w.do, w.alpha, w.beta, w.mu, w.s, causal=w.causal, ssmax=w.ssmax,
                        param="ref" if ref else "alpha")
    for name, x in zip(("dq", "dk", "dv"), got[:3]):
        tol = 1e-2 * max(1.0, float(np.max(np.abs(R[name]))))
        within(max_abs(x, R[name]), tol, name)
    for name, x, A in zip(("dalpha", "dbeta", "dmu", "ds"), got[3:], ("A_alpha", "A_beta", "A_mu", "A_s")):
        err = np.abs(x - R[name])
        tol = 1e-3 * R[A] + 1e-6
        h = int(np.argmax(err / tol))
        within(err[h], tol[h], f"{name} (worst head {h})")


@pytest.mark.parametrize("T,Dh,causal,ssmax", [(64, 64, True, True), (257, 64, True, True), (130, 32, False, True),
                                              (300, 64, False, False)])
def test_bwd_ex_ref(T, Dh, causal, ssmax):
    w = wl.ref_case(1000 + T, 2, 3, T, Dh, "bf16", wl.CAUSAL * causal | wl.SSMAX * ssmax, with_grad=True)
    _check_bwd(w, True)


@pytest.mark.parametrize("T,Dh,causal,mu", [(100, 64, True, 2.5), (257, 32, False, -3.25), (300, 64, True, 0.5)])
def test_bwd_ex_alpha_form_dmu(T, Dh, causal, mu):
    """The offset gradient of the alpha-form (mu not on an integer: no cusp at a visible d)."""
    w = wl.random_case(1100 + T, 2, 3, T, Dh, "bf16", wl.CAUSAL * causal | wl.SSMAX, beta_range=(0.3, 1.6), mu=mu,
                       with_grad=True)
    _check_bwd(w, False)
