"""GPU parity at the special values and ranges of the hot path, against the fp64 oracle.

* beta = 0 (the bias is the constant -1: 0^0 = 1) and alpha = +inf (u = 0, NoPE) through
  the distance table, the bf16 and fp32 forward and the backward, where dbeta = -sum c dZ ln u
  at beta = 0 and every parameter derivative vanishes at alpha = +inf.
* The bfloat16 range of V: the PV product runs on bf16 MFMA, so V with entries near 6e4
  (beyond float16's largest value, 65504, for the largest of them) and V scaled by 2^-16
  (below float16's normal range) are computed like unit-scale V.  The output bar (1e-2 for
  unit-scale values) is applied in V's unit: 1e-2 * scale.
* One dominant key plus a flat tail of keys weighing about 2^-20 of it each, at T = 32768:
  the tail carries 3% of the row's mass, and lse must hold its 1e-3 bar.

Tolerances are the ones the other parity tests state (bf16: max |O - ref| <= 1e-2 on the
fp32 output, |lse - ref| <= 1e-3; fp32: normwise relative 1e-5; gradients: 1e-2 max(1,
max|ref|) per tensor and 1e-3 A_h + 1e-6 per head)."""
import numpy as np
import pytest

import oracle
from gpu_util import within
from gpu_util import BF16_LSE_ABS, BF16_O_ABS, F32_REL, dev, host, lse_rel, max_abs, normwise_rel, params, torch_mod
from positional_prior_bias_amd import workloads as wl

pytestmark = pytest.mark.gpu


def _bam():
    import positional_prior_bias_amd as bam
    return bam


def _special_heads(w):
    """Heads 0 and 1: beta = 0 (alpha kept); head 2: alpha = +inf; the rest as drawn."""
    w.beta[0] = 0.0
    w.beta[1] = 0.0
    w.alpha[2] = np.inf
    return w


def test_table_beta0_and_alpha_inf():
    """bam_prior_table_ex against the oracle's bias and derivatives at beta = 0 (with and
    without an offset) and alpha = +inf."""
    torch = torch_mod()
    alpha = np.array([3.0, 11.5, np.inf, np.inf, 7.0], np.float32)
    beta = np.array([0.0, 0.0, 0.7, 0.4, 1.3], np.float32)
    mu = np.array([0.0, -0.5, 0.0, 0.25, 0.0], np.float32)
    d0, n = -300, 601
    got = _bam().bam_prior_table_ex(dev(alpha), dev(beta), dev(mu), d0, n)
    torch.cuda.synchronize()
    d = np.arange(d0, d0 + n)
    fns = (oracle.prior_bias, oracle.prior_bias_dalpha, oracle.prior_bias_dbeta, oracle.prior_bias_dmu)
    for kind, (f, g) in enumerate(zip(fns, got)):
        g = host(g)
        for h in range(alpha.size):
            r = f(d, float(alpha[h]), float(beta[h]), float(mu[h]))
            tol = 2e-6 * max(1.0, float(np.max(np.abs(r))))
            within(max_abs(g[h], r), tol, f"table {kind} head {h}")


@pytest.mark.parametrize("T,Dh,causal,ssmax,dtype", [(70, 64, True, True, "bf16"), (257, 64, False, True, "bf16"),
                                                     (300, 32, True, False, "bf16"), (1500, 64, True, True, "bf16"),
                                                     (130, 32, True, True, "f32"), (65, 64, False, False, "f32")])
def test_fwd_beta0_alpha_inf(T, Dh, causal, ssmax, dtype):
    torch = torch_mod()
    w = _special_heads(wl.random_case(1700 + T, 2, 4, T, Dh, dtype, wl.CAUSAL * causal | wl.SSMAX * ssmax))
    p = params(w)
    q, k, v = (dev(x, dtype) for x in (w.q, w.k, w.v))
    o, lse = _bam().bam_attn_fwd(q, k, v, p["alpha"], p["beta"], p["mu"], p["s"], causal=causal, ssmax=ssmax,
                                 o_dtype=torch.float32)
    torch.cuda.synchronize()
    O, L = oracle.attn_fwd(w.q, w.k, w.v, w.alpha, w.beta, w.mu, w.s, causal=causal, ssmax=ssmax)
    if dtype == "bf16":
        within(max_abs(host(o), O), BF16_O_ABS, "O")
        within(max_abs(host(lse), L), BF16_LSE_ABS, "lse")
    else:
        within(normwise_rel(host(o), O), F32_REL, "O normwise")
        within(lse_rel(host(lse), L), F32_REL, "lse rel")
    # beta = 0 adds the same constant to every logit of a row: O equals the NoPE head's O
    # for the same inputs (the GPU against itself; each is within the bar of the oracle)
    a2 = w.alpha.copy()
    a2[0] = a2[1] = np.inf
    o2, _ = _bam().bam_attn_fwd(q, k, v, dev(a2), p["beta"], p["mu"], p["s"], causal=causal, ssmax=ssmax,
                                o_dtype=torch.float32)
    torch.cuda.synchronize()
    e2 = max_abs(host(o)[:, :2], host(o2)[:, :2])
    bar = 2 * BF16_O_ABS if dtype == "bf16" else 2e-5 * max(1.0, float(np.abs(O).max()))
    within(e2, bar, "beta = 0 against NoPE")


@pytest.mark.parametrize("T,Dh,causal,ssmax", [(64, 64, True, True), (200, 32, False, True), (300, 64, True, False),
                                               (513, 64, True, True)])
def test_bwd_beta0_alpha_inf(T, Dh, causal, ssmax):
    torch = torch_mod()
    w = _special_heads(wl.random_case(1900 + T, 2, 4, T, Dh, "bf16", wl.CAUSAL * causal | wl.SSMAX * ssmax,
                                      mu=-0.5, with_grad=True))
    p = params(w)
    q, k, v, do = (dev(x, "bf16") for x in (w.q, w.k, w.v, w.do))
    o, lse = _bam().bam_attn_fwd(q, k, v, p["alpha"], p["beta"], p["mu"], p["s"], causal=causal, ssmax=ssmax,
                                 o_dtype=torch.float32)
    g = _bam().bam_attn_bwd_ex(q, k, v, o, lse, do, p["alpha"], p["beta"], p["mu"], p["s"], causal=causal,
                               ssmax=ssmax, grad_dtype=torch.float32)
    torch.cuda.synchronize()
    got = [host(x) for x in g]
    ref = oracle.attn_bwd(w.q, w.k, w.v, w.do, w.alpha, w.beta, w.mu, w.s, causal=causal, ssmax=ssmax)
    for name, x in zip(("dq", "dk", "dv"), got[:3]):
        tol = 1e-2 * max(1.0, float(np.max(np.abs(ref[name]))))
        within(max_abs(x, ref[name]), tol, name)
    for name, x, A in zip(("dalpha", "dbeta", "dmu", "ds"), got[3:], ("A_alpha", "A_beta", "A_mu", "A_s")):
        err = np.abs(x - ref[name])
        tol = 1e-3 * ref[A] + 1e-6
        h = int(np.argmax(err / tol))
        within(err[h], tol[h], f"{name} (worst head {h})")
    # the NoPE head's parameter derivatives vanish
    assert got[3][2] == 0.0 and got[4][2] == 0.0 and got[5][2] == 0.0, (got[3][2], got[4][2], got[5][2])


@pytest.mark.parametrize("scale", [6.0e4 / 5.5, 2.0 ** -16])
def test_fwd_v_range(scale):
    """V = scale * N(0, 1) rounded to bf16: largest |V| near 6e4, or entries around 2^-16."""
    torch = torch_mod()
    w = wl.random_case(2100, 2, 3, 777, 64, "bf16", wl.CAUSAL | wl.SSMAX)
    w.v = wl.bf16_round(w.v * np.float32(scale))
    p = params(w)
    q, k, v = (dev(x, "bf16") for x in (w.q, w.k, w.v))
    o, lse = _bam().bam_attn_fwd(q, k, v, p["alpha"], p["beta"], p["mu"], p["s"], causal=True, ssmax=True,
                                 o_dtype=torch.float32)
    torch.cuda.synchronize()
    O, L = oracle.attn_fwd(w.q, w.k, w.v, w.alpha, w.beta, w.mu, w.s, causal=True, ssmax=True)
    oh = host(o)
    assert np.all(np.isfinite(oh))
    within(max_abs(oh, O), BF16_O_ABS * scale, f"O (max |V| {np.abs(w.v).max():.3e})")
    within(max_abs(host(lse), L), BF16_LSE_ABS, "lse")


def test_dominant_key_flat_tail_T32768():
    """B=1, H=2, T=32768, Dh=64, NoPE, SSMax off.  Every query is 8 e_0; the key at
    position 100 has 13.875 in dimension 0 and every other key 0 there, so each row from
    100 on has one logit of 13.875 and all others 0: each tail key weighs e^-13.875 (about
    2^-20) of the dominant one, and the tail holds about 3% of a late row's mass."""
    torch = torch_mod()
    B, H, T, Dh, p_ = 1, 2, 32768, 64, 100
    rng = np.random.default_rng(2200)
    q = np.zeros((B, H, T, Dh), np.float32)
    q[..., 0] = 8.0
    k = wl.bf16_round(rng.standard_normal((B, H, T, Dh), dtype=np.float32))
    k[..., 0] = 0.0
    k[:, :, p_, 0] = 13.875
    v = wl.bf16_round(rng.standard_normal((B, H, T, Dh), dtype=np.float32))
    alpha = np.full(H, np.inf, np.float32)
    beta = np.ones(H, np.float32)
    mu = np.zeros(H, np.float32)
    s = np.ones(H, np.float32)
    o, lse = _bam().bam_attn_fwd(dev(q, "bf16"), dev(k, "bf16"), dev(v, "bf16"), dev(alpha), dev(beta), dev(mu),
                                 dev(s), causal=True, ssmax=False, o_dtype=torch.float32)
    torch.cuda.synchronize()
    rows = np.unique(np.concatenate([np.arange(0, 300), np.arange(T - 300, T),
                                     rng.integers(0, T, 400)]))
    oh, lh = host(o), host(lse)
    wo = wl_ = 0.0
    for h in range(H):
        O, L = oracle.attn_fwd_rows(q[0, h], k[0, h], v[0, h], rows, alpha[h], beta[h], mu[h], s[h], causal=True,
                                    ssmax=False)
        wo = max(wo, max_abs(oh[0, h, rows], O))
        wl_ = max(wl_, max_abs(lh[0, h, rows], L))
    # the last row's lse in closed form: ln(e^13.875 + 32767)
    closed = np.log(np.exp(13.875) + (T - 1))
    within(abs(lh[0, 0, T - 1] - closed), BF16_LSE_ABS, "last row lse against ln(e^13.875 + 32767)")
    within(wo, BF16_O_ABS, "O")
    within(wl_, BF16_LSE_ABS, "lse")


def test_steep_prior_stays_finite():
    """beta = 20, alpha = 1: u^beta overflows float32 from |d| of about 84 on, so those
    biases are -inf (weight exactly 0) and the parameter derivatives saturate; a tile of
    far keys gives a running max near -2^34, where half an ulp of the max is 2^10.  The
    forward and the backward must stay finite and match the oracle (in fp64 nothing
    overflows and those terms are exactly 0)."""
    torch = torch_mod()
    T, Dh, H = 300, 64, 2
    w = wl.random_case(2300, 1, H, T, Dh, "bf16", wl.CAUSAL | wl.SSMAX, with_grad=True)
    w.alpha[:] = 1.0
    w.beta[:] = np.array([20.0, 1.0], np.float32)
    p = params(w)
    q, k, v, do = (dev(x, "bf16") for x in (w.q, w.k, w.v, w.do))
    o, lse = _bam().bam_attn_fwd(q, k, v, p["alpha"], p["beta"], p["mu"], p["s"], causal=True, ssmax=True,
                                 o_dtype=torch.float32)
    torch.cuda.synchronize()
    O, L = oracle.attn_fwd(w.q, w.k, w.v, w.alpha, w.beta, w.mu, w.s, causal=True, ssmax=True)
    assert np.all(np.isfinite(host(o))) and np.all(np.isfinite(host(lse)))
    within(max_abs(host(o), O), BF16_O_ABS, "O")
    within(max_abs(host(lse), L), BF16_LSE_ABS, "lse")
    g = _bam().bam_attn_bwd_ex(q, k, v, o, lse, do, p["alpha"], p["beta"], p["mu"], p["s"], causal=True,
                               ssmax=True, grad_dtype=torch.float32)
    torch.cuda.synchronize()
    got = [host(x) for x in g]
    assert all(np.all(np.isfinite(x)) for x in got)
    ref = oracle.attn_bwd(w.q, w.k, w.v, w.do, w.alpha, w.beta, w.mu, w.s, causal=True, ssmax=True)
    for name, x, A in zip(("dalpha", "dbeta", "dmu", "ds"), got[3:], ("A_alpha", "A_beta", "A_mu", "A_s")):
        err = np.abs(x - ref[name])
        tol = 1e-3 * ref[A] + 1e-6
        h = int(np.argmax(err / tol))
        within(err[h], tol[h], f"{name} (worst head {h})")
