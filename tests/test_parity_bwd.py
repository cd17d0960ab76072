"""GPU parity of the backward (bam_attn_bwd) against the fp64 oracle.

Tolerances: dQ, dK, dV: max |d - ref| <= 1e-2 * max(1, max |ref|) per tensor; per-head
dalpha, dbeta, ds: |d - ref| <= 1e-3 * A_h (A_h = sum of |terms| of that head's sum, the
scale the cancelling reduction is conditioned on) + 1e-6."""
import numpy as np
import pytest

import oracle
from gpu_util import within
from gpu_util import dev, host, max_abs, params, torch_mod
from positional_prior_bias_amd import workloads as wl

pytestmark = pytest.mark.gpu


def _bam():
    import positional_prior_bias_amd as bam
    return bam


def run_bwd(w):
    torch = torch_mod()
    p = params(w)
    q, k, v, do = (dev(x, "bf16") for x in (w.q, w.k, w.v, w.do))
    o, lse = _bam().bam_attn_fwd(q, k, v, p["alpha"], p["beta"], p["mu"], p["s"], causal=w.causal, ssmax=w.ssmax,
                                 o_dtype=torch.float32)
    g = _bam().bam_attn_bwd(q, k, v, o, lse, do, p["alpha"], p["beta"], p["mu"], p["s"], causal=w.causal,
                            ssmax=w.ssmax, grad_dtype=torch.float32)
    torch.cuda.synchronize()
    return [host(x) for x in g]


def check(w, got):
    ref = oracle.attn_bwd(w.q, w.k, w.v, w.do, w.alpha, w.beta, w.mu, w.s, causal=w.causal, ssmax=w.ssmax)
    for name, x in zip(("dq", "dk", "dv"), got[:3]):
        r = ref[name]
        tol = 1e-2 * max(1.0, float(np.max(np.abs(r))))
        within(max_abs(x, r), tol, name)
    for name, x, A in zip(("dalpha", "dbeta", "ds"), got[3:], ("A_alpha", "A_beta", "A_s")):
        err = np.abs(x - ref[name])
        tol = 1e-3 * ref[A] + 1e-6
        h = int(np.argmax(err / tol))
        within(err[h], tol[h], f"{name} (worst head {h})")


@pytest.mark.parametrize("T,Dh,causal,ssmax,br,mu", [
    (1, 64, True, True, (0.2, 1.2), 0.0),
    (5, 32, False, True, (0.2, 1.2), 0.0),
    (64, 64, True, True, (0.2, 1.2), 0.0),
    (100, 64, True, False, (-0.8, -0.1), -0.5),
    (130, 32, False, False, (0.3, 1.5), 0.0),
    (257, 64, True, True, (0.1, 0.9), 0.0),
    (300, 64, False, True, (-0.8, -0.1), -0.5),
    (600, 64, True, True, (0.2, 1.2), 0.0),       # T > 512: the windows come from the table
    (700, 32, False, True, (-0.8, -0.1), -0.5),
])
def test_bwd_random(T, Dh, causal, ssmax, br, mu):
    w = wl.random_case(300 + T, 2, 3, T, Dh, "bf16", wl.CAUSAL * causal | wl.SSMAX * ssmax, beta_range=br, mu=mu,
                       with_grad=True)
    check(w, run_bwd(w))


def test_bwd_training_shape():
    """B=32, H=12, T=512, Dh=64 with dO from its own seed; every head."""
    w = wl.training_shape(with_grad=True)
    check(w, run_bwd(w))
