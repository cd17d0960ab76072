"""PyTorch training integration of the BAM attention kernels.

``bam_attention`` is a ``torch.autograd.Function`` over ``bam_attn_fwd`` /
``bam_attn_bwd_ex``: gradients flow to q, k, v and to the per-head prior parameters
(and to the SSMax strength s).  ``BamAttention`` is an ``nn.Module`` that owns those
parameters the way the pages' ``AttentionPrior`` module does ("Bayesian Attention
Mechanism" README, "Implementation Details"): theta_alpha and theta_beta trained per head,
theta_mu held fixed unless asked for, and the bias in the reference form
-e^theta_alpha (|(j - i) - mu| + eps)^theta_beta, mu = e^theta_mu - e^-theta_mu.  Unlike
that module it never materialises the (1, H, T, T) bias: the kernels read a per-head
distance table.

Every step runs in libbam's HIP kernels; this file only routes tensors and gradients.
"""
from __future__ import annotations

import math

import torch

from . import bam_attn_bwd_ex, bam_attn_fwd

__all__ = ["bam_attention", "BamAttention"]


class _BamAttentionFn(torch.autograd.Function):
    @staticmethod
    def forward(ctx, q, k, v, alpha, beta, mu, s, causal, ssmax, prior):
        o, lse = bam_attn_fwd(q, k, v, alpha, beta, mu, s, causal=causal, ssmax=ssmax, prior=prior)
        ctx.save_for_backward(q, k, v, o, lse, alpha, beta, mu, s)
        ctx.flags = (causal, ssmax, prior)
        return o

    @staticmethod
    def backward(ctx, do):
        q, k, v, o, lse, alpha, beta, mu, s = ctx.saved_tensors
        causal, ssmax, prior = ctx.flags
        dq, dk, dv, dalpha, dbeta, dmu, ds = bam_attn_bwd_ex(
            q, k, v, o, lse, do.contiguous(), alpha, beta, mu, s, causal=causal, ssmax=ssmax, prior=prior)
        want = ctx.needs_input_grad
        return (dq if want[0] else None, dk if want[1] else None, dv if want[2] else None,
                dalpha if want[3] else None, dbeta if want[4] else None, dmu if want[5] else None,
                ds if (want[6] and ssmax) else None, None, None, None)


def bam_attention(q, k, v, alpha, beta, mu, s=None, causal=True, ssmax=True, prior_ref=True, prior=None):
    """Differentiable BAM attention.  q, k, v: [B, H, T, Dh] (bf16); alpha, beta, mu, s:
    float32 [H] (theta_alpha, theta_beta, theta_mu with prior_ref).  Returns O [B, H, T, Dh].
    prior: "ref", "alpha" or "sandwich" (alpha = ratio_h, beta = d_bar, no parameter
    gradients); when given it overrides prior_ref."""
    if prior is None:
        prior = "ref" if prior_ref else "alpha"
    if mu is None:
        mu = torch.zeros_like(alpha)
    if s is None:
        if ssmax:
            raise ValueError("ssmax needs s")
        s = torch.ones_like(alpha)
    return _BamAttentionFn.apply(q.contiguous(), k.contiguous(), v.contiguous(), alpha, beta, mu, s, causal,
                                 ssmax, prior)


def _alibi_slopes(n_heads):
    """2^(-8 (h + 1) / H): the ALiBi page's get_slopes ("ALiBi: Attention with Linear
    Biases", "Code")."""
    return [2.0 ** (-8.0 * (h + 1) / n_heads) for h in range(n_heads)]


# Initial values of the per-head prior parameters by option name, as the pages'
# AttentionPrior module offers them ("Bayesian Attention Mechanism" README, "Implementation
# Details"); a number instead of a name starts every head at that number.
#
#   parameter     option     initial value of head h (H heads)
#   theta_alpha   "slope"    2^(-8 (h + 1) / H), the ALiBi slopes
#   theta_alpha   "sampled"  exp(z_h), z_h standard normal
#   theta_beta    "linear"   h / (H - 1), evenly from 0 to 1
#   theta_beta    "sampled"  z_h, standard normal
#   theta_beta    (not trained)  1
#   theta_mu      a number only
_NAMED_INIT = {
    ("theta_alpha", "slope"): lambda H, gen: torch.tensor(_alibi_slopes(H), dtype=torch.float32),
    ("theta_alpha", "sampled"): lambda H, gen: torch.randn(H, generator=gen, dtype=torch.float32).exp(),
    ("theta_beta", "linear"): lambda H, gen: torch.linspace(0, 1, H, dtype=torch.float32),
    ("theta_beta", "sampled"): lambda H, gen: torch.randn(H, generator=gen, dtype=torch.float32),
}


def _initial(name, option, H, generator, device):
    if isinstance(option, str):
        if (name, option) not in _NAMED_INIT:
            raise ValueError(f"{name}: unknown initialisation {option!r}")
        return _NAMED_INIT[(name, option)](H, generator).to(device)
    return torch.full((H,), float(option), dtype=torch.float32, device=device)


class BamAttention(torch.nn.Module):
    """Causal attention with a trained BAM prior and SSMax, on the HIP kernels.

    Initialisation options (the table above _NAMED_INIT): theta_alpha_init "slope",
    "sampled" or a number; theta_beta_init "linear", "sampled" or a number (fixed at 1 when
    train_theta_beta is False); theta_mu_init a number, trained only with train_theta_mu.
    s (SSMax strength, one per head) starts at 1 / ln(max_seq_len), so the SSMax factor
    s ln(n) is 1 at the training context length; the pages give no initial value.

    At short steps the host side can outlast the kernels: autograd's per-device worker
    thread costs two thread hand-offs per backward.  Running the backward on the calling
    thread (``torch.autograd.set_multithreading_enabled(False)``) took the training-shape
    step from about 185 to 131 us on one MI355X, where the kernels take about 135 us.
    """

    def __init__(self, n_heads, max_seq_len=512, theta_alpha_init="slope", theta_beta_init="linear",
                 theta_mu_init=0.0, train_theta_alpha=True, train_theta_beta=True, train_theta_mu=False,
                 ssmax=True, train_s=True, device=None, generator=None):
        super().__init__()
        H = n_heads
        f32 = dict(dtype=torch.float32, device=device)   # for s below
        ta = _initial("theta_alpha", theta_alpha_init, H, generator, device)
        tb = _initial("theta_beta", theta_beta_init if train_theta_beta else 1.0, H, generator, device)
        tm = _initial("theta_mu", float(theta_mu_init), H, generator, device)
        self.theta_alpha = torch.nn.Parameter(ta, requires_grad=train_theta_alpha)
        self.theta_beta = torch.nn.Parameter(tb, requires_grad=train_theta_beta)
        self.theta_mu = torch.nn.Parameter(tm, requires_grad=train_theta_mu)
        self.ssmax = ssmax
        self.s = torch.nn.Parameter(torch.full((H,), 1.0 / math.log(max(max_seq_len, 2)), **f32),
                                    requires_grad=ssmax and train_s)

    def forward(self, q, k, v, causal=True):
        return bam_attention(q, k, v, self.theta_alpha, self.theta_beta, self.theta_mu,
                             self.s if self.ssmax else None, causal=causal, ssmax=self.ssmax, prior_ref=True)
