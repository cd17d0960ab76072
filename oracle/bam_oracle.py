"""Plain, slow fp64 CPU oracle for BAM attention.  TEST INFRASTRUCTURE ONLY.

Only the tests, the package smoke check and the benchmark's CPU-baseline leg may
import this module.  The product path never calls it and shares no code with it.

What it computes (the dense definition, written out; no tiling, no online
softmax, no split-KV, no distance table):

* Bayesian Attention Mechanism (stig.sh README), "Implementation Details", and the
  French summary "Résumé Technique : Mécanisme d'Attention Bayésienne (BAM)",
  "Solution Proposée : GGD-BAM": a per-head additive attention bias from a
  Generalized-Gaussian positional prior, b_h(i, j) = -|x / alpha_h|^beta_h.
  Convention adopted here: x = (i - j) - mu_h, with i the query and j the key,
  no epsilon; beta in (0, 1) is heavy-tailed, beta < 0 is the inverted prior.
* ALiBi: Attention with Linear Biases, "Code": scores = Q K^T / sqrt(d_k), then the
  bias is added, then the row softmax, then the weighted sum of V.  NNX
  ALiBi-Style Attention, "Give nearby positions a smaller penalty": the same order.
* Scalable-Softmax: the French summary ("Softmax Évolutif (SSMax)") says only that
  SSMax rescales the logits against attention fading.  Convention adopted here:
  logit_ij = c_i * (q_i.k_j / sqrt(Dh) + b_h(i, j)), c_i = s_h * ln(n_i), with n_i
  the number of keys query i sees; with SSMax off, c_i = 1 (the literal factor).
* Special values of the bias: u = |x| / alpha; u = 0 with beta > 0 gives 0;
  beta = 0 gives -1 (0^0 = 1); alpha = +inf gives u = 0; u = 0 with beta < 0 is a
  precondition violation and raises.
* lse is the natural-log log-sum-exp of the logits of a row.
* Reference parameterisation (Bayesian Attention Mechanism README, "Implementation
  Details", the formula and the AttentionPrior code): b = -e^theta_alpha *
  (|(j - i) - mu| + eps)^theta_beta with mu = e^theta_mu - e^-theta_mu and eps = 1e-5.
  The printed formula writes (i - j) - mu while the code subtracts mu from
  positions[j] - positions[i]; the two agree for mu = 0 (the default, theta_mu = 0)
  and the code's sign is adopted here.  param="ref" selects it; the alpha / beta / mu
  arrays then hold theta_alpha / theta_beta / theta_mu.
* Sandwich (attention-gym "Score Mods", "Sandwich"), param="sandwich": alpha holds the
  per-head compression ratio and beta d_bar; see prior_bias_sandwich.

Pins (tests/test_oracle_pins.py) tie this module to things other than itself:
the printed ALiBi worked example, torch's scaled_dot_product_attention on the
ALiBi / NoPE / Gaussian / square-root reductions, brute force with mpmath on
tiny inputs, closed forms on T = 2 / 3, invariants, and central finite
differences for the backward.  Every function here is pinned; none is
"parity unpinned" except the planted-key readout, which has no page value.
"""
from __future__ import annotations

import math

import numpy as np

__all__ = [
    "prior_bias", "prior_bias_dalpha", "prior_bias_dbeta", "prior_bias_dmu", "ssmax_factor",
    "REF_EPS", "ref_mu", "prior_bias_ref", "prior_bias_ref_dtheta_alpha", "prior_bias_ref_dtheta_beta",
    "prior_bias_ref_dtheta_mu", "prior_bias_sandwich", "sandwich_ratios",
    "attn_fwd", "attn_fwd_rows", "attn_decode", "attn_bwd", "attention_probs",
]


class PreconditionError(ValueError):
    """Raised where the pages' formula is undefined (0 to a negative power)."""


# --------------------------------------------------------------------------------------
# Positional prior (GGD-BAM bias) and its parameter derivatives
# --------------------------------------------------------------------------------------

def _u(d, alpha, mu):
    """u = |(d - mu) / alpha| (alpha = +inf gives 0)."""
    d = np.asarray(d, np.float64)
    x = d - float(mu)
    if math.isinf(float(alpha)):
        return np.zeros_like(x)
    return np.abs(x) / float(alpha)


def prior_bias(d, alpha, beta, mu=0.0):
    """b(d) = -u^beta, u = |(d - mu) / alpha|, for a distance d = i - j (array or scalar).

    Résumé Technique (BAM), "Solution Proposée : GGD-BAM" (the bias matrix B);
    Bayesian Attention Mechanism README, "Implementation Details" (per-head bias,
    learned scale and shape).  Special values as in the module docstring.
    """
    u = _u(d, alpha, mu)
    beta = float(beta)
    if beta == 0.0:
        return -np.ones_like(u)
    zero = u == 0.0
    if beta < 0.0 and np.any(zero):
        raise PreconditionError("bias undefined: u = 0 with beta < 0")
    out = np.zeros_like(u)
    nz = ~zero
    out[nz] = -np.power(u[nz], beta)
    return out


def prior_bias_dalpha(d, alpha, beta, mu=0.0):
    """db/dalpha = beta * u^beta / alpha (0 where u = 0 or alpha = inf)."""
    u = _u(d, alpha, mu)
    beta = float(beta)
    if math.isinf(float(alpha)):
        return np.zeros_like(u)
    out = np.zeros_like(u)
    nz = u != 0.0
    if beta < 0.0 and not np.all(nz):
        raise PreconditionError("bias undefined: u = 0 with beta < 0")
    out[nz] = beta * np.power(u[nz], beta) / float(alpha)
    return out


def prior_bias_dbeta(d, alpha, beta, mu=0.0):
    """db/dbeta = -u^beta * ln(u) (0 where u = 0 and beta >= 0)."""
    u = _u(d, alpha, mu)
    beta = float(beta)
    out = np.zeros_like(u)
    nz = u != 0.0
    if beta < 0.0 and not np.all(nz):
        raise PreconditionError("bias undefined: u = 0 with beta < 0")
    out[nz] = -np.power(u[nz], beta) * np.log(u[nz])
    return out


def prior_bias_dmu(d, alpha, beta, mu=0.0):
    """db/dmu = beta * u^beta / x with x = d - mu (0 where u = 0, beta = 0 or alpha = inf).

    The derivative of -(|x| / alpha)^beta in x is -beta u^beta / x and dx/dmu = -1.  At
    x = 0 the sign of x is taken as 0 (so the term is 0 even where the cusp of
    0 < beta < 1 makes the one-sided derivatives infinite).
    """
    x = np.asarray(d, np.float64) - float(mu)
    u = _u(d, alpha, mu)
    beta = float(beta)
    out = np.zeros_like(u)
    if beta == 0.0 or math.isinf(float(alpha)):
        return out
    nz = u != 0.0
    if beta < 0.0 and not np.all(nz):
        raise PreconditionError("bias undefined: u = 0 with beta < 0")
    out[nz] = beta * np.power(u[nz], beta) / x[nz]
    return out


# --------------------------------------------------------------------------------------
# Reference parameterisation (Bayesian Attention Mechanism README, "Implementation
# Details"): -e^theta_alpha (|(j - i) - mu| + eps)^theta_beta, mu = e^theta_mu - e^-theta_mu
# --------------------------------------------------------------------------------------

REF_EPS = 1e-5


def ref_mu(theta_mu):
    """mu = e^theta_mu - e^-theta_mu."""
    t = float(theta_mu)
    return math.exp(t) - math.exp(-t)


def _ref_x(d, theta_mu):
    """x = (j - i) - mu for a distance d = i - j."""
    return -np.asarray(d, np.float64) - ref_mu(theta_mu)


def prior_bias_ref(d, theta_alpha, theta_beta, theta_mu=0.0, eps=REF_EPS):
    """b(d) = -e^theta_alpha * (|x| + eps)^theta_beta, x = (j - i) - mu, for d = i - j."""
    g = np.abs(_ref_x(d, theta_mu)) + float(eps)
    return -math.exp(float(theta_alpha)) * np.power(g, float(theta_beta))


def prior_bias_ref_dtheta_alpha(d, theta_alpha, theta_beta, theta_mu=0.0, eps=REF_EPS):
    """db/dtheta_alpha = b."""
    return prior_bias_ref(d, theta_alpha, theta_beta, theta_mu, eps)


def prior_bias_ref_dtheta_beta(d, theta_alpha, theta_beta, theta_mu=0.0, eps=REF_EPS):
    """db/dtheta_beta = b * ln(|x| + eps)."""
    g = np.abs(_ref_x(d, theta_mu)) + float(eps)
    return prior_bias_ref(d, theta_alpha, theta_beta, theta_mu, eps) * np.log(g)


def prior_bias_ref_dtheta_mu(d, theta_alpha, theta_beta, theta_mu=0.0, eps=REF_EPS):
    """db/dtheta_mu = (db/dmu)(dmu/dtheta_mu): db/dmu = -b theta_beta sign(x) / (|x| + eps)
    (sign(0) = 0) and dmu/dtheta_mu = e^theta_mu + e^-theta_mu."""
    x = _ref_x(d, theta_mu)
    g = np.abs(x) + float(eps)
    b = prior_bias_ref(d, theta_alpha, theta_beta, theta_mu, eps)
    t = float(theta_mu)
    return -b * float(theta_beta) * np.sign(x) / g * (math.exp(t) + math.exp(-t))


# --------------------------------------------------------------------------------------
# Sandwich relative-position bias (attention-gym "Score Mods", "Sandwich"): the
# position-position inner product of sinusoidal embeddings, sum_i cos(d w_i) / ratio_h,
# w_i = 1 / 10000^(2 i / d_bar), ratio_h = 8 (h + 1) / H, no learned parameters.
# Reading taken: i runs over the d_bar / 2 frequencies of a d_bar-dimensional
# sinusoidal embedding, i = 0 .. d_bar / 2 - 1.
# --------------------------------------------------------------------------------------

def sandwich_ratios(H):
    """ratio_h = 8 (h + 1) / H."""
    return np.array([8.0 * (h + 1) / H for h in range(H)], np.float64)


def prior_bias_sandwich(d, ratio, d_bar=128.0):
    """b(d) = sum_{i < d_bar/2} cos(d / 10000^(2 i / d_bar)) / ratio."""
    d = np.asarray(d, np.float64)
    nf = int(float(d_bar)) // 2
    out = np.zeros_like(d)
    for i in range(nf):
        out += np.cos(d / 10000.0 ** (2.0 * i / float(d_bar)))
    return out / float(ratio)


def _zero_deriv(d, *args):
    return np.zeros_like(np.asarray(d, np.float64))


def _bias_fns(param):
    """(bias, d/dp1, d/dp2, d/dp3) of a parameterisation, each f(d, p1, p2, p3)."""
    if param == "alpha":
        return prior_bias, prior_bias_dalpha, prior_bias_dbeta, prior_bias_dmu
    if param == "ref":
        return (prior_bias_ref, prior_bias_ref_dtheta_alpha, prior_bias_ref_dtheta_beta,
                prior_bias_ref_dtheta_mu)
    if param == "sandwich":   # alpha = ratio_h, beta = d_bar; no trained parameters
        return (lambda d, r, db, _m: prior_bias_sandwich(d, r, db), _zero_deriv, _zero_deriv, _zero_deriv)
    raise ValueError(f"unknown parameterisation {param!r}")


def ssmax_factor(n, s, ssmax: bool):
    """c = s * ln(n) with Scalable-Softmax on, the literal 1 with it off.

    Résumé Technique (BAM), "Solution Proposée : GGD-BAM" (SSMax rescales logits);
    the formula is the convention stated in the module docstring.
    """
    n = np.asarray(n, np.float64)
    if not ssmax:
        return np.ones_like(n)
    return float(s) * np.log(n)


# --------------------------------------------------------------------------------------
# Forward
# --------------------------------------------------------------------------------------

def _head_logits(q, k, rows, alpha, beta, mu, s, causal, ssmax, nkeys=None, param="alpha"):
    """Logits l[r, j] for the query rows `rows` of one head, -inf where not visible.

    q: [T, Dh] (or [R, Dh] already sliced when rows is given as positions),
    k: [Tk, Dh].  Returns (logits, c, scaled_scores, bias) for the selected rows.
    """
    Tk, Dh = k.shape
    i = np.asarray(rows, np.int64)[:, None]
    j = np.arange(Tk, dtype=np.int64)[None, :]
    S = (q @ k.T) / math.sqrt(Dh)                        # content score, q.k / sqrt(Dh)
    visible = (j <= i) if causal else np.ones((i.shape[0], Tk), bool)
    if nkeys is not None:
        visible &= j < nkeys
    n = visible.sum(axis=1).astype(np.float64)           # keys visible to each query
    c = ssmax_factor(n, s, ssmax)[:, None]
    d = np.broadcast_to(i - j, visible.shape)
    bias = np.full(visible.shape, np.nan)
    bias[visible] = _bias_fns(param)[0](d[visible], alpha, beta, mu)
    L = np.full(visible.shape, -np.inf)
    L[visible] = (c * (S + bias))[visible]
    return L, c, S, bias


def _softmax_rows(L):
    m = L.max(axis=1, keepdims=True)
    E = np.exp(L - m)
    Z = E.sum(axis=1, keepdims=True)
    return E / Z, (m + np.log(Z))[:, 0]


def attention_probs(q, k, alpha, beta, mu, s, causal=True, ssmax=False, rows=None, param="alpha"):
    """Attention weights P [R, Tk] of one head (q: [T, Dh], k: [Tk, Dh])."""
    q = np.asarray(q, np.float64)
    k = np.asarray(k, np.float64)
    rows = np.arange(q.shape[0]) if rows is None else np.asarray(rows)
    L, _, _, _ = _head_logits(q[rows], k, rows, alpha, beta, mu, s, causal, ssmax, param=param)
    P, _ = _softmax_rows(L)
    return P


def attn_fwd_rows(q, k, v, rows, alpha, beta, mu, s, causal=True, ssmax=False, chunk=256, param="alpha"):
    """O and lse of the query rows `rows` of one head, dense per row block.

    q, k, v: [T, Dh] arrays of one (b, h).  Returns O [R, Dh], lse [R] (fp64).
    """
    q = np.asarray(q, np.float64)
    k = np.asarray(k, np.float64)
    v = np.asarray(v, np.float64)
    rows = np.asarray(rows, np.int64)
    O = np.empty((rows.size, v.shape[1]))
    lse = np.empty(rows.size)
    for r0 in range(0, rows.size, chunk):
        rr = rows[r0:r0 + chunk]
        L, _, _, _ = _head_logits(q[rr], k, rr, alpha, beta, mu, s, causal, ssmax, param=param)
        P, l = _softmax_rows(L)
        O[r0:r0 + chunk] = P @ v
        lse[r0:r0 + chunk] = l
    return O, lse


def attn_fwd(q, k, v, alpha, beta, mu, s, causal=True, ssmax=False, heads=None, param="alpha"):
    """Full forward: q, k, v [B, H, T, Dh] -> O [B, H, T, Dh], lse [B, H, T] (fp64).

    `heads` optionally restricts the work to a list of (b, h) pairs; other entries
    of the result are NaN.
    """
    q = np.asarray(q)
    B, H, T, Dh = q.shape
    O = np.full((B, H, T, v.shape[-1]), np.nan)
    lse = np.full((B, H, T), np.nan)
    pairs = heads if heads is not None else [(b, h) for b in range(B) for h in range(H)]
    rows = np.arange(T)
    for b, h in pairs:
        O[b, h], lse[b, h] = attn_fwd_rows(q[b, h], k[b, h], v[b, h], rows,
                                           alpha[h], beta[h], mu[h], s[h], causal, ssmax, param=param)
    return O, lse


def attn_decode(q, k_cache, v_cache, kv_len, alpha, beta, mu, s, ssmax=True, heads=None, param="alpha"):
    """One query row per (b, h) against a KV cache.

    q [B, H, Dh]; caches [B, H, Lmax, Dh]; kv_len [B].  The cache holds the current
    token, so the query sits at position i = kv_len - 1 and sees n = kv_len keys
    (causal).  Returns O [B, H, Dh], lse [B, H].
    """
    B, H, Dh = q.shape
    O = np.full((B, H, v_cache.shape[-1]), np.nan)
    lse = np.full((B, H), np.nan)
    pairs = heads if heads is not None else [(b, h) for b in range(B) for h in range(H)]
    for b, h in pairs:
        n = int(kv_len[b])
        qi = np.asarray(q[b, h], np.float64)[None, :]
        kk = np.asarray(k_cache[b, h, :n], np.float64)
        vv = np.asarray(v_cache[b, h, :n], np.float64)
        L, _, _, _ = _head_logits(qi, kk, np.array([n - 1]), alpha[h], beta[h], mu[h], s[h],
                                  True, ssmax, param=param)
        P, l = _softmax_rows(L)
        O[b, h] = (P @ vv)[0]
        lse[b, h] = l[0]
    return O, lse


# --------------------------------------------------------------------------------------
# Backward
# --------------------------------------------------------------------------------------

def attn_bwd(q, k, v, do, alpha, beta, mu, s, causal=True, ssmax=False, heads=None, param="alpha"):
    """Gradients of L = sum(O * dO) for every input of the forward.

    Returns a dict with dq, dk, dv [B, H, T, Dh], dalpha, dbeta, dmu, ds [H] and the
    conditioning scales A_alpha, A_beta, A_mu, A_s [H] (sum of |term| of each parameter
    sum, used to size tolerances of the cancelling reductions).  With param="ref",
    dalpha / dbeta / dmu are the gradients in theta_alpha / theta_beta / theta_mu.

    Chain rule on logit_ij = c_i (S_ij + b_ij), S = q.k / sqrt(Dh):
      dP = dO V^T, D_i = sum_j P_ij dP_ij, dZ = P * (dP - D)  (dZ = dL/dlogit),
      dV = P^T dO, dq_i = c_i sum_j dZ_ij k_j / sqrt(Dh), dk_j = sum_i c_i dZ_ij q_i / sqrt(Dh),
      dalpha = sum c_i dZ_ij db/dalpha, dbeta = sum c_i dZ_ij db/dbeta, dmu likewise,
      ds = sum dZ_ij ln(n_i) (S_ij + b_ij)  (SSMax on; 0 otherwise).
    Bayesian Attention Mechanism README, "Implementation Details": alpha's scale
    and beta are the trained per-head parameters.
    """
    B, H, T, Dh = q.shape
    dq = np.full(q.shape, np.nan)
    dk = np.full(k.shape, np.nan)
    dv = np.full(v.shape, np.nan)
    dalpha = np.zeros(H)
    dbeta = np.zeros(H)
    dmu = np.zeros(H)
    ds = np.zeros(H)
    A = np.zeros((4, H))
    _, f_da, f_db, f_dm = _bias_fns(param)
    pairs = heads if heads is not None else [(b, h) for b in range(B) for h in range(H)]
    rows = np.arange(T)
    for b, h in pairs:
        qq = np.asarray(q[b, h], np.float64)
        kk = np.asarray(k[b, h], np.float64)
        vv = np.asarray(v[b, h], np.float64)
        dd = np.asarray(do[b, h], np.float64)
        L, c, S, bias = _head_logits(qq, kk, rows, alpha[h], beta[h], mu[h], s[h], causal, ssmax,
                                     param=param)
        P, _ = _softmax_rows(L)
        O = P @ vv
        dP = dd @ vv.T
        D = (dd * O).sum(axis=1, keepdims=True)
        dZ = P * (dP - D)
        visible = np.isfinite(L)
        dv[b, h] = P.T @ dd
        G = c * dZ / math.sqrt(Dh)
        dq[b, h] = G @ kk
        dk[b, h] = G.T @ qq
        i = rows[:, None]
        j = np.arange(T)[None, :]
        d = np.broadcast_to(i - j, L.shape)[visible]
        cz = (c * dZ)[visible]
        ta = cz * f_da(d, alpha[h], beta[h], mu[h])
        tb = cz * f_db(d, alpha[h], beta[h], mu[h])
        tm = cz * f_dm(d, alpha[h], beta[h], mu[h])
        dalpha[h] += ta.sum()
        dbeta[h] += tb.sum()
        dmu[h] += tm.sum()
        A[0, h] += np.abs(ta).sum()
        A[1, h] += np.abs(tb).sum()
        A[3, h] += np.abs(tm).sum()
        if ssmax:
            n = visible.sum(axis=1).astype(np.float64)[:, None]
            lnn = np.broadcast_to(np.log(n), L.shape)[visible]
            tsum = dZ[visible] * lnn * (S[visible] + bias[visible])
            ds[h] += tsum.sum()
            A[2, h] += np.abs(tsum).sum()
    return dict(dq=dq, dk=dk, dv=dv, dalpha=dalpha, dbeta=dbeta, dmu=dmu, ds=ds,
                A_alpha=A[0], A_beta=A[1], A_s=A[2], A_mu=A[3])
