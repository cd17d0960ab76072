"""Structural GPU checks that follow from the definition of attention alone
("ALiBi: Attention with Linear Biases", "Code": O = softmax_j(logit) V):

- V = 1 gives O = 1, since every row of the softmax sums to one;
- V = I (T <= Dh, value row j the unit vector e_j) gives O = P, the attention matrix
  itself: compared entry by entry with the fp64 oracle's matrix, masked entries exactly
  zero, rows summing to one;
- the decode result does not depend on how the key range is cut into splits (the split
  size follows from B * H, so the same heads decoded at B = 1 and inside a batch of 8 are
  cut differently).

Bounds: on the fp32 path 1e-5.  On the bf16 path each weight is rounded to bf16 for the PV
product while l sums the unrounded weights, so O_ij = rne(p_ij) / l with |rne(p) - p| <=
2^-8 p (8-bit significand): |O - 1| <= 2^-8 for V = 1 and |O_ij - P_ij| <= 2^-8 P_ij for
V = I, plus float32 rounding (1e-5 of P for the exponent argument and the sum l)."""
import numpy as np
import pytest

import oracle
from gpu_util import dev, host, max_abs, params, torch_mod, within
from positional_prior_bias_amd import workloads as wl

pytestmark = pytest.mark.gpu

BF16_U = 2.0 ** -8


def _bam():
    import positional_prior_bias_amd as bam
    return bam


def _fwd(w, v):
    torch = torch_mod()
    p = params(w)
    q, k = dev(w.q, w.dtype), dev(w.k, w.dtype)
    o, lse = _bam().bam_attn_fwd(q, k, dev(v, w.dtype), p["alpha"], p["beta"], p["mu"], p["s"], causal=w.causal,
                                 ssmax=w.ssmax, o_dtype=torch.float32)
    torch.cuda.synchronize()
    return host(o), host(lse)


@pytest.mark.parametrize("T,Dh,causal,dtype", [(1, 64, True, "bf16"), (77, 32, True, "bf16"),
                                               (300, 64, False, "bf16"), (513, 64, True, "bf16"),
                                               (1500, 64, True, "bf16"), (700, 128, True, "bf16"),
                                               (130, 64, True, "f32"), (200, 32, False, "f32")])
def test_constant_v_gives_constant_output(T, Dh, causal, dtype):
    w = wl.random_case(5100 + T, 2, 3, T, Dh, dtype, wl.CAUSAL * causal | wl.SSMAX, beta_range=(-0.5, 1.3),
                       mu=-0.5)
    o, _ = _fwd(w, np.ones_like(w.v))
    tol = (BF16_U if dtype == "bf16" else 0.0) + 1e-5
    within(max_abs(o, np.ones_like(o)), tol, f"max |O - 1| ({dtype})")


@pytest.mark.parametrize("T,Dh,causal,dtype", [(64, 64, True, "bf16"), (50, 64, False, "bf16"),
                                               (32, 32, True, "bf16"), (128, 128, True, "bf16"),
                                               (64, 64, True, "f32"), (29, 32, False, "f32")])
def test_identity_v_gives_attention_matrix(T, Dh, causal, dtype):
    w = wl.random_case(5200 + T + Dh, 2, 3, T, Dh, dtype, wl.CAUSAL * causal | wl.SSMAX, beta_range=(-0.5, 1.3),
                       mu=-0.5)
    B, H = w.q.shape[:2]
    eye = np.zeros((B, H, T, Dh), np.float32)
    eye[:, :, np.arange(T), np.arange(T)] = 1.0
    o, _ = _fwd(w, eye)
    P = oracle.attn_fwd(w.q, w.k, eye, w.alpha, w.beta, w.mu, w.s, causal=causal, ssmax=True)[0][..., :T]
    got = o[..., :T]
    assert np.all(o[..., T:] == 0.0), "columns beyond T must be exactly zero"
    if causal:
        upper = np.triu(np.ones((T, T), bool), 1)
        assert np.all(got[:, :, upper] == 0.0), "masked (j > i) entries must be exactly zero"
    if dtype == "bf16":
        # |O - P| <= (2^-8 + 1e-5) P, the 1e-5 for the float32 exponent argument and l;
        # reported as the excess over that bound, against an absolute 1e-7
        err = float(np.max(np.abs(got - P) - (BF16_U + 1e-5) * P))
        within(err, 1e-7, "max(|O_ij - P_ij| - (2^-8 + 1e-5) P_ij) (bf16 weights)")
    else:
        within(max_abs(got, P), 1e-5, "max |O_ij - P_ij| (fp32)")
    rows = got.sum(axis=-1)
    within(max_abs(rows, np.ones_like(rows)), (BF16_U if dtype == "bf16" else 0.0) + 1e-5, "max |sum_j O_ij - 1|")


@pytest.mark.parametrize("L,Dh", [(9000, 64), (5000, 32), (3000, 128)])
def test_decode_split_invariance(L, Dh):
    """The heads of sequence 0 decoded alone (few work-groups, so shorter key ranges per
    split) and as sequence 0 of a batch of 8 identical sequences: the same result to float32
    rounding, and V = 1 gives O = 1 in both."""
    torch = torch_mod()
    bam = _bam()
    w = wl.long_decode(seed=5300 + L, B=1, H=12, L=L, Dh=Dh)
    p = params(w)
    q1, k1, v1 = dev(w.q, "bf16"), dev(w.k, "bf16"), dev(w.v, "bf16")
    rep = lambda t: t.expand(8, *t.shape[1:]).contiguous()
    res = {}
    for name, (q, k, v) in (("B=1", (q1, k1, v1)), ("B=8", (rep(q1), rep(k1), rep(v1)))):
        B = q.shape[0]
        kv = torch.full((B,), L, dtype=torch.int32, device="cuda")
        o, lse = bam.bam_attn_decode(q, k, v, kv, p["alpha"], p["beta"], p["mu"], p["s"], ssmax=True,
                                     o_dtype=torch.float32)
        ones, _ = bam.bam_attn_decode(q, k, torch.ones_like(v), kv, p["alpha"], p["beta"], p["mu"], p["s"],
                                      ssmax=True, o_dtype=torch.float32)
        torch.cuda.synchronize()
        res[name] = (host(o), host(lse))
        within(max_abs(host(ones), np.ones(tuple(ones.shape))), 1e-5, f"decode {name}: max |O - 1| for V = 1")
    (o1, l1), (o8, l8) = res["B=1"], res["B=8"]
    for b in range(8):
        within(max_abs(o8[b], o1[0]), 1e-5 * max(1.0, float(np.max(np.abs(o1)))), f"O of sequence {b} vs B=1")
        within(max_abs(l8[b], l1[0]), 1e-5 * max(1.0, float(np.max(np.abs(l1)))), f"lse of sequence {b} vs B=1")


@pytest.mark.parametrize("T,Dh,causal", [(300, 64, True), (700, 64, True), (200, 32, False)])
def test_backward_with_constant_v(T, Dh, causal):
    """V = 1 makes O = 1 whatever the weights, so nothing flows back to q, k or the prior's
    parameters: with O = 1 passed in, dP_ij = sum_e dO_ie = D_i, so dZ = 0, dQ = dK = 0 and
    dalpha = dbeta = ds = 0 up to float32 rounding of the two sums, while dV = P^T dO
    (against the oracle).  The rounding bound: dQ and dK within 1e-3, and each parameter
    gradient within 1e-3 of its head's conditioning scale for a random V."""
    torch = torch_mod()
    bam = _bam()
    w = wl.random_case(5400 + T, 2, 3, T, Dh, "bf16", wl.CAUSAL * causal | wl.SSMAX, beta_range=(0.2, 1.2),
                       with_grad=True)
    p = params(w)
    q, k, do = dev(w.q, "bf16"), dev(w.k, "bf16"), dev(w.do, "bf16")
    ones = np.ones_like(w.v)
    v = dev(ones, "bf16")
    _, lse = bam.bam_attn_fwd(q, k, v, p["alpha"], p["beta"], p["mu"], p["s"], causal=causal, ssmax=True,
                              o_dtype=torch.float32)
    o = torch.ones(tuple(q.shape), dtype=torch.float32, device="cuda")
    g = bam.bam_attn_bwd(q, k, v, o, lse, do, p["alpha"], p["beta"], p["mu"], p["s"], causal=causal, ssmax=True,
                         grad_dtype=torch.float32)
    torch.cuda.synchronize()
    dq, dk, dv, da, db, ds = (host(x) for x in g)
    within(float(np.max(np.abs(dq))), 1e-3, "max |dQ| with V = 1")
    within(float(np.max(np.abs(dk))), 1e-3, "max |dK| with V = 1")
    ref_v = oracle.attn_bwd(w.q, w.k, ones, w.do, w.alpha, w.beta, w.mu, w.s, causal=causal, ssmax=True)
    within(max_abs(dv, ref_v["dv"]), 1e-2 * max(1.0, float(np.max(np.abs(ref_v["dv"])))), "dV = P^T dO with V = 1")
    scale = oracle.attn_bwd(w.q, w.k, w.v, w.do, w.alpha, w.beta, w.mu, w.s, causal=causal, ssmax=True)
    for name, x, A in (("dalpha", da, "A_alpha"), ("dbeta", db, "A_beta"), ("ds", ds, "A_s")):
        r = np.abs(x) / (1e-3 * scale[A] + 1e-6)
        h = int(np.argmax(r))
        within(abs(float(x[h])), 1e-3 * float(scale[A][h]) + 1e-6, f"|{name}| with V = 1 (worst head {h})")
