"""GPU parity of the prefill forward (bam_attn_fwd) against the fp64 oracle.

Tolerances: fp32 path normwise relative 1e-5 on O and lse; bf16 path max |O - ref| <= 1e-2
(on the kernel's fp32 output) and max |lse - ref| <= 1e-3; a bf16 output must be the
round-to-nearest-even of the fp32 output, bit for bit."""
import math

import numpy as np
import pytest

import oracle
import oracle_checks as oc
from gpu_util import within
from gpu_util import (BF16_LSE_ABS, BF16_O_ABS, F32_REL, dev, host, lse_rel, max_abs, normwise_rel, params,
                      torch_mod)
from positional_prior_bias_amd import workloads as wl

pytestmark = pytest.mark.gpu


def _bam():
    import positional_prior_bias_amd as bam
    return bam


def run_fwd(w, o_dtype=None):
    torch = torch_mod()
    p = params(w)
    q, k, v = (dev(x, w.dtype) for x in (w.q, w.k, w.v))
    o, lse = _bam().bam_attn_fwd(q, k, v, p["alpha"], p["beta"], p["mu"], p["s"], causal=w.causal,
                                 ssmax=w.ssmax, o_dtype=o_dtype or torch.float32)
    torch.cuda.synchronize()
    return o, lse


def test_tiny_check_fp32():
    w = wl.tiny_check()
    o, lse = run_fwd(w)
    O, L = oracle.attn_fwd(w.q, w.k, w.v, w.alpha, w.beta, w.mu, w.s, causal=True, ssmax=False)
    within(normwise_rel(host(o), O), F32_REL, "normwise_rel(host(o), O)")
    within(lse_rel(host(lse), L), F32_REL, "lse_rel(host(lse), L)")


@pytest.mark.parametrize("T,Dh,causal,ssmax", [(1, 32, True, True), (5, 64, False, True), (63, 32, True, False),
                                               (64, 64, False, False), (130, 64, True, True), (200, 32, False, True)])
def test_fp32_random(T, Dh, causal, ssmax):
    w = wl.random_case(20 + T, 2, 3, T, Dh, "f32", wl.CAUSAL * causal | wl.SSMAX * ssmax, beta_range=(-0.7, 1.4),
                       mu=-0.5)
    o, lse = run_fwd(w)
    O, L = oracle.attn_fwd(w.q, w.k, w.v, w.alpha, w.beta, w.mu, w.s, causal=causal, ssmax=ssmax)
    within(normwise_rel(host(o), O), F32_REL, "normwise_rel(host(o), O)")
    within(lse_rel(host(lse), L), F32_REL, "lse_rel(host(lse), L)")


def test_worked_example_on_gpu():
    """NNX ALiBi-Style Attention, "A small example", embedded at Dh = 32 (fp32): Q = K = 0,
    V[:, 0] = [0, 1], non-causal, SSMax off, alpha = 1 / slope, beta = 1, mu = 0."""
    torch = torch_mod()
    g = oc.read_golden("alibi_worked_example.txt")
    H, T, Dh = int(g["heads"]), int(g["positions"]), 32
    m = wl.alibi_slopes(H)
    q = torch.zeros((1, H, T, Dh), dtype=torch.float32, device="cuda")
    k = torch.zeros_like(q)
    v = torch.zeros_like(q)
    v[0, :, 1, 0] = 1.0
    alpha = dev((1.0 / m).astype(np.float32))
    beta = dev(np.ones(H, np.float32))
    o, _ = _bam().bam_attn_fwd(q, k, v, alpha, beta, None, None, causal=False, ssmax=False, o_dtype=torch.float32)
    out = host(o)[0, :, :, 0]
    expected = 1.0 / (1.0 + np.exp(m))
    within(max_abs(out[:, 0], expected), 1e-6, "max_abs(out[:, 0], expected)")
    within(max_abs(out[:, 1], 1.0 - expected), 1e-6, "max_abs(out[:, 1], 1.0 - expected)")
    within(max_abs(out[0], [g["head0_pos0"], g["head0_pos1"]]), 5e-7, 'max_abs(out[0], [g["head0_pos0"], g["head0_pos1"]])')


CASES = [
    # T, Dh, causal, ssmax, beta range, mu
    (1, 64, True, True, (0.2, 1.2), 0.0),
    (2, 64, False, True, (0.2, 1.2), 0.0),
    (17, 32, True, False, (0.3, 1.5), 0.0),
    (64, 64, True, True, (0.2, 1.2), 0.0),
    (127, 64, False, False, (-0.8, -0.1), -0.5),
    (129, 128, True, True, (0.1, 0.9), 0.0),
    (300, 64, True, True, (-0.8, -0.1), -0.5),
    (300, 64, False, True, (0.2, 1.2), 0.0),
    (513, 32, True, True, (0.2, 1.2), 0.0),
    (700, 128, False, False, (0.5, 2.0), 0.0),
    # long sequences (many key tiles per work-group, a ragged last tile)
    (2048, 64, True, True, (0.1, 0.9), 0.0),
    (2100, 64, True, True, (-0.8, -0.1), -0.5),
    (2333, 64, False, True, (0.2, 1.2), 0.0),
    (4097, 64, True, False, (0.3, 1.5), 0.0),
]


@pytest.mark.parametrize("T,Dh,causal,ssmax,br,mu", CASES)
def test_bf16_random(T, Dh, causal, ssmax, br, mu):
    B = 2 if T < 2048 else 1
    w = wl.random_case(100 + T + Dh, B, 3, T, Dh, "bf16", wl.CAUSAL * causal | wl.SSMAX * ssmax, beta_range=br,
                       mu=mu)
    o, lse = run_fwd(w)
    O, L = oracle.attn_fwd(w.q, w.k, w.v, w.alpha, w.beta, w.mu, w.s, causal=causal, ssmax=ssmax)
    within(max_abs(host(o), O), BF16_O_ABS, "max_abs(host(o), O)")
    within(max_abs(host(lse), L), BF16_LSE_ABS, "max_abs(host(lse), L)")


def test_bf16_alibi_and_nope():
    torch = torch_mod()
    H = 12
    w = wl.random_case(7, 1, H, 257, 64, "bf16", wl.CAUSAL)
    m = wl.alibi_slopes(H)
    w.alpha = (1.0 / m).astype(np.float32)
    w.beta = np.ones(H, np.float32)
    o, lse = run_fwd(w)
    O, L = oracle.attn_fwd(w.q, w.k, w.v, w.alpha, w.beta, w.mu, w.s, causal=True, ssmax=False)
    within(max_abs(host(o), O), BF16_O_ABS, "ALiBi O")
    within(max_abs(host(lse), L), BF16_LSE_ABS, "ALiBi lse")
    w.alpha = np.full(H, np.inf, np.float32)
    o, lse = run_fwd(w)
    O, L = oracle.attn_fwd(w.q, w.k, w.v, w.alpha, w.beta, w.mu, w.s, causal=True, ssmax=False)
    within(max_abs(host(o), O), BF16_O_ABS, "NoPE O")
    within(max_abs(host(lse), L), BF16_LSE_ABS, "NoPE lse")


def test_bf16_output_is_rne_of_fp32_and_repeatable():
    torch = torch_mod()
    w = wl.random_case(5, 2, 4, 333, 64, "bf16", wl.CAUSAL | wl.SSMAX)
    o32, l32 = run_fwd(w, torch.float32)
    o16, l16 = run_fwd(w, torch.bfloat16)
    assert torch.equal(o16, o32.to(torch.bfloat16))
    assert torch.equal(l16, l32)
    o32b, l32b = run_fwd(w, torch.float32)
    assert torch.equal(o32, o32b) and torch.equal(l32, l32b)


def test_training_shape_full():
    """B=32, H=12, T=512, Dh=64, every row of every head."""
    w = wl.training_shape()
    o, lse = run_fwd(w)
    O, L = oracle.attn_fwd(w.q, w.k, w.v, w.alpha, w.beta, w.mu, w.s, causal=True, ssmax=True)
    print(f"training shape: max|dO|={max_abs(host(o), O):.3e} max|dlse|={max_abs(host(lse), L):.3e}")
    within(max_abs(host(o), O), BF16_O_ABS, "max_abs(host(o), O)")
    within(max_abs(host(lse), L), BF16_LSE_ABS, "max_abs(host(lse), L)")


def long_prefill_rows(T, seed=0, tile=128):
    rng = np.random.default_rng(seed)
    rows = set(range(256)) | set(range(T - 256, T))
    for b in range(tile, T, tile):
        rows |= {b - 1, b, b + 1}
    rows |= set(rng.integers(0, T, 1024).tolist())
    return np.array(sorted(r for r in rows if 0 <= r < T))


def test_long_prefill_sampled_rows():
    """B=1, H=12, T=32768: first/last 256 rows, every 128-row tile boundary +-1, 1024 random rows."""
    w = wl.long_prefill()
    o, lse = run_fwd(w)
    oh, lh = host(o), host(lse)
    rows = long_prefill_rows(w.T)
    worst_o = worst_l = 0.0
    for h in range(w.H):
        O, L = oracle.attn_fwd_rows(w.q[0, h], w.k[0, h], w.v[0, h], rows, w.alpha[h], w.beta[h], w.mu[h], w.s[h],
                                    causal=True, ssmax=True)
        worst_o = max(worst_o, max_abs(oh[0, h, rows], O))
        worst_l = max(worst_l, max_abs(lh[0, h, rows], L))
    within(worst_o, BF16_O_ABS, f"T = 32768 O over {rows.size} rows per head")
    within(worst_l, BF16_LSE_ABS, f"T = 32768 lse over {rows.size} rows per head")


def test_prefill_131072_sampled_rows():
    """B=1, H=12, T=131072, the length sweep's inputs (Q, K, V drawn on the GPU from seed 3,
    the 32,768-token prefill's heads): per head the first and last 64 rows, every 8192-row
    boundary +-1 and 64 random rows, against the oracle on the same bf16 values."""
    torch = torch_mod()
    T = 131072
    w = wl.long_prefill_device(T=T, B=1)
    p = params(w)
    o, lse = _bam().bam_attn_fwd(w.q, w.k, w.v, p["alpha"], p["beta"], p["mu"], p["s"], causal=True, ssmax=True,
                                 o_dtype=torch.float32)
    torch.cuda.synchronize()
    rng = np.random.default_rng(131072)
    rows = set(range(64)) | set(range(T - 64, T))
    for b in range(8192, T, 8192):
        rows |= {b - 1, b, b + 1}
    rows |= set(rng.integers(0, T, 64).tolist())
    rows = np.array(sorted(rows))
    ridx = torch.from_numpy(rows).cuda()
    oh = host(o[0].index_select(1, ridx))
    lh = host(lse[0].index_select(1, ridx))
    worst_o = worst_l = 0.0
    for h in range(w.H):
        qh, kh, vh = (host(x[0, h]) for x in (w.q, w.k, w.v))
        O, L = oracle.attn_fwd_rows(qh, kh, vh, rows, w.alpha[h], w.beta[h], w.mu[h], w.s[h], causal=True,
                                    ssmax=True, chunk=64)
        worst_o = max(worst_o, max_abs(oh[h], O))
        worst_l = max(worst_l, max_abs(lh[h], L))
    within(worst_o, BF16_O_ABS, f"T = 131072 O over {rows.size} rows per head")
    within(worst_l, BF16_LSE_ABS, f"T = 131072 lse over {rows.size} rows per head")
