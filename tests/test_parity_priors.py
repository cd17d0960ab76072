"""GPU parity of the other relative-distance biases carried by the distance table.

* Sandwich (attention-gym "Score Mods", "Sandwich"; BAM_PRIOR_SANDWICH):
  sum_i cos(d / 10000^(2 i / d_bar)) / ratio_h with ratio_h = 8 (h + 1) / H, against the
  fp64 oracle's prior_bias_sandwich, through the table, the prefill forward (bf16 and
  fp32 paths), decode (contiguous and paged) and the backward (whose parameter
  gradients are zero: the bias has no parameters).
* ALiBi with the pages' slopes 2^(-8 (h + 1) / H) ("ALiBi: Attention with Linear Biases",
  "Code"; NNX ALiBi-Style Attention, "One fixed slope per head") as the alpha-form with
  beta = 1 and alpha = 1 / slope, including the printed two-position example of the NNX
  page run on the GPU.

Tolerances as in the other parity tests: table entries 2e-6 of the row's largest entry;
bf16 forward |O| 1e-2, lse 1e-3; fp32 normwise relative 1e-5; backward dQ/dK/dV 1e-2 of
the largest entry."""
import numpy as np
import pytest

import oracle
from gpu_util import within
from gpu_util import BF16_LSE_ABS, BF16_O_ABS, F32_REL, dev, host, max_abs, normwise_rel, params, torch_mod
from oracle_checks import read_golden
from positional_prior_bias_amd import workloads as wl

pytestmark = pytest.mark.gpu


def _bam():
    import positional_prior_bias_amd as bam
    return bam


@pytest.mark.parametrize("d_bar", [2.0, 16.0, 128.0, 1024.0])
def test_prior_table_sandwich(d_bar):
    H, d0, n = 5, -900, 1801
    ratio = np.array([8.0 * (h + 1) / H for h in range(H)], np.float32)
    dbar = np.full(H, d_bar, np.float32)
    got = _bam().bam_prior_table_ex(dev(ratio), dev(dbar), None, d0, n, prior="sandwich")
    torch_mod().cuda.synchronize()
    d = np.arange(d0, d0 + n)
    tab = host(got[0])
    for h in range(H):
        r = oracle.prior_bias_sandwich(d, float(ratio[h]), float(dbar[h]))
        tol = 2e-6 * max(1.0, float(np.max(np.abs(r))))
        within(max_abs(tab[h], r), tol, f"sandwich table head {h}")
    for g in got[1:]:
        assert not np.any(host(g))


def test_prior_table_sandwich_frequency_count_edges():
    """d_bar above 8192 is taken as 8192 and the frequency count is trunc(d_bar) / 2:
    d_bar = 1024 and 1026 (513 frequencies) follow the oracle, d_bar = 9000 and 3e9 that of
    d_bar = 8192; below 2, and for
    a NaN d_bar (a precondition violation), no frequency is kept (zero bias, as the
    oracle's empty sum).  Every entry is finite."""
    ratio = np.ones(7, np.float32)
    dbar = np.array([1024.0, 1026.0, 9000.0, 3e9, np.nan, 1.5, -4.0], np.float32)
    d0, n = -40, 81
    tab = host(_bam().bam_prior_table_ex(dev(ratio), dev(dbar), None, d0, n, prior="sandwich")[0])
    assert np.all(np.isfinite(tab))
    d = np.arange(d0, d0 + n)
    for h, db in ((0, 1024.0), (1, 1026.0), (2, 8192.0), (3, 8192.0)):
        r = oracle.prior_bias_sandwich(d, 1.0, db)
        within(max_abs(tab[h], r), 2e-6 * max(1.0, float(np.abs(r).max())), f"sandwich d_bar {dbar[h]}")
    assert not np.any(tab[4:])
    for h in (5, 6):
        assert np.array_equal(oracle.prior_bias_sandwich(d, 1.0, float(dbar[h])), np.zeros(n))


def test_sandwich_with_prior_ref_rejected():
    bam = _bam()
    a = dev(np.ones(2, np.float32))
    with pytest.raises(bam.BamError):
        bam.bam_prior_table_ex(a, a, None, 0, 4, prior_ref=True, prior="sandwich")
    H, d0, n = 2, 0, 4
    tab = torch_mod().empty((H, n), dtype=torch_mod().float32, device="cuda")
    st = bam.lib().bam_prior_table_ex(a.data_ptr(), a.data_ptr(), None, H, d0, n,
                                      bam.BAM_PRIOR_REF | bam.BAM_PRIOR_SANDWICH, tab.data_ptr(), None, None, None,
                                      None)
    assert st == 1


def _fwd(w, prior):
    """Forward with a float32 output: the Sandwich bias at d = 0 (d_bar / 2 / ratio_h)
    makes rows nearly one-hot, so |O| reaches |v| ~ 4, where one bf16 output rounding
    alone is 2^-6; the float32 output keeps the check on the kernel's arithmetic."""
    p = params(w)
    ty = "bf16" if w.dtype == "bf16" else "f32"
    q, k, v = (dev(x, ty) for x in (w.q, w.k, w.v))
    torch = torch_mod()
    o, lse = _bam().bam_attn_fwd(q, k, v, p["alpha"], p["beta"], p["mu"], p["s"], causal=w.causal, ssmax=w.ssmax,
                                 o_dtype=torch.float32, prior=prior)
    torch.cuda.synchronize()
    return host(o), host(lse)


@pytest.mark.parametrize("T,Dh,causal,ssmax", [(37, 64, True, True), (300, 64, True, True), (513, 64, False, True),
                                              (700, 32, True, False), (200, 128, True, True)])
def test_fwd_sandwich_bf16(T, Dh, causal, ssmax):
    w = wl.sandwich_case(1300 + T, 2, 3, T, Dh, "bf16", wl.CAUSAL * causal | wl.SSMAX * ssmax)
    o, lse = _fwd(w, "sandwich")
    O, L = oracle.attn_fwd(w.q, w.k, w.v, w.alpha, w.beta, w.mu, w.s, causal=causal, ssmax=ssmax, param="sandwich")
    print(f"O err {max_abs(o, O):.3e}  lse err {max_abs(lse, L):.3e}")
    within(max_abs(o, O), BF16_O_ABS, "max_abs(o, O)")
    within(max_abs(lse, L), BF16_LSE_ABS, "max_abs(lse, L)")


@pytest.mark.parametrize("T,Dh,causal,ssmax", [(63, 32, True, True), (200, 64, False, True)])
def test_fwd_sandwich_f32(T, Dh, causal, ssmax):
    w = wl.sandwich_case(1350 + T, 1, 4, T, Dh, "f32", wl.CAUSAL * causal | wl.SSMAX * ssmax, d_bar=64.0)
    o, lse = _fwd(w, "sandwich")
    O, L = oracle.attn_fwd(w.q, w.k, w.v, w.alpha, w.beta, w.mu, w.s, causal=causal, ssmax=ssmax, param="sandwich")
    within(normwise_rel(o, O), F32_REL, "normwise_rel(o, O)")
    within(normwise_rel(lse, L), F32_REL, "normwise_rel(lse, L)")


def test_decode_sandwich():
    torch = torch_mod()
    B, H, L, Dh = 3, 4, 2500, 64
    w = wl.sandwich_case(78, B, H, L, Dh, "bf16")
    kv_len = np.array([2500, 1, 1234], np.int32)
    rng = np.random.default_rng(6)
    q = wl.bf16_round(rng.standard_normal((B, H, Dh)).astype(np.float32))
    p = params(w)
    o, lse = _bam().bam_attn_decode(dev(q, "bf16"), dev(w.k, "bf16"), dev(w.v, "bf16"), torch.from_numpy(kv_len).cuda(),
                                    p["alpha"], p["beta"], p["mu"], p["s"], ssmax=True, o_dtype=torch.float32,
                                    prior="sandwich")
    torch.cuda.synchronize()
    O, Lse = oracle.attn_decode(q, w.k, w.v, kv_len, w.alpha, w.beta, w.mu, w.s, ssmax=True, param="sandwich")
    within(max_abs(host(o), O), BF16_O_ABS, "max_abs(host(o), O)")
    within(max_abs(host(lse), Lse), BF16_LSE_ABS, "max_abs(host(lse), Lse)")


def test_decode_paged_sandwich():
    """Paged cache: the contiguous cache cut into 128-token pages, scattered by a random
    page permutation; same oracle as the contiguous call."""
    torch = torch_mod()
    B, H, L, Dh, P = 2, 3, 1024, 64, 128
    w = wl.sandwich_case(79, B, H, L, Dh, "bf16")
    kv_len = np.array([1024, 515], np.int32)
    rng = np.random.default_rng(7)
    q = wl.bf16_round(rng.standard_normal((B, H, Dh)).astype(np.float32))
    nblk = L // P
    perm = rng.permutation(B * nblk).astype(np.int32)
    block_table = perm.reshape(B, nblk)
    kp = np.zeros((B * nblk, H, P, Dh), np.float32)
    vp = np.zeros_like(kp)
    for b in range(B):
        for j in range(nblk):
            kp[block_table[b, j]] = w.k[b, :, j * P:(j + 1) * P]
            vp[block_table[b, j]] = w.v[b, :, j * P:(j + 1) * P]
    p = params(w)
    o, lse = _bam().bam_attn_decode_paged(dev(q, "bf16"), dev(kp, "bf16"), dev(vp, "bf16"),
                                          torch.from_numpy(block_table).cuda(), torch.from_numpy(kv_len).cuda(),
                                          p["alpha"], p["beta"], p["mu"], p["s"], ssmax=True, o_dtype=torch.float32,
                                          prior="sandwich")
    torch.cuda.synchronize()
    O, Lse = oracle.attn_decode(q, w.k, w.v, kv_len, w.alpha, w.beta, w.mu, w.s, ssmax=True, param="sandwich")
    within(max_abs(host(o), O), BF16_O_ABS, "max_abs(host(o), O)")
    within(max_abs(host(lse), Lse), BF16_LSE_ABS, "max_abs(host(lse), Lse)")


@pytest.mark.parametrize("T,Dh,causal,ssmax", [(64, 64, True, True), (257, 64, True, True), (130, 32, False, True)])
def test_bwd_sandwich(T, Dh, causal, ssmax):
    torch = torch_mod()
    w = wl.sandwich_case(1400 + T, 2, 3, T, Dh, "bf16", wl.CAUSAL * causal | wl.SSMAX * ssmax, with_grad=True)
    p = params(w)
    q, k, v, do = (dev(x, "bf16") for x in (w.q, w.k, w.v, w.do))
    o, lse = _bam().bam_attn_fwd(q, k, v, p["alpha"], p["beta"], p["mu"], p["s"], causal=causal, ssmax=ssmax,
                                 o_dtype=torch.float32, prior="sandwich")
    g = _bam().bam_attn_bwd_ex(q, k, v, o, lse, do, p["alpha"], p["beta"], p["mu"], p["s"], causal=causal,
                               ssmax=ssmax, grad_dtype=torch.float32, prior="sandwich")
    torch.cuda.synchronize()
    got = [host(x) for x in g]
    R = oracle.attn_bwd(w.q, w.k, w.v, w.do, w.alpha, w.beta, w.mu, w.s, causal=causal, ssmax=ssmax,
                        param="sandwich")
    for name, x in zip(("dq", "dk", "dv"), got[:3]):
        tol = 1e-2 * max(1.0, float(np.max(np.abs(R[name]))))
        within(max_abs(x, R[name]), tol, name)
    for name, x in zip(("dalpha", "dbeta", "dmu"), got[3:6]):
        assert not np.any(x), name
    err = np.abs(got[6] - R["ds"])
    tol = 1e-3 * R["A_s"] + 1e-6
    h = int(np.argmax(err / tol))
    within(err[h], tol[h], f"ds (worst head {h})")


def test_alibi_worked_example_on_gpu():
    """NNX ALiBi-Style Attention, "A small example": two positions, four heads, zero
    content scores, values 0 and 1; output at position 0 is 1 / (1 + e^slope_h).  Run
    through the fp32 forward with the alpha-form at beta = 1, alpha = 1 / slope."""
    torch = torch_mod()
    bam = _bam()
    g = read_golden("alibi_worked_example.txt")
    H, T, Dh = int(g["heads"]), int(g["positions"]), 32
    m = host(bam.alibi_slopes(H))
    q = torch.zeros((1, H, T, Dh), dtype=torch.float32, device="cuda")
    v = torch.zeros_like(q)
    v[:, :, 1, :] = 1.0
    a = (1.0 / bam.alibi_slopes(H, device="cuda")).contiguous()
    o, _ = bam.bam_attn_fwd(q, q, v, a, torch.ones_like(a), None, None, causal=False, ssmax=False)
    torch.cuda.synchronize()
    o = host(o)
    expected = 1.0 / (1.0 + np.exp(m))
    assert np.max(np.abs(o[0, :, 0, 0] - expected)) <= 1e-6
    assert np.max(np.abs(o[0, :, 1, 0] - (1.0 - expected))) <= 1e-6
    assert np.max(np.abs(o[0, 0, :, 0] - [g["head0_pos0"], g["head0_pos1"]])) <= 1e-6


@pytest.mark.parametrize("T,H,causal", [(300, 8, False), (700, 12, True)])
def test_fwd_alibi_slopes_bf16(T, H, causal):
    """ALiBi heads with the pages' slope schedule (H = 12 is not a power of two)."""
    torch = torch_mod()
    bam = _bam()
    w = wl.random_case(1500 + T, 1, H, T, 64, "bf16", wl.CAUSAL * causal)
    m = wl.alibi_slopes(H)
    assert np.allclose(host(bam.alibi_slopes(H)), m.astype(np.float32), rtol=0, atol=0)
    alpha = (1.0 / m).astype(np.float32)
    ones, zeros = np.ones(H, np.float32), np.zeros(H, np.float32)
    q, k, v = (dev(x, "bf16") for x in (w.q, w.k, w.v))
    o, lse = bam.bam_attn_fwd(q, k, v, dev(alpha), dev(ones), dev(zeros), None, causal=causal, ssmax=False,
                              o_dtype=torch.float32)
    torch.cuda.synchronize()
    O, L = oracle.attn_fwd(w.q, w.k, w.v, alpha, ones, zeros, ones, causal=causal, ssmax=False)
    within(max_abs(host(o), O), BF16_O_ABS, "max_abs(host(o), O)")
    within(max_abs(host(lse), L), BF16_LSE_ABS, "max_abs(host(lse), L)")
