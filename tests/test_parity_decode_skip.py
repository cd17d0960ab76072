"""Prior-aware decode skipping (bam_attn_decode_skip) and its key-norm pages
(bam_decode_key_norms): the skipping call returns the same bits as bam_attn_decode, leaves
out key ranges where the prior makes every weight zero, and the norm pages bound every key
norm from above."""
import numpy as np
import pytest

import oracle
from gpu_util import within
from gpu_util import BF16_LSE_ABS, BF16_O_ABS, dev, host, max_abs, params, torch_mod
from positional_prior_bias_amd import workloads as wl

pytestmark = pytest.mark.gpu


def _bam():
    import positional_prior_bias_amd as bam
    return bam


def _local_heads(w, H):
    """Priors that decay with distance ("Solution Proposée : GGD-BAM", beta > 0): alpha
    from 2 to 2048, beta from 1 down to 0.5, mu = 0."""
    w.alpha = np.array([2.0 * 4.0 ** (h % 6) for h in range(H)], np.float32)
    w.beta = np.array([1.0 - 0.1 * (h % 6) for h in range(H)], np.float32)
    w.mu = np.zeros(H, np.float32)
    return w


def _both(w, k, v):
    """(full o, lse), (skipping o, lse), skipped fraction, for one workload (k, v on device)."""
    torch, bam = torch_mod(), _bam()
    p = params(w)
    q = dev(w.q, "bf16")
    kv = torch.from_numpy(np.asarray(w.kv_len, np.int32)).cuda()
    B, H, L, Dh = k.shape
    norms = bam.bam_decode_key_norms(k)
    ws = torch.empty(bam.bam_decode_workspace_size(B, H, L, Dh), dtype=torch.uint8, device="cuda")
    full = bam.bam_attn_decode(q, k, v, kv, p["alpha"], p["beta"], p["mu"], p["s"], ssmax=True,
                               o_dtype=torch.float32, workspace=ws)
    full = tuple(t.clone() for t in full)
    skip = bam.bam_attn_decode_skip(q, k, v, kv, p["alpha"], p["beta"], p["mu"], p["s"], key_norms=norms, ssmax=True,
                                    o_dtype=torch.float32, workspace=ws)
    torch.cuda.synchronize()
    frac = bam.decode_skipped_fraction(ws, kv, B, H, L, Dh)
    return full, skip, frac


def _same_bits(a, b, what):
    torch = torch_mod()
    assert a.shape == b.shape and torch.equal(a.view(torch.int32), b.view(torch.int32)), \
        f"{what}: skipping differs from full decode in {(a != b).sum().item()} of {a.numel()} values"


@pytest.mark.parametrize("B,H,L,Dh", [(2, 3, 1000, 64), (1, 2, 4097, 32), (2, 2, 300, 128)])
def test_key_norm_pages_bound_every_key(B, H, L, Dh):
    torch, bam = torch_mod(), _bam()
    rng = np.random.default_rng(L + Dh)
    k = (rng.standard_normal((B, H, L, Dh)) * rng.uniform(0.1, 10.0, (B, H, L, 1))).astype(np.float32)
    kd = dev(k, "bf16")
    norms = host(bam.bam_decode_key_norms(kd))
    npages = bam.bam_decode_norm_pages(L)
    assert norms.shape == (B, H, npages) and npages == (L + 63) // 64
    exact = np.sqrt((host(kd) ** 2).sum(-1))                       # norms of the bf16 keys, fp64
    pad = np.zeros((B, H, npages * 64 - L))
    page_max = np.concatenate([exact, pad], axis=-1).reshape(B, H, npages, 64).max(-1)
    assert np.all(norms >= page_max), "a page's norm is below one of its keys'"
    within(float(np.max(norms / page_max - 1.0)), 2.0 ** -12, "relative excess of the norm pages")


def test_decode_skip_local_heads_same_bits_and_oracle():
    """Local heads at 65,536 tokens (ragged lengths): most ranges are left out, the result has
    the same bits as the full decode and matches the oracle."""
    torch = torch_mod()
    w = _local_heads(wl.long_decode(seed=7, B=2, H=6, L=65536, Dh=64, kv_len=np.array([65536, 40000])), 6)
    k, v = dev(w.k, "bf16"), dev(w.v, "bf16")
    (o, lse), (os_, ls), frac = _both(w, k, v)
    _same_bits(o, os_, "O")
    _same_bits(lse, ls, "lse")
    assert frac > 0.5, f"only {frac:.3f} of the ranges skipped"
    O, LS = oracle.attn_decode(w.q, w.k, w.v, w.kv_len, w.alpha, w.beta, w.mu, w.s, ssmax=True)
    within(max_abs(host(os_), O), BF16_O_ABS, "skipping decode O")
    within(max_abs(host(ls), LS), BF16_LSE_ABS, "skipping decode lse")


@pytest.mark.parametrize("L,kv,Dh", [(20000, [19999, 511], 32), (9000, [1, 8999], 128), (5000, [5000, 1234], 64)])
def test_decode_skip_same_bits_mixed(L, kv, Dh):
    """The extrapolation heads (heavy-tailed and inverted priors, little or nothing to skip)
    next to local heads, ragged lengths down to one key."""
    w = wl.long_decode(seed=60 + L, B=2, H=12, L=L, Dh=Dh, kv_len=np.array(kv))
    loc = _local_heads(wl.long_decode(seed=1, B=1, H=6, L=1, Dh=Dh), 6)
    w.alpha[:6], w.beta[:6], w.mu[:6] = loc.alpha, loc.beta, loc.mu
    k, v = dev(w.k, "bf16"), dev(w.v, "bf16")
    (o, lse), (os_, ls), frac = _both(w, k, v)
    _same_bits(o, os_, "O")
    _same_bits(lse, ls, "lse")


def test_decode_skip_same_bits_256k():
    """The 256,000-token decode workload (B=8, H=12, one planted key per sequence)."""
    w = wl.long_decode_device()
    (o, lse), (os_, ls), frac = _both(w, w.k, w.v)
    _same_bits(o, os_, "O")
    _same_bits(lse, ls, "lse")
    print(f"[decode 256k] skipped range fraction {frac:.4f}")
