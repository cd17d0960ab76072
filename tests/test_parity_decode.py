"""GPU parity of the split-KV decode (bam_attn_decode) against the fp64 oracle.
bf16 caches, fp32 output: max |O - ref| <= 1e-2, max |lse - ref| <= 1e-3."""
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


def run_decode(w, o_dtype=None):
    torch = torch_mod()
    p = params(w)
    q, k, v = dev(w.q, "bf16"), dev(w.k, "bf16"), dev(w.v, "bf16")
    kv = torch.from_numpy(w.kv_len.astype(np.int32)).cuda()
    o, lse = _bam().bam_attn_decode(q, k, v, kv, p["alpha"], p["beta"], p["mu"], p["s"], ssmax=w.ssmax,
                                    o_dtype=o_dtype or torch.float32)
    torch.cuda.synchronize()
    return o, lse


@pytest.mark.parametrize("L,kv,Dh", [(1, [1, 1], 64), (100, [100, 37], 64), (5000, [5000, 1234], 64),
                                     (9000, [1, 8999], 128), (20000, [20000, 4097], 64),
                                     (1, [1, 1], 32), (130, [130, 65], 32), (7000, [6999, 2048], 32),
                                     (20000, [19999, 511], 32)])
def test_decode_random(L, kv, Dh):
    w = wl.long_decode(seed=40 + L, B=2, H=12, L=L, Dh=Dh, kv_len=np.array(kv))
    o, lse = run_decode(w)
    O, LS = oracle.attn_decode(w.q, w.k, w.v, w.kv_len, w.alpha, w.beta, w.mu, w.s, ssmax=True)
    within(max_abs(host(o), O), BF16_O_ABS, "max_abs(host(o), O)")
    within(max_abs(host(lse), LS), BF16_LSE_ABS, "max_abs(host(lse), LS)")


def test_decode_single_key_returns_v0():
    torch = torch_mod()
    w = wl.long_decode(seed=3, B=3, H=12, L=64, Dh=64, kv_len=np.array([1, 1, 1]))
    o, _ = run_decode(w)
    assert torch.equal(o, dev(w.v[:, :, 0, :], "f32"))


def test_decode_equals_last_prefill_row():
    torch = torch_mod()
    w = wl.random_case(9, 2, 12, 777, 64, "bf16", wl.CAUSAL | wl.SSMAX, beta_range=(0.1, 0.9))
    p = params(w)
    q, k, v = (dev(x, "bf16") for x in (w.q, w.k, w.v))
    o, lse = _bam().bam_attn_fwd(q, k, v, p["alpha"], p["beta"], p["mu"], p["s"], causal=True, ssmax=True,
                                 o_dtype=torch.float32)
    kv = torch.full((2,), 777, dtype=torch.int32, device="cuda")
    od, ld = _bam().bam_attn_decode(q[:, :, -1].contiguous(), k, v, kv, p["alpha"], p["beta"], p["mu"], p["s"],
                                    ssmax=True, o_dtype=torch.float32)
    torch.cuda.synchronize()
    within(max_abs(host(od), host(o)[:, :, -1]), 2 * BF16_O_ABS, "max_abs(host(od), host(o)[:, :, -1])")
    within(max_abs(host(ld), host(lse)[:, :, -1]), 2 * BF16_LSE_ABS, "max_abs(host(ld), host(lse)[:, :, -1])")


def test_decode_repeatable_and_bf16_output():
    torch = torch_mod()
    w = wl.long_decode(seed=5, B=2, H=12, L=3000, Dh=64)
    o1, l1 = run_decode(w)
    o2, l2 = run_decode(w)
    ob, _ = run_decode(w, torch.bfloat16)
    assert torch.equal(o1, o2) and torch.equal(l1, l2)
    assert torch.equal(ob, o1.to(torch.bfloat16))


def test_decode_full_context_256k():
    """B=8, H=12, Dh=64, 256,000-token bf16 caches (drawn on the device) with one planted key
    per sequence; every (b, h) checked against the oracle on the same cache values."""
    torch = torch_mod()
    w = wl.long_decode_device()
    p = params(w)
    kv = torch.from_numpy(w.kv_len).cuda()
    o, lse = _bam().bam_attn_decode(dev(w.q, "bf16"), w.k, w.v, kv, p["alpha"], p["beta"], p["mu"], p["s"],
                                    ssmax=True, o_dtype=torch.float32)
    torch.cuda.synchronize()
    O = np.empty((w.B, w.H, w.Dh))
    LS = np.empty((w.B, w.H))
    for b in range(w.B):
        kb = w.k[b].float().cpu().numpy()[None]
        vb = w.v[b].float().cpu().numpy()[None]
        Ob, Lb = oracle.attn_decode(w.q[b:b + 1], kb, vb, w.kv_len[b:b + 1], w.alpha, w.beta, w.mu, w.s, ssmax=True)
        O[b], LS[b] = Ob[0], Lb[0]
    err_o, err_l = max_abs(host(o), O), max_abs(host(lse), LS)
    within(err_o, BF16_O_ABS, "decode 256k O")
    within(err_l, BF16_LSE_ABS, "decode 256k lse")
