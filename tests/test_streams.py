"""Stream semantics of the C ABI (include/bam.h: all work is enqueued on the given stream,
calls return without synchronising, calls on different streams may run concurrently): the
forward, decode and backward on a side stream, two forwards on two streams at once, each
equal bit for bit to the same call on the default stream."""
import numpy as np
import pytest

from gpu_util import dev, params, torch_mod
from positional_prior_bias_amd import workloads as wl

pytestmark = pytest.mark.gpu


def _bam():
    import positional_prior_bias_amd as bam
    return bam


def _inputs(seed, T=700):
    w = wl.random_case(seed, 2, 3, T, 64, "bf16", wl.CAUSAL | wl.SSMAX, beta_range=(0.2, 1.2), with_grad=True)
    q, k, v, do = (dev(x, "bf16") for x in (w.q, w.k, w.v, w.do))
    return w, q, k, v, do, params(w)


def test_side_stream_matches_default_stream():
    torch = torch_mod()
    bam = _bam()
    w, q, k, v, do, p = _inputs(2000)
    args = (q, k, v, p["alpha"], p["beta"], p["mu"], p["s"])
    o0, l0 = bam.bam_attn_fwd(*args, o_dtype=torch.float32)
    g0 = bam.bam_attn_bwd(q, k, v, o0, l0, do, p["alpha"], p["beta"], p["mu"], p["s"], grad_dtype=torch.float32)
    kv = torch.full((2,), 700, dtype=torch.int32, device="cuda")
    qd = q[:, :, -1].contiguous()
    d0 = bam.bam_attn_decode(qd, k, v, kv, p["alpha"], p["beta"], p["mu"], p["s"], o_dtype=torch.float32)
    torch.cuda.synchronize()
    side = torch.cuda.Stream()
    with torch.cuda.stream(side):
        o1, l1 = bam.bam_attn_fwd(*args, o_dtype=torch.float32)
        g1 = bam.bam_attn_bwd(q, k, v, o1, l1, do, p["alpha"], p["beta"], p["mu"], p["s"], grad_dtype=torch.float32)
        d1 = bam.bam_attn_decode(qd, k, v, kv, p["alpha"], p["beta"], p["mu"], p["s"], o_dtype=torch.float32)
    side.synchronize()
    assert torch.equal(o0, o1) and torch.equal(l0, l1)
    for a, b in zip(g0, g1):
        assert torch.equal(a, b)
    assert torch.equal(d0[0], d1[0]) and torch.equal(d0[1], d1[1])


def test_two_streams_at_once():
    """Two forwards with their own workspaces, enqueued on two streams back to back."""
    torch = torch_mod()
    bam = _bam()
    wa, qa, ka, va, _, pa = _inputs(2001, T=1500)
    wb, qb, kb, vb, _, pb = _inputs(2002, T=1500)
    ref_a = bam.bam_attn_fwd(qa, ka, va, pa["alpha"], pa["beta"], pa["mu"], pa["s"], o_dtype=torch.float32)
    ref_b = bam.bam_attn_fwd(qb, kb, vb, pb["alpha"], pb["beta"], pb["mu"], pb["s"], o_dtype=torch.float32)
    torch.cuda.synchronize()
    sa, sb = torch.cuda.Stream(), torch.cuda.Stream()
    outs = []
    for _ in range(3):
        with torch.cuda.stream(sa):
            oa = bam.bam_attn_fwd(qa, ka, va, pa["alpha"], pa["beta"], pa["mu"], pa["s"], o_dtype=torch.float32)
        with torch.cuda.stream(sb):
            ob = bam.bam_attn_fwd(qb, kb, vb, pb["alpha"], pb["beta"], pb["mu"], pb["s"], o_dtype=torch.float32)
        outs.append((oa, ob))
    sa.synchronize()
    sb.synchronize()
    for oa, ob in outs:
        assert torch.equal(oa[0], ref_a[0]) and torch.equal(oa[1], ref_a[1])
        assert torch.equal(ob[0], ref_b[0]) and torch.equal(ob[1], ref_b[1])
