"""The entry points under HIP graph capture.  The library enqueues kernels only (no
allocation, memset or synchronisation inside a call), so a captured forward + decode +
backward replays correctly: the graph is replayed several times with new input values
and eager work in between, and every replay equals the eager calls bit for bit."""
import numpy as np
import pytest

from gpu_util import dev, params, torch_mod
from positional_prior_bias_amd import workloads as wl

pytestmark = pytest.mark.gpu


def test_captured_fwd_decode_bwd_replays():
    torch = torch_mod()
    import positional_prior_bias_amd as bam
    B, H, T, Dh = 2, 3, 600, 64
    w = wl.random_case(2100, B, H, T, Dh, "bf16", wl.CAUSAL | wl.SSMAX, beta_range=(0.2, 1.2), with_grad=True)
    q, k, v, do = (dev(x, "bf16") for x in (w.q, w.k, w.v, w.do))
    p = params(w)
    pa = (p["alpha"], p["beta"], p["mu"], p["s"])
    f32 = torch.float32
    # static outputs and workspaces
    o = torch.empty((B, H, T, Dh), dtype=f32, device="cuda")
    lse = torch.empty((B, H, T), dtype=f32, device="cuda")
    wsf = torch.empty(bam.bam_fwd_workspace_size(B, H, T, Dh, 3), dtype=torch.uint8, device="cuda")
    qd = torch.empty((B, H, Dh), dtype=torch.bfloat16, device="cuda")
    kv = torch.tensor([T, T // 2], dtype=torch.int32, device="cuda")
    od = torch.empty((B, H, Dh), dtype=f32, device="cuda")
    ld = torch.empty((B, H), dtype=f32, device="cuda")
    wsd = torch.empty(bam.bam_decode_workspace_size(B, H, T, Dh), dtype=torch.uint8, device="cuda")
    wsb = torch.empty(bam.bam_bwd_workspace_size(B, H, T, Dh, 3), dtype=torch.uint8, device="cuda")

    def step():
        bam.bam_attn_fwd(q, k, v, *pa, o=o, lse=lse, workspace=wsf)
        qd.copy_(q[:, :, -1])
        bam.bam_attn_decode(qd, k, v, kv, *pa, o=od, lse=ld, workspace=wsd)
        return bam.bam_attn_bwd(q, k, v, o, lse, do, *pa, grad_dtype=f32, workspace=wsb)

    step()                              # warm up outside the capture
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        with torch.cuda.graph(g):
            grads = step()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()

    gen = torch.Generator(device="cuda")
    for rep in range(3):
        gen.manual_seed(rep)
        q.copy_(torch.randn(q.shape, device="cuda", generator=gen).to(torch.bfloat16))
        do.copy_(torch.randn(do.shape, device="cuda", generator=gen).to(torch.bfloat16))
        g.replay()
        torch.cuda.synchronize()
        got = [o.clone(), lse.clone(), od.clone(), ld.clone()] + [x.clone() for x in grads]
        # eager work between replays, then the eager reference on the same inputs
        _ = (torch.randn(1 << 20, device="cuda") * 2).sum().item()
        ref_o, ref_l = bam.bam_attn_fwd(q, k, v, *pa, o_dtype=f32)
        ref_od, ref_ld = bam.bam_attn_decode(q[:, :, -1].contiguous(), k, v, kv, *pa, o_dtype=f32)
        ref_g = bam.bam_attn_bwd(q, k, v, ref_o, ref_l, do, *pa, grad_dtype=f32)
        torch.cuda.synchronize()
        ref = [ref_o, ref_l, ref_od, ref_ld] + list(ref_g)
        for i, (a, b) in enumerate(zip(got, ref)):
            assert torch.equal(a, b), (rep, i)


def test_graphed_training_module_replays():
    """The autograd module under torch.cuda.make_graphed_callables (forward and backward
    captured as graphs): over three replays with new q and dO, eager work in between, the
    output and every gradient (q, k, v and the prior's parameters) equal the eager module's
    bit for bit."""
    torch = torch_mod()
    from positional_prior_bias_amd.autograd import BamAttention
    B, H, T, Dh = 2, 4, 300, 64
    w = wl.random_case(2200, B, H, T, Dh, "bf16", wl.CAUSAL | wl.SSMAX, with_grad=True)
    q0, k0, v0 = (dev(x, "bf16") for x in (w.q, w.k, w.v))
    torch.manual_seed(0)
    mod = BamAttention(H, max_seq_len=T, train_theta_mu=True, device="cuda")
    sample = tuple(x.clone().requires_grad_(True) for x in (q0, k0, v0))
    graphed = torch.cuda.make_graphed_callables(mod, sample)
    gen = torch.Generator(device="cuda")
    for rep in range(3):
        gen.manual_seed(100 + rep)
        qn = torch.randn(q0.shape, device="cuda", generator=gen).to(torch.bfloat16)
        dn = torch.randn(q0.shape, device="cuda", generator=gen).to(torch.bfloat16)
        res = []
        for fn in (graphed, mod):
            x = [t.clone().requires_grad_(True) for t in (qn, k0, v0)]
            for prm in mod.parameters():
                prm.grad = None
            out = fn(*x)
            out.backward(dn)
            torch.cuda.synchronize()
            res.append([out.detach().clone()] + [t.grad.clone() for t in x]
                       + [prm.grad.clone() for prm in mod.parameters() if prm.grad is not None])
            _ = (torch.randn(1 << 20, device="cuda") * 2).sum().item()
        assert len(res[0]) == len(res[1]) == 8, (len(res[0]), len(res[1]))
        for i, (a, b) in enumerate(zip(res[0], res[1])):
            assert torch.equal(a, b), (rep, i)
