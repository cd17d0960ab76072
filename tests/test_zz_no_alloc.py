"""bam_attn_decode_static (no workspace: the library's static device buffer) against
bam_attn_decode on the same inputs, through the C ABI: two calls in a row, the second on a
smaller problem (fewer sequences and heads, a shorter cache, Dh = 32), each bit for bit
equal to the workspace call, which runs the same kernels with the same split of the keys.
The second case is also checked against the fp64 oracle (max |O - ref| <= 1e-2 on the fp32
output, |lse - ref| <= 1e-3)."""
import numpy as np
import pytest

import oracle
from gpu_util import within
from gpu_util import BF16_LSE_ABS, BF16_O_ABS, dev, host, max_abs, params, torch_mod
from positional_prior_bias_amd import workloads as wl

pytestmark = pytest.mark.gpu


def _case(w, o_dtype):
    import positional_prior_bias_amd as bam
    torch = torch_mod()
    p = params(w)
    q, k, v = dev(w.q, "bf16"), dev(w.k, "bf16"), dev(w.v, "bf16")
    kv = torch.from_numpy(w.kv_len.astype(np.int32)).cuda()
    B, H, Dh = w.q.shape
    ref_o, ref_l = bam.bam_attn_decode(q, k, v, kv, p["alpha"], p["beta"], p["mu"], p["s"], ssmax=True,
                                       o_dtype=o_dtype)
    o = torch.empty((B, H, Dh), dtype=o_dtype, device="cuda")
    lse = torch.empty((B, H), dtype=torch.float32, device="cuda")
    bam.bam_attn_decode_static(q, k, v, kv, p["alpha"], p["beta"], p["mu"], p["s"], ssmax=True, o=o, lse=lse)
    torch.cuda.synchronize()
    assert torch.equal(o, ref_o), float((o.float() - ref_o.float()).abs().max())
    assert torch.equal(lse, ref_l), float((lse - ref_l).abs().max())
    return o, lse


def test_static_decode_matches_workspace_decode_twice():
    torch = torch_mod()
    import positional_prior_bias_amd as bam
    big = wl.long_decode(seed=61, B=4, H=12, L=20000, Dh=64, kv_len=np.array([20000, 17, 12345, 4096]))
    need = bam.bam_decode_workspace_size(4, 12, 20000, 64)
    assert need <= bam.bam_decode_static_max_bytes()
    _case(big, torch.bfloat16)
    small = wl.long_decode(seed=62, B=2, H=4, L=3000, Dh=32, kv_len=np.array([2999, 1]))
    o, lse = _case(small, torch.float32)
    O, L = oracle.attn_decode(small.q, small.k, small.v, small.kv_len, small.alpha, small.beta, small.mu, small.s,
                              ssmax=True)
    within(max_abs(host(o), O), BF16_O_ABS, "static decode O")
    within(max_abs(host(lse), L), BF16_LSE_ABS, "static decode lse")
