"""Paged-cache decode (bam_attn_decode_paged): the same result as bam_attn_decode on the
gathered cache, bit for bit (same keys, same splits, same arithmetic), and parity with the
fp64 oracle on that gathered cache (bf16 bar: |O| 1e-2, lse 1e-3).  Ragged kv_len
(1, partial pages, full) in one batch; pages assigned in a shuffled order."""
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


@pytest.mark.parametrize("P,max_blocks,Dh,kv", [(64, 20, 64, (1, 1280, 700, 65)), (256, 9, 64, (2304, 1000, 257, 3)),
                                                 (128, 12, 128, (1536, 129, 1, 800)), (64, 80, 64, (5120, 4099, 64, 1))])
def test_paged_decode(P, max_blocks, Dh, kv):
    torch = torch_mod()
    B, H = len(kv), 3
    Lmax = P * max_blocks
    w = wl.random_case(1300 + P + Dh, B, H, Lmax, Dh, "bf16", wl.SSMAX, beta_range=(0.3, 1.3))
    rng = np.random.default_rng(P + max_blocks)
    q = wl.bf16_round(rng.standard_normal((B, H, Dh)).astype(np.float32))
    kv_len = np.array(kv, np.int32)
    num_pages = B * max_blocks + 5
    perm = rng.permutation(num_pages)[: B * max_blocks].reshape(B, max_blocks).astype(np.int32)
    kp = np.zeros((num_pages, H, P, Dh), np.float32)
    vp = np.zeros((num_pages, H, P, Dh), np.float32)
    for b in range(B):
        for p in range(max_blocks):
            kp[perm[b, p]] = w.k[b, :, p * P:(p + 1) * P]
            vp[perm[b, p]] = w.v[b, :, p * P:(p + 1) * P]
    par = params(w)
    kvt = torch.from_numpy(kv_len).cuda()
    o1, l1 = _bam().bam_attn_decode_paged(dev(q, "bf16"), dev(kp, "bf16"), dev(vp, "bf16"),
                                          torch.from_numpy(perm).cuda(), kvt, par["alpha"], par["beta"], par["mu"],
                                          par["s"], ssmax=True, o_dtype=torch.float32)
    o2, l2 = _bam().bam_attn_decode(dev(q, "bf16"), dev(w.k, "bf16"), dev(w.v, "bf16"), kvt, par["alpha"],
                                    par["beta"], par["mu"], par["s"], ssmax=True, o_dtype=torch.float32)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(l1, l2)
    O, L = oracle.attn_decode(q, w.k, w.v, kv_len, w.alpha, w.beta, w.mu, w.s, ssmax=True)
    within(max_abs(host(o1), O), BF16_O_ABS, "max_abs(host(o1), O)")
    within(max_abs(host(l1), L), BF16_LSE_ABS, "max_abs(host(l1), L)")
