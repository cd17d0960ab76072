"""Seeded synthetic inputs for BAM attention.

This module only draws random numbers and lays them out; it holds none of the
attention arithmetic.  Both the HIP path (through the Python binding) and the
CPU oracle consume exactly these arrays, so a parity test compares the two on
identical inputs.

Conventions
-----------
* numpy ``default_rng(seed)`` (PCG64), arrays drawn in the order documented per
  workload, C order, ``standard_normal(dtype=float32)``.
* "bf16" arrays are the float32 draw rounded to nearest-even bfloat16 and kept
  here as float32 arrays holding exactly-representable bf16 values, so the
  oracle can widen them to float64 without any further rounding.
* Per-head prior parameters are float32 arrays of length H: ``alpha`` (scale,
  > 0, +inf allowed), ``beta`` (shape, any finite value), ``mu`` (offset) and
  ``s`` (Scalable-Softmax strength).

Workload shapes follow the pages' settings: a 12-head model trained at a
512-token context (Bayesian Attention Mechanism, "Usage": sequence length 512
on FineWeb), passkey-style extrapolation to 32k tokens ("Evaluation") and
retrieval at 500x the training context ("Highlights").
"""
from __future__ import annotations

import dataclasses
import math

import numpy as np

CAUSAL = 1
SSMAX = 2


def bf16_round(x: np.ndarray) -> np.ndarray:
    """Round float32 values to the nearest bfloat16 (ties to even).

    Returns a float32 array whose values are exactly representable in bf16.  Inputs
    here are finite draws, so the 32-bit add cannot overflow and NaN handling is not
    needed.
    """
    x = np.ascontiguousarray(x, dtype=np.float32)
    u = x.view(np.uint32)
    r = u + np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1))
    r &= np.uint32(0xFFFF0000)
    return r.view(np.float32).reshape(x.shape)


def to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Upper 16 bits of float32 values that are already bf16-exact."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    return (x.view(np.uint32) >> 16).astype(np.uint16)


@dataclasses.dataclass
class Workload:
    name: str
    B: int
    H: int
    T: int            # query/key length for prefill; Lmax for decode
    Dh: int
    dtype: str        # "bf16" or "f32": the element type Q/K/V are stored in
    flags: int        # CAUSAL | SSMAX bits
    alpha: np.ndarray
    beta: np.ndarray
    mu: np.ndarray
    s: np.ndarray
    q: np.ndarray | None = None
    k: np.ndarray | None = None
    v: np.ndarray | None = None
    do: np.ndarray | None = None
    kv_len: np.ndarray | None = None   # decode only, int32 [B]
    planted: np.ndarray | None = None  # decode only, planted key position per sequence

    @property
    def causal(self) -> bool:
        return bool(self.flags & CAUSAL)

    @property
    def ssmax(self) -> bool:
        return bool(self.flags & SSMAX)


def _normal(rng, shape, bf16: bool) -> np.ndarray:
    x = rng.standard_normal(size=shape, dtype=np.float32)
    return bf16_round(x) if bf16 else x


def tiny_check(seed: int = 0, B: int = 1, H: int = 4, T: int = 256, Dh: int = 32) -> Workload:
    """Small fp32 case the oracle finishes in well under a second.

    Draw order: Q, K, V; alpha ~ U(1,32); beta ~ U(0.3,1.5).  mu = 0, SSMax off.
    """
    rng = np.random.default_rng(seed)
    q = _normal(rng, (B, H, T, Dh), False)
    k = _normal(rng, (B, H, T, Dh), False)
    v = _normal(rng, (B, H, T, Dh), False)
    alpha = rng.uniform(1.0, 32.0, H).astype(np.float32)
    beta = rng.uniform(0.3, 1.5, H).astype(np.float32)
    mu = np.zeros(H, np.float32)
    s = np.ones(H, np.float32)  # unused with SSMax off
    return Workload("tiny_check_fp32", B, H, T, Dh, "f32", CAUSAL, alpha, beta, mu, s, q, k, v)


def training_shape(seed: int = 1, B: int = 32, H: int = 12, T: int = 512, Dh: int = 64,
                   with_grad: bool = False, grad_seed: int = 2) -> Workload:
    """Training-context forward (optionally with dO for the backward).

    Draw order (seed): Q, K, V; alpha = exp(U(0, ln 512)); beta ~ U(0.2, 1.2);
    s ~ U(0.3, 0.6).  mu = 0.  Causal, SSMax on.  dO from its own seed.
    """
    rng = np.random.default_rng(seed)
    q = _normal(rng, (B, H, T, Dh), True)
    k = _normal(rng, (B, H, T, Dh), True)
    v = _normal(rng, (B, H, T, Dh), True)
    alpha = np.exp(rng.uniform(0.0, math.log(512.0), H)).astype(np.float32)
    beta = rng.uniform(0.2, 1.2, H).astype(np.float32)
    s = rng.uniform(0.3, 0.6, H).astype(np.float32)
    mu = np.zeros(H, np.float32)
    w = Workload("train_T%d" % T, B, H, T, Dh, "bf16", CAUSAL | SSMAX, alpha, beta, mu, s, q, k, v)
    if with_grad:
        w.do = _normal(np.random.default_rng(grad_seed), (B, H, T, Dh), True)
        w.name = "train_fwdbwd_T%d" % T
    return w


def extrapolation_heads(rng, H: int = 12):
    """Head parameters of the long-context workloads.

    First half: heavy-tailed heads, alpha = exp(U(0, ln 4096)), beta ~ U(0.1, 0.9), mu = 0.
    Second half: inverted-prior heads, alpha ~ U(0.5, 4), beta ~ U(-0.8, -0.1), mu = -0.5
    (so the distance minus the offset is never zero).  s = 0.45 for every head.
    """
    h1 = H // 2
    h2 = H - h1
    a1 = np.exp(rng.uniform(0.0, math.log(4096.0), h1))
    b1 = rng.uniform(0.1, 0.9, h1)
    a2 = rng.uniform(0.5, 4.0, h2)
    b2 = rng.uniform(-0.8, -0.1, h2)
    alpha = np.concatenate([a1, a2]).astype(np.float32)
    beta = np.concatenate([b1, b2]).astype(np.float32)
    mu = np.concatenate([np.zeros(h1), np.full(h2, -0.5)]).astype(np.float32)
    s = np.full(H, 0.45, np.float32)
    return alpha, beta, mu, s


def long_prefill(seed: int = 3, B: int = 1, H: int = 12, T: int = 32768, Dh: int = 64) -> Workload:
    """Length-extrapolation prefill.  Draw order: Q, K, V, then the head parameters."""
    rng = np.random.default_rng(seed)
    q = _normal(rng, (B, H, T, Dh), True)
    k = _normal(rng, (B, H, T, Dh), True)
    v = _normal(rng, (B, H, T, Dh), True)
    alpha, beta, mu, s = extrapolation_heads(rng, H)
    return Workload("prefill_T%d" % T, B, H, T, Dh, "bf16", CAUSAL | SSMAX, alpha, beta, mu, s, q, k, v)


def long_decode(seed: int = 4, B: int = 8, H: int = 12, L: int = 256000, Dh: int = 64,
                head_seed: int = 3, kv_len: np.ndarray | None = None) -> Workload:
    """One query row per sequence against a long KV cache.

    Draw order (seed): K, then V, each one (b, h) slab of L x Dh at a time (bounds host
    memory); q (B, H, Dh); the planted positions p ~ integers(0, kv_len[b]).  In every
    head of sequence b the key at p[b] is moved along the query direction by 8 units,
    k_p <- bf16(k_p + 8 q / |q|), which raises q.k by 8|q|, i.e. the scaled score by
    about 8 standard deviations.  Head parameters are those of the long prefill
    (drawn from ``head_seed`` the same way).
    """
    rng = np.random.default_rng(seed)
    k = np.empty((B, H, L, Dh), np.float32)
    v = np.empty((B, H, L, Dh), np.float32)
    for b in range(B):
        for h in range(H):
            k[b, h] = _normal(rng, (L, Dh), True)
    for b in range(B):
        for h in range(H):
            v[b, h] = _normal(rng, (L, Dh), True)
    q = _normal(rng, (B, H, Dh), True)
    if kv_len is None:
        kv_len = np.full(B, L, np.int32)
    kv_len = np.asarray(kv_len, np.int32)
    planted = np.array([rng.integers(0, kv_len[b]) for b in range(B)], np.int64)
    for b in range(B):
        p = planted[b]
        for h in range(H):
            qv = q[b, h].astype(np.float64)
            k[b, h, p] = bf16_round((k[b, h, p] + 8.0 * qv / np.linalg.norm(qv)).astype(np.float32))
    # head parameters: same draw as the long prefill (Q, K, V first, then heads)
    hrng = np.random.default_rng(head_seed)
    _ = hrng.standard_normal(size=(1, H, 32768, Dh), dtype=np.float32)
    _ = hrng.standard_normal(size=(1, H, 32768, Dh), dtype=np.float32)
    _ = hrng.standard_normal(size=(1, H, 32768, Dh), dtype=np.float32)
    alpha, beta, mu, s = extrapolation_heads(hrng, H)
    w = Workload("decode_L%d" % L, B, H, L, Dh, "bf16", SSMAX, alpha, beta, mu, s, q, k, v,
                 kv_len=kv_len, planted=planted)
    return w


def random_case(seed: int, B: int, H: int, T: int, Dh: int, dtype: str = "bf16",
                flags: int = CAUSAL | SSMAX, beta_range=(0.2, 1.2), alpha_range=(1.0, 512.0),
                mu: float = 0.0, s_range=(0.3, 0.6), with_grad: bool = False) -> Workload:
    """Generic small case for parity sweeps (ragged T, several tiles).

    Draw order: Q, K, V, alpha = exp(U(ln a0, ln a1)), beta ~ U(beta_range),
    s ~ U(s_range), then dO if requested.
    """
    rng = np.random.default_rng(seed)
    bf = dtype == "bf16"
    q = _normal(rng, (B, H, T, Dh), bf)
    k = _normal(rng, (B, H, T, Dh), bf)
    v = _normal(rng, (B, H, T, Dh), bf)
    alpha = np.exp(rng.uniform(math.log(alpha_range[0]), math.log(alpha_range[1]), H)).astype(np.float32)
    beta = rng.uniform(beta_range[0], beta_range[1], H).astype(np.float32)
    s = rng.uniform(s_range[0], s_range[1], H).astype(np.float32)
    mus = np.full(H, mu, np.float32)
    w = Workload("random_T%d" % T, B, H, T, Dh, dtype, flags, alpha, beta, mus, s, q, k, v)
    if with_grad:
        w.do = _normal(rng, (B, H, T, Dh), bf)
    return w


def ref_case(seed: int, B: int, H: int, T: int, Dh: int, dtype: str = "bf16", flags: int = CAUSAL | SSMAX,
             theta_alpha_range=(-3.0, 0.5), theta_beta_range=(0.0, 1.0), theta_mu_range=(-0.5, 0.5),
             s_range=(0.3, 0.6), with_grad: bool = False) -> Workload:
    """Small case in the reference parameterisation: the workload's alpha / beta / mu
    arrays hold theta_alpha / theta_beta / theta_mu.

    The default theta_beta range is the page's linspace(0, 1) head initialisation
    ("Bayesian Attention Mechanism" README, "Implementation Details").  Draw order: Q, K,
    V, theta_alpha ~ U, theta_beta ~ U, theta_mu ~ U, s ~ U, then dO if requested.
    """
    rng = np.random.default_rng(seed)
    bf = dtype == "bf16"
    q = _normal(rng, (B, H, T, Dh), bf)
    k = _normal(rng, (B, H, T, Dh), bf)
    v = _normal(rng, (B, H, T, Dh), bf)
    ta = rng.uniform(*theta_alpha_range, H).astype(np.float32)
    tb = rng.uniform(*theta_beta_range, H).astype(np.float32)
    tm = rng.uniform(*theta_mu_range, H).astype(np.float32)
    s = rng.uniform(s_range[0], s_range[1], H).astype(np.float32)
    w = Workload("ref_T%d" % T, B, H, T, Dh, dtype, flags, ta, tb, tm, s, q, k, v)
    if with_grad:
        w.do = _normal(rng, (B, H, T, Dh), bf)
    return w


def sandwich_case(seed: int, B: int, H: int, T: int, Dh: int, dtype: str = "bf16", flags: int = CAUSAL | SSMAX,
                  d_bar: float = 128.0, s_range=(0.3, 0.6), with_grad: bool = False) -> Workload:
    """Small case with the Sandwich bias: alpha holds the per-head compression ratios
    8 (h + 1) / H and beta d_bar (attention-gym "Score Mods", "Sandwich": the page's
    defaults); mu is zero.  Draw order: Q, K, V, s ~ U, then dO if requested.
    """
    rng = np.random.default_rng(seed)
    bf = dtype == "bf16"
    q = _normal(rng, (B, H, T, Dh), bf)
    k = _normal(rng, (B, H, T, Dh), bf)
    v = _normal(rng, (B, H, T, Dh), bf)
    ratio = np.array([8.0 * (h + 1) / H for h in range(H)], np.float32)
    dbar = np.full(H, d_bar, np.float32)
    s = rng.uniform(s_range[0], s_range[1], H).astype(np.float32)
    w = Workload("sandwich_T%d" % T, B, H, T, Dh, dtype, flags, ratio, dbar, np.zeros(H, np.float32), s, q, k, v)
    if with_grad:
        w.do = _normal(rng, (B, H, T, Dh), bf)
    return w


def alibi_slopes(H: int) -> np.ndarray:
    """Per-head ALiBi slopes m_h = 2^(-8(h+1)/H) for every H.

    NNX ALiBi-Style Attention, "One fixed slope per head" (the exercise applies this
    schedule to every head count, power of two or not).
    """
    return np.array([2.0 ** (-8.0 * (h + 1) / H) for h in range(H)], np.float64)


def long_decode_device(seed: int = 4, B: int = 8, H: int = 12, L: int = 256000, Dh: int = 64,
                       head_seed: int = 3, kv_len: np.ndarray | None = None, device="cuda") -> Workload:
    """Decode workload with the KV caches drawn directly on the GPU (256k-token caches).

    K and V ([B, H, L, Dh], bf16) come from torch's counter-based Philox generator on
    `device`, seeded with `seed`: for each sequence b, K[b] is one float32 randn draw of
    (H, L, Dh) rounded to bf16, then V[b] likewise, b = 0, 1, ...  q (B, H, Dh) and the
    planted positions come from numpy default_rng(seed) as in long_decode; the planted key
    of sequence b is k_p <- bf16(k_p + 8 q / |q|) in every head.  The returned workload's
    k and v are torch device tensors; everything else is numpy.  Head parameters are those
    of the long prefill.
    """
    import torch
    gen = torch.Generator(device=device)
    gen.manual_seed(seed)
    k = torch.empty((B, H, L, Dh), dtype=torch.bfloat16, device=device)
    v = torch.empty((B, H, L, Dh), dtype=torch.bfloat16, device=device)
    for b in range(B):
        k[b] = torch.randn((H, L, Dh), generator=gen, dtype=torch.float32, device=device).to(torch.bfloat16)
        v[b] = torch.randn((H, L, Dh), generator=gen, dtype=torch.float32, device=device).to(torch.bfloat16)
    rng = np.random.default_rng(seed)
    q = _normal(rng, (B, H, Dh), True)
    if kv_len is None:
        kv_len = np.full(B, L, np.int32)
    kv_len = np.asarray(kv_len, np.int32)
    planted = np.array([rng.integers(0, kv_len[b]) for b in range(B)], np.int64)
    for b in range(B):
        p = int(planted[b])
        dirs = q[b].astype(np.float64)
        dirs = 8.0 * dirs / np.linalg.norm(dirs, axis=1, keepdims=True)
        row = k[b, :, p].to(torch.float64) + torch.from_numpy(dirs).to(device)
        k[b, :, p] = row.to(torch.float32).to(torch.bfloat16)
    hrng = np.random.default_rng(head_seed)
    for _ in range(3):
        hrng.standard_normal(size=(1, H, 32768, Dh), dtype=np.float32)
    alpha, beta, mu, s = extrapolation_heads(hrng, H)
    return Workload("decode_L%d_device" % L, B, H, L, Dh, "bf16", SSMAX, alpha, beta, mu, s, q, k, v,
                    kv_len=kv_len, planted=planted)


def long_prefill_heads(H: int = 12, Dh: int = 64, seed: int = 3):
    """The head parameters of the 32,768-token prefill (drawn after its Q, K, V from `seed`)."""
    rng = np.random.default_rng(seed)
    for _ in range(3):
        rng.standard_normal(size=(1, H, 32768, Dh), dtype=np.float32)
    return extrapolation_heads(rng, H)


def long_prefill_device(seed: int = 3, B: int = 1, H: int = 12, T: int = 262144, Dh: int = 64,
                        device="cuda") -> Workload:
    """Length-sweep prefill with Q, K, V drawn directly on the GPU (lengths past 32k).

    Q, K, V ([B, H, T, Dh], bf16) come from torch's counter-based Philox generator on
    `device`, seeded with `seed`: one float32 randn draw of (B, H, T, Dh) each, in that
    order, rounded to bf16.  The head parameters are those of the 32,768-token prefill
    (long_prefill_heads), so every length of the sweep runs the same heads.  The returned
    workload's q, k and v are torch device tensors.
    """
    import torch
    gen = torch.Generator(device=device)
    gen.manual_seed(seed)
    qkv = [torch.randn((B, H, T, Dh), generator=gen, dtype=torch.float32, device=device).to(torch.bfloat16)
           for _ in range(3)]
    alpha, beta, mu, s = long_prefill_heads(H, Dh, 3)
    return Workload("prefill_T%d_device" % T, B, H, T, Dh, "bf16", CAUSAL | SSMAX, alpha, beta, mu, s, *qkv)
