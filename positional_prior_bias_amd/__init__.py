"""BAM attention on AMD Instinct MI355X (gfx950): Python binding of libbam.so.

The functions here carry the C entry points' names (include/bam.h) and only
marshal arguments: they check every tensor argument's shape, dtype and device
against what the kernels will address (raising BamError before anything is
launched), allocate outputs and the workspace with torch, and pass raw device
pointers plus torch's current HIP stream to the library.  Every step of the computation runs in the library's
HIP kernels; there is no fallback path.  If libbam.so has not been built the
first call raises.
"""
from __future__ import annotations

import ctypes
import functools
import os

__all__ = [
    "BAM_BF16", "BAM_F32", "BAM_CAUSAL", "BAM_SSMAX", "BAM_TABLE_READY", "BAM_PRIOR_REF", "BAM_REF_EPS",
    "BAM_PRIOR_SANDWICH", "sandwich_ratios", "alibi_slopes", "BAM_SKIP_FAR", "bam_fwd_skip_plan_offset",
    "fwd_skipped_fraction", "fwd_rows_per_block",
    "BamError", "lib", "lib_path",
    "bam_prior_table", "bam_prior_table_ex", "bam_attn_fwd", "bam_attn_decode", "bam_attn_decode_paged",
    "bam_attn_bwd",
    "bam_attn_bwd_ex", "bam_attn_decode_static", "bam_decode_static_max_bytes",
    "bam_fwd_workspace_size", "bam_decode_workspace_size", "bam_bwd_workspace_size",
    "EXPORTED_SYMBOLS",
]

BAM_BF16 = 0
BAM_F32 = 1
BAM_CAUSAL = 1
BAM_SSMAX = 2
BAM_TABLE_READY = 4
BAM_PRIOR_REF = 8
BAM_PRIOR_SANDWICH = 16
BAM_SKIP_FAR = 32
BAM_REF_EPS = 1e-5

_DIR = os.path.dirname(os.path.abspath(__file__))
_LIB = None

EXPORTED_SYMBOLS = (
    "bam_status_string", "bam_version", "bam_prior_table", "bam_prior_table_ex",
    "bam_fwd_workspace_size", "bam_attn_fwd", "bam_fwd_skip_plan_offset",
    "bam_decode_workspace_size", "bam_attn_decode", "bam_attn_decode_paged",
    "bam_decode_static_max_bytes", "bam_attn_decode_static",
    "bam_decode_partials_layout", "bam_decode_norm_pages", "bam_decode_key_norms", "bam_attn_decode_skip",
    "bam_bwd_workspace_size", "bam_attn_bwd", "bam_attn_bwd_ex",
)


class BamError(RuntimeError):
    pass


def lib_path() -> str:
    return os.path.join(_DIR, "libbam.so")


def _declare(L):
    vp, i, u, sz, fp = ctypes.c_void_p, ctypes.c_int, ctypes.c_uint, ctypes.c_size_t, ctypes.c_void_p
    L.bam_status_string.restype = ctypes.c_char_p
    L.bam_status_string.argtypes = [i]
    L.bam_version.restype = i
    L.bam_version.argtypes = []
    L.bam_prior_table.restype = i
    L.bam_prior_table.argtypes = [fp, fp, fp, i, i, i, fp, fp, fp, vp]
    L.bam_prior_table_ex.restype = i
    L.bam_prior_table_ex.argtypes = [fp, fp, fp, i, i, i, u, fp, fp, fp, fp, vp]
    L.bam_fwd_workspace_size.restype = sz
    L.bam_fwd_workspace_size.argtypes = [i, i, i, i, u]
    L.bam_attn_fwd.restype = i
    L.bam_fwd_skip_plan_offset.restype = i
    L.bam_fwd_skip_plan_offset.argtypes = [i, i, i, i, u, ctypes.POINTER(sz), ctypes.POINTER(i)]
    L.bam_attn_fwd.argtypes = [vp, vp, vp, i, i, i, i, i, fp, fp, fp, fp, u, vp, i, fp, vp, sz, vp]
    L.bam_decode_workspace_size.restype = sz
    L.bam_decode_workspace_size.argtypes = [i, i, i, i]
    L.bam_attn_decode.restype = i
    L.bam_attn_decode.argtypes = [vp, vp, vp, i, vp, i, i, i, i, fp, fp, fp, fp, u, vp, i, fp, vp, sz, vp]
    L.bam_attn_decode_paged.restype = i
    L.bam_attn_decode_paged.argtypes = [vp, vp, vp, i, vp, i, i, i, vp, i, i, i, fp, fp, fp, fp, u, vp, i, fp, vp,
                                        sz, vp]
    L.bam_decode_static_max_bytes.restype = sz
    L.bam_decode_static_max_bytes.argtypes = []
    L.bam_attn_decode_static.restype = i
    L.bam_attn_decode_static.argtypes = [vp, vp, vp, i, vp, i, i, i, i, fp, fp, fp, fp, u, vp, i, fp, vp]
    L.bam_decode_partials_layout.restype = i
    L.bam_decode_partials_layout.argtypes = [i, i, i, i, ctypes.POINTER(sz), ctypes.POINTER(i), ctypes.POINTER(i)]
    L.bam_decode_norm_pages.restype = i
    L.bam_decode_norm_pages.argtypes = [i]
    L.bam_decode_key_norms.restype = i
    L.bam_decode_key_norms.argtypes = [vp, i, i, i, i, i, fp, vp]
    L.bam_attn_decode_skip.restype = i
    L.bam_attn_decode_skip.argtypes = [vp, vp, vp, i, vp, i, i, i, i, fp, fp, fp, fp, u, fp, vp, i, fp, vp, sz,
                                       vp]
    L.bam_bwd_workspace_size.restype = sz
    L.bam_bwd_workspace_size.argtypes = [i, i, i, i, u]
    L.bam_attn_bwd.restype = i
    L.bam_attn_bwd.argtypes = [vp, vp, vp, vp, i, fp, vp, i, i, i, i, i, fp, fp, fp, fp, u,
                               vp, vp, vp, i, fp, fp, fp, vp, sz, vp]
    L.bam_attn_bwd_ex.restype = i
    L.bam_attn_bwd_ex.argtypes = [vp, vp, vp, vp, i, fp, vp, i, i, i, i, i, fp, fp, fp, fp, u,
                                  vp, vp, vp, i, fp, fp, fp, fp, vp, sz, vp]


def lib():
    """Load libbam.so (once).  Raises BamError if it is missing."""
    global _LIB
    if _LIB is None:
        path = lib_path()
        if not os.path.exists(path):
            raise BamError(f"{path} is not built; run `python -m positional_prior_bias_amd.build`")
        L = ctypes.CDLL(path)
        _declare(L)
        _LIB = L
    return _LIB


def _check(status: int, what: str):
    if status != 0:
        raise BamError(f"{what}: {lib().bam_status_string(status).decode()} (status {status})")


# ---------------------------------------------------------------------------------------
# torch marshalling helpers
# ---------------------------------------------------------------------------------------

_TORCH = None


def _torch():
    global _TORCH
    if _TORCH is None:
        import torch
        _TORCH = torch
    return _TORCH


def _dtype_code(t) -> int:
    torch = _torch()
    if t.dtype == torch.bfloat16:
        return BAM_BF16
    if t.dtype == torch.float32:
        return BAM_F32
    raise BamError(f"unsupported dtype {t.dtype} (bfloat16 or float32)")


def _torch_dtype(code: int):
    torch = _torch()
    return torch.bfloat16 if code == BAM_BF16 else torch.float32


def _dev(t, name):
    if t is None:
        return None
    if not t.is_cuda:
        raise BamError(f"{name} must be a device tensor")
    if not t.is_contiguous():
        raise BamError(f"{name} must be contiguous")
    return t.data_ptr()


def _ptr(t):
    return None if t is None else t.data_ptr()


def _stream(stream=None):
    """The HIP stream handle to launch on: the given stream's, else the current stream of the
    current device (read with torch's C accessors: torch.cuda.current_stream() costs several
    microseconds of Python per call)."""
    if stream is not None:
        return stream.cuda_stream
    C = _torch()._C
    return C._cuda_getCurrentRawStream(C._cuda_getDevice())


def _expect(t, name, shape=None, dtypes=None, device=None):
    """Check a tensor argument's shape, dtype and device against what the kernels will
    address (a mismatch would become an out-of-bounds access on the GPU)."""
    if t is None:
        raise BamError(f"{name} is required")
    if shape is not None and t.shape != shape:
        raise BamError(f"{name} has shape {tuple(t.shape)}, expected {tuple(shape)}")
    if dtypes is not None and t.dtype not in dtypes:
        raise BamError(f"{name} has dtype {t.dtype}, expected one of {tuple(dtypes)}")
    if device is not None and t.device != device:
        raise BamError(f"{name} is on {t.device}, expected {device}")
    return t


def _shape(t, name, ndim):
    if t is None or t.dim() != ndim:
        raise BamError(f"{name} must be a {ndim}-D tensor")
    return tuple(t.shape)


def _check_params(alpha, beta, mu, s, flags, H, device):
    """The per-head prior arrays: float32 with H entries on the data's device (mu may be
    None; s is required with SSMax and otherwise ignored)."""
    f32 = (_torch().float32,)
    for name, t in (("alpha", alpha), ("beta", beta)):
        _expect(t, name, shape=(H,), dtypes=f32, device=device)
    if mu is not None:
        _expect(mu, "mu", shape=(H,), dtypes=f32, device=device)
    if flags & BAM_SSMAX:
        _expect(s, "s", shape=(H,), dtypes=f32, device=device)
    elif s is not None:
        _expect(s, "s", shape=(H,), dtypes=f32, device=device)


def _param_ptrs(alpha, beta, mu, s):
    return _dev(alpha, "alpha"), _dev(beta, "beta"), _dev(mu, "mu"), _dev(s, "s")


def _workspace(nbytes, device, workspace=None):
    torch = _torch()
    if workspace is not None:
        _expect(workspace, "workspace", device=device)
        if not workspace.is_contiguous():
            raise BamError("workspace must be contiguous")
        if workspace.numel() * workspace.element_size() < nbytes:
            raise BamError("workspace too small")
        return workspace
    return torch.empty(max(int(nbytes), 256), dtype=torch.uint8, device=device)


_PRIOR_FLAGS = {None: 0, "alpha": 0, "ref": BAM_PRIOR_REF, "sandwich": BAM_PRIOR_SANDWICH}


def _prior_flag(prior_ref: bool, prior) -> int:
    """prior: "alpha" (the GGD alpha-form), "ref" (theta parameterisation) or "sandwich";
    prior_ref=True is the same as prior="ref"."""
    if prior not in _PRIOR_FLAGS:
        raise BamError(f"unknown prior {prior!r}")
    f = _PRIOR_FLAGS[prior] | (BAM_PRIOR_REF if prior_ref else 0)
    if f == BAM_PRIOR_REF | BAM_PRIOR_SANDWICH:
        raise BamError("prior_ref and the sandwich prior exclude each other")
    return f


def _flags(causal: bool, ssmax: bool, prior_ref: bool = False, prior=None) -> int:
    return (BAM_CAUSAL if causal else 0) | (BAM_SSMAX if ssmax else 0) | _prior_flag(prior_ref, prior)


def sandwich_ratios(n_heads, device=None):
    """Per-head Sandwich compression ratios 8 (h + 1) / H (attention-gym "Score Mods",
    "Sandwich"), float32 [H]: the alpha argument with prior="sandwich"."""
    torch = _torch()
    return torch.tensor([8.0 * (h + 1) / n_heads for h in range(n_heads)], dtype=torch.float32, device=device)


def alibi_slopes(n_heads, device=None):
    """ALiBi slopes 2^(-8 (h + 1) / H), float32 [H] ("ALiBi: Attention with Linear Biases",
    "Code"; NNX ALiBi-Style Attention, "One fixed slope per head").  ALiBi is the alpha-form
    prior with beta = 1, mu = 0 and alpha = 1 / slope."""
    torch = _torch()
    return torch.tensor([2.0 ** (-8.0 * (h + 1) / n_heads) for h in range(n_heads)], dtype=torch.float32,
                        device=device)


# ---------------------------------------------------------------------------------------
# entry points (same names as the C ABI)
# ---------------------------------------------------------------------------------------

@functools.lru_cache(maxsize=256)
def bam_fwd_workspace_size(B, H, T, Dh, flags) -> int:
    return int(lib().bam_fwd_workspace_size(B, H, T, Dh, flags))


@functools.lru_cache(maxsize=256)
def bam_decode_workspace_size(B, H, Lmax, Dh) -> int:
    return int(lib().bam_decode_workspace_size(B, H, Lmax, Dh))


@functools.lru_cache(maxsize=256)
def bam_bwd_workspace_size(B, H, T, Dh, flags) -> int:
    return int(lib().bam_bwd_workspace_size(B, H, T, Dh, flags))


def bam_prior_table(alpha, beta, mu, d0: int, n: int, derivatives: bool = False, stream=None):
    """tab[h, t] = b_h(d0 + t) (float32 [H, n]); with derivatives also db/dalpha, db/dbeta."""
    torch = _torch()
    H = _shape(alpha, "alpha", 1)[0]
    _check_params(alpha, beta, mu, None, 0, H, alpha.device)
    a, b, m, _ = _param_ptrs(alpha, beta, mu, None)
    tab = torch.empty((H, n), dtype=torch.float32, device=alpha.device)
    da = torch.empty_like(tab) if derivatives else None
    db = torch.empty_like(tab) if derivatives else None
    st = lib().bam_prior_table(a, b, m, H, d0, n, _ptr(tab), _ptr(da), _ptr(db), _stream(stream))
    _check(st, "bam_prior_table")
    return (tab, da, db) if derivatives else tab


def bam_prior_table_ex(alpha, beta, mu, d0: int, n: int, prior_ref: bool = False, stream=None, prior=None):
    """(tab, dalpha, dbeta, dmu), each float32 [H, n]: the bias of distance d0 + t and its
    derivatives in the three per-head parameters (theta's with prior_ref)."""
    torch = _torch()
    H = _shape(alpha, "alpha", 1)[0]
    flags = _prior_flag(prior_ref, prior)
    _check_params(alpha, beta, mu, None, 0, H, alpha.device)
    a, b, m, _ = _param_ptrs(alpha, beta, mu, None)
    outs = [torch.empty((H, n), dtype=torch.float32, device=alpha.device) for _ in range(4)]
    st = lib().bam_prior_table_ex(a, b, m, H, d0, n, flags, *(_ptr(t) for t in outs), _stream(stream))
    _check(st, "bam_prior_table_ex")
    return tuple(outs)


def bam_fwd_skip_plan_offset(B, H, T, Dh, flags):
    """(byte offset, count) of the int32 skipping plan a BAM_SKIP_FAR forward leaves in its
    workspace: entry qb * B * H + b * H + h = leading 64-key tiles query block qb skipped."""
    off, cnt = ctypes.c_size_t(0), ctypes.c_int(0)
    _check(lib().bam_fwd_skip_plan_offset(B, H, T, Dh, flags, ctypes.byref(off), ctypes.byref(cnt)),
           "bam_fwd_skip_plan_offset")
    return int(off.value), int(cnt.value)


def fwd_rows_per_block(Dh, T):
    """Query rows per work-group of the bf16 forward (the rule include/bam.h states for the
    skipping plan): 128 for Dh = 128 and for Dh = 64 with T <= 1024, else 256."""
    return 128 if (Dh == 128 or (Dh == 64 and T <= 1024)) else 256


def fwd_skipped_fraction(workspace, B, H, T, Dh, flags):
    """Fraction of the causal forward's (query block, key tile) pairs that the last
    BAM_SKIP_FAR call on `workspace` left out (reads the plan back to the host)."""
    torch = _torch()
    off, cnt = bam_fwd_skip_plan_offset(B, H, T, Dh, flags)
    plan = workspace[off:off + 4 * cnt].view(torch.int32).cpu().long()
    rows = fwd_rows_per_block(Dh, T)
    nqb = cnt // (B * H)
    qb = torch.arange(nqb).repeat_interleave(B * H)
    total = ((torch.clamp((qb + 1) * rows, max=T) + 63) // 64).sum().item()
    return float(plan.sum().item()) / float(total)


def bam_attn_fwd(q, k, v, alpha, beta, mu=None, s=None, causal=True, ssmax=True, o_dtype=None,
                 o=None, lse=None, workspace=None, stream=None, table_ready=False, prior_ref=False,
                 prior=None, skip_far=False):
    """Prefill forward; q, k, v [B, H, T, Dh].  Returns (o, lse).

    table_ready: the given workspace already holds this call's distance table (BAM_TABLE_READY).
    prior_ref: alpha / beta / mu hold theta_alpha / theta_beta / theta_mu (BAM_PRIOR_REF).
    prior="sandwich": the Sandwich bias, alpha = ratio_h, beta = d_bar (BAM_PRIOR_SANDWICH).
    skip_far: leave out the leading key tiles whose weights are zero in float32 (BAM_SKIP_FAR;
    causal bf16 only)."""
    torch = _torch()
    B, H, T, Dh = _shape(q, "q", 4)
    flags = (_flags(causal, ssmax, prior_ref, prior) | (BAM_TABLE_READY if table_ready else 0)
             | (BAM_SKIP_FAR if skip_far else 0))
    if table_ready and workspace is None:
        raise BamError("table_ready needs the workspace of an earlier call")
    in_code = _dtype_code(q)
    dev = q.device
    for name, t in (("k", k), ("v", v)):
        _expect(t, name, shape=q.shape, dtypes=(q.dtype,), device=dev)
    io = (torch.bfloat16, torch.float32)
    oc = in_code if o_dtype is None else (_dtype_code(torch.empty(0, dtype=o_dtype)))
    if o is None:
        o = torch.empty((B, H, T, Dh), dtype=_torch_dtype(oc), device=dev)
    else:
        _expect(o, "o", shape=(B, H, T, Dh), dtypes=io, device=dev)
        oc = _dtype_code(o)
    if lse is None:
        lse = torch.empty((B, H, T), dtype=torch.float32, device=dev)
    else:
        _expect(lse, "lse", shape=(B, H, T), dtypes=(torch.float32,), device=dev)
    _check_params(alpha, beta, mu, s, flags, H, dev)
    nb = bam_fwd_workspace_size(B, H, T, Dh, flags & ~BAM_TABLE_READY)
    ws = _workspace(nb, dev, workspace)
    a, b_, m_, s_ = _param_ptrs(alpha, beta, mu, s)
    st = lib().bam_attn_fwd(_dev(q, "q"), _dev(k, "k"), _dev(v, "v"), in_code, B, H, T, Dh, a, b_, m_, s_,
                            flags, _dev(o, "o"), oc, _dev(lse, "lse"), _ptr(ws),
                            ws.numel() * ws.element_size(), _stream(stream))
    _check(st, "bam_attn_fwd")
    return o, lse


def bam_attn_decode(q, k_cache, v_cache, kv_len, alpha, beta, mu=None, s=None, ssmax=True, o_dtype=None,
                    o=None, lse=None, workspace=None, stream=None, table_ready=False, prior_ref=False,
                 prior=None):
    """Decode; q [B, H, Dh], caches [B, H, Lmax, Dh], kv_len int32 [B].  Returns (o, lse)."""
    return _decode(q, k_cache, v_cache, kv_len, alpha, beta, mu, s, ssmax, o_dtype, o, lse, workspace, stream,
                   table_ready, prior_ref, prior, None)


def bam_attn_decode_skip(q, k_cache, v_cache, kv_len, alpha, beta, mu=None, s=None, key_norms=None, ssmax=True,
                         o_dtype=None, o=None, lse=None, workspace=None, stream=None, table_ready=False,
                         prior_ref=False, prior=None):
    """bam_attn_decode that leaves out the key ranges whose weights are zero in float32;
    key_norms [B, H, bam_decode_norm_pages(Lmax)] float32 from bam_decode_key_norms on the
    same cache.  Same results, bit for bit."""
    if key_norms is None:
        raise BamError("key_norms is required (bam_decode_key_norms of the cache)")
    return _decode(q, k_cache, v_cache, kv_len, alpha, beta, mu, s, ssmax, o_dtype, o, lse, workspace, stream,
                   table_ready, prior_ref, prior, key_norms)


def bam_decode_norm_pages(Lmax) -> int:
    return int(lib().bam_decode_norm_pages(Lmax))


def bam_decode_key_norms(k_cache, norms=None, stream=None):
    """Per-page (64 keys) maxima of the key norms of a cache [B, H, Lmax, Dh]: the float32
    array [B, H, bam_decode_norm_pages(Lmax)] that bam_attn_decode_skip reads."""
    torch = _torch()
    B, H, Lmax, Dh = _shape(k_cache, "k_cache", 4)
    npages = bam_decode_norm_pages(Lmax)
    dev = k_cache.device
    if norms is None:
        norms = torch.empty((B, H, npages), dtype=torch.float32, device=dev)
    else:
        _expect(norms, "norms", shape=(B, H, npages), dtypes=(torch.float32,), device=dev)
    st = lib().bam_decode_key_norms(_dev(k_cache, "k_cache"), _dtype_code(k_cache), B, H, Lmax, Dh,
                                    _dev(norms, "norms"), _stream(stream))
    _check(st, "bam_decode_key_norms")
    return norms


def bam_decode_partials_layout(B, H, Lmax, Dh):
    """(byte offset, nsplit, chunk) of the per-range partials a decode call leaves in its
    workspace: float32 records [B, H, nsplit, Dh + 2] = (m, l, o)."""
    off, ns, ch = ctypes.c_size_t(0), ctypes.c_int(0), ctypes.c_int(0)
    _check(lib().bam_decode_partials_layout(B, H, Lmax, Dh, ctypes.byref(off), ctypes.byref(ns), ctypes.byref(ch)),
           "bam_decode_partials_layout")
    return int(off.value), int(ns.value), int(ch.value)


def decode_skipped_fraction(workspace, kv_len, B, H, Lmax, Dh):
    """Fraction of the key ranges holding visible keys whose partial the last decode call on
    `workspace` left empty (m = -inf): for bam_attn_decode_skip, the ranges it skipped."""
    torch = _torch()
    off, ns, ch = bam_decode_partials_layout(B, H, Lmax, Dh)
    part = workspace[off:off + 4 * B * H * ns * (Dh + 2)].view(torch.float32).view(B, H, ns, Dh + 2)
    m = part[..., 0].cpu()
    L = kv_len.cpu().long().clamp(1, Lmax)
    live = (torch.arange(ns)[None, :] * ch < L[:, None])[:, None, :].expand(B, H, ns)
    empty = torch.isneginf(m) & live
    return float(empty.sum().item()) / float(live.sum().item())


def _decode(q, k_cache, v_cache, kv_len, alpha, beta, mu, s, ssmax, o_dtype, o, lse, workspace, stream, table_ready,
            prior_ref, prior, key_norms):
    torch = _torch()
    B, H, Lmax, Dh = _shape(k_cache, "k_cache", 4)
    flags = _flags(False, ssmax, prior_ref, prior) | (BAM_TABLE_READY if table_ready else 0)
    if table_ready and workspace is None:
        raise BamError("table_ready needs the workspace of an earlier call")
    in_code = _dtype_code(k_cache)
    dev = k_cache.device
    _expect(v_cache, "v_cache", shape=k_cache.shape, dtypes=(k_cache.dtype,), device=dev)
    _expect(q, "q", shape=(B, H, Dh), dtypes=(k_cache.dtype,), device=dev)
    _expect(kv_len, "kv_len", shape=(B,), dtypes=(torch.int32,), device=dev)
    io = (torch.bfloat16, torch.float32)
    oc = in_code if o_dtype is None else _dtype_code(torch.empty(0, dtype=o_dtype))
    if o is None:
        o = torch.empty((B, H, Dh), dtype=_torch_dtype(oc), device=dev)
    else:
        _expect(o, "o", shape=(B, H, Dh), dtypes=io, device=dev)
        oc = _dtype_code(o)
    if lse is None:
        lse = torch.empty((B, H), dtype=torch.float32, device=dev)
    else:
        _expect(lse, "lse", shape=(B, H), dtypes=(torch.float32,), device=dev)
    _check_params(alpha, beta, mu, s, flags, H, dev)
    nb = bam_decode_workspace_size(B, H, Lmax, Dh)
    ws = _workspace(nb, dev, workspace)
    a, b_, m_, s_ = _param_ptrs(alpha, beta, mu, s)
    if key_norms is None:
        st = lib().bam_attn_decode(_dev(q, "q"), _dev(k_cache, "k_cache"), _dev(v_cache, "v_cache"), in_code,
                                   _dev(kv_len, "kv_len"), B, H, Lmax, Dh, a, b_, m_, s_, flags, _dev(o, "o"), oc,
                                   _dev(lse, "lse"), _ptr(ws), ws.numel() * ws.element_size(), _stream(stream))
        _check(st, "bam_attn_decode")
    else:
        _expect(key_norms, "key_norms", shape=(B, H, bam_decode_norm_pages(Lmax)), dtypes=(torch.float32,),
                device=dev)
        st = lib().bam_attn_decode_skip(_dev(q, "q"), _dev(k_cache, "k_cache"), _dev(v_cache, "v_cache"), in_code,
                                        _dev(kv_len, "kv_len"), B, H, Lmax, Dh, a, b_, m_, s_, flags,
                                        _dev(key_norms, "key_norms"), _dev(o, "o"), oc, _dev(lse, "lse"), _ptr(ws),
                                        ws.numel() * ws.element_size(), _stream(stream))
        _check(st, "bam_attn_decode_skip")
    return o, lse


def bam_decode_static_max_bytes() -> int:
    return int(lib().bam_decode_static_max_bytes())


def bam_attn_decode_static(q, k_cache, v_cache, kv_len, alpha, beta, mu=None, s=None, ssmax=True, o=None,
                           lse=None, stream=None, table_ready=False, prior_ref=False, prior=None):
    """Decode with no workspace (the library's static device buffer): for callers that
    cannot allocate.  o [B, H, Dh] (bf16 or fp32) and lse [B, H] fp32 must be given, so the
    call itself allocates nothing.  Calls that overlap on one device race."""
    torch = _torch()
    B, H, Lmax, Dh = _shape(k_cache, "k_cache", 4)
    flags = _flags(False, ssmax, prior_ref, prior) | (BAM_TABLE_READY if table_ready else 0)
    in_code = _dtype_code(k_cache)
    dev = k_cache.device
    _expect(v_cache, "v_cache", shape=k_cache.shape, dtypes=(k_cache.dtype,), device=dev)
    _expect(q, "q", shape=(B, H, Dh), dtypes=(k_cache.dtype,), device=dev)
    _expect(kv_len, "kv_len", shape=(B,), dtypes=(torch.int32,), device=dev)
    _expect(o, "o", shape=(B, H, Dh), dtypes=(torch.bfloat16, torch.float32), device=dev)
    _expect(lse, "lse", shape=(B, H), dtypes=(torch.float32,), device=dev)
    _check_params(alpha, beta, mu, s, flags, H, dev)
    a, b_, m_, s_ = _param_ptrs(alpha, beta, mu, s)
    st = lib().bam_attn_decode_static(_dev(q, "q"), _dev(k_cache, "k_cache"), _dev(v_cache, "v_cache"), in_code,
                                      _dev(kv_len, "kv_len"), B, H, Lmax, Dh, a, b_, m_, s_, flags, _dev(o, "o"),
                                      _dtype_code(o), _dev(lse, "lse"), _stream(stream))
    _check(st, "bam_attn_decode_static")
    return o, lse


def bam_attn_decode_paged(q, k_pages, v_pages, block_table, kv_len, alpha, beta, mu=None, s=None, ssmax=True,
                          o_dtype=None, o=None, lse=None, workspace=None, stream=None, table_ready=False,
                          prior_ref=False, prior=None):
    """Decode on a paged cache: q [B, H, Dh]; k_pages, v_pages [num_pages, H, page_size, Dh];
    block_table int32 [B, max_blocks]; kv_len int32 [B].  Returns (o, lse)."""
    torch = _torch()
    num_pages, H, page_size, Dh = _shape(k_pages, "k_pages", 4)
    B, max_blocks = _shape(block_table, "block_table", 2)
    flags = _flags(False, ssmax, prior_ref, prior) | (BAM_TABLE_READY if table_ready else 0)
    if table_ready and workspace is None:
        raise BamError("table_ready needs the workspace of an earlier call")
    in_code = _dtype_code(k_pages)
    dev = k_pages.device
    _expect(v_pages, "v_pages", shape=k_pages.shape, dtypes=(k_pages.dtype,), device=dev)
    _expect(block_table, "block_table", dtypes=(torch.int32,), device=dev)
    _expect(q, "q", shape=(B, H, Dh), dtypes=(k_pages.dtype,), device=dev)
    _expect(kv_len, "kv_len", shape=(B,), dtypes=(torch.int32,), device=dev)
    io = (torch.bfloat16, torch.float32)
    oc = in_code if o_dtype is None else _dtype_code(torch.empty(0, dtype=o_dtype))
    if o is None:
        o = torch.empty((B, H, Dh), dtype=_torch_dtype(oc), device=dev)
    else:
        _expect(o, "o", shape=(B, H, Dh), dtypes=io, device=dev)
        oc = _dtype_code(o)
    if lse is None:
        lse = torch.empty((B, H), dtype=torch.float32, device=dev)
    else:
        _expect(lse, "lse", shape=(B, H), dtypes=(torch.float32,), device=dev)
    _check_params(alpha, beta, mu, s, flags, H, dev)
    nb = bam_decode_workspace_size(B, H, max_blocks * page_size, Dh)
    ws = _workspace(nb, dev, workspace)
    a, b_, m_, s_ = _param_ptrs(alpha, beta, mu, s)
    st = lib().bam_attn_decode_paged(_dev(q, "q"), _dev(k_pages, "k_pages"), _dev(v_pages, "v_pages"), in_code,
                                     _dev(block_table, "block_table"), max_blocks, num_pages, page_size,
                                     _dev(kv_len, "kv_len"), B, H, Dh, a, b_, m_, s_, flags, _dev(o, "o"), oc,
                                     _dev(lse, "lse"), _ptr(ws), ws.numel() * ws.element_size(), _stream(stream))
    _check(st, "bam_attn_decode_paged")
    return o, lse


def bam_attn_bwd(q, k, v, o, lse, dout, alpha, beta, mu=None, s=None, causal=True, ssmax=True,
                 grad_dtype=None, workspace=None, stream=None, prior_ref=False,
                 prior=None, skip_far=False):
    """Backward.  Returns (dq, dk, dv, dalpha, dbeta, ds).  skip_far: leave out the key /
    query tiles whose weights are zero in float32 (BAM_SKIP_FAR; causal only)."""
    return _bwd(q, k, v, o, lse, dout, alpha, beta, mu, s, causal, ssmax, grad_dtype, workspace, stream,
                prior_ref, False, prior, skip_far)


def bam_attn_bwd_ex(q, k, v, o, lse, dout, alpha, beta, mu=None, s=None, causal=True, ssmax=True,
                    grad_dtype=None, workspace=None, stream=None, prior_ref=False,
                    prior=None, skip_far=False):
    """Backward with the offset gradient.  Returns (dq, dk, dv, dalpha, dbeta, dmu, ds)."""
    return _bwd(q, k, v, o, lse, dout, alpha, beta, mu, s, causal, ssmax, grad_dtype, workspace, stream,
                prior_ref, True, prior, skip_far)


def _bwd(q, k, v, o, lse, dout, alpha, beta, mu, s, causal, ssmax, grad_dtype, workspace, stream, prior_ref,
         want_mu, prior=None, skip_far=False):
    torch = _torch()
    B, H, T, Dh = _shape(q, "q", 4)
    flags = _flags(causal, ssmax, prior_ref, prior) | (BAM_SKIP_FAR if skip_far else 0)
    in_code = _dtype_code(q)
    dev = q.device
    for name, t in (("k", k), ("v", v), ("dout", dout)):
        _expect(t, name, shape=q.shape, dtypes=(q.dtype,), device=dev)
    _expect(o, "o", shape=q.shape, dtypes=(torch.bfloat16, torch.float32), device=dev)
    _expect(lse, "lse", shape=(B, H, T), dtypes=(torch.float32,), device=dev)
    gc = in_code if grad_dtype is None else _dtype_code(torch.empty(0, dtype=grad_dtype))
    gdt = _torch_dtype(gc)
    _check_params(alpha, beta, mu, s, flags, H, dev)
    ws = _workspace(bam_bwd_workspace_size(B, H, T, Dh, flags), dev, workspace)
    a, b_, m_, s_ = _param_ptrs(alpha, beta, mu, s)
    dq = torch.empty_like(q, dtype=gdt)
    dk = torch.empty_like(q, dtype=gdt)
    dv = torch.empty_like(q, dtype=gdt)
    dalpha = torch.empty(H, dtype=torch.float32, device=dev)
    dbeta = torch.empty_like(dalpha)
    dmu = torch.empty_like(dalpha) if want_mu else None
    ds = torch.empty_like(dalpha)
    head = (_dev(q, "q"), _dev(k, "k"), _dev(v, "v"), _dev(o, "o"), _dtype_code(o), _dev(lse, "lse"),
            _dev(dout, "dout"), in_code, B, H, T, Dh, a, b_, m_, s_, flags, _dev(dq, "dq"), _dev(dk, "dk"),
            _dev(dv, "dv"), gc, _dev(dalpha, "dalpha"), _dev(dbeta, "dbeta"))
    tail = (_dev(ds, "ds"), _ptr(ws), ws.numel() * ws.element_size(), _stream(stream))
    if want_mu:
        st = lib().bam_attn_bwd_ex(*head, _dev(dmu, "dmu"), *tail)
        _check(st, "bam_attn_bwd_ex")
        return dq, dk, dv, dalpha, dbeta, dmu, ds
    st = lib().bam_attn_bwd(*head, *tail)
    _check(st, "bam_attn_bwd")
    return dq, dk, dv, dalpha, dbeta, ds
