"""C-ABI library: it loads, exports every symbol include/bam.h declares, and the host-side
argument checks reject bad calls before anything touches the GPU.  No compute calls."""
import ctypes
import os
import re

import pytest

import positional_prior_bias_amd as bam

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "bam.h")


def declared_functions():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(bam_[a-z_0-9]+)\s*\(", src)))


@pytest.fixture(scope="module")
def L():
    if not os.path.exists(bam.lib_path()):
        pytest.fail("libbam.so is not built (run __graft_entry__.build())")
    return bam.lib()


def test_header_declares_the_entry_points():
    names = declared_functions()
    for n in ("bam_attn_fwd", "bam_attn_decode", "bam_attn_bwd", "bam_prior_table"):
        assert n in names
    assert set(names) == set(bam.EXPORTED_SYMBOLS)


def test_library_exports_every_declared_symbol(L):
    raw = ctypes.CDLL(bam.lib_path())
    for n in declared_functions():
        assert hasattr(raw, n), f"libbam.so does not export {n}"


def test_status_strings(L):
    assert L.bam_status_string(0) == b"ok"
    assert L.bam_status_string(3) == b"workspace too small"
    assert L.bam_version() >= 100


def test_workspace_sizes(L):
    # distance table only: H rows of T (causal) or 2T-1 distances, padded by 704 entries on
    # each side, rounded up to 64 entries; 256-byte aligned
    pad64 = lambda n: (n + 63) // 64 * 64  # noqa: E731
    assert L.bam_fwd_workspace_size(32, 12, 512, 64, 3) == 12 * pad64(512 + 2 * 704) * 4
    assert L.bam_fwd_workspace_size(1, 4, 256, 32, 0) == 4 * pad64(511 + 2 * 704) * 4
    assert L.bam_fwd_workspace_size(1, 0, 256, 32, 1) == 0
    assert L.bam_decode_workspace_size(8, 12, 256000, 64) > 12 * 256000 * 4
    assert L.bam_decode_workspace_size(8, 12, 256000, 48) == 0
    assert L.bam_bwd_workspace_size(32, 12, 512, 64, 3) >= 3 * 12 * 512 * 4 + 32 * 12 * 512 * 4


def _fwd(L, **kw):
    a = dict(q=16, k=16, v=16, in_dtype=0, B=1, H=1, T=8, Dh=64, alpha=16, beta=16, mu=None, s=16,
             flags=3, o=16, o_dtype=1, lse=16, ws=256, wsb=1 << 20, stream=None)
    a.update(kw)
    return L.bam_attn_fwd(a["q"], a["k"], a["v"], a["in_dtype"], a["B"], a["H"], a["T"], a["Dh"],
                          a["alpha"], a["beta"], a["mu"], a["s"], a["flags"], a["o"], a["o_dtype"],
                          a["lse"], a["ws"], a["wsb"], a["stream"])


def _no_gpu():
    try:
        import torch
        return not torch.cuda.is_available()
    except Exception:
        return True


# The calls below pass fake device addresses (small integers) that must be rejected by the
# host-side checks before any launch; they run only where no GPU is visible, so a
# regression in those checks can never launch a kernel on them.
host_only = pytest.mark.skipif(not _no_gpu(), reason="fake-pointer host checks run only without a GPU")


@host_only
def test_fwd_rejects_bad_arguments_before_launch(L):
    assert _fwd(L, q=None) == 1
    assert _fwd(L, q=8) == 1                      # misaligned
    assert _fwd(L, T=0) == 1
    assert _fwd(L, flags=64) == 1                 # unknown flag bit
    assert _fwd(L, T=1 << 24, Dh=64) == 2         # one (b, h) slab beyond 32-bit offsets
    assert _fwd(L, flags=2 | 32) == 2             # skipping needs the causal bf16 path
    assert _fwd(L, flags=3 | 8 | 16) == 1         # two prior kinds at once
    assert _fwd(L, s=None) == 1                   # SSMax without s
    assert _fwd(L, Dh=48) == 2
    assert _fwd(L, in_dtype=7) == 2
    assert _fwd(L, in_dtype=1, Dh=128) == 2
    assert _fwd(L, o_dtype=5) == 2
    assert _fwd(L, wsb=16) == 3


@host_only
def test_decode_and_bwd_reject_bad_arguments(L):
    st = L.bam_attn_decode(16, 16, 16, 0, None, 1, 1, 8, 64, 16, 16, None, 16, 2, 16, 1, 16, 256, 1 << 20, None)
    assert st == 1                                 # kv_len NULL
    st = L.bam_attn_decode(16, 16, 16, 1, 16, 1, 1, 8, 64, 16, 16, None, 16, 2, 16, 1, 16, 256, 1 << 20, None)
    assert st == 2                                 # fp32 caches unsupported
    st = L.bam_attn_decode(16, 16, 16, 0, 16, 8, 12, 256000, 64, 16, 16, None, 16, 2, 16, 1, 16, 256, 1024, None)
    assert st == 3
    st = L.bam_attn_bwd(16, 16, 16, 16, 1, 16, 16, 0, 1, 1, 8, 128, 16, 16, None, 16, 3, 16, 16, 16, 0,
                        16, 16, 16, 256, 1 << 20, None)
    assert st == 2                                 # Dh = 128 backward unsupported
    st = L.bam_attn_bwd(16, 16, 16, 16, 1, 16, 16, 0, 1, 1, 8, 64, 16, 16, None, 16, 3, 16, 16, 16, 0,
                        None, 16, 16, 256, 1 << 20, None)
    assert st == 1                                 # dalpha NULL
    st = L.bam_attn_bwd(16, 16, 16, 16, 1, 16, 16, 0, 1, 1, 1 << 24, 64, 16, 16, None, 16, 3, 16, 16, 16, 0,
                        16, 16, 16, 256, 1 << 20, None)
    assert st == 2                                 # one head's Q beyond a 32-bit byte range
    st = L.bam_attn_bwd(16, 16, 16, 16, 1, 16, 16, 0, 1 << 21, 1, 64, 64, 16, 16, None, 16, 3, 16, 16, 16, 0,
                        16, 16, 16, 256, 1 << 20, None)
    assert st == 2                                 # per-row scalars beyond a 32-bit byte range
    assert L.bam_prior_table(None, 16, None, 1, 0, 8, 16, None, None, None) == 1
    st = L.bam_attn_bwd_ex(16, 16, 16, 16, 1, 16, 16, 0, 1, 1, 8, 64, 16, 16, None, 16, 3 | 8, 16, 16, 16, 0,
                           None, 16, 16, 16, 256, 1 << 20, None)
    assert st == 1                                 # dalpha NULL (extended backward)
    st = L.bam_attn_bwd_ex(16, 16, 16, 16, 1, 16, 16, 0, 1, 1, 8, 64, 16, 16, None, 16, 64 | 3, 16, 16, 16, 0,
                           16, 16, 16, 16, 256, 1 << 20, None)
    assert st == 1                                 # unknown flag bit
    assert L.bam_prior_table_ex(16, 16, None, 1, 0, 8, 1, 16, None, None, None, None) == 1   # only prior flags
    assert L.bam_prior_table_ex(16, 16, None, 1, 0, 8, 8 | 16, 16, None, None, None, None) == 1  # two kinds
    pg = L.bam_attn_decode_paged
    assert pg(16, 16, 16, 0, 16, 4, 8, 96, 16, 1, 1, 64, 16, 16, None, 16, 2, 16, 1, 16, 256, 1 << 20, None) == 2
    assert pg(16, 16, 16, 0, None, 4, 8, 64, 16, 1, 1, 64, 16, 16, None, 16, 2, 16, 1, 16, 256, 1 << 20, None) == 1
    assert pg(16, 16, 16, 0, 16, 0, 8, 64, 16, 1, 1, 64, 16, 16, None, 16, 2, 16, 1, 16, 256, 1 << 20, None) == 1


def test_static_decode_host_checks(L):
    """bam_attn_decode_static rejects bad sizes and requests beyond its static buffer before
    touching the device: these calls pass null pointers and never reach a launch."""
    null = None
    args = lambda B, H, Lmax, Dh: (null, null, null, 0, null, B, H, Lmax, Dh, null, null, null, null, 2,  # noqa: E731
                                   null, 1, null, null)
    assert L.bam_decode_static_max_bytes() == 32 << 20
    assert L.bam_attn_decode_static(*args(0, 12, 1000, 64)) == 1          # BAM_EINVAL
    assert L.bam_attn_decode_static(*args(1, 12, 1000, 48)) == 2          # BAM_EUNSUPPORTED
    assert L.bam_decode_workspace_size(64, 64, 1 << 20, 128) > L.bam_decode_static_max_bytes()
    assert L.bam_attn_decode_static(*args(64, 64, 1 << 20, 128)) == 5     # BAM_ETOOLARGE
    assert L.bam_status_string(5).startswith(b"problem exceeds")
