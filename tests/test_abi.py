"""The C ABI: the library loads, exports what include/fa.h declares, and rejects bad
arguments with the documented status before touching the GPU (CPU only)."""
import ctypes
import math
import os
import re

import pytest

import io_aware_exact_fa_amd as fa

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADERS = [os.path.join(ROOT, "include", f) for f in sorted(os.listdir(os.path.join(ROOT, "include")))
           if f.endswith(".h")]

# Valid-looking (non-null) pointers: argument checks must fail before any of them is used.
P = 0x1000


def declared_functions():
    names = []
    for path in HEADERS:
        text = re.sub(r"/\*.*?\*/", "", open(path).read(), flags=re.S)
        names += re.findall(r"^\s*(?:const\s+)?[A-Za-z_][A-Za-z0-9_\s\*]*?\b(fa_[a-z0-9_]+)\s*\(",
                            text, flags=re.M)
    return sorted(set(names))


def test_header_declares_the_entry_points():
    assert declared_functions() == sorted(fa.EXPORTED)


def test_library_exports_every_declared_symbol():
    lib = ctypes.CDLL(fa.LIB_PATH)
    for name in declared_functions():
        assert hasattr(lib, name), name


def test_abi_version_and_status_strings():
    assert fa.fa_abi_version() == 9
    for st in range(6):
        assert fa.fa_status_string(st) and fa.fa_status_string(st) != "unknown status"
    assert fa.fa_status_string(99) == "unknown status"


def _fwd(**kw):
    args = dict(q=P, k=P, v=P, o=P, lse=P, B=1, H=1, N=128, d=64, causal=0, scale=0.125,
                dtype=fa.FA_BF16, stream=None)
    args.update(kw)
    return fa.fa_fwd(**args)


def _bwd(**kw):
    args = dict(q=P, k=P, v=P, o=P, dout=P, lse=P, dq=P, dk=P, dv=P, B=1, H=1, N=128, d=64,
                causal=0, scale=0.125, dtype=fa.FA_BF16, workspace=0x10000,
                workspace_bytes=fa.fa_bwd_workspace_size(1, 1, 128, 64), stream=None)
    args.update(kw)
    return fa.fa_bwd(**args)


@pytest.mark.parametrize("name", ["q", "k", "v", "o", "lse"])
def test_fwd_null_pointer(name):
    assert _fwd(**{name: None}) == fa.FA_ERR_INVALID_ARGUMENT


@pytest.mark.parametrize("kw,status", [
    (dict(B=0), fa.FA_ERR_INVALID_ARGUMENT),
    (dict(H=-1), fa.FA_ERR_INVALID_ARGUMENT),
    (dict(N=0), fa.FA_ERR_INVALID_ARGUMENT),
    (dict(d=0), fa.FA_ERR_INVALID_ARGUMENT),
    (dict(scale=math.nan), fa.FA_ERR_INVALID_ARGUMENT),
    (dict(scale=math.inf), fa.FA_ERR_INVALID_ARGUMENT),
    (dict(B=2**20, H=2**20, N=2**20, d=64), fa.FA_ERR_INVALID_ARGUMENT),   # > 2^62 elements
    (dict(d=96), fa.FA_ERR_UNSUPPORTED),
    (dict(d=32), fa.FA_ERR_UNSUPPORTED),
    (dict(dtype=3), fa.FA_ERR_UNSUPPORTED),
    (dict(dtype=-1), fa.FA_ERR_UNSUPPORTED),
    (dict(H=70000), fa.FA_ERR_UNSUPPORTED),
    (dict(N=2**23 + 1), fa.FA_ERR_UNSUPPORTED),
])
def test_fwd_rejects(kw, status):
    assert _fwd(**kw) == status


@pytest.mark.parametrize("name", ["q", "k", "v", "o", "dout", "lse", "dq", "dk", "dv"])
def test_bwd_null_pointer(name):
    assert _bwd(**{name: None}) == fa.FA_ERR_INVALID_ARGUMENT


@pytest.mark.parametrize("kw,status", [
    (dict(N=-5), fa.FA_ERR_INVALID_ARGUMENT),
    (dict(scale=math.nan), fa.FA_ERR_INVALID_ARGUMENT),
    (dict(d=80), fa.FA_ERR_UNSUPPORTED),
    (dict(dtype=9), fa.FA_ERR_UNSUPPORTED),
    (dict(workspace=None), fa.FA_ERR_WORKSPACE),
    (dict(workspace_bytes=100), fa.FA_ERR_WORKSPACE),
    (dict(workspace=0x10000 + 64), fa.FA_ERR_WORKSPACE),   # not 256-byte aligned
])
def test_bwd_rejects(kw, status):
    assert _bwd(**kw) == status


def test_split_backward_rejects():
    ws, nb = 0x10000, fa.fa_bwd_workspace_size(1, 1, 128, 64)
    assert fa.fa_bwd_preprocess(None, P, P, 1, 1, 128, 64, fa.FA_F16, ws, nb, None) == fa.FA_ERR_INVALID_ARGUMENT
    assert fa.fa_bwd_preprocess(P, P, None, 1, 1, 128, 64, fa.FA_F16, ws, nb, None) == fa.FA_ERR_INVALID_ARGUMENT
    assert fa.fa_bwd_preprocess(P, P, P, 1, 1, 128, 96, fa.FA_F16, ws, nb, None) == fa.FA_ERR_UNSUPPORTED
    assert fa.fa_bwd_preprocess(P, P, P, 1, 1, 128, 64, fa.FA_F16, ws, nb - 1, None) == fa.FA_ERR_WORKSPACE
    assert fa.fa_bwd_dkdv(P, P, P, P, P, P, None, 1, 1, 128, 64, 0, 0.1, fa.FA_F16, ws, nb,
                          None) == fa.FA_ERR_INVALID_ARGUMENT
    assert fa.fa_bwd_dkdv(P, P, P, P, P, P, P, 1, 1, 128, 64, 0, math.nan, fa.FA_F16, ws, nb,
                          None) == fa.FA_ERR_INVALID_ARGUMENT
    assert fa.fa_bwd_dkdv(P, P, P, P, P, P, P, 1, 1, 128, 64, 0, 0.1, fa.FA_F16, ws + 8, nb,
                          None) == fa.FA_ERR_WORKSPACE
    assert fa.fa_bwd_dq(P, P, P, P, P, None, 1, 1, 128, 64, 0, 0.1, fa.FA_F16, ws, nb,
                        None) == fa.FA_ERR_INVALID_ARGUMENT
    assert fa.fa_bwd_dq(P, P, P, P, P, P, 1, 1, 128, 64, 0, 0.1, 5, ws, nb, None) == fa.FA_ERR_UNSUPPORTED
    assert fa.fa_bwd_dq(P, P, P, P, P, P, 1, 1, 128, 64, 0, 0.1, fa.FA_F16, ws, nb - 1,
                        None) == fa.FA_ERR_WORKSPACE


def test_grouped_kv_rejects():
    ws, nb = 0x10000, fa.fa_bwd_workspace_size(1, 8, 128, 64)
    fwd = lambda H, H_kv: fa.fa_fwd_gqa(P, P, P, P, P, 1, H, H_kv, 128, 64, 0, 0.1, fa.FA_F16, None)
    for H, H_kv in ((8, 0), (8, -2), (8, 3), (8, 16), (6, 4)):
        assert fwd(H, H_kv) == fa.FA_ERR_INVALID_ARGUMENT, (H, H_kv)
        assert fa.fa_bwd_gqa(P, P, P, P, P, P, P, P, P, 1, H, H_kv, 128, 64, 0, 0.1, fa.FA_F16,
                             ws, nb, None) == fa.FA_ERR_INVALID_ARGUMENT
        assert fa.fa_bwd_dkdv_gqa(P, P, P, P, P, P, P, 1, H, H_kv, 128, 64, 0, 0.1, fa.FA_F16,
                                  ws, nb, None) == fa.FA_ERR_INVALID_ARGUMENT
        assert fa.fa_bwd_dq_gqa(P, P, P, P, P, P, 1, H, H_kv, 128, 64, 0, 0.1, fa.FA_F16,
                                ws, nb, None) == fa.FA_ERR_INVALID_ARGUMENT
    # The other checks are those of the plain entry points.
    assert fa.fa_fwd_gqa(P, None, P, P, P, 1, 8, 2, 128, 64, 0, 0.1, fa.FA_F16, None) == fa.FA_ERR_INVALID_ARGUMENT
    assert fa.fa_fwd_gqa(P, P, P, P, P, 1, 8, 2, 128, 96, 0, 0.1, fa.FA_F16, None) == fa.FA_ERR_UNSUPPORTED
    assert fa.fa_bwd_gqa(P, P, P, P, P, P, P, P, P, 1, 8, 2, 128, 64, 0, 0.1, fa.FA_F16,
                         ws, nb - 1, None) == fa.FA_ERR_WORKSPACE


def _fwd_varlen(**kw):
    args = dict(q=P, k=P, v=P, o=P, lse=P, cu_seqlens=P, B=3, max_s=128, total=300, H=8, H_kv=2,
                d=64, causal=0, scale=0.125, dtype=fa.FA_BF16, stream=None)
    args.update(kw)
    return fa.fa_fwd_varlen(**args)


def _bwd_varlen(**kw):
    args = dict(q=P, k=P, v=P, o=P, dout=P, lse=P, dq=P, dk=P, dv=P, cu_seqlens=P, B=3, max_s=128,
                total=300, H=8, H_kv=2, d=64, causal=0, scale=0.125, dtype=fa.FA_BF16,
                workspace=0x10000, workspace_bytes=fa.fa_bwd_workspace_size(3, 8, 128, 64),
                stream=None)
    args.update(kw)
    return fa.fa_bwd_varlen(**args)


def test_varlen_rejects():
    E = fa.FA_ERR_INVALID_ARGUMENT
    for call in (_fwd_varlen, _bwd_varlen):
        assert call(cu_seqlens=None) == E
        assert call(q=None) == E
        assert call(total=0) == E and call(total=-5) == E
        assert call(B=0) == E and call(max_s=0) == E
        assert call(H_kv=3) == E and call(H_kv=0) == E
        assert call(scale=math.inf) == E
        assert call(d=96) == fa.FA_ERR_UNSUPPORTED
        assert call(dtype=7) == fa.FA_ERR_UNSUPPORTED
        assert call(max_s=2**23 + 1) == fa.FA_ERR_UNSUPPORTED
        assert call(B=65536) == fa.FA_ERR_UNSUPPORTED
    assert _bwd_varlen(workspace_bytes=fa.fa_bwd_workspace_size(3, 8, 128, 64) - 1) == fa.FA_ERR_WORKSPACE
    assert _bwd_varlen(workspace=0x10008) == fa.FA_ERR_WORKSPACE
    assert _bwd_varlen(dk=None) == E


def test_attn_struct_layout():
    """ctypes mirror of struct fa_attn: natural alignment on x86-64 (the pointer at
    byte 40, the seed at 56, the block mask at 72, the whole 88 bytes)."""
    assert ctypes.sizeof(fa.FaAttn) == 88
    assert fa.FaAttn.cu_seqlens.offset == 40 and fa.FaAttn.total.offset == 48
    assert fa.FaAttn.dropout_p.offset == 52 and fa.FaAttn.seed.offset == 56
    assert fa.FaAttn.rng_offset.offset == 64 and fa.FaAttn.block_mask.offset == 72
    assert fa.FaAttn.block_mask_heads.offset == 80
    assert fa.FaAttn.window_left.offset == 24 and fa.FaAttn.scale.offset == 32


def test_ex_rejects():
    E = fa.FA_ERR_INVALID_ARGUMENT
    good = dict(B=1, H=8, H_kv=2, N=128, d=64, causal=1, scale=0.1, dtype=fa.FA_F16)
    ws, nb = 0x10000, fa.fa_bwd_workspace_size(1, 8, 128, 64)
    fwd = lambda p: fa.fa_fwd_ex(p, P, P, P, P, P, None)
    bwd = lambda p, nb=nb: fa.fa_bwd_ex(p, P, P, P, P, P, P, P, P, P, ws, nb, None)
    assert fwd(None) == E and bwd(None) == E
    for window in ((-2, -1), (-1, -7)):
        assert fwd(fa.attn(**good, window=window)) == E
        assert bwd(fa.attn(**good, window=window)) == E
    assert fwd(fa.attn(**{**good, "H_kv": 3})) == E
    for heads in (0, 3, 9):   # a mask needs 1 or H (= 8) heads
        assert fwd(fa.attn(**good, block_mask=P, block_mask_heads=heads)) == E
    for pd in (-0.1, 1.5, float("nan")):
        assert fwd(fa.attn(**good, dropout=(pd, 1, 0))) == E
        assert bwd(fa.attn(**good, dropout=(pd, 1, 0))) == E
    assert fwd(fa.attn(**{**good, "d": 96})) == fa.FA_ERR_UNSUPPORTED
    assert bwd(fa.attn(**good), nb - 1) == fa.FA_ERR_WORKSPACE
    # Packed batch through the description: total must be positive.
    assert fwd(fa.attn(**good, cu_seqlens=P, total=0)) == E
    assert fa.fa_fwd_ex(fa.attn(**good), P, None, P, P, P, None) == E


def test_too_many_heads_rejected():
    """B*H above 2^24 would overflow the tile grids' 32-bit work index."""
    assert _fwd(B=65535, H=257, N=1) == fa.FA_ERR_UNSUPPORTED
    assert _fwd(B=4097, H=4096, N=1) == fa.FA_ERR_UNSUPPORTED


def _up(x):
    return (x + 255) // 256 * 256


def _stats_bytes(B, H, N):
    """The D and L2 part of the workspace: two float32 arrays [B, H, Np]."""
    return _up(2 * 4 * B * H * ((N + 63) // 64 * 64))


def _one_pass_bytes(B, H, N, d):
    """Workspace of the one-pass steps: D and L2, then the float32 dQ accumulator."""
    return _stats_bytes(B, H, N) + 4 * B * H * ((N + 63) // 64 * 64) * d


def test_workspace_size():
    # Two float32 arrays [B, H, Np], Np = N rounded up to a multiple of 64.
    for B, H, N, d in ((2, 3, 100, 64), (1, 1, 64, 128), (1, 1, 65, 128), (4, 32, 4096, 128)):
        assert fa.fa_bwd_workspace_size(B, H, N, d) == _stats_bytes(B, H, N)
    assert fa.fa_bwd_workspace_size(0, 1, 1, 64) == 0
    assert fa.fa_bwd_workspace_size(1, 1, -3, 64) == 0


def _has_gpu():
    import torch
    return torch.cuda.device_count() > 0


@pytest.mark.skipif(_has_gpu(), reason="would launch kernels on the bogus pointers")
def test_valid_arguments_without_gpu_report_device_error():
    assert _fwd() == fa.FA_ERR_DEVICE
    assert _bwd() == fa.FA_ERR_DEVICE
    ws, nb = 0x10000, fa.fa_bwd_workspace_size(1, 8, 128, 64)
    assert fa.fa_fwd_gqa(P, P, P, P, P, 1, 8, 2, 128, 64, 0, 0.1, fa.FA_F16, None) == fa.FA_ERR_DEVICE
    assert fa.fa_bwd_gqa(P, P, P, P, P, P, P, P, P, 1, 8, 2, 128, 64, 0, 0.1, fa.FA_F16,
                         ws, nb, None) == fa.FA_ERR_DEVICE
    assert _fwd_varlen() == fa.FA_ERR_DEVICE
    assert _bwd_varlen() == fa.FA_ERR_DEVICE
    p = fa.attn(1, 8, 2, 128, 64, 1, 0.1, fa.FA_F16, window=(16, 0))
    assert fa.fa_fwd_ex(p, P, P, P, P, P, None) == fa.FA_ERR_DEVICE
    # Dropout together with a block mask is a valid description.
    pdm = fa.attn(1, 8, 2, 128, 64, 1, 0.1, fa.FA_F16, dropout=(0.25, 1, 0), block_mask=P)
    assert fa.fa_fwd_ex(pdm, P, P, P, P, P, None) == fa.FA_ERR_DEVICE
    assert fa.fa_bwd_ex(pdm, P, P, P, P, P, P, P, P, P, 0x10000,
                        fa.fa_bwd_workspace_size(1, 8, 128, 64), None) == fa.FA_ERR_DEVICE
    assert fa.fa_bwd_ex(p, P, P, P, P, P, P, P, P, P, 0x10000,
                        fa.fa_bwd_workspace_size(1, 8, 128, 64), None) == fa.FA_ERR_DEVICE
    nb = fa.fa_bwd_workspace_size(1, 1, 128, 64)
    assert fa.fa_bwd_preprocess(P, P, P, 1, 1, 128, 64, fa.FA_F16, 0x10000, nb, None) == fa.FA_ERR_DEVICE
    assert fa.fa_bwd_dq(P, P, P, P, P, P, 1, 1, 128, 64, 0, 0.1, fa.FA_F16, 0x10000, nb,
                        None) == fa.FA_ERR_DEVICE


def test_binding_refuses_missing_library(tmp_path, monkeypatch):
    """The binding raises on import when libfa.so is absent; it never falls back."""
    import importlib.util
    import shutil
    pkg = tmp_path / "io_aware_exact_fa_amd"
    pkg.mkdir()
    shutil.copy(os.path.join(ROOT, "io_aware_exact_fa_amd", "__init__.py"), pkg / "__init__.py")
    spec = importlib.util.spec_from_file_location("fa_copy", pkg / "__init__.py")
    mod = importlib.util.module_from_spec(spec)
    with pytest.raises(ImportError):
        spec.loader.exec_module(mod)


@pytest.mark.parametrize("name", ["q", "k", "v", "o"])
def test_fwd_rejects_misaligned_tensor(name):
    """fa.h: tensors are 16-byte aligned (16-byte loads, LDS-direct copies)."""
    for off in (2, 8):
        assert _fwd(**{name: P + off}) == fa.FA_ERR_INVALID_ARGUMENT
    assert fa.fa_fwd_ex(fa.attn(1, 1, 1, 128, 64, 0, 0.125, fa.FA_BF16),
                        *[P + 8 if n == name else P for n in ("q", "k", "v", "o", "lse")],
                        None) == fa.FA_ERR_INVALID_ARGUMENT


@pytest.mark.parametrize("name", ["q", "k", "v", "o", "dout", "dq", "dk", "dv"])
def test_bwd_rejects_misaligned_tensor(name):
    assert _bwd(**{name: P + 4}) == fa.FA_ERR_INVALID_ARGUMENT
    assert _bwd_varlen(**{name: P + 8}) == fa.FA_ERR_INVALID_ARGUMENT


def test_misaligned_statistics_and_offsets_rejected():
    """lse (float32) and cu_seqlens (int32) need 4-byte alignment; the split
    backward entry points check their tensors too."""
    assert _fwd(lse=P + 2) == fa.FA_ERR_INVALID_ARGUMENT
    assert _bwd(lse=P + 1) == fa.FA_ERR_INVALID_ARGUMENT
    assert _fwd_varlen(cu_seqlens=P + 2) == fa.FA_ERR_INVALID_ARGUMENT
    assert _bwd_varlen(cu_seqlens=P + 1) == fa.FA_ERR_INVALID_ARGUMENT
    ws, nb = 0x10000, fa.fa_bwd_workspace_size(1, 1, 128, 64)
    assert fa.fa_bwd_preprocess(P + 8, P, P, 1, 1, 128, 64, fa.FA_F16, ws, nb, None) == fa.FA_ERR_INVALID_ARGUMENT
    assert fa.fa_bwd_dkdv(P, P, P, P, P, P + 8, P, 1, 1, 128, 64, 0, 0.1, fa.FA_F16, ws, nb,
                          None) == fa.FA_ERR_INVALID_ARGUMENT
    assert fa.fa_bwd_dq(P, P + 8, P, P, P, P, 1, 1, 128, 64, 0, 0.1, fa.FA_F16, ws, nb,
                        None) == fa.FA_ERR_INVALID_ARGUMENT
    p = fa.attn(3, 8, 2, 128, 64, 0, 0.1, fa.FA_F16, cu_seqlens=P + 2, total=300)
    assert fa.fa_fwd_ex(p, P, P, P, P, P, None) == fa.FA_ERR_INVALID_ARGUMENT


def test_binding_rejects_misaligned_view():
    """A contiguous view at an odd element offset passes the shape checks but not
    the alignment check, before any launch (CPU tensors are refused earlier)."""
    import torch

    class FakeCuda:
        shape, dtype, is_cuda = (1, 1, 8, 64), torch.bfloat16, True

        def is_contiguous(self):
            return True

        def data_ptr(self):
            return 0x10002

    with pytest.raises(ValueError, match="not 16-byte aligned"):
        fa._check("q", FakeCuda(), (1, 1, 8, 64), torch.bfloat16)


def _bwd_noalloc(**kw):
    args = dict(q=P, k=P, v=P, o=P, dout=P, lse=P, dq=P, dk=P, dv=P, B=1, H=1, N=128, d=64,
                causal=0, scale=0.125, dtype=fa.FA_BF16, stream=None)
    args.update(kw)
    return fa.fa_bwd_noalloc(**args)


def test_noalloc_rejects():
    """The allocation-free backward checks what fa_bwd checks, and refuses shapes
    whose D and L2 do not fit its static array (B*H*Np > 4 Mi rows)."""
    E = fa.FA_ERR_INVALID_ARGUMENT
    for name in ("q", "k", "v", "o", "dout", "lse", "dq", "dk", "dv"):
        assert _bwd_noalloc(**{name: None}) == E
    assert _bwd_noalloc(dq=P + 8) == E and _bwd_noalloc(lse=P + 2) == E
    assert _bwd_noalloc(N=0) == E and _bwd_noalloc(scale=math.nan) == E
    assert _bwd_noalloc(d=96) == fa.FA_ERR_UNSUPPORTED
    rows = fa.FA_NOALLOC_SCRATCH_BYTES // 8            # D and L2, 4 bytes each per row
    assert _stats_bytes(1, 64, rows // 64) <= fa.FA_NOALLOC_SCRATCH_BYTES
    assert _stats_bytes(1, 64, rows // 64 + 64) > fa.FA_NOALLOC_SCRATCH_BYTES
    assert _bwd_noalloc(B=1, H=64, N=rows // 64 + 64, d=128) == fa.FA_ERR_WORKSPACE
    assert _bwd_noalloc(B=2, H=32, N=131072, d=128) == fa.FA_ERR_WORKSPACE


def test_noalloc_scratch_size_matches_header():
    text = open(os.path.join(ROOT, "include", "fa.h")).read()
    m = re.search(r"#define FA_NOALLOC_SCRATCH_BYTES \((\d+)u << (\d+)\)", text)
    assert m and int(m[1]) << int(m[2]) == fa.FA_NOALLOC_SCRATCH_BYTES


@pytest.mark.skipif(_has_gpu(), reason="would launch kernels on the bogus pointers")
def test_noalloc_valid_arguments_without_gpu_report_device_error():
    assert _bwd_noalloc() == fa.FA_ERR_DEVICE


def _dkdv_dq(**kw):
    args = dict(q=P, k=P, v=P, dout=P, lse=P, dk=P, dv=P, B=1, H=8, H_kv=2, N=128, d=64, causal=1,
                scale=0.125, dtype=fa.FA_BF16, workspace=0x10000,
                workspace_bytes=_one_pass_bytes(1, 8, 128, 64), stream=None)
    args.update(kw)
    return fa.fa_bwd_dkdv_dq(**args)


def _dq_fin(**kw):
    args = dict(dq=P, B=1, H=8, N=128, d=64, scale=0.125, dtype=fa.FA_BF16, workspace=0x10000,
                workspace_bytes=_one_pass_bytes(1, 8, 128, 64), stream=None)
    args.update(kw)
    return fa.fa_bwd_dq_finalize(**args)


def test_one_pass_steps_reject():
    """fa_bwd_dkdv_dq and fa_bwd_dq_finalize: the usual checks, 16-bit types only,
    and a workspace that also holds the accumulator."""
    E = fa.FA_ERR_INVALID_ARGUMENT
    for name in ("q", "k", "v", "dout", "lse", "dk", "dv"):
        assert _dkdv_dq(**{name: None}) == E
    assert _dkdv_dq(dk=P + 8) == E and _dq_fin(dq=None) == E and _dq_fin(dq=P + 4) == E
    assert _dkdv_dq(H_kv=3) == E and _dkdv_dq(N=0) == E and _dq_fin(scale=math.inf) == E
    assert _dkdv_dq(dtype=fa.FA_F32) == fa.FA_ERR_UNSUPPORTED
    assert _dq_fin(dtype=fa.FA_F32) == fa.FA_ERR_UNSUPPORTED
    assert _dkdv_dq(d=96) == fa.FA_ERR_UNSUPPORTED and _dq_fin(d=96) == fa.FA_ERR_UNSUPPORTED
    full = _one_pass_bytes(1, 8, 128, 64)
    assert _dkdv_dq(workspace_bytes=full - 1) == fa.FA_ERR_WORKSPACE
    assert _dq_fin(workspace_bytes=fa.fa_bwd_workspace_size(1, 8, 128, 64)) == fa.FA_ERR_WORKSPACE
    assert _dkdv_dq(workspace=0x10008) == fa.FA_ERR_WORKSPACE


@pytest.mark.skipif(_has_gpu(), reason="would launch kernels on the bogus pointers")
def test_one_pass_steps_without_gpu_report_device_error():
    assert _dkdv_dq() == fa.FA_ERR_DEVICE and _dq_fin() == fa.FA_ERR_DEVICE
    nb = fa.fa_bwd_workspace_size(1, 1, 128, 64)
    assert fa.fa_bwd_preprocess(P, P, P, 1, 1, 128, 64, fa.FA_F16, 0x10000, nb, None) == fa.FA_ERR_DEVICE
    assert fa.fa_bwd_dkdv(P, P, P, P, P, P, P, 1, 1, 128, 64, 0, 0.1, fa.FA_F16, 0x10000, nb,
                          None) == fa.FA_ERR_DEVICE
