"""Python binding of libfa.so, the gfx950 exact-attention library.

Argument marshalling only: every step of the forward and backward runs in
the library's HIP kernels.  PyTorch supplies device memory and the current
stream.  If libfa.so is missing, importing the binding raises instead of
falling back to anything else.

Two layers:
  * ``fa_fwd`` / ``fa_bwd`` / ``fa_bwd_workspace_size`` / ``fa_status_string``
    / ``fa_abi_version``: the C entry points with the same names and the same
    arguments (device pointers as Python ints, sizes, dtype code, stream
    handle); they return the status code.
  * ``forward`` / ``backward`` (and ``forward_varlen`` / ``backward_varlen``
    for packed variable-length batches): torch tensors in, torch tensors out; they
    check shapes, allocate outputs (and the backward workspace) with torch
    and raise ``FaError`` on a non-zero status.
"""
from __future__ import annotations

import ctypes
import os

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libfa.so")

FA_OK = 0
FA_ERR_INVALID_ARGUMENT = 1
FA_ERR_UNSUPPORTED = 2
FA_ERR_WORKSPACE = 3
FA_ERR_DEVICE = 4
FA_ERR_LAUNCH = 5

FA_F32 = 0
FA_F16 = 1
FA_BF16 = 2

EXPORTED = ("fa_abi_version", "fa_status_string", "fa_fwd", "fa_bwd_workspace_size", "fa_bwd",
            "fa_bwd_preprocess", "fa_bwd_dkdv", "fa_bwd_dq", "fa_fwd_gqa", "fa_bwd_gqa",
            "fa_bwd_dkdv_gqa", "fa_bwd_dq_gqa", "fa_fwd_varlen", "fa_bwd_varlen", "fa_fwd_ex",
            "fa_bwd_ex", "fa_bwd_noalloc", "fa_bwd_dkdv_dq", "fa_bwd_dq_finalize")

FA_NOALLOC_SCRATCH_BYTES = 32 << 20


class FaAttn(ctypes.Structure):
    """struct fa_attn of include/fa.h: one call's shape, mask, window and packing."""
    _fields_ = [("B", ctypes.c_int), ("H", ctypes.c_int), ("H_kv", ctypes.c_int),
                ("N", ctypes.c_int), ("d", ctypes.c_int), ("causal", ctypes.c_int),
                ("window_left", ctypes.c_int), ("window_right", ctypes.c_int),
                ("scale", ctypes.c_float), ("dtype", ctypes.c_int),
                ("cu_seqlens", ctypes.c_void_p), ("total", ctypes.c_int),
                ("dropout_p", ctypes.c_float), ("seed", ctypes.c_ulonglong),
                ("rng_offset", ctypes.c_uint), ("block_mask", ctypes.c_void_p),
                ("block_mask_heads", ctypes.c_int)]

FA_BLOCK_Q = 256
FA_BLOCK_K = 128


class FaError(RuntimeError):
    def __init__(self, status: int, where: str):
        super().__init__(f"{where}: {fa_status_string(status)} (status {status})")
        self.status = status


def _load() -> ctypes.CDLL:
    if not os.path.exists(LIB_PATH):
        raise ImportError(
            f"{LIB_PATH} is not built; run `python io_aware_exact_fa_amd/_build.py` "
            "(or __graft_entry__.build()) first")
    # torch ships its own HIP runtime (same soname as the system one).  Load torch
    # first so libfa.so binds to that runtime: device memory and streams come from
    # torch, and two HIP runtimes in one process would not share them.
    import torch  # noqa: F401
    lib = ctypes.CDLL(LIB_PATH)
    _check_single_runtime()
    vp, i, f, sz = ctypes.c_void_p, ctypes.c_int, ctypes.c_float, ctypes.c_size_t
    lib.fa_abi_version.restype = i
    lib.fa_abi_version.argtypes = []
    lib.fa_status_string.restype = ctypes.c_char_p
    lib.fa_status_string.argtypes = [i]
    lib.fa_fwd.restype = i
    lib.fa_fwd.argtypes = [vp, vp, vp, vp, vp, i, i, i, i, i, f, i, vp]
    lib.fa_bwd_workspace_size.restype = sz
    lib.fa_bwd_workspace_size.argtypes = [i, i, i, i]
    lib.fa_bwd.restype = i
    lib.fa_bwd.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, vp, i, i, i, i, i, f, i, vp, sz, vp]
    lib.fa_bwd_noalloc.restype = i
    lib.fa_bwd_noalloc.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, vp, i, i, i, i, i, f, i, vp]
    lib.fa_bwd_dkdv_dq.restype = i
    lib.fa_bwd_dkdv_dq.argtypes = [vp, vp, vp, vp, vp, vp, vp, i, i, i, i, i, i, f, i, vp, sz, vp]
    lib.fa_bwd_dq_finalize.restype = i
    lib.fa_bwd_dq_finalize.argtypes = [vp, i, i, i, i, f, i, vp, sz, vp]
    lib.fa_bwd_preprocess.restype = i
    lib.fa_bwd_preprocess.argtypes = [vp, vp, vp, i, i, i, i, i, vp, sz, vp]
    lib.fa_bwd_dkdv.restype = i
    lib.fa_bwd_dkdv.argtypes = [vp, vp, vp, vp, vp, vp, vp, i, i, i, i, i, f, i, vp, sz, vp]
    lib.fa_bwd_dq.restype = i
    lib.fa_bwd_dq.argtypes = [vp, vp, vp, vp, vp, vp, i, i, i, i, i, f, i, vp, sz, vp]
    lib.fa_fwd_gqa.restype = i
    lib.fa_fwd_gqa.argtypes = [vp, vp, vp, vp, vp, i, i, i, i, i, i, f, i, vp]
    lib.fa_bwd_gqa.restype = i
    lib.fa_bwd_gqa.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, vp, i, i, i, i, i, i, f, i, vp, sz,
                               vp]
    lib.fa_bwd_dkdv_gqa.restype = i
    lib.fa_bwd_dkdv_gqa.argtypes = [vp, vp, vp, vp, vp, vp, vp, i, i, i, i, i, i, f, i, vp, sz, vp]
    lib.fa_bwd_dq_gqa.restype = i
    lib.fa_bwd_dq_gqa.argtypes = [vp, vp, vp, vp, vp, vp, i, i, i, i, i, i, f, i, vp, sz, vp]
    lib.fa_fwd_varlen.restype = i
    lib.fa_fwd_varlen.argtypes = [vp, vp, vp, vp, vp, vp, i, i, i, i, i, i, i, f, i, vp]
    lib.fa_bwd_varlen.restype = i
    lib.fa_bwd_varlen.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, i, i, i, i, i, i, i, f,
                                  i, vp, sz, vp]
    pa = ctypes.POINTER(FaAttn)
    lib.fa_fwd_ex.restype = i
    lib.fa_fwd_ex.argtypes = [pa, vp, vp, vp, vp, vp, vp]
    lib.fa_bwd_ex.restype = i
    lib.fa_bwd_ex.argtypes = [pa, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, sz, vp]
    return lib


def _check_single_runtime() -> None:
    try:
        with open("/proc/self/maps") as f:
            paths = {line.split()[-1] for line in f if "libamdhip64" in line}
    except OSError:
        return
    if len(paths) > 1:
        raise ImportError(f"two HIP runtimes are loaded in this process: {sorted(paths)}")


_lib = _load()


# ------------------------------------------------------------------ C entry points


def fa_abi_version() -> int:
    return _lib.fa_abi_version()


def fa_status_string(status: int) -> str:
    return _lib.fa_status_string(int(status)).decode()


def fa_fwd(q, k, v, o, lse, B, H, N, d, causal, scale, dtype, stream) -> int:
    return _lib.fa_fwd(q, k, v, o, lse, B, H, N, d, int(causal), float(scale), int(dtype), stream)


def fa_bwd_workspace_size(B, H, N, d) -> int:
    return _lib.fa_bwd_workspace_size(B, H, N, d)


def fa_bwd(q, k, v, o, dout, lse, dq, dk, dv, B, H, N, d, causal, scale, dtype,
           workspace, workspace_bytes, stream) -> int:
    return _lib.fa_bwd(q, k, v, o, dout, lse, dq, dk, dv, B, H, N, d, int(causal), float(scale),
                       int(dtype), workspace, workspace_bytes, stream)


def fa_bwd_noalloc(q, k, v, o, dout, lse, dq, dk, dv, B, H, N, d, causal, scale, dtype,
                   stream) -> int:
    return _lib.fa_bwd_noalloc(q, k, v, o, dout, lse, dq, dk, dv, B, H, N, d, int(causal),
                               float(scale), int(dtype), stream)


def fa_bwd_dkdv_dq(q, k, v, dout, lse, dk, dv, B, H, H_kv, N, d, causal, scale, dtype,
                   workspace, workspace_bytes, stream) -> int:
    return _lib.fa_bwd_dkdv_dq(q, k, v, dout, lse, dk, dv, B, H, H_kv, N, d, int(causal),
                               float(scale), int(dtype), workspace, workspace_bytes, stream)


def fa_bwd_dq_finalize(dq, B, H, N, d, scale, dtype, workspace, workspace_bytes, stream) -> int:
    return _lib.fa_bwd_dq_finalize(dq, B, H, N, d, float(scale), int(dtype), workspace,
                                   workspace_bytes, stream)


def fa_bwd_preprocess(o, dout, lse, B, H, N, d, dtype, workspace, workspace_bytes, stream) -> int:
    return _lib.fa_bwd_preprocess(o, dout, lse, B, H, N, d, int(dtype), workspace, workspace_bytes,
                                  stream)


def fa_bwd_dkdv(q, k, v, dout, lse, dk, dv, B, H, N, d, causal, scale, dtype,
                workspace, workspace_bytes, stream) -> int:
    return _lib.fa_bwd_dkdv(q, k, v, dout, lse, dk, dv, B, H, N, d, int(causal), float(scale),
                            int(dtype), workspace, workspace_bytes, stream)


def fa_bwd_dq(q, k, v, dout, lse, dq, B, H, N, d, causal, scale, dtype,
              workspace, workspace_bytes, stream) -> int:
    return _lib.fa_bwd_dq(q, k, v, dout, lse, dq, B, H, N, d, int(causal), float(scale),
                          int(dtype), workspace, workspace_bytes, stream)


def fa_fwd_gqa(q, k, v, o, lse, B, H, H_kv, N, d, causal, scale, dtype, stream) -> int:
    return _lib.fa_fwd_gqa(q, k, v, o, lse, B, H, H_kv, N, d, int(causal), float(scale),
                           int(dtype), stream)


def fa_bwd_gqa(q, k, v, o, dout, lse, dq, dk, dv, B, H, H_kv, N, d, causal, scale, dtype,
               workspace, workspace_bytes, stream) -> int:
    return _lib.fa_bwd_gqa(q, k, v, o, dout, lse, dq, dk, dv, B, H, H_kv, N, d, int(causal),
                           float(scale), int(dtype), workspace, workspace_bytes, stream)


def fa_bwd_dkdv_gqa(q, k, v, dout, lse, dk, dv, B, H, H_kv, N, d, causal, scale, dtype,
                    workspace, workspace_bytes, stream) -> int:
    return _lib.fa_bwd_dkdv_gqa(q, k, v, dout, lse, dk, dv, B, H, H_kv, N, d, int(causal),
                                float(scale), int(dtype), workspace, workspace_bytes, stream)


def fa_bwd_dq_gqa(q, k, v, dout, lse, dq, B, H, H_kv, N, d, causal, scale, dtype,
                  workspace, workspace_bytes, stream) -> int:
    return _lib.fa_bwd_dq_gqa(q, k, v, dout, lse, dq, B, H, H_kv, N, d, int(causal), float(scale),
                              int(dtype), workspace, workspace_bytes, stream)


def fa_fwd_varlen(q, k, v, o, lse, cu_seqlens, B, max_s, total, H, H_kv, d, causal, scale, dtype,
                  stream) -> int:
    return _lib.fa_fwd_varlen(q, k, v, o, lse, cu_seqlens, B, max_s, total, H, H_kv, d,
                              int(causal), float(scale), int(dtype), stream)


def fa_bwd_varlen(q, k, v, o, dout, lse, dq, dk, dv, cu_seqlens, B, max_s, total, H, H_kv, d,
                  causal, scale, dtype, workspace, workspace_bytes, stream) -> int:
    return _lib.fa_bwd_varlen(q, k, v, o, dout, lse, dq, dk, dv, cu_seqlens, B, max_s, total, H,
                              H_kv, d, int(causal), float(scale), int(dtype), workspace,
                              workspace_bytes, stream)


def fa_fwd_ex(p, q, k, v, o, lse, stream) -> int:
    return _lib.fa_fwd_ex(ctypes.byref(p) if p is not None else None, q, k, v, o, lse, stream)


def fa_bwd_ex(p, q, k, v, o, dout, lse, dq, dk, dv, workspace, workspace_bytes, stream) -> int:
    return _lib.fa_bwd_ex(ctypes.byref(p) if p is not None else None, q, k, v, o, dout, lse, dq,
                          dk, dv, workspace, workspace_bytes, stream)


def attn(B, H, H_kv, N, d, causal, scale, dtype, window=(-1, -1), cu_seqlens=None,
         total=0, dropout=None, block_mask=None, block_mask_heads=1) -> FaAttn:
    """Fill an fa_attn (window sides -1 = open; cu_seqlens and block_mask device
    addresses or None; dropout = (p, seed, offset) or None)."""
    p, seed, offset = dropout if dropout is not None else (0.0, 0, 0)
    return FaAttn(B, H, H_kv, N, d, int(causal), int(window[0]), int(window[1]), float(scale),
                  int(dtype), cu_seqlens, int(total), float(p), int(seed), int(offset),
                  block_mask, int(block_mask_heads))


# ------------------------------------------------------------------ torch helpers


def dtype_code(torch_dtype) -> int:
    import torch
    codes = {torch.float32: FA_F32, torch.float16: FA_F16, torch.bfloat16: FA_BF16}
    if torch_dtype not in codes:
        raise TypeError(f"unsupported dtype {torch_dtype}")
    return codes[torch_dtype]


def _check(name, t, shape, dtype):
    if tuple(t.shape) != tuple(shape) or t.dtype != dtype or not t.is_contiguous() or not t.is_cuda:
        raise ValueError(f"{name}: expected contiguous {dtype} cuda tensor of shape {tuple(shape)}, "
                         f"got {t.dtype} {tuple(t.shape)} contiguous={t.is_contiguous()} "
                         f"device={t.device}")
    # fa.h: [.., d] tensors 16-byte aligned (16-byte loads and LDS-direct copies),
    # float32 row statistics 4-byte aligned.
    align = 4 if name == "lse" else 16
    if t.data_ptr() % align != 0:
        raise ValueError(f"{name}: data pointer {t.data_ptr():#x} is not {align}-byte aligned "
                         "(a view at an offset into another tensor?)")



def _stream(stream):
    import torch
    if stream is None:
        return torch.cuda.current_stream().cuda_stream
    return stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream)


def forward(q, k, v, causal: bool, scale: float, o=None, lse=None, stream=None, window=None,
            dropout=None, block_mask=None):
    """O, LSE for q [B, H, N, d] and k, v [B, H_kv, N, d] (H_kv divides H; all one
    dtype, on the GPU).  ``window`` = (left, right), -1 = open side; ``dropout`` =
    (p, seed, offset)."""
    import torch
    B, H, N, d = q.shape
    H_kv = k.shape[1]
    _check("q", q, (B, H, N, d), q.dtype)
    _check("k", k, (B, H_kv, N, d), q.dtype)
    _check("v", v, (B, H_kv, N, d), q.dtype)
    if o is None:
        o = torch.empty_like(q)
    if lse is None:
        lse = torch.empty((B, H, N), dtype=torch.float32, device=q.device)
    _check("o", o, (B, H, N, d), q.dtype)
    _check("lse", lse, (B, H, N), torch.float32)
    if window is not None or dropout is not None or block_mask is not None:
        p = attn(B, H, H_kv, N, d, causal, scale, dtype_code(q.dtype), window or (-1, -1),
                 dropout=dropout, **_bm(block_mask, H, N, q.device))
        st = fa_fwd_ex(p, q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), lse.data_ptr(),
                       _stream(stream))
        if st != FA_OK:
            raise FaError(st, "fa_fwd_ex")
        return o, lse
    st = fa_fwd_gqa(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), lse.data_ptr(),
                    B, H, H_kv, N, d, causal, scale, dtype_code(q.dtype), _stream(stream))
    if st != FA_OK:
        raise FaError(st, "fa_fwd_gqa")
    return o, lse


def workspace(B, H, N, d, device, one_pass=False):
    """A torch uint8 buffer big enough (and aligned) for fa_bwd at this shape; with
    one_pass, also for the one-pass steps (fa_bwd_dkdv_dq, fa_bwd_dq_finalize):
    fa_bwd_workspace_size plus the float32 dQ accumulator [B, H, Np, d]."""
    import torch
    n = fa_bwd_workspace_size(B, H, N, d)
    if n == 0:
        raise FaError(FA_ERR_INVALID_ARGUMENT, "fa_bwd_workspace_size")
    if one_pass:
        n += 4 * B * H * ((N + 63) // 64 * 64) * d
    return torch.empty(n, dtype=torch.uint8, device=device)   # caching allocator: 512 B aligned


def backward(q, k, v, o, dout, lse, causal: bool, scale: float, dq=None, dk=None, dv=None,
             ws=None, stream=None, window=None, dropout=None, block_mask=None):
    """dQ, dK, dV for the forward that produced o and lse."""
    import torch
    B, H, N, d = q.shape
    H_kv = k.shape[1]
    for name, t in (("q", q), ("o", o), ("dout", dout)):
        _check(name, t, (B, H, N, d), q.dtype)
    for name, t in (("k", k), ("v", v)):
        _check(name, t, (B, H_kv, N, d), q.dtype)
    _check("lse", lse, (B, H, N), torch.float32)
    dq = torch.empty_like(q) if dq is None else dq
    dk = torch.empty_like(k) if dk is None else dk
    dv = torch.empty_like(k) if dv is None else dv
    _check("dq", dq, (B, H, N, d), q.dtype)
    for name, t in (("dk", dk), ("dv", dv)):
        _check(name, t, (B, H_kv, N, d), q.dtype)
    ws = workspace(B, H, N, d, q.device) if ws is None else ws
    if window is not None or dropout is not None or block_mask is not None:
        p = attn(B, H, H_kv, N, d, causal, scale, dtype_code(q.dtype), window or (-1, -1),
                 dropout=dropout, **_bm(block_mask, H, N, q.device))
        st = fa_bwd_ex(p, q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), dout.data_ptr(),
                       lse.data_ptr(), dq.data_ptr(), dk.data_ptr(), dv.data_ptr(), ws.data_ptr(),
                       ws.numel(), _stream(stream))
        if st != FA_OK:
            raise FaError(st, "fa_bwd_ex")
        return dq, dk, dv
    st = fa_bwd_gqa(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), dout.data_ptr(),
                    lse.data_ptr(), dq.data_ptr(), dk.data_ptr(), dv.data_ptr(), B, H, H_kv, N, d,
                    causal, scale, dtype_code(q.dtype), ws.data_ptr(), ws.numel(),
                    _stream(stream))
    if st != FA_OK:
        raise FaError(st, "fa_bwd_gqa")
    return dq, dk, dv


def _bm(block_mask, H, N, device):
    """fa_attn fields of a block mask: a contiguous uint8 device tensor
    [1 or H, ceil(N / FA_BLOCK_Q), ceil(N / FA_BLOCK_K)]."""
    import torch
    if block_mask is None:
        return {}
    nbq, nbk = -(-N // FA_BLOCK_Q), -(-N // FA_BLOCK_K)
    if (block_mask.dtype != torch.uint8 or block_mask.dim() != 3 or block_mask.shape[0] not in (1, H)
            or tuple(block_mask.shape[1:]) != (nbq, nbk) or not block_mask.is_contiguous()
            or block_mask.device != device):
        raise ValueError(f"block_mask: expected a contiguous uint8 tensor [1 or {H}, {nbq}, {nbk}] "
                         f"on {device}, got {block_mask.dtype} {tuple(block_mask.shape)}")
    return {"block_mask": block_mask.data_ptr(), "block_mask_heads": block_mask.shape[0]}


def _check_cu(cu_seqlens, device):
    import torch
    if (cu_seqlens.dtype != torch.int32 or cu_seqlens.dim() != 1 or cu_seqlens.numel() < 2
            or not cu_seqlens.is_contiguous() or cu_seqlens.device != device):
        raise ValueError("cu_seqlens: expected a contiguous 1-D int32 tensor of B + 1 offsets on "
                         f"{device}, got {cu_seqlens.dtype} {tuple(cu_seqlens.shape)} on "
                         f"{cu_seqlens.device}")
    return cu_seqlens.numel() - 1


def forward_varlen(q, k, v, cu_seqlens, max_s: int, causal: bool, scale: float, o=None, lse=None,
                   stream=None, window=None, dropout=None, block_mask=None):
    """O [H, total, d], LSE [B, H, max_s] for packed q [H, total, d], k, v
    [H_kv, total, d] and device int32 cu_seqlens [B + 1] (offsets are read on the
    device, not checked here)."""
    import torch
    H, total, d = q.shape
    H_kv = k.shape[0]
    B = _check_cu(cu_seqlens, q.device)
    _check("q", q, (H, total, d), q.dtype)
    _check("k", k, (H_kv, total, d), q.dtype)
    _check("v", v, (H_kv, total, d), q.dtype)
    o = torch.empty_like(q) if o is None else o
    lse = torch.empty((B, H, max_s), dtype=torch.float32, device=q.device) if lse is None else lse
    _check("o", o, (H, total, d), q.dtype)
    _check("lse", lse, (B, H, max_s), torch.float32)
    if window is not None or dropout is not None or block_mask is not None:
        p = attn(B, H, H_kv, max_s, d, causal, scale, dtype_code(q.dtype), window or (-1, -1),
                 cu_seqlens.data_ptr(), total, dropout, **_bm(block_mask, H, max_s, q.device))
        st = fa_fwd_ex(p, q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), lse.data_ptr(),
                       _stream(stream))
    else:
        st = fa_fwd_varlen(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), lse.data_ptr(),
                           cu_seqlens.data_ptr(), B, max_s, total, H, H_kv, d, causal, scale,
                           dtype_code(q.dtype), _stream(stream))
    if st != FA_OK:
        raise FaError(st, "fa_fwd_varlen")
    return o, lse


def backward_varlen(q, k, v, o, dout, lse, cu_seqlens, max_s: int, causal: bool, scale: float,
                    dq=None, dk=None, dv=None, ws=None, stream=None, window=None, dropout=None,
                    block_mask=None):
    """dQ, dK, dV for the packed forward that produced o and lse."""
    import torch
    H, total, d = q.shape
    H_kv = k.shape[0]
    B = _check_cu(cu_seqlens, q.device)
    for name, t in (("q", q), ("o", o), ("dout", dout)):
        _check(name, t, (H, total, d), q.dtype)
    for name, t in (("k", k), ("v", v)):
        _check(name, t, (H_kv, total, d), q.dtype)
    _check("lse", lse, (B, H, max_s), torch.float32)
    dq = torch.empty_like(q) if dq is None else dq
    dk = torch.empty_like(k) if dk is None else dk
    dv = torch.empty_like(k) if dv is None else dv
    _check("dq", dq, (H, total, d), q.dtype)
    for name, t in (("dk", dk), ("dv", dv)):
        _check(name, t, (H_kv, total, d), q.dtype)
    ws = workspace(B, H, max_s, d, q.device) if ws is None else ws
    if window is not None or dropout is not None or block_mask is not None:
        p = attn(B, H, H_kv, max_s, d, causal, scale, dtype_code(q.dtype), window or (-1, -1),
                 cu_seqlens.data_ptr(), total, dropout, **_bm(block_mask, H, max_s, q.device))
        st = fa_bwd_ex(p, q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), dout.data_ptr(),
                       lse.data_ptr(), dq.data_ptr(), dk.data_ptr(), dv.data_ptr(), ws.data_ptr(),
                       ws.numel(), _stream(stream))
    else:
        st = fa_bwd_varlen(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(),
                           dout.data_ptr(), lse.data_ptr(), dq.data_ptr(), dk.data_ptr(),
                           dv.data_ptr(), cu_seqlens.data_ptr(), B, max_s, total, H, H_kv, d,
                           causal, scale, dtype_code(q.dtype), ws.data_ptr(), ws.numel(),
                           _stream(stream))
    if st != FA_OK:
        raise FaError(st, "fa_bwd_varlen")
    return dq, dk, dv
