"""Seeded synthetic attention workloads, shared by the tests and the benchmark.

This module only draws random numbers and rounds them to the storage dtype.
It holds none of the attention arithmetic: the HIP library computes attention,
and the fp64 oracle under ``oracle/`` recomputes it for checking.  Both sides
receive the very same rounded tensors from here.

Every workload is Q, K, V and an upstream gradient dO, each [B, H, N, d] and
contiguous with d fastest (K and V [B, H_kv, N, d] when H_kv key/value heads are
shared by the H query heads), plus the softmax scale (1/sqrt(d)).  Draw order for
one workload, from a CPU ``torch.Generator`` seeded with the workload's seed:
[the per-head offset, only when ``offset`` is set], Q, K, V, dO, all as fp32
standard normals.  Q and K are then multiplied by ``qk_std``; with ``offset``
the per-head vector c[h] (one N(0,1)^d draw per head index, shared by every Q
and K row of that head in every batch entry) is added to Q and K.  Finally all
four tensors are rounded to the workload dtype (round to nearest even).
"""
from __future__ import annotations

import dataclasses
import math

import torch

_TORCH_DTYPES = {"f32": torch.float32, "f16": torch.float16, "bf16": torch.bfloat16}


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    B: int
    H: int
    N: int
    d: int
    dtype: str          # "f32" | "f16" | "bf16"
    causal: bool
    seed: int
    qk_std: float = 1.0
    offset: bool = False
    H_kv: int = 0       # key/value heads (0: one per query head)
    window: tuple = (-1, -1)   # local window (left, right); -1: open side
    dropout: tuple = ()        # (p, seed, offset): dropout on P, regenerated in the backward
    block_density: float = 0.0   # > 0: a block-sparse mask per head (block_mask())

    @property
    def kv_heads(self) -> int:
        return self.H_kv or self.H

    @property
    def windowed(self) -> bool:
        return tuple(self.window) != (-1, -1)

    @property
    def sparse(self) -> bool:
        return self.block_density > 0

    @property
    def scale(self) -> float:
        return 1.0 / math.sqrt(self.d)

    @property
    def torch_dtype(self) -> torch.dtype:
        return _TORCH_DTYPES[self.dtype]

    def fwd_flops(self) -> float:
        """Forward FLOPs counted as 4*B*H*N^2*d, halved under the causal mask; with a
        local window, 4*B*H*d per visible (query, key) pair."""
        if self.sparse:
            bm = block_mask(self)
            return 4.0 * self.B * self.d * sum(block_pairs(self.N, self.causal, bm[h])
                                               for h in range(self.H))
        if self.windowed:
            return 4.0 * self.B * self.H * self.d * visible_pairs(self.N, self.causal, self.window)
        f = 4.0 * self.B * self.H * self.N * self.N * self.d
        return f / 2 if self.causal else f

    def bwd_flops(self) -> float:
        """Backward FLOPs counted as 2.5x the forward count."""
        return 2.5 * self.fwd_flops()

    def with_(self, **kw) -> "Workload":
        return dataclasses.replace(self, **kw)


def visible_pairs(n: int, causal: bool, window) -> int:
    """Number of (query, key) pairs with max(0, i - left) <= j <= min(n - 1, i + right)
    (right = 0 under the causal mask; -1 = open side), summed row by row."""
    left, right = window
    left = n if left < 0 else left
    right = (n if right < 0 else right) if not causal else min(0 if right < 0 else right, 0)
    total = 0
    for i in range(n):   # n is at most a few tens of thousands
        total += min(n - 1, i + right) - max(0, i - left) + 1
    return total


BLOCK_Q, BLOCK_K = 256, 128   # block sizes of a block-sparse mask (queries x keys)


def block_mask(w) -> torch.Tensor:
    """uint8 [H, ceil(N / 256), ceil(N / 128)]: each block kept with probability
    block_density (seeded with seed + 1), the key blocks of a query block's own
    rows always kept (so that no row is empty)."""
    nbq, nbk = -(-w.N // BLOCK_Q), -(-w.N // BLOCK_K)
    g = torch.Generator(device="cpu").manual_seed(w.seed + 1)
    m = (torch.rand((w.H, nbq, nbk), generator=g) < w.block_density).to(torch.uint8)
    for qb in range(nbq):
        m[:, qb, (qb * BLOCK_Q) // BLOCK_K:min(nbk, ((qb + 1) * BLOCK_Q + BLOCK_K - 1) // BLOCK_K)] = 1
    return m.contiguous()


def block_pairs(n: int, causal: bool, bm) -> int:
    """(query, key) pairs a block mask [nbq, nbk] keeps (under the causal mask,
    those with key <= query), counted block by block."""
    total = 0
    nbq, nbk = bm.shape
    for qb in range(nbq):
        q0, q1 = qb * BLOCK_Q, min(n, (qb + 1) * BLOCK_Q)
        for kb in range(nbk):
            if not bm[qb, kb]:
                continue
            k0, k1 = kb * BLOCK_K, min(n, (kb + 1) * BLOCK_K)
            if not causal:
                total += (q1 - q0) * (k1 - k0)
            else:
                for i in range(q0, q1):
                    total += max(0, min(k1, i + 1) - k0)
    return total


# The five workloads of the method's measurement plan, named by what they are.
SINGLE_HEAD_F32 = Workload("b1h1n128d64-f32", 1, 1, 128, 64, "f32", False, 1001)
SHORT_F16 = Workload("b8h16n1024d64-f16", 8, 16, 1024, 64, "f16", False, 1002)
CAUSAL_BF16 = Workload("b4h32n4096d128-bf16-causal", 4, 32, 4096, 128, "bf16", True, 1003)
LONG_CAUSAL_F16 = Workload("b1h16n16384d64-f16-causal-qkstd2", 1, 16, 16384, 64, "f16",
                           True, 1004, qk_std=2.0)
PEAKED_BF16 = Workload("b2h32n8192d128-bf16-offset", 2, 32, 8192, 128, "bf16", False, 1005,
                       offset=True)

ALL = (SINGLE_HEAD_F32, SHORT_F16, CAUSAL_BF16, LONG_CAUSAL_F16, PEAKED_BF16)

# Grouped key/value heads (32 query heads over 8 or 4 K/V heads) at the shapes of
# the two d = 128 workloads above.
GQA_BF16 = Workload("b2h32kv8n8192d128-bf16-gqa", 2, 32, 8192, 128, "bf16", False, 1006, H_kv=8)
GQA_CAUSAL_BF16 = Workload("b4h32kv4n4096d128-bf16-causal-gqa", 4, 32, 4096, 128, "bf16", True,
                           1007, H_kv=4)
GQA = (GQA_BF16, GQA_CAUSAL_BF16)

# Sliding-window attention: each query sees its 4096 most recent keys (window
# left 4095, causal), with grouped K/V heads: the local-attention configuration of
# the efficiency page's sliding-window section, at N = 16384.
WINDOW_BF16 = Workload("b2h32kv8n16384d128-bf16-causal-window4096", 2, 32, 16384, 128, "bf16",
                       True, 1010, H_kv=8, window=(4095, -1))
WINDOWED = (WINDOW_BF16,)

# Training-time dropout at the rate of the original paper's runtime benchmark
# (p = 0.1: "FlashAttention 원 논문 해부", section "원 논문 benchmark는 조건을
# 떼지 않고 읽는다"), at the shape of the offset workload.
DROPOUT_BF16 = Workload("b2h32n8192d128-bf16-dropout0.1", 2, 32, 8192, 128, "bf16", False, 1011,
                        dropout=(0.1, 0x5EED_0001_2345_6789, 7))
DROPOUT = (DROPOUT_BF16,)

# Block-sparse attention at the offset workload's shape: a quarter of the
# 256 x 128 blocks kept at random per head (the block-diagonal always).
SPARSE_BF16 = Workload("b2h32n8192d128-bf16-blocksparse25", 2, 32, 8192, 128, "bf16", False, 1012,
                       block_density=0.25)
SPARSE = (SPARSE_BF16,)

BY_NAME = {w.name: w for w in ALL + GQA + WINDOWED + DROPOUT + SPARSE}


def make_inputs(w: Workload) -> dict:
    """Return {"q","k","v","do"} as contiguous CPU tensors in the workload dtype."""
    g = torch.Generator(device="cpu").manual_seed(w.seed)
    shape = (w.B, w.H, w.N, w.d)
    kv_shape = (w.B, w.kv_heads, w.N, w.d)
    if w.offset and w.kv_heads != w.H:
        raise ValueError("the per-head offset is defined for one K/V head per query head")
    c = torch.randn((w.H, w.d), generator=g, dtype=torch.float32) if w.offset else None
    q = torch.randn(shape, generator=g, dtype=torch.float32)
    k = torch.randn(kv_shape, generator=g, dtype=torch.float32)
    v = torch.randn(kv_shape, generator=g, dtype=torch.float32)
    do = torch.randn(shape, generator=g, dtype=torch.float32)
    if w.qk_std != 1.0:
        q.mul_(w.qk_std)
        k.mul_(w.qk_std)
    if c is not None:
        q.add_(c[None, :, None, :])
        k.add_(c[None, :, None, :])
    dt = w.torch_dtype
    return {name: t.to(dt).contiguous() for name, t in (("q", q), ("k", k), ("v", v), ("do", do))}


# ----------------------------------------------------------- packed variable-length batches
#
# A padding-free batch: sequences of different lengths packed one after another,
# one slab per head: Q and dO [H, total, d], K and V [H_kv, total, d], with
# cu_seqlens the B + 1 cumulative offsets.  Draw order from a CPU generator
# seeded with the workload's seed: Q, K, V, dO (fp32 standard normals, rounded
# to the dtype).  The lengths are part of the workload's definition.


@dataclasses.dataclass(frozen=True)
class Varlen:
    name: str
    lens: tuple         # sequence lengths (zeros allowed)
    H: int
    d: int
    dtype: str
    causal: bool
    seed: int
    H_kv: int = 0

    @property
    def B(self) -> int:
        return len(self.lens)

    @property
    def kv_heads(self) -> int:
        return self.H_kv or self.H

    @property
    def total(self) -> int:
        return int(sum(self.lens))

    @property
    def max_s(self) -> int:
        return max(max(self.lens), 1)

    @property
    def cu_seqlens(self) -> torch.Tensor:
        cu = [0]
        for n in self.lens:
            cu.append(cu[-1] + int(n))
        return torch.tensor(cu, dtype=torch.int32)

    @property
    def scale(self) -> float:
        return 1.0 / math.sqrt(self.d)

    @property
    def torch_dtype(self) -> torch.dtype:
        return _TORCH_DTYPES[self.dtype]

    def fwd_flops(self) -> float:
        """4*H*n^2*d per sequence of length n (halved under the causal mask)."""
        f = sum(4.0 * self.H * n * n * self.d for n in self.lens)
        return f / 2 if self.causal else f

    def bwd_flops(self) -> float:
        return 2.5 * self.fwd_flops()


def uniform_lengths(B: int, lo: int, hi: int, seed: int) -> tuple:
    """B lengths drawn uniformly from [lo, hi] with a seeded CPU generator."""
    g = torch.Generator(device="cpu").manual_seed(seed)
    return tuple(int(x) for x in torch.randint(lo, hi + 1, (B,), generator=g))


# 16 sequences of 512 to 8192 tokens (uniform), 32 query heads, d = 128: the
# token budget of the dense b2h32n8192d128 workloads spread over a realistic
# length mix; one full-mask and one causal with grouped K/V heads.
VARLEN_BF16 = Varlen("varlen16-512to8192-h32d128-bf16", uniform_lengths(16, 512, 8192, 1008), 32,
                     128, "bf16", False, 1008)
VARLEN_CAUSAL_BF16 = Varlen("varlen16-512to8192-h32kv8d128-bf16-causal",
                            uniform_lengths(16, 512, 8192, 1009), 32, 128, "bf16", True, 1009,
                            H_kv=8)
VARLEN = (VARLEN_BF16, VARLEN_CAUSAL_BF16)
VARLEN_BY_NAME = {w.name: w for w in VARLEN}


def make_varlen_inputs(w: Varlen, extra_rows: int = 0) -> dict:
    """{"q","k","v","do"} packed per head ([H or H_kv, total + extra_rows, d]) and
    "cu_seqlens" (int32, B + 1); ``extra_rows`` trailing rows belong to no sequence."""
    g = torch.Generator(device="cpu").manual_seed(w.seed)
    rows = w.total + extra_rows
    q = torch.randn((w.H, rows, w.d), generator=g, dtype=torch.float32)
    k = torch.randn((w.kv_heads, rows, w.d), generator=g, dtype=torch.float32)
    v = torch.randn((w.kv_heads, rows, w.d), generator=g, dtype=torch.float32)
    do = torch.randn((w.H, rows, w.d), generator=g, dtype=torch.float32)
    dt = w.torch_dtype
    out = {name: t.to(dt).contiguous() for name, t in (("q", q), ("k", k), ("v", v), ("do", do))}
    out["cu_seqlens"] = w.cu_seqlens
    return out


def make_random(shape, dtype: str, seed: int, std: float = 1.0) -> torch.Tensor:
    """One seeded N(0, std^2) tensor rounded to ``dtype`` (for edge-case tests)."""
    g = torch.Generator(device="cpu").manual_seed(seed)
    t = torch.randn(shape, generator=g, dtype=torch.float32)
    if std != 1.0:
        t.mul_(std)
    return t.to(_TORCH_DTYPES[dtype]).contiguous()
