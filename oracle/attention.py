"""The plain definition of exact softmax attention, in float64, on the CPU.

TEST INFRASTRUCTURE ONLY (see the package docstring): only the tests, the
smoke check and the benchmark's CPU baseline may use this module.

Per head, with Q, K in R^{N x d}, V in R^{N x dv} and softmax scale tau:

    S = tau * Q K^T                          (N x N, materialized)
    S_ij = -inf for j > i  under the causal mask
    P = row-wise softmax(S), computed stably by subtracting the row max
    O = P V,   LSE_i = m_i + ln(sum_j exp(S_ij - m_i))

Sources, by page and section:
  * definition S = tau Q K^T, P = softmax(S), O = P V and the causal mask
    s_ij = -inf for j > i: "FlashAttention 원 논문 해부" (sj-techlog),
    sections "원 논문의 정의" and "Q·K·V와 한 행의 의미";
  * stable softmax (subtract the row max m; the value is unchanged): same page,
    section "stable softmax는 overflow를 막는 필수 변형이다";
  * LSE L = m + log(l), with P = exp(S - L) recovered from it in the backward:
    "FlashAttention-2: Faster Attention with Better Parallelism and Work
    Partitioning" (wonbeomjang.kr), section "개선 2: m과 l 대신 L만 저장".
    "log" is read as the natural log, since P = exp(S - L) must hold.
  * backward dV = P^T dO, dP = dO V^T, dS_ij = P_ij (dP_ij - D_i) with
    D_i = sum_j P_ij dP_ij, dQ = dS K, dK = dS^T Q: the FlashAttention-2 page,
    section "Standard Attention Implementation / Backward Pass".  That page
    writes S = Q K^T without tau; with S = tau Q K^T the chain rule puts one
    factor tau on dQ and dK (dV is unaffected), and the oracle includes it.
    Finite-difference tests pin this reading.

Fully masked rows (impossible under the square causal mask, but defined here
so the functions are total): P row = 0, O row = 0, LSE = -inf, no gradient.

Every array is converted to float64 on entry.  No blocking, fusion or
reordering: each step is one numpy expression of the definition above.
"""
from __future__ import annotations

import numpy as np

from . import philox


def _f64(x) -> np.ndarray:
    return np.asarray(x, dtype=np.float64)


def causal_visible(n_q: int, n_k: int) -> np.ndarray:
    """Boolean [n_q, n_k]: key j is visible to query i iff j <= i."""
    i = np.arange(n_q)[:, None]
    j = np.arange(n_k)[None, :]
    return j <= i


def window_visible(n_q: int, n_k: int, window) -> np.ndarray:
    """Boolean [n_q, n_k]: key j is inside the window (left, right) of query i iff
    i - left <= j <= i + right; a side given as None or a negative number is
    open.  Local attention: "어텐션 비용 줄이기" (ailab.paldyn.com), sections
    "지역 윈도와 글로벌 토큰" (w keys on each side) and "슬라이딩 윈도와 수용 영역"
    (the most recent W keys: causal with left = W - 1)."""
    left, right = window
    i = np.arange(n_q)[:, None]
    j = np.arange(n_k)[None, :]
    vis = np.ones((n_q, n_k), dtype=bool)
    if left is not None and left >= 0:
        vis &= j >= i - left
    if right is not None and right >= 0:
        vis &= j <= i + right
    return vis


BLOCK_Q, BLOCK_K = 256, 128


def block_visible(n_q: int, n_k: int, blocks) -> np.ndarray:
    """Boolean [n_q, n_k] from a block mask [ceil(n_q / BLOCK_Q), ceil(n_k / BLOCK_K)]:
    key j is visible to query i iff block (i // BLOCK_Q, j // BLOCK_K) is nonzero.
    Block-sparse attention skips the zero blocks of a given mask ("FlashAttention 원
    논문 해부", section "대안, 비교와 선택 기준"); the dense attention with this
    element mask is its exact result."""
    b = np.asarray(blocks) != 0
    return b[np.arange(n_q)[:, None] // BLOCK_Q, np.arange(n_k)[None, :] // BLOCK_K]


def scores(q, k, scale: float, causal: bool, window=None, blocks=None) -> np.ndarray:
    """S = scale * Q K^T for one head, with -inf where the causal mask, the window
    or a block mask hides a key."""
    q, k = _f64(q), _f64(k)
    s = float(scale) * (q @ k.T)
    if causal:
        s = np.where(causal_visible(q.shape[0], k.shape[0]), s, -np.inf)
    if window is not None:
        s = np.where(window_visible(q.shape[0], k.shape[0], window), s, -np.inf)
    if blocks is not None:
        s = np.where(block_visible(q.shape[0], k.shape[0], blocks), s, -np.inf)
    return s


def row_softmax(s) -> tuple[np.ndarray, np.ndarray]:
    """Stable row softmax of S.  Returns (P, LSE) with LSE in natural-log units."""
    s = _f64(s)
    m = s.max(axis=1)                      # row maximum
    has_key = np.isfinite(m)
    m_ref = np.where(has_key, m, 0.0)      # reference point (0 for empty rows)
    e = np.exp(s - m_ref[:, None])         # exp(-inf) = 0 for hidden keys
    l = e.sum(axis=1)                      # normalizer
    p = np.zeros_like(e)
    np.divide(e, l[:, None], out=p, where=l[:, None] > 0)
    lse = np.full(l.shape, -np.inf)
    pos = l > 0
    lse[pos] = m_ref[pos] + np.log(l[pos])
    return p, lse


def probabilities(q, k, scale: float, causal: bool, window=None) -> np.ndarray:
    """P = softmax(scale * Q K^T + mask) for one head."""
    p, _ = row_softmax(scores(q, k, scale, causal, window))
    return p


def dropped(p, drop):
    """Dropout applied to P: drop = (keep mask [n_q, n_k], scale) or None.  Kept
    entries are multiplied by the scale (the inverse keep probability), so the
    expectation over masks is P itself."""
    if drop is None:
        return p
    mask, sc = drop
    return np.where(mask, p * float(sc), 0.0)


def forward_head(q, k, v, scale: float, causal: bool, window=None,
                 drop=None, blocks=None) -> tuple[np.ndarray, np.ndarray]:
    """O = dropout(P) V and LSE for one head (q: [N,d], k: [N,d], v: [N,dv]).  LSE
    is that of the undropped softmax (it is what the backward recomputes P from)."""
    p, lse = row_softmax(scores(q, k, scale, causal, window, blocks))
    o = dropped(p, drop) @ _f64(v)
    return o, lse


def backward_head(q, k, v, do, scale: float, causal: bool, window=None, drop=None,
                  blocks=None) -> dict:
    """Analytic gradients of sum(O * dO) for one head.

    Returns dict(dq, dk, dv, D, p, dp, ds); D is computed as rowsum(P * dP).
    """
    q, k, v, do = _f64(q), _f64(k), _f64(v), _f64(do)
    p, _ = row_softmax(scores(q, k, scale, causal, window, blocks))
    dv = dropped(p, drop).T @ do           # dV = dropout(P)^T dO
    dp = dropped(do @ v.T, drop)           # dP = dropout'(dO V^T): the chain rule
                                           # through the kept entries and the scale
    D = (p * dp).sum(axis=1)               # D_i = sum_j P_ij dP_ij
    ds = p * (dp - D[:, None])             # dS_ij = P_ij (dP_ij - D_i)
    dq = float(scale) * (ds @ k)           # dQ = tau dS K
    dk = float(scale) * (ds.T @ q)         # dK = tau dS^T Q
    return {"dq": dq, "dk": dk, "dv": dv, "D": D, "p": p, "dp": dp, "ds": ds}


def _heads(shape):
    return np.ndindex(*shape[:-2])


def head_drop(dropout, hd: int, n: int):
    """The (mask, scale) of attention head hd = b H + h for dropout = (p_drop, seed,
    offset), or None.  The scale is 2^16 / threshold, the inverse of the keep
    probability the 16-bit threshold realizes (0 when everything is dropped)."""
    if dropout is None:
        return None
    p_drop, seed, offset = dropout
    t = philox.keep_threshold(p_drop)
    return philox.keep_mask(hd, n, n, p_drop, seed, offset), (65536.0 / t if t > 0 else 0.0)


def _hd(idx, shape):
    """Head index b H + h of a [B, H, ...] leading index."""
    return int(idx[0]) * int(shape[1]) + int(idx[1])


def forward(q, k, v, scale: float, causal: bool, heads=None, window=None, dropout=None):
    """Batched forward over leading axes ([..., N, d]); returns (O, LSE).

    ``heads`` optionally restricts the work to a list of leading-index tuples;
    the other heads of the returned arrays are left as NaN.
    """
    q, k, v = _f64(q), _f64(k), _f64(v)
    lead = q.shape[:-2]
    o = np.full(lead + (q.shape[-2], v.shape[-1]), np.nan)
    lse = np.full(lead + (q.shape[-2],), np.nan)
    for idx in (heads if heads is not None else _heads(q.shape)):
        drop = head_drop(dropout, _hd(idx, q.shape), q.shape[-2])
        o[idx], lse[idx] = forward_head(q[idx], k[idx], v[idx], scale, causal, window, drop)
    return o, lse


def backward(q, k, v, do, scale: float, causal: bool, heads=None, window=None, dropout=None):
    """Batched backward over leading axes; returns (dQ, dK, dV, D)."""
    q, k, v, do = _f64(q), _f64(k), _f64(v), _f64(do)
    lead = q.shape[:-2]
    dq = np.full(q.shape, np.nan)
    dk = np.full(k.shape, np.nan)
    dv = np.full(v.shape, np.nan)
    D = np.full(lead + (q.shape[-2],), np.nan)
    for idx in (heads if heads is not None else _heads(q.shape)):
        drop = head_drop(dropout, _hd(idx, q.shape), q.shape[-2])
        g = backward_head(q[idx], k[idx], v[idx], do[idx], scale, causal, window, drop)
        dq[idx], dk[idx], dv[idx], D[idx] = g["dq"], g["dk"], g["dv"], g["D"]
    return dq, dk, dv, D


# ---------------------------------------------------------------- grouped K/V heads
#
# Grouped-query attention: the page "Transformer 효율화 기법" (ailab.paldyn.com),
# section "v1에서 v3까지", names GQA among FlashAttention-2's features but does
# not define it.  Reading: H query heads share H_kv key/value heads (H_kv
# divides H); query head h attends with key/value head h // (H // H_kv) of the
# same batch entry.  Each query head is the plain definition above; the
# gradient of a shared K or V head is the sum over the query heads that use it
# (the chain rule through every use).


def _group(h_q: int, h_kv: int) -> int:
    if h_kv <= 0 or h_q % h_kv:
        raise ValueError(f"{h_q} query heads cannot share {h_kv} key/value heads")
    return h_q // h_kv


def _blocks(block_mask, h):
    """Block mask of query head h from [1 or H, nbq, nbk], or None."""
    if block_mask is None:
        return None
    bm = np.asarray(block_mask)
    return bm[h % bm.shape[0]]


def forward_gqa(q, k, v, scale: float, causal: bool, window=None, dropout=None,
                block_mask=None):
    """q [B, H, N, d], k [B, H_kv, N, d], v [B, H_kv, N, dv] -> (O [B, H, N, dv],
    LSE [B, H, N])."""
    q, k, v = _f64(q), _f64(k), _f64(v)
    B, H = q.shape[:2]
    g = _group(H, k.shape[1])
    o = np.empty((B, H, q.shape[2], v.shape[-1]))
    lse = np.empty((B, H, q.shape[2]))
    for b in range(B):
        for h in range(H):
            drop = head_drop(dropout, b * H + h, q.shape[2])
            o[b, h], lse[b, h] = forward_head(q[b, h], k[b, h // g], v[b, h // g], scale, causal,
                                              window, drop, _blocks(block_mask, h))
    return o, lse


def backward_gqa(q, k, v, do, scale: float, causal: bool, window=None, dropout=None,
                 block_mask=None):
    """Gradients of sum(O * dO) for forward_gqa: (dQ [B, H, N, d], dK [B, H_kv, N, d],
    dV [B, H_kv, N, dv])."""
    q, k, v, do = _f64(q), _f64(k), _f64(v), _f64(do)
    B, H = q.shape[:2]
    g = _group(H, k.shape[1])
    dq = np.empty(q.shape)
    dk = np.zeros(k.shape)
    dv = np.zeros(v.shape)
    for b in range(B):
        for h in range(H):
            drop = head_drop(dropout, b * H + h, q.shape[2])
            r = backward_head(q[b, h], k[b, h // g], v[b, h // g], do[b, h], scale, causal, window,
                              drop, _blocks(block_mask, h))
            dq[b, h] = r["dq"]
            dk[b, h // g] += r["dk"]
            dv[b, h // g] += r["dv"]
    return dq, dk, dv


# ---------------------------------------------------------------- variable-length batches
#
# Dropout (every batched function's `dropout` = (p_drop, seed, offset)): the
# keep mask of head b H + h is philox.keep_mask; in a packed batch, b is the
# sequence and positions count inside it.
#
# Padding-free batches: the 2022 interface described on "FlashAttention 원 논문
# 해부" (section "내부 구조와 실제 실행 흐름", items 2 and 3) packs the valid tokens
# of all sequences one after another and passes cu_seqlens (the cumulative token
# offset of each sequence, B + 1 entries from 0 to the token total) and max_s
# (the longest length); the softmax statistics stay [B, heads, max_s].
# Reading: sequence b owns packed rows cu[b] <= t < cu[b + 1]; its attention is
# the plain definition over its own tokens only (the causal mask top-left
# aligned at its first token), so tokens of different sequences never see one
# another.  Layout here: one packed slab per head, q [H, total, d],
# k and v [H_kv, total, d] (grouped heads as above); rows outside every
# sequence and LSE entries past a sequence's length are left as NaN.


def _spans(cu_seqlens, total: int, max_s: int):
    cu = [int(x) for x in np.asarray(cu_seqlens).reshape(-1)]
    if len(cu) < 2 or cu[0] != 0 or cu[-1] > total:
        raise ValueError("cu_seqlens must start at 0 and end at most at the token total")
    for b in range(len(cu) - 1):
        if not 0 <= cu[b + 1] - cu[b] <= max_s:
            raise ValueError(f"sequence {b} has length {cu[b + 1] - cu[b]} outside [0, {max_s}]")
    return cu


def forward_varlen(q, k, v, cu_seqlens, max_s: int, scale: float, causal: bool, seqs=None,
                   window=None, dropout=None, block_mask=None):
    """q [H, total, d], k [H_kv, total, d], v [H_kv, total, dv] -> (O [H, total, dv],
    LSE [B, H, max_s]).  ``seqs`` optionally restricts the work to some sequences."""
    q, k, v = _f64(q), _f64(k), _f64(v)
    H, total = q.shape[:2]
    g = _group(H, k.shape[0])
    cu = _spans(cu_seqlens, total, max_s)
    B = len(cu) - 1
    o = np.full((H, total, v.shape[-1]), np.nan)
    lse = np.full((B, H, max_s), np.nan)
    for b in (seqs if seqs is not None else range(B)):
        s0, s1 = cu[b], cu[b + 1]
        if s1 == s0:
            continue   # an empty sequence has no rows
        for h in range(H):
            drop = head_drop(dropout, b * H + h, s1 - s0)
            o[h, s0:s1], lse[b, h, : s1 - s0] = forward_head(
                q[h, s0:s1], k[h // g, s0:s1], v[h // g, s0:s1], scale, causal, window, drop,
                _blocks(block_mask, h))
    return o, lse


def backward_varlen(q, k, v, do, cu_seqlens, max_s: int, scale: float, causal: bool, seqs=None,
                    window=None, dropout=None, block_mask=None):
    """Gradients of sum(O * dO) for forward_varlen: (dQ [H, total, d],
    dK [H_kv, total, d], dV [H_kv, total, dv]); rows outside the computed
    sequences are NaN."""
    q, k, v, do = _f64(q), _f64(k), _f64(v), _f64(do)
    H, total = q.shape[:2]
    g = _group(H, k.shape[0])
    cu = _spans(cu_seqlens, total, max_s)
    dq = np.full(q.shape, np.nan)
    dk = np.full(k.shape, np.nan)
    dv = np.full(v.shape, np.nan)
    for b in (seqs if seqs is not None else range(len(cu) - 1)):
        s0, s1 = cu[b], cu[b + 1]
        if s1 == s0:
            continue
        dk[:, s0:s1] = 0.0
        dv[:, s0:s1] = 0.0
        for h in range(H):
            drop = head_drop(dropout, b * H + h, s1 - s0)
            r = backward_head(q[h, s0:s1], k[h // g, s0:s1], v[h // g, s0:s1], do[h, s0:s1],
                              scale, causal, window, drop, _blocks(block_mask, h))
            dq[h, s0:s1] = r["dq"]
            dk[h // g, s0:s1] += r["dk"]
            dv[h // g, s0:s1] += r["dv"]
    return dq, dk, dv
