"""The online-softmax tile recurrence and the two-tile merge, in float64.

TEST INFRASTRUCTURE ONLY (see the package docstring).  These functions are not
the reference the GPU path is compared with (that is ``attention.py``, the
plain definition).  They restate the recurrence the pages prove exact, so that
tests can pin the recurrence itself against the states and values the pages
print, and against the plain definition.

Sources:
  * two-tile merge of per-row states (m, l, u):
        m~ = max(new scores), l~ = sum e^{s - m~}, u~ = sum e^{s - m~} v,
        m' = max(m, m~), a = e^{m - m'}, b = e^{m~ - m'},
        l' = a l + b l~, u' = a u + b u~, o' = u' / l',
    starting from m = -inf, l = 0, u = 0:
    "FlashAttention 원 논문 해부" (sj-techlog), section
    "두 tile을 한 row로 합치는 식";
  * the forward loop over key/value tiles with the unnormalized accumulator,
    rescaled by diag(e^{m_old - m_new}) per tile and divided by l once at the
    end, and L = m + log l:
    "FlashAttention-2: Faster Attention with Better Parallelism and Work
    Partitioning" (wonbeomjang.kr), sections "개선 1: Rescaling을 마지막에 한
    번만", "개선 2: m과 l 대신 L만 저장" and
    "결과: FlashAttention-2 Forward 알고리즘".
"""
from __future__ import annotations

import numpy as np


def merge_tile(m: float, l: float, u, s_new, v_new) -> dict:
    """Fold one tile (scores s_new[k], values v_new[k, dv]) into a row state.

    Returns the tile state (m_t, l_t, u_t), the factors (a, b) and the merged
    state (m, l, u, o).  Hidden keys carry s = -inf and contribute nothing.
    """
    s_new = np.asarray(s_new, dtype=np.float64)
    v_new = np.asarray(v_new, dtype=np.float64).reshape(s_new.shape[0], -1)
    u = np.asarray(u, dtype=np.float64).reshape(-1)
    m_t = float(s_new.max())
    if np.isfinite(m_t):
        w = np.exp(s_new - m_t)
    else:                                   # the whole tile is hidden
        w = np.zeros_like(s_new)
    l_t = float(w.sum())
    u_t = w @ v_new
    m_new = max(m, m_t)
    if not np.isfinite(m_new):              # nothing visible so far
        return {"m_t": m_t, "l_t": l_t, "u_t": u_t, "a": 0.0, "b": 0.0,
                "m": m_new, "l": 0.0, "u": np.zeros_like(u_t), "o": np.full_like(u_t, np.nan)}
    a = float(np.exp(m - m_new))            # e^{-inf} = 0 for the initial state
    b = float(np.exp(m_t - m_new)) if np.isfinite(m_t) else 0.0
    l_new = a * l + b * l_t
    u_new = a * u + b * u_t
    return {"m_t": m_t, "l_t": l_t, "u_t": u_t, "a": a, "b": b,
            "m": m_new, "l": l_new, "u": u_new, "o": u_new / l_new}


def online_forward_head(q, k, v, scale: float, causal: bool, block_cols: int,
                        record_row: int | None = None):
    """Forward for one head by the tile recurrence over key blocks of width block_cols.

    Keeps, per query row, the running max m, normalizer l and the unnormalized
    accumulator; rescales by e^{m_old - m_new} per tile and divides by l once.
    Returns (O, LSE, states) where ``states`` lists (start, end, m, l) after
    each tile for row ``record_row`` (empty if None).
    """
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    n_q, n_k = q.shape[0], k.shape[0]
    m = np.full(n_q, -np.inf)
    l = np.zeros(n_q)
    acc = np.zeros((n_q, v.shape[1]))
    rows = np.arange(n_q)[:, None]
    states = []
    for start in range(0, n_k, block_cols):
        end = min(start + block_cols, n_k)
        s = float(scale) * (q @ k[start:end].T)             # tile S_ij
        if causal:
            s = np.where(np.arange(start, end)[None, :] <= rows, s, -np.inf)
        m_new = np.maximum(m, s.max(axis=1))
        m_ref = np.where(np.isfinite(m_new), m_new, 0.0)
        alpha = np.exp(m - m_ref)                            # e^{m_old - m_new}
        p = np.exp(s - m_ref[:, None])                       # unnormalized tile probs
        l = alpha * l + p.sum(axis=1)
        acc = alpha[:, None] * acc + p @ v[start:end]
        m = m_new
        if record_row is not None:
            states.append((start, end, float(m[record_row]), float(l[record_row])))
    o = np.zeros_like(acc)
    np.divide(acc, l[:, None], out=o, where=l[:, None] > 0)
    lse = np.full(n_q, -np.inf)
    pos = l > 0
    lse[pos] = m[pos] + np.log(l[pos])
    return o, lse, states
