"""Plant plausible mistakes in the oracle's windows, packed batches, block masks and
dropout, and require that one of the pins in test_oracle.py catches each.

Each mutant replaces one oracle function for the duration of a test
(monkeypatch); the pins are then run against the mutated oracle.  Everything
here runs on the CPU.
"""
import numpy as np
import pytest

import oracle
from oracle import attention as att
from oracle import philox
from tests import test_oracle as T


def _fails(fn):
    """A pin catches a mutant when it fails on it: an assertion, or an error raised
    by the oracle's own checks."""
    try:
        fn()
    except (AssertionError, ValueError):
        return True
    return False


WINDOW_PINS = [
    lambda: T.test_window_wider_than_the_sequence_changes_nothing(True),
    T.test_window_of_one_key_is_the_value_row,
    lambda: T.test_sliding_window_brute_force(2),
    lambda: T.test_local_window_zero_query(3, 1),
    lambda: T.test_local_window_zero_query(0, 4),
    T.test_window_cell_count_matches_the_page,
]

VARLEN_PINS = [
    lambda: T.test_varlen_equal_lengths_is_the_padded_batch(True),
    lambda: T.test_varlen_is_block_diagonal_attention(True),
    T.test_varlen_sequences_do_not_interact,
    lambda: T.test_varlen_zero_query(True),
]

BLOCK_PINS = [
    T.test_full_block_mask_changes_nothing,
    lambda: T.test_block_diagonal_mask_is_a_packed_batch(False),
    T.test_block_mask_empty_rows_and_zero_query,
]

DROPOUT_PINS = [
    T.test_philox_known_answers,
    T.test_uniform_layout_of_one_call,
    T.test_keep_rate_and_uniformity,
    T.test_dropout_zero_query_closed_form,
    T.test_dropout_is_unbiased,
    lambda: T.test_dropout_finite_differences(False),
]


def test_unmutated_oracle_passes_every_pin():
    for pin in WINDOW_PINS + VARLEN_PINS + BLOCK_PINS + DROPOUT_PINS:
        pin()


def _window_off_by_one(n_q, n_k, window):
    left, right = window
    i, j = np.arange(n_q)[:, None], np.arange(n_k)[None, :]
    vis = np.ones((n_q, n_k), dtype=bool)
    if left is not None and left >= 0:
        vis &= j > i - left                       # mistake: excludes key i - left
    if right is not None and right >= 0:
        vis &= j <= i + right
    return vis


def _window_sides_swapped(n_q, n_k, window):
    return att.__dict__["_orig_window_visible"](n_q, n_k, (window[1], window[0]))


@pytest.mark.parametrize("name,fn", [("off by one on the left", _window_off_by_one),
                                     ("left and right swapped", _window_sides_swapped)])
def test_window_mistake_is_caught(monkeypatch, name, fn):
    monkeypatch.setitem(att.__dict__, "_orig_window_visible", att.window_visible)
    monkeypatch.setattr(att, "window_visible", fn)
    assert any(_fails(p) for p in WINDOW_PINS), name


def test_varlen_offset_mistake_is_caught(monkeypatch):
    """Sequences shifted by one packed row (a wrong offset convention)."""
    orig = att._spans

    def shifted(cu_seqlens, total, max_s):
        cu = orig(cu_seqlens, total, max_s)
        return [0] + [min(total, c + 1) for c in cu[1:-1]] + [cu[-1]]
    monkeypatch.setattr(att, "_spans", shifted)
    assert any(_fails(p) for p in VARLEN_PINS)


def test_varlen_head_mapping_mistake_is_caught(monkeypatch):
    """Query head h reading K/V head h mod H_kv instead of h // (H / H_kv)."""
    def wrong(q, k, v, cu_seqlens, max_s, scale, causal, seqs=None, window=None, dropout=None,
              block_mask=None):
        q, k, v = (np.asarray(x, dtype=np.float64) for x in (q, k, v))
        H, total = q.shape[:2]
        hk = k.shape[0]
        cu = att._spans(cu_seqlens, total, max_s)
        o = np.full((H, total, v.shape[-1]), np.nan)
        lse = np.full((len(cu) - 1, H, max_s), np.nan)
        for b in range(len(cu) - 1):
            s0, s1 = cu[b], cu[b + 1]
            if s1 == s0:
                continue
            for h in range(H):
                o[h, s0:s1], lse[b, h, :s1 - s0] = att.forward_head(
                    q[h, s0:s1], k[h % hk, s0:s1], v[h % hk, s0:s1], scale, causal)
        return o, lse
    monkeypatch.setattr(oracle, "forward_varlen", wrong)
    assert any(_fails(p) for p in VARLEN_PINS)


def test_block_mask_mistake_is_caught(monkeypatch):
    """Block sizes swapped (128 queries x 256 keys)."""
    def swapped(n_q, n_k, blocks):
        b = np.asarray(blocks) != 0
        qi = np.minimum(np.arange(n_q) // 128, b.shape[0] - 1)
        kj = np.minimum(np.arange(n_k) // 256, b.shape[1] - 1)
        return b[qi[:, None], kj[None, :]]
    monkeypatch.setattr(att, "block_visible", swapped)
    assert any(_fails(p) for p in BLOCK_PINS)


@pytest.mark.parametrize("name", ["multiplier", "halves swapped", "scale dropped", "dP unmasked"])
def test_dropout_mistake_is_caught(monkeypatch, name):
    if name == "multiplier":
        orig = philox.philox4x32

        def wrong(c0, c1, c2, c3, k0, k1, rounds=10):
            return orig(c2, c1, c0, c3, k0, k1, rounds)    # counter words 0 and 2 swapped
        monkeypatch.setattr(philox, "philox4x32", wrong)
    elif name == "halves swapped":
        orig = philox.uniforms16

        def wrong(head, n_q, n_k, seed, offset):
            u = orig(head, n_q, n_k, seed, offset).astype(np.int64)
            return (((u & 0xFF) << 8) | (u >> 8)).astype(np.uint16)   # bytes swapped
        monkeypatch.setattr(philox, "uniforms16", wrong)
    elif name == "scale dropped":
        monkeypatch.setattr(att, "dropped", lambda p, drop: p if drop is None
                            else np.where(drop[0], p, 0.0))
    else:
        orig = att.dropped
        calls = {"n": 0}

        def wrong(p, drop):
            calls["n"] += 1
            # the backward's second use (on dO V^T) is left undropped
            return p if (drop is not None and calls["n"] % 3 == 0) else orig(p, drop)
        monkeypatch.setattr(att, "dropped", wrong)
    assert any(_fails(p) for p in DROPOUT_PINS), name
