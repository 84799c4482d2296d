"""Pins of the fp64 oracle against what the pages and the mathematics fix (CPU only)."""
import math

import numpy as np
import pytest

import oracle
from tests import pins


def fwd(q, k, v, scale, causal):
    return oracle.forward_head(q, k, v, scale, causal)


def bwd(q, k, v, do, scale, causal):
    g = oracle.backward_head(q, k, v, do, scale, causal)
    return g["dq"], g["dk"], g["dv"]


# ----------------------------------------------------------------- page values


def test_page_causal_first_row():
    pins.check_page_cpu_vectors(fwd)


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("block", [1, 2, 3])
def test_page_tiled_recurrence_equals_standard(causal, block):
    """The page checks tile widths 1, 2, 3, causal on and off, to 1e-12."""
    g = pins.load_golden("cpu_check_vectors.json")
    q, k, v = (np.array(g[n], dtype=np.float64) for n in ("q", "k", "v"))
    scale = 1.0 / math.sqrt(3.0)
    o_ref, lse_ref = oracle.forward_head(q, k, v, scale, causal)
    o, lse, _ = oracle.online_forward_head(q, k, v, scale, causal, block)
    assert np.max(np.abs(o - o_ref)) <= g["tiled_vs_standard_tolerance"]
    assert np.max(np.abs(lse - lse_ref)) <= g["tiled_vs_standard_tolerance"]


@pytest.mark.parametrize("causal", [False, True])
def test_page_printed_row_states(causal):
    """Row 4 (0-based) with tile width 2 passes through the printed (m, l) states."""
    g = pins.load_golden("cpu_check_vectors.json")
    q, k, v = (np.array(g[n], dtype=np.float64) for n in ("q", "k", "v"))
    _, _, states = oracle.online_forward_head(q, k, v, 1.0 / math.sqrt(3.0), causal, 2,
                                              record_row=4)
    printed = g["printed"]["row4_block2_states"]
    half_ulp = 0.5 * 10.0 ** -g["printed"]["printed_decimals"]
    assert len(states) == len(printed)
    for (start, end, m, l), p in zip(states, printed):
        assert (start, end) == (p["start"], p["end"])
        assert abs(m - p["m"]) <= half_ulp + 1e-12
        assert abs(l - p["l"]) <= half_ulp + 1e-12


def test_page_merge_example():
    g = pins.load_golden("merge_example.json")
    st = g["state"]
    r = oracle.merge_tile(st["m"], st["l"], [st["u"]], g["tile_scores"],
                          np.array(g["tile_values"])[:, None])
    p = g["printed"]
    assert r["m_t"] == p["m_tile"] and r["m"] == p["m_new"] and r["b"] == p["b"]
    for key, name in (("l_t", "l_tile"), ("a", "a"), ("l", "l_new")):
        assert abs(float(np.ravel(r[key])[0]) - p[name]) <= 1e-4, key
    assert abs(float(r["u_t"][0]) - p["u_tile"]) <= 1e-4
    assert abs(float(r["u"][0]) - p["u_new"]) <= 1e-4
    assert abs(float(r["o"][0]) - p["o_new"]) <= 5e-4


def test_page_rescale_example():
    g = pins.load_golden("rescale_example.json")
    # A block whose maximum is 5 (its other score is far below, so it barely matters).
    r = oracle.merge_tile(g["m_old"], g["l_old"], [0.0], [g["m_block"], -50.0], np.zeros((2, 1)))
    p = g["printed"]
    assert r["m"] == g["m_block"]
    assert abs(r["a"] - p["factor"]) <= 5e-3 * p["factor"]
    assert abs(r["a"] * g["l_old"] - p["l_old_rescaled"]) <= 5e-3 * p["l_old_rescaled"]


def test_merge_equals_softmax_of_concatenation():
    """Merging tile by tile from (m, l, u) = (-inf, 0, 0) is the softmax of the whole row."""
    r = np.random.default_rng(11)
    s = 4.0 * r.standard_normal(13)
    v = r.standard_normal((13, 3))
    state = {"m": -np.inf, "l": 0.0, "u": np.zeros(3)}
    for a, b in ((0, 4), (4, 5), (5, 13)):
        state = oracle.merge_tile(state["m"], state["l"], state["u"], s[a:b], v[a:b])
    w = np.exp(s - s.max())
    np.testing.assert_allclose(state["o"], (w / w.sum()) @ v, atol=1e-14)
    np.testing.assert_allclose(state["m"] + math.log(state["l"]),
                               s.max() + math.log(w.sum()), atol=1e-14)


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("block", [1, 2, 3, 7, 16, 40])
def test_recurrence_equals_definition(causal, block):
    r = np.random.default_rng(12)
    q, k, v = (3.0 * r.standard_normal((40, 8)) for _ in range(3))
    o_ref, lse_ref = oracle.forward_head(q, k, v, 0.35, causal)
    o, lse, _ = oracle.online_forward_head(q, k, v, 0.35, causal, block)
    assert np.max(np.abs(o - o_ref)) <= 1e-12
    assert np.max(np.abs(lse - lse_ref)) <= 1e-12


# ----------------------------------------------------------------- closed forms


@pytest.mark.parametrize("causal", [False, True])
def test_zero_query_mean_of_values(causal):
    pins.check_zero_query(fwd, causal=causal)


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("jstar", [0, 3, 7])
def test_dominant_score(causal, jstar):
    pins.check_dominant_score(fwd, causal=causal, jstar=jstar)


def test_dominant_score_selects_one_row():
    """As the dominant score grows, O_i tends to v_{j*}."""
    r = np.random.default_rng(13)
    n, d = 6, 4
    q = np.zeros((n, d))
    q[:, 0] = 200.0
    k = r.standard_normal((n, d))
    k[:, 0] = 0.0
    k[2] = np.eye(d)[0]
    v = r.standard_normal((n, 2))
    o, _ = oracle.forward_head(q, k, v, 1.0, False)
    np.testing.assert_allclose(o, np.repeat(v[2:3], n, axis=0), atol=1e-12)


def test_single_key():
    pins.check_single_key(fwd, bwd)


# ----------------------------------------------------------------- invariants


@pytest.mark.parametrize("causal", [False, True])
def test_probability_rows(causal):
    """P >= 0, rows sum to 1, hidden keys get exactly 0."""
    r = np.random.default_rng(14)
    q, k = 2.0 * r.standard_normal((12, 5)), 2.0 * r.standard_normal((12, 5))
    p = oracle.probabilities(q, k, 0.5, causal)
    assert np.all(p >= 0)
    np.testing.assert_allclose(p.sum(axis=1), 1.0, atol=1e-14)
    if causal:
        assert np.all(p[~oracle.causal_visible(12, 12)] == 0.0)
        assert np.all(p[oracle.causal_visible(12, 12)] > 0.0)


def test_large_scores_do_not_overflow():
    """Scores around 1e3 would overflow exp without the max subtraction."""
    r = np.random.default_rng(15)
    q, k, v = 40.0 * r.standard_normal((8, 4)), 40.0 * r.standard_normal((8, 4)), r.standard_normal((8, 3))
    o, lse = oracle.forward_head(q, k, v, 1.0, False)
    assert np.all(np.isfinite(o)) and np.all(np.isfinite(lse))
    o2, lse2 = oracle.forward_head(q, k + 7.0, v, 1.0, False)   # shift by a row constant
    np.testing.assert_allclose(o2, o, atol=1e-10)


@pytest.mark.parametrize("causal", [False, True])
def test_key_shift_invariance(causal):
    pins.check_key_shift(fwd, bwd, causal=causal)


def test_value_linearity():
    pins.check_value_linearity(fwd)


def test_fully_hidden_rows_are_zero():
    """A row with no visible key (possible only with a non-causal mask pattern) is defined as
    O = 0, LSE = -inf."""
    s = np.array([[0.0, 1.0], [-np.inf, -np.inf]])
    p, lse = oracle.row_softmax(s)
    assert np.all(p[1] == 0.0) and lse[1] == -np.inf
    np.testing.assert_allclose(p[0].sum(), 1.0)


# ----------------------------------------------------------------- backward


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("n", [2, 5, 16])
def test_finite_differences(causal, n):
    pins.check_finite_differences(fwd, bwd, n=n, causal=causal)


def test_finite_differences_unit_scale_wide_values():
    pins.check_finite_differences(fwd, bwd, n=7, d=3, dv=5, scale=1.0, causal=True, seed=21)


@pytest.mark.parametrize("causal", [False, True])
def test_zero_query_gradients(causal):
    pins.check_zero_query_gradients(bwd, causal=causal)


@pytest.mark.parametrize("causal", [False, True])
def test_delta_identity(causal):
    """D_i = rowsum(P * dP) equals rowsum(dO * O)."""
    r = np.random.default_rng(16)
    q, k, v, do = (r.standard_normal((11, 6)) for _ in range(4))
    g = oracle.backward_head(q, k, v, do, 0.4, causal)
    o, _ = oracle.forward_head(q, k, v, 0.4, causal)
    np.testing.assert_allclose(g["D"], (do * o).sum(axis=1), atol=1e-13)
    np.testing.assert_allclose(g["ds"].sum(axis=1), 0.0, atol=1e-13)


def test_batched_wrappers_match_heads():
    r = np.random.default_rng(17)
    q, k, v, do = (r.standard_normal((2, 3, 9, 4)) for _ in range(4))
    o, lse = oracle.forward(q, k, v, 0.5, True)
    dq, dk, dv, D = oracle.backward(q, k, v, do, 0.5, True)
    for b in range(2):
        for h in range(3):
            o1, l1 = oracle.forward_head(q[b, h], k[b, h], v[b, h], 0.5, True)
            g = oracle.backward_head(q[b, h], k[b, h], v[b, h], do[b, h], 0.5, True)
            np.testing.assert_array_equal(o[b, h], o1)
            np.testing.assert_array_equal(lse[b, h], l1)
            np.testing.assert_array_equal(dq[b, h], g["dq"])
            np.testing.assert_array_equal(dk[b, h], g["dk"])
            np.testing.assert_array_equal(dv[b, h], g["dv"])
            np.testing.assert_array_equal(D[b, h], g["D"])
    o_s, _ = oracle.forward(q, k, v, 0.5, True, heads=[(1, 2)])
    np.testing.assert_array_equal(o_s[1, 2], o[1, 2])
    assert np.isnan(o_s[0, 0]).all()


# ----------------------------------------------------------- grouped K/V heads


def _gqa_inputs(B=2, H=6, H_kv=2, n=5, d=3, dv=4, seed=11):
    r = np.random.default_rng(seed)
    return (r.standard_normal((B, H, n, d)), r.standard_normal((B, H_kv, n, d)),
            r.standard_normal((B, H_kv, n, dv)), r.standard_normal((B, H, n, dv)))


@pytest.mark.parametrize("causal", [False, True])
def test_gqa_with_one_query_head_per_kv_head_is_plain_attention(causal):
    q, k, v, do = _gqa_inputs(H=3, H_kv=3)
    o, lse = oracle.forward_gqa(q, k, v, 0.6, causal)
    for b in range(2):
        for h in range(3):
            o1, l1 = oracle.forward_head(q[b, h], k[b, h], v[b, h], 0.6, causal)
            np.testing.assert_array_equal(o[b, h], o1)
            np.testing.assert_array_equal(lse[b, h], l1)


def test_gqa_head_mapping():
    """Key/value head j holds values equal to j + 1 in every entry, so every output
    row of query head h is exactly 1 + (the K/V head it reads): h // (H / H_kv)."""
    q, k, _, _ = _gqa_inputs(H=6, H_kv=3)
    v = np.broadcast_to(np.arange(1.0, 4.0)[None, :, None, None], (2, 3, 5, 4)).copy()
    o, _ = oracle.forward_gqa(q, k, v, 0.9, False)
    for h in range(6):
        np.testing.assert_allclose(o[:, h], 1.0 + h // 2, rtol=0, atol=1e-14)


@pytest.mark.parametrize("causal", [False, True])
def test_gqa_zero_query(causal):
    """Q = 0: every query head's rows are means of the (visible) rows of its shared V."""
    _, k, v, _ = _gqa_inputs(H=4, H_kv=2, n=7)
    o, lse = oracle.forward_gqa(np.zeros((2, 4, 7, 3)), k, v, 0.4, causal)
    for b in range(2):
        for h in range(4):
            for i in range(7):
                vis = i + 1 if causal else 7
                np.testing.assert_allclose(o[b, h, i], v[b, h // 2, :vis].mean(axis=0), atol=1e-13)
                np.testing.assert_allclose(lse[b, h, i], math.log(vis), atol=1e-13)


@pytest.mark.parametrize("causal", [False, True])
def test_gqa_finite_differences(causal):
    """Central differences of L = sum(O * dO) with respect to the shared K and V
    (each element feeds several query heads) and to Q."""
    q, k, v, do = _gqa_inputs(B=1, H=4, H_kv=2, n=4, d=3, dv=2)
    scale, hstep = 0.8, 1e-6
    dq, dk, dv = oracle.backward_gqa(q, k, v, do, scale, causal)

    def loss(qq, kk, vv):
        o, _ = oracle.forward_gqa(qq, kk, vv, scale, causal)
        return float((o * do).sum())

    for which, (x, g) in enumerate(zip((q, k, v), (dq, dk, dv))):
        fd = np.zeros_like(x)
        for idx in np.ndindex(*x.shape):
            xp, xm = x.copy(), x.copy()
            xp[idx] += hstep
            xm[idx] -= hstep
            ap, am = [q, k, v], [q, k, v]
            ap[which], am[which] = xp, xm
            fd[idx] = (loss(*ap) - loss(*am)) / (2 * hstep)
        np.testing.assert_allclose(g, fd, rtol=0, atol=1e-7, err_msg="qkv"[which])


def test_gqa_query_head_order_within_a_group():
    """Swapping two query heads of one group swaps their outputs and dQ and leaves
    the shared dK, dV unchanged."""
    q, k, v, do = _gqa_inputs(H=4, H_kv=2)
    perm = [1, 0, 2, 3]
    o, _ = oracle.forward_gqa(q, k, v, 0.5, True)
    o2, _ = oracle.forward_gqa(q[:, perm], k, v, 0.5, True)
    np.testing.assert_allclose(o2, o[:, perm], atol=1e-14)
    g = oracle.backward_gqa(q, k, v, do, 0.5, True)
    g2 = oracle.backward_gqa(q[:, perm], k, v, do[:, perm], 0.5, True)
    np.testing.assert_allclose(g2[0], g[0][:, perm], atol=1e-13)
    np.testing.assert_allclose(g2[1], g[1], atol=1e-13)
    np.testing.assert_allclose(g2[2], g[2], atol=1e-13)


def test_gqa_rejects_uneven_groups():
    q, k, v, _ = _gqa_inputs(H=6, H_kv=4)
    with pytest.raises(ValueError):
        oracle.forward_gqa(q, k, v, 0.5, False)


# ----------------------------------------------------------- variable-length batches


def _varlen_inputs(lens=(3, 0, 5, 1), H=4, H_kv=2, d=3, dv=4, seed=21, extra=0):
    """Packed [H, total, d] inputs for the given sequence lengths (plus ``extra``
    trailing rows that belong to no sequence)."""
    r = np.random.default_rng(seed)
    cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
    total = int(cu[-1]) + extra
    return (cu, r.standard_normal((H, total, d)), r.standard_normal((H_kv, total, d)),
            r.standard_normal((H_kv, total, dv)), r.standard_normal((H, total, dv)))


@pytest.mark.parametrize("causal", [False, True])
def test_varlen_equal_lengths_is_the_padded_batch(causal):
    """B sequences of one length N packed head-major are the [B, H, N, d] batch."""
    B, H, H_kv, N = 3, 4, 2, 6
    cu, q, k, v, do = _varlen_inputs(lens=(N,) * B, H=H, H_kv=H_kv)
    to_batch = lambda x: x.reshape(x.shape[0], B, N, x.shape[-1]).transpose(1, 0, 2, 3)
    o, lse = oracle.forward_varlen(q, k, v, cu, N, 0.7, causal)
    ob, lseb = oracle.forward_gqa(to_batch(q), to_batch(k), to_batch(v), 0.7, causal)
    np.testing.assert_allclose(to_batch(o), ob, rtol=0, atol=1e-14)
    np.testing.assert_allclose(lse, lseb, rtol=0, atol=1e-14)
    g = oracle.backward_varlen(q, k, v, do, cu, N, 0.7, causal)
    gb = oracle.backward_gqa(to_batch(q), to_batch(k), to_batch(v), to_batch(do), 0.7, causal)
    for x, y in zip(g, gb):
        np.testing.assert_allclose(to_batch(x), y, rtol=0, atol=1e-13)


@pytest.mark.parametrize("causal", [False, True])
def test_varlen_is_block_diagonal_attention(causal):
    """The packed batch equals one attention over all packed tokens in which
    token t sees token u only inside its own sequence (and u <= t if causal):
    a mask-based formulation with no per-sequence slicing."""
    cu, q, k, v, _ = _varlen_inputs(lens=(3, 0, 5, 1, 4), H=2, H_kv=1)
    total = q.shape[1]
    seq = np.searchsorted(cu, np.arange(total), side="right") - 1
    pos = np.arange(total)
    visible = seq[:, None] == seq[None, :]
    if causal:
        visible &= pos[None, :] <= pos[:, None]
    o, lse = oracle.forward_varlen(q, k, v, cu, 5, 0.9, causal)
    for h in range(2):
        s = np.where(visible, 0.9 * q[h] @ k[0].T, -np.inf)
        m = s.max(axis=1, keepdims=True)
        e = np.exp(s - m)
        p = e / e.sum(axis=1, keepdims=True)
        np.testing.assert_allclose(o[h], p @ v[0], rtol=0, atol=1e-13)
        ref_lse = (m[:, 0] + np.log(e.sum(axis=1)))
        for b in range(len(cu) - 1):
            n = cu[b + 1] - cu[b]
            np.testing.assert_allclose(lse[b, h, :n], ref_lse[cu[b]:cu[b + 1]], atol=1e-13)
            assert np.isnan(lse[b, h, n:]).all()


def test_varlen_sequences_do_not_interact():
    """Changing every input of one sequence changes no output or gradient of
    another sequence."""
    cu, q, k, v, do = _varlen_inputs(lens=(4, 3, 5))
    base = oracle.forward_varlen(q, k, v, cu, 5, 0.5, True)
    gbase = oracle.backward_varlen(q, k, v, do, cu, 5, 0.5, True)
    s0, s1 = cu[1], cu[2]
    q2, k2, v2, do2 = q.copy(), k.copy(), v.copy(), do.copy()
    for x in (q2, k2, v2, do2):
        x[:, s0:s1] = np.random.default_rng(5).standard_normal(x[:, s0:s1].shape)
    o2, lse2 = oracle.forward_varlen(q2, k2, v2, cu, 5, 0.5, True)
    g2 = oracle.backward_varlen(q2, k2, v2, do2, cu, 5, 0.5, True)
    keep = np.r_[0:s0, s1:q.shape[1]]
    np.testing.assert_array_equal(o2[:, keep], base[0][:, keep])
    np.testing.assert_array_equal(lse2[[0, 2]], base[1][[0, 2]])
    assert not np.allclose(o2[:, s0:s1], base[0][:, s0:s1])
    for x, y in zip(g2, gbase):
        np.testing.assert_array_equal(x[:, keep], y[:, keep])


@pytest.mark.parametrize("causal", [False, True])
def test_varlen_zero_query(causal):
    """Q = 0: each row is the mean of the visible V rows of its own sequence and
    LSE = ln(number visible); empty sequences and unowned rows are untouched."""
    cu, _, k, v, _ = _varlen_inputs(lens=(3, 0, 5, 1), extra=2)
    q = np.zeros((4,) + k.shape[1:])
    o, lse = oracle.forward_varlen(q, k, v, cu, 6, 0.4, causal)
    for b in range(4):
        for h in range(4):
            for i in range(cu[b + 1] - cu[b]):
                vis = i + 1 if causal else cu[b + 1] - cu[b]
                np.testing.assert_allclose(o[h, cu[b] + i], v[h // 2, cu[b]:cu[b] + vis].mean(axis=0),
                                           atol=1e-13)
                np.testing.assert_allclose(lse[b, h, i], math.log(vis), atol=1e-13)
    assert np.isnan(lse[1]).all() and np.isnan(o[:, cu[-1]:]).all()


@pytest.mark.parametrize("causal", [False, True])
def test_varlen_finite_differences(causal):
    """Central differences of L = sum(O * dO) over every packed input element,
    with an empty sequence and a row that belongs to no sequence (gradient 0)."""
    cu, q, k, v, do = _varlen_inputs(lens=(2, 0, 3), H=2, H_kv=1, d=2, dv=2, extra=1)
    scale, hstep = 0.8, 1e-6
    dq, dk, dv = oracle.backward_varlen(q, k, v, do, cu, 3, scale, causal)

    def loss(qq, kk, vv):
        o, _ = oracle.forward_varlen(qq, kk, vv, cu, 3, scale, causal)
        return float(np.nansum(o * do))

    for which, (x, g) in enumerate(zip((q, k, v), (dq, dk, dv))):
        fd = np.zeros_like(x)
        for idx in np.ndindex(*x.shape):
            xp, xm = x.copy(), x.copy()
            xp[idx] += hstep
            xm[idx] -= hstep
            ap, am = [q, k, v], [q, k, v]
            ap[which], am[which] = xp, xm
            fd[idx] = (loss(*ap) - loss(*am)) / (2 * hstep)
        owned = np.nan_to_num(g, nan=0.0)
        np.testing.assert_allclose(owned, fd, rtol=0, atol=1e-7, err_msg="qkv"[which])
        assert np.isnan(g[:, -1]).all()


def test_varlen_rejects_bad_offsets():
    cu, q, k, v, _ = _varlen_inputs(lens=(3, 4))
    for bad, max_s in (([1, 3, 7], 4), ([0, 4, 3], 4), ([0, 3, 8], 5), ([0, 3, 7], 3)):
        with pytest.raises(ValueError):
            oracle.forward_varlen(q, k, v, np.array(bad), max_s, 0.5, False)


# ----------------------------------------------------------- local windows


def _win_inputs(n=9, d=3, dv=2, seed=31):
    r = np.random.default_rng(seed)
    return (r.standard_normal((n, d)), r.standard_normal((n, d)), r.standard_normal((n, dv)),
            r.standard_normal((n, dv)))


@pytest.mark.parametrize("causal", [False, True])
def test_window_wider_than_the_sequence_changes_nothing(causal):
    q, k, v, do = _win_inputs()
    o, lse = oracle.forward_head(q, k, v, 0.7, causal)
    for window in ((-1, -1), (None, None), (8, 8), (100, 3 if causal else 100)):
        o2, lse2 = oracle.forward_head(q, k, v, 0.7, causal, window)
        np.testing.assert_array_equal(o2, o)
        np.testing.assert_array_equal(lse2, lse)


def test_window_of_one_key_is_the_value_row():
    """Window (0, 0): each query sees only its own key, so O_i = v_i exactly and
    LSE_i = scale q_i . k_i; dQ and dK vanish (a softmax over one key is constant)."""
    q, k, v, do = _win_inputs()
    o, lse = oracle.forward_head(q, k, v, 0.7, False, (0, 0))
    np.testing.assert_allclose(o, v, rtol=0, atol=1e-15)
    np.testing.assert_allclose(lse, 0.7 * (q * k).sum(axis=1), rtol=0, atol=1e-14)
    g = oracle.backward_head(q, k, v, do, 0.7, False, (0, 0))
    np.testing.assert_allclose(g["dv"], do, atol=1e-15)
    assert np.abs(g["dq"]).max() < 1e-14 and np.abs(g["dk"]).max() < 1e-14


@pytest.mark.parametrize("W", [1, 2, 4])
def test_sliding_window_brute_force(W):
    """The most recent W keys (causal, left = W - 1), written as a per-row loop over
    an explicit key list with math.exp: no mask matrix, no numpy softmax."""
    q, k, v, _ = _win_inputs(n=7)
    o, lse = oracle.forward_head(q, k, v, 0.8, True, (W - 1, -1))
    for i in range(7):
        keys = list(range(max(0, i - W + 1), i + 1))
        sc = [0.8 * sum(q[i, t] * k[j, t] for t in range(3)) for j in keys]
        mx = max(sc)
        w = [math.exp(x - mx) for x in sc]
        tot = sum(w)
        for c in range(2):
            assert abs(o[i, c] - sum(wj * v[j, c] for wj, j in zip(w, keys)) / tot) < 1e-13
        assert abs(lse[i] - (mx + math.log(tot))) < 1e-13


@pytest.mark.parametrize("left,right", [(2, 2), (3, 1), (0, 4), (5, 0)])
def test_local_window_zero_query(left, right):
    """Q = 0: row i is the mean of v over keys max(0, i - left) .. min(n - 1, i + right)
    and LSE = ln(their number); an asymmetric window pins which side is which."""
    _, k, v, _ = _win_inputs(n=10)
    o, lse = oracle.forward_head(np.zeros((10, 3)), k, v, 0.5, False, (left, right))
    for i in range(10):
        lo, hi = max(0, i - left), min(9, i + right)
        np.testing.assert_allclose(o[i], v[lo:hi + 1].mean(axis=0), atol=1e-14)
        np.testing.assert_allclose(lse[i], math.log(hi - lo + 1), atol=1e-14)


def test_window_cell_count_matches_the_page():
    """The efficiency page counts N = 4096 with a 512-wide window (256 on each side) as
    4096 x 512 = 2,097,152 cells, one eighth of full attention; the mask's count
    differs from that only by the rows whose window is cut at the sequence ends."""
    n, half = 4096, 256
    cells = int(oracle.window_visible(n, n, (half, half - 1)).sum())
    edge = half * (half + 1) // 2 + half * (half - 1) // 2   # keys cut at both ends
    assert cells == n * 2 * half - edge
    assert abs(cells / (n * n) - 1 / 8) < 0.01


@pytest.mark.parametrize("causal,window", [(False, (2, 1)), (True, (2, -1)), (False, (0, 3))])
def test_window_finite_differences(causal, window):
    q, k, v, do = _win_inputs(n=6, d=2, dv=2)
    scale, hstep = 0.9, 1e-6
    g = oracle.backward_head(q, k, v, do, scale, causal, window)

    def loss(qq, kk, vv):
        return float((oracle.forward_head(qq, kk, vv, scale, causal, window)[0] * do).sum())

    for which, (x, gg) in enumerate(zip((q, k, v), (g["dq"], g["dk"], g["dv"]))):
        fd = np.zeros_like(x)
        for idx in np.ndindex(*x.shape):
            xp, xm = x.copy(), x.copy()
            xp[idx] += hstep
            xm[idx] -= hstep
            ap, am = [q, k, v], [q, k, v]
            ap[which], am[which] = xp, xm
            fd[idx] = (loss(*ap) - loss(*am)) / (2 * hstep)
        np.testing.assert_allclose(gg, fd, rtol=0, atol=1e-7, err_msg="qkv"[which])


# ----------------------------------------------------------- dropout


def test_philox_known_answers():
    """Philox4x32-10 against the generator's published known-answer vectors."""
    from oracle import philox
    path = __import__("os").path.join(__import__("os").path.dirname(__file__), "golden",
                                      "philox4x32_10_kat.txt")
    rows = [l.split() for l in open(path) if l.strip() and not l.startswith("#")]
    assert len(rows) == 3
    for r in rows:
        v = [int(x, 16) for x in r]
        out = philox.philox4x32(*v[:4], v[4], v[5])
        assert [int(x) for x in out] == v[6:], r


def test_uniform_layout_of_one_call():
    """One call (query i, group g, parity p) feeds keys 16 g + p + 2 t, t = 0..7, with
    its eight 16-bit halves in order (low half of word 0 first)."""
    from oracle import philox
    u = philox.uniforms16(5, 4, 48, seed=0x1234_5678_9abc_def0, offset=77)
    for i, g, par in ((0, 0, 0), (3, 2, 1), (2, 1, 0)):
        w = philox.philox4x32(i, 2 * g + par, 5, 77, 0x9abcdef0, 0x12345678)
        halves = []
        for x in w:
            halves += [int(x) & 0xFFFF, int(x) >> 16]
        assert [int(u[i, 16 * g + par + 2 * t]) for t in range(8)] == halves


def test_keep_rate_and_uniformity():
    """Over 2^20 draws the keep fraction is within 5 sigma of threshold / 2^16, and the
    16-bit uniforms fill 16 equal bins evenly (chi-square below 50 at 15 dof)."""
    from oracle import philox
    u = philox.uniforms16(3, 1024, 1024, seed=42, offset=0).astype(np.int64)
    for p in (0.1, 0.5, 0.9):
        t = philox.keep_threshold(p)
        rate = (u < t).mean()
        q = t / 65536
        assert abs(rate - q) < 5 * math.sqrt(q * (1 - q) / u.size), (p, rate, q)
    hist = np.bincount(u.reshape(-1) >> 12, minlength=16)
    exp = u.size / 16
    assert ((hist - exp) ** 2 / exp).sum() < 50


def test_masks_depend_on_head_seed_and_offset():
    from oracle import philox
    base = philox.keep_mask(1, 64, 64, 0.5, 9, 0)
    assert np.array_equal(base, philox.keep_mask(1, 64, 64, 0.5, 9, 0))
    for other in (philox.keep_mask(2, 64, 64, 0.5, 9, 0), philox.keep_mask(1, 64, 64, 0.5, 10, 0),
                  philox.keep_mask(1, 64, 64, 0.5, 9, 1), philox.keep_mask(1, 64, 64, 0.5, 9 + (1 << 32), 0)):
        assert 0.4 < (other != base).mean() < 0.6


@pytest.mark.parametrize("causal", [False, True])
def test_dropout_probability_zero_is_no_dropout(causal):
    q, k, v, do = _gqa_inputs(H=4, H_kv=2, n=9)
    o, lse = oracle.forward_gqa(q, k, v, 0.6, causal)
    o2, lse2 = oracle.forward_gqa(q, k, v, 0.6, causal, dropout=(0.0, 5, 0))
    np.testing.assert_array_equal(o, o2)
    np.testing.assert_array_equal(lse, lse2)
    for a, b in zip(oracle.backward_gqa(q, k, v, do, 0.6, causal),
                    oracle.backward_gqa(q, k, v, do, 0.6, causal, dropout=(0.0, 5, 0))):
        np.testing.assert_array_equal(a, b)


def test_dropout_zero_query_closed_form():
    """Q = 0, causal: row i averages the i + 1 visible rows of V, so with dropout it is
    (scale / (i + 1)) times the sum of the kept visible rows; LSE = ln(i + 1)."""
    _, k, v, _ = _win_inputs(n=12)
    from oracle import philox
    p_drop, seed, offset, hd = 0.3, 123, 4, 7
    mask = philox.keep_mask(hd, 12, 12, p_drop, seed, offset)
    sc = 65536.0 / philox.keep_threshold(p_drop)
    o, lse = oracle.forward_head(np.zeros((12, 3)), k, v, 0.5, True, drop=(mask, sc))
    for i in range(12):
        want = sc / (i + 1) * v[:i + 1][mask[i, :i + 1]].sum(axis=0)
        np.testing.assert_allclose(o[i], want, atol=1e-14)
        assert abs(lse[i] - math.log(i + 1)) < 1e-14


def test_dropout_is_unbiased():
    """Averaged over 400 seeds, dropout(P) V approaches P V (the scale is the inverse
    keep probability): the mean error shrinks like 1 / sqrt(seeds)."""
    q, k, v, _ = _win_inputs(n=8)
    o_ref, _ = oracle.forward_head(q, k, v, 0.9, False)
    acc = np.zeros_like(o_ref)
    from oracle import philox
    n = 400
    for seed in range(n):
        mask = philox.keep_mask(0, 8, 8, 0.5, seed, 0)
        acc += oracle.forward_head(q, k, v, 0.9, False, drop=(mask, 2.0))[0]
    err = np.abs(acc / n - o_ref).max()
    assert err < 4 * np.abs(v).max() / math.sqrt(n)


@pytest.mark.parametrize("causal", [False, True])
def test_dropout_finite_differences(causal):
    """With the mask fixed, the gradients of sum(O * dO) match central differences,
    and D = rowsum(dO * O) (the dropped O) equals rowsum(P * dP)."""
    from oracle import philox
    q, k, v, do = _win_inputs(n=6, d=2, dv=2)
    mask = philox.keep_mask(3, 6, 6, 0.4, 99, 1)
    drop = (mask, 65536.0 / philox.keep_threshold(0.4))
    scale, hstep = 0.9, 1e-6
    g = oracle.backward_head(q, k, v, do, scale, causal, drop=drop)
    o, _ = oracle.forward_head(q, k, v, scale, causal, drop=drop)
    np.testing.assert_allclose(g["D"], (do * o).sum(axis=1), atol=1e-13)

    def loss(qq, kk, vv):
        return float((oracle.forward_head(qq, kk, vv, scale, causal, drop=drop)[0] * do).sum())

    for which, (x, gg) in enumerate(zip((q, k, v), (g["dq"], g["dk"], g["dv"]))):
        fd = np.zeros_like(x)
        for idx in np.ndindex(*x.shape):
            xp, xm = x.copy(), x.copy()
            xp[idx] += hstep
            xm[idx] -= hstep
            ap, am = [q, k, v], [q, k, v]
            ap[which], am[which] = xp, xm
            fd[idx] = (loss(*ap) - loss(*am)) / (2 * hstep)
        np.testing.assert_allclose(gg, fd, rtol=0, atol=1e-7, err_msg="qkv"[which])


# ----------------------------------------------------------- block-sparse masks


def test_full_block_mask_changes_nothing():
    q, k, v, do = _win_inputs(n=300)
    o, lse = oracle.forward_head(q, k, v, 0.5, True)
    o2, lse2 = oracle.forward_head(q, k, v, 0.5, True, blocks=np.ones((2, 3)))
    np.testing.assert_array_equal(o, o2)
    np.testing.assert_array_equal(lse, lse2)


@pytest.mark.parametrize("causal", [False, True])
def test_block_diagonal_mask_is_a_packed_batch(causal):
    """Query block b sees key blocks 2 b and 2 b + 1 only (256 queries x 2 x 128 keys):
    exactly a packed batch of sequences of 256 tokens, a formulation by slicing."""
    r = np.random.default_rng(3)
    n, H = 768, 2
    q, k, v, do = (r.standard_normal((1, H, n, 3)) for _ in range(4))
    bm = np.zeros((1, 3, 6), dtype=np.uint8)
    for b in range(3):
        bm[0, b, 2 * b:2 * b + 2] = 1
    o, lse = oracle.forward_gqa(q, k, v, 0.7, causal, block_mask=bm)
    ov, lsev = oracle.forward_varlen(q[0], k[0], v[0], [0, 256, 512, 768], 256, 0.7, causal)
    np.testing.assert_allclose(o[0], ov, rtol=0, atol=1e-13)
    for b in range(3):
        np.testing.assert_allclose(lse[0, :, 256 * b:256 * b + 256], lsev[b], rtol=0, atol=1e-13)
    g = oracle.backward_gqa(q, k, v, do, 0.7, causal, block_mask=bm)
    gv = oracle.backward_varlen(q[0], k[0], v[0], do[0], [0, 256, 512, 768], 256, 0.7, causal)
    for x, y in zip(g, gv):
        np.testing.assert_allclose(x[0], y, rtol=0, atol=1e-12)


def test_block_mask_empty_rows_and_zero_query():
    """A query block with no kept key block: O = 0, LSE = -inf, no gradient; the
    other rows with Q = 0 average V over exactly the kept key blocks."""
    r = np.random.default_rng(4)
    n = 300
    k, v, do = (r.standard_normal((n, 3)) for _ in range(3))
    blocks = np.array([[1, 0, 1], [0, 0, 0]])
    o, lse = oracle.forward_head(np.zeros((n, 3)), k, v, 0.5, False, blocks=blocks)
    keep = np.r_[0:128, 256:300]
    np.testing.assert_allclose(o[:256], np.broadcast_to(v[keep].mean(axis=0), (256, 3)), atol=1e-14)
    np.testing.assert_allclose(lse[:256], math.log(len(keep)), atol=1e-14)
    assert (o[256:] == 0).all() and np.isneginf(lse[256:]).all()
    g = oracle.backward_head(r.standard_normal((n, 3)), k, v, do, 0.5, False, blocks=blocks)
    assert (g["dq"][256:] == 0).all()
    assert (g["dk"][128:256] == 0).all() and (g["dv"][128:256] == 0).all()


def test_block_mask_finite_differences():
    r = np.random.default_rng(5)
    n = 260
    q, k, v, do = (r.standard_normal((n, 2)) for _ in range(4))
    blocks = np.array([[1, 0, 1], [0, 1, 1]])
    scale, hstep = 0.9, 1e-6
    g = oracle.backward_head(q, k, v, do, scale, True, blocks=blocks)

    def loss(qq, kk, vv):
        return float((oracle.forward_head(qq, kk, vv, scale, True, blocks=blocks)[0] * do).sum())

    for which, (x, gg) in enumerate(zip((q, k, v), (g["dq"], g["dk"], g["dv"]))):
        idxs = [(i, c) for i in (0, 5, 127, 128, 200, 255, 256, 259) for c in range(2)]
        for idx in idxs:
            xp, xm = x.copy(), x.copy()
            xp[idx] += hstep
            xm[idx] -= hstep
            ap, am = [q, k, v], [q, k, v]
            ap[which], am[which] = xp, xm
            fd = (loss(*ap) - loss(*am)) / (2 * hstep)
            assert abs(gg[idx] - fd) < 1e-6, ("qkv"[which], idx, gg[idx], fd)


# ----------------------------------------------------------- dropout with a block mask


def test_dropout_with_block_mask_reduces_to_each_alone():
    """With both, the block mask hides keys before the softmax and dropout acts on
    the resulting P: a full block mask gives dropout alone, no dropped element
    (p = 0) gives the block mask alone, and the kept P of a block-masked row is
    exactly the block-masked P with the dropped elements zeroed and the rest
    scaled by 1 / keep."""
    from oracle import philox
    q, k, v, do = _win_inputs(n=300)
    blocks = np.array([[1, 0, 1], [0, 1, 1]])
    mask = philox.keep_mask(5, 300, 300, 0.3, 77, 2)
    sc = 65536.0 / philox.keep_threshold(0.3)
    drop = (mask, sc)
    o_d, lse_d = oracle.forward_head(q, k, v, 0.6, False, drop=drop)
    o_fd, lse_fd = oracle.forward_head(q, k, v, 0.6, False, drop=drop, blocks=np.ones((2, 3)))
    np.testing.assert_array_equal(o_d, o_fd)
    np.testing.assert_array_equal(lse_d, lse_fd)
    o_b, lse_b = oracle.forward_head(q, k, v, 0.6, False, blocks=blocks)
    keep_all = (np.ones((300, 300), dtype=bool), 1.0)
    o_b0, _ = oracle.forward_head(q, k, v, 0.6, False, drop=keep_all, blocks=blocks)
    np.testing.assert_allclose(o_b0, o_b, rtol=0, atol=1e-14)
    # O of the combination = (block-masked P, then dropped and scaled) V, by hand.
    s = 0.6 * q @ k.T
    vis = oracle.block_visible(300, 300, blocks)
    s = np.where(vis, s, -np.inf)
    m = s.max(axis=1, keepdims=True)
    p = np.exp(s - m)
    p /= p.sum(axis=1, keepdims=True)
    o_both, lse_both = oracle.forward_head(q, k, v, 0.6, False, drop=drop, blocks=blocks)
    np.testing.assert_allclose(o_both, (np.where(mask, p * sc, 0.0)) @ v, rtol=0, atol=1e-12)
    np.testing.assert_array_equal(lse_both, lse_b)


def test_dropout_with_block_mask_finite_differences():
    """Gradients with both a block mask and a (fixed) dropout mask match central
    differences, at block edges, and D = rowsum(dO * O) holds."""
    from oracle import philox
    r = np.random.default_rng(6)
    n = 260
    q, k, v, do = (r.standard_normal((n, 2)) for _ in range(4))
    blocks = np.array([[1, 0, 1], [0, 1, 1]])
    drop = (philox.keep_mask(2, n, n, 0.25, 31, 4), 65536.0 / philox.keep_threshold(0.25))
    scale, hstep = 0.9, 1e-6
    g = oracle.backward_head(q, k, v, do, scale, True, drop=drop, blocks=blocks)
    o, _ = oracle.forward_head(q, k, v, scale, True, drop=drop, blocks=blocks)
    np.testing.assert_allclose(g["D"], (do * o).sum(axis=1), atol=1e-12)

    def loss(qq, kk, vv):
        return float((oracle.forward_head(qq, kk, vv, scale, True, drop=drop, blocks=blocks)[0]
                      * do).sum())

    for which, (x, gg) in enumerate(zip((q, k, v), (g["dq"], g["dk"], g["dv"]))):
        for idx in [(i, c) for i in (0, 5, 127, 128, 200, 255, 256, 259) for c in range(2)]:
            xp, xm = x.copy(), x.copy()
            xp[idx] += hstep
            xm[idx] -= hstep
            ap, am = [q, k, v], [q, k, v]
            ap[which], am[which] = xp, xm
            fd = (loss(*ap) - loss(*am)) / (2 * hstep)
            assert abs(gg[idx] - fd) < 1e-6, ("qkv"[which], idx, gg[idx], fd)
