"""Plant plausible mistakes in copies of the oracle and require that a pin catches each.

This shows the pins of ``tests/pins.py`` are strong enough that a dropped term,
a wrong sign or index, or a transposed operand in the oracle would be noticed.
Everything here runs on the CPU.
"""
import numpy as np
import pytest

import oracle
from tests import pins


def _softmax_rows(s, log=np.log):
    m = s.max(axis=1)
    e = np.exp(s - m[:, None])
    l = e.sum(axis=1)
    return e / l[:, None], m + log(l)


def _scores(q, k, scale, causal, mask=lambda i, j: j <= i, use_scale=True):
    s = (scale if use_scale else 1.0) * (np.asarray(q, float) @ np.asarray(k, float).T)
    if causal:
        i = np.arange(s.shape[0])[:, None]
        j = np.arange(s.shape[1])[None, :]
        s = np.where(mask(i, j), s, -np.inf)
    return s


def make_fwd(**kw):
    log = kw.pop("log", np.log)

    def fwd(q, k, v, scale, causal):
        p, lse = _softmax_rows(_scores(q, k, scale, causal, **kw), log=log)
        return p @ np.asarray(v, float), lse
    return fwd


def make_bwd(variant):
    def bwd(q, k, v, do, scale, causal):
        q, k, v, do = (np.asarray(x, float) for x in (q, k, v, do))
        p, _ = _softmax_rows(_scores(q, k, scale, causal))
        dv = p.T @ do
        dp = do @ v.T
        D = (p * dp).sum(axis=1)
        ds = p * (dp - D[:, None])
        dq = scale * (ds @ k)
        dk = scale * (ds.T @ q)
        if variant == "dk_no_transpose":
            dk = scale * (ds @ q)
        elif variant == "dv_no_transpose":
            dv = p @ do
        elif variant == "dq_no_scale":
            dq = ds @ k
        elif variant == "dk_no_scale":
            dk = ds.T @ q
        elif variant == "delta_sign":
            ds = p * (dp + D[:, None])
            dq = scale * (ds @ k)
            dk = scale * (ds.T @ q)
        elif variant == "delta_dropped":
            ds = p * dp
            dq = scale * (ds @ k)
            dk = scale * (ds.T @ q)
        return dq, dk, dv
    return bwd


good_fwd = make_fwd()
good_bwd = make_bwd(None)


def _fails(fn):
    try:
        fn()
    except AssertionError:
        return True
    return False


def forward_pins(fwd):
    return [
        lambda: pins.check_page_cpu_vectors(fwd),
        lambda: pins.check_zero_query(fwd, causal=False),
        lambda: pins.check_zero_query(fwd, causal=True),
        lambda: pins.check_dominant_score(fwd, causal=False),
        lambda: pins.check_dominant_score(fwd, causal=True),
        lambda: pins.check_value_linearity(fwd),
        lambda: pins.check_key_shift(fwd, good_bwd, causal=True),
    ]


def backward_pins(bwd):
    return [
        lambda: pins.check_finite_differences(good_fwd, bwd, causal=False),
        lambda: pins.check_finite_differences(good_fwd, bwd, causal=True),
        lambda: pins.check_zero_query_gradients(bwd, causal=False),
        lambda: pins.check_zero_query_gradients(bwd, causal=True),
    ]


def test_copy_without_mistakes_passes_every_pin():
    for check in forward_pins(good_fwd) + backward_pins(good_bwd):
        check()
    pins.check_single_key(good_fwd, good_bwd)


@pytest.mark.parametrize("name,fwd", [
    ("scale dropped from the scores", make_fwd(use_scale=False)),
    ("mask hides the past instead of the future", make_fwd(mask=lambda i, j: j >= i)),
    ("mask also hides the diagonal", make_fwd(mask=lambda i, j: j < i)),
    ("LSE in base 2", make_fwd(log=np.log2)),
])
@pytest.mark.filterwarnings("ignore::RuntimeWarning")
def test_forward_mistake_is_caught(name, fwd):
    assert any(_fails(c) for c in forward_pins(fwd)), name


@pytest.mark.parametrize("variant", [
    "dk_no_transpose", "dv_no_transpose", "dq_no_scale", "dk_no_scale",
    "delta_sign", "delta_dropped",
])
def test_backward_mistake_is_caught(variant):
    assert any(_fails(c) for c in backward_pins(make_bwd(variant))), variant


def test_real_oracle_agrees_with_unmutated_copy():
    r = np.random.default_rng(3)
    q, k, v, do = (r.standard_normal((9, 5)) for _ in range(4))
    for causal in (False, True):
        o, lse = oracle.forward_head(q, k, v, 0.3, causal)
        o2, lse2 = good_fwd(q, k, v, 0.3, causal)
        np.testing.assert_allclose(o, o2, atol=1e-14)
        np.testing.assert_allclose(lse, lse2, atol=1e-14)
