"""Parity of local-window attention (fa_fwd_ex / fa_bwd_ex) with the fp64 oracle on
the GPU, through the C ABI: dense and packed batches, grouped K/V heads, windows
that cut tiles on either side, and bitwise agreement with the plain entry points
when the window covers every key."""
import numpy as np
import pytest
import torch

import oracle
import workloads
from tests.test_parity import TOL, f64, rel_err, say

pytestmark = pytest.mark.gpu

DEV = "cuda:0"


@pytest.fixture(scope="module")
def fa():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import io_aware_exact_fa_amd
    return io_aware_exact_fa_amd


def run_dense(fa, inp, causal, scale, window):
    q, k, v, do = (inp[n].to(DEV) for n in ("q", "k", "v", "do"))
    o, lse = fa.forward(q, k, v, causal, scale, window=window)
    dq, dk, dv = fa.backward(q, k, v, o, do, lse, causal, scale, window=window)
    torch.cuda.synchronize()
    return {"o": o, "lse": lse, "dq": dq, "dk": dk, "dv": dv}


def check_dense(out, inp, causal, scale, dtype, window, tag):
    tol = TOL[dtype]
    q, k, v, do = (f64(inp[n]) for n in ("q", "k", "v", "do"))
    o_ref, lse_ref = oracle.forward_gqa(q, k, v, scale, causal, window)
    dq_ref, dk_ref, dv_ref = oracle.backward_gqa(q, k, v, do, scale, causal, window)
    err_o = float(np.max(np.abs(f64(out["o"]) - o_ref)))
    err_l = float(np.max(np.abs(f64(out["lse"]) - lse_ref)))
    errs = {n: rel_err(f64(out[n]), r) for n, r in (("dq", dq_ref), ("dk", dk_ref), ("dv", dv_ref))}
    say(f"  {tag} O {err_o:.3e} LSE {err_l:.3e} " + " ".join(f"{n} {e:.3e}" for n, e in errs.items()))
    assert err_o <= tol["o"] and err_l <= tol["lse"], (err_o, err_l)
    for n, e in errs.items():
        assert e <= tol["grad"], (n, e)


# (causal, window): one-key windows, windows that cut tiles on both sides, a causal
# sliding window, windows wider than one tile but narrower than the sequence.
WINDOWS = [(False, (0, 0)), (False, (5, 3)), (True, (64, -1)), (True, (100, 7)),
           (False, (-1, 70)), (False, (130, 130)), (True, (1, -1))]


def cases():
    for dtype in ("bf16", "f16", "f32"):
        for d in (64, 128):
            for causal, window in WINDOWS:
                yield dtype, d, causal, window


@pytest.mark.parametrize("dtype,d,causal,window", list(cases()))
def test_windows_small(fa, dtype, d, causal, window):
    """N = 300 (four 64-key tiles and a tail), two batch entries, 4 query heads over 2
    K/V heads; every element against the oracle."""
    w = workloads.Workload(f"win-{dtype}-d{d}", 2, 4, 300, d, dtype, causal,
                           seed=81 + d + window[0] + 3 * window[1], H_kv=2)
    inp = workloads.make_inputs(w)
    say(f"case {w.name} causal={causal} window={window}")
    out = run_dense(fa, inp, causal, w.scale, window)
    check_dense(out, inp, causal, w.scale, dtype, window, w.name)


@pytest.mark.parametrize("dtype", ["bf16", "f16"])
@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("causal", [False, True])
def test_covering_window_is_bitwise_the_plain_call(fa, dtype, d, causal):
    """A window at least as wide as the sequence hides nothing: fa_fwd_ex and fa_bwd_ex
    then run the same tiles as the plain entry points, bit for bit."""
    w = workloads.Workload(f"cover-{dtype}-d{d}", 2, 4, 333, d, dtype, causal, 91 + d, H_kv=2)
    inp = workloads.make_inputs(w)
    say(f"case {w.name} causal={causal}")
    q, k, v, do = (inp[n].to(DEV) for n in ("q", "k", "v", "do"))
    o, lse = fa.forward(q, k, v, causal, w.scale)
    dq, dk, dv = fa.backward(q, k, v, o, do, lse, causal, w.scale)
    for window in ((-1, -1), (333, 400)):
        o2, lse2 = fa.forward(q, k, v, causal, w.scale, window=window)
        dq2, dk2, dv2 = fa.backward(q, k, v, o2, do, lse2, causal, w.scale, window=window)
        torch.cuda.synchronize()
        for a, b in ((o, o2), (lse, lse2), (dq, dq2), (dk, dk2), (dv, dv2)):
            assert torch.equal(a, b), window


@pytest.mark.parametrize("dtype,d", [("bf16", 128), ("f16", 64), ("f32", 128)])
@pytest.mark.parametrize("causal,window", [(True, (40, -1)), (False, (30, 30))])
def test_windows_packed(fa, dtype, d, causal, window):
    """Windows inside packed sequences (positions count from each sequence's start)."""
    lens = (1, 0, 17, 64, 65, 200, 3, 130)
    w = workloads.Varlen(f"varlen-win-{dtype}-d{d}", lens, 4, d, dtype, causal, 101 + d, H_kv=2)
    inp = workloads.make_varlen_inputs(w)
    say(f"case {w.name} causal={causal} window={window}")
    q, k, v, do = (inp[n].to(DEV) for n in ("q", "k", "v", "do"))
    cu = inp["cu_seqlens"].to(DEV)
    o, lse = fa.forward_varlen(q, k, v, cu, w.max_s, causal, w.scale, window=window)
    dq, dk, dv = fa.backward_varlen(q, k, v, o, do, lse, cu, w.max_s, causal, w.scale,
                                    window=window)
    torch.cuda.synchronize()
    out = {"o": o, "lse": lse, "dq": dq, "dk": dk, "dv": dv}
    tol = TOL[dtype]
    qq, kk, vv, dd = (f64(inp[n]) for n in ("q", "k", "v", "do"))
    o_ref, lse_ref = oracle.forward_varlen(qq, kk, vv, inp["cu_seqlens"].numpy(), w.max_s,
                                           w.scale, causal, window=window)
    g_ref = oracle.backward_varlen(qq, kk, vv, dd, inp["cu_seqlens"].numpy(), w.max_s, w.scale,
                                   causal, window=window)
    own = ~np.isnan(lse_ref)
    err_o = float(np.nanmax(np.abs(f64(o) - o_ref)))
    err_l = float(np.max(np.abs(f64(lse)[own] - lse_ref[own])))
    say(f"  O {err_o:.3e} LSE {err_l:.3e}")
    assert err_o <= tol["o"] and err_l <= tol["lse"]
    for n, r in zip(("dq", "dk", "dv"), g_ref):
        e = rel_err(np.nan_to_num(f64(out[n]) * (~np.isnan(r))), np.nan_to_num(r))
        say(f"  {n} {e:.3e}")
        assert e <= tol["grad"], (n, e)


@pytest.mark.parametrize("w", workloads.WINDOWED, ids=lambda w: w.name)
def test_large_window_sampled(fa, w):
    """The sliding-window workload at full size (the launch the benchmark times): the
    oracle on the last query head of each batch entry and the gradients of its K/V
    head; on every head, sum_j dV_j = sum_i dO_i and sum_j dK_j = 0."""
    inp = workloads.make_inputs(w)
    say(f"case {w.name} full size")
    out = run_dense(fa, inp, w.causal, w.scale, w.window)
    tol = TOL[w.dtype]
    G = w.H // w.kv_heads
    for b in range(w.B):
        h = w.H - 1
        j = h // G
        q, k, v, do = (f64(inp[n][b, x]) for n, x in (("q", h), ("k", j), ("v", j), ("do", h)))
        o_ref, lse_ref = oracle.forward_head(q, k, v, w.scale, w.causal, w.window)
        err_o = float(np.max(np.abs(f64(out["o"][b, h]) - o_ref)))
        err_l = float(np.max(np.abs(f64(out["lse"][b, h]) - lse_ref)))
        g = oracle.backward_head(q, k, v, do, w.scale, w.causal, w.window)
        e_dq = rel_err(f64(out["dq"][b, h]), g["dq"])
        say(f"  b{b} h{h}: O {err_o:.3e} LSE {err_l:.3e} dq {e_dq:.3e}")
        assert err_o <= tol["o"] and err_l <= tol["lse"] and e_dq <= tol["grad"]
    dv = out["dv"].double().sum(dim=2)
    dk = out["dk"].double().sum(dim=2)
    do = inp["do"].to(DEV).double().sum(dim=2).reshape(w.B, w.kv_heads, G, w.d).sum(dim=2)
    t4 = 4 * tol["grad"]
    assert (dv - do).abs().max().item() <= t4 * out["dv"].double().abs().sum(dim=2).max().item()
    assert dk.abs().max().item() <= t4 * out["dk"].double().abs().sum(dim=2).max().item()
