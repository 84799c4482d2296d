"""Parity of dropout (fa_fwd_ex / fa_bwd_ex with dropout_p > 0) with the fp64 oracle
on the GPU, through the C ABI.  The oracle builds the keep mask from its own
Philox4x32-10; besides the tolerance checks, two tests read every keep bit off
the outputs (the forward's and the dK/dV kernel's, which generate the mask in
different lane layouts) and require them to equal the oracle's bit for bit."""
import numpy as np
import pytest
import torch

import oracle
import workloads
from oracle import philox
from tests.test_parity import TOL, f64, rel_err, say
from tests.tolerances import o_bound

pytestmark = pytest.mark.gpu

DEV = "cuda:0"


@pytest.fixture(scope="module")
def fa():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import io_aware_exact_fa_amd
    return io_aware_exact_fa_amd


def p32(p):
    """The dropout probability as the ABI's float carries it."""
    return float(np.float32(p))


def o_tol(dtype, o_ref):
    """The O bound scaled to the binade of the largest output (dropout's 1 / keep
    scaling lets |O| reach past 4; tests/tolerances.py)."""
    return o_bound(dtype, o_ref)


@pytest.mark.parametrize("dtype", ["bf16", "f16", "f32"])
@pytest.mark.parametrize("d", [64, 128])
def test_keep_bits_exact(fa, dtype, d):
    """N = 128, Q = 0, no mask: P = 1/128 everywhere.  With V = [I; 0] and [0; I]
    (identity over 64 keys) O[i, c] = Z[i, key] * scale / 128, and with dO = [I; 0]
    and [0; I] dV[key, c] = Z[query, key] * scale / 128: every keep bit of both the
    forward and the dK/dV kernel, compared with the oracle's mask (two heads, two
    batch entries: the head index enters the counter)."""
    B, H, N = 2, 2, 128
    pd, seed, off = p32(0.3), 0xABCDEF0123, 5
    dt = {"bf16": torch.bfloat16, "f16": torch.float16, "f32": torch.float32}[dtype]
    q = torch.zeros((B, H, N, d), dtype=dt, device=DEV)
    k = workloads.make_random((B, H, N, d), dtype, 7).to(DEV)
    sc = 65536.0 / philox.keep_threshold(pd)
    for half in range(2):
        v = torch.zeros((B, H, N, d), dtype=dt)
        v[:, :, 64 * half:64 * half + 64, :64] = torch.eye(64, dtype=dt)
        v = v.to(DEV)
        o, lse = fa.forward(q, k, v, False, 0.125, dropout=(pd, seed, off))
        do = v.clone()   # [I; 0] or [0; I] over queries
        dq, dk, dv = fa.backward(q, k, v, o, do, lse, False, 0.125, dropout=(pd, seed, off))
        torch.cuda.synchronize()
        for b in range(B):
            for h in range(H):
                want = philox.keep_mask(b * H + h, N, N, pd, seed, off)
                got_fwd = f64(o[b, h, :, :64]) > 0.5 * sc / N
                assert np.array_equal(got_fwd, want[:, 64 * half:64 * half + 64]), (b, h, half)
                got_bwd = f64(dv[b, h, :, :64]) > 0.5 * sc / N   # dV[key, query - 64 half]
                assert np.array_equal(got_bwd, want[64 * half:64 * half + 64, :].T), (b, h, half)
    say(f"keep bits exact ({dtype}, d = {d})")


def cases():
    for dtype in ("bf16", "f16", "f32"):
        for d in (64, 128):
            for causal in (False, True):
                yield dtype, d, causal


@pytest.mark.parametrize("dtype,d,causal", list(cases()))
def test_dropout_small(fa, dtype, d, causal):
    """N = 300 (several tiles, ragged tail), 4 query heads over 2 K/V heads, p = 0.25;
    every element against the oracle."""
    w = workloads.Workload(f"drop-{dtype}-d{d}", 2, 4, 300, d, dtype, causal, 111 + d, H_kv=2)
    inp = workloads.make_inputs(w)
    drop = (p32(0.25), 0x1234_5678_9ABC + d, 3)
    say(f"case {w.name} causal={causal}")
    qd, kd, vd, dod = (inp[n].to(DEV) for n in ("q", "k", "v", "do"))
    o, lse = fa.forward(qd, kd, vd, causal, w.scale, dropout=drop)
    dq, dk, dv = fa.backward(qd, kd, vd, o, dod, lse, causal, w.scale, dropout=drop)
    torch.cuda.synchronize()
    tol = TOL[dtype]
    q, k, v, do = (f64(inp[n]) for n in ("q", "k", "v", "do"))
    o_ref, lse_ref = oracle.forward_gqa(q, k, v, w.scale, causal, dropout=drop)
    g_ref = oracle.backward_gqa(q, k, v, do, w.scale, causal, dropout=drop)
    err_o = float(np.max(np.abs(f64(o) - o_ref)))
    err_l = float(np.max(np.abs(f64(lse) - lse_ref)))
    errs = [rel_err(f64(x), r) for x, r in zip((dq, dk, dv), g_ref)]
    say(f"  O {err_o:.3e} (tol {o_tol(dtype, o_ref):.1e}) LSE {err_l:.3e} dq/dk/dv "
        + " ".join(f"{e:.3e}" for e in errs))
    assert err_o <= o_tol(dtype, o_ref) and err_l <= tol["lse"]
    assert max(errs) <= tol["grad"], errs


def test_dropout_everything(fa):
    """p = 1 drops every element: O = 0 and every gradient 0; LSE is unchanged."""
    w = workloads.Workload("drop-all", 1, 2, 200, 128, "bf16", True, 121)
    inp = workloads.make_inputs(w)
    qd, kd, vd, dod = (inp[n].to(DEV) for n in ("q", "k", "v", "do"))
    o, lse = fa.forward(qd, kd, vd, True, w.scale, dropout=(1.0, 9, 0))
    o0, lse0 = fa.forward(qd, kd, vd, True, w.scale)
    dq, dk, dv = fa.backward(qd, kd, vd, o, dod, lse, True, w.scale, dropout=(1.0, 9, 0))
    torch.cuda.synchronize()
    assert not o.any() and not dq.any() and not dk.any() and not dv.any()
    assert torch.equal(lse, lse0)


@pytest.mark.parametrize("dtype,d", [("bf16", 128), ("f16", 64)])
def test_dropout_packed_and_windowed(fa, dtype, d):
    """Dropout inside packed sequences (positions count from each sequence's start,
    the sequence index enters the counter) together with a causal window."""
    lens = (1, 0, 17, 64, 65, 200, 3, 130)
    w = workloads.Varlen(f"varlen-drop-{dtype}-d{d}", lens, 4, d, dtype, True, 131 + d, H_kv=2)
    inp = workloads.make_varlen_inputs(w)
    drop, window = (p32(0.2), 77, 11), (50, -1)
    q, k, v, do = (inp[n].to(DEV) for n in ("q", "k", "v", "do"))
    cu = inp["cu_seqlens"].to(DEV)
    o, lse = fa.forward_varlen(q, k, v, cu, w.max_s, True, w.scale, window=window, dropout=drop)
    dq, dk, dv = fa.backward_varlen(q, k, v, o, do, lse, cu, w.max_s, True, w.scale,
                                    window=window, dropout=drop)
    torch.cuda.synchronize()
    tol = TOL[dtype]
    qq, kk, vv, dd = (f64(inp[n]) for n in ("q", "k", "v", "do"))
    cun = inp["cu_seqlens"].numpy()
    o_ref, lse_ref = oracle.forward_varlen(qq, kk, vv, cun, w.max_s, w.scale, True, window=window,
                                           dropout=drop)
    g_ref = oracle.backward_varlen(qq, kk, vv, dd, cun, w.max_s, w.scale, True, window=window,
                                   dropout=drop)
    own = ~np.isnan(lse_ref)
    err_o = float(np.nanmax(np.abs(f64(o) - o_ref)))
    err_l = float(np.max(np.abs(f64(lse)[own] - lse_ref[own])))
    errs = [rel_err(f64(x), r) for x, r in zip((dq, dk, dv), g_ref)]
    say(f"  {w.name}: O {err_o:.3e} LSE {err_l:.3e} grads " + " ".join(f"{e:.3e}" for e in errs))
    assert err_o <= o_tol(dtype, o_ref) and err_l <= tol["lse"] and max(errs) <= tol["grad"]


@pytest.mark.parametrize("w", workloads.DROPOUT, ids=lambda w: w.name)
def test_large_dropout_sampled(fa, w):
    """The dropout workload at full size (the launch the benchmark times): the oracle
    on the last head; on every head, sum_j dK_j = 0 (rows of dS still sum to 0)."""
    inp = workloads.make_inputs(w)
    say(f"case {w.name} full size")
    drop = (p32(w.dropout[0]),) + tuple(w.dropout[1:])
    qd, kd, vd, dod = (inp[n].to(DEV) for n in ("q", "k", "v", "do"))
    o, lse = fa.forward(qd, kd, vd, w.causal, w.scale, dropout=drop)
    dq, dk, dv = fa.backward(qd, kd, vd, o, dod, lse, w.causal, w.scale, dropout=drop)
    torch.cuda.synchronize()
    b, h = w.B - 1, w.H - 1
    q, k, v, do = (f64(inp[n][b, h]) for n in ("q", "k", "v", "do"))
    hdrop = oracle.head_drop(drop, b * w.H + h, w.N)
    o_ref, lse_ref = oracle.forward_head(q, k, v, w.scale, w.causal, drop=hdrop)
    g = oracle.backward_head(q, k, v, do, w.scale, w.causal, drop=hdrop)
    tol = TOL[w.dtype]
    err_o = float(np.max(np.abs(f64(o[b, h]) - o_ref)))
    err_l = float(np.max(np.abs(f64(lse[b, h]) - lse_ref)))
    errs = [rel_err(f64(x[b, h]), g[n]) for x, n in zip((dq, dk, dv), ("dq", "dk", "dv"))]
    say(f"  O {err_o:.3e} LSE {err_l:.3e} grads " + " ".join(f"{e:.3e}" for e in errs))
    assert err_o <= o_tol(w.dtype, o_ref) and err_l <= tol["lse"] and max(errs) <= tol["grad"]
    dks = dk.double().sum(dim=2)
    assert dks.abs().max().item() <= 4 * tol["grad"] * dk.double().abs().sum(dim=2).max().item()
