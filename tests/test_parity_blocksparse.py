"""Parity of block-sparse attention (fa_fwd_ex / fa_bwd_ex with a block mask) with
the fp64 oracle on the GPU, through the C ABI: random masks per head with empty
query blocks, all dtypes and head sizes, causal and not, packed batches, the
equivalence of a block-diagonal mask with a packed batch, block masks together
with dropout, and the full-size workload."""
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


def random_mask(heads, n, density, seed, empty_row=True):
    nbq, nbk = -(-n // 256), -(-n // 128)
    g = torch.Generator(device="cpu").manual_seed(seed)
    m = (torch.rand((heads, nbq, nbk), generator=g) < density).to(torch.uint8)
    if empty_row:
        m[0, nbq - 1, :] = 0   # head 0: the last query block sees nothing
    return m.contiguous()


def check(out, inp, w, bm, causal, tag):
    tol = TOL[w.dtype]
    q, k, v, do = (f64(inp[n]) for n in ("q", "k", "v", "do"))
    o_ref, lse_ref = oracle.forward_gqa(q, k, v, w.scale, causal, block_mask=bm.numpy())
    g_ref = oracle.backward_gqa(q, k, v, do, w.scale, causal, block_mask=bm.numpy())
    err_o = float(np.max(np.abs(f64(out["o"]) - o_ref)))
    fin = np.isfinite(lse_ref)
    lse = f64(out["lse"])
    assert np.array_equal(np.isneginf(lse), ~fin), "empty rows must have LSE = -inf"
    err_l = float(np.max(np.abs(lse[fin] - lse_ref[fin])))
    errs = [rel_err(f64(x), r) for x, r in zip((out["dq"], out["dk"], out["dv"]), g_ref)]
    say(f"  {tag}: O {err_o:.3e} LSE {err_l:.3e} grads " + " ".join(f"{e:.3e}" for e in errs))
    assert err_o <= tol["o"] and err_l <= tol["lse"] and max(errs) <= tol["grad"]


def run(fa, inp, causal, scale, bm, window=None):
    q, k, v, do = (inp[n].to(DEV) for n in ("q", "k", "v", "do"))
    bmd = bm.to(DEV)
    o, lse = fa.forward(q, k, v, causal, scale, window=window, block_mask=bmd)
    dq, dk, dv = fa.backward(q, k, v, o, do, lse, causal, scale, window=window, block_mask=bmd)
    torch.cuda.synchronize()
    return {"o": o, "lse": lse, "dq": dq, "dk": dk, "dv": dv}


def cases():
    for dtype in ("bf16", "f16", "f32"):
        for d in (64, 128):
            for causal in (False, True):
                yield dtype, d, causal


@pytest.mark.parametrize("dtype,d,causal", list(cases()))
def test_block_sparse_small(fa, dtype, d, causal):
    """N = 600 (3 query blocks, 5 key blocks, ragged ends), 4 query heads over 2 K/V
    heads, one random mask per head at density 0.5 (head 0's last query block
    empty)."""
    w = workloads.Workload(f"bs-{dtype}-d{d}", 2, 4, 600, d, dtype, causal, 141 + d, H_kv=2)
    inp = workloads.make_inputs(w)
    bm = random_mask(4, 600, 0.5, 7 + d + causal)
    say(f"case {w.name} causal={causal} density {bm.float().mean().item():.2f}")
    check(run(fa, inp, causal, w.scale, bm), inp, w, bm, causal, w.name)


@pytest.mark.parametrize("dtype", ["bf16", "f16"])
def test_shared_mask_with_window(fa, dtype):
    """One mask for every head, together with a causal window."""
    w = workloads.Workload(f"bs-shared-{dtype}", 1, 4, 700, 128, dtype, True, 151, H_kv=4)
    inp = workloads.make_inputs(w)
    bm = random_mask(1, 700, 0.6, 3, empty_row=False)
    window = (300, -1)
    out = run(fa, inp, True, w.scale, bm, window)
    tol = TOL[dtype]
    q, k, v, do = (f64(inp[n]) for n in ("q", "k", "v", "do"))
    o_ref, lse_ref = oracle.forward_gqa(q, k, v, w.scale, True, window, block_mask=bm.numpy())
    g_ref = oracle.backward_gqa(q, k, v, do, w.scale, True, window, block_mask=bm.numpy())
    fin = np.isfinite(lse_ref)
    err_o = float(np.max(np.abs(f64(out["o"]) - o_ref)))
    err_l = float(np.max(np.abs(f64(out["lse"])[fin] - lse_ref[fin])))
    errs = [rel_err(f64(x), r) for x, r in zip((out["dq"], out["dk"], out["dv"]), g_ref)]
    say(f"  shared+window {dtype}: O {err_o:.3e} LSE {err_l:.3e} " + " ".join(f"{e:.3e}" for e in errs))
    assert err_o <= tol["o"] and err_l <= tol["lse"] and max(errs) <= tol["grad"]


@pytest.mark.parametrize("dtype,d", [("bf16", 128), ("f16", 64), ("bf16", 64)])
def test_block_diagonal_equals_packed_batch(fa, dtype, d):
    """Query block b keeping only key blocks 2 b, 2 b + 1 is a packed batch of
    256-token sequences: the two calls agree to rounding (same tiles, same order)."""
    B, H, N = 1, 4, 768
    w = workloads.Workload(f"bs-diag-{dtype}-d{d}", B, H, N, d, dtype, False, 161 + d, H_kv=2)
    inp = workloads.make_inputs(w)
    bm = torch.zeros((1, 3, 6), dtype=torch.uint8)
    for b in range(3):
        bm[0, b, 2 * b:2 * b + 2] = 1
    out = run(fa, inp, False, w.scale, bm)
    q, k, v, do = (inp[n][0].to(DEV).contiguous() for n in ("q", "k", "v", "do"))
    cu = torch.tensor([0, 256, 512, 768], dtype=torch.int32, device=DEV)
    o, lse = fa.forward_varlen(q, k, v, cu, 256, False, w.scale)
    dq, dk, dv = fa.backward_varlen(q, k, v, o, do, lse, cu, 256, False, w.scale)
    torch.cuda.synchronize()
    tol = TOL[dtype]
    assert (out["o"][0] - o).abs().max().item() <= tol["o"] / 4
    for bb in range(3):
        assert (out["lse"][0, :, 256 * bb:256 * bb + 256] - lse[bb]).abs().max().item() <= tol["lse"] / 4
    for x, y in ((out["dq"][0], dq), (out["dk"][0], dk), (out["dv"][0], dv)):
        assert rel_err(f64(x), f64(y)) <= tol["grad"] / 4


def test_block_sparse_packed(fa):
    """Block masks inside packed sequences (blocks count from each sequence's start)."""
    lens = (300, 0, 17, 520, 129)
    w = workloads.Varlen("bs-varlen", lens, 4, 128, "bf16", False, 171, H_kv=2)
    inp = workloads.make_varlen_inputs(w)
    bm = random_mask(4, w.max_s, 0.6, 9, empty_row=False)
    q, k, v, do = (inp[n].to(DEV) for n in ("q", "k", "v", "do"))
    cu = inp["cu_seqlens"].to(DEV)
    bmd = bm.to(DEV)
    o, lse = fa.forward_varlen(q, k, v, cu, w.max_s, False, w.scale, block_mask=bmd)
    dq, dk, dv = fa.backward_varlen(q, k, v, o, do, lse, cu, w.max_s, False, w.scale, block_mask=bmd)
    torch.cuda.synchronize()
    qq, kk, vv, dd = (f64(inp[n]) for n in ("q", "k", "v", "do"))
    cun = inp["cu_seqlens"].numpy()
    o_ref, lse_ref = oracle.forward_varlen(qq, kk, vv, cun, w.max_s, w.scale, False,
                                           block_mask=bm.numpy())
    g_ref = oracle.backward_varlen(qq, kk, vv, dd, cun, w.max_s, w.scale, False,
                                   block_mask=bm.numpy())
    tol = TOL["bf16"]
    own = np.isfinite(lse_ref)
    err_o = float(np.nanmax(np.abs(f64(o) - o_ref)))
    err_l = float(np.max(np.abs(f64(lse)[own] - lse_ref[own])))
    errs = [rel_err(np.nan_to_num(f64(x)), np.nan_to_num(r)) for x, r in zip((dq, dk, dv), g_ref)]
    say(f"  packed: O {err_o:.3e} LSE {err_l:.3e} " + " ".join(f"{e:.3e}" for e in errs))
    assert err_o <= tol["o"] and err_l <= tol["lse"] and max(errs) <= tol["grad"]


@pytest.mark.parametrize("w", workloads.SPARSE, ids=lambda w: w.name)
def test_large_block_sparse_sampled(fa, w):
    """The block-sparse workload at full size (the launch the benchmark times): the
    oracle on the last head of each batch entry (dq, and dk, dv of that head)."""
    inp = workloads.make_inputs(w)
    bm = workloads.block_mask(w)
    say(f"case {w.name} full size, density {bm.float().mean().item():.3f}")
    out = run(fa, inp, w.causal, w.scale, bm)
    tol = TOL[w.dtype]
    for b in range(w.B):
        h = w.H - 1
        q, k, v, do = (f64(inp[n][b, h]) for n in ("q", "k", "v", "do"))
        o_ref, lse_ref = oracle.forward_head(q, k, v, w.scale, w.causal, blocks=bm[h].numpy())
        g = oracle.backward_head(q, k, v, do, w.scale, w.causal, blocks=bm[h].numpy())
        err_o = float(np.max(np.abs(f64(out["o"][b, h]) - o_ref)))
        err_l = float(np.max(np.abs(f64(out["lse"][b, h]) - lse_ref)))
        errs = [rel_err(f64(out[n][b, h]), g[n]) for n in ("dq", "dk", "dv")]
        say(f"  b{b} h{h}: O {err_o:.3e} LSE {err_l:.3e} " + " ".join(f"{e:.3e}" for e in errs))
        assert err_o <= tol["o"] and err_l <= tol["lse"] and max(errs) <= tol["grad"]


@pytest.mark.parametrize("dtype,d,causal", list(cases()))
def test_block_sparse_with_dropout(fa, dtype, d, causal):
    """A block mask per head (one head with an empty query block) together with
    dropout p = 0.25: the mask hides keys before the softmax, dropout acts on the
    kept P; every element against the oracle.  N = 300, 4 query heads over 2 K/V
    heads, two batch entries."""
    from tests.test_parity_dropout import o_tol, p32
    w = workloads.Workload(f"bsdrop-{dtype}-d{d}", 2, 4, 300, d, dtype, causal, 171 + d, H_kv=2)
    inp = workloads.make_inputs(w)
    bm = random_mask(4, 300, 0.6, 181 + d)
    drop = (p32(0.25), 0x5EED_0000_4242 + d, 5)
    say(f"case {w.name} causal={causal}")
    q, k, v, do = (inp[n].to(DEV) for n in ("q", "k", "v", "do"))
    bmd = bm.to(DEV)
    o, lse = fa.forward(q, k, v, causal, w.scale, dropout=drop, block_mask=bmd)
    dq, dk, dv = fa.backward(q, k, v, o, do, lse, causal, w.scale, dropout=drop, block_mask=bmd)
    torch.cuda.synchronize()
    tol = TOL[dtype]
    qh, kh, vh, doh = (f64(inp[n]) for n in ("q", "k", "v", "do"))
    o_ref, lse_ref = oracle.forward_gqa(qh, kh, vh, w.scale, causal, dropout=drop,
                                        block_mask=bm.numpy())
    g_ref = oracle.backward_gqa(qh, kh, vh, doh, w.scale, causal, dropout=drop,
                                block_mask=bm.numpy())
    fin = np.isfinite(lse_ref)
    lg = f64(lse)
    assert np.array_equal(np.isneginf(lg), ~fin), "empty rows must have LSE = -inf"
    err_o = float(np.max(np.abs(f64(o) - o_ref)))
    err_l = float(np.max(np.abs(lg[fin] - lse_ref[fin])))
    errs = [rel_err(f64(x), r) for x, r in zip((dq, dk, dv), g_ref)]
    say(f"  O {err_o:.3e} (tol {o_tol(dtype, o_ref):.1e}) LSE {err_l:.3e} grads "
        + " ".join(f"{e:.3e}" for e in errs))
    assert err_o <= o_tol(dtype, o_ref) and err_l <= tol["lse"] and max(errs) <= tol["grad"]
