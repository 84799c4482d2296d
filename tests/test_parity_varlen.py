"""Parity of the packed variable-length entry points (fa_fwd_varlen, fa_bwd_varlen)
with the fp64 oracle, on the GPU, through the C ABI.  Tolerances as for the dense
path (the same kernels run; only the rows each workgroup addresses differ)."""
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


def run_varlen(fa, inp, w, sentinel=False):
    """Forward and backward on the GPU.  With ``sentinel`` the outputs start as NaN so
    that rows no sequence owns (and LSE entries past a length) show if written."""
    q, k, v, do = (inp[n].to(DEV) for n in ("q", "k", "v", "do"))
    cu = inp["cu_seqlens"].to(DEV)
    fill = (lambda t: t.fill_(float("nan"))) if sentinel else (lambda t: t)
    o = fill(torch.empty_like(q))
    lse = fill(torch.empty((w.B, w.H, w.max_s), dtype=torch.float32, device=DEV))
    o, lse = fa.forward_varlen(q, k, v, cu, w.max_s, w.causal, w.scale, o=o, lse=lse)
    dq, dk, dv = (fill(torch.empty_like(t)) for t in (q, k, k))
    dq, dk, dv = fa.backward_varlen(q, k, v, o, do, lse, cu, w.max_s, w.causal, w.scale,
                                    dq=dq, dk=dk, dv=dv)
    torch.cuda.synchronize()
    return {"o": o, "lse": lse, "dq": dq, "dk": dk, "dv": dv}


def check_sequences(out, inp, w, seqs, heads=None, tag=""):
    """Oracle on the given sequences (all query heads, or the listed ones, with
    their K/V heads' gradients summed over every query head of the group)."""
    tol = TOL[w.dtype]
    q, k, v, do = (f64(inp[n]) for n in ("q", "k", "v", "do"))
    cu = inp["cu_seqlens"].tolist()
    G = w.H // w.kv_heads
    got = {n: f64(out[n]) for n in out}
    err = {"o": 0.0, "lse": 0.0, "dq": 0.0, "dk": 0.0, "dv": 0.0}
    for b in seqs:
        s0, s1 = cu[b], cu[b + 1]
        if s1 == s0:
            continue
        hs = heads if heads is not None else range(w.H)
        kv_done = set()
        for h in hs:
            j = h // G
            o_ref, lse_ref = oracle.forward_head(q[h, s0:s1], k[j, s0:s1], v[j, s0:s1], w.scale,
                                                 w.causal)
            err["o"] = max(err["o"], float(np.max(np.abs(got["o"][h, s0:s1] - o_ref))))
            err["lse"] = max(err["lse"], float(np.max(np.abs(got["lse"][b, h, :s1 - s0] - lse_ref))))
            g = oracle.backward_head(q[h, s0:s1], k[j, s0:s1], v[j, s0:s1], do[h, s0:s1],
                                     w.scale, w.causal)
            err["dq"] = max(err["dq"], rel_err(got["dq"][h, s0:s1], g["dq"]))
            if j in kv_done:
                continue
            kv_done.add(j)
            dk = np.zeros((s1 - s0, w.d))
            dv = np.zeros((s1 - s0, w.d))
            for hh in range(j * G, (j + 1) * G):
                gg = oracle.backward_head(q[hh, s0:s1], k[j, s0:s1], v[j, s0:s1], do[hh, s0:s1],
                                          w.scale, w.causal)
                dk += gg["dk"]
                dv += gg["dv"]
            err["dk"] = max(err["dk"], rel_err(got["dk"][j, s0:s1], dk))
            err["dv"] = max(err["dv"], rel_err(got["dv"][j, s0:s1], dv))
    say(f"  {tag} " + ", ".join(f"{n} {e:.3e}" for n, e in err.items()))
    assert err["o"] <= tol["o"] and err["lse"] <= tol["lse"], err
    for n in ("dq", "dk", "dv"):
        assert err[n] <= tol["grad"], (n, err)


LENS = (1, 0, 17, 64, 65, 200, 3, 130)   # single token, empty, ragged, tile-exact, multi-tile


def small_cases():
    for dtype in ("bf16", "f16", "f32"):
        for d in (64, 128):
            for causal in (False, True):
                yield dtype, d, causal


@pytest.mark.parametrize("dtype,d,causal", list(small_cases()))
def test_varlen_small(fa, dtype, d, causal):
    """Eight sequences (one empty, one of a single token, ragged tails) packed with 5
    trailing rows that belong to none; 4 query heads over 2 K/V heads.  Every owned
    element against the oracle; unowned rows and LSE past each length untouched."""
    w = workloads.Varlen(f"varlen-small-{dtype}-d{d}", LENS, 4, d, dtype, causal,
                         seed=61 + d + causal, H_kv=2)
    inp = workloads.make_varlen_inputs(w, extra_rows=5)
    say(f"case {w.name} causal={causal}")
    out = run_varlen(fa, inp, w, sentinel=True)
    check_sequences(out, inp, w, range(w.B), tag=w.name)
    total = w.total
    for n in ("o", "dq", "dk", "dv"):
        assert torch.isnan(out[n][:, total:]).all(), f"{n}: unowned rows were written"
        assert not torch.isnan(out[n][:, :total]).any(), f"{n}: owned rows left unwritten"
    for b, n in enumerate(LENS):
        assert torch.isnan(out["lse"][b, :, n:]).all(), "LSE past the length was written"
        assert not torch.isnan(out["lse"][b, :, :n]).any()


@pytest.mark.parametrize("dtype", ["bf16", "f16"])
@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("causal", [False, True])
def test_equal_lengths_match_the_dense_entry_points_bitwise(fa, dtype, d, causal):
    """B sequences of one length packed head-major run the same tile arithmetic as
    the dense [B, H, N, d] call: every output equal bit for bit."""
    B, H, Hkv, N = 3, 4, 2, 300
    wd = workloads.Workload(f"dense-{dtype}-d{d}", B, H, N, d, dtype, causal, 71 + d, H_kv=Hkv)
    dense = workloads.make_inputs(wd)
    dev = {n: t.to(DEV) for n, t in dense.items()}
    o, lse = fa.forward(dev["q"], dev["k"], dev["v"], causal, wd.scale)
    dq, dk, dv = fa.backward(dev["q"], dev["k"], dev["v"], o, dev["do"], lse, causal, wd.scale)
    pack = lambda t: t.permute(1, 0, 2, 3).reshape(t.shape[1], B * N, d).contiguous()
    cu = torch.arange(0, B * N + 1, N, dtype=torch.int32, device=DEV)
    pq, pk, pv, pdo = (pack(dev[n]) for n in ("q", "k", "v", "do"))
    po, plse = fa.forward_varlen(pq, pk, pv, cu, N, causal, wd.scale)
    pdq, pdk, pdv = fa.backward_varlen(pq, pk, pv, po, pdo, plse, cu, N, causal, wd.scale)
    torch.cuda.synchronize()
    say(f"case {wd.name} causal={causal}")
    assert torch.equal(po, pack(o))
    assert torch.equal(plse, lse)
    assert torch.equal(pdq, pack(dq))
    assert torch.equal(pdk, pack(dk))
    assert torch.equal(pdv, pack(dv))


@pytest.mark.parametrize("w", workloads.VARLEN, ids=lambda w: w.name)
def test_large_varlen_sampled(fa, w):
    """The packed workloads at full size (the launch the benchmark times): the oracle
    on the shortest sequence (all heads) and on the first and last query head of
    the longest; on every sequence, sum_j dV_j = sum_i dO_i over the group's query
    heads and sum_j dK_j = 0."""
    inp = workloads.make_varlen_inputs(w)
    say(f"case {w.name} full size")
    out = run_varlen(fa, inp, w)
    lens = list(w.lens)
    check_sequences(out, inp, w, [lens.index(min(lens))], tag=w.name + " shortest")
    check_sequences(out, inp, w, [lens.index(max(lens))], heads=[0, w.H - 1],
                    tag=w.name + " longest")
    cu = inp["cu_seqlens"].tolist()
    G = w.H // w.kv_heads
    do = inp["do"].to(DEV).double()
    tol = 4 * TOL[w.dtype]["grad"]
    for b in range(w.B):
        s0, s1 = cu[b], cu[b + 1]
        dv = out["dv"][:, s0:s1].double()
        dk = out["dk"][:, s0:s1].double()
        want = do[:, s0:s1].sum(dim=1).reshape(w.kv_heads, G, w.d).sum(dim=1)
        assert (dv.sum(dim=1) - want).abs().max().item() <= tol * dv.abs().sum(dim=1).max().item()
        assert dk.sum(dim=1).abs().max().item() <= tol * dk.abs().sum(dim=1).max().item()
    assert torch.isfinite(out["o"]).all() and torch.isfinite(out["lse"]).all()
