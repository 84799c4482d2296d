"""Parity of the HIP path (through the C ABI) with the fp64 oracle, on the GPU.

Tolerances (tests/tolerances.py): O max-abs 2e-3 (fp16) / 1e-2 (bf16); dQ,
dK, dV max-abs error relative to the reference's max-abs 5e-3 (fp16) / 2e-2
(bf16).  LSE max-abs 1e-3 (fp16) / 4e-3 (bf16): the forward's row sum adds P~
as rounded to the input type, so ln l carries up to that type's unit roundoff.
fp32 has no stated tolerance; 1e-5 on O and 1e-4 on LSE and gradients is
derived from fp32 accumulation over at most a few thousand terms.
"""
import math
import sys

import numpy as np
import pytest
import torch

import oracle
import workloads
from tests import pins
from tests.tolerances import TOL, o_bound

pytestmark = pytest.mark.gpu

TORCH = {"f32": torch.float32, "f16": torch.float16, "bf16": torch.bfloat16}


@pytest.fixture(scope="module")
def fa():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import io_aware_exact_fa_amd
    return io_aware_exact_fa_amd


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def gpu_run(fa, inp, causal, scale, backward=True):
    dev = torch.device("cuda:0")
    q, k, v, do = (inp[n].to(dev) for n in ("q", "k", "v", "do"))
    o, lse = fa.forward(q, k, v, causal, scale)
    out = {"o": o, "lse": lse}
    if backward:
        ws = fa.workspace(*q.shape, dev)
        dq, dk, dv = fa.backward(q, k, v, o, do, lse, causal, scale, ws=ws)
        out.update(dq=dq, dk=dk, dv=dv, ws=ws)
    torch.cuda.synchronize()
    return out


def f64(t):
    return t.detach().to("cpu", torch.float64).numpy()


def rel_err(got, ref):
    den = np.max(np.abs(ref))
    return float(np.max(np.abs(got - ref)) / (den if den > 0 else 1.0))


def same_but_summation_order(a, b, dtype):
    """dQ of the one-pass backward, which sums the key tiles' shares by atomic
    adds in an order that may change, against another summation: equal up to
    one unit in the last place of the storage type (relative to the largest
    element)."""
    ulp = {"f32": 2.0 ** -23, "f16": 2.0 ** -10, "bf16": 2.0 ** -7}[dtype]
    da, db_ = a.double(), b.double()
    return (da - db_).abs().max().item() <= ulp * max(da.abs().max().item(), 1e-30)


def compare(out, inp, causal, scale, dtype, heads=None, backward=True, tag=""):
    """Compare GPU outputs with the oracle on the given (b, h) heads (all if None)."""
    tol = TOL[dtype]
    q, k, v, do = (f64(inp[n]) for n in ("q", "k", "v", "do"))
    B, H = q.shape[:2]
    heads = heads if heads is not None else [(b, h) for b in range(B) for h in range(H)]
    o_ref, lse_ref = oracle.forward(q, k, v, scale, causal, heads=heads)
    sel = tuple(np.array(x) for x in zip(*heads))
    o_gpu, lse_gpu = f64(out["o"])[sel], f64(out["lse"])[sel]
    err_o = float(np.max(np.abs(o_gpu - o_ref[sel])))
    err_l = float(np.max(np.abs(lse_gpu - lse_ref[sel])))
    say(f"  {tag} O max-abs {err_o:.3e} (tol {tol['o']}), LSE max-abs {err_l:.3e}")
    assert err_o <= tol["o"], f"O error {err_o}"
    assert err_l <= tol["lse"], f"LSE error {err_l}"
    if not backward:
        return
    dq_ref, dk_ref, dv_ref, D_ref = oracle.backward(q, k, v, do, scale, causal, heads=heads)
    for name, ref in (("dq", dq_ref), ("dk", dk_ref), ("dv", dv_ref)):
        e = rel_err(f64(out[name])[sel], ref[sel])
        say(f"  {tag} {name} rel-to-max {e:.3e} (tol {tol['grad']})")
        assert e <= tol["grad"], f"{name} error {e}"


# ------------------------------------------------------------------ small seeded grid


def grid_cases():
    for dtype in ("bf16", "f16", "f32"):
        for d in (64, 128):
            for causal in (False, True):
                for n in (1, 17, 128, 129, 300):
                    yield dtype, d, causal, n


@pytest.mark.parametrize("dtype,d,causal,n", list(grid_cases()))
def test_small_shapes(fa, dtype, d, causal, n):
    w = workloads.Workload(f"grid-{dtype}-d{d}-n{n}", 2, 2, n, d, dtype, causal, seed=7 + n + d)
    inp = workloads.make_inputs(w)
    say(f"case {w.name} causal={causal}")
    out = gpu_run(fa, inp, causal, w.scale)
    compare(out, inp, causal, w.scale, dtype, tag=w.name)


@pytest.mark.parametrize("dtype", ["bf16", "f16"])
@pytest.mark.parametrize("causal", [False, True])
def test_several_tiles_with_ragged_tail(fa, dtype, causal):
    """N = 520: eight 64-key tiles plus a tail of 8 keys; five query tiles forward,
    five key tiles backward, with a ragged last tile."""
    w = workloads.Workload("ragged-520", 1, 3, 520, 128, dtype, causal, seed=31, qk_std=1.5)
    inp = workloads.make_inputs(w)
    say(f"case {w.name} {dtype} causal={causal}")
    compare(gpu_run(fa, inp, causal, w.scale), inp, causal, w.scale, dtype, tag=w.name)


# ------------------------------------------------------------------ page vectors


@pytest.mark.parametrize("dtype", ["f32", "bf16", "f16"])
@pytest.mark.parametrize("causal", [False, True])
def test_page_vectors_zero_padded(fa, dtype, causal):
    """The page's 5x3 / 5x2 integer vectors, zero-padded to d = 64 (zeros leave the dot
    products unchanged), scale 1/sqrt(3); all values are exact in every dtype."""
    g = pins.load_golden("cpu_check_vectors.json")
    qkv = {}
    for n in ("q", "k", "v"):
        a = np.array(g[n], dtype=np.float32)
        pad = np.zeros((5, 64), dtype=np.float32)
        pad[:, : a.shape[1]] = a
        qkv[n] = torch.from_numpy(pad)[None, None].to(TORCH[dtype]).contiguous()
    qkv["do"] = workloads.make_random((1, 1, 5, 64), dtype, seed=5)
    scale = 1.0 / math.sqrt(3.0)
    say(f"case page-vectors {dtype} causal={causal}")
    out = gpu_run(fa, qkv, causal, scale)
    compare(out, qkv, causal, scale, dtype, tag="page")
    if causal:
        o = f64(out["o"])[0, 0]
        np.testing.assert_allclose(o[0, :2], g["printed"]["causal_row0_output"], atol=TOL[dtype]["o"])


# ------------------------------------------------------------------ closed forms / invariants


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("causal", [False, True])
def test_zero_query_gives_prefix_mean(fa, dtype, causal):
    w = workloads.Workload("zeroq", 1, 2, 200, 64, dtype, causal, seed=41)
    inp = workloads.make_inputs(w)
    inp["q"] = torch.zeros_like(inp["q"])
    out = gpu_run(fa, inp, causal, w.scale, backward=False)
    v = f64(inp["v"])
    n = np.arange(1, 201)[:, None] if causal else 200
    expect = (np.cumsum(v, axis=2) / n) if causal else np.repeat(v.mean(axis=2, keepdims=True), 200, 2)
    assert np.max(np.abs(f64(out["o"]) - expect)) <= TOL[dtype]["o"]
    lse_expect = np.log(np.arange(1, 201)) if causal else np.full(200, math.log(200))
    assert np.max(np.abs(f64(out["lse"]) - lse_expect)) <= 1e-4


@pytest.mark.parametrize("dtype", ["bf16", "f16"])
def test_key_shift_invariance(fa, dtype):
    """K + 1 c^T shifts row i of the scores by scale q_i.c: O and the gradients stay put
    (to tolerance), LSE moves by exactly that amount."""
    w = workloads.Workload("shift", 1, 2, 150, 64, dtype, False, seed=43)
    inp = workloads.make_inputs(w)
    c = torch.zeros(64)
    c[:8] = 1.0                               # exact in every dtype
    inp2 = dict(inp)
    inp2["k"] = (inp["k"].float() + c).to(TORCH[dtype])
    a, b = gpu_run(fa, inp, False, w.scale), gpu_run(fa, inp2, False, w.scale)
    # Compare each against the oracle of its own inputs, and LSE shift directly.
    compare(a, inp, False, w.scale, dtype, tag="shift-a")
    compare(b, inp2, False, w.scale, dtype, tag="shift-b")
    # the shifted keys are exact in dtype only where k + c rounds exactly; use the oracle's shift
    q = f64(inp["q"])
    shift = w.scale * (q @ c.double().numpy())
    dl = f64(b["lse"]) - f64(a["lse"])
    k_exact = torch.equal(inp2["k"].float(), inp["k"].float() + c)
    if k_exact:
        assert np.max(np.abs(dl - shift)) <= 2e-3


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_scale_sign_and_zero(fa, dtype):
    for scale in (-0.2, 0.0, 0.9):
        w = workloads.Workload("scale", 1, 2, 100, 64, dtype, True, seed=47)
        inp = workloads.make_inputs(w)
        say(f"case scale={scale} {dtype}")
        compare(gpu_run(fa, inp, True, scale), inp, True, scale, dtype, tag=f"scale{scale}")


def test_peaked_rows_stress_rescaling(fa):
    """Scores with std ~8 make the running max jump between tiles."""
    w = workloads.Workload("peaked", 1, 2, 400, 64, "f16", True, seed=53, qk_std=2.8)
    inp = workloads.make_inputs(w)
    compare(gpu_run(fa, inp, True, w.scale), inp, True, w.scale, "f16", tag="peaked")


@pytest.mark.parametrize("dtype", ["bf16", "f16"])
@pytest.mark.parametrize("d,causal,n", [(128, False, 2085), (128, True, 700), (64, False, 700),
                                        (64, True, 700)])
def test_rising_scores_rescale_every_tile(fa, dtype, d, causal, n):
    """Keys along one direction with a norm that grows with the key index, so
    that every 64-key tile raises each row's max by more than the forward's
    rescale slack (2^8): the growth test, the half-row exchange and the rescale
    run on every tile (the 64-row forward at d = 128 without the mask, the
    32-row one otherwise), against the oracle on every element of O and LSE.
    The forward alone: with every key along one direction, dQ = scale sum_j dS_ij
    k_j cancels almost completely (the dS_ij of a row sum to zero and the k_j
    differ little against their norm), so rounding dS to bf16 alone moves dQ by
    about 14 % of its largest element on this input (fp64 emulation) -- a
    property of the input, not of the path, which the backward tests cover."""
    rng = np.random.default_rng(881 + d + n + int(causal))
    B, H = 1, 2
    u = np.ones(d)
    gamma = 2.4 * math.sqrt(d) / 8    # s c grows by 15-30 log2 units per 64-key tile
    alpha = (0.5 + gamma * np.arange(n) / d)[:, None]
    qn = u[None, None, None, :] + 0.3 * rng.standard_normal((B, H, n, d))
    kn = alpha[None, None] * u[None, None, None, :] + 0.3 * rng.standard_normal((B, H, n, d))
    vn = rng.standard_normal((B, H, n, d))
    don = rng.standard_normal((B, H, n, d))
    t = TORCH[dtype]
    inp = {name: torch.from_numpy(x).to(t) for name, x in (("q", qn), ("k", kn), ("v", vn), ("do", don))}
    scale = 1.0 / math.sqrt(d)
    say(f"case rising d={d} causal={causal} n={n} {dtype}")
    compare(gpu_run(fa, inp, causal, scale, backward=False), inp, causal, scale, dtype,
            backward=False, tag="rising")


# ------------------------------------------------------------------ repeatability, workspace


def test_repeatable_and_delta(fa):
    w = workloads.Workload("repeat", 2, 2, 333, 128, "bf16", True, seed=59)
    inp = workloads.make_inputs(w)
    a = gpu_run(fa, inp, True, w.scale)
    b = gpu_run(fa, inp, True, w.scale)
    for name in ("o", "lse", "dq", "dk", "dv"):
        assert torch.equal(a[name], b[name]), f"{name} differs between runs"
    # Workspace: D = rowsum(dO * O), then L2 = LSE log2(e), each [B, H, Np]
    # with Np = 384 (333 rounded up to 64); padding rows hold D = 0, L2 = +inf.
    Np = 384
    ws = a["ws"][: 2 * 4 * 4 * Np].view(torch.float32).reshape(2, 2, 2, Np)
    D, L2 = f64(ws[0]), f64(ws[1])
    expect = (f64(inp["do"]) * f64(a["o"])).sum(-1)
    assert np.max(np.abs(D[..., :333] - expect)) <= 1e-4
    l2_expect = f64(a["lse"]) * 1.4426950408889634
    assert np.max(np.abs(L2[..., :333] - l2_expect)) <= 1e-6 * max(1.0, np.max(np.abs(l2_expect)))
    assert np.all(D[..., 333:] == 0) and np.all(np.isposinf(L2[..., 333:]))


def test_non_default_stream(fa):
    w = workloads.Workload("stream", 1, 2, 256, 64, "f16", False, seed=61)
    inp = workloads.make_inputs(w)
    s = torch.cuda.Stream()
    dev = torch.device("cuda:0")
    with torch.cuda.stream(s):
        q, k, v, do = (inp[n].to(dev) for n in ("q", "k", "v", "do"))
        o, lse = fa.forward(q, k, v, False, w.scale, stream=s)
        dq, dk, dv = fa.backward(q, k, v, o, do, lse, False, w.scale, stream=s)
    s.synchronize()
    compare(dict(o=o, lse=lse, dq=dq, dk=dk, dv=dv), inp, False, w.scale, "f16", tag="stream")


# ------------------------------------------------------------------ the five workloads


@pytest.mark.parametrize("w", [workloads.SINGLE_HEAD_F32, workloads.SHORT_F16], ids=lambda w: w.name)
def test_small_workloads_full(fa, w):
    inp = workloads.make_inputs(w)
    say(f"case {w.name} (every head)")
    compare(gpu_run(fa, inp, w.causal, w.scale), inp, w.causal, w.scale, w.dtype, tag=w.name)


LARGE = [workloads.CAUSAL_BF16, workloads.LONG_CAUSAL_F16, workloads.PEAKED_BF16]


def xcd_sample_heads(B, H, limit=9):
    """(b, h) pairs of the flat heads 0, n/8, 2n/8, ..., 7n/8 and n - 1 (n = B H):
    the first head of each of the 8 contiguous head ranges that the kernels hand
    to the 8 XCDs, and the last head.  With more than ``limit`` of them (oracle
    memory at long N), the first and the last only."""
    n = B * H
    flat = sorted({(x * n) // 8 for x in range(8)} | {n - 1})
    if len(flat) > limit:
        flat = [0, n - 1]
    return [(f // H, f % H) for f in flat]


def test_xcd_sample_heads():
    assert xcd_sample_heads(2, 32) == [(0, 0), (0, 8), (0, 16), (0, 24), (1, 0), (1, 8), (1, 16),
                                       (1, 24), (1, 31)]
    assert xcd_sample_heads(1, 16, limit=2) == [(0, 0), (0, 15)]
    assert len(xcd_sample_heads(4, 32)) == 9 and xcd_sample_heads(4, 32)[-1] == (3, 31)


@pytest.mark.parametrize("w", LARGE, ids=lambda w: w.name)
def test_large_workloads_sampled_heads(fa, w):
    """Full-size launch (the configuration the benchmark times).  The oracle checks
    every element of one head in each XCD's range of heads and of the last head
    (the XCD-aware and heavy-first work orders decide which workgroup gets which
    head; the N = 16384 workload: the first and the last head, for oracle
    memory), and properties that hold for every head are checked on all."""
    inp = workloads.make_inputs(w)
    say(f"case {w.name} full size")
    out = gpu_run(fa, inp, w.causal, w.scale)
    heads = xcd_sample_heads(w.B, w.H, limit=9 if w.N <= 8192 else 2)
    say(f"  oracle heads {heads}")
    compare(out, inp, w.causal, w.scale, w.dtype, heads=heads, tag=w.name)
    # Every head: sum_j dV_j = sum_i dO_i (rows of P sum to 1) and sum_j dK_j = 0
    # (rows of dS sum to 0), both in fp64 over the GPU's outputs.
    dv = out["dv"].double().sum(dim=2)
    do = inp["do"].to("cuda").double().sum(dim=2)
    dk = out["dk"].double().sum(dim=2)
    scale_dv = out["dv"].double().abs().sum(dim=2).max().item()
    scale_dk = out["dk"].double().abs().sum(dim=2).max().item()
    tol = 4 * TOL[w.dtype]["grad"]
    assert (dv - do).abs().max().item() <= tol * scale_dv
    assert dk.abs().max().item() <= tol * scale_dk
    assert torch.isfinite(out["lse"]).all() and torch.isfinite(out["o"]).all()


# ------------------------------------------------------------------ grouped K/V heads


def compare_gqa(out, inp, causal, scale, dtype, tag="", groups=None):
    """Compare with the grouped-K/V oracle; ``groups`` restricts the check to a list of
    (b, kv head) pairs (their query heads and the shared dK, dV)."""
    tol = TOL[dtype]
    q, k, v, do = (f64(inp[n]) for n in ("q", "k", "v", "do"))
    B, H = q.shape[:2]
    Hkv = k.shape[1]
    G = H // Hkv
    if groups is not None:
        # The oracle on just those groups: one batch entry and K/V head at a time.
        sel_q = [(b, j * G + g) for b, j in groups for g in range(G)]
        qi = tuple(np.array(x) for x in zip(*sel_q))
        ki = tuple(np.array(x) for x in zip(*groups))
    if groups is None:
        o_ref, lse_ref = oracle.forward_gqa(q, k, v, scale, causal)
        err_o = float(np.max(np.abs(f64(out["o"]) - o_ref)))
        err_l = float(np.max(np.abs(f64(out["lse"]) - lse_ref)))
        dq_ref, dk_ref, dv_ref = oracle.backward_gqa(q, k, v, do, scale, causal)
        got = {n: f64(out[n]) for n in ("dq", "dk", "dv")}
        refs = {"dq": dq_ref, "dk": dk_ref, "dv": dv_ref}
    else:
        fw = [oracle.forward_gqa(q[b:b + 1, j * G:(j + 1) * G], k[b:b + 1, j:j + 1],
                                 v[b:b + 1, j:j + 1], scale, causal) for b, j in groups]
        bw = [oracle.backward_gqa(q[b:b + 1, j * G:(j + 1) * G], k[b:b + 1, j:j + 1],
                                  v[b:b + 1, j:j + 1], do[b:b + 1, j * G:(j + 1) * G], scale, causal)
              for b, j in groups]
        o_ref = np.concatenate([f[0][0] for f in fw])
        lse_ref = np.concatenate([f[1][0] for f in fw])
        err_o = float(np.max(np.abs(f64(out["o"])[qi] - o_ref)))
        err_l = float(np.max(np.abs(f64(out["lse"])[qi] - lse_ref)))
        got = {"dq": f64(out["dq"])[qi], "dk": f64(out["dk"])[ki], "dv": f64(out["dv"])[ki]}
        refs = {"dq": np.concatenate([x[0][0] for x in bw]),
                "dk": np.concatenate([x[1][0] for x in bw]),
                "dv": np.concatenate([x[2][0] for x in bw])}
    say(f"  {tag} O max-abs {err_o:.3e} (tol {tol['o']}), LSE max-abs {err_l:.3e}")
    assert err_o <= tol["o"], f"O error {err_o}"
    assert err_l <= tol["lse"], f"LSE error {err_l}"
    for name in ("dq", "dk", "dv"):
        e = rel_err(got[name], refs[name])
        say(f"  {tag} {name} rel-to-max {e:.3e} (tol {tol['grad']})")
        assert e <= tol["grad"], f"{name} error {e}"


def gqa_cases():
    for dtype in ("bf16", "f16", "f32"):
        for d in (64, 128):
            for causal in (False, True):
                for H, Hkv in ((8, 2), (6, 1)):
                    yield dtype, d, causal, H, Hkv


@pytest.mark.parametrize("dtype,d,causal,H,Hkv", list(gqa_cases()))
def test_grouped_kv_heads(fa, dtype, d, causal, H, Hkv):
    """H query heads over Hkv shared K/V heads (Hkv = 1: multi-query), N = 200 (three
    64-row tiles and a tail of 8), two batch entries."""
    w = workloads.Workload(f"gqa-{dtype}-d{d}-h{H}kv{Hkv}", 2, H, 200, d, dtype, causal,
                           seed=41 + H + Hkv + d, H_kv=Hkv)
    inp = workloads.make_inputs(w)
    say(f"case {w.name} causal={causal}")
    compare_gqa(gpu_run(fa, inp, causal, w.scale), inp, causal, w.scale, dtype, tag=w.name)


@pytest.mark.parametrize("w", workloads.GQA, ids=lambda w: w.name)
def test_large_gqa_sampled_groups(fa, w):
    """The grouped-K/V workloads at full size, in the launch the benchmark times; the
    oracle on the first and last K/V group."""
    inp = workloads.make_inputs(w)
    say(f"case {w.name}")
    out = gpu_run(fa, inp, w.causal, w.scale)
    groups = [(0, 0), (w.B - 1, w.kv_heads - 1)]
    compare_gqa(out, inp, w.causal, w.scale, w.dtype, tag=w.name, groups=groups)


# ------------------------------------------------------------------ the plain entry points


@pytest.mark.parametrize("dtype,d", [("bf16", 128), ("f16", 128), ("bf16", 64), ("f16", 64)])
def test_plain_entry_points_by_name(fa, dtype, d):
    """fa_fwd, fa_bwd, the two-pass steps (fa_bwd_preprocess + fa_bwd_dkdv +
    fa_bwd_dq) and the one-pass steps (fa_bwd_preprocess + fa_bwd_dkdv_dq +
    fa_bwd_dq_finalize) called by those names through ctypes (not through their
    grouped forms), causal, ragged N = 333 over 3 heads of 2 batch entries:
    every element against the oracle; the two-pass steps bit for bit equal to
    fa_bwd; the one-pass dK and dV too (at d = 64 the two-pass dK/dV kernel is the
    pipelined one, which accumulates in the same order), its dQ up to the order
    of its sums."""
    w = workloads.Workload(f"plain-{dtype}-d{d}", 2, 3, 333, d, dtype, True, seed=83)
    inp = workloads.make_inputs(w)
    dev = torch.device("cuda:0")
    q, k, v, do = (inp[n].to(dev) for n in ("q", "k", "v", "do"))
    B, H, N, d = q.shape
    code = fa.dtype_code(q.dtype)
    sh = torch.cuda.current_stream().cuda_stream
    P = lambda t: t.data_ptr()
    o = torch.full_like(q, float("nan"))
    lse = torch.full((B, H, N), float("nan"), dtype=torch.float32, device=dev)
    say(f"case {w.name}: fa_fwd")
    assert fa.fa_fwd(P(q), P(k), P(v), P(o), P(lse), B, H, N, d, 1, w.scale, code, sh) == fa.FA_OK
    ws = fa.workspace(B, H, N, d, dev)
    g1 = [torch.full_like(q, float("nan")) for _ in range(3)]
    say(f"case {w.name}: fa_bwd")
    assert fa.fa_bwd(P(q), P(k), P(v), P(o), P(do), P(lse), *(P(t) for t in g1), B, H, N, d, 1,
                     w.scale, code, P(ws), ws.numel(), sh) == fa.FA_OK
    g2 = [torch.full_like(q, float("nan")) for _ in range(3)]
    ws2 = fa.workspace(B, H, N, d, dev)
    say(f"case {w.name}: fa_bwd_preprocess, fa_bwd_dkdv, fa_bwd_dq")
    assert fa.fa_bwd_preprocess(P(o), P(do), P(lse), B, H, N, d, code, P(ws2), ws2.numel(),
                                sh) == fa.FA_OK
    assert fa.fa_bwd_dkdv(P(q), P(k), P(v), P(do), P(lse), P(g2[1]), P(g2[2]), B, H, N, d, 1,
                          w.scale, code, P(ws2), ws2.numel(), sh) == fa.FA_OK
    assert fa.fa_bwd_dq(P(q), P(k), P(v), P(do), P(lse), P(g2[0]), B, H, N, d, 1, w.scale, code,
                        P(ws2), ws2.numel(), sh) == fa.FA_OK
    g3 = [torch.full_like(q, float("nan")) for _ in range(3)]
    ws3 = fa.workspace(B, H, N, d, dev, one_pass=True)
    ws3.fill_(255)   # NaN in every float32 of the workspace: the accumulator must be zeroed
    say(f"case {w.name}: fa_bwd_preprocess, fa_bwd_dkdv_dq, fa_bwd_dq_finalize")
    assert fa.fa_bwd_preprocess(P(o), P(do), P(lse), B, H, N, d, code, P(ws3), ws3.numel(),
                                sh) == fa.FA_OK
    assert fa.fa_bwd_dkdv_dq(P(q), P(k), P(v), P(do), P(lse), P(g3[1]), P(g3[2]), B, H, H, N, d,
                             1, w.scale, code, P(ws3), ws3.numel(), sh) == fa.FA_OK
    assert fa.fa_bwd_dq_finalize(P(g3[0]), B, H, N, d, w.scale, code, P(ws3), ws3.numel(),
                                 sh) == fa.FA_OK
    torch.cuda.synchronize()
    out = dict(o=o, lse=lse, dq=g1[0], dk=g1[1], dv=g1[2])
    compare(out, inp, True, w.scale, dtype, tag=w.name)
    compare(dict(o=o, lse=lse, dq=g3[0], dk=g3[1], dv=g3[2]), inp, True, w.scale, dtype,
            tag=w.name + " one-pass")
    # fa_bwd is the two-pass backward, bit for bit; the one-pass kernel does the
    # same dK/dV arithmetic, and sums dQ by atomic adds instead.
    for name, a, b, c in zip(("dq", "dk", "dv"), g1, g2, g3):
        assert torch.equal(a, b), f"{name}: fa_bwd differs from its steps"
        if name != "dq":
            assert torch.equal(a, c), f"{name}: the one-pass kernel differs"
    assert same_but_summation_order(g3[0], g1[0], dtype)


# ------------------------------------------------------------------ the 64-row forward


@pytest.mark.parametrize("dtype", ["bf16", "f16"])
@pytest.mark.parametrize("case", ["plain", "window", "gqa-blocks", "negative-scale", "peaked"])
def test_long_rows_forward_kernel(fa, dtype, case):
    """Without the causal mask and dropout, at N >= 2048, the forward runs 64 query
    rows per wave (its own kernel).  N = 2085: eight full 256-row workgroups and a
    ragged ninth, a ragged last key tile; every element of every head against the
    oracle, with a window (both edges masked), grouped K/V heads with a block
    mask, a negative scale, and peaked scores (row maxima that keep growing,
    so the accumulators are rescaled)."""
    n = 2085
    qk_std = 3.0 if case == "peaked" else 1.0
    H, Hkv = (4, 2) if case == "gqa-blocks" else (2, 2)
    w = workloads.Workload(f"rows64-{case}-{dtype}", 1, H, n, 128, dtype, False, 191 + len(case),
                           qk_std=qk_std, H_kv=Hkv)
    inp = workloads.make_inputs(w)
    say(f"case {w.name}")
    dev = torch.device("cuda:0")
    q, k, v = (inp[x].to(dev) for x in ("q", "k", "v"))
    scale = -w.scale if case == "negative-scale" else w.scale
    window = (300, 100) if case == "window" else None
    bm = None
    if case == "gqa-blocks":
        g = torch.Generator(device="cpu").manual_seed(7)
        bm = (torch.rand((H, -(-n // 256), -(-n // 128)), generator=g) < 0.6).to(torch.uint8)
        bm[0, -1, :] = 0   # head 0: the last query block sees nothing
    o, lse = fa.forward(q, k, v, False, scale, window=window,
                        block_mask=bm.to(dev) if bm is not None else None)
    torch.cuda.synchronize()
    qh, kh, vh = (f64(inp[x]) for x in ("q", "k", "v"))
    o_ref, lse_ref = oracle.forward_gqa(qh, kh, vh, scale, False, window=window,
                                        block_mask=bm.numpy() if bm is not None else None)
    fin = np.isfinite(lse_ref)
    lg = f64(lse)
    assert np.array_equal(np.isneginf(lg), ~fin)
    err_o = float(np.max(np.abs(f64(o) - o_ref)))
    err_l = float(np.max(np.abs(lg[fin] - lse_ref[fin])))
    say(f"  O max-abs {err_o:.3e} (bound {o_bound(dtype, o_ref):.1e}) LSE {err_l:.3e}")
    assert err_o <= o_bound(dtype, o_ref) and err_l <= TOL[dtype]["lse"]
