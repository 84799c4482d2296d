"""fa_bwd_noalloc (the backward whose D and L2 live in the library's static
device array) against fa_bwd (caller-allocated workspace), through the C ABI.

Two calls in a row, the second on a smaller shape, so that the second call
finds the array holding the first call's D and L2: both must give exactly
fa_bwd's gradients (the same kernels run on the same values), and those lie
within the parity bounds of the fp64 oracle.  Collected last (test_zz_...):
it also passes alone in a fresh process."""
import sys

import numpy as np
import pytest
import torch

import oracle
import workloads
from tests.tolerances import TOL

pytestmark = pytest.mark.gpu


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module")
def fa():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import io_aware_exact_fa_amd
    return io_aware_exact_fa_amd


def _case(fa, B, H, N, d, dtype, causal, seed):
    w = workloads.Workload(f"noalloc-b{B}h{H}n{N}d{d}-{dtype}", B, H, N, d, dtype, causal, seed)
    inp = workloads.make_inputs(w)
    dev = torch.device("cuda:0")
    q, k, v, do = (inp[n].to(dev) for n in ("q", "k", "v", "do"))
    o, lse = fa.forward(q, k, v, causal, w.scale)
    code = fa.dtype_code(q.dtype)
    sh = torch.cuda.current_stream().cuda_stream
    P = lambda t: t.data_ptr()
    ref = [torch.empty_like(q) for _ in range(3)]
    ws = fa.workspace(B, H, N, d, dev)
    st = fa.fa_bwd(P(q), P(k), P(v), P(o), P(do), P(lse), *(P(t) for t in ref), B, H, N, d,
                   causal, w.scale, code, P(ws), ws.numel(), sh)
    assert st == fa.FA_OK, fa.fa_status_string(st)
    got = [torch.full_like(q, float("nan")) for _ in range(3)]
    st = fa.fa_bwd_noalloc(P(q), P(k), P(v), P(o), P(do), P(lse), *(P(t) for t in got), B, H, N,
                           d, causal, w.scale, code, sh)
    assert st == fa.FA_OK, fa.fa_status_string(st)
    torch.cuda.synchronize()
    return w, inp, ref, got


def _check(w, inp, ref, got):
    for name, r, g in zip(("dq", "dk", "dv"), ref, got):
        assert torch.equal(r, g), f"{w.name}: {name} differs from fa_bwd's"
    f64 = lambda t: t.detach().to("cpu", torch.float64).numpy()
    g_ref = oracle.backward(*(f64(inp[n]) for n in ("q", "k", "v", "do")), w.scale, w.causal)
    tol = TOL[w.dtype]["grad"]
    for name, g, r in zip(("dq", "dk", "dv"), got, g_ref):
        err = float(np.max(np.abs(f64(g) - r)) / np.max(np.abs(r)))
        say(f"  {w.name} {name} rel {err:.2e} (tol {tol})")
        assert err <= tol


def test_noalloc_matches_fa_bwd_twice_second_smaller(fa):
    say("noalloc: first call b2h4n700d128 bf16 causal")
    first = _case(fa, 2, 4, 700, 128, "bf16", True, 71)
    _check(*first)
    say("noalloc: second call b1h2n130d64 f16 (smaller)")
    second = _case(fa, 1, 2, 130, 64, "f16", False, 72)
    _check(*second)


def test_noalloc_refuses_oversized_shape(fa):
    """Past the static array's size the call fails before any launch."""
    t = torch.empty(16, dtype=torch.bfloat16, device="cuda")
    lse = torch.empty(4, dtype=torch.float32, device="cuda")
    P = t.data_ptr()
    st = fa.fa_bwd_noalloc(P, P, P, P, P, lse.data_ptr(), P, P, P, 2, 32, 131072, 128, 0, 0.088,
                           fa.FA_BF16, torch.cuda.current_stream().cuda_stream)
    assert st == fa.FA_ERR_WORKSPACE
