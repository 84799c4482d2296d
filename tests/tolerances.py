"""Parity bounds of the HIP path against the fp64 oracle, per storage type.

O and the gradients (max-abs error; gradients relative to the reference's
max-abs) for fp16 and bf16 are the bounds the method is held to.  LSE: the
16-bit forward sums P~ as rounded to the input type (the values the P~V
product uses), so ln l carries up to that type's unit roundoff u: 2^-11
(fp16), 2^-8 (bf16); the bounds are 1e-3 and 4e-3.  fp32 has no stated bound:
1e-5 on O, 1e-4 on LSE and gradients, from fp32 MFMA accumulation over a few
thousand terms.  Shared by the GPU parity tests and ``smoke()``."""
TOL = {
    "f32": dict(o=1e-5, lse=1e-4, grad=1e-4),
    "f16": dict(o=2e-3, lse=1e-3, grad=5e-3),
    "bf16": dict(o=1e-2, lse=4e-3, grad=2e-2),
}


def o_bound(dtype, o_ref):
    """The O bound scaled to the binade of the largest output.  The plain bounds
    hold for |O| < 4 (a convex combination of N(0,1) rows rarely leaves it);
    where |O| reaches higher binades (dropout's 1 / keep scaling, or very
    peaked rows that select single large values of V), the final rounding of O
    to the storage type alone is proportionally larger (a half ulp of bf16 at
    |O| in [4, 8) is 2^-6 = 0.0156)."""
    import math

    import numpy as np
    m = float(np.nanmax(np.abs(o_ref)))
    return TOL[dtype]["o"] * max(1.0, 2.0 ** math.ceil(math.log2(max(m, 1e-30))) / 4.0)
