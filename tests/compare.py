"""The comparison rule for attention outputs against the fp64 oracle.

|gpu_i - ref_i| <= tol * max_j |ref_j| + ulp_out(ref_i), elementwise, where
tol is 2e-3 for fp16/bf16 outputs and 1e-5 for fp32 outputs (max abs error
relative to the output magnitude), and ulp_out is one unit in the last place
of the output dtype at ref_i (the output itself is rounded to that dtype).
"""

import numpy as np

TOL = {"f32": 1e-5, "f16": 2e-3, "bf16": 2e-3}
MANT = {"f32": 23, "f16": 10, "bf16": 7}
MIN_EXP = {"f32": -126, "f16": -14, "bf16": -126}


def ulp(x, dtype):
    """One unit in the last place of `dtype` at |x| (subnormal spacing below
    the smallest normal)."""
    a = np.abs(np.asarray(x, dtype=np.float64))
    e = np.floor(np.log2(np.where(a > 0, a, 1.0)))
    e = np.maximum(e, MIN_EXP[dtype])
    return np.ldexp(1.0, (e - MANT[dtype]).astype(np.int64))


def check(gpu, ref, dtype, what=""):
    """Assert the rule; return (max relative error, elements needing the ulp)."""
    g = np.asarray(gpu, dtype=np.float64)
    r = np.asarray(ref, dtype=np.float64)
    assert g.shape == r.shape, (g.shape, r.shape)
    assert np.all(np.isfinite(g)), "%s: non-finite output" % what
    if r.size == 0:
        return 0.0, 0
    scale = np.abs(r).max()
    err = np.abs(g - r)
    bound = TOL[dtype] * scale + ulp(r, dtype)
    bad = err > bound
    if bad.any():
        i = np.unravel_index(np.argmax(err - bound), err.shape)
        raise AssertionError(
            "%s: %d of %d elements outside tolerance; worst at %s: gpu %r ref %r "
            "(err %.3g, bound %.3g, max|ref| %.3g)" % (what, bad.sum(), bad.size, i, g[i], r[i],
                                                       err[i], bound[i], scale))
    rel = float(err.max() / scale) if scale > 0 else float(err.max())
    return rel, int((err > TOL[dtype] * scale).sum())
