"""Acceptance gates for GPU results against the oracle (tests only).

Tolerance (element-wise, fp64):  |C_gpu - S| <= 2^-8 |C_ref| + 1e-5 sum_k |a_ik b_jk|
  S      the oracle's unrounded fp64 sum,
  C_ref  the oracle's bf16 result (S rounded once, nearest-even),
  absS   the oracle's sum of |products|.
2^-8 is bf16's unit roundoff (one nearest-even rounding) for normal values;
below 2^-126 the rounding error is at most half the subnormal spacing, 2^-134,
which every bound includes (SUBNORMAL_HALF_ULP).  1e-5 absS allows for fp32
accumulation in any order.  Read against the rounded C_ref (the
"literal" form) a correct fp32 GEMM can differ from C_ref by one bf16 ulp where
S sits next to a rounding midpoint; the literal form is reported, and each of
its failures must be exactly such a flip.

Fused epilogues (y = act(S + bias)) use the same form with S replaced by the
oracle's unrounded Y and a wider allowance: the fp32 sum's error passes
through the activation with slope at most 1.13 (GELU; SiLU 1.10, ReLU 1), so
1.2e-5 absS; the fp32 bias add, exp/erfc and the products around them add a
few fp32 ulps, bounded by 2^-20 (|Y| + |bias|).
"""
import numpy as np

from tests.exact import widen

REL = 2.0 ** -8
SUBNORMAL_HALF_ULP = 2.0 ** -134
ABS_SUM = 1e-5


def compare(c_bits, c_ref_bits, S, absS, acc=ABS_SUM, extra=0.0):
    """Check one result; returns a dict of counts; raises AssertionError on a real mismatch.

    acc: allowance per unit of absS; extra: further absolute allowance
    (scalar or array), used by the epilogue gate."""
    c = widen(c_bits)
    cref = widen(c_ref_bits)
    S = np.asarray(S, dtype=np.float64)
    absS = np.asarray(absS, dtype=np.float64)
    assert c.shape == cref.shape == S.shape == absS.shape
    finite = np.isfinite(c)
    assert finite.all(), "non-finite outputs: %d" % int((~finite).sum())
    allow = acc * absS + np.asarray(extra, dtype=np.float64)
    bound = REL * np.abs(cref) + SUBNORMAL_HALF_ULP + allow
    err_g = np.abs(c - S)
    bad_g = err_g > bound
    if bad_g.any():
        idx = np.argwhere(bad_g)[:5]
        det = [(tuple(int(v) for v in i), float(c[tuple(i)]), float(S[tuple(i)]), float(bound[tuple(i)]))
               for i in idx]
        raise AssertionError("tolerance violated at %d of %d elements, e.g. (index, gpu, S, bound): %s"
                             % (int(bad_g.sum()), c.size, det))
    # Literal form against the rounded C_ref, with each failure explained.
    bad_l = np.abs(c - cref) > bound
    flips = 0
    if bad_l.any():
        for i in np.argwhere(bad_l):
            i = tuple(i)
            cb, rb = int(np.asarray(c_bits)[i]), int(np.asarray(c_ref_bits)[i])
            # 1-ulp neighbour: same sign, adjacent bit patterns
            assert (cb ^ rb) & 0x8000 == 0 and abs(cb - rb) == 1, ("not a 1-ulp flip", i, hex(cb), hex(rb))
            mid = (float(c[i]) + float(cref[i])) / 2.0
            assert abs(S[i] - mid) <= np.broadcast_to(allow, S.shape)[i], ("flip far from a midpoint", i)
            flips += 1
    exact = int((np.asarray(c_bits) == np.asarray(c_ref_bits)).sum())
    return dict(elements=int(c.size), bit_exact=exact, literal_flips=flips,
                max_err_over_absS=float(np.max(err_g / np.maximum(absS, 1e-300))) if c.size else 0.0)


EPI_ACC = 1.2e-5
EPI_REL_EXTRA = 2.0 ** -20


def compare_epilogue(c_bits, c_ref_bits, Y, absS, bias_vals):
    """Gate for a fused epilogue: Y the oracle's unrounded act(S + bias),
    bias_vals the bias value of each element's column (float64)."""
    Y = np.asarray(Y, dtype=np.float64)
    extra = EPI_REL_EXTRA * (np.abs(Y) + np.abs(np.asarray(bias_vals, dtype=np.float64)))
    return compare(c_bits, c_ref_bits, Y, absS, acc=EPI_ACC, extra=extra)
