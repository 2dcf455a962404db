"""Acceptance gates for GPU results against the oracle (tests only).

Tolerance (element-wise, fp64):  |C_gpu - S| <= 2^-8 |C_ref| + 1e-5 sum_k |a_ik b_jk|
  S      the oracle's unrounded fp64 sum,
  C_ref  the oracle's bf16 result (S rounded once, nearest-even),
  absS   the oracle's sum of |products|.
2^-8 is bf16's unit roundoff (one nearest-even rounding); 1e-5 absS allows
for fp32 accumulation in any order.  Read against the rounded C_ref (the
"literal" form) a correct fp32 GEMM can differ from C_ref by one bf16 ulp where
S sits next to a rounding midpoint; the literal form is reported, and each of
its failures must be exactly such a flip.
"""
import numpy as np

from tests.exact import widen

REL = 2.0 ** -8
ABS_SUM = 1e-5


def compare(c_bits, c_ref_bits, S, absS):
    """Check one result; returns a dict of counts; raises AssertionError on a real mismatch."""
    c = widen(c_bits)
    cref = widen(c_ref_bits)
    S = np.asarray(S, dtype=np.float64)
    absS = np.asarray(absS, dtype=np.float64)
    assert c.shape == cref.shape == S.shape == absS.shape
    finite = np.isfinite(c)
    assert finite.all(), "non-finite outputs: %d" % int((~finite).sum())
    bound = REL * np.abs(cref) + ABS_SUM * absS
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
            assert abs(S[i] - mid) <= ABS_SUM * absS[i], ("flip far from a midpoint", i)
            flips += 1
    exact = int((np.asarray(c_bits) == np.asarray(c_ref_bits)).sum())
    return dict(elements=int(c.size), bit_exact=exact, literal_flips=flips,
                max_err_over_absS=float(np.max(err_g / np.maximum(absS, 1e-300))) if c.size else 0.0)
