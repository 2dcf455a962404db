"""Pins for the CPU oracle (no GPU).

The oracle computes C = A * B^T with fp64 sums and one nearest-even bf16
rounding (FlyDSL "Prebuilt kernels guide", section 3.1 for the operation,
section 1.1 for the bf16 rounding).  Every check here compares it with
something other than itself: the bf16 format definition and IEEE ties-to-even
(golden cases), numpy's and torch's conversions, exact integer and rational
arithmetic, identities (all-ones, identity matrices) and the fp64 summation
error bound.  The mutation test plants plausible mistakes in a copy of the
oracle source and checks that these pins catch every one.
"""
import os
import shutil
import tempfile
from fractions import Fraction

import math

import numpy as np
import pytest

import oracle
from tests import exact
import workloads

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "bf16_rne_cases.txt")


def _golden_cases():
    cases = []
    for ln in open(GOLDEN):
        if ln.startswith("#") or not ln.strip():
            continue
        x, e = ln.split()[:2]
        cases.append((float.fromhex(x), int(e, 16)))
    return cases


# ---------------------------------------------------------------- pin checks
# Each check takes an Oracle so the mutation test can run it on a variant.

def check_value_exhaustive(O):
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    ref = exact.widen(bits)
    got = np.array([O.bf16_value(int(b)) for b in bits], dtype=np.float64)
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(got), nan)
    assert np.array_equal(got[~nan], ref[~nan])
    # signs of zeros
    assert np.signbit(got[0x8000]) and not np.signbit(got[0])


def check_roundtrip_exhaustive(O):
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    vals = exact.widen(bits)
    fin = np.isfinite(vals)
    back = O.bf16_rne_array(vals[fin])
    assert np.array_equal(back, bits[fin])


def check_golden_ties(O):
    for x, e in _golden_cases():
        assert O.bf16_rne(x) == e, (x.hex(), hex(e), hex(O.bf16_rne(x)))


def check_rne_vs_float32_bit_rounding(O, n=100_000):
    # For inputs that are exactly float32, f64 -> bf16 and f32 -> bf16 rounding
    # agree; the latter is the integer bit recipe (and torch's conversion).
    rng = np.random.default_rng(1234)
    u = rng.integers(0, 2**32, size=n, dtype=np.uint64).astype(np.uint32)
    x32 = u.view(np.float32)
    keep = np.isfinite(x32) & (np.abs(x32) < np.float32(3.0e38))
    x32 = x32[keep]
    ref = workloads.f32_to_bf16_bits(x32)
    got = O.bf16_rne_array(x32.astype(np.float64))
    assert np.array_equal(got, ref)
    try:
        import torch
    except ImportError:
        return
    tref = torch.from_numpy(x32.copy()).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(got, tref)


def check_all_ones(O):
    for K in (256, 4096, 8192, 12288):
        A = np.full((3, K), 0x3F80, dtype=np.uint16)
        B = np.full((5, K), 0x3F80, dtype=np.uint16)
        C, S, absS = O.gemm(A, B)
        assert np.all(S == K) and np.all(absS == K)
        assert np.all(C == exact.round_exact(K))


def check_identity(O):
    rng = np.random.default_rng(7)
    K = 64
    I = np.zeros((K, K), dtype=np.uint16)
    I[np.arange(K), np.arange(K)] = 0x3F80
    Bm = workloads.draw(rng, (40, K), ("normal", 0.0, 1.0))
    C, _, _ = O.gemm(I, Bm)                 # A = I  ->  C = B^T
    assert np.array_equal(C, Bm.T)
    Am = workloads.draw(rng, (33, K), ("uniform", -1.0, 1.0))
    C, _, _ = O.gemm(Am, I)                 # B = I  ->  C = A
    assert np.array_equal(C, Am)


def check_small_integers(O):
    # Integer entries in [-4, 4]: every partial sum is an exact integer, so the
    # result must equal the exact int64 product A @ B^T, rounded once.
    rng = np.random.default_rng(11)
    M, N, K = 37, 29, 131
    ai = rng.integers(-4, 5, size=(M, K))
    bi = rng.integers(-4, 5, size=(N, K))
    A = workloads.f32_to_bf16_bits(ai.astype(np.float32))
    B = workloads.f32_to_bf16_bits(bi.astype(np.float32))
    C, S, absS = O.gemm(A, B)
    ref = ai.astype(np.int64) @ bi.astype(np.int64).T
    assert np.array_equal(S, ref.astype(np.float64))
    assert np.array_equal(absS, (np.abs(ai)[:, None, :] * np.abs(bi)[None, :, :]).sum(-1).astype(np.float64))
    want = np.array([[exact.round_exact(int(v)) for v in row] for row in ref], dtype=np.uint16)
    assert np.array_equal(C, want)


def check_brute_force_tiny(O):
    # Random bf16 over a wide exponent range, tiny shapes, exact rationals.
    rng = np.random.default_rng(5)
    for trial in range(6):
        M, N, K = [int(v) for v in rng.integers(1, 9, size=3)]
        mant = rng.uniform(-2.0, 2.0, size=(M + N, K))
        scale = 2.0 ** rng.integers(-20, 21, size=(M + N, K))
        bits = workloads.f32_to_bf16_bits((mant * scale).astype(np.float32))
        A, B = bits[:M], bits[M:]
        C, S, absS = O.gemm(A, B)
        for i in range(M):
            for j in range(N):
                s, sa = exact.exact_dot(A[i], B[j])
                assert abs(Fraction(S[i, j]) - s) <= K * Fraction(2) ** -53 * sa
                assert abs(Fraction(absS[i, j]) - sa) <= K * Fraction(2) ** -53 * sa
                assert C[i, j] == exact.round_exact(s), (trial, i, j)


def check_fp64_bound_workload(O):
    # tiny_256 inputs: sampled entries against the exact sum.
    A, B = workloads.workload_inputs("tiny_256")
    K = A.shape[1]
    rng = np.random.default_rng(3)
    ii = rng.integers(0, A.shape[0], size=120)
    jj = rng.integers(0, B.shape[0], size=120)
    C, S, absS = O.gemm_entries(A, B, ii, jj)
    for t in range(ii.size):
        s, sa = exact.exact_dot(A[ii[t]], B[jj[t]])
        assert abs(Fraction(S[t]) - s) <= K * Fraction(2) ** -53 * sa
        assert Fraction(absS[t]) == sa or abs(Fraction(absS[t]) - sa) <= K * Fraction(2) ** -53 * sa
        assert C[t] == exact.round_exact(s)


def check_transpose_symmetry(O):
    # C(A, B) = C(B, A)^T element for element (same dot products, same k order);
    # and (A, -B) negates every element.
    A, B = workloads.make_inputs(19, 23, 77, seed=9)
    C1, S1, _ = O.gemm(A, B)
    C2, S2, _ = O.gemm(B, A)
    assert np.array_equal(C1, C2.T) and np.array_equal(S1, S2.T)
    C3, S3, _ = O.gemm(A, B ^ np.uint16(0x8000))
    assert np.array_equal(S3, -S1)


# ---------------------------------------------------------------- epilogue
# Fused epilogues of the FlyDSL prebuilt kernels guide (section 3.1): bias
# per column, then ReLU, SiLU or GELU, on the unrounded sum, rounded once.

def check_epilogue_bias_exact(O):
    # All-ones operands make S = K exactly; x = K + b is then known exactly
    # in rationals (fp64 holds it to one rounding) and the results are known
    # in closed form for bias and ReLU: C = round(K + b), round(max(K + b, 0)).
    K = 256
    A = np.full((3, K), 0x3F80, dtype=np.uint16)
    B = np.full((7, K), 0x3F80, dtype=np.uint16)
    bvals = [-300.0, -256.0, -0.5, 0.0, 1.0, 3.5, 2.0 ** -130]
    bias = workloads.f32_to_bf16_bits(np.array(bvals, dtype=np.float32))
    bias[3] = 0x8000                                  # -0 adds nothing
    _, S, _ = O.gemm(A, B)
    xs = [Fraction(K) + Fraction(float(v)) for v in exact.widen(bias).tolist()]
    C, Y = O.epilogue(S, bias, "bias")
    ulp = Fraction(2) ** -52
    for j, x in enumerate(xs):
        assert abs(Fraction(Y[0, j]) - x) <= ulp * abs(x) and C[1, j] == exact.round_exact(x), j
    C, Y = O.epilogue(S, bias, "bias_relu")
    for j, x in enumerate(xs):
        want = x if x > 0 else Fraction(0)
        assert abs(Fraction(Y[2, j]) - want) <= ulp * want and C[2, j] == exact.round_exact(want), j
    assert C[0, 1] == 0x0000                          # relu(0) is +0
    C0, Y0 = O.epilogue(S, bias, "none")              # plain GEMM: bias unused
    assert np.all(Y0 == K) and np.all(C0 == exact.round_exact(K))


def check_epilogue_closed_forms(O):
    # sigmoid(ln 3) = 3/4 exactly, so SiLU(ln 3) = (3/4) ln 3; the 0.975
    # quantile of the standard normal, 1.959963984540054, gives
    # GELU(q) = 0.975 q; both activations have slope 1/2 at 0.
    l3 = math.log(3.0)
    assert abs(O.activation(l3, "bias_silu") - 0.75 * l3) <= 1e-15
    q = 1.959963984540054
    assert abs(O.activation(q, "bias_gelu") - 0.975 * q) <= 1e-14
    assert abs(O.activation(-q, "bias_gelu") + 0.025 * q) <= 1e-14
    for name in ("bias_silu", "bias_gelu"):
        h = 1e-9
        assert abs(O.activation(h, name) / h - 0.5) <= 1e-8, name
        assert O.activation(0.0, name) == 0.0
    assert O.activation(-2.5, "bias_relu") == 0.0 and O.activation(2.5, "bias_relu") == 2.5
    assert O.activation(-2.5, "bias") == -2.5


def check_epilogue_odd_parts(O):
    # x sigmoid(x) - (-x) sigmoid(-x) = x and x Phi(x) - (-x) Phi(-x) = x.
    for x in (0.125, 0.5, 1.0, 2.5, 7.0, 20.0, 40.0):
        for name in ("bias_silu", "bias_gelu"):
            d = O.activation(x, name) - O.activation(-x, name)
            assert abs(d - x) <= 4e-16 * x, (name, x, d)
    # the far left tail stays a tiny negative number, not a cancellation zero
    g = O.activation(-10.0, "bias_gelu")
    assert -1e-21 < g < -1e-24


def check_epilogue_columns(O):
    # One bias value per column: row layout and explicit column indices agree,
    # and a column shift is visible.
    rng = np.random.default_rng(21)
    S = rng.normal(0.0, 3.0, size=(5, 9))
    bias = workloads.f32_to_bf16_bits(rng.normal(0.0, 1.0, size=9).astype(np.float32))
    for name in ("bias", "bias_relu", "bias_silu", "bias_gelu"):
        C, Y = O.epilogue(S, bias, name)
        jj = np.tile(np.arange(9), 5)
        Ce, Ye = O.epilogue(S.ravel(), bias, name, cols=jj)
        assert np.array_equal(Ce, C.ravel()) and np.array_equal(Ye, Y.ravel())
        for j in (0, 4, 8):
            x = S[2, j] + float(exact.widen(bias[j]))
            assert Y[2, j] == O.activation(x, name)
            assert C[2, j] == O.bf16_rne(Y[2, j])


# ------------------------------------------------------------------ MXFP8
# Block-scaled FP8 GEMM (FlyDSL-in-PyTorch blog, MXFP section): E4M3 values,
# one E8M0 scale per 32 along K.

def _torch_e4m3(codes):
    import torch
    return torch.from_numpy(np.ascontiguousarray(codes, dtype=np.uint8)).view(torch.float8_e4m3fn).double().numpy()


def check_e4m3_exhaustive(O):
    # Every E4M3 code against torch's float8_e4m3fn (an independent decoder).
    ref = _torch_e4m3(np.arange(256, dtype=np.uint8))
    got = np.array([O.e4m3_value(b) for b in range(256)])
    nan = np.isnan(ref)
    assert np.array_equal(nan, np.isnan(got))
    assert np.array_equal(got[~nan], ref[~nan])
    assert np.array_equal(np.signbit(got[~nan]), np.signbit(ref[~nan]))
    assert O.e4m3_value(0x7E) == 448.0 and nan.sum() == 2


def check_e8m0_exhaustive(O):
    import torch
    ref = torch.arange(256, dtype=torch.uint8).view(torch.float8_e8m0fnu).double().numpy()
    got = np.array([O.e8m0_value(b) for b in range(256)])
    assert np.isnan(got[255]) and np.isnan(ref[255])
    assert np.array_equal(got[:255], ref[:255])
    assert all(got[e] == 2.0 ** (e - 127) for e in range(255))


def check_mx_all_ones(O):
    # E4M3 0x38 is 1.0; unit scales (code 127): C = K exactly.
    for K in (128, 4096):
        A = np.full((3, K), 0x38, dtype=np.uint8)
        B = np.full((5, K), 0x38, dtype=np.uint8)
        s = np.full((3, K // 32), 127, dtype=np.uint8)
        t = np.full((5, K // 32), 127, dtype=np.uint8)
        C, S, absS = O.mx_gemm(A, s, B, t)
        assert np.all(S == K) and np.all(absS == K) and np.all(C == exact.round_exact(K))


def check_mx_unit_scales_equal_bf16_gemm(O):
    # With unit scales the MX product is the bf16 product of the same values
    # (every E4M3 value is a bf16 value): pinned to the bf16 oracle.
    A, SA, B, SB = workloads.make_mx_inputs(9, 7, 96, seed=3)
    SA[:] = 127
    SB[:] = 127
    ab = workloads.f32_to_bf16_bits(_torch_e4m3(A).astype(np.float32))
    bb = workloads.f32_to_bf16_bits(_torch_e4m3(B).astype(np.float32))
    C1, S1, a1 = O.mx_gemm(A, SA, B, SB)
    C2, S2, a2 = O.gemm(ab, bb)
    assert np.array_equal(S1, S2) and np.array_equal(a1, a2) and np.array_equal(C1, C2)


def check_mx_scales_are_powers_of_two(O):
    # Raising row i's scales by d multiplies row i of S by 2^d exactly; a
    # column's scales likewise; and a block's scale reaches only its block:
    # with all codes zero outside block b, the row equals block b's product.
    A, SA, B, SB = workloads.make_mx_inputs(6, 5, 128, seed=4)
    _, S, _ = O.mx_gemm(A, SA, B, SB)
    SA2 = SA.copy(); SA2[2] += 3
    SB2 = SB.copy(); SB2[4] -= 2
    _, S2, _ = O.mx_gemm(A, SA2, B, SB2)
    want = S.copy(); want[2] *= 8.0; want[:, 4] *= 0.25
    assert np.array_equal(S2, want)
    Az = A.copy(); Az[:, :64] = 0; Az[:, 96:] = 0          # keep block 2 only
    _, Sz, _ = O.mx_gemm(Az, SA, B, SB)
    SA3 = SA.copy(); SA3[:, 0] += 5; SA3[:, 1] -= 4; SA3[:, 3] += 1
    _, Sz3, _ = O.mx_gemm(Az, SA3, B, SB)
    assert np.array_equal(Sz, Sz3)


def check_mx_brute_force_tiny(O):
    # Exact rationals from torch's decode and the scale definition.
    rng = np.random.default_rng(17)
    for trial in range(4):
        M, N = [int(v) for v in rng.integers(1, 5, size=2)]
        K = 64
        A = rng.integers(0, 256, size=(M, K)).astype(np.uint8)
        B = rng.integers(0, 256, size=(N, K)).astype(np.uint8)
        A[(A & 0x7F) == 0x7F] = 0x11                      # no NaN codes
        B[(B & 0x7F) == 0x7F] = 0x22
        SA = rng.integers(100, 150, size=(M, 2)).astype(np.uint8)
        SB = rng.integers(100, 150, size=(N, 2)).astype(np.uint8)
        av, bv = _torch_e4m3(A), _torch_e4m3(B)
        C, S, absS = O.mx_gemm(A, SA, B, SB)
        for i in range(M):
            for j in range(N):
                s = sum(Fraction(float(av[i, k])) * Fraction(2) ** (int(SA[i, k // 32]) - 127) *
                        Fraction(float(bv[j, k])) * Fraction(2) ** (int(SB[j, k // 32]) - 127) for k in range(K))
                sa = sum(abs(Fraction(float(av[i, k])) * Fraction(float(bv[j, k]))) *
                         Fraction(2) ** (int(SA[i, k // 32]) + int(SB[j, k // 32]) - 254) for k in range(K))
                assert abs(Fraction(S[i, j]) - s) <= K * Fraction(2) ** -53 * sa, (trial, i, j)
                assert C[i, j] == exact.round_exact(s), (trial, i, j)


# ------------------------------------------------------------ grouped GEMM
# FlyDSL-in-PyTorch blog, grouped GEMM section: concatenated expert rows,
# one weight per expert, cumulative row-end offsets.

def check_grouped_one_expert_is_dense(O):
    A, B = workloads.make_inputs(37, 21, 96, seed=11)
    C1, S1, a1 = O.grouped_gemm(A, B[None], np.array([37], np.int32))
    C2, S2, a2 = O.gemm(A, B)
    assert np.array_equal(C1, C2) and np.array_equal(S1, S2) and np.array_equal(a1, a2)


def check_grouped_expert_identity(O):
    # All-ones activations; expert g's weight is all (g + 1) (exact bf16
    # integers), so row i's outputs are K (g + 1) with g its expert: fixes
    # every boundary, empty experts (repeated offsets) included.
    K, N = 64, 5
    offs = np.array([0, 3, 3, 9, 10, 10, 17], dtype=np.int32)       # experts 0, 2, 5 empty
    G, M = offs.size, 20
    A = np.full((M, K), 0x3F80, dtype=np.uint16)
    vals = np.arange(1, G + 1, dtype=np.float32)
    B = np.repeat(workloads.f32_to_bf16_bits(vals)[:, None, None], N, axis=1).repeat(K, axis=2)
    C, S, _ = O.grouped_gemm(A, B, offs)
    assert C.shape == (17, N)
    want_g = np.searchsorted(offs, np.arange(17), side="right")
    assert np.array_equal(S, np.repeat((K * (want_g + 1.0))[:, None], N, axis=1))


def check_grouped_permutation(O):
    # Reordering the experts (with their rows) reorders the output rows.
    rng = np.random.default_rng(4)
    sizes = np.array([5, 0, 9, 3])
    A, _ = workloads.make_inputs(int(sizes.sum()), 1, 64, seed=5)
    B = workloads.draw(rng, (4, 11, 64), ("uniform", -1.0, 1.0))
    offs = np.cumsum(sizes).astype(np.int32)
    C, S, _ = O.grouped_gemm(A, B, offs)
    perm = [2, 0, 3, 1]
    starts = np.concatenate([[0], offs[:-1]])
    rows = np.concatenate([np.arange(starts[g], offs[g]) for g in perm]).astype(np.int64)
    C2, S2, _ = O.grouped_gemm(A[rows], B[perm], np.cumsum(sizes[perm]).astype(np.int32))
    assert np.array_equal(C2, C[rows]) and np.array_equal(S2, S[rows])


def check_grouped_brute_force_tiny(O):
    rng = np.random.default_rng(12)
    A = workloads.draw(rng, (6, 16), ("normal", 0.0, 1.0))
    B = workloads.draw(rng, (3, 4, 16), ("normal", 0.0, 1.0))
    offs = np.array([2, 2, 6], dtype=np.int32)
    C, S, absS = O.grouped_gemm(A, B, offs)
    av, bv = exact.widen(A), exact.widen(B)
    for i in range(6):
        g = 0 if i < 2 else 2
        for j in range(4):
            s = sum(Fraction(float(av[i, k])) * Fraction(float(bv[g, j, k])) for k in range(16))
            assert abs(Fraction(S[i, j]) - s) <= 16 * Fraction(2) ** -53 * Fraction(absS[i, j])
            assert C[i, j] == exact.round_exact(s)


# ------------------------------------------------------------------ layouts
def _stored(X, col, ld, fill):
    """X (rows x K logical) stored in row layout (rows x ld) or column layout
    (K x ld), padding filled with `fill`."""
    rows, K = X.shape
    if col:
        st = np.full((K, ld), fill, dtype=np.uint16)
        st[:, :rows] = X.T
    else:
        st = np.full((rows, ld), fill, dtype=np.uint16)
        st[:, :K] = X
    return st


def check_layouts_equal_dense(O):
    # Every layout pair with padded leading dimensions; padding is a NaN
    # pattern, so a read of it would show as NaN sums.
    A, B = workloads.make_inputs(13, 9, 40, seed=21)
    C0, S0, a0 = O.gemm(A, B)
    for a_col in (False, True):
        for b_col in (False, True):
            lda = (13 if a_col else 40) + 3
            ldb = (9 if b_col else 40) + 5
            C, S, absS = O.gemm_layout(_stored(A, a_col, lda, 0x7FC1), lda, a_col,
                                       _stored(B, b_col, ldb, 0xFFC3), ldb, b_col, 13, 9, 40)
            assert np.array_equal(C, C0) and np.array_equal(S, S0) and np.array_equal(absS, a0), (a_col, b_col)


def check_layout_index_roles(O):
    # A square case where a transposed read would be in bounds: column layout
    # of A must read A^T's storage as A, not as A^T.
    rng = np.random.default_rng(8)
    A = workloads.draw(rng, (16, 16), ("uniform", -1.0, 1.0))
    B = workloads.draw(rng, (16, 16), ("uniform", -1.0, 1.0))
    C0, S0, _ = O.gemm(A, B)
    C1, S1, _ = O.gemm_layout(np.ascontiguousarray(A.T), 16, True, B, 16, False, 16, 16, 16)
    C2, S2, _ = O.gemm_layout(A, 16, False, np.ascontiguousarray(B.T), 16, True, 16, 16, 16)
    assert np.array_equal(S1, S0) and np.array_equal(S2, S0)
    C3, S3, _ = O.gemm(np.ascontiguousarray(A.T), B)
    assert not np.array_equal(S3, S0)                       # the check above can fail


# ------------------------------------------------------------------ MXFP4
# Block-scaled FP4 GEMM (FlyDSL-in-PyTorch blog, MXFP section): packed E2M1
# values, one E8M0 scale per 32 along K.

# The E2M1 magnitudes of codes 0-7 as the OCP MX format defines them (sign
# bit 3, two exponent bits with bias 1, one fraction bit: 0, 0.5 subnormal;
# then 1.f * 2^(e - 1)).
E2M1_MAGNITUDES = [0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0]


def _e2m1_as_e4m3(code):
    # The E4M3 code of the same value, by bit fields (an independent route to
    # the value through torch's float8_e4m3fn decoder).
    s, e, f = (code >> 3) & 1, (code >> 1) & 3, code & 1
    if e == 0 and f == 0:
        return s << 7
    if e == 0:                                   # 0.5 = 1.0 * 2^-1
        return (s << 7) | (6 << 3)
    return (s << 7) | ((e + 6) << 3) | (f << 2)


def check_e2m1_magnitudes(O):
    got = [O.e2m1_value(c) for c in range(16)]
    assert got[:8] == E2M1_MAGNITUDES
    assert got[8:] == [-m for m in E2M1_MAGNITUDES]
    assert np.signbit(got[8]) and not np.signbit(got[0])


def check_e2m1_via_e4m3(O):
    ref = _torch_e4m3(np.array([_e2m1_as_e4m3(c) for c in range(16)], dtype=np.uint8))
    got = np.array([O.e2m1_value(c) for c in range(16)])
    assert np.array_equal(got, ref) and np.array_equal(np.signbit(got), np.signbit(ref))


def check_mx4_equals_mx8_of_same_values(O):
    # Every E2M1 value is an E4M3 value: the MXFP4 product equals the (pinned)
    # MXFP8 product of the re-encoded codes with the same scales, bit for bit.
    to8 = np.array([_e2m1_as_e4m3(c) for c in range(16)], dtype=np.uint8)
    for (M, N, K, seed) in ((7, 9, 128, 1), (3, 20, 256, 2)):
        A, SA, B, SB = workloads.make_mx4_inputs(M, N, K, sa=(110, 140), sb=(110, 140), seed=seed)
        A8, B8 = to8[workloads.unpack_e2m1(A)], to8[workloads.unpack_e2m1(B)]
        C4, S4, a4 = O.mx4_gemm(A, SA, B, SB)
        C8, S8, a8 = O.mx_gemm(A8, SA, B8, SB)
        assert np.array_equal(S4, S8) and np.array_equal(a4, a8) and np.array_equal(C4, C8)


def check_mx4_all_ones(O):
    # E2M1 code 2 is 1.0 (byte 0x22 holds two); unit scales: C = K exactly.
    for K in (128, 4096):
        A = np.full((3, K // 2), 0x22, dtype=np.uint8)
        B = np.full((5, K // 2), 0x22, dtype=np.uint8)
        C, S, absS = O.mx4_gemm(A, np.full((3, K // 32), 127, np.uint8), B, np.full((5, K // 32), 127, np.uint8))
        assert np.all(S == K) and np.all(absS == K) and np.all(C == exact.round_exact(K))


def check_mx4_blocks_and_pairing(O):
    # A one-hot at k in both operands gives exactly the product of the two
    # values times 2^(sa + sb) with the scales of block k / 32, and a one-hot
    # in the other nibble of the same byte pairs with nothing.  (Which nibble
    # holds k even changes only the order of the fp64 sum, which the exact
    # MXFP8 comparison above sees.)
    K = 128
    for k in (0, 1, 31, 32, 77, 127):
        A = np.zeros((1, K // 2), np.uint8)
        B = np.zeros((1, K // 2), np.uint8)
        A[0, k // 2] = 0x3 << (4 * (k & 1))                # 1.5 at k
        B[0, k // 2] = 0x7 << (4 * (k & 1))                # 6.0 at k
        SA = np.full((1, K // 32), 127, np.uint8); SA[0, k // 32] = 130
        SB = np.full((1, K // 32), 127, np.uint8); SB[0, k // 32] = 125
        _, S, _ = O.mx4_gemm(A, SA, B, SB)
        assert S[0, 0] == 1.5 * 6.0 * 2.0 ** (3 - 2), k
        B2 = np.zeros_like(B); B2[0, k // 2] = 0x7 << (4 * (1 - (k & 1)))
        _, S2, _ = O.mx4_gemm(A, SA, B2, SB)
        assert S2[0, 0] == 0.0, k


def check_mx4_brute_force_tiny(O):
    # Exact rationals from the magnitude list and the scale definition.
    rng = np.random.default_rng(23)
    val = [Fraction(m) for m in E2M1_MAGNITUDES] + [-Fraction(m) for m in E2M1_MAGNITUDES]
    for trial in range(4):
        M, N = [int(v) for v in rng.integers(1, 5, size=2)]
        K = 64
        a = rng.integers(0, 16, size=(M, K)).astype(np.uint8)
        b = rng.integers(0, 16, size=(N, K)).astype(np.uint8)
        SA = rng.integers(100, 150, size=(M, 2)).astype(np.uint8)
        SB = rng.integers(100, 150, size=(N, 2)).astype(np.uint8)
        C, S, absS = O.mx4_gemm(workloads.pack_e2m1(a), SA, workloads.pack_e2m1(b), SB)
        for i in range(M):
            for j in range(N):
                s = sum(val[a[i, k]] * val[b[j, k]] * Fraction(2) ** (int(SA[i, k // 32]) + int(SB[j, k // 32]) - 254)
                        for k in range(K))
                sa = sum(abs(val[a[i, k]] * val[b[j, k]]) * Fraction(2) ** (int(SA[i, k // 32]) + int(SB[j, k // 32]) - 254)
                         for k in range(K))
                assert abs(Fraction(S[i, j]) - s) <= K * Fraction(2) ** -53 * sa, (trial, i, j)
                assert Fraction(absS[i, j]) == sa or abs(Fraction(absS[i, j]) - sa) <= K * Fraction(2) ** -53 * sa
                assert C[i, j] == exact.round_exact(s), (trial, i, j)


ALL_CHECKS = [check_value_exhaustive, check_roundtrip_exhaustive, check_golden_ties,
              check_rne_vs_float32_bit_rounding, check_all_ones, check_identity,
              check_small_integers, check_brute_force_tiny, check_fp64_bound_workload,
              check_transpose_symmetry, check_epilogue_bias_exact, check_epilogue_closed_forms,
              check_epilogue_odd_parts, check_epilogue_columns, check_e4m3_exhaustive,
              check_e8m0_exhaustive, check_mx_all_ones, check_mx_unit_scales_equal_bf16_gemm,
              check_mx_scales_are_powers_of_two, check_mx_brute_force_tiny, check_grouped_one_expert_is_dense,
              check_grouped_expert_identity, check_grouped_permutation, check_grouped_brute_force_tiny,
              check_layouts_equal_dense, check_layout_index_roles, check_e2m1_magnitudes, check_e2m1_via_e4m3,
              check_mx4_equals_mx8_of_same_values, check_mx4_all_ones, check_mx4_blocks_and_pairing,
              check_mx4_brute_force_tiny]


@pytest.fixture(scope="module")
def O():
    oracle.build()
    return oracle.Oracle()


@pytest.mark.parametrize("check", ALL_CHECKS, ids=lambda c: c.__name__)
def test_oracle_pin(O, check):
    check(O)


def test_empty_and_degenerate(O):
    A = np.zeros((4, 0), dtype=np.uint16)
    B = np.zeros((3, 0), dtype=np.uint16)
    C, S, absS = O.gemm(A, B)          # K = 0: the empty sum is +0
    assert C.shape == (4, 3) and np.all(C == 0) and np.all(S == 0)
    C, _, _ = O.gemm(np.zeros((0, 5), np.uint16), np.zeros((2, 5), np.uint16))
    assert C.shape == (0, 2)


def test_rows_and_entries_consistent(O):
    A, B = workloads.make_inputs(70, 45, 96, seed=2)
    C, S, absS = O.gemm(A, B)
    Cr, Sr, _ = O.gemm(A, B, rows=(13, 51))
    assert np.array_equal(Cr, C[13:51]) and np.array_equal(Sr, S[13:51])
    ii = np.array([0, 69, 13, 40]); jj = np.array([44, 0, 7, 21])
    Ce, Se, ae = O.gemm_entries(A, B, ii, jj)
    assert np.array_equal(Ce, C[ii, jj]) and np.array_equal(Se, S[ii, jj])
    assert np.array_equal(ae, absS[ii, jj])


def test_mx_rows_and_entries_consistent(O):
    A, SA, B, SB = workloads.make_mx_inputs(40, 33, 160, seed=6)
    C, S, absS = O.mx_gemm(A, SA, B, SB)
    Cr, Sr, _ = O.mx_gemm(A, SA, B, SB, rows=(7, 29))
    assert np.array_equal(Cr, C[7:29]) and np.array_equal(Sr, S[7:29])
    ii = np.array([0, 39, 7, 20]); jj = np.array([32, 0, 5, 17])
    Ce, Se, ae = O.mx_gemm_entries(A, SA, B, SB, ii, jj)
    assert np.array_equal(Ce, C[ii, jj]) and np.array_equal(Se, S[ii, jj])
    assert np.array_equal(ae, absS[ii, jj])
    C1, S1, _ = O.mx_gemm(A, SA, B, SB, nthreads=1)
    assert np.array_equal(C1, C) and np.array_equal(S1, S)


def test_mx4_rows_and_entries_consistent(O):
    A, SA, B, SB = workloads.make_mx4_inputs(40, 33, 256, seed=6)
    C, S, absS = O.mx4_gemm(A, SA, B, SB)
    Cr, Sr, _ = O.mx4_gemm(A, SA, B, SB, rows=(7, 29))
    assert np.array_equal(Cr, C[7:29]) and np.array_equal(Sr, S[7:29])
    ii = np.array([0, 39, 7, 20]); jj = np.array([32, 0, 5, 17])
    Ce, Se, ae = O.mx4_gemm_entries(A, SA, B, SB, ii, jj)
    assert np.array_equal(Ce, C[ii, jj]) and np.array_equal(Se, S[ii, jj])
    assert np.array_equal(ae, absS[ii, jj])


def test_mx4_pack_round_trip():
    rng = np.random.default_rng(9)
    codes = rng.integers(0, 16, size=(5, 64)).astype(np.uint8)
    packed = workloads.pack_e2m1(codes)
    assert packed.shape == (5, 32) and np.array_equal(workloads.unpack_e2m1(packed), codes)
    assert packed[0, 0] == codes[0, 0] | (codes[0, 1] << 4)


def test_mx_quantizer_round_trips(O):
    # The input generator's MX quantisation: every block's largest magnitude
    # lands in [224, 448] after scaling and rounding (or the block is zero), and the decoded
    # values stay within one E4M3 rounding (2^-4 relative, or the subnormal
    # spacing 2^-9 of the scaled value) of the drawn ones.
    rng = np.random.default_rng(5)
    x = rng.normal(0.0, 1.0, size=(8, 256))
    x[3, 32:64] = 0.0
    A, SA = workloads.mx_quantize(x)
    dec = np.array([[O.e4m3_value(c) for c in row] for row in A])
    scale = np.repeat(np.array([[O.e8m0_value(e) for e in row] for row in SA]), 32, axis=1)
    amax = np.abs(dec).reshape(8, 8, 32).max(axis=2)
    assert np.all((amax >= 224) | (amax == 0)) and amax.max() <= 448
    assert amax[3, 1] == 0
    assert np.all(np.abs(dec * scale - x) <= (2.0 ** -4 * np.abs(x) + 2.0 ** -10 * scale))


def test_thread_count_does_not_change_result(O):
    A, B = workloads.make_inputs(64, 40, 300, seed=4)
    C1, S1, _ = O.gemm(A, B, nthreads=1)
    C4, S4, _ = O.gemm(A, B, nthreads=4)
    assert np.array_equal(C1, C4) and np.array_equal(S1, S4)


# ------------------------------------------------------------ mutation test
# Plausible mistakes planted in a copy of the oracle source; each must be
# caught by at least one pin above.
MUTANTS = {
    "sign_of_sum": ("double p = g_val[a_row[k]] * g_val[b_row[k]];\n        s += p;",
                    "double p = g_val[a_row[k]] * g_val[b_row[k]];\n        s -= p;"),
    "dropped_last_term": ("for (int64_t k = 0; k < K; ++k) {\n        double p = g_val",
                          "for (int64_t k = 0; k < K - 1; ++k) {\n        double p = g_val"),
    "mx_dropped_last_term": ("for (int64_t k = 0; k < K; ++k) {\n        double p = (g_e4m3",
                             "for (int64_t k = 0; k < K - 1; ++k) {\n        double p = (g_e4m3"),
    "mx_transposed_operands": ("mx_dot_one(A + i * K, SA + i * KB, B + j * K, SB + j * KB, K, &s, &sa);",
                               "mx_dot_one(A + j * K, SA + j * KB, B + i * K, SB + i * KB, K, &s, &sa);"),
    "reversed_b_index": ("g_val[b_row[k]]", "g_val[b_row[K - 1 - k]]"),
    "transposed_operands": ("dot_one(A + i * K, B + j * K, K, &s, &sa);",
                            "dot_one(A + j * K, B + i * K, K, &s, &sa);"),
    "truncating_rounding": ("double n = rint(ax / q);", "double n = floor(ax / q);"),
    "ties_away_from_zero": ("double n = rint(ax / q);", "double n = round(ax / q);"),
    "one_bit_too_many": ("double q = ldexp(1.0, E - 7);", "double q = ldexp(1.0, E - 8);"),
    "no_subnormal_clamp": ("        E = -126;                   /* bf16 subnormal range: fixed quantum */",
                           "        E = E;"),
    "abs_sum_signed": ("s += p;\n        sa += fabs(p);\n    }\n    *s_out = s;\n    *abs_out = sa;\n}\n\n/*\n * Rows",
                       "s += p;\n        sa += p;\n    }\n    *s_out = s;\n    *abs_out = sa;\n}\n\n/*\n * Rows"),
    "exponent_bias": ("mag = ldexp(1.0 + (double)f / 128.0, e - 127);",
                      "mag = ldexp(1.0 + (double)f / 128.0, e - 126);"),
    "negative_zero_sign": ("uint16_t sign = signbit(x) ? 0x8000 : 0;",
                           "uint16_t sign = (x < 0) ? 0x8000 : 0;"),
    "relu_as_abs": ("return x > 0.0 ? x : 0.0;", "return fabs(x);"),
    "silu_sign": ("return x / (1.0 + exp(-x));", "return x / (1.0 + exp(x));"),
    "gelu_tanh_form": ("return 0.5 * x * erfc(-x * M_SQRT1_2);",
                       "return 0.5 * x * (1.0 + tanh(0.7978845608028654 * (x + 0.044715 * x * x * x)));"),
    "gelu_wrong_tail": ("return 0.5 * x * erfc(-x * M_SQRT1_2);", "return 0.5 * x * erfc(x * M_SQRT1_2);"),
    "gelu_no_half": ("return 0.5 * x * erfc(-x * M_SQRT1_2);", "return x * erfc(-x * M_SQRT1_2);"),
    "gelu_cancelling_tail": ("return 0.5 * x * erfc(-x * M_SQRT1_2);",
                             "return 0.5 * x * (1.0 + erf(x * M_SQRT1_2));"),
    "bias_after_activation": ("y = hkg_oracle_activation(S[t] + hkg_oracle_bf16_value(bias[j]), epi);",
                              "y = hkg_oracle_activation(S[t], epi) + hkg_oracle_bf16_value(bias[j]);"),
    "bias_shifted_column": ("const int64_t j = cols ? cols[t] : t % N;",
                            "const int64_t j = cols ? cols[t] : (t + 1) % N;"),
    "layout_a_col_transposed": ("const uint16_t a = a_col ? A[k * lda + i] : A[i * lda + k];",
                                "const uint16_t a = a_col ? A[i * lda + k] : A[i * lda + k];"),
    "layout_b_stride_ignored": ("const uint16_t b = b_col ? B[k * ldb + j] : B[j * ldb + k];",
                                "const uint16_t b = b_col ? B[k * ldb + j] : B[j * K + k];"),
    "group_boundary_inclusive": ("if ((int64_t)offs[mid] > i)", "if ((int64_t)offs[mid] >= i)"),
    "group_next_expert": ("dot_one(A + i * K, B + (g * N + j) * K, K, &s, &sa);",
                          "dot_one(A + i * K, B + (((g + 1) % G) * N + j) * K, K, &s, &sa);"),
    "group_always_first": ("const int64_t g = group_of_row(offs, G, i);",
                           "const int64_t g = group_of_row(offs, G, i) < G ? 0 : G;"),
    "mx_one_scale_per_row": ("(g_e4m3[a_row[k]] * hkg_oracle_e8m0_value(sa_row[k / 32]))",
                             "(g_e4m3[a_row[k]] * hkg_oracle_e8m0_value(sa_row[0]))"),
    "mx_b_scaled_by_a": ("(g_e4m3[b_row[k]] * hkg_oracle_e8m0_value(sb_row[k / 32]))",
                         "(g_e4m3[b_row[k]] * hkg_oracle_e8m0_value(sa_row[k / 32]))"),
    "e8m0_bias": ("ldexp(1.0, (int)bits - 127)", "ldexp(1.0, (int)bits - 128)"),
    "e4m3_bias": ("mag = ldexp(1.0 + (double)f / 8.0, e - 7);", "mag = ldexp(1.0 + (double)f / 8.0, e - 8);"),
    "e4m3_subnormal_scale": ("mag = ldexp((double)f / 8.0, -6);", "mag = ldexp((double)f / 8.0, -7);"),
    "e4m3_ieee_style_nan": ("if (e == 0xF && f == 0x7)", "if (e == 0xF)"),
    "e2m1_exponent_bias": ("ldexp(1.0 + (double)f / 2.0, e - 1);", "ldexp(1.0 + (double)f / 2.0, e - 2);"),
    "e2m1_subnormal_scale": ("? (double)f / 2.0 ", "? (double)f "),
    "e2m1_sign_bit": ("int sign = (code >> 3) & 1;", "int sign = (code >> 2) & 1;"),
    "mx4_high_nibble_shift": ("(k & 1) ? byte >> 4 : byte & 0xF", "(k & 1) ? byte >> 3 : byte & 0xF"),
    "mx4_dropped_last_term": ("for (int64_t k = 0; k < K; ++k) {\n        double p = (mx4_element",
                              "for (int64_t k = 0; k < K - 1; ++k) {\n        double p = (mx4_element"),
    "mx4_one_scale_per_row": ("(mx4_element(a_row, k) * hkg_oracle_e8m0_value(sa_row[k / 32]))",
                              "(mx4_element(a_row, k) * hkg_oracle_e8m0_value(sa_row[0]))"),
    "mx4_b_scaled_by_a": ("(mx4_element(b_row, k) * hkg_oracle_e8m0_value(sb_row[k / 32]))",
                          "(mx4_element(b_row, k) * hkg_oracle_e8m0_value(sa_row[k / 32]))"),
    "mx4_scale_block_of_16": ("(mx4_element(a_row, k) * hkg_oracle_e8m0_value(sa_row[k / 32]))",
                              "(mx4_element(a_row, k) * hkg_oracle_e8m0_value(sa_row[k / 16]))"),
    "mx_abs_sum_signed": ("s += p;\n        sa += fabs(p);\n    }\n    *s_out = s;\n    *abs_out = sa;\n}\n\n/* Rows [row_begin, row_end) of the MXFP8",
                          "s += p;\n        sa += p;\n    }\n    *s_out = s;\n    *abs_out = sa;\n}\n\n/* Rows [row_begin, row_end) of the MXFP8"),
}


def _mutant_caught(path):
    O = oracle.Oracle(path)
    for check in ALL_CHECKS:
        try:
            check(O)
        except AssertionError:
            return check.__name__
    return None


@pytest.mark.skipif(shutil.which("gcc") is None, reason="gcc not available")
def test_pins_catch_planted_mistakes():
    src = open(oracle.SRC).read()
    tmp = tempfile.mkdtemp(prefix="hkg_mutants_")
    try:
        uncaught = []
        for name, (old, new) in MUTANTS.items():
            assert src.count(old) == 1, "mutation site not unique: " + name
            msrc = os.path.join(tmp, name + ".c")
            with open(msrc, "w") as f:
                f.write(src.replace(old, new))
            lib = os.path.join(tmp, "lib_" + name + ".so")
            oracle.build(force=True, src=msrc, out=lib)
            if _mutant_caught(lib) is None:
                uncaught.append(name)
        assert not uncaught, "mutants not caught by any pin: %s" % uncaught
    finally:
        shutil.rmtree(tmp, ignore_errors=True)
