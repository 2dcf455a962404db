"""The acceptance gates on the CPU: a float32 emulation of a correct GPU
result passes them, and plausible GPU mistakes fail them.

The emulation sums bf16 products in float32 in blocks of 32 k (the MFMA's k
step) then across blocks, adds the bias in float32, applies the activation in
float32 and rounds to bf16 nearest-even: what the kernels do, in another
order.  This checks that the tolerance derived in tests/gates.py is neither
too tight for a correct fp32 implementation nor so loose that a dropped
bias, a shifted column or the wrong activation passes.
"""
import numpy as np
import pytest
from scipy import special

import oracle
import workloads
from tests import exact, gates


def _emulate(A, B, bias, epi, bias_shift=0, act=None, skip_bias=False):
    a = exact.widen(A).astype(np.float32)
    b = exact.widen(B).astype(np.float32)
    M, K = a.shape
    s = np.zeros((M, b.shape[0]), dtype=np.float32)
    for k0 in range(0, K, 32):
        s = (s + (a[:, k0:k0 + 32] @ b[:, k0:k0 + 32].T).astype(np.float32)).astype(np.float32)
    if epi == "none":
        y = s
    else:
        bv = exact.widen(np.roll(bias, bias_shift)).astype(np.float32)
        x = s if skip_bias else (s + bv[None, :]).astype(np.float32)
        kind = act or epi
        if kind == "bias":
            y = x
        elif kind == "bias_relu":
            y = np.where(x > 0, x, np.float32(0.0)).astype(np.float32)
        elif kind == "bias_silu":
            y = (x / (np.float32(1.0) + np.exp(-x))).astype(np.float32)
        else:
            y = (np.float32(0.5) * x * special.erfc(-x.astype(np.float64) * np.sqrt(0.5)).astype(np.float32))
            y = y.astype(np.float32)
    return workloads.f32_to_bf16_bits(y)


@pytest.fixture(scope="module")
def case():
    oracle.build()
    A, B = workloads.make_inputs(48, 40, 608, seed=31)
    bias = workloads.f32_to_bf16_bits(np.random.default_rng(9).normal(0.0, 4.0, size=40).astype(np.float32))
    Cr, S, absS = oracle.gemm(A, B)
    return A, B, bias, Cr, S, absS


@pytest.mark.parametrize("epi", ["none", "bias", "bias_relu", "bias_silu", "bias_gelu"])
def test_fp32_emulation_passes(case, epi):
    A, B, bias, Cr, S, absS = case
    C = _emulate(A, B, bias, epi)
    if epi == "none":
        gates.compare(C, Cr, S, absS)
        return
    Ce, Y = oracle.epilogue(S, bias, epi)
    gates.compare_epilogue(C, Ce, Y, absS, np.broadcast_to(exact.widen(bias), S.shape))


@pytest.mark.parametrize("mistake", ["dropped_bias", "shifted_column", "silu_for_gelu", "relu_for_silu",
                                     "bias_not_applied_to_none"])
def test_planted_gpu_mistakes_fail(case, mistake):
    A, B, bias, Cr, S, absS = case
    epi = {"dropped_bias": "bias_gelu", "shifted_column": "bias", "silu_for_gelu": "bias_gelu",
           "relu_for_silu": "bias_silu", "bias_not_applied_to_none": "bias"}[mistake]
    if mistake == "dropped_bias":
        C = _emulate(A, B, bias, epi, skip_bias=True)
    elif mistake == "shifted_column":
        C = _emulate(A, B, bias, epi, bias_shift=1)
    elif mistake == "silu_for_gelu":
        C = _emulate(A, B, bias, epi, act="bias_silu")
    elif mistake == "relu_for_silu":
        C = _emulate(A, B, bias, epi, act="bias_relu")
    else:
        C = _emulate(A, B, bias, "none")
    Ce, Y = oracle.epilogue(S, bias, epi)
    with pytest.raises(AssertionError):
        gates.compare_epilogue(C, Ce, Y, absS, np.broadcast_to(exact.widen(bias), S.shape))


def test_plain_gate_rejects_truncation(case):
    A, B, bias, Cr, S, absS = case
    # rounding toward zero instead of nearest-even: one ulp off on about
    # half of the elements, beyond 2^-8 |C| for many of them
    a = exact.widen(A).astype(np.float64)
    b = exact.widen(B).astype(np.float64)
    s = (a @ b.T).astype(np.float32)
    C = (s.view(np.uint32) >> np.uint32(16)).astype(np.uint16)
    with pytest.raises(AssertionError):
        gates.compare(C, Cr, S, absS)


def test_correct_rounding_of_subnormal_results_passes():
    # Results in bf16's subnormal range round with an absolute error up to
    # half the subnormal spacing, 2^-134, not 2^-8 of the value: a correctly
    # rounded result must pass, one a spacing off must fail.
    oracle.build()
    O = oracle.default()
    S = np.array([5.0509e-40, -5.0509e-40, 1.3e-40, 2.0 ** -133 * 2.5, 3e-39, 1.5e-38])
    C = O.bf16_rne_array(S)
    gates.compare(C, C, S, np.zeros_like(S))
    with pytest.raises(AssertionError):
        gates.compare(C + np.uint16(1), C, S, np.zeros_like(S))


# ------------------------------------------------------------------ MXFP8
# An emulation of the scaled MFMA's measured arithmetic (groups of 8 k
# truncated toward zero to 2^-13 of the group's largest product's power of
# two, then fp32 accumulation) must pass the MXFP8 gate; plausible kernel
# mistakes must fail it.

def _e4m3(codes):
    O = oracle.default()
    table = np.array([O.e4m3_value(c) for c in range(256)])
    return table[np.asarray(codes, dtype=np.uint8)]


def _mx_emulate(av, bv, K, mistake=None):
    M, N = av.shape[0], bv.shape[0]
    acc = np.zeros((M, N), dtype=np.float32)
    for k0 in range(0, K, 128):
        p = av[:, None, k0:k0 + 128] * bv[None, :, k0:k0 + 128]          # exact in float64
        g = p.reshape(M, N, 16, 8)
        mx = np.abs(g).max(axis=-1)
        with np.errstate(divide="ignore"):
            E = np.floor(np.log2(np.where(mx > 0, mx, 1.0)))
        q = np.ldexp(1.0, (E - 13).astype(np.int64))[..., None]
        g = np.trunc(g / q) * q
        if mistake == "dropped_group" and k0 == 0:
            g[:, :, 5, :] = 0.0
        acc = (acc + g.sum(axis=(-1, -2)).astype(np.float32)).astype(np.float32)
    return workloads.f32_to_bf16_bits(acc)


@pytest.fixture(scope="module")
def mx_case():
    oracle.build()
    A, SA, B, SB = workloads.make_mx_inputs(40, 36, 384, a=("normal", 0.0, 1.0), b=("normal", 0.0, 0.02), seed=21)
    C, S, absS = oracle.mx_gemm(A, SA, B, SB)
    a_op = gates.mx_operand(A, SA, _e4m3)
    b_op = gates.mx_operand(B, SB, _e4m3)
    T = gates.mx_truncation_allowance(a_op, b_op)
    return A, SA, B, SB, C, S, absS, a_op[0], b_op[0], T


def test_mx_emulation_passes(mx_case):
    A, SA, B, SB, C, S, absS, av, bv, T = mx_case
    stats = gates.compare_mx(_mx_emulate(av, bv, 384), C, S, absS, T, 384)
    assert stats["elements"] == 40 * 36


def test_mx_truncation_allowance_is_needed():
    # Groups of +1, -1 and six products 1.875 * 2^-13 (codes 0x0F * 0x04):
    # the large pair cancels, the small ones are truncated to 2^-13 each,
    # an error far above 1e-5 absS and 2^-8 |C|.  The gate passes the
    # emulated hardware with T and fails it without.
    oracle.build()
    K = 256
    row = np.tile(np.array([0x38, 0xB8] + [0x0F] * 6, dtype=np.uint8), K // 8)
    col = np.tile(np.array([0x38, 0x38] + [0x04] * 6, dtype=np.uint8), K // 8)
    A = np.tile(row, (4, 1)); B = np.tile(col, (3, 1))
    SA = np.full((4, K // 32), 127, np.uint8); SB = np.full((3, K // 32), 127, np.uint8)
    C, S, absS = oracle.mx_gemm(A, SA, B, SB)
    a_op = gates.mx_operand(A, SA, _e4m3); b_op = gates.mx_operand(B, SB, _e4m3)
    T = gates.mx_truncation_allowance(a_op, b_op)
    av, bv = a_op[0], b_op[0]
    Cg = _mx_emulate(av, bv, K)
    gates.compare_mx(Cg, C, S, absS, T, K)
    with pytest.raises(AssertionError):
        gates.compare(Cg, C, S, absS, acc=gates.mx_acc(K))


@pytest.mark.parametrize("mistake", ["b_scaled_by_a", "scale_block_shift", "dropped_group", "transposed_b_scales"])
def test_mx_planted_mistakes_fail(mx_case, mistake):
    A, SA, B, SB, C, S, absS, av, bv, T = mx_case
    if mistake == "b_scaled_by_a":
        # B's codes with A's scale rows (the wrong operand's scale pointer)
        b2 = gates.mx_operand(B, SA[:36], _e4m3)[0]
        Cg = _mx_emulate(av, b2, 384)
    elif mistake == "scale_block_shift":
        a2 = gates.mx_operand(A, np.roll(SA, 1, axis=1), _e4m3)[0]
        Cg = _mx_emulate(a2, bv, 384)
    elif mistake == "transposed_b_scales":
        b2 = gates.mx_operand(B, SB[::-1], _e4m3)[0]
        Cg = _mx_emulate(av, b2, 384)
    else:
        Cg = _mx_emulate(av, bv, 384, mistake="dropped_group")
    with pytest.raises(AssertionError):
        gates.compare_mx(Cg, C, S, absS, T, 384)


def test_mx_allowance_matches_definition_on_a_tiny_case():
    # One group: 1.0 * 1.0, 2^-7 * 2^-7 (subnormal codes 0x04) and six zero
    # products.  Es = 0 (exponent fields 7 + 7 - 14), En = 0, q = 2^-13; the
    # products 1 and 0 are multiples of q, 2^-14 is not: T = 2^-14.
    codes_a = np.array([[0x38, 0x04, 0, 0, 0, 0, 0, 0]], dtype=np.uint8)
    codes_b = codes_a.copy()
    s = np.full((1, 1), 127, np.uint8)
    pad = lambda c: np.concatenate([c, np.zeros((1, 24), np.uint8)], axis=1)
    a_op = gates.mx_operand(pad(codes_a), s, _e4m3)
    b_op = gates.mx_operand(pad(codes_b), s, _e4m3)
    T = gates.mx_truncation_allowance(a_op, b_op)
    assert T[0, 0] == 2.0 ** -14
    assert gates.mx_truncation_allowance(a_op, b_op, ii=np.array([0]), jj=np.array([0]))[0] == T[0, 0]
    # A subnormal-led group: largest operands 2^-7 (exponent field 0, so
    # Es = -12) against En = -14: q = 2^-25 and 2^-14 is a multiple: T = 0.
    a_op = gates.mx_operand(pad(np.array([[0x04, 0, 0, 0, 0, 0, 0, 0]], np.uint8)), s, _e4m3)
    assert gates.mx_truncation_allowance(a_op, a_op)[0, 0] == 0.0
