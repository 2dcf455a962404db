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
