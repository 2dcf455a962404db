"""GPU parity of the fused epilogues (bias, bias+ReLU, bias+SiLU, bias+GELU).

Each kernel of the library (tile schedules, tile split-K, skinny, skinny
split-K, general, K = 0) runs through the C ABI with every epilogue, and the
result is compared element by element with the oracle's act(S + bias) on the
same seeded inputs (tests/gates.py, compare_epilogue, states the tolerance).
Inputs whose fp32 sums and epilogue are exact must match bit for bit.
"""
import numpy as np
import pytest

import oracle
import workloads
from tests import exact, gates

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")

EPIS = ["bias", "bias_relu", "bias_silu", "bias_gelu"]


def _say(*a):
    print("[gpu-epilogue]", *a, flush=True)


@pytest.fixture(scope="module")
def hkg():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import tile_level_dense_amd as lib
    lib.lib()
    return lib


def dev(bits):
    t = torch.from_numpy(np.ascontiguousarray(bits).view(np.int16))
    return t.view(torch.bfloat16).to("cuda")


def host(t):
    return t.view(torch.int16).cpu().numpy().view(np.uint16)


def make_bias(N, seed, scale=4.0):
    rng = np.random.default_rng(1000 + seed)
    return workloads.f32_to_bf16_bits(rng.normal(0.0, scale, size=N).astype(np.float32))


def check(C, A, B, bias, epi):
    Cr, S, absS = oracle.gemm(A, B)
    Ce, Y = oracle.epilogue(S, bias, epi)
    bvals = np.broadcast_to(exact.widen(bias), S.shape)
    return gates.compare_epilogue(C, Ce, Y, absS, bvals)


def run_forced(hkg, A, B, bias, epi, edit=None):
    M, K = A.shape
    N = B.shape[0]
    p = hkg.plan(M, N, K)
    if edit is not None:
        edit(p)
    c = hkg.run_plan(p, dev(A), dev(B), bias=dev(bias), epilogue=epi)
    torch.cuda.synchronize()
    return host(c), p


def _tile(hkg, variant, split=1):
    from tile_level_dense_amd import build as hkg_build
    bm, bn, bk, stages, wm, wn, sc = hkg_build.tile_configs()[variant]

    def edit(p):
        p.kernel_id = hkg.HKG_KERNEL_TILE
        p.variant = variant
        p.tile_m, p.tile_n, p.tile_k, p.waves = bm, bn, bk, wm * wn * (2 if sc == 7 else 1)
        p.split_k = split
        p.grid_y = split
        p.workspace_bytes = split * p.M * p.N * 4 if split > 1 else 0
    return edit


def _skinny(hkg, variant, split):
    from tile_level_dense_amd import build as hkg_build
    mb, nb, wk, u, cp, al = hkg_build.skinny_configs()[variant]

    def edit(p):
        p.kernel_id = hkg.HKG_KERNEL_SKINNY
        p.variant = variant
        p.tile_m, p.tile_n, p.waves = 16 * mb, 16 * nb, wk
        p.split_k = split
        p.grid_y = split
        p.workspace_bytes = split * p.M * p.N * 4 if split > 1 else 0
    return edit


def _generic(hkg):
    def edit(p):
        p.kernel_id = hkg.HKG_KERNEL_GENERIC
    return edit


# (name, shape, plan edit factory or None for the planner's choice)
CASES = [
    ("planner_tile", (520, 1000, 392), None),
    ("pingpong_256", (300, 500, 136), lambda h: _tile(h, 0)),
    ("pingpong_256_w2x4", (260, 270, 200), lambda h: _tile(h, 5)),
    ("pipelined_256", (300, 500, 136), lambda h: _tile(h, 4)),
    ("tile_256x128", (129, 300, 264), lambda h: _tile(h, 1)),
    ("tile_128_split3", (200, 333, 1032), lambda h: _tile(h, 2, 3)),
    ("kinter_128x256", (300, 530, 392), lambda h: _tile(h, 14)),
    ("kinter_128x128", (129, 270, 136), lambda h: _tile(h, 15)),
    ("kinter_128x128_s5", (200, 300, 456), lambda h: _tile(h, 16)),
    ("split_tail", (4400, 4200, 136), None),
    ("tile256_one_round", (700, 900, 200), lambda h: _tile(h, 11)),
    ("tile256_many_rounds", (4400, 4200, 72), lambda h: _tile(h, 11)),
    ("planner_skinny", (16, 1000, 2056), None),
    ("skinny_split3", (20, 300, 4096), lambda h: _skinny(h, 1, 3)),
    ("skinny_nb4", (9, 100, 520), lambda h: _skinny(h, 5, 1)),
    ("skinny_lds_split3", (12, 300, 4104), lambda h: _skinny(h, 10, 3)),
    ("generic", (70, 45, 100), lambda h: _generic(h)),
]


@pytest.mark.parametrize("epi", EPIS)
@pytest.mark.parametrize("name,shape,make_edit", CASES, ids=[c[0] for c in CASES])
def test_epilogue_parity(hkg, epi, name, shape, make_edit):
    M, N, K = shape
    _say(name, epi, shape)
    A, B = workloads.make_inputs(M, N, K, seed=len(name) + K)
    bias = make_bias(N, seed=M)
    C, p = run_forced(hkg, A, B, bias, epi, make_edit(hkg) if make_edit else None)
    check(C, A, B, bias, epi)


@pytest.mark.parametrize("epi", ["bias", "bias_relu"])
@pytest.mark.parametrize("shape", [(256, 256, 256), (16, 4096, 256), (300, 130, 256)])
def test_exact_bias_epilogue_bit_exact(hkg, epi, shape):
    # All-ones operands: every fp32 sum is K = 256 exactly; 256 + b is exact
    # in fp32 for these biases, and so is max(., 0): the result must equal
    # the oracle's bit for bit.
    M, N, K = shape
    _say("exact", epi, shape)
    A = np.full((M, K), 0x3F80, dtype=np.uint16)
    B = np.full((N, K), 0x3F80, dtype=np.uint16)
    vals = np.array([-300.0, -256.0, -0.5, 0.0, 1.0, 3.5, -1000.0, 17.25], dtype=np.float32)
    bias = workloads.f32_to_bf16_bits(np.resize(vals, N))
    C = host(hkg.gemm(dev(A), dev(B), bias=dev(bias), epilogue=epi))
    _, S, _ = oracle.gemm(A[:1], B)
    Ce, _ = oracle.epilogue(S, bias, epi)
    assert np.array_equal(C, np.broadcast_to(Ce, C.shape))


@pytest.mark.parametrize("epi", EPIS)
def test_k_zero_is_epilogue_of_bias(hkg, epi):
    _say("K = 0", epi)
    M, N = 37, 29
    bias = make_bias(N, seed=3)
    a = torch.empty((M, 0), dtype=torch.bfloat16, device="cuda")
    b = torch.empty((N, 0), dtype=torch.bfloat16, device="cuda")
    out = torch.full((M, N), 3.0, dtype=torch.bfloat16, device="cuda")
    hkg.gemm(a, b, out=out, bias=dev(bias), epilogue=epi)
    torch.cuda.synchronize()
    Ce, Y = oracle.epilogue(np.zeros((M, N)), bias, epi)
    gates.compare_epilogue(host(out), Ce, Y, np.zeros((M, N)), np.broadcast_to(exact.widen(bias), (M, N)))


@pytest.mark.parametrize("epi", EPIS)
def test_misaligned_operands_take_generic(hkg, epi):
    M, N, K = 33, 48, 200
    _say("misaligned", epi)
    A, B = workloads.make_inputs(M, N, K, seed=8)
    bias = make_bias(N, seed=4)
    a_buf = torch.zeros(M * K + 1, dtype=torch.bfloat16, device="cuda")
    b_buf = torch.zeros(N * K + 1, dtype=torch.bfloat16, device="cuda")
    c_buf = torch.zeros(M * N + 1, dtype=torch.bfloat16, device="cuda")
    bias_buf = torch.zeros(N + 1, dtype=torch.bfloat16, device="cuda")
    a_buf[1:] = dev(A).reshape(-1)
    b_buf[1:] = dev(B).reshape(-1)
    bias_buf[1:] = dev(bias)
    st = hkg.hkg_gemm_bf16_epilogue(a_buf.data_ptr() + 2, b_buf.data_ptr() + 2, bias_buf.data_ptr() + 2,
                                    c_buf.data_ptr() + 2, M, N, K, hkg.EPILOGUES[epi],
                                    torch.cuda.current_stream().cuda_stream)
    assert st == hkg.HKG_OK
    torch.cuda.synchronize()
    check(host(c_buf[1:]).reshape(M, N), A, B, bias, epi)


def test_none_epilogue_is_plain_gemm(hkg):
    M, N, K = 300, 200, 264
    A, B = workloads.make_inputs(M, N, K, seed=12)
    a, b = dev(A), dev(B)
    c1 = host(hkg.gemm(a, b))
    c2 = host(hkg.gemm(a, b, bias=None, epilogue="none"))
    assert np.array_equal(c1, c2)


def test_workload_epilogues(hkg):
    # The MLP-up workload (a feed-forward projection) with bias + GELU and the
    # decode workload with bias + SiLU, whole outputs.
    for name, epi in (("mlp_up_128x12288x4096", "bias_gelu"), ("decode_16x4096x4096", "bias_silu")):
        _say("workload", name, epi)
        A, B = workloads.workload_inputs(name)
        N = B.shape[0]
        bias = make_bias(N, seed=7, scale=0.1)
        C = host(hkg.gemm(dev(A), dev(B), bias=dev(bias), epilogue=epi))
        check(C, A, B, bias, epi)


@pytest.mark.parametrize("epi", EPIS)
def test_activation_over_its_range(hkg, epi):
    # K = 0 makes every output epilogue(bias): a sweep of the activation
    # itself over [-40, 40], tiny and subnormal values, signed zeros and
    # values where exp under- or overflows, against the oracle's fp64.
    _say("activation sweep", epi)
    xs = np.concatenate([np.linspace(-40.0, 40.0, 3001),
                         [0.0, -0.0, 1e-30, -1e-30, 1e-39, -1e-39, 88.0, -88.0, 90.0, -90.0, 100.0, -100.0,
                          1e4, -1e4, 3e38, -3e38]]).astype(np.float32)
    bias = workloads.f32_to_bf16_bits(xs)
    N = bias.size
    M = 3
    a = torch.empty((M, 0), dtype=torch.bfloat16, device="cuda")
    b = torch.empty((N, 0), dtype=torch.bfloat16, device="cuda")
    out = hkg.gemm(a, b, bias=dev(bias), epilogue=epi)
    torch.cuda.synchronize()
    Ce, Y = oracle.epilogue(np.zeros((M, N)), bias, epi)
    gates.compare_epilogue(host(out), Ce, Y, np.zeros((M, N)), np.broadcast_to(exact.widen(bias), (M, N)))
