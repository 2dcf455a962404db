"""GPU parity of the MXFP8 (block-scaled FP8) GEMM against the oracle.

Every MXFP8 kernel variant (the 256 x 256 ping-pong, the 128 x 128 ring,
the small-M kernels, with and without split-K) runs through the C ABI on seeded inputs; each
output is compared with the oracle's exact sum under the MXFP8 gate of
tests/gates.py (compare_mx: the bf16 rounding, the scaled MFMA's measured
group truncation and fp32 accumulation).  Inputs whose every product and
sum the hardware forms exactly must match the oracle bit for bit.
"""
import numpy as np
import pytest

import oracle
import workloads
from tests import exact, gates

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


def _say(*a):
    print("[gpu-mx]", *a, flush=True)


@pytest.fixture(scope="module")
def hkg():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import tile_level_dense_amd as lib
    lib.lib()
    return lib


_E4M3 = None


def e4m3(codes):
    global _E4M3
    if _E4M3 is None:
        O = oracle.default()
        _E4M3 = np.array([O.e4m3_value(c) for c in range(256)])
    return _E4M3[np.asarray(codes, dtype=np.uint8)]


def dev8(x):
    return torch.from_numpy(np.ascontiguousarray(x, dtype=np.uint8)).to("cuda")


def dev16(bits):
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).to("cuda")


def host(t):
    return t.view(torch.int16).cpu().numpy().view(np.uint16)


def check(C, A, SA, B, SB, bias=None, epi="none"):
    K = A.shape[1]
    Cr, S, absS = oracle.mx_gemm(A, SA, B, SB)
    T = gates.mx_truncation_allowance(gates.mx_operand(A, SA, e4m3), gates.mx_operand(B, SB, e4m3))
    if epi == "none":
        return gates.compare_mx(C, Cr, S, absS, T, K)
    Ce, Y = oracle.epilogue(S, bias, epi)
    return gates.compare_mx_epilogue(C, Ce, Y, absS, np.broadcast_to(exact.widen(bias), S.shape), T, K)


def forced(hkg, variant, split=1):
    """Plan edit forcing one kernel variant: an int picks an MXFP8 tile
    variant, "s<i>" the small-M (skinny) variant i."""
    from tile_level_dense_amd import build as hkg_build
    if isinstance(variant, str):
        mb, nb, wk, u, cp, al = hkg_build.skinny_configs(mx=True)[int(variant[1:])]

        def edit(p):
            assert p.M <= 16 * mb
            p.kernel_id = hkg.HKG_KERNEL_MX_SKINNY
            p.variant = int(variant[1:])
            p.tile_m, p.tile_n, p.tile_k, p.waves = 16 * mb, 16 * nb, 128, wk
            p.split_k = split
            p.grid_x = -(-p.N // (16 * nb))
            p.grid_y = split
            p.workspace_bytes = split * p.M * p.N * 4 if split > 1 else 0
        return edit
    bm, bn, bk, stages, wm, wn, _ = hkg_build.tile_configs(mx=True)[variant]

    def edit(p):
        p.kernel_id = hkg.HKG_KERNEL_MX_TILE
        p.variant = variant
        p.tile_m, p.tile_n, p.tile_k, p.waves = bm, bn, bk, wm * wn
        p.split_k = split
        p.grid_y = split
        p.workspace_bytes = split * p.M * p.N * 4 if split > 1 else 0
    return edit


def run(hkg, A, SA, B, SB, edit=None, bias=None, epi="none"):
    M, K = A.shape
    N = B.shape[0]
    a, b = dev8(A), dev8(B)
    bias_t = dev16(bias) if bias is not None else None
    if edit is None:
        c = hkg.gemm_mxfp8(a, dev8(SA), b, dev8(SB), bias=bias_t, epilogue=epi)
    else:
        p = hkg.mx_plan(M, N, K)
        edit(p)
        c = hkg.run_mx_plan(p, a, hkg.mx_pack_scales(dev8(SA), K), b, hkg.mx_pack_scales(dev8(SB), K),
                            bias=bias_t, epilogue=epi)
    torch.cuda.synchronize()
    return host(c)


def make_bias(N, seed, scale=4.0):
    rng = np.random.default_rng(2000 + seed)
    return workloads.f32_to_bf16_bits(rng.normal(0.0, scale, size=N).astype(np.float32))


# (name, shape, variant or None for the planner, split)
CASES = [
    ("planner_tiny", (256, 256, 256), None, 1),
    ("planner_ragged", (300, 500, 384), None, 1),
    ("pingpong_ragged", (300, 500, 384), 0, 1),
    ("pingpong_one_stage", (256, 256, 128), 0, 1),
    ("pingpong_long_k", (513, 260, 1024), 0, 1),
    ("ring_ragged", (129, 260, 256), 1, 1),
    ("ring_small", (17, 33, 128), 1, 1),
    ("ring_split3", (200, 333, 1536), 1, 3),
    ("ring_split2_decode", (32, 512, 1024), 1, 2),
    ("single_element", (1, 1, 128), 1, 1),
    # small-M kernel: 16-row and 32-row covers, ragged N, split-K with
    # splits that get unequal (or no) steps of 128 k
    ("skinny16_single", (1, 1, 128), "s0", 1),
    ("skinny16_ragged", (13, 300, 1024), "s0", 1),
    ("skinny16_split4", (7, 2000, 4096), "s0", 4),
    ("skinny16_split3_short", (16, 48, 384), "s0", 3),
    ("skinny16_split5_uneven", (16, 100, 896), "s0", 5),
    ("skinny32_ragged", (17, 260, 256), "s1", 1),
    ("skinny32_split2", (32, 512, 1024), "s1", 2),
    ("skinny32_one_row", (1, 70, 512), "s1", 3),
    # the same covers with A staged through LDS
    ("skinny16_lds_ragged", (13, 300, 1024), "s2", 1),
    ("skinny16_lds_split3_short", (16, 48, 384), "s2", 3),
    ("skinny16_lds_single", (1, 1, 128), "s2", 1),
    ("skinny32_lds_ragged", (17, 260, 256), "s3", 1),
    ("skinny32_lds_split5_uneven", (32, 100, 1792), "s3", 5),
    ("skinny32_lds_long_k", (29, 64, 8192), "s3", 1),
    ("planner_decode_32", (32, 1024, 4096), None, 1),
    ("planner_decode_small", (16, 2048, 4096), None, 1),
]


@pytest.mark.parametrize("name,shape,variant,split", CASES, ids=[c[0] for c in CASES])
def test_mx_parity(hkg, name, shape, variant, split):
    M, N, K = shape
    _say(name, shape, variant, split)
    A, SA, B, SB = workloads.make_mx_inputs(M, N, K, b=("normal", 0.0, 0.02), seed=len(name) + K)
    C = run(hkg, A, SA, B, SB, None if variant is None else forced(hkg, variant, split))
    check(C, A, SA, B, SB)


def _exact_inputs(M, N, K, seed):
    # E4M3 magnitudes in [1, 3.75] (exponent fields 7 and 8), both signs,
    # block scales 2^-1 .. 2^1: products are multiples of 2^-8 below 2^6,
    # so no group truncates anything (its quantum is at most 2^-10 of the
    # scale), and every partial sum, bounded by absS < 2^16, is a multiple
    # of 2^-8 that fp32's 24 bits hold exactly.
    rng = np.random.default_rng(seed)
    def codes(shape):
        e = rng.integers(7, 9, size=shape); f = rng.integers(0, 8, size=shape); s = rng.integers(0, 2, size=shape)
        return ((s << 7) | (e << 3) | f).astype(np.uint8)
    A, B = codes((M, K)), codes((N, K))
    SA = rng.integers(126, 129, size=(M, K // 32)).astype(np.uint8)
    SB = rng.integers(126, 129, size=(N, K // 32)).astype(np.uint8)
    return A, SA, B, SB


@pytest.mark.parametrize("variant,split,shape", [(0, 1, (256, 512, 512)), (1, 1, (200, 136, 512)),
                                                 (1, 4, (64, 256, 1024)), ("s0", 1, (16, 256, 512)),
                                                 ("s1", 4, (32, 272, 1024)), ("s2", 2, (16, 256, 512)),
                                                 ("s3", 1, (32, 272, 1024))])
def test_mx_exact_inputs_bit_exact(hkg, variant, split, shape):
    M, N, K = shape
    _say("exact", variant, split, shape)
    A, SA, B, SB = _exact_inputs(M, N, K, seed=M + K)
    C = run(hkg, A, SA, B, SB, forced(hkg, variant, split))
    Cr, S, absS = oracle.mx_gemm(A, SA, B, SB)
    assert absS.max() < 2.0 ** 16
    assert np.array_equal(C, Cr)


@pytest.mark.parametrize("epi", ["bias", "bias_relu", "bias_silu", "bias_gelu"])
@pytest.mark.parametrize("variant,split,shape", [(0, 1, (300, 260, 256)), (1, 2, (100, 200, 1024)),
                                                 ("s0", 1, (9, 130, 256)), ("s1", 2, (20, 200, 1024))])
def test_mx_epilogue_parity(hkg, epi, variant, split, shape):
    M, N, K = shape
    _say("epilogue", epi, variant, split, shape)
    A, SA, B, SB = workloads.make_mx_inputs(M, N, K, seed=K + len(epi))
    bias = make_bias(N, seed=M)
    C = run(hkg, A, SA, B, SB, forced(hkg, variant, split), bias=bias, epi=epi)
    check(C, A, SA, B, SB, bias=bias, epi=epi)


def test_mx_k_zero_is_epilogue_of_bias(hkg):
    _say("K = 0")
    M, N = 19, 40
    bias = make_bias(N, seed=5)
    a = torch.empty((M, 0), dtype=torch.uint8, device="cuda")
    b = torch.empty((N, 0), dtype=torch.uint8, device="cuda")
    sa = torch.empty((M, 0), dtype=torch.uint8, device="cuda")
    sb = torch.empty((N, 0), dtype=torch.uint8, device="cuda")
    out = hkg.gemm_mxfp8(a, sa, b, sb, bias=dev16(bias), epilogue="bias_silu")
    torch.cuda.synchronize()
    Ce, Y = oracle.epilogue(np.zeros((M, N)), bias, "bias_silu")
    gates.compare_epilogue(host(out), Ce, Y, np.zeros((M, N)), np.broadcast_to(exact.widen(bias), (M, N)))


def test_mx_pack_layout(hkg):
    # The documented packed layout, written out with numpy.
    rows, K = 130, 512
    rng = np.random.default_rng(3)
    S = rng.integers(0, 255, size=(rows, K // 32)).astype(np.uint8)
    P = hkg.mx_pack_scales(dev8(S), K).cpu().numpy()
    KT, groups = K // 128, (rows + 63) // 64
    assert P.size == groups * KT * 256
    want = np.zeros((groups, KT, 64, 4), dtype=np.uint8)
    for R in range(groups):
        for t in range(KT):
            for l in range(64):
                for f in range(4):
                    r = 64 * R + 16 * f + l % 16
                    if r < rows:
                        want[R, t, l, f] = S[r, 4 * t + l // 16]
    assert np.array_equal(P, want.reshape(-1))


def test_mx_prepacked_equals_natural_and_is_deterministic(hkg):
    M, N, K = 300, 270, 640
    A, SA, B, SB = workloads.make_mx_inputs(M, N, K, seed=77)
    a, b, sa, sb = dev8(A), dev8(B), dev8(SA), dev8(SB)
    c1 = hkg.gemm_mxfp8(a, sa, b, sb)
    c2 = hkg.gemm_mxfp8(a, hkg.mx_pack_scales(sa, K), b, hkg.mx_pack_scales(sb, K), packed=True)
    c3 = hkg.gemm_mxfp8(a, sa, b, sb)
    torch.cuda.synchronize()
    assert torch.equal(c1.view(torch.int16), c2.view(torch.int16))
    assert torch.equal(c1.view(torch.int16), c3.view(torch.int16))


@pytest.mark.parametrize("shape", [(13, 300, 1024), (32, 260, 256), (1, 70, 512), (7, 2000, 4096), (16, 48, 384)])
def test_mx_small_m_natural_scales(hkg, shape):
    # The small-M kernel reads natural-layout scales itself: the result must
    # match the packed path bit for bit and the oracle under the gate; scale
    # arrays at an odd address take the packing path and agree as well.
    M, N, K = shape
    _say("natural scales", shape)
    p = hkg.mx_plan(M, N, K)
    assert p.kernel_id == hkg.HKG_KERNEL_MX_SKINNY
    A, SA, B, SB = workloads.make_mx_inputs(M, N, K, b=("normal", 0.0, 0.02), seed=M + N)
    a, b, sa, sb = dev8(A), dev8(B), dev8(SA), dev8(SB)
    c_nat = hkg.gemm_mxfp8(a, sa, b, sb)
    c_pk = hkg.gemm_mxfp8(a, hkg.mx_pack_scales(sa, K), b, hkg.mx_pack_scales(sb, K), packed=True)
    odd_a = torch.empty(SA.size + 1, dtype=torch.uint8, device="cuda")[1:].view(SA.shape)
    odd_b = torch.empty(SB.size + 1, dtype=torch.uint8, device="cuda")[1:].view(SB.shape)
    odd_a.copy_(sa)
    odd_b.copy_(sb)
    c_odd = hkg.gemm_mxfp8(a, odd_a, b, odd_b)
    torch.cuda.synchronize()
    assert torch.equal(c_nat.view(torch.int16), c_pk.view(torch.int16))
    assert torch.equal(c_nat.view(torch.int16), c_odd.view(torch.int16))
    check(host(c_nat), A, SA, B, SB)


def test_mx_workload_decode_whole_output(hkg):
    # mx_decode_32x4096x4096: a decode projection, every output checked.
    _say("workload mx_decode_32x4096x4096")
    A, SA, B, SB = workloads.mx_workload_inputs("mx_decode_32x4096x4096")
    assert hkg.mx_plan(*A.shape, B.shape[0]).kernel_id == hkg.HKG_KERNEL_MX_SKINNY
    C = run(hkg, A, SA, B, SB)
    check(C, A, SA, B, SB)


def _tile_edges(n, tile):
    """First and last index of every tile along one dimension, and the 17th."""
    idx = {0, n - 1}
    for t in range(0, n, tile):
        idx.update({t, min(n - 1, t + tile - 1), min(n - 1, t + 17)})
    return np.array(sorted(idx), dtype=np.int64)


def test_mx_workload_square_sampled(hkg):
    # mx_square_8192 in the planner's launch configuration, checked against
    # the oracle entry by entry: every tile's edge rows crossed with every
    # tile's edge columns, the two whole rows and the two whole columns on
    # each side of the first tile boundary, and 4096 random outputs.
    _say("workload mx_square_8192")
    A, SA, B, SB = workloads.mx_workload_inputs("mx_square_8192")
    M, K = A.shape
    N = B.shape[0]
    p = hkg.mx_plan(M, N, K)
    assert p.kernel_id == hkg.HKG_KERNEL_MX_TILE and p.variant == 0
    tm, tn = p.tile_m, p.tile_n
    C = run(hkg, A, SA, B, SB)
    rng = np.random.default_rng(8)
    er, ec = _tile_edges(M, tm), _tile_edges(N, tn)
    gi, gj = np.meshgrid(er, ec, indexing="ij")
    full = np.arange(N, dtype=np.int64)
    fullm = np.arange(M, dtype=np.int64)
    ii = np.concatenate([gi.ravel(), np.full(N, tm - 1), np.full(N, tm), fullm, fullm,
                         rng.integers(0, M, 4096)])
    jj = np.concatenate([gj.ravel(), full, full, np.full(M, tn - 1), np.full(M, tn),
                         rng.integers(0, N, 4096)])
    _say("mx_square_8192: %d entries (%d edge rows x %d edge columns)" % (ii.size, er.size, ec.size))
    Cr, S, absS = oracle.mx_gemm_entries(A, SA, B, SB, ii, jj)
    T = gates.mx_truncation_allowance(gates.mx_operand(A, SA, e4m3), gates.mx_operand(B, SB, e4m3), ii=ii, jj=jj)
    stats = gates.compare_mx(C[ii, jj], Cr, S, absS, T, K)
    _say("mx_square_8192", stats)
    assert np.isfinite(exact.widen(C)).all()
