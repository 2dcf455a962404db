"""GPU parity of the MXFP4 (block-scaled FP4) GEMM against the oracle.

Both MXFP4 tile variants (the 256 x 256 ping-pong and the 128 x 128 ring,
with and without split-K) run through the C ABI on seeded inputs; each
output is compared with the oracle's exact sum under the MXFP4 gate of
tests/gates.py (compare_mx4: the bf16 rounding and fp32 accumulation; the
products of a scale block are summed exactly).  Inputs whose every partial
sum fp32 holds exactly must match the oracle bit for bit.  K multiples of
128 that are not multiples of 256 leave the last 256-k stage half empty;
those cases are included.
"""
import numpy as np
import pytest

import oracle
import workloads
from tests import exact, gates

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


def _say(*a):
    print("[gpu-mx4]", *a, flush=True)


@pytest.fixture(scope="module")
def hkg():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import tile_level_dense_amd as lib
    lib.lib()
    return lib


def dev8(x):
    return torch.from_numpy(np.ascontiguousarray(x, dtype=np.uint8)).to("cuda")


def dev16(bits):
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).to("cuda")


def host(t):
    return t.view(torch.int16).cpu().numpy().view(np.uint16)


def check(C, A, SA, B, SB, bias=None, epi="none"):
    K = 2 * A.shape[1]
    Cr, S, absS = oracle.mx4_gemm(A, SA, B, SB)
    if epi == "none":
        return gates.compare_mx4(C, Cr, S, absS, K)
    Ce, Y = oracle.epilogue(S, bias, epi)
    return gates.compare_mx4_epilogue(C, Ce, Y, absS, np.broadcast_to(exact.widen(bias), S.shape), K)


def forced(hkg, variant, split=1):
    """Plan edit forcing MXFP4 tile variant `variant` with `split` K splits."""
    from tile_level_dense_amd import build as hkg_build
    bm, bn, bk, stages, wm, wn, _ = hkg_build.tile_configs(mx4=True)[variant]

    def edit(p):
        p.kernel_id = hkg.HKG_KERNEL_MX4_TILE
        p.variant = variant
        p.tile_m, p.tile_n, p.tile_k, p.waves = bm, bn, bk, wm * wn
        p.split_k = split
        p.grid_y = split
        p.workspace_bytes = split * p.M * p.N * 4 if split > 1 else 0
    return edit


def run(hkg, A, SA, B, SB, edit=None, bias=None, epi="none", packed=False):
    M = A.shape[0]
    K = 2 * A.shape[1]
    N = B.shape[0]
    a, b = dev8(A), dev8(B)
    bias_t = dev16(bias) if bias is not None else None
    if edit is None and not packed:
        c = hkg.gemm_mxfp4(a, dev8(SA), b, dev8(SB), bias=bias_t, epilogue=epi)
    elif edit is None:
        c = hkg.gemm_mxfp4(a, hkg.mx_pack_scales(dev8(SA), K), b, hkg.mx_pack_scales(dev8(SB), K), bias=bias_t,
                           epilogue=epi, packed=True)
    else:
        p = hkg.mx4_plan(M, N, K)
        edit(p)
        c = hkg.run_mx4_plan(p, a, hkg.mx_pack_scales(dev8(SA), K), b, hkg.mx_pack_scales(dev8(SB), K),
                             bias=bias_t, epilogue=epi)
    torch.cuda.synchronize()
    return host(c)


def make_bias(N, seed, scale=4.0):
    rng = np.random.default_rng(3000 + seed)
    return workloads.f32_to_bf16_bits(rng.normal(0.0, scale, size=N).astype(np.float32))


# (name, shape, variant or None for the planner, split)
CASES = [
    ("planner_tiny", (256, 256, 256), None, 1),
    ("planner_ragged", (300, 500, 384), None, 1),
    ("pingpong_ragged_half_stage", (300, 500, 384), 0, 1),
    ("pingpong_one_step", (256, 256, 128), 0, 1),
    ("pingpong_long_k", (513, 260, 1024), 0, 1),
    ("pingpong_two_tiles_each_way", (512, 512, 768), 0, 1),
    ("ring_ragged", (129, 260, 256), 1, 1),
    ("ring_small_one_step", (17, 33, 128), 1, 1),
    ("ring_split3", (200, 333, 1536), 1, 3),
    ("ring_split2_decode", (32, 512, 1024), 1, 2),
    ("ring_split4_half_stage", (40, 300, 1152), 1, 4),
    ("ring_split5_empty_split", (16, 128, 768), 1, 5),
    ("single_element", (1, 1, 128), 1, 1),
    ("planner_decode_32", (32, 1024, 4096), None, 1),
    ("planner_pingpong", (4096, 4096, 512), None, 1),
]


@pytest.mark.parametrize("name,shape,variant,split", CASES, ids=[c[0] for c in CASES])
def test_mx4_parity(hkg, name, shape, variant, split):
    M, N, K = shape
    _say(name, shape, variant, split)
    A, SA, B, SB = workloads.make_mx4_inputs(M, N, K, sb=(118, 122), seed=len(name) + K)
    C = run(hkg, A, SA, B, SB, None if variant is None else forced(hkg, variant, split))
    stats = check(C, A, SA, B, SB)
    _say(name, stats)


def test_mx4_planner_choices(hkg):
    p = hkg.mx4_plan(8192, 8192, 8192)
    assert p.kernel_id == hkg.HKG_KERNEL_MX4_TILE and p.variant == 0 and p.split_k == 1
    p = hkg.mx4_plan(64, 14336, 4096)
    assert p.kernel_id == hkg.HKG_KERNEL_MX4_TILE and p.variant == 1 and p.split_k == 3
    p = hkg.mx4_plan(32, 14336, 4096)
    assert p.kernel_id == hkg.HKG_KERNEL_MX4_SKINNY and p.tile_m == 32 and p.tile_n == 64 and p.split_k == 1
    p = hkg.mx4_plan(32, 8192, 8192)
    assert p.kernel_id == hkg.HKG_KERNEL_MX4_SKINNY and p.tile_n == 32 and p.split_k == 1
    p = hkg.mx4_plan(16, 14336, 4096)
    assert p.kernel_id == hkg.HKG_KERNEL_MX4_SKINNY and p.tile_m == 32 and p.tile_n == 64
    p = hkg.mx4_plan(32, 1024, 4096)
    assert p.kernel_id == hkg.HKG_KERNEL_MX4_SKINNY and p.tile_n == 16 and p.split_k == 2
    p = hkg.mx4_plan(9, 4096, 4096)
    assert p.kernel_id == hkg.HKG_KERNEL_MX4_SKINNY and p.tile_m == 16


def forced_skinny(hkg, variant, split=1):
    """Plan edit forcing MXFP4 small-M variant `variant` with `split` K splits."""
    from tile_level_dense_amd import build as hkg_build
    mb, nb, wk, u, cp, al = hkg_build.skinny_configs(mx4=True)[variant]

    def edit(p):
        p.kernel_id = hkg.HKG_KERNEL_MX4_SKINNY
        p.variant = variant
        p.tile_m, p.tile_n, p.tile_k, p.waves = 16 * mb, 16 * nb, 256, wk
        p.split_k = split
        p.grid_x = -(-p.N // (16 * nb))
        p.grid_y = split
        p.workspace_bytes = split * p.M * p.N * 4 if split > 1 else 0
    return edit


# (name, shape, small-M variant, split): ragged N and M, K with a half-empty
# last 256-k step, splits that leave some workgroups no steps.
SKINNY_CASES = [
    ("m16_ragged", (13, 300, 1152), 0, 1),
    ("m16_one_row_half_step", (1, 50, 128), 0, 1),
    ("m32_n16", (32, 260, 1024), 1, 1),
    ("m32_n16_split3_half_step", (17, 200, 1408), 1, 3),
    ("m32_n32", (30, 333, 2048), 2, 1),
    ("m32_n32_split5_empty", (32, 96, 768), 2, 5),
    ("m32_n64", (25, 520, 1536), 3, 1),
    ("m32_n64_split2_half_step", (32, 700, 640), 3, 2),
]


@pytest.mark.parametrize("name,shape,variant,split", SKINNY_CASES, ids=[c[0] for c in SKINNY_CASES])
def test_mx4_skinny_parity(hkg, name, shape, variant, split):
    M, N, K = shape
    _say("skinny", name, shape, variant, split)
    A, SA, B, SB = workloads.make_mx4_inputs(M, N, K, sb=(118, 122), seed=len(name) + K)
    C = run(hkg, A, SA, B, SB, forced_skinny(hkg, variant, split))
    stats = check(C, A, SA, B, SB)
    _say(name, stats)


@pytest.mark.parametrize("variant,split,shape", [(0, 1, (16, 200, 896)), (1, 1, (32, 136, 512)),
                                                 (2, 3, (20, 100, 1024)), (3, 1, (32, 300, 384))])
def test_mx4_skinny_exact_inputs_bit_exact(hkg, variant, split, shape):
    M, N, K = shape
    _say("skinny exact", variant, split, shape)
    A, SA, B, SB = _exact_inputs(M, N, K, seed=M + K)
    C = run(hkg, A, SA, B, SB, forced_skinny(hkg, variant, split))
    Cr, S, absS = oracle.mx4_gemm(A, SA, B, SB)
    assert absS.max() < 2.0 ** 18
    assert np.array_equal(C, Cr)


def test_mx4_skinny_epilogue_and_nan_neighbours(hkg):
    # bias + SiLU on the small-M kernel; NaN scale codes in columns 64-127 of
    # B (block 0) leave every other output as specified, with K = 384 (a
    # half-empty last step).
    M, N, K = 32, 192, 384
    A, SA, B, SB = workloads.make_mx4_inputs(M, N, K, seed=43)
    bias = make_bias(N, 5)
    for variant in (1, 3):
        C = run(hkg, A, SA, B, SB, forced_skinny(hkg, variant), bias=bias, epi="bias_silu")
        stats = check(C, A, SA, B, SB, bias=bias, epi="bias_silu")
        _say("skinny epilogue", variant, stats)
    SB[64:128, 0] = 0xFF
    keep = np.r_[0:64, 128:192]
    Cr, S, absS = oracle.mx4_gemm(A, SA, B[keep], SB[keep])
    for variant in (1, 2, 3):
        C = run(hkg, A, SA, B, SB, forced_skinny(hkg, variant))
        stats = gates.compare_mx4(C[:, keep], Cr, S, absS, K)
        _say("skinny NaN neighbours", variant, stats)


def _exact_inputs(M, N, K, seed):
    # Uniform codes (multiples of 1/2 up to 6) with block scales 2^-1 .. 2^1:
    # products are multiples of 2^-4, every partial sum is bounded by
    # absS <= 36 * 4 * K < 2^18 for K <= 1024 and so a multiple of 2^-4 that
    # fp32's 24 bits hold exactly; the oracle's sum is then the hardware's.
    return workloads.make_mx4_inputs(M, N, K, sa=(126, 129), sb=(126, 129), seed=seed)


@pytest.mark.parametrize("variant,split,shape", [(0, 1, (256, 512, 512)), (0, 1, (300, 260, 384)),
                                                 (1, 1, (200, 136, 512)), (1, 4, (64, 256, 1024)),
                                                 (1, 3, (33, 100, 896))])
def test_mx4_exact_inputs_bit_exact(hkg, variant, split, shape):
    M, N, K = shape
    _say("exact", variant, split, shape)
    A, SA, B, SB = _exact_inputs(M, N, K, seed=M + K)
    C = run(hkg, A, SA, B, SB, forced(hkg, variant, split))
    Cr, S, absS = oracle.mx4_gemm(A, SA, B, SB)
    assert absS.max() < 2.0 ** 18
    assert np.array_equal(C, Cr)


def test_mx4_all_ones_and_one_hot_scales(hkg):
    # 1.0 everywhere with unit scales gives K; one block of one row scaled
    # by 2^3 and one block of one column by 2^-2 move only the outputs they
    # touch, by 7 * 32 and -0.75 * 32 (exact in bf16).
    M, N, K = 130, 70, 512
    A = np.full((M, K // 2), 0x22, np.uint8)
    B = np.full((N, K // 2), 0x22, np.uint8)
    SA = np.full((M, K // 32), 127, np.uint8)
    SB = np.full((N, K // 32), 127, np.uint8)
    SA[5, 7] = 130
    SB[9, 12] = 125
    for variant in (0, 1):
        C = run(hkg, A, SA, B, SB, forced(hkg, variant))
        want = np.full((M, N), float(K))
        want[5, :] += 7 * 32
        want[:, 9] -= 0.75 * 32
        assert np.array_equal(exact.widen(C), want), variant


def test_mx4_half_stage_ignores_next_groups_scales(hkg):
    # K = 384 leaves the last 256-k stage half empty; its empty 128-k step
    # must not pick up the scales the packed layout stores next (the next
    # 64-row group's first step).  NaN codes (0xFF) in block 0 of rows 64-127
    # of A and of columns 64-127 of B: the outputs whose sums they enter are
    # unspecified, every other output is checked.
    M, N, K = 192, 192, 384
    A, SA, B, SB = workloads.make_mx4_inputs(M, N, K, seed=41)
    SA[64:128, 0] = 0xFF
    SB[64:128, 0] = 0xFF
    keep_r = np.r_[0:64, 128:192]
    keep_c = np.r_[0:64, 128:192]
    Cr, S, absS = oracle.mx4_gemm(A[keep_r], SA[keep_r], B[keep_c], SB[keep_c])
    for variant in (0, 1):
        _say("half stage, NaN scales next door, variant", variant)
        C = run(hkg, A, SA, B, SB, forced(hkg, variant))
        stats = gates.compare_mx4(C[np.ix_(keep_r, keep_c)], Cr, S, absS, K)
        _say("variant", variant, stats, "NaN in the rows with NaN codes:",
             bool(np.isnan(exact.widen(C[64:128, :])).all()))


def test_mx4_packed_and_natural_scales_agree(hkg):
    A, SA, B, SB = workloads.make_mx4_inputs(300, 260, 512, seed=11)
    C1 = run(hkg, A, SA, B, SB)
    C2 = run(hkg, A, SA, B, SB, packed=True)
    assert np.array_equal(C1, C2)
    check(C1, A, SA, B, SB)


@pytest.mark.parametrize("epi", ["bias", "bias_relu", "bias_silu", "bias_gelu"])
@pytest.mark.parametrize("variant,split,shape", [(0, 1, (300, 260, 256)), (1, 2, (100, 200, 1024))])
def test_mx4_epilogue_parity(hkg, epi, variant, split, shape):
    M, N, K = shape
    _say("epilogue", epi, variant, split, shape)
    A, SA, B, SB = workloads.make_mx4_inputs(M, N, K, sb=(120, 124), seed=K + len(epi))
    bias = make_bias(N, seed=M)
    C = run(hkg, A, SA, B, SB, forced(hkg, variant, split), bias=bias, epi=epi)
    check(C, A, SA, B, SB, bias=bias, epi=epi)


def test_mx4_errors(hkg):
    import ctypes
    a = dev8(np.zeros((64, 96), np.uint8))
    s = dev8(np.zeros((64, 6), np.uint8))
    c = torch.empty((64, 64), dtype=torch.bfloat16, device="cuda")
    st = hkg.hkg_gemm_mxfp4(a.data_ptr(), s.data_ptr(), a.data_ptr(), s.data_ptr(), None, c.data_ptr(),
                            64, 64, 192, 0, None)
    assert st == hkg.HKG_ERR_INVALID_ARG                    # K % 128 != 0
    a2 = dev8(np.zeros((64, 65), np.uint8))
    st = hkg.hkg_gemm_mxfp4(a2.data_ptr() + 1, s.data_ptr(), a.data_ptr(), s.data_ptr(), None, c.data_ptr(),
                            64, 64, 128, 0, None)
    assert st == hkg.HKG_ERR_MISALIGNED
    st, p = hkg.hkg_gemm_mxfp4_plan(64, 64, 128)
    assert st == hkg.HKG_OK
    p.split_k = 17
    sp = dev8(np.zeros(hkg.hkg_mx_packed_scales_bytes(64, 128), np.uint8))
    st = hkg.hkg_gemm_mxfp4_run_plan(p, a.data_ptr(), sp.data_ptr(), a.data_ptr(), sp.data_ptr(), None,
                                     c.data_ptr(), 64, 64, 128, 0, None)
    assert st == hkg.HKG_ERR_UNSUPPORTED
    torch.cuda.synchronize()


def test_mx4_k_zero_and_empty(hkg):
    a = dev8(np.zeros((8, 0), np.uint8))
    s = dev8(np.zeros((8, 0), np.uint8))
    c = hkg.gemm_mxfp4(a, s, a, s)
    torch.cuda.synchronize()
    assert c.shape == (8, 8) and np.all(host(c) == 0)


def test_mx4_workload_decode_whole_output(hkg):
    # mx4_decode_32x14336x4096 (the blog's best MXFP4 shape) in the
    # planner's launch configuration, every output against the oracle.
    _say("workload mx4_decode_32x14336x4096")
    A, SA, B, SB = workloads.mx4_workload_inputs("mx4_decode_32x14336x4096")
    C = run(hkg, A, SA, B, SB)
    stats = check(C, A, SA, B, SB)
    _say("mx4_decode_32x14336x4096", stats)


def _tile_edges(n, t):
    e = set()
    for b in range(0, n, t):
        e.update((b, min(n, b + t) - 1))
    return np.array(sorted(e), dtype=np.int64)


def test_mx4_workload_square_sampled(hkg):
    # mx4_square_8192 in the planner's launch configuration, checked against
    # the oracle entry by entry: every tile's edge rows crossed with every
    # tile's edge columns, the two whole rows and the two whole columns on
    # each side of the first tile boundary, and 4096 random outputs.
    _say("workload mx4_square_8192")
    A, SA, B, SB = workloads.mx4_workload_inputs("mx4_square_8192")
    M = A.shape[0]
    K = 2 * A.shape[1]
    N = B.shape[0]
    p = hkg.mx4_plan(M, N, K)
    assert p.kernel_id == hkg.HKG_KERNEL_MX4_TILE and p.variant == 0
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
    _say("mx4_square_8192: %d entries" % ii.size)
    Cr, S, absS = oracle.mx4_gemm_entries(A, SA, B, SB, ii, jj)
    stats = gates.compare_mx4(C[ii, jj], Cr, S, absS, K)
    _say("mx4_square_8192", stats)
    assert np.isfinite(exact.widen(C)).all()
