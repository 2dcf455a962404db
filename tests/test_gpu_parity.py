"""GPU parity: the HIP library against the CPU oracle, through the C ABI.

Every case runs libhkg.so on an MI355X and compares element by element with
the oracle on the same seeded inputs (tests/gates.py states the tolerance).
Special inputs whose fp32 sums are exact (all-ones, identity, small
integers) must match bit for bit.  The full-size workloads are compared on
sampled rows spread over tiles and on random elements, plus properties of
the whole output (finite, bit-identical on a repeat run).
"""
import numpy as np
import pytest

import oracle
import workloads
from tests import gates

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


def _say(*a):
    print("[gpu-parity]", *a, flush=True)


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


def run(hkg, A, B, **kw):
    a, b = dev(A), dev(B)
    c = hkg.gemm(a, b, **kw)
    torch.cuda.synchronize()
    return host(c)


def full_check(C, A, B, exact=False):
    Cr, S, absS = oracle.gemm(A, B)
    if exact:
        assert np.array_equal(C, Cr), "not bit-exact: %d of %d differ" % (int((C != Cr).sum()), C.size)
        return None
    return gates.compare(C, Cr, S, absS)


def oracle_rows(A, B, rows):
    """Oracle (C_ref, S, absS) for the listed rows of C."""
    parts = [oracle.gemm(A, B, rows=(r, r + 1)) for r in rows]
    return tuple(np.concatenate([p[t] for p in parts]) for t in range(3))


def sample_rows(M, tile=256, extra=8, seed=0):
    rows = {0, 1, M - 1, M // 2}
    for t in range(0, M, tile):
        rows.update({t, min(M - 1, t + tile - 1), min(M - 1, t + 17)})
    rng = np.random.default_rng(seed)
    rows.update(int(r) for r in rng.integers(0, M, size=extra))
    return sorted(r for r in rows if 0 <= r < M)


# ------------------------------------------------------------- workloads
@pytest.mark.parametrize("name", workloads.ORDER)
def test_workload_parity(hkg, name):
    w = workloads.WORKLOADS[name]
    M, N, K = w["M"], w["N"], w["K"]
    _say("workload", name, (M, N, K), "seed 0", "plan", hkg.plan(M, N, K).kernel_name.decode())
    A, B = workloads.workload_inputs(name)
    a, b = dev(A), dev(B)
    c = hkg.gemm(a, b)
    c2 = hkg.gemm(a, b)
    torch.cuda.synchronize()
    C = host(c)
    assert np.array_equal(C, host(c2)), "repeat run differs"
    assert torch.isfinite(c.float()).all().item()
    if M * N * K <= 8 * 10**9:
        stats = full_check(C, A, B)
    else:
        rows = sample_rows(M)
        stats = gates.compare(C[rows], *oracle_rows(A, B, rows))
        rng = np.random.default_rng(1)
        ii = rng.integers(0, M, size=20000)
        jj = rng.integers(0, N, size=20000)
        Ce, Se, ae = oracle.gemm_entries(A, B, ii, jj)
        gates.compare(C[ii, jj], Ce, Se, ae)
    _say(name, stats)


# -------------------------------------------------------- exact inputs
EXACT_SHAPES = [(512, 512, 512), (300, 260, 136), (16, 1024, 4096), (128, 640, 1024), (5, 48, 8192)]


@pytest.mark.parametrize("shape", EXACT_SHAPES)
def test_all_ones_is_K(hkg, shape):
    M, N, K = shape
    _say("all-ones", shape)
    A = np.full((M, K), 0x3F80, np.uint16)
    B = np.full((N, K), 0x3F80, np.uint16)
    C = run(hkg, A, B)
    want = oracle.bf16_rne(float(K))
    assert np.all(C == want)


@pytest.mark.parametrize("shape", EXACT_SHAPES)
def test_small_integers_bit_exact(hkg, shape):
    # |entries| <= 4 and K * 16 < 2^24: every fp32 partial sum is exact.
    M, N, K = shape
    _say("small-int", shape)
    rng = np.random.default_rng(21)
    A = workloads.f32_to_bf16_bits(rng.integers(-4, 5, size=(M, K)).astype(np.float32))
    B = workloads.f32_to_bf16_bits(rng.integers(-4, 5, size=(N, K)).astype(np.float32))
    C = run(hkg, A, B)
    full_check(C, A, B, exact=True)


@pytest.mark.parametrize("side", ["A", "B"])
def test_identity_bit_exact(hkg, side):
    K = 384
    _say("identity", side)
    I = np.zeros((K, K), np.uint16)
    I[np.arange(K), np.arange(K)] = 0x3F80
    rng = np.random.default_rng(3)
    X = workloads.draw(rng, (200, K), ("normal", 0.0, 1.0))
    if side == "A":
        C = run(hkg, I, X)          # C = X^T
        assert np.array_equal(C, X.T)
    else:
        C = run(hkg, X, I)          # C = X
        assert np.array_equal(C, X)


def test_identity_skinny(hkg):
    K = 1024
    _say("identity skinny")
    I = np.zeros((K, K), np.uint16)
    I[np.arange(K), np.arange(K)] = 0x3F80
    X = workloads.draw(np.random.default_rng(4), (40, K), ("uniform", -1.0, 1.0))
    assert np.array_equal(run(hkg, X, I), X)


# ------------------------------------------------------------ ragged
RAGGED = [(1, 1, 8), (15, 17, 24), (17, 33, 40), (16, 4096, 64), (33, 100, 520), (127, 129, 136),
          (128, 257, 72), (129, 127, 72), (255, 257, 264), (257, 255, 128), (300, 520, 200),
          (513, 385, 1000), (1000, 36, 64), (64, 7, 4096), (7, 3000, 8),
          (33, 47, 13), (130, 70, 99), (3, 5, 1), (200, 90, 1001)]


@pytest.mark.parametrize("shape", RAGGED, ids=lambda s: "%dx%dx%d" % s)
def test_ragged_shapes(hkg, shape):
    M, N, K = shape
    p = hkg.plan(M, N, K)
    _say("ragged", shape, p.kernel_name.decode())
    A, B = workloads.make_inputs(M, N, K, ("normal", 0.0, 1.0), ("normal", 0.0, 0.02), seed=M * 7 + N)
    full_check(run(hkg, A, B), A, B)


# One round of k-interleaved tiles (two 4-wave groups over the whole tile,
# alternate 64-k stages, partials added through LDS), as the planner picks
# them: ragged M, N and K, an odd number of stages (the last one padded
# with zeros), every output; a second run is bit-identical.
KINTER_SHAPES = [((1300, 4000, 1032), "tile_128x256x64_s3_w2x2_p7"),
                 ((1280, 4096, 1096), "tile_128x256x64_s3_w2x2_p7"),
                 ((1000, 3600, 1160), "tile_128x128x64_s3_w2x2_p7"),
                 ((250, 16384, 1032), "tile_128x128x64_s3_w2x2_p7")]


@pytest.mark.parametrize("shape,name", KINTER_SHAPES, ids=lambda v: "%dx%dx%d" % v if isinstance(v, tuple) else v)
def test_kinter_planner_shapes(hkg, shape, name):
    M, N, K = shape
    p = hkg.plan(M, N, K)
    _say("k-interleaved", shape, p.kernel_name.decode())
    assert p.kernel_name.decode() == name, p
    A, B = workloads.make_inputs(M, N, K, ("normal", 0.0, 1.0), ("normal", 0.0, 0.02), seed=M + N)
    C1 = run(hkg, A, B)
    full_check(C1, A, B)
    assert np.array_equal(C1, run(hkg, A, B))


def test_kinter_strided(hkg):
    """Padded leading dimensions of A, B and C on the k-interleaved tile
    (through the layout entry point's in-place path); C's padding kept."""
    M, N, K = 1300, 4000, 1032
    lda, ldb, ldc = K + 24, K + 8, N + 40
    assert hkg.plan(M, N, K).kernel_name.decode() == "tile_128x256x64_s3_w2x2_p7"
    A, B = workloads.make_inputs(M, N, K, ("normal", 0.0, 1.0), ("normal", 0.0, 0.02), seed=7)
    As = np.full((M, lda), 0x7FC1, dtype=np.uint16)
    As[:, :K] = A
    Bs = np.full((N, ldb), 0xFFC3, dtype=np.uint16)
    Bs[:, :K] = B
    a, b = dev(As), dev(Bs)
    c = dev(np.full((M, ldc), 0x4B80, dtype=np.uint16))
    _say("k-interleaved strided", (M, N, K))
    st = hkg.hkg_gemm_bf16_ex(a.data_ptr(), lda, hkg.LAYOUT_ROW, b.data_ptr(), ldb, hkg.LAYOUT_ROW, None,
                              c.data_ptr(), ldc, M, N, K, 0, torch.cuda.current_stream().cuda_stream)
    assert st == hkg.HKG_OK
    torch.cuda.synchronize()
    Cs = host(c)
    assert (Cs[:, N:] == 0x4B80).all()
    full_check(np.ascontiguousarray(Cs[:, :N]), A, B)


@pytest.mark.parametrize("workload,name", [("middle_2048x4096x4096", "tile_128x256x64_s3_w2x2_p7"),
                                           ("middle_1024x4096x4096", "tile_128x128x64_s5_w2x2_p7")])
def test_kinter_full_size_sampled(hkg, workload, name):
    """The compute-bound middle workloads the benchmark times, at their
    size and inputs: rows at every tile boundary and 20000 random outputs
    against the oracle."""
    w = workloads.MIDDLE_WORKLOADS[workload]
    M, N, K = w["M"], w["N"], w["K"]
    p = hkg.plan(M, N, K)
    _say("k-interleaved full size", workload, p.kernel_name.decode())
    assert p.kernel_name.decode() == name, p
    A, B = workloads.workload_inputs(workload)
    C = run(hkg, A, B)
    rows = sample_rows(M, tile=128)
    gates.compare(C[rows], *oracle_rows(A, B, rows))
    rng = np.random.default_rng(2)
    ii = rng.integers(0, M, size=20000)
    jj = rng.integers(0, N, size=20000)
    Ce, Se, ae = oracle.gemm_entries(A, B, ii, jj)
    gates.compare(C[ii, jj], Ce, Se, ae)


def test_planner_wide_n_streaming_tile(hkg):
    # Mid-size M, wide N: the planner's 128 x 96 streaming tile (one round of
    # 256 tiles; 128 x 128 would leave 64 CUs idle), ragged M and K, every
    # output against the oracle.
    M, N, K = 200, 12288, 520
    p = hkg.plan(M, N, K)
    _say("wide-N streaming tile", (M, N, K), p.kernel_name.decode())
    assert (p.tile_m, p.tile_n, p.split_k, p.grid_x) == (128, 96, 1, 256), p
    A, B = workloads.make_inputs(M, N, K, ("normal", 0.0, 1.0), ("normal", 0.0, 0.02), seed=96)
    full_check(run(hkg, A, B), A, B)


@pytest.mark.parametrize("shape", [(16, 8192, 4096), (13, 6000, 1000), (1, 4112, 256)],
                         ids=lambda s: "%dx%dx%d" % s)
def test_planner_skinny_two_rounds(hkg, shape):
    # M <= 16 with 257 to 512 column blocks of 16: the planner's small-M
    # kernel over two rounds of workgroups, every output against the oracle.
    M, N, K = shape
    p = hkg.plan(M, N, K)
    _say("skinny, two rounds", shape, p.kernel_name.decode())
    assert hkg.KERNEL_NAMES[p.kernel_id] == "SKINNY" and p.grid_x == -(-N // 16), p
    A, B = workloads.make_inputs(M, N, K, ("normal", 0.0, 1.0), ("normal", 0.0, 0.02), seed=N + K)
    full_check(run(hkg, A, B), A, B)


# ---------------------------------------------------- forced plans
def forced(hkg, A, B, edit):
    M, K = A.shape
    N = B.shape[0]
    p = hkg.plan(M, N, K)
    edit(p)
    c = hkg.run_plan(p, dev(A), dev(B))
    torch.cuda.synchronize()
    return host(c)


def force_tile(hkg, p, variant, win_w=None, chunk_c=None, split=1):
    """Edit plan p to run tile-kernel variant `variant` (hkg_tile_configs.h)."""
    from tile_level_dense_amd import build as hkg_build
    bm, bn, bk, stages, wm, wn, sc = hkg_build.tile_configs()[variant]
    p.kernel_id = hkg.HKG_KERNEL_TILE
    p.variant = variant
    # schedule 7: two groups, each a wm x wn grid over the whole tile
    p.tile_m, p.tile_n, p.tile_k, p.waves = bm, bn, bk, wm * wn * (2 if sc == 7 else 1)
    p.split_k = split
    p.grid_y = split
    p.workspace_bytes = split * p.M * p.N * 4 if split > 1 else 0
    if win_w is not None:
        p.xcd_window_w = win_w
    if chunk_c is not None:
        p.xcd_chunk_c = chunk_c


def _n_tile_variants():
    from tile_level_dense_amd import build as hkg_build
    return len(hkg_build.tile_configs())


TILE_SHAPES = [(300, 500, 136), (256, 256, 64), (129, 1, 8), (700, 260, 520), (200, 1030, 72),
               (520, 1000, 392)]


@pytest.mark.parametrize("variant", range(_n_tile_variants()))
@pytest.mark.parametrize("shape", TILE_SHAPES, ids=lambda s: "%dx%dx%d" % s)
def test_forced_tile_variants(hkg, variant, shape):
    M, N, K = shape
    _say("tile variant", variant, shape)
    A, B = workloads.make_inputs(M, N, K, seed=variant + 10)
    full_check(forced(hkg, A, B, lambda p: force_tile(hkg, p, variant)), A, B)


TILE_SPLIT_SHAPES = [(300, 500, 136), (520, 1000, 392), (129, 40, 4104)]


def _split_variants():
    from tile_level_dense_amd import build as hkg_build
    return [v for v, (bm, bn, bk, st, wm, wn, sc) in enumerate(hkg_build.tile_configs())
            if (bm // wm // 16) * (bn // wn // 16) <= 16 and sc != 7]


@pytest.mark.parametrize("variant", _split_variants())
@pytest.mark.parametrize("split", (2, 3, 5))
@pytest.mark.parametrize("shape", TILE_SPLIT_SHAPES, ids=lambda s: "%dx%dx%d" % s)
def test_forced_tile_split(hkg, variant, split, shape):
    """Split-K tile runs, including splits whose K range is empty (K of 2
    or 3 k-tiles over 5 splits); two runs agree bit for bit (the partials
    are summed in split order)."""
    M, N, K = shape
    _say("tile variant", variant, "split", split, shape)
    A, B = workloads.make_inputs(M, N, K, ("normal", 0.0, 1.0), ("normal", 0.0, 0.05), seed=split + 10)
    C1 = forced(hkg, A, B, lambda p: force_tile(hkg, p, variant, split=split))
    full_check(C1, A, B)
    C2 = forced(hkg, A, B, lambda p: force_tile(hkg, p, variant, split=split))
    assert np.array_equal(C1, C2)


def _persistent_variant():
    from tile_level_dense_amd import build as hkg_build
    return [v for v, c in enumerate(hkg_build.tile_configs()) if c[6] == 6][0]


# More tiles than the persistent grid's 256 workgroups, so workgroups walk
# two to four tiles: ragged M, N and K; one stage per tile (K = 64: the
# copies running ahead are always in the next tile); three or four tiles.
PERSISTENT_SHAPES = [(4400, 4200, 200), (4352, 4352, 64), (7168, 7000, 72), (4608, 4352, 8)]


@pytest.mark.parametrize("shape", PERSISTENT_SHAPES, ids=lambda s: "%dx%dx%d" % s)
def test_persistent_pingpong_multi_tile(hkg, shape):
    """The persistent ping-pong over every output of shapes whose workgroups
    walk several tiles; a second run is bit-identical."""
    M, N, K = shape
    v = _persistent_variant()
    _say("persistent ping-pong", shape, "tiles", -(-M // 256) * -(-N // 256))
    A, B = workloads.make_inputs(M, N, K, ("normal", 0.0, 1.0), ("normal", 0.0, 0.02), seed=M + K)
    C1 = forced(hkg, A, B, lambda p: force_tile(hkg, p, v))
    full_check(C1, A, B)
    C2 = forced(hkg, A, B, lambda p: force_tile(hkg, p, v))
    assert np.array_equal(C1, C2)


# More 256 x 256 tiles than compute units with a last round of at most half
# of them: the planner splits that round's tiles into two halves of K (the
# grouped kernel's streamed schedule with one expert).  Ragged M, N and K,
# every output; a second run is bit-identical (each split tile's two fp32
# partials are added once, a commutative sum).
SPLIT_TAIL_SHAPES = [(4400, 4200, 136), (4352, 4096, 520), (4100, 4608, 72)]


@pytest.mark.parametrize("shape", SPLIT_TAIL_SHAPES, ids=lambda s: "%dx%dx%d" % s)
def test_split_tail_planner_shapes(hkg, shape):
    M, N, K = shape
    p = hkg.plan(M, N, K)
    _say("split last round", shape, p.reason.decode())
    assert p.split_k == 2 and "last round split" in p.reason.decode(), p
    A, B = workloads.make_inputs(M, N, K, ("normal", 0.0, 1.0), ("normal", 0.0, 0.02), seed=M + N + K)
    C1 = run(hkg, A, B)
    full_check(C1, A, B)
    assert np.array_equal(C1, run(hkg, A, B))


def test_persistent_pingpong_strided(hkg):
    """Row-layout operands and C with padded leading dimensions on the
    persistent ping-pong (through the layout entry point's in-place path)."""
    M, N, K = 4352, 4224, 136
    lda, ldb, ldc = K + 24, K + 8, N + 40
    A, B = workloads.make_inputs(M, N, K, ("normal", 0.0, 1.0), ("normal", 0.0, 0.02), seed=3)
    As = np.full((M, lda), 0x7FC1, dtype=np.uint16)
    As[:, :K] = A
    Bs = np.full((N, ldb), 0xFFC3, dtype=np.uint16)
    Bs[:, :K] = B
    a, b = dev(As), dev(Bs)
    c = dev(np.full((M, ldc), 0x4B80, dtype=np.uint16))
    p = hkg.plan(M, N, K)
    _say("persistent strided plan", p.kernel_name.decode())
    st = hkg.hkg_gemm_bf16_ex(a.data_ptr(), lda, hkg.LAYOUT_ROW, b.data_ptr(), ldb, hkg.LAYOUT_ROW, None,
                              c.data_ptr(), ldc, M, N, K, 0, torch.cuda.current_stream().cuda_stream)
    assert st == hkg.HKG_OK
    torch.cuda.synchronize()
    Cs = host(c)
    assert (Cs[:, N:] == 0x4B80).all()
    full_check(np.ascontiguousarray(Cs[:, :N]), A, B)


def _skinny_configs():
    from tile_level_dense_amd import build as hkg_build
    return hkg_build.skinny_configs()


SKINNY_SHAPES = [(16, 512, 8192), (20, 300, 4096), (64, 1000, 2056), (128, 96, 8192), (100, 33, 1000),
                 (1, 4100, 1024), (9, 64, 264)]
SKINNY_CASES = [(v, s, shape) for v, cfg in enumerate(_skinny_configs()) for shape in SKINNY_SHAPES
                if shape[0] <= 16 * cfg[0] for s in (1, 3, 7)]


@pytest.mark.parametrize("variant,split,shape", SKINNY_CASES)
def test_forced_skinny_split(hkg, variant, split, shape):
    M, N, K = shape
    _say("skinny variant", variant, "split", split, shape)
    A, B = workloads.make_inputs(M, N, K, ("normal", 0.0, 1.0), ("normal", 0.0, 0.02), seed=split)

    mb, nb, wk, u, cp, al = _skinny_configs()[variant]

    def edit(p):
        p.kernel_id = hkg.HKG_KERNEL_SKINNY
        p.variant = variant
        p.tile_m, p.tile_n, p.waves = 16 * mb, 16 * nb, wk
        p.split_k = split
    C1 = forced(hkg, A, B, edit)
    C2 = forced(hkg, A, B, edit)       # counters must be back at zero
    assert np.array_equal(C1, C2)
    full_check(C1, A, B)


def test_forced_generic(hkg):
    M, N, K = 150, 70, 264
    _say("generic forced", (M, N, K))
    A, B = workloads.make_inputs(M, N, K, seed=5)

    def edit(p):
        p.kernel_id = hkg.HKG_KERNEL_GENERIC
    full_check(forced(hkg, A, B, edit), A, B)


@pytest.mark.parametrize("w,c", [(0, 0), (1, 0), (3, 2), (8, 4), (5, 1), (9, 0), (8, 32), (2, 1)])
def test_tile_orders(hkg, w, c):
    M = N = 2304          # 9 x 9 tiles of 256: ragged against 8 XCDs and windows
    K = 128
    _say("tile order", w, c)
    A, B = workloads.make_inputs(M, N, K, seed=w * 10 + c)

    def edit(p):
        force_tile(hkg, p, 0, win_w=w, chunk_c=c)
    C = forced(hkg, A, B, edit)
    rows = sample_rows(M, extra=16)
    gates.compare(C[rows], *oracle_rows(A, B, rows))
    # every tile written: compare a column sample over all rows
    cols = np.arange(0, N, 97)
    ii, jj = np.meshgrid(np.arange(M), cols, indexing="ij")
    Ce, Se, ae = oracle.gemm_entries(A, B, ii.ravel(), jj.ravel())
    gates.compare(C[ii.ravel(), jj.ravel()], Ce, Se, ae)


# ----------------------------------------------------- edge handling
def test_misaligned_pointers_take_generic(hkg):
    M, N, K = 64, 48, 200
    _say("misaligned", (M, N, K))
    A, B = workloads.make_inputs(M, N, K, seed=6)
    a_buf = torch.zeros(M * K + 1, dtype=torch.bfloat16, device="cuda")
    b_buf = torch.zeros(N * K + 1, dtype=torch.bfloat16, device="cuda")
    c_buf = torch.zeros(M * N + 1, dtype=torch.bfloat16, device="cuda")
    a_buf[1:] = dev(A).reshape(-1)
    b_buf[1:] = dev(B).reshape(-1)
    st = hkg.hkg_gemm_bf16(a_buf.data_ptr() + 2, b_buf.data_ptr() + 2, c_buf.data_ptr() + 2, M, N, K,
                           torch.cuda.current_stream().cuda_stream)
    assert st == hkg.HKG_OK
    torch.cuda.synchronize()
    full_check(host(c_buf[1:]).reshape(M, N), A, B)
    p = hkg.plan(M, N, K)
    st = hkg.hkg_gemm_bf16_run_plan(p, a_buf.data_ptr() + 2, b_buf.data_ptr() + 2, c_buf.data_ptr() + 2,
                                    M, N, K, None)
    assert st == hkg.HKG_ERR_MISALIGNED


def test_k_zero_fills_zero(hkg):
    _say("K = 0")
    a = torch.empty((37, 0), dtype=torch.bfloat16, device="cuda")
    b = torch.empty((29, 0), dtype=torch.bfloat16, device="cuda")
    out = torch.full((37, 29), 3.0, dtype=torch.bfloat16, device="cuda")
    hkg.gemm(a, b, out=out)
    torch.cuda.synchronize()
    assert np.all(host(out) == 0)


def test_empty_output_is_noop(hkg):
    _say("M = 0")
    a = torch.empty((0, 64), dtype=torch.bfloat16, device="cuda")
    b = torch.ones((8, 64), dtype=torch.bfloat16, device="cuda")
    assert hkg.gemm(a, b).shape == (0, 8)


def test_device_status_ok(hkg):
    p = hkg.plan(256, 256, 256)
    a = torch.zeros((256, 256), dtype=torch.bfloat16, device="cuda")
    out = hkg.run_plan(p, a, a)
    torch.cuda.synchronize()
    assert out.shape == (256, 256)
