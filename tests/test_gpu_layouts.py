"""GPU parity of the four operand layouts and leading dimensions.

hkg_gemm_bf16_ex runs through the C ABI with A and B stored in row or column
layout, padded leading dimensions (padding filled with NaN patterns: a read
of it would poison the result) and a padded C (whose padding must stay as it
was), on the tile, skinny and general paths, with and without epilogues.
Results are compared element by element with the oracle's layout GEMM on the
same stored arrays (tests/gates.py); hkg_pack_bf16 must produce the exact
row-layout copy.
"""
import numpy as np
import pytest

import oracle
import workloads
from tests import exact, gates

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")

NAN_A, NAN_B = 0x7FC1, 0xFFC3
SENTINEL = 0x4B80


def _say(*a):
    print("[gpu-layouts]", *a, flush=True)


@pytest.fixture(scope="module")
def hkg():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import tile_level_dense_amd as lib
    lib.lib()
    return lib


def stored(X, col, ld, fill):
    rows, K = X.shape
    if col:
        st = np.full((K, ld), fill, dtype=np.uint16)
        st[:, :rows] = X.T
    else:
        st = np.full((rows, ld), fill, dtype=np.uint16)
        st[:, :K] = X
    return st


def dev(bits):
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).to("cuda")


def run_ex(hkg, As, lda, a_col, Bs, ldb, b_col, M, N, K, ldc, bias=None, epi="none"):
    a, b = dev(As), dev(Bs)
    c = dev(np.full((max(M, 1), ldc), SENTINEL, dtype=np.uint16))
    bias_t = dev(bias) if bias is not None else None
    st = hkg.hkg_gemm_bf16_ex(a.data_ptr(), lda, int(a_col), b.data_ptr(), ldb, int(b_col),
                              bias_t.data_ptr() if bias_t is not None else None, c.data_ptr(), ldc, M, N, K,
                              hkg.EPILOGUES[epi], torch.cuda.current_stream().cuda_stream)
    assert st == hkg.HKG_OK, hkg.STATUS.get(st)
    torch.cuda.synchronize()
    return c.view(torch.int16).cpu().numpy().view(np.uint16)


# (name, M, N, K, pad): pad added to every leading dimension; pads keeping
# ld % 8 == 0 run the fast kernels, others the general one
SHAPES = [
    ("tile", 300, 260, 264, 8),
    ("tile_split", 200, 136, 1024, 16),
    ("skinny", 16, 1000, 520, 8),
    ("general_odd_ld", 40, 50, 64, 3),
    ("general_odd_k", 37, 45, 100, 5),
]


@pytest.mark.parametrize("a_col,b_col", [(False, False), (False, True), (True, True), (True, False)],
                         ids=["NT", "NN", "TN", "TT"])
@pytest.mark.parametrize("name,M,N,K,pad", SHAPES, ids=[s[0] for s in SHAPES])
def test_layout_parity(hkg, name, M, N, K, pad, a_col, b_col):
    _say(name, M, N, K, pad, a_col, b_col)
    A, B = workloads.make_inputs(M, N, K, seed=M + N)
    lda = (M if a_col else K) + pad
    ldb = (N if b_col else K) + pad
    ldc = N + 8
    As, Bs = stored(A, a_col, lda, NAN_A), stored(B, b_col, ldb, NAN_B)
    C = run_ex(hkg, As, lda, a_col, Bs, ldb, b_col, M, N, K, ldc)
    Cr, S, absS = oracle.gemm_layout(As, lda, a_col, Bs, ldb, b_col, M, N, K)
    gates.compare(C[:, :N], Cr, S, absS)
    assert np.all(C[:, N:] == SENTINEL), "C padding was written"


@pytest.mark.parametrize("epi", ["bias", "bias_gelu"])
@pytest.mark.parametrize("a_col,b_col", [(False, True), (True, False)], ids=["NN", "TT"])
def test_layout_epilogue(hkg, epi, a_col, b_col):
    M, N, K = 130, 200, 192
    A, B = workloads.make_inputs(M, N, K, seed=7)
    bias = workloads.f32_to_bf16_bits(np.random.default_rng(2).normal(0, 3, size=N).astype(np.float32))
    lda, ldb = (M if a_col else K) + 8, (N if b_col else K) + 8
    As, Bs = stored(A, a_col, lda, NAN_A), stored(B, b_col, ldb, NAN_B)
    C = run_ex(hkg, As, lda, a_col, Bs, ldb, b_col, M, N, K, N, bias=bias, epi=epi)
    _, S, absS = oracle.gemm_layout(As, lda, a_col, Bs, ldb, b_col, M, N, K)
    Ce, Y = oracle.epilogue(S, bias, epi)
    gates.compare_epilogue(C, Ce, Y, absS, np.broadcast_to(exact.widen(bias), S.shape))


def test_layout_k_zero_with_ldc(hkg):
    M, N = 5, 9
    C = run_ex(hkg, np.zeros((1, 8), np.uint16), 8, False, np.zeros((1, 8), np.uint16), 8, False, M, N, 0, 16)
    assert np.all(C[:, :N] == 0) and np.all(C[:, N:] == SENTINEL)


def test_torch_views_pick_layouts(hkg):
    # The binding maps row-major tensors and transposed views to the layouts.
    M, N, K = 96, 80, 128
    A, B = workloads.make_inputs(M, N, K, seed=4)
    a, b = dev(A), dev(B)
    ref = hkg.gemm(a, b)
    for av in (a, a.t().contiguous().t()):
        for bv in (b, b.t().contiguous().t()):
            out = hkg.gemm_ex(av, bv)
            torch.cuda.synchronize()
            assert torch.equal(out.view(torch.int16), ref.view(torch.int16))
    wide = torch.zeros((M, N + 24), dtype=torch.bfloat16, device="cuda")
    hkg.gemm_ex(a, b, out=wide[:, 8:8 + N])
    torch.cuda.synchronize()
    assert torch.equal(wide[:, 8:8 + N].contiguous().view(torch.int16), ref.view(torch.int16))
    assert torch.count_nonzero(wide[:, :8]) == 0 and torch.count_nonzero(wide[:, 8 + N:]) == 0


@pytest.mark.parametrize("col", [False, True])
def test_pack(hkg, col):
    rows, K = 333, 200
    X, _ = workloads.make_inputs(rows, 1, K, seed=9)
    ld = (rows if col else K) + 11
    Xs = stored(X, col, ld, NAN_A)
    y = torch.empty((rows, K), dtype=torch.bfloat16, device="cuda")
    x = dev(Xs)
    st = hkg.hkg_pack_bf16(x.data_ptr(), ld, int(col), y.data_ptr(), rows, K,
                           torch.cuda.current_stream().cuda_stream)
    assert st == hkg.HKG_OK
    torch.cuda.synchronize()
    assert np.array_equal(y.view(torch.int16).cpu().numpy().view(np.uint16), X)


def test_square_8192_with_column_layout_weight(hkg):
    # square_8192 with B in column layout (x @ W with W stored K x N), in the
    # launch the benchmark times; sampled outputs against the oracle.
    A, B = workloads.workload_inputs("square_8192")
    M, K = A.shape
    N = B.shape[0]
    _say("square_8192 NN")
    a, bt = dev(A), dev(np.ascontiguousarray(B.T))
    c = torch.empty((M, N), dtype=torch.bfloat16, device="cuda")
    st = hkg.hkg_gemm_bf16_ex(a.data_ptr(), K, 0, bt.data_ptr(), N, 1, None, c.data_ptr(), N, M, N, K, 0,
                              torch.cuda.current_stream().cuda_stream)
    assert st == hkg.HKG_OK
    torch.cuda.synchronize()
    Cg = c.view(torch.int16).cpu().numpy().view(np.uint16)
    rng = np.random.default_rng(12)
    ii, jj = rng.integers(0, M, 3000), rng.integers(0, N, 3000)
    Cr, S, absS = oracle.gemm_entries(A, B, ii, jj)
    gates.compare(Cg[ii, jj], Cr, S, absS)


# C's leading dimension picks the store path of the tile kernels: a
# multiple of 8 elements takes the 16-byte stores of 8 rows x 128 bytes,
# 4 mod 8 the 8-byte ones, an odd one element stores.  One shape per planner
# tile family (persistent 256 x 256, two-stage 128 x 128, k-interleaved
# 128 x 256, streaming 64 x 64), ragged in N so the last 8-column chunks
# are partial, every output against the oracle and C's padding untouched.
STORE_SHAPES = [("persistent", 4100, 3004, 64, "tile_256x256x64_s2_w4x2_p6"),
                ("ring_128", 2600, 4100, 136, "tile_128x128x64_s2_w2x2_p2"),
                ("kinter", 1300, 4004, 1032, "tile_128x256x64_s3_w2x2_p7"),
                ("streaming", 300, 500, 136, "tile_64x64x64_s4_w2x2_p2")]


@pytest.mark.parametrize("ldc_pad", [8, 4, 1], ids=["wide", "eight_byte", "elements"])
@pytest.mark.parametrize("name,M,N,K,kernel", STORE_SHAPES, ids=[s[0] for s in STORE_SHAPES])
def test_store_paths_by_ldc(hkg, name, M, N, K, kernel, ldc_pad):
    assert hkg.plan(M, N, K).kernel_name.decode() == kernel
    assert N % 8 == 4                        # the last 8-column chunk of a row is partial
    ldc = (N + 7) // 8 * 8 + ldc_pad         # 0, 4 or an odd remainder mod 8
    _say("store path", name, M, N, K, "ldc", ldc)
    A, B = workloads.make_inputs(M, N, K, ("normal", 0.0, 1.0), ("normal", 0.0, 0.05), seed=N + ldc_pad)
    C = run_ex(hkg, A, K, False, B, K, False, M, N, K, ldc)
    assert np.all(C[:, N:] == SENTINEL), "C padding was written"
    Cr, S, absS = oracle.gemm(A, B)
    gates.compare(np.ascontiguousarray(C[:, :N]), Cr, S, absS)
