"""hkg_gemm_bf16_noalloc against hkg_gemm_bf16 through the C ABI.

The no-allocation form runs the same plan and kernels with its split-K
scratch in a fixed device array, so its output must equal hkg_gemm_bf16's
bit for bit.  Two calls in a row on split-K shapes (tile and small-M
kernels), the second smaller than the first, so the second runs on scratch
the first left behind; plus unsplit shapes (no scratch) and the oracle gate
on one of them.
"""
import numpy as np
import pytest

import oracle
import workloads
from tests import gates

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


def _say(*a):
    print("[gpu-noalloc]", *a, flush=True)


@pytest.fixture(scope="module")
def hkg():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import tile_level_dense_amd as lib
    lib.lib()
    return lib


def dev16(bits):
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).to("cuda")


def host16(t):
    return t.view(torch.int16).cpu().numpy().view(np.uint16)


def both(hkg, M, N, K, seed):
    A, B = workloads.make_inputs(M, N, K, ("normal", 0.0, 1.0), ("normal", 0.0, 0.02), seed=seed)
    a, b = dev16(A), dev16(B)
    c_ref = torch.full((M, N), 7.0, dtype=torch.bfloat16, device="cuda")
    c_na = torch.full((M, N), -7.0, dtype=torch.bfloat16, device="cuda")
    stream = torch.cuda.current_stream().cuda_stream
    st = hkg.hkg_gemm_bf16(a.data_ptr(), b.data_ptr(), c_ref.data_ptr(), M, N, K, stream)
    assert st == hkg.HKG_OK, hkg.hkg_status_string(st)
    st = hkg.hkg_gemm_bf16_noalloc(a.data_ptr(), b.data_ptr(), c_na.data_ptr(), M, N, K, stream)
    assert st == hkg.HKG_OK, hkg.hkg_status_string(st)
    torch.cuda.synchronize()
    return A, B, host16(c_ref), host16(c_na)


# pairs of (first, second smaller) shapes; the planner's split for each is checked
PAIRS = [
    ((64, 512, 4096), (32, 256, 2048)),        # tile 64 x 64, split 8 then 4
    ((16, 256, 8192), (8, 128, 4096)),         # small-M kernel, split 4 then 4 on fewer columns
    ((128, 1024, 8192), (64, 512, 4096)),      # tile split 8, the larger partials first
]


@pytest.mark.parametrize("first,second", PAIRS, ids=["%dx%dx%d" % p[0] for p in PAIRS])
def test_noalloc_equals_gemm_two_calls(hkg, first, second):
    for i, (M, N, K) in enumerate((first, second)):
        p = hkg.plan(M, N, K)
        assert p.split_k > 1, (M, N, K, p.kernel_name)
        A, B, c_ref, c_na = both(hkg, M, N, K, seed=40 + i)
        _say("%dx%dx%d" % (M, N, K), p.kernel_name.decode(), "split", p.split_k,
             "workspace", p.workspace_bytes)
        assert np.array_equal(c_na, c_ref), ("call", i, (M, N, K))
        if i == 1:
            Cr, S, absS = oracle.gemm(A, B)
            _say("gate", gates.compare(c_na, Cr, S, absS))


def test_noalloc_unsplit_and_tiny(hkg):
    for (M, N, K) in ((256, 256, 256), (16, 4096, 512), (3, 5, 24)):
        A, B, c_ref, c_na = both(hkg, M, N, K, seed=7)
        assert np.array_equal(c_na, c_ref), (M, N, K)


def test_noalloc_split_last_round_runs_whole(hkg):
    """Where the plan splits the last round of 256 x 256 tiles (64 MiB of
    partials, more than the fixed scratch), the no-allocation form runs
    those tiles whole: every output against the oracle, twice, the second
    call after a split-K call has left partials and counters behind."""
    M, N, K = 4352, 4096, 200
    p = hkg.plan(M, N, K)
    assert p.split_k == 2 and "last round split" in p.reason.decode(), p
    for i in range(2):
        A, B, c_ref, c_na = both(hkg, M, N, K, seed=60 + i)
        _say("split last round", (M, N, K), "call", i)
        Cr, S, absS = oracle.gemm(A, B)
        gates.compare(c_na, Cr, S, absS)
        gates.compare(c_ref, Cr, S, absS)
        if i == 0:
            both(hkg, 64, 512, 4096, seed=5)       # a split-K call on the fixed scratch in between
