"""GPU parity at the library's size limits, through the C ABI.

The fast kernels address a tile's operand rows and the split-K partials with
32-bit byte offsets; the planner keeps every launch inside those ranges and
sends larger shapes to the general kernel.  These cases sit on both sides of
each limit, at full size, and compare sampled outputs with the oracle (the
operand rows the samples need are copied back to the host): the largest K a
256-row tile holds (and one step past it), the largest split-K partial
buffer, and the largest K of the small-M kernel.  Inputs are small integers
drawn on the device (bf16-exact), so each case needs no host-side input
generation of its gigabytes.
"""
import numpy as np
import pytest

import oracle
from tests import gates

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")

# Largest K whose 256-row operand range (256 rows x 2K bytes) stays below
# 2^31 bytes, rounded down to the 8-k granule of the fast kernels.
K_TILE_MAX = ((2**31 - 1) // 2 // 256) // 8 * 8


def _say(*a):
    print("[gpu-limits]", *a, flush=True)


@pytest.fixture(scope="module")
def hkg():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import tile_level_dense_amd as lib
    lib.lib()
    return lib


def small_ints(rows, cols, seed):
    g = torch.Generator(device="cuda")
    g.manual_seed(seed)
    return torch.randint(-3, 4, (rows, cols), device="cuda", generator=g, dtype=torch.int8).to(torch.bfloat16)


def bits(t):
    return t.view(torch.int16).cpu().numpy().view(np.uint16)


def check_sampled(c, a, b, n=24, seed=0):
    """Oracle check of n sampled outputs (and the four corners) of c = a b^T."""
    M, N = c.shape
    rng = np.random.default_rng(seed)
    ii = np.concatenate([[0, 0, M - 1, M - 1], rng.integers(0, M, n)])
    jj = np.concatenate([[0, N - 1, 0, N - 1], rng.integers(0, N, n)])
    ui, li = np.unique(ii, return_inverse=True)
    uj, lj = np.unique(jj, return_inverse=True)
    A = bits(a[torch.from_numpy(ui).to("cuda")])
    B = bits(b[torch.from_numpy(uj).to("cuda")])
    Cr, S, absS = oracle.gemm_entries(A, B, li, lj)
    C = bits(c)[ii, jj]
    return gates.compare(C, Cr, S, absS)


@pytest.mark.parametrize("forced", [False, True], ids=["planner", "forced_256x256"])
def test_tile_at_k_limit(hkg, forced):
    # The largest K a 256-row tile addresses: the planner's choice (a split
    # 128-row tile) and the 256 x 256 ping-pong tile forced over all of K.
    M = N = 256
    K = K_TILE_MAX
    p = hkg.plan(M, N, K)
    assert hkg.KERNEL_NAMES[p.kernel_id] == "TILE"
    if forced:
        from tile_level_dense_amd import build as hkg_build
        assert hkg_build.tile_configs()[0][:2] == (256, 256)
        p.variant, p.tile_m, p.tile_n, p.tile_k, p.waves = 0, 256, 256, 64, 8
        p.split_k, p.grid_y, p.workspace_bytes = 1, 1, 0
    _say("K", K, "variant", p.variant, (p.tile_m, p.tile_n), "split", p.split_k)
    a, b = small_ints(M, K, 1), small_ints(N, K, 2)
    c = hkg.run_plan(p, a, b)
    torch.cuda.synchronize()
    assert torch.isfinite(c.float()).all().item()
    _say(check_sampled(c, a, b))
    del a, b, c
    torch.cuda.empty_cache()


def test_generic_past_k_limit(hkg):
    M = N = 64
    K = K_TILE_MAX + 8
    p = hkg.plan(M, N, K)
    _say("K", K, p.kernel_name.decode())
    assert hkg.KERNEL_NAMES[p.kernel_id] == "GENERIC"
    a, b = small_ints(M, K, 7), small_ints(N, K, 8)
    c = hkg.gemm(a, b)
    torch.cuda.synchronize()
    _say(check_sampled(c, a, b))
    del a, b, c
    torch.cuda.empty_cache()


def test_largest_split_k_partials(hkg):
    # M N 4 bytes of fp32 partials per split just below 2^31: the planner's
    # bound for split-K; forced onto the 128 x 128 tile with 3 splits.
    from tile_level_dense_amd import build as hkg_build
    M, N, K = 8192, 65528, 640
    assert M * N < 2**29 and (M * N + 8 * 128) * 4 >= 2**31 - 2**20
    variant = next(v for v, cfg in enumerate(hkg_build.tile_configs()) if cfg == (128, 128, 64, 2, 2, 2, 2))
    p = hkg.plan(M, N, K)
    p.kernel_id = hkg.HKG_KERNEL_TILE
    p.variant = variant
    p.tile_m, p.tile_n, p.tile_k, p.waves = 128, 128, 64, 4
    p.split_k, p.grid_y = 3, 3
    p.workspace_bytes = 3 * M * N * 4
    _say("split-K partials", (M, N, K), "workspace", p.workspace_bytes)
    a, b = small_ints(M, K, 3), small_ints(N, K, 4)
    c = hkg.run_plan(p, a, b)
    c2 = hkg.run_plan(p, a, b)
    torch.cuda.synchronize()
    assert torch.equal(c.view(torch.int16), c2.view(torch.int16))
    assert torch.isfinite(c.float()).all().item()
    _say(check_sampled(c, a, b, n=200))
    del a, b, c, c2
    torch.cuda.empty_cache()


def test_small_m_kernel_longest_k(hkg):
    M, N, K = 16, 4096, K_TILE_MAX
    p = hkg.plan(M, N, K)
    _say("small-M", (M, N, K), p.kernel_name.decode(), "split", p.split_k)
    assert hkg.KERNEL_NAMES[p.kernel_id] == "SKINNY"
    a, b = small_ints(M, K, 5), small_ints(N, K, 6)
    c = hkg.gemm(a, b)
    torch.cuda.synchronize()
    _say(check_sampled(c, a, b, n=64))
    del a, b, c
    torch.cuda.empty_cache()
