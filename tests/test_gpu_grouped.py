"""GPU parity of the grouped (mixture-of-experts) GEMM against the oracle.

Every grouped tile variant runs through the C ABI on the persistent grid, with
the planner's grid and with forced grids (one workgroup walking every tile,
grids that are not a multiple of the 8 chiplets, the chiplet-contiguous walk
on and off, a last round split into two halves of K and the same launches
unsplit), on ragged expert sizes with empty experts, more than 64 experts
(several steps of the wave-parallel expert walk), every epilogue, and the
MoE workloads on row ranges across expert boundaries.  Each row of an expert
is compared element by element with the oracle (tests/gates.py); rows that
belong to no expert must keep what the output held.
"""
import numpy as np
import pytest

import oracle
import workloads
from tests import exact, gates

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")

SENTINEL = 0x4B80          # bf16 16777216.0: no GEMM here produces it


def _say(*a):
    print("[gpu-grouped]", *a, flush=True)


@pytest.fixture(scope="module")
def hkg():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import tile_level_dense_amd as lib
    lib.lib()
    return lib


def dev(bits):
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).to("cuda")


def host(t):
    return t.view(torch.int16).cpu().numpy().view(np.uint16)


def run(hkg, A, B, offs, variant=None, grid=None, xcd=None, bias=None, epi="none", split=None):
    M, K = A.shape
    G, N = B.shape[0], B.shape[1]
    out = torch.from_numpy(np.full((M, N), SENTINEL, dtype=np.uint16).view(np.int16)).view(torch.bfloat16).to("cuda")
    plan = None
    if variant is not None or grid is not None or xcd is not None or split is not None:
        from tile_level_dense_amd import build as hkg_build
        plan = hkg.grouped_plan(G, M, N, K)
        if variant is not None:
            bm, bn, bk, st, wm, wn, _ = hkg_build.tile_configs(grouped=True)[variant]
            plan.variant, plan.tile_m, plan.tile_n, plan.tile_k, plan.waves = variant, bm, bn, bk, wm * wn
        if grid is not None:
            plan.grid_x = grid
        if xcd is not None:
            plan.xcd_chunk_c = xcd
        if split is not None:
            plan.split_k = split
            plan.workspace_bytes = plan.grid_x * plan.tile_m * plan.tile_n * 4 if split == 2 else 0
    offs_t = torch.from_numpy(np.ascontiguousarray(offs, dtype=np.int32)).to("cuda")
    hkg.grouped_gemm(dev(A), dev(B), offs_t, out=out, bias=dev(bias) if bias is not None else None, epilogue=epi,
                     plan=plan)
    torch.cuda.synchronize()
    return host(out)


def check(C, A, B, offs, bias=None, epi="none", rows=None):
    end = int(offs[-1])
    r0, r1 = (0, end) if rows is None else rows
    Cr, S, absS = oracle.grouped_gemm(A, B, offs, rows=(r0, r1))
    if epi == "none":
        gates.compare(C[r0:r1], Cr, S, absS)
    else:
        # the oracle's epilogue takes one bias row: apply it expert by expert
        g = np.searchsorted(offs, np.arange(r0, r1), side="right")
        bvals = exact.widen(bias)[g]
        Ce = np.empty_like(Cr)
        Y = np.empty_like(S)
        for e in np.unique(g):
            sel = g == e
            Ce[sel], Y[sel] = oracle.epilogue(S[sel], bias[e], epi)
        gates.compare_epilogue(C[r0:r1], Ce, Y, absS, bvals)
    if rows is None:
        assert np.all(C[end:] == SENTINEL), "rows of no expert were written"


CASES = [
    # name, sizes, N, K, variant, grid, xcd
    ("planner_tiny", [64, 0, 100, 92], 256, 256, None, None, None),
    ("v256_ragged", [1, 255, 0, 300, 17], 300, 192, 0, None, None),
    ("v128_ragged", [1, 255, 0, 300, 17], 300, 192, 1, None, None),
    ("v128_one_workgroup", [33, 0, 129, 7], 140, 128, 1, 1, 0),
    ("v256_one_workgroup", [300, 5, 0, 260], 260, 64, 0, 1, 0),
    ("v128_grid7_round_robin", [100, 200, 0, 3], 333, 136, 1, 7, 1),
    ("v128_grid16_xcd", [129, 0, 0, 511, 64], 270, 200, 1, 16, 1),
    ("v256_grid24_xcd", [513, 0, 257], 530, 128, 0, 24, 1),
    ("leading_empty_experts", [0, 0, 0, 70, 0], 96, 64, 1, None, None),
    # the ping-pong tile (variant 2): several tiles per workgroup, one-stage
    # and ragged K, XCD-chunked walk
    ("pp_ragged", [1, 255, 0, 300, 17], 300, 192, 2, None, None),
    ("pp_one_workgroup_one_stage", [300, 5, 0, 260], 260, 64, 2, 1, 0),
    ("pp_grid3_ragged_k", [300, 70], 260, 520, 2, 3, None),
    ("pp_grid24_xcd", [513, 0, 257], 530, 128, 2, 24, 1),
    # the ping-pong whose workgroups stream their tiles' stages (variant 3):
    # items crossing experts of different row counts, one-stage and ragged
    # K, round-robin and chiplet walks
    ("ps_ragged", [1, 255, 0, 300, 17], 300, 192, 3, None, None),
    ("ps_one_workgroup_one_stage", [300, 5, 0, 260], 260, 64, 3, 1, 0),
    ("ps_one_workgroup_many_experts", [300, 0, 1, 257, 600, 0, 40], 520, 200, 3, 1, 0),
    ("ps_grid3_ragged_k", [300, 70], 260, 520, 3, 3, None),
    ("ps_grid7_two_stages", [700, 3, 0, 513], 300, 128, 3, 7, 1),
    ("ps_grid24_xcd", [513, 0, 257], 530, 128, 3, 24, 1),
    ("single_expert", [300], 200, 264, None, None, None),
]


@pytest.mark.parametrize("name,sizes,N,K,variant,grid,xcd", CASES, ids=[c[0] for c in CASES])
def test_grouped_parity(hkg, name, sizes, N, K, variant, grid, xcd):
    _say(name, sizes, N, K, variant, grid, xcd)
    A, B, offs = workloads.make_grouped_inputs(sizes, N, K, seed=len(name) + K)
    C = run(hkg, A, B, offs, variant, grid, xcd)
    check(C, A, B, offs)


def last_round(sizes, N, tile_m, tile_n, grid):
    """(tiles, tiles in the last round, experts holding a tile of it) of the
    grouped tile list: experts in order, ceil(rows / tile_m) x ceil(N / tile_n)
    tiles each."""
    per = [-(-int(r) // tile_m) * -(-N // tile_n) for r in sizes]
    total = sum(per)
    rem = total % grid
    ends = np.cumsum(per)
    experts = [g for g in range(len(sizes)) if per[g] and ends[g] > total - rem]
    return total, rem, experts


# name, sizes, N, K, variant, grid, xcd: each with a last round of at most
# half the grid, so its tiles are split into two halves of K.
SPLIT_CASES = [
    # 20 tiles on 8 workgroups: two whole rounds (chiplet walk), 4 tiles split
    # in 8 halves; 5 stages of K (halves of 3 and 2)
    ("pp_whole_rounds_then_split", [1000, 300, 500, 260], 512, 320, 2, 8, 1),
    # every tile in the split round; ragged K (halves of 2 and 2 stages, the
    # last one partial)
    ("pp_all_split_ragged_k", [300, 0, 17, 260], 300, 200, 2, 24, 0),
    # two stages: one each
    ("pp_two_stages", [513, 0, 257], 530, 128, 2, 32, 1),
    ("v128_split", [129, 0, 0, 511, 64], 270, 200, 1, 48, 1),
    ("v256_ring_split", [300, 5, 0, 260], 260, 320, 0, 8, 0),
    # the streaming ping-pong: its unit is the last item of a workgroup's
    # stream (after whole tiles, or alone), halves of 3 and 2, 2 and 2 (the
    # last partial), 1 and 1 stages
    ("ps_whole_rounds_then_split", [1000, 300, 500, 260], 512, 320, 3, 8, 1),
    ("ps_split_after_round", [700, 3, 0, 513, 90], 300, 320, 3, 12, 0),
    ("ps_all_split_ragged_k", [300, 0, 17, 260], 300, 200, 3, 24, 0),
    ("ps_two_stages", [513, 0, 257], 530, 128, 3, 32, 1),
]


@pytest.mark.parametrize("name,sizes,N,K,variant,grid,xcd", SPLIT_CASES, ids=[c[0] for c in SPLIT_CASES])
def test_grouped_last_round_split(hkg, name, sizes, N, K, variant, grid, xcd):
    from tile_level_dense_amd import build as hkg_build
    bm, bn = hkg_build.tile_configs(grouped=True)[variant][:2]
    total, rem, _ = last_round(sizes, N, bm, bn, grid)
    assert 0 < rem and 2 * rem <= grid, (total, rem)
    _say(name, sizes, N, K, variant, grid, xcd, "tiles", total, "split", rem)
    A, B, offs = workloads.make_grouped_inputs(sizes, N, K, seed=len(name) + K)
    C2 = run(hkg, A, B, offs, variant, grid, xcd, split=2)
    check(C2, A, B, offs)
    assert np.array_equal(run(hkg, A, B, offs, variant, grid, xcd, split=2), C2), "split run not deterministic"
    C1 = run(hkg, A, B, offs, variant, grid, xcd, split=1)
    check(C1, A, B, offs)


def test_grouped_split_with_one_stage_is_whole(hkg):
    # K of one stage: split_k 2 in the plan leaves every tile whole, so the
    # output equals the unsplit run's bit for bit.
    sizes = [300, 0, 17, 260]
    assert last_round(sizes, 300, 256, 256, 24)[1] == 10
    A, B, offs = workloads.make_grouped_inputs(sizes, 300, 64, seed=12)
    for variant in (2, 3):
        C2 = run(hkg, A, B, offs, variant, 24, 0, split=2)
        check(C2, A, B, offs)
        assert np.array_equal(C2, run(hkg, A, B, offs, variant, 24, 0, split=1))


@pytest.mark.parametrize("variant", [2, 3])
@pytest.mark.parametrize("epi", ["bias", "bias_gelu"])
def test_grouped_split_epilogue(hkg, epi, variant):
    sizes, N, K = [1000, 300, 500, 260], 512, 320
    assert last_round(sizes, N, 256, 256, 8)[1] == 4
    A, B, offs = workloads.make_grouped_inputs(sizes, N, K, seed=31)
    rng = np.random.default_rng(6)
    bias = workloads.f32_to_bf16_bits(rng.normal(0.0, 2.0, size=(4, N)).astype(np.float32))
    C = run(hkg, A, B, offs, variant, 8, 1, bias=bias, epi=epi, split=2)
    check(C, A, B, offs, bias=bias, epi=epi)


# The two 256 x 256 ping-pong variants (one tile at a time, and tiles streamed
# stage after stage) multiply every tile in the same order and split a last
# round at the same stage, so their outputs are identical bit for bit.
@pytest.mark.parametrize("sizes,N,K,grid,xcd", [
    ([1000, 300, 500, 260], 512, 320, 8, 1),
    ([700, 3, 0, 513, 90], 300, 320, 12, 0),
    ([1, 255, 0, 300, 17, 0, 1200], 700, 136, 16, 1),
])
def test_grouped_streamed_equals_one_tile(hkg, sizes, N, K, grid, xcd):
    A, B, offs = workloads.make_grouped_inputs(sizes, N, K, seed=N + K)
    for split in (1, 2):
        C2 = run(hkg, A, B, offs, 2, grid, xcd, split=split)
        C3 = run(hkg, A, B, offs, 3, grid, xcd, split=split)
        assert np.array_equal(C2, C3), ("split", split)
    check(C3, A, B, offs)


def test_grouped_many_experts(hkg):
    # 150 experts (three steps of the 64-expert walk), a third of them empty.
    rng = np.random.default_rng(40)
    sizes = rng.integers(0, 40, size=150)
    sizes[rng.random(150) < 0.33] = 0
    _say("many experts", int(sizes.sum()))
    A, B, offs = workloads.make_grouped_inputs(sizes, 72, 64, seed=41)
    for variant, grid in ((1, None), (0, 5), (2, 5), (3, 5)):
        C = run(hkg, A, B, offs, variant, grid)
        check(C, A, B, offs)


def test_grouped_rows_past_last_expert_untouched(hkg):
    A, B, offs = workloads.make_grouped_inputs([40, 0, 50], 64, 64, seed=3)
    M = A.shape[0]
    A = np.concatenate([A, A[:30]])              # 30 more rows that belong to no expert
    C = run(hkg, A, B, offs)
    assert C.shape[0] == M + 30
    check(C, A, B, offs)


def test_grouped_offsets_are_clamped(hkg):
    # An offset past M is read as M: expert 1 gets rows [100, 300).
    A, B, offs = workloads.make_grouped_inputs([100, 200], 64, 128, seed=9)
    C = run(hkg, A, B, np.array([100, 5000], np.int32))
    check(C, A, B, offs)


@pytest.mark.parametrize("epi", ["bias", "bias_relu", "bias_silu", "bias_gelu"])
def test_grouped_epilogue(hkg, epi):
    _say("epilogue", epi)
    A, B, offs = workloads.make_grouped_inputs([70, 0, 130, 3], 200, 256, seed=len(epi))
    rng = np.random.default_rng(5)
    bias = workloads.f32_to_bf16_bits(rng.normal(0.0, 2.0, size=(4, 200)).astype(np.float32))
    for variant in (0, 1, 2, 3):
        C = run(hkg, A, B, offs, variant, bias=bias, epi=epi)
        check(C, A, B, offs, bias=bias, epi=epi)


@pytest.mark.parametrize("name", ["moe_uniform_8x1024_4096x4096", "moe_ragged_16_8192_4096x4096"])
def test_grouped_workloads_rows(hkg, name):
    # The MoE workloads in the planner's launch; oracle rows across expert
    # boundaries (and the first and last rows), every column.
    _say("workload", name)
    A, B, offs = workloads.grouped_workload_inputs(name)
    C = run(hkg, A, B, offs)
    bounds = sorted(set(int(o) for o in offs))
    picks = [(0, 4)] + [(max(0, b - 3), min(int(offs[-1]), b + 3)) for b in bounds[:-1]] + \
            [(int(offs[-1]) - 4, int(offs[-1]))]
    # every row of the experts whose tiles fall in the last round (split over
    # K when it fills at most half the grid)
    p = hkg.grouped_plan(len(offs), A.shape[0], B.shape[1], A.shape[1])
    sizes = np.diff(np.concatenate([[0], offs]))
    total, rem, experts = last_round(sizes, B.shape[1], p.tile_m, p.tile_n, p.grid_x)
    _say(name, "tiles", total, "last round", rem, "experts", experts)
    for g in experts:
        picks.append((int(offs[g - 1]) if g else 0, int(offs[g])))
    for r0, r1 in picks:
        if r1 > r0:
            check(C, A, B, offs, rows=(r0, r1))
    assert np.all(C[: int(offs[-1])] != SENTINEL)
