"""Host-side tests of the C-ABI library (no GPU needed).

The library must load and export every function include/hkg.h declares,
the ctypes mirror of hkg_plan_t must match the C layout, plans must follow
the documented selection rules, and every argument error must come back as
its status code before any device work.  The build must refuse kernels that
spill registers to scratch.
"""
import ctypes
import os
import re
import shutil
import subprocess
import tempfile

import pytest

import tile_level_dense_amd as hkg
from tile_level_dense_amd import build as hkg_build

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "hkg.h")


def _no_gpu():
    try:
        import torch
        return torch.cuda.device_count() == 0
    except Exception:
        return True


@pytest.fixture(scope="module")
def lib():
    return hkg.lib()


def _declared_functions():
    text = open(HEADER).read()
    return sorted(set(re.findall(r"^\s*(?:const\s+)?[A-Za-z_][A-Za-z0-9_]*\**\s+\**(hkg_[a-z0-9_]+)\s*\(",
                                 text, re.M)))


def test_header_declares_the_abi():
    names = _declared_functions()
    assert names == sorted(hkg.EXPORTED_SYMBOLS), names


def test_library_exports_every_declared_symbol(lib):
    for name in _declared_functions():
        assert hasattr(lib, name), name
    nm = shutil.which("nm")
    if nm:
        out = subprocess.run([nm, "-D", "--defined-only", hkg.library_path()], stdout=subprocess.PIPE,
                             text=True, check=True).stdout
        exported = set(re.findall(r"\bT (hkg_[a-z0-9_]+)", out))
        assert set(_declared_functions()) <= exported


@pytest.mark.skipif(shutil.which("gcc") is None, reason="gcc not available")
def test_plan_struct_layout_matches_header():
    fields = [f for f, _ in hkg.Plan._fields_]
    prog = ['#include <stdio.h>', '#include <stddef.h>', '#include "hkg.h"', 'int main(void){',
            'printf("size %zu\\n", sizeof(hkg_plan_t));']
    for f in fields:
        prog.append('printf("%s %%zu\\n", offsetof(hkg_plan_t, %s));' % (f, f))
    prog.append("return 0;}")
    tmp = tempfile.mkdtemp()
    try:
        src = os.path.join(tmp, "layout.c")
        exe = os.path.join(tmp, "layout")
        open(src, "w").write("\n".join(prog))
        subprocess.check_call(["gcc", "-std=c11", "-I" + os.path.join(ROOT, "include"), src, "-o", exe])
        out = subprocess.run([exe], stdout=subprocess.PIPE, text=True, check=True).stdout.split("\n")
        got = dict(ln.split() for ln in out if ln.strip())
        assert int(got["size"]) == ctypes.sizeof(hkg.Plan)
        for f in fields:
            assert int(got[f]) == getattr(hkg.Plan, f).offset, f
    finally:
        shutil.rmtree(tmp, ignore_errors=True)


def test_abi_version(lib):
    assert lib.hkg_abi_version() == hkg.HKG_ABI_VERSION


def test_status_strings(lib):
    for code in list(hkg.STATUS) + [-99]:
        s = hkg.hkg_status_string(code)
        assert isinstance(s, str) and s


WORKLOAD_PLANS = {
    (256, 256, 256): ("TILE", "tile_64x64x64_s4"),
    (16, 4096, 4096): ("SKINNY", "skinny_m16"),
    (128, 12288, 4096): ("TILE", "tile_64x96x64_s4"),
    (4096, 4096, 12288): ("TILE", "tile_256x256x64_"),
    (8192, 8192, 8192): ("TILE", "tile_256x256x64_"),
}


@pytest.mark.parametrize("shape", list(WORKLOAD_PLANS))
def test_plan_for_workloads(shape):
    M, N, K = shape
    p = hkg.plan(M, N, K)
    kind, name = WORKLOAD_PLANS[shape]
    assert hkg.KERNEL_NAMES[p.kernel_id] == kind
    assert p.kernel_name.decode().startswith(name)
    assert p.flops == 2.0 * M * N * K
    assert p.algorithmic_bytes == 2.0 * (M * K + N * K + M * N)
    assert p.scratch_bytes == 0 and p.vgprs > 0
    assert p.M == M and p.N == N and p.K == K
    # deterministic
    q = hkg.plan(M, N, K)
    assert bytes(p) == bytes(q)


def test_plan_square_8192_geometry():
    p = hkg.plan(8192, 8192, 8192)
    assert (p.tile_m, p.tile_n, p.tile_k, p.waves) == (256, 256, 64, 8)
    # persistent ping-pong: one workgroup per compute unit, 4 tiles each
    assert p.grid_x == 256 and p.block_x == 512
    assert p.kernel_name.decode().endswith("_p6")
    assert p.xcd_window_w == 8 and p.xcd_chunk_c == 32
    # ping-pong schedule: A halves double-, B triple-buffered
    assert p.lds_bytes == (4 * 128 + 3 * 256) * 64 * 2
    assert p.workspace_bytes == 0 and p.split_k == 1


@pytest.mark.parametrize("M", [16, 9, 8, 1])
def test_plan_small_m_a_staging(M):
    # Every M <= 16 takes the 16-row cover with A staged through LDS: 8
    # waves, chunks of 4 steps, two chunk buffers of 16 rows x 256 bytes per
    # wave.
    p = hkg.plan(M, 4096, 4096)
    assert p.kernel_name.decode() == "skinny_m16_n16_w8_u4_c0_lds"
    assert p.lds_bytes >= 8 * 2 * 16 * 4 * 64


def test_plan_decode_geometry():
    p = hkg.plan(16, 4096, 4096)
    assert p.grid_x == 256 and p.split_k == 1 and p.workspace_bytes == 0


def test_plan_boundaries():
    assert hkg.KERNEL_NAMES[hkg.plan(16, 4096, 4096).kernel_id] == "SKINNY"
    assert hkg.KERNEL_NAMES[hkg.plan(17, 4096, 4096).kernel_id] == "TILE"
    assert hkg.KERNEL_NAMES[hkg.plan(16, 4112, 4096).kernel_id] == "SKINNY"    # 257 column blocks
    assert hkg.KERNEL_NAMES[hkg.plan(16, 8192, 4096).kernel_id] == "SKINNY"    # 512: two rounds
    assert hkg.KERNEL_NAMES[hkg.plan(16, 8208, 4096).kernel_id] == "TILE"      # 513 column blocks
    assert hkg.KERNEL_NAMES[hkg.plan(32, 4096, 4096).kernel_id] == "TILE"
    p = hkg.plan(128, 12288, 4096)       # 256 tiles of 64 x 96: one per CU, unsplit
    assert hkg.KERNEL_NAMES[p.kernel_id] == "TILE" and (p.tile_m, p.tile_n, p.split_k, p.grid_x) == (64, 96, 1, 256)
    assert hkg.KERNEL_NAMES[hkg.plan(512, 512, 100).kernel_id] == "GENERIC"     # K % 8
    assert hkg.KERNEL_NAMES[hkg.plan(512, 512, 0).kernel_id] == "ZERO"
    assert hkg.KERNEL_NAMES[hkg.plan(0, 512, 64).kernel_id] == "NONE"
    assert hkg.KERNEL_NAMES[hkg.plan(5, 0, 64).kernel_id] == "NONE"
    assert hkg.KERNEL_NAMES[hkg.plan(1, 1, 8).kernel_id] == "SKINNY"
    # small N at decode M: split-K across workgroups with a workspace
    p = hkg.plan(16, 256, 8192)
    assert p.split_k > 1 and p.workspace_bytes == p.split_k * 16 * 256 * 4
    # streaming tiles: the fewest splits that keep one workgroup per CU
    p = hkg.plan(256, 4096, 4096)        # 128 x 128 needs split 4, 64 x 64 fills unsplit
    assert (p.tile_m, p.tile_n, p.split_k, p.grid_x) == (64, 64, 1, 256)
    p = hkg.plan(512, 4096, 4096)        # 128 x 128 needs split 2, 128 x 64 fills unsplit
    assert (p.tile_m, p.tile_n, p.split_k, p.grid_x) == (128, 64, 1, 256)
    p = hkg.plan(256, 12288, 4096)       # unsplit: the smallest tile filling one round (128 x 128: 192 tiles)
    assert (p.tile_m, p.tile_n, p.split_k, p.grid_x) == (128, 96, 1, 256)
    p = hkg.plan(256, 16384, 4096)       # 128 x 96 would take two rounds: 128 x 128 fills one
    assert (p.tile_m, p.tile_n, p.split_k, p.grid_x) == (128, 128, 1, 256)
    # tile grid under one workgroup per CU: split-K across workgroups,
    # at least 8 k-tiles per split; the 128-row tile is skipped at M = 64
    # (half its rows would be padding)
    p = hkg.plan(64, 4096, 4096)
    assert (p.tile_m, p.tile_n) == (64, 64) and p.grid_x == 64
    assert p.split_k == 4 and p.grid_y == 4 and p.workspace_bytes == 4 * 64 * 4096 * 4
    p = hkg.plan(64, 4096, 1024)
    assert p.split_k == 2
    p = hkg.plan(64, 4096, 512)
    assert p.split_k == 1
    # equal splits: the smallest tile whose grid fits one workgroup per CU
    for shape in [(256, 256, 256), (512, 512, 512), (1024, 1024, 1024)]:
        p = hkg.plan(*shape)
        assert (p.tile_m, p.tile_n, p.split_k) == (64, 64, 1), shape
    p = hkg.plan(64, 4096, 128)
    assert p.split_k == 1 and p.workspace_bytes == 0
    # compute-bound ladder: 256 x 256 from 3/4 of the CUs on; then one round
    # of k-interleaved 128 x 256 tiles (160 to 256 of them, K >= 1024); the
    # two-stage 128 x 128 tile while its tiles outnumber the CUs; one round
    # of k-interleaved 128 x 128 tiles (224 to 256, K >= 1024)
    for shape, name in [((3072, 4096, 1024), "tile_256x256x64_s2"),
                        ((2048, 2048, 1024), "tile_128x128x64_s3_w2x2_p7"),
                        ((4096, 2048, 1024), "tile_128x256x64_s3_w2x2_p7"),
                        ((1024, 8192, 4096), "tile_128x256x64_s3_w2x2_p7"),
                        ((1280, 4096, 4096), "tile_128x256x64_s3_w2x2_p7"),     # 160 tiles
                        ((1152, 4096, 4096), "tile_128x128x64_s2_w2x2_p2"),     # 144 tiles of 128 x 256
                        ((2560, 4096, 1024), "tile_128x128x64_s2_w2x2_p2"),     # 320 tiles of 128 x 256
                        ((2048, 4096, 256), "tile_128x128x64_s2_w2x2_p2"),      # K under 1024
                        ((150, 40960, 4096), "tile_128x128x64_s2_w2x2_p2"),     # rows 41% padding
                        ((256, 16384, 4096), "tile_128x128x64_s5_w2x2_p7"),     # five stages from K = 4096
                        ((1024, 3584, 4096), "tile_128x128x64_s5_w2x2_p7"),     # 224 tiles
                        ((1024, 3584, 2048), "tile_128x128x64_s3_w2x2_p7"),
                        ((8192, 8192, 8192), "tile_256x256x64_s2")]:
        p = hkg.plan(*shape)
        assert hkg.KERNEL_NAMES[p.kernel_id] == "TILE" and p.split_k == 1
        assert p.kernel_name.decode().startswith(name), (shape, p)
    p = hkg.plan(1024, 4096, 4096)
    assert (p.waves, p.block_x, p.grid_x, p.lds_bytes) == (8, 512, 256, 5 * 256 * 128), p
    assert "k-interleaved" in p.reason.decode()
    # more 256 x 256 tiles than CUs with a last round of at most half the
    # device: that round split in two halves of K (one partial tile of
    # workspace per workgroup, one grid)
    for shape, split in [((4352, 4096, 4096), 2), ((6144, 4096, 4096), 2), ((4400, 4200, 136), 2),
                         ((5120, 5120, 4096), 1), ((8192, 8192, 8192), 1), ((4096, 4096, 12288), 1),
                         ((4352, 4096, 64), 1)]:
        p = hkg.plan(*shape)
        assert p.kernel_name.decode() == "tile_256x256x64_s2_w4x2_p6" and p.split_k == split, (shape, p)
        assert p.workspace_bytes == (256 * 256 * 256 * 4 if split == 2 else 0) and p.grid_y == 1, (shape, p)
        assert ("last round split" in p.reason.decode()) == (split == 2)
    p = hkg.plan(1024, 3072, 4096)          # 192 tiles of 128 x 128: the streaming 128 x 96 fills a round
    assert (p.tile_m, p.tile_n, p.grid_x) == (128, 96, 256)


@pytest.mark.parametrize("shape", [(-1, 4, 8), (4, -1, 8), (4, 4, -8), (2**31, 4, 8), (4, 4, 2**31),
                                   (2**31 - 1, 2**31 - 1, 2**31 - 1)])
def test_plan_rejects_bad_dims(shape):
    st, _ = hkg.hkg_gemm_bf16_plan(*shape)
    assert st == hkg.HKG_ERR_INVALID_ARG


def test_plan_null_out(lib):
    assert lib.hkg_gemm_bf16_plan(4, 4, 8, None) == hkg.HKG_ERR_INVALID_ARG


def test_argument_errors_precede_device_work():
    M, N, K = 64, 64, 64
    # null pointers with nonzero sizes
    assert hkg.hkg_gemm_bf16(None, 4096, 8192, M, N, K) == hkg.HKG_ERR_INVALID_ARG
    assert hkg.hkg_gemm_bf16(4096, None, 8192, M, N, K) == hkg.HKG_ERR_INVALID_ARG
    assert hkg.hkg_gemm_bf16(4096, 1 << 20, None, M, N, K) == hkg.HKG_ERR_INVALID_ARG
    # C overlapping A or B
    base = 1 << 30
    assert hkg.hkg_gemm_bf16(base, base + (1 << 20), base + 64, M, N, K) == hkg.HKG_ERR_INVALID_ARG
    assert hkg.hkg_gemm_bf16(base, base + (1 << 20), base + (1 << 20) + 128, M, N, K) == hkg.HKG_ERR_INVALID_ARG
    # negative dims
    assert hkg.hkg_gemm_bf16(base, base, base, -1, N, K) == hkg.HKG_ERR_INVALID_ARG
    # empty output: nothing to do, even with null pointers
    assert hkg.hkg_gemm_bf16(None, None, None, 0, 0, 0) == hkg.HKG_OK
    assert hkg.hkg_gemm_bf16(None, 4096, None, 0, 64, 64) == hkg.HKG_OK


def test_epilogue_errors_precede_device_work():
    M, N, K = 64, 64, 64
    A, B, C = 1 << 30, (1 << 30) + (1 << 22), (1 << 30) + (1 << 23)
    bias = (1 << 30) + (1 << 24)
    # unknown codes
    for code in (-1, 5, 99):
        assert hkg.hkg_gemm_bf16_epilogue(A, B, bias, C, M, N, K, code) == hkg.HKG_ERR_INVALID_ARG
    # a bias is needed for every code but none
    for code in (1, 2, 3, 4):
        assert hkg.hkg_gemm_bf16_epilogue(A, B, None, C, M, N, K, code) == hkg.HKG_ERR_INVALID_ARG
    # bias overlapping C, bias at an odd address
    assert hkg.hkg_gemm_bf16_epilogue(A, B, C + 128, C, M, N, K, 1) == hkg.HKG_ERR_INVALID_ARG
    assert hkg.hkg_gemm_bf16_epilogue(A, B, bias + 1, C, M, N, K, 1) == hkg.HKG_ERR_MISALIGNED
    # empty output: nothing to do, any bias
    assert hkg.hkg_gemm_bf16_epilogue(None, 4096, None, None, 0, 8, 8, 4) == hkg.HKG_OK
    # the same checks on the plan path
    p = hkg.plan(M, N, K)
    assert hkg.hkg_gemm_bf16_run_plan_epilogue(p, A, B, None, C, M, N, K, 2) == hkg.HKG_ERR_INVALID_ARG
    assert hkg.hkg_gemm_bf16_run_plan_epilogue(p, A, B, bias, C, M, N, K, 7) == hkg.HKG_ERR_INVALID_ARG
    assert hkg.EPILOGUES == {"none": 0, "bias": 1, "bias_relu": 2, "bias_silu": 3, "bias_gelu": 4}


@pytest.mark.skipif(not _no_gpu(), reason="a GPU is present")
def test_epilogue_calls_report_no_device():
    M, N, K = 64, 64, 64
    A, B, C = 1 << 30, (1 << 30) + (1 << 22), (1 << 30) + (1 << 23)
    bias = (1 << 30) + (1 << 24)
    assert hkg.hkg_gemm_bf16_epilogue(A, B, bias, C, M, N, K, 3) == hkg.HKG_ERR_NO_DEVICE
    assert hkg.hkg_gemm_bf16_epilogue(A, B, None, C, M, N, K, 0) == hkg.HKG_ERR_NO_DEVICE


def test_run_plan_errors_precede_device_work():
    M, N, K = 512, 512, 512
    p = hkg.plan(M, N, K)
    A, B, C = 1 << 30, (1 << 30) + (1 << 22), (1 << 30) + (1 << 23)
    assert hkg.hkg_gemm_bf16_run_plan(p, A, B, C, M + 1, N, K) == hkg.HKG_ERR_INVALID_ARG
    q = hkg.Plan.from_buffer_copy(p)
    q.variant = 99
    assert hkg.hkg_gemm_bf16_run_plan(q, A, B, C, M, N, K) == hkg.HKG_ERR_UNSUPPORTED
    q = hkg.Plan.from_buffer_copy(p)
    q.split_k = 17           # tile split range is 1..16
    assert hkg.hkg_gemm_bf16_run_plan(q, A, B, C, M, N, K) == hkg.HKG_ERR_UNSUPPORTED
    q.split_k = 0
    assert hkg.hkg_gemm_bf16_run_plan(q, A, B, C, M, N, K) == hkg.HKG_ERR_UNSUPPORTED
    # split-K exists only in tile variants with at most 16 accumulator
    # blocks per wave (256 x 256 over 8 waves has 32); the persistent
    # 256 x 256 tile takes split 2 only, meaning its last round split
    q = hkg.plan(8192, 8192, 8192)
    assert (q.tile_m, q.tile_n, q.waves) == (256, 256, 8)
    q.split_k = 3
    assert hkg.hkg_gemm_bf16_run_plan(q, 1 << 40, 2 << 40, 3 << 40, 8192, 8192, 8192) == hkg.HKG_ERR_UNSUPPORTED
    q = hkg.Plan.from_buffer_copy(p)
    q.abi_version = 7
    assert hkg.hkg_gemm_bf16_run_plan(q, A, B, C, M, N, K) == hkg.HKG_ERR_INVALID_ARG
    # a fast-kernel plan on 2-byte aligned pointers
    assert hkg.hkg_gemm_bf16_run_plan(p, A + 2, B, C, M, N, K) == hkg.HKG_ERR_MISALIGNED
    # skinny split range
    s = hkg.plan(16, 4096, 4096)
    s.split_k = 65
    assert hkg.hkg_gemm_bf16_run_plan(s, 1 << 30, 1 << 32, 1 << 33, 16, 4096, 4096) == hkg.HKG_ERR_UNSUPPORTED


@pytest.mark.skipif(not _no_gpu(), reason="checks the no-device status; a GPU is present")
def test_no_device_status():
    M, N, K = 64, 64, 64
    A, B, C = 1 << 30, (1 << 30) + (1 << 20), (1 << 30) + (1 << 21)
    assert hkg.hkg_gemm_bf16(A, B, C, M, N, K) == hkg.HKG_ERR_NO_DEVICE
    p = hkg.plan(M, N, K)
    assert hkg.hkg_gemm_bf16_run_plan(p, A, B, C, M, N, K) == hkg.HKG_ERR_NO_DEVICE


def test_build_resources_have_no_scratch():
    import json
    path = os.path.join(hkg_build.BUILD, "kernel_resources.json")
    if not os.path.exists(path):
        hkg_build.build()
    res = json.load(open(path))
    entries = res["tile"] + res["mx_tile"] + res["grouped"] + res["skinny"] + res["mx_skinny"] + [res["generic"]]
    for e in entries:
        assert e["scratch"] == 0 and e["vgpr_spill"] <= 0, e


@pytest.mark.skipif(not os.path.exists(hkg_build.HIPCC), reason="hipcc not available")
def test_build_gate_refuses_a_spilling_kernel():
    src = r'''
#include <hip/hip_runtime.h>
__global__ __launch_bounds__(1024) void spills(const float* in, float* out, int n) {
  float v[512];
#pragma unroll
  for (int i = 0; i < 512; ++i) v[i] = in[threadIdx.x * 512 + i] * (float)i;
  float s = 0.f;
  for (int r = 0; r < n; ++r)
#pragma unroll
    for (int i = 0; i < 512; ++i) s += v[(i * 7 + r) & 511] * v[i];
  out[threadIdx.x] = s;
}
'''
    tmp = tempfile.mkdtemp()
    try:
        f = os.path.join(tmp, "spill.hip")
        open(f, "w").write(src)
        p = subprocess.run([hkg_build.HIPCC, "-O3", "--offload-arch=gfx950", "-c", f, "-o",
                            os.path.join(tmp, "spill.o"), "-Rpass-analysis=kernel-resource-usage"],
                           stdout=subprocess.PIPE, stderr=subprocess.PIPE, text=True)
        assert p.returncode == 0
        res = hkg_build._parse_resources(p.stderr)
        (name, r), = res.items()
        e = hkg_build._entry(name, r)
        assert e["scratch"] > 0
        with pytest.raises(hkg_build.BuildError):
            hkg_build._gate([e])
    finally:
        shutil.rmtree(tmp, ignore_errors=True)


def _tile_order_fn(lib):
    f = lib.hkg_internal_tile_order
    f.argtypes = [ctypes.c_int32] * 5 + [ctypes.POINTER(ctypes.c_int32)] * 2
    f.restype = ctypes.c_int32
    return f


def test_tile_order_is_a_bijection(lib):
    """The kernel's workgroup -> tile order (same inline function, host build)
    must visit every tile exactly once for any grid and (W, C)."""
    f = _tile_order_fn(lib)
    tm, tn = ctypes.c_int32(), ctypes.c_int32()
    grids = [(tm_, tn_) for tm_ in range(1, 20) for tn_ in range(1, 20)] + [(32, 32), (16, 16), (57, 57), (9, 9)]
    for gm, gn in grids:
        for w in (0, 1, 2, 3, 5, 8, 16):
            for c in (0, 1, 2, 4, 7, 32):
                seen = set()
                for b in range(gm * gn):
                    assert f(b, gm, gn, w, c, ctypes.byref(tm), ctypes.byref(tn)) == 0
                    assert 0 <= tm.value < gm and 0 <= tn.value < gn
                    seen.add((tm.value, tn.value))
                assert len(seen) == gm * gn, (gm, gn, w, c)


def test_tile_order_chiplet_blocks(lib):
    """At 32 x 32 tiles with W = 8, C = 32 the 32 workgroups that one XCD
    receives first (ids x, x + 8, ..., x + 248) cover an 8 x 4 block of tiles."""
    f = _tile_order_fn(lib)
    tm, tn = ctypes.c_int32(), ctypes.c_int32()
    for xcd in range(8):
        tiles = set()
        for r in range(32):
            f(xcd + 8 * r, 32, 32, 8, 32, ctypes.byref(tm), ctypes.byref(tn))
            tiles.add((tm.value, tn.value))
        rows = {t[0] for t in tiles}
        cols = {t[1] for t in tiles}
        assert len(tiles) == 32 and len(rows) == 8 and len(cols) == 4
        assert cols == set(range(4 * xcd, 4 * xcd + 4))


# ------------------------------------------------------------------ MXFP8
@pytest.mark.parametrize("shape,kernel,variant,split", [
    ((8192, 8192, 8192), "MX_TILE", 0, 1),     # 32 x 32 ping-pong tiles fill the device
    ((4096, 4096, 12288), "MX_TILE", 0, 1),
    ((32, 4096, 4096), "MX_SKINNY", 3, 1),     # decode: 256 column blocks of 16 already fill it
    ((16, 2048, 4096), "MX_SKINNY", 2, 2),     # 128 column blocks: split 2 (at least 2 steps per wave)
    # A through LDS (variants 2, 3) once M fills more than half of the
    # cover: 16-row cover up to 16 rows, 32-row cover above
    ((8, 4096, 4096), "MX_SKINNY", 0, 1),
    ((9, 4096, 4096), "MX_SKINNY", 2, 1),
    ((17, 4096, 4096), "MX_SKINNY", 3, 1),
    ((33, 4096, 4096), "MX_TILE", 1, 8),       # above 32 rows: 32 tiles of 128 x 128, split to fill
    ((128, 12288, 4096), "MX_TILE", 1, 3),
    ((256, 256, 256), "MX_TILE", 1, 1),        # 4 tiles; K / 128 / 4 = 0 splits -> 1
    ((1000, 1000, 384), "MX_TILE", 1, 1),
])
def test_mx_plan_selection(shape, kernel, variant, split):
    p = hkg.mx_plan(*shape)
    M, N, K = shape
    assert hkg.KERNEL_NAMES[p.kernel_id] == kernel and p.variant == variant and p.split_k == split, p
    assert p.tile_k == 128 and p.flops == 2.0 * M * N * K
    assert p.algorithmic_bytes == M * K + N * K + (M + N) * (K // 32) + 2 * M * N
    assert p.workspace_bytes == (split * M * N * 4 if split > 1 else 0)
    assert p.vgprs > 0 and p.scratch_bytes == 0


def test_mx_plan_edge_shapes():
    assert hkg.hkg_gemm_mxfp8_plan(64, 64, 100)[0] == hkg.HKG_ERR_INVALID_ARG      # K % 128
    assert hkg.hkg_gemm_mxfp8_plan(-1, 64, 128)[0] == hkg.HKG_ERR_INVALID_ARG
    st, p = hkg.hkg_gemm_mxfp8_plan(0, 64, 128)
    assert st == hkg.HKG_OK and p.kernel_id == hkg.HKG_KERNEL_NONE
    st, p = hkg.hkg_gemm_mxfp8_plan(5, 7, 0)
    assert st == hkg.HKG_OK and p.kernel_id == hkg.HKG_KERNEL_ZERO
    # K beyond the 32-bit offsets of one 256-row tile
    assert hkg.hkg_gemm_mxfp8_plan(64, 64, 8388608)[0] == hkg.HKG_ERR_UNSUPPORTED


def test_mx_packed_scale_bytes():
    assert hkg.hkg_mx_packed_scales_bytes(1, 128) == 64 * 4
    assert hkg.hkg_mx_packed_scales_bytes(64, 128) == 64 * 4
    assert hkg.hkg_mx_packed_scales_bytes(65, 256) == 128 * 8
    assert hkg.hkg_mx_packed_scales_bytes(0, 256) == 0
    assert hkg.hkg_mx_packed_scales_bytes(10, 96) == -1
    assert hkg.hkg_mx_packed_scales_bytes(-1, 128) == -1


def test_mx_argument_errors_precede_device_work():
    M, N, K = 64, 64, 256
    A, SA, B, SB, C = [(1 << 30) + i * (1 << 22) for i in range(5)]
    bias = (1 << 30) + 5 * (1 << 22)
    f = hkg.hkg_gemm_mxfp8
    assert f(A, SA, B, SB, None, C, M, N, 200) == hkg.HKG_ERR_INVALID_ARG          # K % 128
    assert f(None, SA, B, SB, None, C, M, N, K) == hkg.HKG_ERR_INVALID_ARG
    assert f(A, None, B, SB, None, C, M, N, K) == hkg.HKG_ERR_INVALID_ARG
    assert f(A, SA, B, None, None, C, M, N, K) == hkg.HKG_ERR_INVALID_ARG
    assert f(A, SA, B, SB, None, SA + 16, M, N, K) == hkg.HKG_ERR_INVALID_ARG       # C overlaps SA
    assert f(A, SA, B, SB, None, C, M, N, K, 3) == hkg.HKG_ERR_INVALID_ARG          # epilogue without bias
    assert f(A, SA, B, SB, bias + 1, C, M, N, K, 1) == hkg.HKG_ERR_MISALIGNED
    assert f(A + 8, SA, B, SB, None, C, M, N, K) == hkg.HKG_ERR_MISALIGNED
    assert f(None, None, B, SB, None, None, 0, N, K) == hkg.HKG_OK                  # empty output
    g = hkg.hkg_gemm_mxfp8_prepacked
    assert g(A, SA + 2, B, SB, None, C, M, N, K) == hkg.HKG_ERR_MISALIGNED           # packed scales: 4 bytes
    assert g(A, SA, B, SB, None, C + 8, M, N, K) == hkg.HKG_ERR_MISALIGNED
    assert hkg.hkg_mx_pack_scales(SA, SB, M, 100) == hkg.HKG_ERR_INVALID_ARG
    assert hkg.hkg_mx_pack_scales(SA, SA + 64, M, K) == hkg.HKG_ERR_INVALID_ARG      # overlap
    assert hkg.hkg_mx_pack_scales(SA, SB + 2, M, K) == hkg.HKG_ERR_MISALIGNED
    assert hkg.hkg_mx_pack_scales(None, None, 0, K) == hkg.HKG_OK


def test_mx_run_plan_checks():
    M, N, K = 512, 512, 512
    A, PA, B, PB, C = [(1 << 30) + i * (1 << 22) for i in range(5)]
    p = hkg.mx_plan(M, N, K)
    r = hkg.hkg_gemm_mxfp8_run_plan
    assert r(p, A, PA, B, PB, None, C, M + 1, N, K) == hkg.HKG_ERR_INVALID_ARG
    q = hkg.Plan.from_buffer_copy(p)
    q.variant = 7
    assert r(q, A, PA, B, PB, None, C, M, N, K) == hkg.HKG_ERR_UNSUPPORTED
    # a bf16 plan is not an MXFP8 plan, and the other way round
    assert r(hkg.plan(M, N, K), A, PA, B, PB, None, C, M, N, K) == hkg.HKG_ERR_UNSUPPORTED
    assert hkg.hkg_gemm_bf16_run_plan(p, A, B, C, M, N, K) == hkg.HKG_ERR_UNSUPPORTED
    # split-K only in the 128 x 128 variant
    q = hkg.mx_plan(8192, 8192, 8192)
    q.split_k = 2
    assert r(q, 1 << 40, 2 << 40, 3 << 40, 4 << 40, None, 5 << 40, 8192, 8192, 8192) == hkg.HKG_ERR_UNSUPPORTED


@pytest.mark.skipif(not _no_gpu(), reason="checks the no-device status; a GPU is present")
def test_mx_no_device_status():
    M, N, K = 64, 64, 256
    A, SA, B, SB, C = [(1 << 30) + i * (1 << 22) for i in range(5)]
    assert hkg.hkg_gemm_mxfp8(A, SA, B, SB, None, C, M, N, K) == hkg.HKG_ERR_NO_DEVICE
    assert hkg.hkg_mx_pack_scales(SA, SB, M, K) == hkg.HKG_ERR_NO_DEVICE


# ------------------------------------------------------------ grouped GEMM
@pytest.mark.parametrize("shape,variant,grid", [
    ((8, 8192, 4096, 4096), 3, 256),      # experts of 1024 rows: 256 x 256 ping-pong, one workgroup per CU
    ((16, 8192, 4096, 4096), 3, 256),
    ((64, 4096, 2048, 1024), 1, 512),     # 64 rows per expert: 128 x 128, two per CU
    ((4, 256, 256, 256), 1, 12),          # grid capped at the most tiles the experts can have
])
def test_grouped_plan_selection(shape, variant, grid):
    G, M, N, K = shape
    p = hkg.grouped_plan(*shape)
    assert p.kernel_id == hkg.HKG_KERNEL_GROUPED and p.variant == variant and p.grid_x == grid, p
    # a last round filling at most half the grid is split over K (two halves)
    assert p.split_k == 2 and p.xcd_chunk_c == 1
    assert p.workspace_bytes == grid * p.tile_m * p.tile_n * 4
    assert p.algorithmic_bytes == 2 * (M * K + G * N * K + M * N)
    assert p.vgprs > 0 and p.scratch_bytes == 0
    assert p.lds_bytes == (160 * 1024 if variant == 3 else 2 * (p.tile_m + p.tile_n) * 128)
    assert p.kernel_name.decode() == ("grouped_256x256x64_s2_w4x2_p6" if variant == 3 else "grouped_128x128x64_s2_w2x2_p2")


def test_grouped_plan_edges():
    for shape in ((0, 64, 64, 64), (4, 0, 64, 64), (4, 64, 0, 64)):
        st, p = hkg.hkg_grouped_gemm_bf16_plan(*shape)
        assert st == hkg.HKG_OK and p.kernel_id == hkg.HKG_KERNEL_NONE
    # one stage of K: nothing to split
    p = hkg.grouped_plan(4, 512, 256, 64)
    assert p.split_k == 1 and p.workspace_bytes == 0
    assert hkg.hkg_grouped_gemm_bf16_plan(-1, 64, 64, 64)[0] == hkg.HKG_ERR_INVALID_ARG
    assert hkg.hkg_grouped_gemm_bf16_plan(4, 64, 64, 100)[0] == hkg.HKG_ERR_UNSUPPORTED     # K % 8


def test_grouped_argument_errors_precede_device_work():
    G, M, N, K = 4, 256, 128, 64
    A, B, offs, C, bias = [(1 << 30) + i * (1 << 24) for i in range(5)]
    f = hkg.hkg_grouped_gemm_bf16
    assert f(None, B, offs, None, C, G, M, N, K) == hkg.HKG_ERR_INVALID_ARG
    assert f(A, B, None, None, C, G, M, N, K) == hkg.HKG_ERR_INVALID_ARG
    assert f(A, B, offs, None, offs, G, M, N, K) == hkg.HKG_ERR_INVALID_ARG          # C overlaps offs
    assert f(A, B, offs, None, C, G, M, N, K, 2) == hkg.HKG_ERR_INVALID_ARG          # bias needed
    assert f(A, B, offs, bias + 1, C, G, M, N, K, 1) == hkg.HKG_ERR_MISALIGNED
    assert f(A + 8, B, offs, None, C, G, M, N, K) == hkg.HKG_ERR_MISALIGNED
    assert f(A, B, offs + 2, None, C, G, M, N, K) == hkg.HKG_ERR_MISALIGNED
    assert f(A, B, offs, None, C, G, M, N, K, 9) == hkg.HKG_ERR_INVALID_ARG
    assert f(None, None, None, None, None, 0, 0, N, K) == hkg.HKG_OK
    p = hkg.grouped_plan(G, M, N, K)
    r = hkg.hkg_grouped_gemm_bf16_run_plan
    assert r(p, A, B, offs, None, C, G, M + 1, N, K) == hkg.HKG_ERR_INVALID_ARG
    q = hkg.Plan.from_buffer_copy(p)
    q.variant = 5
    assert r(q, A, B, offs, None, C, G, M, N, K) == hkg.HKG_ERR_UNSUPPORTED
    assert r(hkg.plan(M, N, K), A, B, offs, None, C, G, M, N, K) == hkg.HKG_ERR_UNSUPPORTED
    q = hkg.Plan.from_buffer_copy(p)
    q.grid_x = 0
    assert r(q, A, B, offs, None, C, G, M, N, K) == hkg.HKG_ERR_UNSUPPORTED
    q = hkg.Plan.from_buffer_copy(p)
    q.split_k = 3
    assert r(q, A, B, offs, None, C, G, M, N, K) == hkg.HKG_ERR_UNSUPPORTED


@pytest.mark.skipif(not _no_gpu(), reason="checks the no-device status; a GPU is present")
def test_grouped_no_device_status():
    G, M, N, K = 4, 256, 128, 64
    A, B, offs, C = [(1 << 30) + i * (1 << 24) for i in range(4)]
    assert hkg.hkg_grouped_gemm_bf16(A, B, offs, None, C, G, M, N, K) == hkg.HKG_ERR_NO_DEVICE


# ------------------------------------------------------------------ layouts
def test_layout_argument_errors_precede_device_work():
    M, N, K = 64, 48, 32
    A, B, C = [(1 << 30) + i * (1 << 24) for i in range(3)]
    f = hkg.hkg_gemm_bf16_ex
    assert f(A, K, 2, B, K, 0, None, C, N, M, N, K) == hkg.HKG_ERR_INVALID_ARG      # unknown layout
    assert f(A, K - 1, 0, B, K, 0, None, C, N, M, N, K) == hkg.HKG_ERR_INVALID_ARG  # lda < K (row)
    assert f(A, M - 1, 1, B, K, 0, None, C, N, M, N, K) == hkg.HKG_ERR_INVALID_ARG  # lda < M (column)
    assert f(A, K, 0, B, N - 1, 1, None, C, N, M, N, K) == hkg.HKG_ERR_INVALID_ARG  # ldb < N (column)
    assert f(A, K, 0, B, K, 0, None, C, N - 1, M, N, K) == hkg.HKG_ERR_INVALID_ARG  # ldc < N
    assert f(None, K, 0, B, K, 0, None, C, N, M, N, K) == hkg.HKG_ERR_INVALID_ARG
    # C with a large ldc reaches into B
    assert f(A, K, 0, C + 2 * 1000 * 10, K, 0, None, C, 1000, M, N, K) == hkg.HKG_ERR_INVALID_ARG
    assert f(A, K, 0, B, K, 0, None, C, N, M, N, K, 2) == hkg.HKG_ERR_INVALID_ARG   # epilogue without bias
    assert f(None, K, 0, B, K, 0, None, None, N, 0, N, K) == hkg.HKG_OK               # empty output
    p = hkg.hkg_pack_bf16
    assert p(A, K - 1, 0, B, M, K) == hkg.HKG_ERR_INVALID_ARG
    assert p(A, M, 1, A + 16, M, K) == hkg.HKG_ERR_INVALID_ARG                        # overlap
    assert p(A, K, 3, B, M, K) == hkg.HKG_ERR_INVALID_ARG
    assert p(None, K, 0, None, 0, K) == hkg.HKG_OK


@pytest.mark.skipif(not _no_gpu(), reason="checks the no-device status; a GPU is present")
def test_layout_no_device_status():
    M, N, K = 64, 48, 32
    A, B, C = [(1 << 30) + i * (1 << 24) for i in range(3)]
    assert hkg.hkg_gemm_bf16_ex(A, M, 1, B, N, 1, None, C, N, M, N, K) == hkg.HKG_ERR_NO_DEVICE
    assert hkg.hkg_pack_bf16(A, M, 1, B, M, K) == hkg.HKG_ERR_NO_DEVICE
