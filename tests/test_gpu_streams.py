"""Library workspaces per (device, stream): calls on two streams at once, and
workspaces under graph capture.

Each stream has its own split-K partials and arrival counters, packed MXFP8
scales and row-layout copies (include/hkg.h, "Thread safety").  The first
test enqueues split-K, MXFP8-with-packing and column-layout calls of
different sizes on two streams, interleaved, several rounds without a host
synchronisation, and checks every output against the oracle (and each
round's outputs bit-identical to the first's).  The others check that a
workspace is never grown while its stream is being captured (the call is
refused with HKG_ERR_WORKSPACE) and that a graph captured before its stream's
workspace grew still replays correctly (the outgrown buffer is kept).
"""
import ctypes

import numpy as np
import pytest

import oracle
import workloads
from tests import gates

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


def _say(*a):
    print("[gpu-streams]", *a, flush=True)


@pytest.fixture(scope="module")
def hkg():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import tile_level_dense_amd as lib
    lib.lib()
    return lib


def dev16(bits):
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).to("cuda")


def dev8(x):
    return torch.from_numpy(np.ascontiguousarray(x, dtype=np.uint8)).to("cuda")


def host16(t):
    return t.view(torch.int16).cpu().numpy().view(np.uint16)


_E4M3 = None


def e4m3(codes):
    global _E4M3
    if _E4M3 is None:
        O = oracle.default()
        _E4M3 = np.array([O.e4m3_value(c) for c in range(256)])
    return _E4M3[np.asarray(codes, dtype=np.uint8)]


class DenseJob:
    """hkg_gemm_bf16 on a shape whose plan splits K (tile or skinny kernel)."""

    def __init__(self, hkg, M, N, K, seed):
        self.name = "dense %dx%dx%d" % (M, N, K)
        self.A, self.B = workloads.make_inputs(M, N, K, ("normal", 0.0, 1.0), ("normal", 0.0, 0.02), seed=seed)
        self.a, self.b = dev16(self.A), dev16(self.B)
        self.M, self.N = M, N
        p = hkg.plan(M, N, K)
        assert p.split_k > 1, (self.name, p.kernel_name)
        self.kernel = p.kernel_name.decode()
        self.hkg = hkg

    def out(self):
        return torch.empty((self.M, self.N), dtype=torch.bfloat16, device="cuda")

    def launch(self, c):
        self.hkg.gemm(self.a, self.b, out=c)

    def check(self, C):
        Cr, S, absS = oracle.gemm(self.A, self.B)
        return gates.compare(C, Cr, S, absS)


class MxJob:
    """hkg_gemm_mxfp8 with natural scales on the tile kernel (packs the scales
    into the stream's workspace on every call)."""

    def __init__(self, hkg, M, N, K, seed):
        self.name = "mxfp8 %dx%dx%d" % (M, N, K)
        rng = np.random.default_rng(seed)
        self.A, self.SA = workloads.mx_quantize(rng.normal(0.0, 1.0, size=(M, K)))
        self.B, self.SB = workloads.mx_quantize(rng.normal(0.0, 1.0, size=(N, K)))
        self.t = [dev8(x) for x in (self.A, self.SA, self.B, self.SB)]
        self.M, self.N, self.K = M, N, K
        p = hkg.mx_plan(M, N, K)
        assert p.kernel_id == hkg.HKG_KERNEL_MX_TILE, p.kernel_name
        self.kernel = p.kernel_name.decode()
        self.hkg = hkg

    def out(self):
        return torch.empty((self.M, self.N), dtype=torch.bfloat16, device="cuda")

    def launch(self, c):
        a, sa, b, sb = self.t
        self.hkg.gemm_mxfp8(a, sa, b, sb, out=c)

    def check(self, C):
        Cr, S, absS = oracle.mx_gemm(self.A, self.SA, self.B, self.SB)
        T = gates.mx_truncation_allowance(gates.mx_operand(self.A, self.SA, e4m3),
                                          gates.mx_operand(self.B, self.SB, e4m3))
        return gates.compare_mx(C, Cr, S, absS, T, self.K)


class LayoutJob:
    """hkg_gemm_bf16_ex with column-layout operands (transposed into the
    stream's workspace on every call)."""

    def __init__(self, hkg, M, N, K, a_col, seed):
        self.name = "layout %s%s %dx%dx%d" % ("T" if a_col else "N", "N", M, N, K)
        self.A, self.B = workloads.make_inputs(M, N, K, ("normal", 0.0, 1.0), ("normal", 0.0, 0.02), seed=seed)
        self.at = dev16(self.A.T.copy())          # stored K x M
        self.bt = dev16(self.B.T.copy())          # stored K x N
        self.a = dev16(self.A)
        self.a_col = a_col
        self.M, self.N = M, N
        self.hkg = hkg

    def out(self):
        return torch.empty((self.M, self.N), dtype=torch.bfloat16, device="cuda")

    def launch(self, c):
        self.hkg.gemm_ex(self.at.t() if self.a_col else self.a, self.bt.t(), out=c)

    def check(self, C):
        Cr, S, absS = oracle.gemm(self.A, self.B)
        return gates.compare(C, Cr, S, absS)


def test_two_streams_at_once(hkg):
    jobs1 = [DenseJob(hkg, 64, 512, 4096, 1), DenseJob(hkg, 16, 256, 8192, 2), MxJob(hkg, 100, 300, 1024, 3),
             LayoutJob(hkg, 96, 200, 512, False, 4)]
    jobs2 = [DenseJob(hkg, 96, 640, 2048, 5), DenseJob(hkg, 8, 384, 6144, 6), MxJob(hkg, 70, 260, 768, 7),
             LayoutJob(hkg, 80, 150, 384, True, 8)]
    for j in jobs1 + jobs2:
        _say(j.name, getattr(j, "kernel", ""))
    rounds = 6
    outs1 = [[j.out() for j in jobs1] for _ in range(rounds)]
    outs2 = [[j.out() for j in jobs2] for _ in range(rounds)]
    s1, s2 = torch.cuda.Stream(), torch.cuda.Stream()
    assert s1.cuda_stream != s2.cuda_stream
    torch.cuda.synchronize()
    for r in range(rounds):
        for j1, c1, j2, c2 in zip(jobs1, outs1[r], jobs2, outs2[r]):
            with torch.cuda.stream(s1):
                j1.launch(c1)
            with torch.cuda.stream(s2):
                j2.launch(c2)
    torch.cuda.synchronize()
    for jobs, outs in ((jobs1, outs1), (jobs2, outs2)):
        for i, j in enumerate(jobs):
            first = host16(outs[0][i])
            stats = j.check(first)
            _say(j.name, stats)
            for r in range(1, rounds):
                assert np.array_equal(host16(outs[r][i]), first), (j.name, "round", r)


def _new_stream():
    """A HIP stream created here (never used by the library before), wrapped
    for torch; default priority."""
    hip = ctypes.CDLL("libamdhip64.so")
    h = ctypes.c_void_p()
    assert hip.hipStreamCreateWithFlags(ctypes.byref(h), ctypes.c_uint(1)) == 0     # non-blocking
    return hip, h, torch.cuda.ExternalStream(h.value)


def test_workspace_not_grown_during_capture(hkg):
    job = DenseJob(hkg, 96, 640, 2048, 11)
    hip, h, s = _new_stream()
    try:
        c = job.out()
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        with pytest.raises(hkg.HkgError) as err:
            with torch.cuda.graph(g, stream=s):
                c.zero_()
                job.launch(c)
        assert err.value.status == hkg.HKG_ERR_WORKSPACE, str(err.value)
        _say("refused during capture:", str(err.value)[:160])
        torch.cuda.synchronize()
        # the same call outside capture allocates; then capturing it works
        with torch.cuda.stream(s):
            job.launch(c)
        torch.cuda.synchronize()
        ref = host16(c)
        job.check(ref)
        g2 = torch.cuda.CUDAGraph()
        c2 = job.out()
        with torch.cuda.graph(g2, stream=s):
            job.launch(c2)
        for r in range(3):
            c2.fill_(0)
            torch.cuda.synchronize()
            g2.replay()
            torch.cuda.synchronize()
            assert np.array_equal(host16(c2), ref), ("replay", r)
        del g, g2
    finally:
        torch.cuda.synchronize()
        hip.hipStreamDestroy(h)


def test_graph_outlives_workspace_growth(hkg):
    small = DenseJob(hkg, 32, 256, 2048, 21)
    big = DenseJob(hkg, 128, 1024, 8192, 22)
    big_plan = hkg.plan(128, 1024, 8192)
    small_plan = hkg.plan(32, 256, 2048)
    assert big_plan.workspace_bytes > 2 * small_plan.workspace_bytes
    hip, h, s = _new_stream()
    try:
        c = small.out()
        with torch.cuda.stream(s):
            small.launch(c)                       # allocates the stream's workspace
        torch.cuda.synchronize()
        ref = host16(c)
        small.check(ref)
        g = torch.cuda.CUDAGraph()
        cg = small.out()
        with torch.cuda.graph(g, stream=s):
            small.launch(cg)                      # the graph holds the small workspace
        cb = big.out()
        for r in range(3):
            cg.fill_(0)
            with torch.cuda.stream(s):
                big.launch(cb)                    # first round grows it; the old buffer is retired
            torch.cuda.synchronize()
            g.replay()
            torch.cuda.synchronize()
            assert np.array_equal(host16(cg), ref), ("replay", r)
        big.check(host16(cb))
        del g
    finally:
        torch.cuda.synchronize()
        hip.hipStreamDestroy(h)


def test_grouped_capture_without_workspace_runs_whole_tiles(hkg):
    # A grouped plan that splits its last round (72 tiles of 128 x 128 on 64
    # workgroups: 8 tiles split in two halves of K) captured on a stream that
    # has no workspace yet: the captured call runs every tile whole (the
    # unsplit eager result, bit for bit); once an eager call has allocated
    # the workspace, a new capture splits (the split eager result).
    sizes, N, K = [1000, 300, 500, 260], 512, 320
    A, B, offs = workloads.make_grouped_inputs(sizes, N, K, seed=51)
    G, M = len(sizes), A.shape[0]
    a, b = dev16(A), dev16(B)
    offs_t = torch.from_numpy(np.ascontiguousarray(offs, dtype=np.int32)).to("cuda")

    def plan(split):
        p = hkg.grouped_plan(G, M, N, K)
        assert p.tile_m == 128 and p.tile_n == 128, p.kernel_name
        p.grid_x = 64
        p.split_k = split
        return p

    def eager(split):
        c = torch.zeros((M, N), dtype=torch.bfloat16, device="cuda")
        hkg.grouped_gemm(a, b, offs_t, out=c, plan=plan(split))
        torch.cuda.synchronize()
        return host16(c)

    whole, split = eager(1), eager(2)
    Cr, S, absS = oracle.grouped_gemm(A, B, offs)
    gates.compare(whole, Cr, S, absS)
    gates.compare(split, Cr, S, absS)
    assert not np.array_equal(whole, split), "the split should change some roundings"
    for allocated, want in ((False, whole), (True, split)):
        hip, h, s = _new_stream()
        try:
            if allocated:
                with torch.cuda.stream(s):
                    hkg.grouped_gemm(a, b, offs_t, out=torch.zeros((M, N), dtype=torch.bfloat16, device="cuda"),
                                     plan=plan(2))
            torch.cuda.synchronize()
            c = torch.zeros((M, N), dtype=torch.bfloat16, device="cuda")
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g, stream=s):
                hkg.grouped_gemm(a, b, offs_t, out=c, plan=plan(2))
            for r in range(3):
                c.fill_(0)
                torch.cuda.synchronize()
                g.replay()
                torch.cuda.synchronize()
                assert np.array_equal(host16(c), want), ("allocated", allocated, "replay", r)
            _say("grouped capture, workspace allocated before:", allocated)
            del g
        finally:
            torch.cuda.synchronize()
            hip.hipStreamDestroy(h)
