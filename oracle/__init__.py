"""CPU oracle for C = A * B^T (bf16 in, fp64 sums, one bf16 rounding).

TEST INFRASTRUCTURE ONLY.  Only the tests, the smoke check and the
benchmark's CPU-baseline leg import this package.  It shares no code with the
HIP library (``tile_level_dense_amd``) and never imports it.

The arithmetic lives in ``hkg_oracle.c`` (plain C, built by gcc); this module
only marshals numpy arrays through ctypes.  The operation is the NT projection
GEMM of the FlyDSL "Prebuilt kernels guide" (section 3.1, Preshuffle GEMM:
C[M,N] = A[M,K] @ B[N,K]^T); the bf16 output rounding is nearest-even, as in
that guide's section 1.1 (bf16 handling on gfx950: hardware cvt_pk_bf16_f32).

Arrays of bf16 are numpy ``uint16`` holding the raw bit patterns.
"""
import ctypes
import os
import subprocess

import numpy as np

_DIR = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(_DIR, "hkg_oracle.c")
LIB = os.path.join(_DIR, "libhkg_oracle.so")


def build(force=False, src=SRC, out=LIB):
    """Compile the oracle with gcc (no fast-math; k order is the loop order)."""
    if force or not os.path.exists(out) or os.path.getmtime(out) < os.path.getmtime(src):
        tmp = out + ".tmp%d" % os.getpid()
        subprocess.check_call(
            ["gcc", "-O2", "-fopenmp", "-shared", "-fPIC", "-std=c11",
             "-fno-fast-math", "-ffp-contract=off", src, "-o", tmp, "-lm"])
        os.replace(tmp, out)
    return out


def _bind(path):
    lib = ctypes.CDLL(path)
    u16p = ctypes.POINTER(ctypes.c_uint16)
    f64p = ctypes.POINTER(ctypes.c_double)
    i64p = ctypes.POINTER(ctypes.c_int64)
    i64 = ctypes.c_int64
    lib.hkg_oracle_bf16_value.argtypes = [ctypes.c_uint16]
    lib.hkg_oracle_bf16_value.restype = ctypes.c_double
    lib.hkg_oracle_bf16_rne.argtypes = [ctypes.c_double]
    lib.hkg_oracle_bf16_rne.restype = ctypes.c_uint16
    lib.hkg_oracle_gemm_rows.argtypes = [u16p, u16p, i64, i64, i64, i64, i64,
                                         u16p, f64p, f64p, ctypes.c_int]
    lib.hkg_oracle_gemm_rows.restype = None
    lib.hkg_oracle_gemm_entries.argtypes = [u16p, u16p, i64, i64, i64, i64p, i64p, i64,
                                            u16p, f64p, f64p, ctypes.c_int]
    lib.hkg_oracle_gemm_entries.restype = None
    lib.hkg_oracle_gemm_layout_rows.argtypes = [u16p, i64, ctypes.c_int, u16p, i64, ctypes.c_int, i64, i64, i64,
                                                i64, i64, u16p, f64p, f64p, ctypes.c_int]
    lib.hkg_oracle_gemm_layout_rows.restype = None
    i32p = ctypes.POINTER(ctypes.c_int32)
    lib.hkg_oracle_grouped_gemm_rows.argtypes = [u16p, u16p, i32p, i64, i64, i64, i64, i64, i64,
                                                 u16p, f64p, f64p, ctypes.c_int]
    lib.hkg_oracle_grouped_gemm_rows.restype = ctypes.c_int
    lib.hkg_oracle_max_threads.argtypes = []
    lib.hkg_oracle_max_threads.restype = ctypes.c_int
    u8p = ctypes.POINTER(ctypes.c_uint8)
    lib.hkg_oracle_e4m3_value.argtypes = [ctypes.c_uint8]
    lib.hkg_oracle_e4m3_value.restype = ctypes.c_double
    lib.hkg_oracle_e8m0_value.argtypes = [ctypes.c_uint8]
    lib.hkg_oracle_e8m0_value.restype = ctypes.c_double
    lib.hkg_oracle_mx_gemm_rows.argtypes = [u8p, u8p, u8p, u8p, i64, i64, i64, i64, i64,
                                            u16p, f64p, f64p, ctypes.c_int]
    lib.hkg_oracle_mx_gemm_rows.restype = None
    lib.hkg_oracle_mx_gemm_entries.argtypes = [u8p, u8p, u8p, u8p, i64, i64, i64, i64p, i64p, i64,
                                               u16p, f64p, f64p, ctypes.c_int]
    lib.hkg_oracle_mx_gemm_entries.restype = None
    lib.hkg_oracle_e2m1_value.argtypes = [ctypes.c_uint8]
    lib.hkg_oracle_e2m1_value.restype = ctypes.c_double
    lib.hkg_oracle_mx4_gemm_rows.argtypes = lib.hkg_oracle_mx_gemm_rows.argtypes
    lib.hkg_oracle_mx4_gemm_rows.restype = None
    lib.hkg_oracle_mx4_gemm_entries.argtypes = lib.hkg_oracle_mx_gemm_entries.argtypes
    lib.hkg_oracle_mx4_gemm_entries.restype = None
    lib.hkg_oracle_activation.argtypes = [ctypes.c_double, ctypes.c_int]
    lib.hkg_oracle_activation.restype = ctypes.c_double
    lib.hkg_oracle_epilogue.argtypes = [f64p, u16p, i64, i64, i64p, ctypes.c_int, f64p, u16p]
    lib.hkg_oracle_epilogue.restype = ctypes.c_int
    return lib


def _ptr(a, ctype):
    return None if a is None else a.ctypes.data_as(ctypes.POINTER(ctype))


def _check_operands(A, B):
    A = np.ascontiguousarray(A, dtype=np.uint16)
    B = np.ascontiguousarray(B, dtype=np.uint16)
    if A.ndim != 2 or B.ndim != 2 or A.shape[1] != B.shape[1]:
        raise ValueError("A must be M x K and B N x K (bf16 bit patterns)")
    return A, B


class Oracle:
    """One loaded build of the oracle: the default one, or a variant a test built."""

    def __init__(self, path=None):
        if path is None:
            path = LIB
            if not os.path.exists(path):
                build()
        self.path = path
        self.lib = _bind(path)

    def bf16_value(self, bits):
        """f64 value of one bf16 bit pattern (from the format definition)."""
        return self.lib.hkg_oracle_bf16_value(int(bits))

    def bf16_rne(self, x):
        """Nearest-even bf16 bit pattern of one double."""
        return int(self.lib.hkg_oracle_bf16_rne(float(x)))

    def bf16_rne_array(self, x):
        x = np.asarray(x, dtype=np.float64)
        out = np.empty(x.shape, dtype=np.uint16)
        flat = out.reshape(-1)
        f = self.lib.hkg_oracle_bf16_rne
        for t, v in enumerate(x.reshape(-1).tolist()):
            flat[t] = f(v)
        return out

    def max_threads(self):
        return int(self.lib.hkg_oracle_max_threads())

    def gemm(self, A, B, rows=None, nthreads=0, want_sums=True):
        """C = A * B^T over rows [r0, r1) of C (all rows by default).

        Returns (C bits uint16, S float64, absS float64); S and absS are None
        when want_sums is False.
        """
        A, B = _check_operands(A, B)
        M, K = A.shape
        N = B.shape[0]
        r0, r1 = (0, M) if rows is None else rows
        if not (0 <= r0 <= r1 <= M):
            raise ValueError("row range out of bounds")
        C = np.zeros((r1 - r0, N), dtype=np.uint16)
        S = np.zeros((r1 - r0, N), dtype=np.float64) if want_sums else None
        absS = np.zeros((r1 - r0, N), dtype=np.float64) if want_sums else None
        if r1 > r0 and N > 0:
            self.lib.hkg_oracle_gemm_rows(
                _ptr(A, ctypes.c_uint16), _ptr(B, ctypes.c_uint16), M, N, K, r0, r1,
                _ptr(C, ctypes.c_uint16), _ptr(S, ctypes.c_double),
                _ptr(absS, ctypes.c_double), int(nthreads))
        return C, S, absS

    def gemm_layout(self, A, lda, a_col, B, ldb, b_col, M, N, K, rows=None, nthreads=0):
        """C = A * B^T with operands in stored form: A flat bf16 bits read as
        a(i,k) = A[i lda + k] (a_col False) or A[k lda + i] (a_col True); B as
        b(j,k) = B[j ldb + k] or B[k ldb + j].  Returns dense (C, S, absS)."""
        A = np.ascontiguousarray(A, dtype=np.uint16).reshape(-1)
        B = np.ascontiguousarray(B, dtype=np.uint16).reshape(-1)
        need_a = ((K - 1) * lda + M if a_col else (M - 1) * lda + K) if M and K else 0
        need_b = ((K - 1) * ldb + N if b_col else (N - 1) * ldb + K) if N and K else 0
        if A.size < need_a or B.size < need_b or lda < (M if a_col else K) or ldb < (N if b_col else K):
            raise ValueError("stored operands too small for the layout")
        r0, r1 = (0, M) if rows is None else rows
        C = np.zeros((r1 - r0, N), dtype=np.uint16)
        S = np.zeros((r1 - r0, N), dtype=np.float64)
        absS = np.zeros((r1 - r0, N), dtype=np.float64)
        if r1 > r0 and N > 0:
            self.lib.hkg_oracle_gemm_layout_rows(
                _ptr(A, ctypes.c_uint16), int(lda), int(bool(a_col)), _ptr(B, ctypes.c_uint16), int(ldb),
                int(bool(b_col)), M, N, K, r0, r1, _ptr(C, ctypes.c_uint16), _ptr(S, ctypes.c_double),
                _ptr(absS, ctypes.c_double), int(nthreads))
        return C, S, absS

    def grouped_gemm(self, A, B, offs, rows=None, nthreads=0):
        """Grouped C: A (M x K bf16 bits), B (G x N x K), offs (G int, row ends
        of each expert, non-decreasing, <= M).  Rows [r0, r1), default all rows
        of experts [0, offs[-1]).  Returns (C, S, absS)."""
        A = np.ascontiguousarray(A, dtype=np.uint16)
        B = np.ascontiguousarray(B, dtype=np.uint16)
        offs = np.ascontiguousarray(offs, dtype=np.int32)
        if A.ndim != 2 or B.ndim != 3 or A.shape[1] != B.shape[2] or offs.shape != (B.shape[0],):
            raise ValueError("A must be M x K, B G x N x K and offs G values")
        M, K = A.shape
        G, N = B.shape[0], B.shape[1]
        if G and (np.any(np.diff(offs) < 0) or offs[0] < 0 or offs[-1] > M):
            raise ValueError("offsets must be non-decreasing within [0, M]")
        end = int(offs[-1]) if G else 0
        r0, r1 = (0, end) if rows is None else rows
        if not (0 <= r0 <= r1 <= M):
            raise ValueError("row range out of bounds")
        C = np.zeros((r1 - r0, N), dtype=np.uint16)
        S = np.zeros((r1 - r0, N), dtype=np.float64)
        absS = np.zeros((r1 - r0, N), dtype=np.float64)
        if r1 > r0 and N > 0:
            self.lib.hkg_oracle_grouped_gemm_rows(
                _ptr(A, ctypes.c_uint16), _ptr(B, ctypes.c_uint16), _ptr(offs, ctypes.c_int32), G, M, N, K,
                r0, r1, _ptr(C, ctypes.c_uint16), _ptr(S, ctypes.c_double), _ptr(absS, ctypes.c_double),
                int(nthreads))
        return C, S, absS

    def gemm_entries(self, A, B, ii, jj, nthreads=0):
        """Selected elements C[ii[t], jj[t]] with their S and absS."""
        A, B = _check_operands(A, B)
        M, K = A.shape
        N = B.shape[0]
        ii = np.ascontiguousarray(ii, dtype=np.int64)
        jj = np.ascontiguousarray(jj, dtype=np.int64)
        if ii.shape != jj.shape:
            raise ValueError("index arrays differ in shape")
        if ii.size and (ii.min() < 0 or ii.max() >= M or jj.min() < 0 or jj.max() >= N):
            raise ValueError("index out of bounds")
        n = ii.size
        C = np.zeros(n, dtype=np.uint16)
        S = np.zeros(n, dtype=np.float64)
        absS = np.zeros(n, dtype=np.float64)
        if n:
            self.lib.hkg_oracle_gemm_entries(
                _ptr(A, ctypes.c_uint16), _ptr(B, ctypes.c_uint16), M, N, K,
                _ptr(ii, ctypes.c_int64), _ptr(jj, ctypes.c_int64), n,
                _ptr(C, ctypes.c_uint16), _ptr(S, ctypes.c_double),
                _ptr(absS, ctypes.c_double), int(nthreads))
        return C, S, absS


    def e4m3_value(self, bits):
        """f64 value of one E4M3 (OCP e4m3fn) code, from the format definition."""
        return self.lib.hkg_oracle_e4m3_value(int(bits))

    def e8m0_value(self, bits):
        """f64 value 2^(e - 127) of one E8M0 scale code (0xFF: NaN)."""
        return self.lib.hkg_oracle_e8m0_value(int(bits))

    def _mx_operands(self, A, SA, B, SB):
        A = np.ascontiguousarray(A, dtype=np.uint8)
        B = np.ascontiguousarray(B, dtype=np.uint8)
        SA = np.ascontiguousarray(SA, dtype=np.uint8)
        SB = np.ascontiguousarray(SB, dtype=np.uint8)
        if A.ndim != 2 or B.ndim != 2 or A.shape[1] != B.shape[1] or A.shape[1] % 32:
            raise ValueError("A must be M x K and B N x K E4M3 codes, K a multiple of 32")
        K = A.shape[1]
        if SA.shape != (A.shape[0], K // 32) or SB.shape != (B.shape[0], K // 32):
            raise ValueError("scales must be M x K/32 and N x K/32 E8M0 codes")
        return A, SA, B, SB

    def mx_gemm(self, A, SA, B, SB, rows=None, nthreads=0, want_sums=True):
        """MXFP8 C = (A * 2^SA) (B * 2^SB)^T over rows [r0, r1) (FlyDSL blog, MXFP
        section): (C bits uint16, S, absS) like gemm()."""
        A, SA, B, SB = self._mx_operands(A, SA, B, SB)
        M, K = A.shape
        N = B.shape[0]
        r0, r1 = (0, M) if rows is None else rows
        if not (0 <= r0 <= r1 <= M):
            raise ValueError("row range out of bounds")
        C = np.zeros((r1 - r0, N), dtype=np.uint16)
        S = np.zeros((r1 - r0, N), dtype=np.float64) if want_sums else None
        absS = np.zeros((r1 - r0, N), dtype=np.float64) if want_sums else None
        if r1 > r0 and N > 0:
            self.lib.hkg_oracle_mx_gemm_rows(
                _ptr(A, ctypes.c_uint8), _ptr(SA, ctypes.c_uint8), _ptr(B, ctypes.c_uint8),
                _ptr(SB, ctypes.c_uint8), M, N, K, r0, r1, _ptr(C, ctypes.c_uint16),
                _ptr(S, ctypes.c_double), _ptr(absS, ctypes.c_double), int(nthreads))
        return C, S, absS

    def mx_gemm_entries(self, A, SA, B, SB, ii, jj, nthreads=0):
        """Selected elements of the MXFP8 product with their S and absS."""
        A, SA, B, SB = self._mx_operands(A, SA, B, SB)
        M, K = A.shape
        N = B.shape[0]
        ii = np.ascontiguousarray(ii, dtype=np.int64)
        jj = np.ascontiguousarray(jj, dtype=np.int64)
        if ii.shape != jj.shape:
            raise ValueError("index arrays differ in shape")
        if ii.size and (ii.min() < 0 or ii.max() >= M or jj.min() < 0 or jj.max() >= N):
            raise ValueError("index out of bounds")
        n = ii.size
        C = np.zeros(n, dtype=np.uint16)
        S = np.zeros(n, dtype=np.float64)
        absS = np.zeros(n, dtype=np.float64)
        if n:
            self.lib.hkg_oracle_mx_gemm_entries(
                _ptr(A, ctypes.c_uint8), _ptr(SA, ctypes.c_uint8), _ptr(B, ctypes.c_uint8),
                _ptr(SB, ctypes.c_uint8), M, N, K, _ptr(ii, ctypes.c_int64), _ptr(jj, ctypes.c_int64), n,
                _ptr(C, ctypes.c_uint16), _ptr(S, ctypes.c_double), _ptr(absS, ctypes.c_double),
                int(nthreads))
        return C, S, absS

    def e2m1_value(self, code):
        """f64 value of one E2M1 code (0..15), from the format definition."""
        return self.lib.hkg_oracle_e2m1_value(int(code))

    def _mx4_operands(self, A, SA, B, SB):
        A = np.ascontiguousarray(A, dtype=np.uint8)
        B = np.ascontiguousarray(B, dtype=np.uint8)
        SA = np.ascontiguousarray(SA, dtype=np.uint8)
        SB = np.ascontiguousarray(SB, dtype=np.uint8)
        if A.ndim != 2 or B.ndim != 2 or A.shape[1] != B.shape[1] or A.shape[1] % 16:
            raise ValueError("A must be M x K/2 and B N x K/2 bytes of E2M1 pairs, K a multiple of 32")
        K = 2 * A.shape[1]
        if SA.shape != (A.shape[0], K // 32) or SB.shape != (B.shape[0], K // 32):
            raise ValueError("scales must be M x K/32 and N x K/32 E8M0 codes")
        return A, SA, B, SB, K

    def mx4_gemm(self, A, SA, B, SB, rows=None, nthreads=0, want_sums=True):
        """MXFP4 C = (A * 2^SA) (B * 2^SB)^T over rows [r0, r1) (FlyDSL blog, MXFP
        section; A, B packed two E2M1 codes per byte, k even in the low nibble):
        (C bits uint16, S, absS) like gemm()."""
        A, SA, B, SB, K = self._mx4_operands(A, SA, B, SB)
        M = A.shape[0]
        N = B.shape[0]
        r0, r1 = (0, M) if rows is None else rows
        if not (0 <= r0 <= r1 <= M):
            raise ValueError("row range out of bounds")
        C = np.zeros((r1 - r0, N), dtype=np.uint16)
        S = np.zeros((r1 - r0, N), dtype=np.float64) if want_sums else None
        absS = np.zeros((r1 - r0, N), dtype=np.float64) if want_sums else None
        if r1 > r0 and N > 0:
            self.lib.hkg_oracle_mx4_gemm_rows(
                _ptr(A, ctypes.c_uint8), _ptr(SA, ctypes.c_uint8), _ptr(B, ctypes.c_uint8),
                _ptr(SB, ctypes.c_uint8), M, N, K, r0, r1, _ptr(C, ctypes.c_uint16),
                _ptr(S, ctypes.c_double), _ptr(absS, ctypes.c_double), int(nthreads))
        return C, S, absS

    def mx4_gemm_entries(self, A, SA, B, SB, ii, jj, nthreads=0):
        """Selected elements of the MXFP4 product with their S and absS."""
        A, SA, B, SB, K = self._mx4_operands(A, SA, B, SB)
        M = A.shape[0]
        N = B.shape[0]
        ii = np.ascontiguousarray(ii, dtype=np.int64)
        jj = np.ascontiguousarray(jj, dtype=np.int64)
        if ii.shape != jj.shape:
            raise ValueError("index arrays differ in shape")
        if ii.size and (ii.min() < 0 or ii.max() >= M or jj.min() < 0 or jj.max() >= N):
            raise ValueError("index out of bounds")
        n = ii.size
        C = np.zeros(n, dtype=np.uint16)
        S = np.zeros(n, dtype=np.float64)
        absS = np.zeros(n, dtype=np.float64)
        if n:
            self.lib.hkg_oracle_mx4_gemm_entries(
                _ptr(A, ctypes.c_uint8), _ptr(SA, ctypes.c_uint8), _ptr(B, ctypes.c_uint8),
                _ptr(SB, ctypes.c_uint8), M, N, K, _ptr(ii, ctypes.c_int64), _ptr(jj, ctypes.c_int64), n,
                _ptr(C, ctypes.c_uint16), _ptr(S, ctypes.c_double), _ptr(absS, ctypes.c_double),
                int(nthreads))
        return C, S, absS

    def activation(self, x, epilogue):
        """act(x) in fp64 for one epilogue (x already includes the bias)."""
        return float(self.lib.hkg_oracle_activation(float(x), EPILOGUES[epilogue]))

    def epilogue(self, S, bias, epilogue, cols=None):
        """Fused epilogue on unrounded sums (FlyDSL prebuilt kernels guide,
        section 3.1): Y = act(S + bias[column]) in fp64 and its bf16 rounding.

        S: sums, any shape; whole rows of an N-column C unless `cols` gives
        each element's column.  bias: uint16 bf16 bits, one per column.
        Returns (C bits uint16, Y float64), both shaped like S.
        """
        S = np.ascontiguousarray(S, dtype=np.float64)
        bias = np.ascontiguousarray(bias, dtype=np.uint16)
        epi = EPILOGUES[epilogue]
        N = bias.size
        if cols is not None:
            cols = np.ascontiguousarray(cols, dtype=np.int64).reshape(-1)
            if cols.size != S.size or (cols.size and (cols.min() < 0 or cols.max() >= N)):
                raise ValueError("column indices do not match S or bias")
        elif epi != 0 and S.size and (S.ndim < 1 or S.shape[-1] != N):
            raise ValueError("bias must hold one value per column")
        C = np.zeros(S.shape, dtype=np.uint16)
        Y = np.zeros(S.shape, dtype=np.float64)
        if S.size:
            rc = self.lib.hkg_oracle_epilogue(_ptr(S, ctypes.c_double), _ptr(bias, ctypes.c_uint16) if N else None,
                                              S.size, max(N, 1), _ptr(cols, ctypes.c_int64),
                                              epi, _ptr(Y, ctypes.c_double), _ptr(C, ctypes.c_uint16))
            if rc != 0:
                raise ValueError("unknown epilogue")
        return C, Y


# Fused epilogues by name (FlyDSL prebuilt kernels guide, section 3.1).
EPILOGUES = {"none": 0, "bias": 1, "bias_relu": 2, "bias_silu": 3, "bias_gelu": 4}

_default = None


def default():
    global _default
    if _default is None:
        _default = Oracle()
    return _default


def bf16_value(bits):
    return default().bf16_value(bits)


def bf16_rne(x):
    return default().bf16_rne(x)


def bf16_rne_array(x):
    return default().bf16_rne_array(x)


def max_threads():
    return default().max_threads()


def gemm(A, B, rows=None, nthreads=0, want_sums=True):
    return default().gemm(A, B, rows, nthreads, want_sums)


def gemm_layout(A, lda, a_col, B, ldb, b_col, M, N, K, rows=None, nthreads=0):
    return default().gemm_layout(A, lda, a_col, B, ldb, b_col, M, N, K, rows, nthreads)


def grouped_gemm(A, B, offs, rows=None, nthreads=0):
    return default().grouped_gemm(A, B, offs, rows, nthreads)


def gemm_entries(A, B, ii, jj, nthreads=0):
    return default().gemm_entries(A, B, ii, jj, nthreads)


def activation(x, epilogue):
    return default().activation(x, epilogue)


def mx_gemm(A, SA, B, SB, rows=None, nthreads=0, want_sums=True):
    return default().mx_gemm(A, SA, B, SB, rows, nthreads, want_sums)


def mx_gemm_entries(A, SA, B, SB, ii, jj, nthreads=0):
    return default().mx_gemm_entries(A, SA, B, SB, ii, jj, nthreads)


def e2m1_value(code):
    return default().e2m1_value(code)


def mx4_gemm(A, SA, B, SB, rows=None, nthreads=0, want_sums=True):
    return default().mx4_gemm(A, SA, B, SB, rows, nthreads, want_sums)


def mx4_gemm_entries(A, SA, B, SB, ii, jj, nthreads=0):
    return default().mx4_gemm_entries(A, SA, B, SB, ii, jj, nthreads)


def epilogue(S, bias, epilogue, cols=None):
    return default().epilogue(S, bias, epilogue, cols)
