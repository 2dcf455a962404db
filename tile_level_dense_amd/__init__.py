"""Python binding of libhkg.so, the gfx950 dense BF16 GEMM C = A * B^T (and
its block-scaled forms, MXFP8 and MXFP4).

Argument marshalling only: every step of the GEMM runs in the library's HIP
kernels.  The binding uses ctypes and mirrors the C ABI of include/hkg.h with
the same names (``hkg_gemm_bf16``, ``hkg_gemm_bf16_epilogue``,
``hkg_gemm_bf16_plan``, ``hkg_gemm_bf16_run_plan``,
``hkg_gemm_bf16_run_plan_epilogue``, ``hkg_status_string``, and the MXFP8
calls ``hkg_gemm_mxfp8``, ``hkg_gemm_mxfp8_plan``, ``hkg_mx_pack_scales``,
``hkg_mx_packed_scales_bytes``, ``hkg_gemm_mxfp8_prepacked``,
``hkg_gemm_mxfp8_run_plan``, the MXFP4 calls ``hkg_gemm_mxfp4``,
``hkg_gemm_mxfp4_plan``, ``hkg_gemm_mxfp4_prepacked``,
``hkg_gemm_mxfp4_run_plan``, the grouped calls
``hkg_grouped_gemm_bf16``, ``hkg_grouped_gemm_bf16_plan``,
``hkg_grouped_gemm_bf16_run_plan``, and the layout calls ``hkg_gemm_bf16_ex``,
``hkg_pack_bf16``); ``gemm``, ``gemm_ex``, ``pack``, ``gemm_mxfp8``,
``gemm_mxfp4`` and ``grouped_gemm`` are the torch-facing convenience wrappers
(with ``bias=`` and ``epilogue=`` for the fused epilogues).  torch supplies
device memory and streams.

There is no fallback: if the library is not built and cannot be built, or a
call fails, an exception is raised.
"""
import ctypes
import os

__all__ = ["HkgError", "Plan", "hkg_gemm_bf16", "hkg_gemm_bf16_epilogue", "hkg_gemm_bf16_plan",
           "hkg_gemm_bf16_run_plan", "hkg_gemm_bf16_run_plan_epilogue", "hkg_status_string",
           "hkg_last_hip_error", "gemm", "plan", "run_plan", "library_path", "EXPORTED_SYMBOLS",
           "KERNEL_NAMES", "EPILOGUES", "hkg_gemm_mxfp8", "hkg_gemm_mxfp8_plan", "hkg_mx_pack_scales",
           "hkg_mx_packed_scales_bytes", "hkg_gemm_mxfp8_prepacked", "hkg_gemm_mxfp8_run_plan", "gemm_mxfp8",
           "mx_plan", "mx_pack_scales", "run_mx_plan", "hkg_grouped_gemm_bf16", "hkg_grouped_gemm_bf16_plan",
           "hkg_grouped_gemm_bf16_run_plan", "grouped_gemm", "grouped_plan", "hkg_gemm_bf16_ex", "hkg_pack_bf16",
           "gemm_ex", "pack", "LAYOUT_ROW", "LAYOUT_COL", "hkg_gemm_bf16_noalloc", "hkg_gemm_mxfp4",
           "hkg_gemm_mxfp4_plan", "hkg_gemm_mxfp4_prepacked", "hkg_gemm_mxfp4_run_plan", "gemm_mxfp4",
           "mx4_plan", "run_mx4_plan"]

_DIR = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_DIR, "libhkg.so")

HKG_ABI_VERSION = 1
STATUS = {0: "HKG_OK", -1: "HKG_ERR_INVALID_ARG", -2: "HKG_ERR_MISALIGNED", -3: "HKG_ERR_UNSUPPORTED",
          -4: "HKG_ERR_NO_DEVICE", -5: "HKG_ERR_ARCH", -6: "HKG_ERR_HIP", -7: "HKG_ERR_WORKSPACE"}
HKG_OK = 0
HKG_ERR_INVALID_ARG = -1
HKG_ERR_MISALIGNED = -2
HKG_ERR_UNSUPPORTED = -3
HKG_ERR_NO_DEVICE = -4
HKG_ERR_ARCH = -5
HKG_ERR_HIP = -6
HKG_ERR_WORKSPACE = -7
KERNEL_NAMES = {0: "NONE", 1: "TILE", 2: "SKINNY", 3: "GENERIC", 4: "ZERO", 5: "MX_TILE", 6: "GROUPED",
                7: "MX_SKINNY", 8: "MX4_TILE", 9: "MX4_SKINNY"}
(HKG_KERNEL_NONE, HKG_KERNEL_TILE, HKG_KERNEL_SKINNY, HKG_KERNEL_GENERIC, HKG_KERNEL_ZERO, HKG_KERNEL_MX_TILE,
 HKG_KERNEL_GROUPED, HKG_KERNEL_MX_SKINNY, HKG_KERNEL_MX4_TILE, HKG_KERNEL_MX4_SKINNY) = range(10)

LAYOUT_ROW, LAYOUT_COL = 0, 1          # hkg_layout_t

# hkg_epilogue_t codes by the FlyDSL guide's names
EPILOGUES = {"none": 0, "bias": 1, "bias_relu": 2, "bias_silu": 3, "bias_gelu": 4}

EXPORTED_SYMBOLS = ["hkg_gemm_bf16", "hkg_gemm_bf16_epilogue", "hkg_gemm_bf16_plan", "hkg_gemm_bf16_run_plan",
                    "hkg_gemm_bf16_run_plan_epilogue", "hkg_status_string", "hkg_last_hip_error",
                    "hkg_abi_version", "hkg_gemm_mxfp8", "hkg_gemm_mxfp8_plan", "hkg_mx_pack_scales",
                    "hkg_mx_packed_scales_bytes", "hkg_gemm_mxfp8_prepacked", "hkg_gemm_mxfp8_run_plan",
                    "hkg_grouped_gemm_bf16", "hkg_grouped_gemm_bf16_plan", "hkg_grouped_gemm_bf16_run_plan",
                    "hkg_gemm_bf16_ex", "hkg_pack_bf16", "hkg_gemm_bf16_noalloc", "hkg_gemm_mxfp4",
                    "hkg_gemm_mxfp4_plan", "hkg_gemm_mxfp4_prepacked", "hkg_gemm_mxfp4_run_plan"]


class Plan(ctypes.Structure):
    """Mirror of hkg_plan_t (include/hkg.h)."""
    _fields_ = [
        ("abi_version", ctypes.c_int32), ("kernel_id", ctypes.c_int32), ("variant", ctypes.c_int32),
        ("tile_m", ctypes.c_int32), ("tile_n", ctypes.c_int32), ("tile_k", ctypes.c_int32),
        ("waves", ctypes.c_int32), ("split_k", ctypes.c_int32),
        ("grid_x", ctypes.c_int32), ("grid_y", ctypes.c_int32), ("grid_z", ctypes.c_int32),
        ("block_x", ctypes.c_int32),
        ("xcd_window_w", ctypes.c_int32), ("xcd_chunk_c", ctypes.c_int32),
        ("workspace_bytes", ctypes.c_int64),
        ("lds_bytes", ctypes.c_int32), ("vgprs", ctypes.c_int32), ("agprs", ctypes.c_int32),
        ("sgprs", ctypes.c_int32), ("scratch_bytes", ctypes.c_int32),
        ("M", ctypes.c_int64), ("N", ctypes.c_int64), ("K", ctypes.c_int64),
        ("flops", ctypes.c_double), ("algorithmic_bytes", ctypes.c_double),
        ("kernel_name", ctypes.c_char * 64), ("reason", ctypes.c_char * 128),
    ]

    def as_dict(self):
        d = {}
        for name, _ in self._fields_:
            v = getattr(self, name)
            d[name] = v.decode() if isinstance(v, bytes) else v
        d["kernel"] = KERNEL_NAMES.get(self.kernel_id, "?")
        return d

    def __repr__(self):
        return "Plan(%s)" % ", ".join("%s=%r" % kv for kv in self.as_dict().items())


class HkgError(RuntimeError):
    def __init__(self, status, where=""):
        self.status = status
        msg = "%s: %s (%d)" % (where or "hkg", STATUS.get(status, "?"), status)
        detail = hkg_last_hip_error() if _lib is not None else ""
        if detail:
            msg += " -- " + detail
        super().__init__(msg)


_lib = None


def library_path():
    return LIB_PATH


def _load():
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        # Nothing built yet: build in-tree (hipcc for gfx950); errors propagate.
        from . import build as _build
        _build.build()
    lib = ctypes.CDLL(LIB_PATH)
    vp = ctypes.c_void_p
    i64 = ctypes.c_int64
    lib.hkg_gemm_bf16.argtypes = [vp, vp, vp, i64, i64, i64, vp]
    lib.hkg_gemm_bf16.restype = ctypes.c_int
    lib.hkg_gemm_bf16_noalloc.argtypes = [vp, vp, vp, i64, i64, i64, vp]
    lib.hkg_gemm_bf16_noalloc.restype = ctypes.c_int
    lib.hkg_gemm_bf16_plan.argtypes = [i64, i64, i64, ctypes.POINTER(Plan)]
    lib.hkg_gemm_bf16_plan.restype = ctypes.c_int
    lib.hkg_gemm_bf16_run_plan.argtypes = [ctypes.POINTER(Plan), vp, vp, vp, i64, i64, i64, vp]
    lib.hkg_gemm_bf16_run_plan.restype = ctypes.c_int
    lib.hkg_gemm_bf16_epilogue.argtypes = [vp, vp, vp, vp, i64, i64, i64, ctypes.c_int32, vp]
    lib.hkg_gemm_bf16_epilogue.restype = ctypes.c_int
    lib.hkg_gemm_bf16_run_plan_epilogue.argtypes = [ctypes.POINTER(Plan), vp, vp, vp, vp, i64, i64, i64,
                                                    ctypes.c_int32, vp]
    lib.hkg_gemm_bf16_run_plan_epilogue.restype = ctypes.c_int
    lib.hkg_status_string.argtypes = [ctypes.c_int]
    lib.hkg_status_string.restype = ctypes.c_char_p
    lib.hkg_last_hip_error.argtypes = []
    lib.hkg_last_hip_error.restype = ctypes.c_char_p
    lib.hkg_abi_version.argtypes = []
    lib.hkg_abi_version.restype = ctypes.c_int32
    i32 = ctypes.c_int32
    lib.hkg_gemm_mxfp8_plan.argtypes = [i64, i64, i64, ctypes.POINTER(Plan)]
    lib.hkg_gemm_mxfp8_plan.restype = ctypes.c_int
    lib.hkg_gemm_mxfp8.argtypes = [vp, vp, vp, vp, vp, vp, i64, i64, i64, i32, vp]
    lib.hkg_gemm_mxfp8.restype = ctypes.c_int
    lib.hkg_mx_packed_scales_bytes.argtypes = [i64, i64]
    lib.hkg_mx_packed_scales_bytes.restype = i64
    lib.hkg_mx_pack_scales.argtypes = [vp, vp, i64, i64, vp]
    lib.hkg_mx_pack_scales.restype = ctypes.c_int
    lib.hkg_gemm_mxfp8_prepacked.argtypes = [vp, vp, vp, vp, vp, vp, i64, i64, i64, i32, vp]
    lib.hkg_gemm_mxfp8_prepacked.restype = ctypes.c_int
    lib.hkg_gemm_mxfp8_run_plan.argtypes = [ctypes.POINTER(Plan), vp, vp, vp, vp, vp, vp, i64, i64, i64, i32, vp]
    lib.hkg_gemm_mxfp8_run_plan.restype = ctypes.c_int
    lib.hkg_gemm_mxfp4_plan.argtypes = [i64, i64, i64, ctypes.POINTER(Plan)]
    lib.hkg_gemm_mxfp4_plan.restype = ctypes.c_int
    lib.hkg_gemm_mxfp4.argtypes = [vp, vp, vp, vp, vp, vp, i64, i64, i64, i32, vp]
    lib.hkg_gemm_mxfp4.restype = ctypes.c_int
    lib.hkg_gemm_mxfp4_prepacked.argtypes = [vp, vp, vp, vp, vp, vp, i64, i64, i64, i32, vp]
    lib.hkg_gemm_mxfp4_prepacked.restype = ctypes.c_int
    lib.hkg_gemm_mxfp4_run_plan.argtypes = [ctypes.POINTER(Plan), vp, vp, vp, vp, vp, vp, i64, i64, i64, i32, vp]
    lib.hkg_gemm_mxfp4_run_plan.restype = ctypes.c_int
    lib.hkg_grouped_gemm_bf16_plan.argtypes = [i64, i64, i64, i64, ctypes.POINTER(Plan)]
    lib.hkg_grouped_gemm_bf16_plan.restype = ctypes.c_int
    lib.hkg_grouped_gemm_bf16.argtypes = [vp, vp, vp, vp, vp, i64, i64, i64, i64, i32, vp]
    lib.hkg_grouped_gemm_bf16.restype = ctypes.c_int
    lib.hkg_grouped_gemm_bf16_run_plan.argtypes = [ctypes.POINTER(Plan), vp, vp, vp, vp, vp, i64, i64, i64, i64, i32,
                                                   vp]
    lib.hkg_grouped_gemm_bf16_run_plan.restype = ctypes.c_int
    lib.hkg_gemm_bf16_ex.argtypes = [vp, i64, i32, vp, i64, i32, vp, vp, i64, i64, i64, i64, i32, vp]
    lib.hkg_gemm_bf16_ex.restype = ctypes.c_int
    lib.hkg_pack_bf16.argtypes = [vp, i64, i32, vp, i64, i64, vp]
    lib.hkg_pack_bf16.restype = ctypes.c_int
    if lib.hkg_abi_version() != HKG_ABI_VERSION:
        raise ImportError("libhkg.so ABI version %d, binding expects %d" % (lib.hkg_abi_version(), HKG_ABI_VERSION))
    _lib = lib
    return lib


def lib():
    return _load()


# ------------------------------------------------------------ raw C names
def hkg_gemm_bf16(A, B, C, M, N, K, stream=None):
    """C-ABI call with raw device addresses (ints); returns the status code."""
    return _load().hkg_gemm_bf16(A, B, C, M, N, K, stream)


def hkg_gemm_bf16_noalloc(A, B, C, M, N, K, stream=None):
    """C-ABI call of the no-allocation form (raw device addresses); status code."""
    return _load().hkg_gemm_bf16_noalloc(A, B, C, M, N, K, stream)


def hkg_gemm_bf16_plan(M, N, K):
    """(status, Plan) for an aligned call of this shape; host only."""
    p = Plan()
    st = _load().hkg_gemm_bf16_plan(M, N, K, ctypes.byref(p))
    return st, p


def hkg_gemm_bf16_run_plan(plan_, A, B, C, M, N, K, stream=None):
    return _load().hkg_gemm_bf16_run_plan(ctypes.byref(plan_), A, B, C, M, N, K, stream)


def hkg_gemm_bf16_epilogue(A, B, bias, C, M, N, K, epilogue, stream=None):
    """C-ABI call with raw device addresses (ints) and an epilogue code."""
    return _load().hkg_gemm_bf16_epilogue(A, B, bias, C, M, N, K, epilogue, stream)


def hkg_gemm_bf16_run_plan_epilogue(plan_, A, B, bias, C, M, N, K, epilogue, stream=None):
    return _load().hkg_gemm_bf16_run_plan_epilogue(ctypes.byref(plan_), A, B, bias, C, M, N, K, epilogue,
                                                   stream)


def hkg_gemm_mxfp8(A, SA, B, SB, bias, C, M, N, K, epilogue=0, stream=None):
    """C-ABI call with raw device addresses (ints); returns the status code."""
    return _load().hkg_gemm_mxfp8(A, SA, B, SB, bias, C, M, N, K, epilogue, stream)


def hkg_gemm_mxfp8_plan(M, N, K):
    p = Plan()
    st = _load().hkg_gemm_mxfp8_plan(M, N, K, ctypes.byref(p))
    return st, p


def hkg_mx_packed_scales_bytes(rows, K):
    return _load().hkg_mx_packed_scales_bytes(rows, K)


def hkg_mx_pack_scales(S, P, rows, K, stream=None):
    return _load().hkg_mx_pack_scales(S, P, rows, K, stream)


def hkg_gemm_mxfp8_prepacked(A, PA, B, PB, bias, C, M, N, K, epilogue=0, stream=None):
    return _load().hkg_gemm_mxfp8_prepacked(A, PA, B, PB, bias, C, M, N, K, epilogue, stream)


def hkg_gemm_mxfp8_run_plan(plan_, A, PA, B, PB, bias, C, M, N, K, epilogue=0, stream=None):
    return _load().hkg_gemm_mxfp8_run_plan(ctypes.byref(plan_), A, PA, B, PB, bias, C, M, N, K, epilogue, stream)


def hkg_gemm_mxfp4(A, SA, B, SB, bias, C, M, N, K, epilogue=0, stream=None):
    """C-ABI call with raw device addresses (ints); returns the status code."""
    return _load().hkg_gemm_mxfp4(A, SA, B, SB, bias, C, M, N, K, epilogue, stream)


def hkg_gemm_mxfp4_plan(M, N, K):
    p = Plan()
    st = _load().hkg_gemm_mxfp4_plan(M, N, K, ctypes.byref(p))
    return st, p


def hkg_gemm_mxfp4_prepacked(A, PA, B, PB, bias, C, M, N, K, epilogue=0, stream=None):
    return _load().hkg_gemm_mxfp4_prepacked(A, PA, B, PB, bias, C, M, N, K, epilogue, stream)


def hkg_gemm_mxfp4_run_plan(plan_, A, PA, B, PB, bias, C, M, N, K, epilogue=0, stream=None):
    return _load().hkg_gemm_mxfp4_run_plan(ctypes.byref(plan_), A, PA, B, PB, bias, C, M, N, K, epilogue, stream)


def hkg_gemm_bf16_ex(A, lda, a_layout, B, ldb, b_layout, bias, C, ldc, M, N, K, epilogue=0, stream=None):
    """C-ABI call with raw device addresses (ints); returns the status code."""
    return _load().hkg_gemm_bf16_ex(A, lda, a_layout, B, ldb, b_layout, bias, C, ldc, M, N, K, epilogue, stream)


def hkg_pack_bf16(X, ldx, layout, Y, rows, K, stream=None):
    return _load().hkg_pack_bf16(X, ldx, layout, Y, rows, K, stream)


def hkg_grouped_gemm_bf16(A, B, offs, bias, C, G, M, N, K, epilogue=0, stream=None):
    """C-ABI call with raw device addresses (ints); returns the status code."""
    return _load().hkg_grouped_gemm_bf16(A, B, offs, bias, C, G, M, N, K, epilogue, stream)


def hkg_grouped_gemm_bf16_plan(G, M, N, K):
    p = Plan()
    st = _load().hkg_grouped_gemm_bf16_plan(G, M, N, K, ctypes.byref(p))
    return st, p


def hkg_grouped_gemm_bf16_run_plan(plan_, A, B, offs, bias, C, G, M, N, K, epilogue=0, stream=None):
    return _load().hkg_grouped_gemm_bf16_run_plan(ctypes.byref(plan_), A, B, offs, bias, C, G, M, N, K, epilogue,
                                                  stream)


def hkg_status_string(status):
    return _load().hkg_status_string(status).decode()


def hkg_last_hip_error():
    return _load().hkg_last_hip_error().decode()


# ---------------------------------------------------------- torch helpers
def _stream_handle(stream, device):
    import torch
    if stream is None:
        stream = torch.cuda.current_stream(device)
    return stream.cuda_stream


def _check(a, b, out):
    import torch
    if a.dtype != torch.bfloat16 or b.dtype != torch.bfloat16:
        raise TypeError("A and B must be torch.bfloat16")
    if a.dim() != 2 or b.dim() != 2 or a.shape[1] != b.shape[1]:
        raise ValueError("A must be M x K and B N x K, got %s and %s" % (tuple(a.shape), tuple(b.shape)))
    if not (a.is_cuda and b.is_cuda):
        raise ValueError("A and B must be device tensors")
    if a.device != b.device:
        raise ValueError("A and B on different devices")
    if not (a.is_contiguous() and b.is_contiguous()):
        raise ValueError("A and B must be contiguous (row-major, K contiguous)")
    M, K = a.shape
    N = b.shape[0]
    if out is not None:
        if out.dtype != torch.bfloat16 or tuple(out.shape) != (M, N) or not out.is_contiguous() \
                or out.device != a.device:
            raise ValueError("out must be a contiguous bf16 %d x %d tensor on A's device" % (M, N))
    return M, N, K


def _epilogue_args(a, N, bias, epilogue):
    import torch
    code = EPILOGUES[epilogue]
    if code == 0:
        return 0, 0
    if bias is None or bias.dtype != torch.bfloat16 or tuple(bias.shape) != (N,) or not bias.is_contiguous() \
            or bias.device != a.device:
        raise ValueError("epilogue %r needs a contiguous bf16 bias of %d values on A's device" % (epilogue, N))
    return bias.data_ptr(), code


def gemm(a, b, out=None, stream=None, bias=None, epilogue="none"):
    """C = epilogue(a @ b.T + bias) for bf16 device tensors a (M x K), b (N x K)
    and bias (N); epilogue one of EPILOGUES ("none" ignores bias)."""
    import torch
    M, N, K = _check(a, b, out)
    bias_ptr, code = _epilogue_args(a, N, bias, epilogue)
    if out is None:
        out = torch.empty((M, N), dtype=torch.bfloat16, device=a.device)
    with torch.cuda.device(a.device):
        if code == 0:
            st = _load().hkg_gemm_bf16(a.data_ptr(), b.data_ptr(), out.data_ptr(), M, N, K,
                                       _stream_handle(stream, a.device))
        else:
            st = _load().hkg_gemm_bf16_epilogue(a.data_ptr(), b.data_ptr(), bias_ptr, out.data_ptr(), M, N, K,
                                                code, _stream_handle(stream, a.device))
    if st != HKG_OK:
        raise HkgError(st, "hkg_gemm_bf16" if code == 0 else "hkg_gemm_bf16_epilogue")
    return out


def plan(M, N, K):
    st, p = hkg_gemm_bf16_plan(M, N, K)
    if st != HKG_OK:
        raise HkgError(st, "hkg_gemm_bf16_plan")
    return p


def run_plan(plan_, a, b, out=None, stream=None, bias=None, epilogue="none"):
    import torch
    M, N, K = _check(a, b, out)
    bias_ptr, code = _epilogue_args(a, N, bias, epilogue)
    if out is None:
        out = torch.empty((M, N), dtype=torch.bfloat16, device=a.device)
    with torch.cuda.device(a.device):
        if code == 0:
            st = _load().hkg_gemm_bf16_run_plan(ctypes.byref(plan_), a.data_ptr(), b.data_ptr(),
                                                out.data_ptr(), M, N, K, _stream_handle(stream, a.device))
        else:
            st = _load().hkg_gemm_bf16_run_plan_epilogue(ctypes.byref(plan_), a.data_ptr(), b.data_ptr(), bias_ptr,
                                                         out.data_ptr(), M, N, K, code,
                                                         _stream_handle(stream, a.device))
    if st != HKG_OK:
        raise HkgError(st, "hkg_gemm_bf16_run_plan" if code == 0 else "hkg_gemm_bf16_run_plan_epilogue")
    return out


# ------------------------------------------------------------------ MXFP8
def _check_mx(a, sa, b, sb, out, packed, fp4=False):
    """Shapes of uint8 device tensors: a M x K and b N x K E4M3 codes (fp4:
    M x K/2 and N x K/2 bytes of E2M1 pairs); sa, sb the E8M0 scales, M x K/32
    and N x K/32 (or, packed, the packed byte counts)."""
    import torch
    for t, name in ((a, "A"), (b, "B"), (sa, "SA"), (sb, "SB")):
        if t.dtype != torch.uint8 or not t.is_cuda or not t.is_contiguous() or t.device != a.device:
            raise ValueError("%s must be a contiguous uint8 device tensor on A's device" % name)
    if a.dim() != 2 or b.dim() != 2 or a.shape[1] != b.shape[1]:
        raise ValueError("A must be M x K and B N x K, got %s and %s" % (tuple(a.shape), tuple(b.shape)))
    M, K = a.shape
    N = b.shape[0]
    if fp4:
        K *= 2
    if packed:
        if sa.numel() != max(0, hkg_mx_packed_scales_bytes(M, K)) or \
                sb.numel() != max(0, hkg_mx_packed_scales_bytes(N, K)):
            raise ValueError("packed scales must hold hkg_mx_packed_scales_bytes(rows, K) bytes")
    elif tuple(sa.shape) != (M, K // 32) or tuple(sb.shape) != (N, K // 32):
        raise ValueError("SA must be M x K/32 and SB N x K/32")
    if out is not None and (out.dtype != torch.bfloat16 or tuple(out.shape) != (M, N) or not out.is_contiguous()
                            or out.device != a.device):
        raise ValueError("out must be a contiguous bf16 %d x %d tensor on A's device" % (M, N))
    return M, N, K


def gemm_mxfp8(a, sa, b, sb, out=None, stream=None, bias=None, epilogue="none", packed=False):
    """C = epilogue(MXFP8 a @ b.T + bias): a (M x K) and b (N x K) uint8 E4M3
    codes, sa / sb their E8M0 scales (M x K/32, N x K/32; or packed by
    mx_pack_scales when packed=True), K % 128 == 0."""
    import torch
    M, N, K = _check_mx(a, sa, b, sb, out, packed)
    bias_ptr, code = _epilogue_args(a, N, bias, epilogue)
    if out is None:
        out = torch.empty((M, N), dtype=torch.bfloat16, device=a.device)
    fn = _load().hkg_gemm_mxfp8_prepacked if packed else _load().hkg_gemm_mxfp8
    with torch.cuda.device(a.device):
        st = fn(a.data_ptr(), sa.data_ptr(), b.data_ptr(), sb.data_ptr(), bias_ptr or None, out.data_ptr(), M, N, K,
                code, _stream_handle(stream, a.device))
    if st != HKG_OK:
        raise HkgError(st, "hkg_gemm_mxfp8_prepacked" if packed else "hkg_gemm_mxfp8")
    return out


def gemm_mxfp4(a, sa, b, sb, out=None, stream=None, bias=None, epilogue="none", packed=False):
    """C = epilogue(MXFP4 a @ b.T + bias): a (M x K/2) and b (N x K/2) uint8,
    two E2M1 codes per byte (k even in the low nibble), sa / sb their E8M0
    scales (M x K/32, N x K/32; or packed by mx_pack_scales when packed=True),
    K % 128 == 0."""
    import torch
    M, N, K = _check_mx(a, sa, b, sb, out, packed, fp4=True)
    bias_ptr, code = _epilogue_args(a, N, bias, epilogue)
    if out is None:
        out = torch.empty((M, N), dtype=torch.bfloat16, device=a.device)
    fn = _load().hkg_gemm_mxfp4_prepacked if packed else _load().hkg_gemm_mxfp4
    with torch.cuda.device(a.device):
        st = fn(a.data_ptr(), sa.data_ptr(), b.data_ptr(), sb.data_ptr(), bias_ptr or None, out.data_ptr(), M, N, K,
                code, _stream_handle(stream, a.device))
    if st != HKG_OK:
        raise HkgError(st, "hkg_gemm_mxfp4_prepacked" if packed else "hkg_gemm_mxfp4")
    return out


def mx4_plan(M, N, K):
    st, p = hkg_gemm_mxfp4_plan(M, N, K)
    if st != HKG_OK:
        raise HkgError(st, "hkg_gemm_mxfp4_plan")
    return p


def run_mx4_plan(plan_, a, pa, b, pb, out=None, stream=None, bias=None, epilogue="none"):
    """Runs an MXFP4 plan on packed scales pa, pb (a, b as gemm_mxfp4)."""
    import torch
    M, N, K = _check_mx(a, pa, b, pb, out, True, fp4=True)
    bias_ptr, code = _epilogue_args(a, N, bias, epilogue)
    if out is None:
        out = torch.empty((M, N), dtype=torch.bfloat16, device=a.device)
    with torch.cuda.device(a.device):
        st = _load().hkg_gemm_mxfp4_run_plan(ctypes.byref(plan_), a.data_ptr(), pa.data_ptr(), b.data_ptr(),
                                             pb.data_ptr(), bias_ptr or None, out.data_ptr(), M, N, K, code,
                                             _stream_handle(stream, a.device))
    if st != HKG_OK:
        raise HkgError(st, "hkg_gemm_mxfp4_run_plan")
    return out


def mx_pack_scales(s, K, stream=None):
    """Packed form (uint8 device tensor) of E8M0 scales s (rows x K/32)."""
    import torch
    if s.dtype != torch.uint8 or s.dim() != 2 or not s.is_cuda or not s.is_contiguous() or s.shape[1] * 32 != K:
        raise ValueError("scales must be a contiguous uint8 rows x K/32 device tensor")
    rows = s.shape[0]
    n = hkg_mx_packed_scales_bytes(rows, K)
    if n < 0:
        raise HkgError(HKG_ERR_INVALID_ARG, "hkg_mx_packed_scales_bytes")
    p = torch.empty(n, dtype=torch.uint8, device=s.device)
    with torch.cuda.device(s.device):
        st = _load().hkg_mx_pack_scales(s.data_ptr(), p.data_ptr(), rows, K, _stream_handle(stream, s.device))
    if st != HKG_OK:
        raise HkgError(st, "hkg_mx_pack_scales")
    return p


def mx_plan(M, N, K):
    st, p = hkg_gemm_mxfp8_plan(M, N, K)
    if st != HKG_OK:
        raise HkgError(st, "hkg_gemm_mxfp8_plan")
    return p


def run_mx_plan(plan_, a, pa, b, pb, out=None, stream=None, bias=None, epilogue="none"):
    """Runs an MXFP8 plan on packed scales pa, pb."""
    import torch
    M, N, K = _check_mx(a, pa, b, pb, out, True)
    bias_ptr, code = _epilogue_args(a, N, bias, epilogue)
    if out is None:
        out = torch.empty((M, N), dtype=torch.bfloat16, device=a.device)
    with torch.cuda.device(a.device):
        st = _load().hkg_gemm_mxfp8_run_plan(ctypes.byref(plan_), a.data_ptr(), pa.data_ptr(), b.data_ptr(),
                                             pb.data_ptr(), bias_ptr or None, out.data_ptr(), M, N, K, code,
                                             _stream_handle(stream, a.device))
    if st != HKG_OK:
        raise HkgError(st, "hkg_gemm_mxfp8_run_plan")
    return out


# ----------------------------------------------------------- grouped GEMM
def grouped_plan(G, M, N, K):
    st, p = hkg_grouped_gemm_bf16_plan(G, M, N, K)
    if st != HKG_OK:
        raise HkgError(st, "hkg_grouped_gemm_bf16_plan")
    return p


def grouped_gemm(a, b, offs, out=None, stream=None, bias=None, epilogue="none", plan=None):
    """Mixture-of-experts GEMM: a (M x K bf16, experts' rows concatenated),
    b (G x N x K bf16, one weight per expert), offs (G int32 row ends, device),
    bias (G x N bf16) for epilogues.  Rows of no expert in `out` are left as
    they are (zeros when out is None)."""
    import torch
    if a.dtype != torch.bfloat16 or b.dtype != torch.bfloat16 or offs.dtype != torch.int32:
        raise TypeError("A, B must be torch.bfloat16 and offs torch.int32")
    if a.dim() != 2 or b.dim() != 3 or a.shape[1] != b.shape[2] or offs.dim() != 1 or offs.shape[0] != b.shape[0]:
        raise ValueError("A must be M x K, B G x N x K and offs G values")
    for t in (a, b, offs):
        if not t.is_cuda or not t.is_contiguous() or t.device != a.device:
            raise ValueError("operands must be contiguous device tensors on one device")
    M, K = a.shape
    G, N = b.shape[0], b.shape[1]
    code = EPILOGUES[epilogue]
    bias_ptr = None
    if code:
        if bias is None or bias.dtype != torch.bfloat16 or tuple(bias.shape) != (G, N) or not bias.is_contiguous() \
                or bias.device != a.device:
            raise ValueError("epilogue %r needs a contiguous bf16 G x N bias on A's device" % epilogue)
        bias_ptr = bias.data_ptr()
    if out is None:
        out = torch.zeros((M, N), dtype=torch.bfloat16, device=a.device)
    elif out.dtype != torch.bfloat16 or tuple(out.shape) != (M, N) or not out.is_contiguous() or out.device != a.device:
        raise ValueError("out must be a contiguous bf16 %d x %d tensor on A's device" % (M, N))
    with torch.cuda.device(a.device):
        args = (a.data_ptr(), b.data_ptr(), offs.data_ptr(), bias_ptr, out.data_ptr(), G, M, N, K, code,
                _stream_handle(stream, a.device))
        if plan is None:
            st = _load().hkg_grouped_gemm_bf16(*args)
        else:
            st = _load().hkg_grouped_gemm_bf16_run_plan(ctypes.byref(plan), *args)
    if st != HKG_OK:
        raise HkgError(st, "hkg_grouped_gemm_bf16")
    return out


# ------------------------------------------------------------------ layouts
def _layout_of(t, name):
    """(layout, leading dimension) of a 2-D tensor view with one unit stride:
    row layout when its last dimension is contiguous, column layout when its
    first is (e.g. W.t() of a K x N weight W)."""
    if t.dim() != 2:
        raise ValueError("%s must be 2-D" % name)
    r, c = t.shape
    s0, s1 = t.stride()
    if s1 == 1 or c <= 1:
        return LAYOUT_ROW, max(s0 if r > 1 else c, c, 1)
    if s0 == 1 or r <= 1:
        return LAYOUT_COL, max(s1 if c > 1 else r, r, 1)
    raise ValueError("%s needs one unit stride (got strides %s)" % (name, (s0, s1)))


def gemm_ex(a, b, out=None, stream=None, bias=None, epilogue="none"):
    """C = epilogue(a @ b.T + bias) for bf16 device views a (M x K) and b
    (N x K) in any layout: each may be row-major or a transposed view (one
    unit stride), with any leading dimension; out may be a row-major view
    with a leading dimension (its other elements are left alone)."""
    import torch
    if a.dtype != torch.bfloat16 or b.dtype != torch.bfloat16:
        raise TypeError("A and B must be torch.bfloat16")
    if a.dim() != 2 or b.dim() != 2 or a.shape[1] != b.shape[1] or not (a.is_cuda and b.is_cuda) \
            or a.device != b.device:
        raise ValueError("A must be M x K and B N x K device views")
    M, K = a.shape
    N = b.shape[0]
    la, lda = _layout_of(a, "A")
    lb, ldb = _layout_of(b, "B")
    if out is None:
        out = torch.empty((M, N), dtype=torch.bfloat16, device=a.device)
    if out.dtype != torch.bfloat16 or tuple(out.shape) != (M, N) or out.device != a.device or \
            (N > 1 and out.stride(1) != 1):
        raise ValueError("out must be a bf16 %d x %d view with unit column stride" % (M, N))
    ldc = max(out.stride(0) if M > 1 else N, N, 1)
    bias_ptr, code = _epilogue_args(a, N, bias, epilogue)
    with torch.cuda.device(a.device):
        st = _load().hkg_gemm_bf16_ex(a.data_ptr(), lda, la, b.data_ptr(), ldb, lb, bias_ptr or None,
                                      out.data_ptr(), ldc, M, N, K, code, _stream_handle(stream, a.device))
    if st != HKG_OK:
        raise HkgError(st, "hkg_gemm_bf16_ex")
    return out


def pack(x, stream=None):
    """Row-layout, dense copy (rows x K) of a bf16 device view x (rows x K) in
    any layout, by hkg_pack_bf16: the form the fast kernels read in place."""
    import torch
    if x.dtype != torch.bfloat16 or not x.is_cuda:
        raise TypeError("x must be a bf16 device tensor")
    rows, K = x.shape
    layout, ld = _layout_of(x, "x")
    y = torch.empty((rows, K), dtype=torch.bfloat16, device=x.device)
    with torch.cuda.device(x.device):
        st = _load().hkg_pack_bf16(x.data_ptr(), ld, layout, y.data_ptr(), rows, K, _stream_handle(stream, x.device))
    if st != HKG_OK:
        raise HkgError(st, "hkg_pack_bf16")
    return y
