"""Python binding of libhkg.so, the gfx950 dense BF16 GEMM C = A * B^T.

Argument marshalling only: every step of the GEMM runs in the library's HIP
kernels.  The binding uses ctypes and mirrors the C ABI of include/hkg.h with
the same names (``hkg_gemm_bf16``, ``hkg_gemm_bf16_epilogue``,
``hkg_gemm_bf16_plan``, ``hkg_gemm_bf16_run_plan``,
``hkg_gemm_bf16_run_plan_epilogue``, ``hkg_status_string``); ``gemm`` is the
torch-facing convenience wrapper (with ``bias=`` and ``epilogue=`` for the
fused epilogues).  torch supplies device memory and streams.

There is no fallback: if the library is not built and cannot be built, or a
call fails, an exception is raised.
"""
import ctypes
import os

__all__ = ["HkgError", "Plan", "hkg_gemm_bf16", "hkg_gemm_bf16_epilogue", "hkg_gemm_bf16_plan",
           "hkg_gemm_bf16_run_plan", "hkg_gemm_bf16_run_plan_epilogue", "hkg_status_string",
           "hkg_last_hip_error", "gemm", "plan", "run_plan", "library_path", "EXPORTED_SYMBOLS",
           "KERNEL_NAMES", "EPILOGUES"]

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
KERNEL_NAMES = {0: "NONE", 1: "TILE", 2: "SKINNY", 3: "GENERIC", 4: "ZERO"}
HKG_KERNEL_NONE, HKG_KERNEL_TILE, HKG_KERNEL_SKINNY, HKG_KERNEL_GENERIC, HKG_KERNEL_ZERO = range(5)

# hkg_epilogue_t codes by the FlyDSL guide's names
EPILOGUES = {"none": 0, "bias": 1, "bias_relu": 2, "bias_silu": 3, "bias_gelu": 4}

EXPORTED_SYMBOLS = ["hkg_gemm_bf16", "hkg_gemm_bf16_epilogue", "hkg_gemm_bf16_plan", "hkg_gemm_bf16_run_plan",
                    "hkg_gemm_bf16_run_plan_epilogue", "hkg_status_string", "hkg_last_hip_error",
                    "hkg_abi_version"]


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
