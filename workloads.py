"""Seeded synthetic inputs for the dense BF16 GEMM C = A * B^T and its
block-scaled FP8 (MXFP8) variant.

This module is shared by the tests, the benchmark and the smoke check.  It
holds no GEMM arithmetic: it only draws input matrices (and, for MXFP8,
encodes them as E4M3 codes with per-block E8M0 scales) and names the
workload shapes.  Neither the oracle nor the HIP library imports it; the
callers hand its arrays to both.

Recipe (the same for every workload): numpy ``default_rng(seed)`` (PCG64),
draw A first and then B from that one stream as float64, narrow to float32
(numpy, nearest-even), then to bf16 with nearest-even on the float32 bit
pattern.  Arrays are numpy ``uint16`` bit patterns, row-major.

Workload shapes stand in for transformer projection and feed-forward layers,
the use the FlyDSL-in-PyTorch blog post gives its dense NT GEMMs (section
"Dense GEMM"); uniform [-1, 1] and N(0, 1) inputs follow the random-input
protocol of the HipKittens talk notes (section "Experiments").
"""
import numpy as np

# name, M, N, K, distribution of A, distribution of B.
# ("uniform", lo, hi) or ("normal", mean, std); std 0.02 is the usual
# weight-init scale for projection weights.
WORKLOADS = {
    "tiny_256": dict(M=256, N=256, K=256,
                     a=("uniform", -1.0, 1.0), b=("uniform", -1.0, 1.0)),
    "decode_16x4096x4096": dict(M=16, N=4096, K=4096,
                                a=("normal", 0.0, 1.0), b=("normal", 0.0, 0.02)),
    "mlp_up_128x12288x4096": dict(M=128, N=12288, K=4096,
                                  a=("normal", 0.0, 1.0), b=("normal", 0.0, 0.02)),
    "prefill_down_4096x4096x12288": dict(M=4096, N=4096, K=12288,
                                         a=("normal", 0.0, 1.0), b=("normal", 0.0, 0.02)),
    "square_8192": dict(M=8192, N=8192, K=8192,
                        a=("uniform", -1.0, 1.0), b=("uniform", -1.0, 1.0)),
}
ORDER = ["tiny_256", "decode_16x4096x4096", "mlp_up_128x12288x4096",
         "prefill_down_4096x4096x12288", "square_8192"]


def f32_to_bf16_bits(x32):
    """float32 array -> bf16 bit patterns (nearest-even); inputs are finite."""
    u = np.ascontiguousarray(x32, dtype=np.float32).view(np.uint32)
    lsb = (u >> np.uint32(16)) & np.uint32(1)
    return ((u + np.uint32(0x7FFF) + lsb) >> np.uint32(16)).astype(np.uint16)


def bf16_bits_to_f32(b):
    """bf16 bit patterns -> float32 (exact widening)."""
    return (np.asarray(b, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def draw_values(rng, shape, dist):
    """float64 draws of one distribution."""
    kind = dist[0]
    if kind == "uniform":
        return rng.uniform(dist[1], dist[2], size=shape)
    if kind == "normal":
        return rng.normal(dist[1], dist[2], size=shape)
    raise ValueError("unknown distribution %r" % (kind,))


def draw(rng, shape, dist):
    """bf16 bit patterns of one distribution (float64 -> float32 -> bf16)."""
    return f32_to_bf16_bits(draw_values(rng, shape, dist).astype(np.float32))


def make_inputs(M, N, K, a=("uniform", -1.0, 1.0), b=("uniform", -1.0, 1.0), seed=0):
    """(A bits M x K, B bits N x K) from one seeded stream, A drawn first."""
    rng = np.random.default_rng(seed)
    A = draw(rng, (M, K), a)
    B = draw(rng, (N, K), b)
    return A, B


# The compute-bound middle: prefill chunks of 1024 and 2048 tokens through a
# 4096-wide projection, where 256 x 256 output tiles are too few to fill the
# device (64 and 128 tiles for 256 compute units).  Context for the
# benchmark and the parity tests, beside the workloads above.
MIDDLE_WORKLOADS = {
    "middle_1024x4096x4096": dict(M=1024, N=4096, K=4096,
                                  a=("normal", 0.0, 1.0), b=("normal", 0.0, 0.02)),
    "middle_2048x4096x4096": dict(M=2048, N=4096, K=4096,
                                  a=("normal", 0.0, 1.0), b=("normal", 0.0, 0.02)),
}


def workload_inputs(name, seed=0):
    w = WORKLOADS[name] if name in WORKLOADS else MIDDLE_WORKLOADS[name]
    return make_inputs(w["M"], w["N"], w["K"], w["a"], w["b"], seed)


# ------------------------------------------------------------ MXFP8 inputs
# Block-scaled FP8 operands (FlyDSL-in-PyTorch blog, MXFP section: E4M3
# values, one E8M0 scale per 32 values along K).  Recipe: draw float64
# values as above (A first, then B, one stream), then for every block of 32
# along K pick the scale 2^e with e = ceil(log2(max|x| / 448)) (so the
# block's largest magnitude fits E4M3's 448; all-zero blocks get e = 0),
# store e + 127 as the E8M0 code, and the E4M3 codes of x / 2^e rounded to
# nearest-even (torch's float8_e4m3fn conversion).  Returns uint8 arrays
# (A, SA, B, SB) with SA M x K/32 and SB N x K/32.
MX_WORKLOADS = {
    "mx_tiny_256": dict(M=256, N=256, K=256, a=("normal", 0.0, 1.0), b=("normal", 0.0, 1.0)),
    "mx_decode_32x4096x4096": dict(M=32, N=4096, K=4096, a=("normal", 0.0, 1.0), b=("normal", 0.0, 0.02)),
    "mx_square_8192": dict(M=8192, N=8192, K=8192, a=("normal", 0.0, 1.0), b=("normal", 0.0, 1.0)),
}


def mx_quantize(x):
    """float64 rows (R x K, K % 32 == 0) -> (E4M3 codes R x K, E8M0 codes R x K/32)."""
    import torch
    x = np.asarray(x, dtype=np.float64)
    R, K = x.shape
    blocks = x.reshape(R, K // 32, 32)
    amax = np.abs(blocks).max(axis=2)
    with np.errstate(divide="ignore"):
        e = np.where(amax > 0, np.ceil(np.log2(amax / 448.0)), 0.0)
    e = np.clip(e, -127, 127).astype(np.int64)
    scaled = blocks / np.ldexp(1.0, e)[:, :, None]
    codes = torch.from_numpy(scaled.astype(np.float32)).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    return codes.reshape(R, K).copy(), (e + 127).astype(np.uint8)


def make_mx_inputs(M, N, K, a=("normal", 0.0, 1.0), b=("normal", 0.0, 1.0), seed=0):
    rng = np.random.default_rng(seed)
    xa = draw_values(rng, (M, K), a)
    xb = draw_values(rng, (N, K), b)
    A, SA = mx_quantize(xa)
    B, SB = mx_quantize(xb)
    return A, SA, B, SB


def mx_workload_inputs(name, seed=0):
    w = MX_WORKLOADS[name]
    return make_mx_inputs(w["M"], w["N"], w["K"], w["a"], w["b"], seed)


# ------------------------------------------------------------------ MXFP4
# Block-scaled FP4 GEMMs (FlyDSL-in-PyTorch blog, MXFP section: packed E2M1
# operands, one E8M0 scale per 32 k; its MXFP4 gains peak at 32 x 14336 x
# 4096, which the decode workload takes).  Recipe: E2M1 codes drawn
# uniformly from all 16 codes (values 0, +-0.5, ..., +-6; the format has no
# special codes) and packed two per byte, element 2c in the low nibble of
# byte c; E8M0 scale codes drawn uniformly from a small range per operand
# (activations 2^-2 .. 2^1, the decode weights 2^-9 .. 2^-6, the magnitudes
# quantised N(0, 1) activations and N(0, 0.02) weights carry).  A's codes,
# A's scales, B's codes, B's scales, in that order, from one seeded stream.
MX4_WORKLOADS = {
    "mx4_tiny_256": dict(M=256, N=256, K=256, sa=(125, 129), sb=(125, 129)),
    "mx4_decode_32x14336x4096": dict(M=32, N=14336, K=4096, sa=(125, 129), sb=(118, 122)),
    "mx4_square_8192": dict(M=8192, N=8192, K=8192, sa=(125, 129), sb=(125, 129)),
}


def pack_e2m1(codes):
    """R x K codes (0..15, K even) -> R x K/2 bytes, element 2c in the low nibble of byte c."""
    codes = np.asarray(codes, dtype=np.uint8)
    return (codes[:, 0::2] | (codes[:, 1::2] << 4)).astype(np.uint8)


def unpack_e2m1(packed):
    """Inverse of pack_e2m1: R x K/2 bytes -> R x K codes."""
    packed = np.asarray(packed, dtype=np.uint8)
    out = np.empty((packed.shape[0], 2 * packed.shape[1]), dtype=np.uint8)
    out[:, 0::2] = packed & 0xF
    out[:, 1::2] = packed >> 4
    return out


def make_mx4_inputs(M, N, K, sa=(125, 129), sb=(125, 129), seed=0):
    """(A M x K/2, SA M x K/32, B N x K/2, SB N x K/32) uint8; scale codes in [lo, hi)."""
    rng = np.random.default_rng(seed)
    a = rng.integers(0, 16, size=(M, K), dtype=np.uint8)
    SA = rng.integers(sa[0], sa[1], size=(M, K // 32)).astype(np.uint8)
    b = rng.integers(0, 16, size=(N, K), dtype=np.uint8)
    SB = rng.integers(sb[0], sb[1], size=(N, K // 32)).astype(np.uint8)
    return pack_e2m1(a), SA, pack_e2m1(b), SB


def mx4_workload_inputs(name, seed=0):
    w = MX4_WORKLOADS[name]
    return make_mx4_inputs(w["M"], w["N"], w["K"], w["sa"], w["sb"], seed)


# ------------------------------------------------------------ grouped GEMM
# Mixture-of-experts GEMMs (FlyDSL-in-PyTorch blog, grouped GEMM section):
# the rows of all experts concatenated in A (sum of M_g rows), one N x K
# weight per expert stacked in B (G x N x K), and int32 offsets holding each
# expert's row end (cumulative sums of the sizes).  The blog measures uniform
# expert loads and ragged ones with empty and heavily skewed experts; these
# stand in for both.  Recipe: A drawn first, then B, from one seeded stream,
# as for the dense workloads.
GROUPED_WORKLOADS = {
    "grouped_tiny": dict(sizes=[64, 0, 100, 92], N=256, K=256,
                         a=("uniform", -1.0, 1.0), b=("uniform", -1.0, 1.0)),
    "moe_uniform_8x1024_4096x4096": dict(sizes=[1024] * 8, N=4096, K=4096,
                                         a=("normal", 0.0, 1.0), b=("normal", 0.0, 0.02)),
    "moe_ragged_16_8192_4096x4096": dict(sizes=[0, 1500, 37, 0, 800, 3000, 1, 255, 256, 257, 0, 1024, 500, 62,
                                                300, 200], N=4096, K=4096,
                                         a=("normal", 0.0, 1.0), b=("normal", 0.0, 0.02)),
}


def make_grouped_inputs(sizes, N, K, a=("uniform", -1.0, 1.0), b=("uniform", -1.0, 1.0), seed=0):
    """(A bits sum(sizes) x K, B bits G x N x K, offs int32 G) from one seeded stream."""
    rng = np.random.default_rng(seed)
    sizes = np.asarray(sizes, dtype=np.int64)
    A = draw(rng, (int(sizes.sum()), K), a)
    B = draw(rng, (sizes.size, N, K), b)
    return A, B, np.cumsum(sizes).astype(np.int32)


def grouped_workload_inputs(name, seed=0):
    w = GROUPED_WORKLOADS[name]
    return make_grouped_inputs(w["sizes"], w["N"], w["K"], w["a"], w["b"], seed)
