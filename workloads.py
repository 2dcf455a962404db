"""Seeded synthetic inputs for the dense BF16 GEMM C = A * B^T.

This module is shared by the tests, the benchmark and the smoke check.  It
holds no GEMM arithmetic: it only draws input matrices and names the five
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


def draw(rng, shape, dist):
    kind = dist[0]
    if kind == "uniform":
        x = rng.uniform(dist[1], dist[2], size=shape)
    elif kind == "normal":
        x = rng.normal(dist[1], dist[2], size=shape)
    else:
        raise ValueError("unknown distribution %r" % (kind,))
    return f32_to_bf16_bits(x.astype(np.float32))


def make_inputs(M, N, K, a=("uniform", -1.0, 1.0), b=("uniform", -1.0, 1.0), seed=0):
    """(A bits M x K, B bits N x K) from one seeded stream, A drawn first."""
    rng = np.random.default_rng(seed)
    A = draw(rng, (M, K), a)
    B = draw(rng, (N, K), b)
    return A, B


def workload_inputs(name, seed=0):
    w = WORKLOADS[name]
    return make_inputs(w["M"], w["N"], w["K"], w["a"], w["b"], seed)
