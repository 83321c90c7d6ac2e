"""Seeded synthetic inputs for the fused GEMM C = act(A @ B + bias).

This module only draws numbers: it holds none of the multiply, the epilogue or
the tile selection.  Both the HIP path and the oracle consume the arrays it
returns, so the two sides always see identical bytes.

Conventions (stated here because the pages leave them open):
  * A is [M, K] row-major, B is [K, N] row-major, bias is [N] float32 or None.
  * Random numbers come from numpy's PCG64 (``numpy.random.default_rng``).
    Draw order is A, then B, then bias; each is drawn in float64, scaled,
    cast to float32 and, for bf16 workloads, rounded to bf16 with
    round-to-nearest-even.  bf16 arrays are returned as uint16 bit patterns.
  * "N(0, s)" means mean 0 and standard deviation s; "uniform[-1,1)" is
    half-open.

The five workloads are the shapes the pages reason about (page "Compilers and
Kernel Languages", section "A different tile for every shape": a large square
multiply, the 1000 x 1000 x 8192 wave-quantisation case, a 16-token decode)
plus an fp32 sweep case and a ragged-edge case.
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field

import numpy as np

# dtype codes shared with the C ABI (input -> output)
F32 = 0            # fp32 in, fp32 out
BF16 = 1           # bf16 in, fp32 accumulate, bf16 out
BF16_F32OUT = 2    # bf16 in, fp32 accumulate, fp32 out

ACT_NONE, ACT_RELU, ACT_GELU = 0, 1, 2

DTYPE_NAMES = {F32: "f32", BF16: "bf16", BF16_F32OUT: "bf16_f32out"}
ACT_NAMES = {ACT_NONE: "none", ACT_RELU: "relu", ACT_GELU: "gelu"}


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 values to bf16 (round to nearest, ties to even).

    Returns the 16-bit patterns as uint16.  Inputs here are finite.
    """
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32).astype(np.uint64)
    lsb = (u >> np.uint64(16)) & np.uint64(1)
    return ((u + np.uint64(0x7FFF) + lsb) >> np.uint64(16)).astype(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    """Widen bf16 bit patterns to float32 (exact)."""
    return (np.asarray(b, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


@dataclass(frozen=True)
class Dist:
    """A value distribution: ``kind`` is "normal" (mean 0, std ``scale``) or
    "uniform" (on [-scale, scale)), or "int" (integers in [-scale, scale])."""
    kind: str
    scale: float = 1.0

    def draw(self, rng: np.random.Generator, shape) -> np.ndarray:
        if self.kind == "normal":
            return rng.standard_normal(shape) * self.scale
        if self.kind == "uniform":
            return rng.uniform(-self.scale, self.scale, shape)
        if self.kind == "int":
            s = int(self.scale)
            return rng.integers(-s, s + 1, shape).astype(np.float64)
        raise ValueError(f"unknown distribution {self.kind!r}")


@dataclass(frozen=True)
class Workload:
    name: str
    M: int
    N: int
    K: int
    dtype: int
    act: int
    a_dist: Dist
    b_dist: Dist
    bias_dist: Dist | None
    seed: int
    note: str = ""

    @property
    def flops(self) -> float:
        return 2.0 * self.M * self.N * self.K

    @property
    def in_bytes(self) -> int:
        return 4 if self.dtype == F32 else 2

    @property
    def out_bytes(self) -> int:
        return 2 if self.dtype == BF16 else 4

    @property
    def compulsory_bytes(self) -> int:
        """Bytes every implementation must move: A, B, C once, bias once."""
        eb, ec = self.in_bytes, self.out_bytes
        b = eb * (self.M * self.K + self.K * self.N) + ec * self.M * self.N
        if self.bias_dist is not None:
            b += 4 * self.N
        return b

    def key(self) -> str:
        return f"{self.M}x{self.N}x{self.K}_{DTYPE_NAMES[self.dtype]}_{ACT_NAMES[self.act]}"


_SK = 1.0 / math.sqrt(8192.0)

# The five workloads, indexed 1..5; the seed is the index.
WORKLOADS: dict[int, Workload] = {
    1: Workload("fp32_relu_256", 256, 256, 256, F32, ACT_RELU,
                Dist("uniform"), Dist("uniform"), Dist("uniform"), 1,
                "fp32 sweep case: every feasible (BM,BN,BK) in {32,64,128}^2 x {16,32}"),
    2: Workload("bf16_1000x1000x8192", 1000, 1000, 8192, BF16_F32OUT, ACT_NONE,
                Dist("normal", _SK), Dist("normal", _SK), None, 2,
                "wave-quantisation case: few 128x128 tiles against 256 CUs"),
    3: Workload("bf16_square_8192_gelu", 8192, 8192, 8192, BF16, ACT_GELU,
                Dist("normal", _SK), Dist("normal", _SK), Dist("normal", 0.1), 3,
                "compute-bound large-tile case"),
    4: Workload("bf16_decode_m16", 16, 28672, 8192, BF16, ACT_NONE,
                Dist("normal", 1.0), Dist("normal", 0.02), None, 4,
                "HBM-bound weight-streaming decode case"),
    5: Workload("bf16_ragged_4100x3000x1000", 4100, 3000, 1000, BF16, ACT_RELU,
                Dist("normal", 1.0), Dist("normal", 1.0), Dist("uniform"), 5,
                "ragged edges: M mod 128 = 4, N mod 128 = 56, K mod 64 = 40"),
}


def _finish(x64: np.ndarray, dtype: int) -> np.ndarray:
    x32 = x64.astype(np.float32)
    return x32 if dtype == F32 else f32_to_bf16_bits(x32)


def make_inputs(M: int, N: int, K: int, dtype: int, a_dist: Dist, b_dist: Dist,
                bias_dist: Dist | None, seed: int):
    """Draw (A, B, bias) for one problem.

    A and B are float32 arrays (dtype F32) or uint16 bf16 bit patterns
    (BF16, BF16_F32OUT); bias is float32 [N] or None.
    """
    rng = np.random.default_rng(seed)
    A = _finish(a_dist.draw(rng, (M, K)), dtype)
    B = _finish(b_dist.draw(rng, (K, N)), dtype)
    bias = None
    if bias_dist is not None:
        bias = bias_dist.draw(rng, (N,)).astype(np.float32)
    return A, B, bias


def workload_inputs(index: int):
    w = WORKLOADS[index]
    return make_inputs(w.M, w.N, w.K, w.dtype, w.a_dist, w.b_dist, w.bias_dist, w.seed)


def as_float64(x: np.ndarray, dtype: int) -> np.ndarray:
    """Exact float64 view of an input array (used by tests for closed forms)."""
    if dtype == F32:
        return np.asarray(x, dtype=np.float32).astype(np.float64)
    return bf16_bits_to_f32(x).astype(np.float64)
