"""Seeded synthetic inputs shared by the HIP path's tests/bench and the CPU oracle.

This module holds no arithmetic of the method itself: it only draws numbers.
Both sides of every parity check receive the very same bytes from here.

Generator (stated so that it can be re-implemented anywhere):

* Uniform source: SplitMix64 (S. Vigna, public domain), used as a counter-based
  hash.  For sub-stream ``k`` of seed ``s`` the key is
  ``key = mix64(s * 0x9E3779B97F4A7C15 + (k + 1) * 0xD1B54A32D192ED03)`` and the
  ``i``-th 64-bit word is ``mix64(key + (i + 1) * 0x9E3779B97F4A7C15)``, where
  ``mix64(z) = z ^ (z >> 31)`` after ``z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9``
  and ``z = (z ^ (z >> 27)) * 0x94D049BB133111EB`` (all mod 2**64).
* 53-bit uniforms: ``u = ((w >> 11) + 1) * 2**-53`` lies in (0, 1].
* Normals: Box-Muller, cosine branch, in float64:
  ``sqrt(-2 ln u[2j]) * cos(2 pi u[2j+1])``.
* Rounding: float64 -> float32 (round to nearest even) -> bfloat16 (round to
  nearest even on the float32 bit pattern) for bf16 tensors.

Workload shapes are those of the vision-backbone stages the method targets
("Seeing Both Ways, Running One Way", section 2: stage-3 and stage-4 patch
sequences of 196 and 49 tokens), plus two aux tokens per sequence (section 3.2).
"""
from __future__ import annotations

import dataclasses
import math

import numpy as np

_GOLDEN = np.uint64(0x9E3779B97F4A7C15)
_STREAM = np.uint64(0xD1B54A32D192ED03)
_M1 = np.uint64(0xBF58476D1CE4E5B9)
_M2 = np.uint64(0x94D049BB133111EB)
_BLOCK = 1 << 22

# Sub-stream ids, in the documented draw order.
STREAM_X, STREAM_DELTA, STREAM_B, STREAM_C, STREAM_DT0, STREAM_CONVW, STREAM_ARAND = range(7)


def _mix64(z: np.ndarray) -> np.ndarray:
    z = (z ^ (z >> np.uint64(30))) * _M1
    z = (z ^ (z >> np.uint64(27))) * _M2
    return z ^ (z >> np.uint64(31))


def _key(seed: int, stream: int) -> np.uint64:
    with np.errstate(over="ignore"):
        z = np.array([np.uint64(seed) * _GOLDEN + np.uint64(stream + 1) * _STREAM], dtype=np.uint64)
        return _mix64(z)[0]


def uniform53(seed: int, stream: int, count: int, start: int = 0) -> np.ndarray:
    """float64 uniforms in (0, 1], words ``start .. start+count-1`` of a sub-stream."""
    key = _key(seed, stream)
    out = np.empty(count, dtype=np.float64)
    with np.errstate(over="ignore"):
        for lo in range(0, count, _BLOCK):
            n = min(_BLOCK, count - lo)
            idx = np.arange(start + lo + 1, start + lo + 1 + n, dtype=np.uint64)
            w = _mix64(key + idx * _GOLDEN)
            out[lo:lo + n] = ((w >> np.uint64(11)).astype(np.float64) + 1.0) * (2.0 ** -53)
    return out


def normal(seed: int, stream: int, count: int) -> np.ndarray:
    """float64 standard normals (Box-Muller, cosine branch)."""
    out = np.empty(count, dtype=np.float64)
    for lo in range(0, count, _BLOCK):
        n = min(_BLOCK, count - lo)
        u = uniform53(seed, stream, 2 * n, start=2 * lo)
        out[lo:lo + n] = np.sqrt(-2.0 * np.log(u[0::2])) * np.cos(2.0 * math.pi * u[1::2])
    return out


def f32_to_bf16_bits(a: np.ndarray) -> np.ndarray:
    """Round float32 values to bfloat16 (nearest even); returns uint16 bit patterns."""
    bits = np.ascontiguousarray(a, dtype=np.float32).view(np.uint32).astype(np.uint64)
    rounded = (bits + np.uint64(0x7FFF) + ((bits >> np.uint64(16)) & np.uint64(1))) >> np.uint64(16)
    return rounded.astype(np.uint16)


def bf16_bits_to_f64(b: np.ndarray) -> np.ndarray:
    """Exact upcast of bfloat16 bit patterns to float64."""
    return (b.astype(np.uint32) << np.uint32(16)).view(np.float32).astype(np.float64)


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    B: int          # images in the batch
    D: int          # channels
    N: int          # SSM state size
    T: int          # patch tokens per image (before the two aux tokens)
    io: str         # "f32" or "bf16"
    B2_list: tuple  # fold ratios exercised
    K: int = 4      # depthwise conv width

    @property
    def L(self) -> int:
        return self.T + 2

    @property
    def token_channels(self) -> int:
        return self.B * self.D * self.L


WORKLOADS = {
    "tiny": Workload("tiny", B=4, D=16, N=4, T=8, io="f32", B2_list=(1, 2, 4)),
    "stage4": Workload("stage4", B=256, D=640, N=8, T=49, io="bf16", B2_list=(1, 2, 4, 8, 16, 32)),
    "stage3": Workload("stage3", B=256, D=320, N=8, T=196, io="bf16", B2_list=(1, 2, 4, 8)),
    "base_stage3": Workload("base_stage3", B=512, D=512, N=16, T=196, io="bf16",
                            B2_list=(1, 2, 4, 8, 16, 32, 64)),
    "long": Workload("long", B=16, D=320, N=16, T=4000, io="bf16", B2_list=(1,)),
}
WORKLOAD_ORDER = ("tiny", "stage4", "stage3", "base_stage3", "long")


@dataclasses.dataclass
class LayerInputs:
    """One scan layer's inputs.  io tensors are float32 arrays (f32 io) or uint16
    bf16 bit patterns (bf16 io); parameters are float32."""
    io: str
    x: np.ndarray          # [B, D, T] patch tokens (stage input, before the aux pad)
    delta: np.ndarray      # [B, D, L] raw step input (before bias and softplus)
    Bm: np.ndarray         # [B, N, L]
    Cm: np.ndarray         # [B, N, L]
    A: np.ndarray          # [D, N] float32
    Dskip: np.ndarray      # [D] float32
    delta_bias: np.ndarray  # [D] float32
    conv_w: np.ndarray     # [D, K] float32

    def as_f64(self, name: str) -> np.ndarray:
        a = getattr(self, name)
        if a.dtype == np.uint16:
            return bf16_bits_to_f64(a)
        return a.astype(np.float64)


def _io_cast(v64: np.ndarray, io: str) -> np.ndarray:
    v32 = v64.astype(np.float32)
    if io == "f32":
        return v32
    if io == "bf16":
        return f32_to_bf16_bits(v32)
    raise ValueError(f"unknown io dtype {io!r}")


def make_layer(w: Workload, seed: int, layer: int = 0, a_mode: str = "structured") -> LayerInputs:
    """Inputs of one layer.  ``layer`` selects independent draws for a second layer
    (streams are offset by 16 per layer); ``a_mode='random'`` gives the control A
    with a random per-(d, n) scale."""
    B, D, N, T, L, K = w.B, w.D, w.N, w.T, w.L, w.K
    off = 16 * layer
    x = _io_cast(normal(seed, STREAM_X + off, B * D * T), w.io).reshape(B, D, T)
    delta = _io_cast(normal(seed, STREAM_DELTA + off, B * D * L), w.io).reshape(B, D, L)
    Bm = _io_cast(normal(seed, STREAM_B + off, B * N * L), w.io).reshape(B, N, L)
    Cm = _io_cast(normal(seed, STREAM_C + off, B * N * L), w.io).reshape(B, N, L)
    # step-size bias: inverse softplus of a log-uniform draw in [1e-3, 1e-1]
    u = uniform53(seed, STREAM_DT0 + off, D)
    dt0 = np.exp(math.log(1e-3) + u * (math.log(1e-1) - math.log(1e-3)))
    delta_bias = np.log(np.expm1(dt0)).astype(np.float32)
    conv_w = (uniform53(seed, STREAM_CONVW + off, D * K) - 0.5).astype(np.float32).reshape(D, K)
    A = -np.tile(np.arange(1, N + 1, dtype=np.float64), (D, 1))
    if a_mode == "random":
        A = A * np.exp(0.5 * normal(seed, STREAM_ARAND + off, D * N)).reshape(D, N)
    elif a_mode != "structured":
        raise ValueError(a_mode)
    return LayerInputs(io=w.io, x=x, delta=delta, Bm=Bm, Cm=Cm, A=A.astype(np.float32),
                       Dskip=np.ones(D, dtype=np.float32), delta_bias=delta_bias, conv_w=conv_w)


# ---------------------------------------------------------------- mixer block
STREAM_BLOCK = 32  # first sub-stream of the mixer-block draws (independent of the layer draws)


class BlockInputs:
    """Random-weight mixer block around one scan layer, channel-last.  io arrays are
    float32 (f32 io) or uint16 bf16 bit patterns; A, Dskip, delta_bias, conv_w float32.

    X [B, L, C] is the (already padded) stage token sequence; W_x, W_z [C, D] give
    the scan input and the gate, W_b, W_c [C, N] give B and C, W_dt1 [C, R] and
    W_dt2 [R, D] the low-rank step input, W_out [D, C] the output projection.
    Weights are N(0, 1) / sqrt(fan_in)."""

    def __init__(self, **kw):
        self.__dict__.update(kw)


def make_block(B: int, T: int, C: int, D: int, N: int, K: int, R: int, io: str, seed: int) -> BlockInputs:
    L = T + 2
    s = STREAM_BLOCK
    g = lambda k, n, scale=1.0: normal(seed, s + k, n) * scale
    X = _io_cast(g(0, B * L * C), io).reshape(B, L, C)
    W = {}
    for k, (name, rows, cols) in enumerate([("W_x", C, D), ("W_z", C, D), ("W_b", C, N), ("W_c", C, N),
                                             ("W_dt1", C, R), ("W_dt2", R, D), ("W_out", D, C)]):
        W[name] = _io_cast(g(1 + k, rows * cols, 1.0 / math.sqrt(rows)), io).reshape(rows, cols)
    u = uniform53(seed, s + 8, D)
    dt0 = np.exp(math.log(1e-3) + u * (math.log(1e-1) - math.log(1e-3)))
    return BlockInputs(io=io, B=B, T=T, L=L, C=C, D=D, N=N, K=K, R=R, X=X, **W,
                       A=-np.tile(np.arange(1, N + 1, dtype=np.float32), (D, 1)),
                       Dskip=np.ones(D, dtype=np.float32),
                       delta_bias=np.log(np.expm1(dt0)).astype(np.float32),
                       conv_w=(uniform53(seed, s + 9, D * K) - 0.5).astype(np.float32).reshape(D, K))
