"""Seeded synthetic inputs for the attention-forward workloads.

This module holds no attention arithmetic: it only turns (seed, counter) pairs
into numbers, and names the workload shapes. Both the CPU oracle tests and the
GPU path consume its arrays as inputs.

Uniform source (pulsatrix HIPBackend page, ``dropout_forward`` note): the k-th
uniform of a seed is the SplitMix64 output for state ``seed + (k + 1) * gamma``
(gamma = 0x9E3779B97F4A7C15), keeping the top 24 bits as a float in [0, 1).
SplitMix64 is the generator of Steele, Lea and Flood (OOPSLA 2014).

Normals: Box-Muller in float64 on consecutive counter pairs, scaled by sigma,
rounded once to float32 (round to nearest even). bf16 inputs are a second
round-to-nearest-even step from that float32, which is how the oxicuda
``gemm_mixed_precision`` documentation describes emulating 16-bit storage.

Counter streams: tensor ``t`` (Q=0, K=1, V=2) draws counters ``t * 2**40 + n``.
"""
from __future__ import annotations

import ctypes
import dataclasses
import math
import os
import subprocess
from typing import Dict, Tuple

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_HERE, "libgen.so")
_lib = None


def build_native(force: bool = True) -> str:
    """Compile gen.c (host C, OpenMP) into gen/libgen.so."""
    if force or not os.path.exists(_LIB_PATH):
        tmp = _LIB_PATH + ".tmp%d" % os.getpid()
        subprocess.check_call(["gcc", "-O2", "-fopenmp", "-fPIC", "-shared",
                               os.path.join(_HERE, "gen.c"), "-o", tmp, "-lm"])
        os.replace(tmp, _LIB_PATH)
    return _LIB_PATH


def _native():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB_PATH):
            build_native(force=False)
        lib = ctypes.CDLL(_LIB_PATH)
        lib.gen_normal_f32.argtypes = [ctypes.c_uint64, ctypes.c_uint64, ctypes.c_int64,
                                       ctypes.c_double, ctypes.c_void_p]
        lib.gen_normal_f32.restype = None
        lib.gen_f32_to_bf16.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int64]
        lib.gen_f32_to_bf16.restype = None
        lib.gen_bf16_to_f32.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int64]
        lib.gen_bf16_to_f32.restype = None
        _lib = lib
    return _lib

GAMMA = np.uint64(0x9E3779B97F4A7C15)
_M1 = np.uint64(0xBF58476D1CE4E5B9)
_M2 = np.uint64(0x94D049BB133111EB)
STREAM_STRIDE = 1 << 40
TENSOR_STREAM = {"q": 0, "k": 1, "v": 2, "dout": 3, "mask": 4}

_CHUNK = 1 << 22  # elements per vectorised block; bounds temporaries to ~100 MB


def splitmix64(x: np.ndarray) -> np.ndarray:
    """SplitMix64 output function applied to state values ``x`` (uint64, wrapping)."""
    z = np.asarray(x, dtype=np.uint64).copy()
    with np.errstate(over="ignore"):
        z ^= z >> np.uint64(30)
        z *= _M1
        z ^= z >> np.uint64(27)
        z *= _M2
        z ^= z >> np.uint64(31)
    return z


def uniform24(seed: int, counters: np.ndarray) -> np.ndarray:
    """uniform(seed, k) for each counter k: top 24 bits of splitmix64(seed + (k+1)*gamma), in [0, 1)."""
    k = np.asarray(counters, dtype=np.uint64)
    with np.errstate(over="ignore"):
        state = np.uint64(seed & 0xFFFFFFFFFFFFFFFF) + (k + np.uint64(1)) * GAMMA
    z = splitmix64(state)
    return (z >> np.uint64(40)).astype(np.float64) * (1.0 / (1 << 24))


def normal_f64(seed: int, first_counter: int, n: int) -> np.ndarray:
    """n standard normals from counters [first_counter, first_counter + 2*ceil(n/2)).

    Pair p uses u1 = uniform(2p), u2 = uniform(2p+1); element 2p is
    sqrt(-2 ln(1-u1)) cos(2 pi u2) and element 2p+1 the matching sine.
    """
    out = np.empty(n, dtype=np.float64)
    npairs = (n + 1) // 2
    for p0 in range(0, npairs, _CHUNK):
        p1 = min(npairs, p0 + _CHUNK)
        idx = np.arange(p0, p1, dtype=np.uint64)
        base = np.uint64(first_counter) + np.uint64(2) * idx
        u1 = uniform24(seed, base)
        u2 = uniform24(seed, base + np.uint64(1))
        r = np.sqrt(-2.0 * np.log1p(-u1))
        th = (2.0 * math.pi) * u2
        e0 = 2 * p0
        e1 = min(n, 2 * p1)
        blk = np.empty(2 * (p1 - p0), dtype=np.float64)
        blk[0::2] = r * np.cos(th)
        blk[1::2] = r * np.sin(th)
        out[e0:e1] = blk[: e1 - e0]
    return out


def normal_f32(seed: int, first_counter: int, n: int, sigma: float) -> np.ndarray:
    """The same draws as ``(normal_f64(...) * sigma).astype(float32)``, computed by gen.c."""
    out = np.empty(n, dtype=np.float32)
    if n:
        _native().gen_normal_f32(seed & 0xFFFFFFFFFFFFFFFF, first_counter, n, float(sigma),
                                 out.ctypes.data)
    return out


def f32_to_bf16_bits_native(x: np.ndarray) -> np.ndarray:
    """gen.c's float32 -> bfloat16 rounding (same rule as ``f32_to_bf16_bits``)."""
    a = np.ascontiguousarray(x, dtype=np.float32)
    out = np.empty(a.shape, dtype=np.uint16)
    if a.size:
        _native().gen_f32_to_bf16(a.ctypes.data, out.ctypes.data, a.size)
    return out


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 values to bfloat16 (nearest, ties to even); returns uint16 bit patterns.

    NaN inputs map to a quiet NaN; infinities and overflow to infinity follow
    from the integer rounding of the bit pattern.
    """
    b = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32).astype(np.uint64)
    lsb = (b >> np.uint64(16)) & np.uint64(1)
    r = ((b + np.uint64(0x7FFF) + lsb) >> np.uint64(16)).astype(np.uint16)
    nan = np.isnan(np.asarray(x, dtype=np.float32))
    if nan.any():
        r = r.copy()
        r[nan] = np.uint16(0x7FC0)
    return r


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    """Exact widening of bfloat16 bit patterns to float32."""
    a = np.ascontiguousarray(b, dtype=np.uint16)
    out = np.empty(a.shape, dtype=np.float32)
    if a.size:
        _native().gen_bf16_to_f32(a.ctypes.data, out.ctypes.data, a.size)
    return out


def f32_to_f16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 values to IEEE binary16 (nearest, ties to even, numpy's conversion);
    returns uint16 bit patterns."""
    with np.errstate(over="ignore"):  # beyond the largest finite value: infinity, as IEEE rounds
        return np.ascontiguousarray(x, dtype=np.float32).astype(np.float16).view(np.uint16)


def f16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    """Exact widening of binary16 bit patterns to float32."""
    return np.ascontiguousarray(b, dtype=np.uint16).view(np.float16).astype(np.float32)


def to_16bit(x: np.ndarray, dtype: str):
    """(exact float32 values, uint16 bit patterns) of x rounded to the 16-bit type dtype."""
    if dtype == "bf16":
        b = f32_to_bf16_bits_native(x)
        return bf16_bits_to_f32(b), b
    if dtype == "f16":
        b = f32_to_f16_bits(x)
        return f16_bits_to_f32(b), b
    raise ValueError(f"not a 16-bit dtype: {dtype}")


def tensor_f32(seed: int, which: str, shape: Tuple[int, ...], sigma: float) -> np.ndarray:
    """A float32 tensor of N(0, sigma^2) draws for stream ``which`` in {"q","k","v","dout"}."""
    n = int(np.prod(shape, dtype=np.int64))
    return normal_f32(seed, TENSOR_STREAM[which] * STREAM_STRIDE, n, sigma).reshape(shape)


@dataclasses.dataclass(frozen=True)
class Workload:
    """One attention-forward workload: shapes, dtype, mask, scale and input distribution."""

    name: str
    dtype: str  # "f32", "bf16" or "f16" (input element type; accumulation and O are fp32)
    batch: int
    heads: int
    seq_q: int
    seq_kv: int
    head_dim: int
    causal: bool
    scale: float
    sigma_qk: float
    sigma_v: float
    seed: int

    @property
    def q_shape(self):
        return (self.batch, self.heads, self.seq_q, self.head_dim)

    @property
    def kv_shape(self):
        return (self.batch, self.heads, self.seq_kv, self.head_dim)


def _w(name, dtype, b, h, sq, skv, d, causal, scale, sqk, sv, seed):
    return Workload(name, dtype, b, h, sq, skv, d, causal, scale, sqk, sv, seed)


# The benchmark workload shapes, keyed by what they are: input dtype, mask,
# batch x heads, query/key lengths, head dim. The cross-attention shape runs
# both unmasked and with the bottom-right causal mask, on the same inputs.
WORKLOADS: Dict[str, Workload] = {w.name: w for w in (
    _w("f32_causal_b1h2_s128_d64", "f32", 1, 2, 128, 128, 64, True, 1.0 / 8.0, 1.0, 1.0, 20261202),
    _w("f32_b4h8_s512_d64", "f32", 4, 8, 512, 512, 64, False, 1.0 / math.sqrt(64), 1.0, 1.0, 20261203),
    _w("f32_causal_b8h16_s2048_d128", "f32", 8, 16, 2048, 2048, 128, True, 1.0 / math.sqrt(128), 1.0, 1.0, 20261204),
    _w("f32_cross_b2h32_q256_kv4096_d128", "f32", 2, 32, 256, 4096, 128, False, 1.0 / math.sqrt(128), 1.0, 1.0, 20261205),
    _w("f32_cross_causal_b2h32_q256_kv4096_d128", "f32", 2, 32, 256, 4096, 128, True, 1.0 / math.sqrt(128), 1.0, 1.0, 20261205),
    _w("bf16_causal_b1h32_s16384_d128", "bf16", 1, 32, 16384, 16384, 128, True, 1.0 / math.sqrt(128), 3.0, 1.0, 20261206),
    _w("f16_causal_b1h32_s16384_d128", "f16", 1, 32, 16384, 16384, 128, True, 1.0 / math.sqrt(128), 3.0, 1.0, 20261207),
    _w("f32_causal_b8h16_s2048_d32", "f32", 8, 16, 2048, 2048, 32, True, 1.0 / math.sqrt(32), 1.0, 1.0, 20261220),
    _w("f32_causal_b8h16_s2048_d256", "f32", 8, 16, 2048, 2048, 256, True, 1.0 / math.sqrt(256), 1.0, 1.0, 20261221),
    _w("bf16_causal_b1h32_s16384_d32", "bf16", 1, 32, 16384, 16384, 32, True, 1.0 / math.sqrt(32), 3.0, 1.0, 20261222),
    _w("bf16_causal_b1h32_s16384_d256", "bf16", 1, 32, 16384, 16384, 256, True, 1.0 / math.sqrt(256), 3.0, 1.0, 20261223),
)}


def make_inputs(w: Workload):
    """Host inputs for a workload.

    Returns (q, k, v) as float32 arrays holding the exact input values, plus,
    for 16-bit workloads, the uint16 bit patterns (qb, kb, vb) the device consumes.
    """
    q = tensor_f32(w.seed, "q", w.q_shape, w.sigma_qk)
    k = tensor_f32(w.seed, "k", w.kv_shape, w.sigma_qk)
    v = tensor_f32(w.seed, "v", w.kv_shape, w.sigma_v)
    if w.dtype == "f32":
        return (q, k, v), None
    pairs = [to_16bit(t, w.dtype) for t in (q, k, v)]
    return tuple(p[0] for p in pairs), tuple(p[1] for p in pairs)


@dataclasses.dataclass(frozen=True)
class RowWorkload:
    """A row-primitive workload: a (batch x rows x cols) fp32 score matrix and its op."""

    name: str
    op: str          # softmax_rows | logsumexp_rows | masked_softmax_rows | scaled_causal_softmax
                     # | softmax_rows_backward (x: the forward's scores; dy ~ N(0, 1))
    batch: int
    rows: int        # rows per matrix
    cols: int
    scale: float     # scaled_causal_softmax only
    causal: bool     # scaled_causal_softmax only
    sigma: float     # input scores ~ N(0, sigma^2)
    density: float   # masked_softmax_rows: probability that an entry is admitted
    seed: int


# Score matrices of the attention shapes (one row per query row of every head):
# the 4x8-head 512x512 shape and the 32-head 16384x16384 causal shape.
ROW_WORKLOADS: Dict[str, RowWorkload] = {w.name: w for w in (
    RowWorkload("softmax_rows_r16384_c512", "softmax_rows", 1, 16384, 512, 1.0, False, 4.0, 1.0, 20261211),
    RowWorkload("logsumexp_rows_r16384_c512", "logsumexp_rows", 1, 16384, 512, 1.0, False, 4.0, 1.0, 20261212),
    RowWorkload("masked_softmax_rows_r16384_c512", "masked_softmax_rows", 1, 16384, 512, 1.0, False, 4.0, 0.5, 20261213),
    RowWorkload("scaled_causal_softmax_b32_r512_c512", "scaled_causal_softmax", 32, 512, 512, 0.125, True, 4.0, 1.0, 20261214),
    RowWorkload("softmax_rows_r32768_c16384", "softmax_rows", 1, 32768, 16384, 1.0, False, 4.0, 1.0, 20261215),
    RowWorkload("scaled_causal_softmax_b2_r16384_c16384", "scaled_causal_softmax", 2, 16384, 16384,
                1.0 / math.sqrt(128), True, 4.0, 1.0, 20261216),
    RowWorkload("softmax_rows_backward_r16384_c512", "softmax_rows_backward", 1, 16384, 512, 1.0, False,
                4.0, 1.0, 20261217),
    RowWorkload("softmax_rows_backward_r32768_c16384", "softmax_rows_backward", 1, 32768, 16384, 1.0,
                False, 4.0, 1.0, 20261218),
)}


def make_row_inputs(w: RowWorkload):
    """(x, mask) for a row workload: x [batch*rows, cols] float32 (or [batch, rows, cols] for the
    scaled op); mask float32 of the same shape (1 admitted, 0 blocked) or None."""
    shape = (w.batch, w.rows, w.cols) if w.op == "scaled_causal_softmax" else (w.batch * w.rows, w.cols)
    x = tensor_f32(w.seed, "q", shape, w.sigma)
    mask = None
    if w.op == "masked_softmax_rows":
        n = int(np.prod(shape, dtype=np.int64))
        u = uniform24(w.seed, np.uint64(TENSOR_STREAM["k"] * STREAM_STRIDE) + np.arange(n, dtype=np.uint64))
        mask = (u < w.density).astype(np.float32).reshape(shape)
    return x, mask


def make_row_grad(w: RowWorkload) -> np.ndarray:
    """dL/dy for a softmax-backward row workload: float32 N(0, 1), the shape of its scores."""
    return tensor_f32(w.seed, "v", (w.batch * w.rows, w.cols), 1.0)


def random_case(seed: int, shape_q, shape_kv, sigma_qk=1.0, sigma_v=1.0, dtype="f32"):
    """Inputs for an ad-hoc (test) shape, from the same streams as ``make_inputs``."""
    q = tensor_f32(seed, "q", tuple(shape_q), sigma_qk)
    k = tensor_f32(seed, "k", tuple(shape_kv), sigma_qk)
    v = tensor_f32(seed, "v", tuple(shape_kv), sigma_v)
    if dtype == "f32":
        return (q, k, v), None
    pairs = [to_16bit(t, dtype) for t in (q, k, v)]
    return tuple(p[0] for p in pairs), tuple(p[1] for p in pairs)


def upstream_grad(seed: int, shape, sigma: float = 1.0) -> np.ndarray:
    """The upstream gradient dL/dO of a backward case: N(0, sigma^2) float32 on its own stream."""
    return tensor_f32(seed, "dout", tuple(shape), sigma)


def bernoulli_mask(seed: int, shape, density: float) -> np.ndarray:
    """A uint8 0/1 mask of the given shape: entry n is 1 iff uniform(seed, mask stream + n) < density."""
    n = int(np.prod(shape, dtype=np.int64))
    u = uniform24(seed, np.uint64(TENSOR_STREAM["mask"] * STREAM_STRIDE) + np.arange(n, dtype=np.uint64))
    return (u < density).astype(np.uint8).reshape(tuple(shape))
