"""Attention forward/backward and row-softmax oracle -- TEST INFRASTRUCTURE ONLY.

Plain double-precision CPU statements of the attention forward pass
(attention_oracle.c: the ``attention`` call of the oxicuda ComputeBackend page,
max-subtracted softmax and log-sum-exp as on the pulsatrix HIPBackend page,
and the empty-row convention of the TorchLean hard-masked softmax) and of the
row primitives on a materialised score matrix (rows_oracle.c: pulsatrix
``softmax_rows`` / ``logsumexp_rows``, the TorchLean hard-masked softmax and
MicroGPT's fused scale + causal mask + softmax), the gradients of the
attention forward (attention_bwd_oracle.c: the chain rule through the
softmax, recomputed from q, k, v and the upstream gradient), the forward
with an explicit hard mask (attention_masked_oracle.c: the TorchLean
hard-masked softmax inside the attention), and its gradients
(attention_bwd_masked_oracle.c: the same chain rule over each row's admitted
keys).

Only ``tests/``, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` may import this package. The attention library never does, and
the two share no code.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRCS = [os.path.join(_HERE, "attention_oracle.c"), os.path.join(_HERE, "rows_oracle.c"),
         os.path.join(_HERE, "attention_bwd_oracle.c"), os.path.join(_HERE, "attention_masked_oracle.c"),
         os.path.join(_HERE, "attention_bwd_masked_oracle.c")]
_LIB_PATH = os.path.join(_HERE, "liboracle.so")
_lib = None


def build(force: bool = True, out: str | None = None, defines=()) -> str:
    """Compile the oracle with gcc (host only). ``defines`` is for planted-mistake builds."""
    out = out or _LIB_PATH
    if force or not os.path.exists(out):
        tmp = out + ".tmp%d" % os.getpid()
        cmd = ["gcc", "-O2", "-fopenmp", "-fPIC", "-shared"] + ["-D" + d for d in defines]
        cmd += _SRCS + ["-o", tmp, "-lm"]
        subprocess.check_call(cmd)
        os.replace(tmp, out)
    return out


def _bind(lib):
    dp = ctypes.c_void_p
    L = ctypes.c_long
    lib.oracle_attention_fwd.argtypes = [dp, dp, dp, L, L, L, L, L, ctypes.c_double, ctypes.c_int,
                                         dp, L, dp, dp]
    lib.oracle_attention_fwd.restype = ctypes.c_int
    lib.oracle_attention_probs.argtypes = [dp, dp, L, L, L, ctypes.c_double, ctypes.c_int, dp]
    lib.oracle_attention_probs.restype = ctypes.c_int
    for name in ("oracle_softmax_rows", "oracle_logsumexp_rows"):
        getattr(lib, name).argtypes = [dp, L, L, dp]
        getattr(lib, name).restype = ctypes.c_int
    lib.oracle_masked_softmax_rows.argtypes = [dp, dp, L, L, dp]
    lib.oracle_masked_softmax_rows.restype = ctypes.c_int
    lib.oracle_softmax_rows_backward.argtypes = [dp, dp, L, L, ctypes.c_double, dp]
    lib.oracle_softmax_rows_backward.restype = ctypes.c_int
    lib.oracle_scaled_causal_softmax.argtypes = [dp, L, L, L, ctypes.c_double, ctypes.c_int, dp]
    lib.oracle_scaled_causal_softmax.restype = ctypes.c_int
    lib.oracle_attention_bwd.argtypes = [dp, dp, dp, dp, L, L, L, L, L, ctypes.c_double, ctypes.c_int,
                                         dp, dp, dp]
    lib.oracle_attention_bwd.restype = ctypes.c_int
    lib.oracle_attention_bwd_bound.argtypes = lib.oracle_attention_bwd.argtypes
    lib.oracle_attention_bwd_bound.restype = ctypes.c_int
    lib.oracle_attention_fwd_masked.argtypes = [dp, dp, dp, dp, L, L, L, L, L, L, L, ctypes.c_double,
                                                ctypes.c_int, dp, dp]
    lib.oracle_attention_fwd_masked.restype = ctypes.c_int
    for name in ("oracle_attention_bwd_masked", "oracle_attention_bwd_masked_bound"):
        getattr(lib, name).argtypes = [dp, dp, dp, dp, dp, L, L, L, L, L, L, L, ctypes.c_double,
                                       ctypes.c_int, dp, dp, dp]
        getattr(lib, name).restype = ctypes.c_int
    lib.oracle_num_threads.argtypes = []
    lib.oracle_num_threads.restype = ctypes.c_int
    return lib


def load(path: str | None = None):
    """The oracle library at ``path`` (default: the in-tree build, built if missing)."""
    global _lib
    if path is not None:
        return _bind(ctypes.CDLL(path))
    if _lib is None:
        if not os.path.exists(_LIB_PATH):
            build(force=False)
        _lib = _bind(ctypes.CDLL(_LIB_PATH))
    return _lib


def _f32(a):
    return np.ascontiguousarray(a, dtype=np.float32)


def attention_fwd(q, k, v, scale: float, causal: bool, rows=None, lib=None):
    """O and LSE in float64.

    q: [B,H,Sq,D]; k, v: [B,H,Skv,D] (values as float32, exact for bf16 inputs).
    rows: optional flat row ids (b*H + h)*Sq + i; then O is [len(rows), D] and LSE [len(rows)].
    """
    lib = lib or load()
    q, k, v = _f32(q), _f32(k), _f32(v)
    B, H, Sq, D = q.shape
    Skv = k.shape[2]
    assert k.shape == (B, H, Skv, D) and v.shape == (B, H, Skv, D)
    if rows is None:
        o = np.empty((B, H, Sq, D), dtype=np.float64)
        lse = np.empty((B, H, Sq), dtype=np.float64)
        rp, nr = None, 0
    else:
        rows = np.ascontiguousarray(rows, dtype=np.int64)
        o = np.empty((rows.size, D), dtype=np.float64)
        lse = np.empty((rows.size,), dtype=np.float64)
        rp, nr = rows.ctypes.data, rows.size
    rc = lib.oracle_attention_fwd(q.ctypes.data, k.ctypes.data, v.ctypes.data, B, H, Sq, Skv, D,
                                  float(scale), int(bool(causal)), rp, nr, o.ctypes.data,
                                  lse.ctypes.data)
    if rc != 0:
        raise ValueError("oracle_attention_fwd rejected its arguments")
    return o, lse


def softmax_probs(q_bh, k_bh, scale: float, causal: bool, lib=None):
    """P[i, j] for one (batch, head): q_bh [Sq, D], k_bh [Skv, D]."""
    lib = lib or load()
    q_bh, k_bh = _f32(q_bh), _f32(k_bh)
    Sq, D = q_bh.shape
    Skv = k_bh.shape[0]
    p = np.empty((Sq, Skv), dtype=np.float64)
    rc = lib.oracle_attention_probs(q_bh.ctypes.data, k_bh.ctypes.data, Sq, Skv, D, float(scale),
                                    int(bool(causal)), p.ctypes.data)
    if rc != 0:
        raise ValueError("oracle_attention_probs rejected its arguments")
    return p


def attention_bwd(q, k, v, dout, scale: float, causal: bool, lib=None):
    """dQ, dK, dV (float64) of the attention forward for upstream gradient dout = dL/dO."""
    lib = lib or load()
    q, k, v, dout = _f32(q), _f32(k), _f32(v), _f32(dout)
    B, H, Sq, D = q.shape
    Skv = k.shape[2]
    assert k.shape == (B, H, Skv, D) and v.shape == (B, H, Skv, D) and dout.shape == q.shape
    dq = np.empty(q.shape, dtype=np.float64)
    dk = np.empty(k.shape, dtype=np.float64)
    dv = np.empty(v.shape, dtype=np.float64)
    rc = lib.oracle_attention_bwd(q.ctypes.data, k.ctypes.data, v.ctypes.data, dout.ctypes.data, B, H,
                                  Sq, Skv, D, float(scale), int(bool(causal)), dq.ctypes.data,
                                  dk.ctypes.data, dv.ctypes.data)
    if rc != 0:
        raise ValueError("oracle_attention_bwd rejected its arguments")
    return dq, dk, dv


def attention_bwd_bound(q, k, v, dout, scale: float, causal: bool, lib=None):
    """Error scale (mq, mk, mv) of the gradients: their sums with every factor in magnitude."""
    lib = lib or load()
    q, k, v, dout = _f32(q), _f32(k), _f32(v), _f32(dout)
    B, H, Sq, D = q.shape
    Skv = k.shape[2]
    assert k.shape == (B, H, Skv, D) and v.shape == (B, H, Skv, D) and dout.shape == q.shape
    mq = np.empty(q.shape, dtype=np.float64)
    mk = np.empty(k.shape, dtype=np.float64)
    mv = np.empty(v.shape, dtype=np.float64)
    rc = lib.oracle_attention_bwd_bound(q.ctypes.data, k.ctypes.data, v.ctypes.data, dout.ctypes.data,
                                        B, H, Sq, Skv, D, float(scale), int(bool(causal)),
                                        mq.ctypes.data, mk.ctypes.data, mv.ctypes.data)
    if rc != 0:
        raise ValueError("oracle_attention_bwd_bound rejected its arguments")
    return mq, mk, mv


def attention_fwd_masked(q, k, v, mask, scale: float, causal: bool, lib=None):
    """O and LSE (float64) with a hard mask: mask is [B or 1, H or 1, Sq, Skv], nonzero admits
    (combined with the causal bound when causal)."""
    lib = lib or load()
    q, k, v = _f32(q), _f32(k), _f32(v)
    B, H, Sq, D = q.shape
    Skv = k.shape[2]
    assert k.shape == (B, H, Skv, D) and v.shape == (B, H, Skv, D)
    m = np.ascontiguousarray(np.asarray(mask) != 0, dtype=np.uint8)
    if m.ndim != 4 or m.shape[2:] != (Sq, Skv) or m.shape[0] not in (1, B) or m.shape[1] not in (1, H):
        raise ValueError(f"mask shape {m.shape} does not broadcast to {(B, H, Sq, Skv)}")
    sh = Sq * Skv if m.shape[1] == H else 0
    sb = m.shape[1] * Sq * Skv if m.shape[0] == B else 0
    o = np.empty((B, H, Sq, D), dtype=np.float64)
    lse = np.empty((B, H, Sq), dtype=np.float64)
    rc = lib.oracle_attention_fwd_masked(q.ctypes.data, k.ctypes.data, v.ctypes.data, m.ctypes.data,
                                         sb, sh, B, H, Sq, Skv, D, float(scale), int(bool(causal)),
                                         o.ctypes.data, lse.ctypes.data)
    if rc != 0:
        raise ValueError("oracle_attention_fwd_masked rejected its arguments")
    return o, lse


def _mask_bytes(mask, B, H, Sq, Skv):
    """The mask as contiguous 0/1 bytes and its (batch, head) strides (0 broadcasts)."""
    m = np.ascontiguousarray(np.asarray(mask) != 0, dtype=np.uint8)
    if m.ndim != 4 or m.shape[2:] != (Sq, Skv) or m.shape[0] not in (1, B) or m.shape[1] not in (1, H):
        raise ValueError(f"mask shape {m.shape} does not broadcast to {(B, H, Sq, Skv)}")
    sh = Sq * Skv if m.shape[1] == H else 0
    sb = m.shape[1] * Sq * Skv if m.shape[0] == B else 0
    return m, sb, sh


def _bwd_masked_call(fn, q, k, v, dout, mask, scale, causal, lib):
    lib = lib or load()
    q, k, v, dout = _f32(q), _f32(k), _f32(v), _f32(dout)
    B, H, Sq, D = q.shape
    Skv = k.shape[2]
    assert k.shape == (B, H, Skv, D) and v.shape == (B, H, Skv, D) and dout.shape == q.shape
    m, sb, sh = _mask_bytes(mask, B, H, Sq, Skv)
    a = np.empty(q.shape, dtype=np.float64)
    b = np.empty(k.shape, dtype=np.float64)
    c = np.empty(v.shape, dtype=np.float64)
    rc = getattr(lib, fn)(q.ctypes.data, k.ctypes.data, v.ctypes.data, dout.ctypes.data, m.ctypes.data,
                          sb, sh, B, H, Sq, Skv, D, float(scale), int(bool(causal)), a.ctypes.data,
                          b.ctypes.data, c.ctypes.data)
    if rc != 0:
        raise ValueError(f"{fn} rejected its arguments")
    return a, b, c


def attention_bwd_masked(q, k, v, dout, mask, scale: float, causal: bool, lib=None):
    """dQ, dK, dV (float64) of the hard-masked forward (mask as attention_fwd_masked takes it)."""
    return _bwd_masked_call("oracle_attention_bwd_masked", q, k, v, dout, mask, scale, causal, lib)


def attention_bwd_masked_bound(q, k, v, dout, mask, scale: float, causal: bool, lib=None):
    """Error scale (mq, mk, mv) of the masked gradients, as attention_bwd_bound over the admitted pairs."""
    return _bwd_masked_call("oracle_attention_bwd_masked_bound", q, k, v, dout, mask, scale, causal, lib)


def _rows2d(x):
    x = _f32(x)
    if x.ndim != 2:
        raise ValueError("expected a (rows, cols) matrix")
    return x


def softmax_rows(x, lib=None):
    """Row softmax of a (rows, cols) matrix, float64."""
    lib = lib or load()
    x = _rows2d(x)
    out = np.empty(x.shape, dtype=np.float64)
    if lib.oracle_softmax_rows(x.ctypes.data, x.shape[0], x.shape[1], out.ctypes.data) != 0:
        raise ValueError("oracle_softmax_rows rejected its arguments")
    return out


def logsumexp_rows(x, lib=None):
    """Per-row natural-log log-sum-exp of a (rows, cols) matrix, float64 [rows]."""
    lib = lib or load()
    x = _rows2d(x)
    out = np.empty((x.shape[0],), dtype=np.float64)
    if lib.oracle_logsumexp_rows(x.ctypes.data, x.shape[0], x.shape[1], out.ctypes.data) != 0:
        raise ValueError("oracle_logsumexp_rows rejected its arguments")
    return out


def softmax_rows_backward(y, dy, scale: float = 1.0, lib=None):
    """dx = scale * y * (dy - rowsum(y * dy)) in float64, from the softmax output y and dL/dy."""
    lib = lib or load()
    y, dy = _rows2d(y), _rows2d(dy)
    if y.shape != dy.shape:
        raise ValueError("y and dy differ in shape")
    out = np.empty(y.shape, dtype=np.float64)
    if lib.oracle_softmax_rows_backward(y.ctypes.data, dy.ctypes.data, y.shape[0], y.shape[1],
                                        float(scale), out.ctypes.data) != 0:
        raise ValueError("oracle_softmax_rows_backward rejected its arguments")
    return out


def masked_softmax_rows(x, mask, lib=None):
    """Hard-masked row softmax: entries with mask != 0 are admitted."""
    lib = lib or load()
    x, mask = _rows2d(x), _rows2d(mask)
    if mask.shape != x.shape:
        raise ValueError("mask shape differs")
    out = np.empty(x.shape, dtype=np.float64)
    if lib.oracle_masked_softmax_rows(x.ctypes.data, mask.ctypes.data, x.shape[0], x.shape[1],
                                      out.ctypes.data) != 0:
        raise ValueError("oracle_masked_softmax_rows rejected its arguments")
    return out


def scaled_causal_softmax(x, scale: float, causal: bool, lib=None):
    """softmax(scale * x) per row of each (rows, cols) matrix of x [batch, rows, cols], with the
    bottom-right causal mask when causal."""
    lib = lib or load()
    x = _f32(x)
    if x.ndim != 3:
        raise ValueError("expected a (batch, rows, cols) array")
    out = np.empty(x.shape, dtype=np.float64)
    if lib.oracle_scaled_causal_softmax(x.ctypes.data, x.shape[0], x.shape[1], x.shape[2],
                                        float(scale), int(bool(causal)), out.ctypes.data) != 0:
        raise ValueError("oracle_scaled_causal_softmax rejected its arguments")
    return out


def num_threads(lib=None) -> int:
    return int((lib or load()).oracle_num_threads())
