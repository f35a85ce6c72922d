"""Scaled masked attention forward for MI355X (gfx950).

A thin ctypes binding over libsma.so (C ABI in include/sma.h). This module only
marshals arguments: torch provides device memory and the current stream, and
every step of the computation runs in the library's HIP kernels. If the
library has not been built, importing works but every call raises.
"""
from __future__ import annotations

import ctypes
import math
import os

PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(PKG, "libsma.so")

SMA_DTYPE_F32 = 0
SMA_DTYPE_BF16 = 1
SMA_DTYPE_F16 = 2
SMA_LAYOUT_BHSD = 0
SMA_LAYOUT_BSHD = 1
LAYOUTS = {"bhsd": SMA_LAYOUT_BHSD, "bshd": SMA_LAYOUT_BSHD}
SMA_OK = 0
SMA_KERNEL_AUTO = -1
SMA_KERNEL_F32_QBLOCK = 0
SMA_KERNEL_F32_KSPLIT = 1
SMA_KERNEL_BF16_QBLOCK = 2
KERNEL_NAMES = {SMA_KERNEL_F32_QBLOCK: "f32_qblock", SMA_KERNEL_F32_KSPLIT: "f32_ksplit",
                SMA_KERNEL_BF16_QBLOCK: "bf16_qblock"}
STATUS_NAMES = {0: "SMA_OK", 1: "SMA_ERR_NULL_POINTER", 2: "SMA_ERR_INVALID_VALUE",
                3: "SMA_ERR_UNSUPPORTED", 4: "SMA_ERR_MISALIGNED", 5: "SMA_ERR_ALIASING",
                6: "SMA_ERR_HIP", 7: "SMA_ERR_SCRATCH"}
SMA_ERR_NULL_POINTER = 1
SMA_ERR_INVALID_VALUE = 2
SMA_ERR_UNSUPPORTED = 3
SMA_ERR_MISALIGNED = 4
SMA_ERR_ALIASING = 5
SMA_ERR_HIP = 6
SMA_ERR_SCRATCH = 7
NOALLOC_SCRATCH_BYTES = 72 * 1024 * 1024  # SMA_NOALLOC_SCRATCH_BYTES

_lib = None


class Plan(ctypes.Structure):
    """struct sma_plan: kernel, key splits, workgroups, workspace bytes."""
    _fields_ = [("kernel", ctypes.c_int), ("nsplit", ctypes.c_int),
                ("workgroups", ctypes.c_size_t), ("workspace_bytes", ctypes.c_size_t)]

    def __repr__(self):
        return (f"Plan(kernel={KERNEL_NAMES.get(self.kernel, self.kernel)}, nsplit={self.nsplit}, "
                f"workgroups={self.workgroups}, workspace_bytes={self.workspace_bytes})")


class SMAError(RuntimeError):
    """A non-zero status from libsma."""

    def __init__(self, status: int, message: str):
        super().__init__(message)
        self.status = status


def library():
    """The loaded libsma (raises if it was never built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it with "
                               "`python -m scaled_masked_attention_amd.build` (hipcc, gfx950)")
        lib = ctypes.CDLL(LIB_PATH)
        vp, sz = ctypes.c_void_p, ctypes.c_size_t
        lib.sma_attention_fwd.argtypes = [vp, vp, vp, vp, vp, ctypes.c_int, ctypes.c_int, sz, sz,
                                          sz, sz, sz, ctypes.c_double, ctypes.c_int, vp, sz, vp]
        lib.sma_attention_fwd.restype = ctypes.c_int
        lib.sma_attention_fwd_timed.argtypes = lib.sma_attention_fwd.argtypes + [vp, vp]
        lib.sma_attention_fwd_timed.restype = ctypes.c_int
        lib.sma_attention_fwd_validate.argtypes = [vp, vp, vp, vp, vp, ctypes.c_int, ctypes.c_int,
                                                   sz, sz, sz, sz, sz, ctypes.c_double,
                                                   ctypes.c_int, vp, sz]
        lib.sma_attention_fwd_validate.restype = ctypes.c_int
        lib.sma_attention_fwd_workspace_bytes.argtypes = [ctypes.c_int, sz, sz, sz, sz, sz,
                                                          ctypes.c_int]
        lib.sma_attention_fwd_workspace_bytes.restype = sz
        lib.sma_attention_fwd_plan.argtypes = [ctypes.c_int, sz, sz, sz, sz, sz, ctypes.c_int,
                                               ctypes.c_int, ctypes.c_int, ctypes.c_int,
                                               ctypes.c_int, ctypes.POINTER(Plan)]
        lib.sma_attention_fwd_plan.restype = ctypes.c_int
        fwd = lib.sma_attention_fwd.argtypes
        lib.sma_attention_fwd_ex.argtypes = (fwd[:14] + [ctypes.c_int] + fwd[14:16] +
                                             [ctypes.POINTER(Plan), vp, vp, vp])
        lib.sma_attention_fwd_ex.restype = ctypes.c_int
        lib.sma_attention_fwd_layout.argtypes = fwd[:14] + [ctypes.c_int] + fwd[14:17]
        lib.sma_attention_fwd_layout.restype = ctypes.c_int
        lib.sma_attention_fwd_noalloc.argtypes = fwd[:14] + [ctypes.c_int, ctypes.POINTER(Plan), vp]
        lib.sma_attention_fwd_noalloc.restype = ctypes.c_int
        lib.sma_attention_fwd_masked.argtypes = (fwd[:5] + [vp, sz, sz] + fwd[5:14] + [ctypes.c_int] +
                                                 fwd[14:16] + [ctypes.POINTER(Plan), vp, vp, vp])
        lib.sma_attention_fwd_masked.restype = ctypes.c_int
        lib.sma_attention_fwd_masked_workspace_bytes.argtypes = [ctypes.c_int, sz, sz, sz, sz, sz,
                                                                 ctypes.c_int, ctypes.c_int, sz, sz]
        lib.sma_attention_fwd_masked_workspace_bytes.restype = sz
        fp = ctypes.c_void_p
        lib.sma_softmax_rows.argtypes = [fp, fp, sz, sz, vp]
        lib.sma_logsumexp_rows.argtypes = [fp, fp, sz, sz, vp]
        lib.sma_masked_softmax_rows.argtypes = [fp, fp, fp, sz, sz, vp]
        lib.sma_scaled_causal_softmax.argtypes = [fp, fp, sz, sz, sz, ctypes.c_double, ctypes.c_int, vp]
        lib.sma_softmax_rows_backward.argtypes = [fp, fp, fp, sz, sz, ctypes.c_double, vp]
        for n in ("sma_softmax_rows", "sma_logsumexp_rows", "sma_masked_softmax_rows",
                  "sma_scaled_causal_softmax", "sma_softmax_rows_backward"):
            getattr(lib, n).restype = ctypes.c_int
        bwd = [vp] * 9 + [ctypes.c_int, sz, sz, sz, sz, sz, ctypes.c_double, ctypes.c_int, vp, sz, vp]
        lib.sma_attention_bwd.argtypes = bwd
        lib.sma_attention_bwd.restype = ctypes.c_int
        lib.sma_attention_bwd_timed.argtypes = bwd + [vp, vp]
        lib.sma_attention_bwd_timed.restype = ctypes.c_int
        lib.sma_attention_bwd_layout.argtypes = bwd[:17] + [ctypes.c_int] + bwd[17:]
        lib.sma_attention_bwd_layout.restype = ctypes.c_int
        lib.sma_attention_bwd_masked.argtypes = bwd[:9] + [vp, sz, sz] + bwd[9:17] + [ctypes.c_int] + bwd[17:]
        lib.sma_attention_bwd_masked.restype = ctypes.c_int
        lib.sma_attention_bwd_masked_workspace_bytes.argtypes = [ctypes.c_int, sz, sz, sz, sz, sz,
                                                                 ctypes.c_int, ctypes.c_int, sz, sz]
        lib.sma_attention_bwd_masked_workspace_bytes.restype = sz
        lib.sma_attention_bwd_workspace_bytes.argtypes = [ctypes.c_int, sz, sz, sz, sz, sz, ctypes.c_int]
        lib.sma_attention_bwd_workspace_bytes.restype = sz
        lib.sma_status_string.argtypes = [ctypes.c_int]
        lib.sma_status_string.restype = ctypes.c_char_p
        lib.sma_abi_version.argtypes = []
        lib.sma_abi_version.restype = ctypes.c_int
        _lib = lib
    return _lib


def status_string(status: int) -> str:
    return library().sma_status_string(int(status)).decode()


def abi_version() -> int:
    return int(library().sma_abi_version())


def _raise(st: int):
    if st != SMA_OK:
        raise SMAError(st, status_string(st))


def workspace_bytes(in_dtype: int, batch: int, heads: int, seq_q: int, seq_kv: int,
                    head_dim: int, causal: bool, num_cus: int = 0, layout: str = "bhsd") -> int:
    """Workspace that enables the library's key split (0: it never splits this shape, or
    the arguments are invalid). With the defaults this is sma_attention_fwd_workspace_bytes;
    another CU count or the [B,S,H,d] layout goes through sma_attention_fwd_plan."""
    if num_cus == 0 and layout == "bhsd":
        return int(library().sma_attention_fwd_workspace_bytes(in_dtype, batch, heads, seq_q,
                                                               seq_kv, head_dim, int(bool(causal))))
    try:
        return int(plan(in_dtype, batch, heads, seq_q, seq_kv, head_dim, causal, num_cus=num_cus,
                        layout=layout).workspace_bytes)
    except SMAError:
        return 0


def plan(in_dtype: int, batch: int, heads: int, seq_q: int, seq_kv: int, head_dim: int,
         causal: bool, kernel: int = SMA_KERNEL_AUTO, nsplit: int = 0, num_cus: int = 0,
         layout: str = "bhsd") -> Plan:
    """sma_attention_fwd_plan: the kernel, split and workspace a call would use."""
    if layout not in LAYOUTS:
        raise ValueError(f"layout must be one of {sorted(LAYOUTS)}")
    out = Plan()
    _raise(library().sma_attention_fwd_plan(in_dtype, batch, heads, seq_q, seq_kv, head_dim,
                                            int(bool(causal)), LAYOUTS[layout], kernel, nsplit,
                                            num_cus, ctypes.byref(out)))
    return out


def validate(q_ptr, k_ptr, v_ptr, o_ptr, lse_ptr, in_dtype, o_dtype, batch, heads, seq_q, seq_kv,
             head_dim, scale, causal, ws_ptr=None, ws_bytes=0) -> int:
    """Host-only argument check on raw integer addresses (no HIP call); returns the status."""
    return int(library().sma_attention_fwd_validate(q_ptr, k_ptr, v_ptr, o_ptr, lse_ptr, in_dtype,
                                                    o_dtype, batch, heads, seq_q, seq_kv, head_dim,
                                                    float(scale), int(bool(causal)), ws_ptr,
                                                    ws_bytes))


def attention_fwd_raw(q_ptr, k_ptr, v_ptr, o_ptr, lse_ptr, in_dtype, o_dtype, batch, heads,
                      seq_q, seq_kv, head_dim, scale, causal, ws_ptr, ws_bytes, stream) -> None:
    """sma_attention_fwd on raw addresses; raises SMAError on a non-zero status."""
    _raise(library().sma_attention_fwd(q_ptr, k_ptr, v_ptr, o_ptr, lse_ptr, in_dtype, o_dtype,
                                       batch, heads, seq_q, seq_kv, head_dim, float(scale),
                                       int(bool(causal)), ws_ptr, ws_bytes, stream))


def attention_fwd_timed_raw(q_ptr, k_ptr, v_ptr, o_ptr, lse_ptr, in_dtype, o_dtype, batch, heads,
                            seq_q, seq_kv, head_dim, scale, causal, ws_ptr, ws_bytes, stream,
                            event_before, event_after) -> None:
    """sma_attention_fwd_timed: also records two caller-owned hipEvent_t around the main kernel."""
    _raise(library().sma_attention_fwd_timed(q_ptr, k_ptr, v_ptr, o_ptr, lse_ptr, in_dtype,
                                             o_dtype, batch, heads, seq_q, seq_kv, head_dim,
                                             float(scale), int(bool(causal)), ws_ptr, ws_bytes,
                                             stream, event_before, event_after))


def attention_fwd_ex_raw(q_ptr, k_ptr, v_ptr, o_ptr, lse_ptr, in_dtype, o_dtype, batch, heads,
                         seq_q, seq_kv, head_dim, scale, causal, ws_ptr, ws_bytes, plan_, stream,
                         event_before=None, event_after=None, layout=SMA_LAYOUT_BHSD) -> None:
    """sma_attention_fwd_ex: explicit plan (a Plan, or None for the library's choice) and layout."""
    _raise(library().sma_attention_fwd_ex(q_ptr, k_ptr, v_ptr, o_ptr, lse_ptr, in_dtype, o_dtype,
                                          batch, heads, seq_q, seq_kv, head_dim, float(scale),
                                          int(bool(causal)), int(layout), ws_ptr, ws_bytes,
                                          ctypes.byref(plan_) if plan_ is not None else None,
                                          stream, event_before, event_after))


def attention_fwd_noalloc_raw(q_ptr, k_ptr, v_ptr, o_ptr, lse_ptr, in_dtype, o_dtype, batch, heads,
                              seq_q, seq_kv, head_dim, scale, causal, plan_, stream,
                              layout=SMA_LAYOUT_BHSD) -> None:
    """sma_attention_fwd_noalloc: no workspace argument, nothing allocated (the key split uses
    the library's device scratch); plan_ a Plan or None. Raises SMAError."""
    _raise(library().sma_attention_fwd_noalloc(q_ptr, k_ptr, v_ptr, o_ptr, lse_ptr, in_dtype,
                                               o_dtype, batch, heads, seq_q, seq_kv, head_dim,
                                               float(scale), int(bool(causal)), int(layout),
                                               ctypes.byref(plan_) if plan_ is not None else None,
                                               stream))


def attention_fwd_masked_raw(q_ptr, k_ptr, v_ptr, o_ptr, lse_ptr, mask_ptr, mask_batches, mask_heads,
                             in_dtype, o_dtype, batch, heads, seq_q, seq_kv, head_dim, scale, causal,
                             layout, ws_ptr, ws_bytes, plan_, stream, event_before=None,
                             event_after=None) -> None:
    """sma_attention_fwd_masked on raw addresses; raises SMAError on a non-zero status."""
    _raise(library().sma_attention_fwd_masked(q_ptr, k_ptr, v_ptr, o_ptr, lse_ptr, mask_ptr,
                                              mask_batches, mask_heads, in_dtype, o_dtype, batch,
                                              heads, seq_q, seq_kv, head_dim, float(scale),
                                              int(bool(causal)), int(layout), ws_ptr, ws_bytes,
                                              ctypes.byref(plan_) if plan_ is not None else None,
                                              stream, event_before, event_after))


def attention_fwd(q, k, v, scale=None, causal=False, return_lse=False, out=None, lse=None,
                  workspace=None, stream=None, kernel=None, nsplit=0, out_dtype=None, layout="bhsd",
                  mask=None):
    """O = softmax(scale * Q K^T + mask) V on the GPU.

    q [B,H,Sq,D], k and v [B,H,Skv,D]: contiguous torch tensors on the current
    HIP device, all float32, all bfloat16 or all float16. Returns O ([B,H,Sq,D], float32, or
    bfloat16 / float16 rounded to nearest even with out_dtype=torch.bfloat16 /
    torch.float16 or an ``out`` of that dtype) and, with return_lse, the per-row natural-log LSE
    (float32, [B,H,Sq]).
    scale=None means 1/sqrt(D). causal uses the bottom-right alignment.
    layout="bshd" takes q [B,Sq,H,D], k and v [B,Skv,H,D] and returns O in that
    layout (LSE stays [B,H,Sq]). mask: a bool or uint8 tensor [Sq,Skv] or
    [B or 1, H or 1, Sq, Skv] on the device; key j is admitted to row i only
    where it is nonzero (and, with causal, under the causal bound too).
    kernel (an SMA_KERNEL_* code) and nsplit force a plan; by default the
    library chooses. A forced split gets a workspace of the size it needs.
    stream: the torch.cuda.Stream to launch on (default: the current stream); the
    outputs and workspace allocated here are allocated on it.
    """
    import torch

    if stream is None:
        stream = torch.cuda.current_stream()
    # Outputs and workspace are allocated on the launch stream: the caching
    # allocator then never hands their blocks to other work while the kernels
    # still use them, whichever stream the caller launches on.
    with torch.cuda.stream(stream):
        return _attention_fwd(q, k, v, scale, causal, return_lse, out, lse, workspace, stream,
                              kernel, nsplit, out_dtype, layout, mask)


def _attention_fwd(q, k, v, scale, causal, return_lse, out, lse, workspace, stream, kernel, nsplit,
                   out_dtype, layout, mask):
    import torch

    if not (isinstance(q, torch.Tensor) and isinstance(k, torch.Tensor) and isinstance(v, torch.Tensor)):
        raise TypeError("q, k, v must be torch tensors")
    if q.dim() != 4 or k.dim() != 4 or v.dim() != 4:
        raise ValueError("q, k, v must be 4-D [batch, heads, seq, head_dim]")
    if layout not in LAYOUTS:
        raise ValueError(f"layout must be one of {sorted(LAYOUTS)}")
    bshd = layout == "bshd"
    if bshd:
        B, Sq, H, D = q.shape
        Skv = k.shape[1]
        kv_shape, o_shape = (B, Skv, H, D), (B, Sq, H, D)
    else:
        B, H, Sq, D = q.shape
        Skv = k.shape[2]
        kv_shape, o_shape = (B, H, Skv, D), (B, H, Sq, D)
    if tuple(k.shape) != kv_shape or tuple(v.shape) != kv_shape:
        raise ValueError(f"shape mismatch: q {tuple(q.shape)}, k {tuple(k.shape)}, v {tuple(v.shape)}")
    if not (q.dtype == k.dtype == v.dtype):
        raise ValueError("q, k, v must share one dtype")
    if q.dtype == torch.float32:
        in_dt = SMA_DTYPE_F32
    elif q.dtype == torch.bfloat16:
        in_dt = SMA_DTYPE_BF16
    elif q.dtype == torch.float16:
        in_dt = SMA_DTYPE_F16
    else:
        raise ValueError(f"unsupported dtype {q.dtype}")
    dev = torch.device("cuda", torch.cuda.current_device())
    for name, t in (("q", q), ("k", k), ("v", v)):
        if t.device != dev:
            raise ValueError(f"{name} is on {t.device}, the current HIP device is {dev}")
        if not t.is_contiguous():
            raise ValueError(f"{name} must be contiguous")
    if scale is None:
        scale = 1.0 / math.sqrt(D)
    if out_dtype is None:
        out_dtype = out.dtype if out is not None else torch.float32
    if out_dtype not in (torch.float32, torch.bfloat16, torch.float16):
        raise ValueError(f"unsupported out_dtype {out_dtype}")
    o_dt = {torch.float32: SMA_DTYPE_F32, torch.bfloat16: SMA_DTYPE_BF16,
            torch.float16: SMA_DTYPE_F16}[out_dtype]
    if out is None:
        out = torch.empty(o_shape, dtype=out_dtype, device=dev)
    if return_lse and lse is None:
        lse = torch.empty((B, H, Sq), dtype=torch.float32, device=dev)
    if out.device != dev or out.dtype != out_dtype or not out.is_contiguous():
        raise ValueError(f"out must be a contiguous {out_dtype} tensor on {dev}")
    if lse is not None and (lse.device != dev or lse.dtype != torch.float32 or not lse.is_contiguous()):
        raise ValueError(f"lse must be a contiguous float32 tensor on {dev}")
    if tuple(out.shape) != o_shape or (lse is not None and lse.shape != (B, H, Sq)):
        raise ValueError("out/lse shape mismatch")
    forced = None
    if kernel is not None and kernel != SMA_KERNEL_AUTO:
        forced = plan(in_dt, B, H, Sq, Skv, D, causal, kernel, nsplit, layout=layout)
        need = forced.workspace_bytes
    else:
        need = 0 if mask is not None else workspace_bytes(in_dt, B, H, Sq, Skv, D, causal,
                                                          layout=layout)
    if mask is not None:
        if not isinstance(mask, torch.Tensor) or mask.dtype not in (torch.bool, torch.uint8):
            raise ValueError("mask must be a bool or uint8 torch tensor")
        if mask.dim() == 2:
            mask = mask.view(1, 1, *mask.shape)
        if (mask.dim() != 4 or tuple(mask.shape[2:]) != (Sq, Skv) or mask.shape[0] not in (1, B)
                or mask.shape[1] not in (1, H)):
            raise ValueError(f"mask shape {tuple(mask.shape)} does not broadcast to {(B, H, Sq, Skv)}")
        if mask.device != dev or not mask.is_contiguous():
            raise ValueError(f"mask must be a contiguous tensor on {dev}")
        mb, mh = mask.shape[0], mask.shape[1]
        need += library().sma_attention_fwd_masked_workspace_bytes(in_dt, B, H, Sq, Skv, D,
                                                                   int(bool(causal)),
                                                                   LAYOUTS[layout], mb, mh)
    if workspace is None and need > 0:
        workspace = torch.empty(need, dtype=torch.uint8, device=dev)
    ws_ptr = workspace.data_ptr() if workspace is not None else None
    ws_bytes = workspace.numel() * workspace.element_size() if workspace is not None else 0
    if stream is None:
        stream = torch.cuda.current_stream()
    if mask is not None:
        attention_fwd_masked_raw(q.data_ptr(), k.data_ptr() if Skv else None,
                                 v.data_ptr() if Skv else None, out.data_ptr(),
                                 lse.data_ptr() if lse is not None else None,
                                 mask.data_ptr() if mask.numel() else None, mb, mh, in_dt, o_dt, B, H,
                                 Sq, Skv, D, scale, causal, LAYOUTS[layout], ws_ptr, ws_bytes, forced,
                                 stream.cuda_stream)
    else:
        attention_fwd_ex_raw(q.data_ptr(), k.data_ptr() if Skv else None, v.data_ptr() if Skv else None,
                             out.data_ptr(), lse.data_ptr() if lse is not None else None, in_dt,
                             o_dt, B, H, Sq, Skv, D, scale, causal, ws_ptr, ws_bytes, forced,
                             stream.cuda_stream, layout=LAYOUTS[layout])
    return (out, lse) if return_lse else out


# ------------------------------------------------------------------ backward
def attention_bwd_workspace_bytes(in_dtype: int, batch: int, heads: int, seq_q: int, seq_kv: int,
                                  head_dim: int, causal: bool) -> int:
    return library().sma_attention_bwd_workspace_bytes(in_dtype, batch, heads, seq_q, seq_kv,
                                                       head_dim, int(bool(causal)))


def attention_bwd_raw(q_ptr, k_ptr, v_ptr, o_ptr, lse_ptr, dout_ptr, dq_ptr, dk_ptr, dv_ptr,
                      in_dtype, batch, heads, seq_q, seq_kv, head_dim, scale, causal, ws_ptr,
                      ws_bytes, stream, event_after_pre=None, event_after_dkdv=None) -> None:
    """sma_attention_bwd_timed on raw addresses (events may be None); raises SMAError."""
    _raise(library().sma_attention_bwd_timed(q_ptr, k_ptr, v_ptr, o_ptr, lse_ptr, dout_ptr, dq_ptr,
                                             dk_ptr, dv_ptr, in_dtype, batch, heads, seq_q, seq_kv,
                                             head_dim, float(scale), int(bool(causal)), ws_ptr,
                                             ws_bytes, stream, event_after_pre, event_after_dkdv))


def attention_bwd(q, k, v, o, lse, dout, scale=None, causal=False, workspace=None, stream=None,
                  layout="bhsd", mask=None):
    """(dQ, dK, dV) of O = softmax(scale * Q K^T + mask) V for the upstream gradient dout.

    q, o, dout [B,H,Sq,D] and k, v [B,H,Skv,D] contiguous tensors on the current
    HIP device: q, k, v all float32, all bfloat16 or all float16 (then on 16-bit MFMA;
    float16 is not rescaled, so dout must keep dS inside its range), o, dout
    and lse ([B,H,Sq]) float32, o and lse as attention_fwd returned them for the
    same q, k, v, scale and causal. layout="bshd" takes q, o, dout [B,Sq,H,D] and
    k, v [B,Skv,H,D] (lse stays [B,H,Sq]). mask: the hard mask attention_fwd was
    given (bool or uint8, [Sq,Skv] or [B or 1, H or 1, Sq, Skv]). Returns three
    float32 tensors shaped like q, k and v. The workspace is allocated when not given.
    """
    import torch

    if stream is None:
        stream = torch.cuda.current_stream()
    with torch.cuda.stream(stream):  # allocations on the launch stream, as in attention_fwd
        return _attention_bwd(q, k, v, o, lse, dout, scale, causal, workspace, stream, layout, mask)


def _attention_bwd(q, k, v, o, lse, dout, scale, causal, workspace, stream, layout, mask):
    import torch

    ts = {"q": q, "k": k, "v": v, "o": o, "lse": lse, "dout": dout}
    for name, t in ts.items():
        if not isinstance(t, torch.Tensor):
            raise TypeError(f"{name} must be a torch tensor")
    if q.dim() != 4 or k.dim() != 4 or v.dim() != 4:
        raise ValueError("q, k, v must be 4-D [batch, heads, seq, head_dim]")
    if layout not in LAYOUTS:
        raise ValueError(f"layout must be one of {sorted(LAYOUTS)}")
    if layout == "bshd":
        B, Sq, H, D = q.shape
        Skv = k.shape[1]
        kv_shape, q_shape = (B, Skv, H, D), (B, Sq, H, D)
    else:
        B, H, Sq, D = q.shape
        Skv = k.shape[2]
        kv_shape, q_shape = (B, H, Skv, D), (B, H, Sq, D)
    if (tuple(k.shape) != kv_shape or tuple(v.shape) != kv_shape or tuple(o.shape) != q_shape or
            tuple(dout.shape) != q_shape or tuple(lse.shape) != (B, H, Sq)):
        raise ValueError("shape mismatch among q, k, v, o, lse, dout")
    dev = torch.device("cuda", torch.cuda.current_device())
    dts = {torch.float32: SMA_DTYPE_F32, torch.bfloat16: SMA_DTYPE_BF16, torch.float16: SMA_DTYPE_F16}
    if not (q.dtype == k.dtype == v.dtype) or q.dtype not in dts:
        raise ValueError("q, k, v must be all float32, all bfloat16 or all float16")
    in_dt = dts[q.dtype]
    for name, t in ts.items():
        if name in ("o", "lse", "dout") and t.dtype != torch.float32:
            raise ValueError(f"{name} must be float32")
        if t.device != dev:
            raise ValueError(f"{name} is on {t.device}, the current HIP device is {dev}")
        if not t.is_contiguous():
            raise ValueError(f"{name} must be contiguous")
    if scale is None:
        scale = 1.0 / math.sqrt(D)
    dq = torch.empty(q.shape, dtype=torch.float32, device=dev)
    dk = torch.empty(k.shape, dtype=torch.float32, device=dev)
    dv = torch.empty(v.shape, dtype=torch.float32, device=dev)
    if mask is not None:
        if not isinstance(mask, torch.Tensor) or mask.dtype not in (torch.bool, torch.uint8):
            raise ValueError("mask must be a bool or uint8 torch tensor")
        if mask.dim() == 2:
            mask = mask.view(1, 1, *mask.shape)
        if (mask.dim() != 4 or tuple(mask.shape[2:]) != (Sq, Skv) or mask.shape[0] not in (1, B)
                or mask.shape[1] not in (1, H)):
            raise ValueError(f"mask shape {tuple(mask.shape)} does not broadcast to {(B, H, Sq, Skv)}")
        if mask.device != dev or not mask.is_contiguous():
            raise ValueError(f"mask must be a contiguous tensor on {dev}")
        need = library().sma_attention_bwd_masked_workspace_bytes(in_dt, B, H, Sq, Skv, D,
                                                                  int(bool(causal)), LAYOUTS[layout],
                                                                  mask.shape[0], mask.shape[1])
    else:
        need = attention_bwd_workspace_bytes(in_dt, B, H, Sq, Skv, D, causal)
    if workspace is None and need > 0:
        workspace = torch.empty(need, dtype=torch.uint8, device=dev)
    ws_ptr = workspace.data_ptr() if workspace is not None else None
    ws_bytes = workspace.numel() * workspace.element_size() if workspace is not None else 0
    if stream is None:
        stream = torch.cuda.current_stream()
    if mask is not None:
        _raise(library().sma_attention_bwd_masked(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse),
                                                  _ptr(dout), _ptr(dq), _ptr(dk), _ptr(dv),
                                                  _ptr(mask), mask.shape[0], mask.shape[1], in_dt,
                                                  B, H, Sq, Skv, D, float(scale),
                                                  int(bool(causal)), LAYOUTS[layout], ws_ptr,
                                                  ws_bytes, stream.cuda_stream))
    elif layout == "bhsd":
        attention_bwd_raw(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), _ptr(dout), _ptr(dq),
                          _ptr(dk), _ptr(dv), in_dt, B, H, Sq, Skv, D, scale, causal, ws_ptr,
                          ws_bytes, stream.cuda_stream)
    else:
        _raise(library().sma_attention_bwd_layout(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse),
                                                  _ptr(dout), _ptr(dq), _ptr(dk), _ptr(dv), in_dt,
                                                  B, H, Sq, Skv, D, float(scale),
                                                  int(bool(causal)), LAYOUTS[layout], ws_ptr,
                                                  ws_bytes, stream.cuda_stream))
    return dq, dk, dv


# ------------------------------------------------------------------ row primitives
def _row_input(x, name, ndim):
    import torch

    if not isinstance(x, torch.Tensor) or x.dtype != torch.float32 or not x.is_contiguous():
        raise ValueError(f"{name} must be a contiguous float32 tensor")
    if x.dim() != ndim:
        raise ValueError(f"{name} must be {ndim}-D")
    if x.device != torch.device("cuda", torch.cuda.current_device()):
        raise ValueError(f"{name} must be on the current HIP device")
    return x


def _ptr(t):
    return t.data_ptr() if t is not None and t.numel() > 0 else None


def softmax_rows(x, out=None, stream=None):
    """Row softmax of a contiguous float32 [rows, cols] tensor; out may be x (in place)."""
    import torch

    stream = stream or torch.cuda.current_stream()
    with torch.cuda.stream(stream):  # allocate on the launch stream
        x = _row_input(x, "x", 2)
        out = torch.empty_like(x) if out is None else _row_input(out, "out", 2)
        if out.shape != x.shape:
            raise ValueError("out shape differs")
        s = stream.cuda_stream
        _raise(library().sma_softmax_rows(_ptr(x), _ptr(out), x.shape[0], x.shape[1], s))
        return out


def logsumexp_rows(x, out=None, stream=None):
    """Per-row natural-log log-sum-exp of a contiguous float32 [rows, cols] tensor -> [rows]."""
    import torch

    stream = stream or torch.cuda.current_stream()
    with torch.cuda.stream(stream):  # allocate on the launch stream
        x = _row_input(x, "x", 2)
        out = torch.empty(x.shape[0], dtype=torch.float32, device=x.device) if out is None else out
        if out.shape != (x.shape[0],):
            raise ValueError("out must be [rows]")
        s = stream.cuda_stream
        _raise(library().sma_logsumexp_rows(_ptr(x), _ptr(out), x.shape[0], x.shape[1], s))
        return out


def masked_softmax_rows(x, mask, out=None, stream=None):
    """Hard-masked row softmax: mask (float32, same shape) nonzero admits an entry."""
    import torch

    stream = stream or torch.cuda.current_stream()
    with torch.cuda.stream(stream):  # allocate on the launch stream
        x, mask = _row_input(x, "x", 2), _row_input(mask, "mask", 2)
        if mask.shape != x.shape:
            raise ValueError("mask shape differs")
        out = torch.empty_like(x) if out is None else _row_input(out, "out", 2)
        s = stream.cuda_stream
        _raise(library().sma_masked_softmax_rows(_ptr(x), _ptr(mask), _ptr(out), x.shape[0], x.shape[1], s))
        return out


def softmax_rows_backward(y, dy, scale=1.0, out=None, stream=None):
    """dx = scale * y * (dy - rowsum(y * dy)) for contiguous float32 [rows, cols] tensors y (the
    softmax output) and dy; out may be y or dy (in place)."""
    import torch

    stream = stream or torch.cuda.current_stream()
    with torch.cuda.stream(stream):  # allocate on the launch stream
        y, dy = _row_input(y, "y", 2), _row_input(dy, "dy", 2)
        if dy.shape != y.shape:
            raise ValueError("dy shape differs")
        out = torch.empty_like(y) if out is None else _row_input(out, "out", 2)
        if out.shape != y.shape:
            raise ValueError("out shape differs")
        s = stream.cuda_stream
        _raise(library().sma_softmax_rows_backward(_ptr(y), _ptr(dy), _ptr(out), y.shape[0], y.shape[1],
                                                   float(scale), s))
        return out


def scaled_causal_softmax(x, scale, causal=True, out=None, stream=None):
    """softmax(scale * x) per row of each matrix of a float32 [batch, rows, cols] tensor, with the
    bottom-right causal mask when causal."""
    import torch

    stream = stream or torch.cuda.current_stream()
    with torch.cuda.stream(stream):  # allocate on the launch stream
        x = _row_input(x, "x", 3)
        out = torch.empty_like(x) if out is None else _row_input(out, "out", 3)
        if out.shape != x.shape:
            raise ValueError("out shape differs")
        s = stream.cuda_stream
        _raise(library().sma_scaled_causal_softmax(_ptr(x), _ptr(out), x.shape[0], x.shape[1], x.shape[2],
                                                   float(scale), int(bool(causal)), s))
        return out
