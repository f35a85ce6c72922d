"""Shared test helpers: run the HIP path through the C ABI, run the oracle, compare."""
from __future__ import annotations

import math

import numpy as np

import gen
import oracle

# Parity bars for O: fp32 max-abs 2e-5; bf16 max-abs 2e-2 and relative L2 1e-2. fp16 inputs:
# P is rounded to fp16 (unit roundoff 2^-11, against bf16's 2^-8) for P V, so |dO| is at most
# 2^-11 sum_j p_j |v_j| / l, about 2.8e-3 for |v| <= 5.8: max-abs 4e-3, relative L2 2e-3.
F32_MAX_ABS = 2e-5
BF16_MAX_ABS = 2e-2
BF16_REL_L2 = 1e-2
F16_MAX_ABS = 4e-3
F16_REL_L2 = 2e-3
# Lines printed at the end of the session by the terminal-summary hook in conftest.py.
SUMMARY = []

# LSE (natural log): |d| <= tol * max(1, |lse|).
F32_LSE_TOL = 1e-5
BF16_LSE_TOL = 1e-4

# A second, tighter bar for the backward gradients. The derived bars of the backward tests
# (elementwise and L2, from the oracle's error scale) are the parity claim; the errors the
# kernels show use only a small part of them. A gradient tensor whose worst element, or whose
# L2 error, uses more than BWD_REGRESSION[dtype] = (element, L2) of its derived bars fails:
# about three times the largest fractions measured over all backward GPU tests (element and
# L2: fp32 0.022 and 0.061, bf16 0.100 and 0.198, fp16 0.095 and 0.142; the kernels are
# deterministic, so these do not vary between runs), so that a drift of that size is caught.
# BWD_WORST keeps the largest fractions seen in the session (printed at the end).
BWD_REGRESSION = {"f32": (0.07, 0.2), "bf16": (0.3, 0.6), "f16": (0.3, 0.4)}
BWD_WORST = {}


def bwd_regression(dtype, frac_elem, frac_l2, label):
    """Record a gradient tensor's error as fractions of its derived bars; hold it to the
    regression bar."""
    e, l2, _, _ = BWD_WORST.get(dtype, (0.0, 0.0, "", ""))
    BWD_WORST[dtype] = (max(e, frac_elem), max(l2, frac_l2),
                        label if frac_elem >= e else BWD_WORST[dtype][2],
                        label if frac_l2 >= l2 else BWD_WORST[dtype][3])
    bar_e, bar_l2 = BWD_REGRESSION[dtype]
    assert frac_elem <= bar_e, (f"{label}: worst element uses {frac_elem:.3f} of its derived bar "
                                f"(regression bar {bar_e} for {dtype})")
    assert frac_l2 <= bar_l2, (f"{label}: L2 error uses {frac_l2:.3f} of its derived bar "
                               f"(regression bar {bar_l2} for {dtype})")


def allowed_keys(i, sq, skv, causal):
    """Test-side bookkeeping of the bottom-right mask (which rows are empty)."""
    if not causal:
        return skv
    return int(min(max(i + skv - sq + 1, 0), skv))


def empty_rows(sq, skv, causal):
    return np.array([allowed_keys(i, sq, skv, causal) == 0 for i in range(sq)], dtype=bool)


def to_device(vals, bits, dtype):
    """Host inputs -> contiguous torch tensors on cuda:0 (16-bit types from the exact bit patterns)."""
    import torch

    if dtype == "f32":
        return tuple(torch.from_numpy(np.ascontiguousarray(x)).to("cuda") for x in vals)
    tdt = torch.bfloat16 if dtype == "bf16" else torch.float16
    return tuple(torch.from_numpy(np.ascontiguousarray(b).view(np.int16)).to("cuda").view(tdt)
                 for b in bits)


def run_gpu(tq, tk, tv, scale, causal, **kw):
    import torch

    import scaled_masked_attention_amd as sma

    o, lse = sma.attention_fwd(tq, tk, tv, scale=scale, causal=causal, return_lse=True, **kw)
    torch.cuda.synchronize()
    return o.cpu().numpy().astype(np.float64), lse.cpu().numpy().astype(np.float64)


def check_parity(o, lse, o_ref, lse_ref, dtype, label=""):
    """Compare GPU O/LSE (float64 arrays) with the oracle's; raise AssertionError with numbers."""
    assert o.shape == o_ref.shape, (o.shape, o_ref.shape)
    ref_empty = np.isneginf(lse_ref)
    assert np.array_equal(np.isneginf(lse), ref_empty), f"{label}: -inf LSE pattern differs"
    if ref_empty.any():
        assert np.all(o[ref_empty] == 0.0), f"{label}: rows without keys are not exactly zero"
        assert not np.any(np.signbit(o[ref_empty])), f"{label}: -0.0 in an empty row"
    assert np.all(np.isfinite(o)), f"{label}: non-finite output"
    err = np.abs(o - o_ref)
    max_abs = float(err.max()) if err.size else 0.0
    nrm = float(np.linalg.norm(o_ref))
    rel_l2 = float(np.linalg.norm(o - o_ref) / nrm) if nrm > 0 else float(np.linalg.norm(o - o_ref))
    fin = ~ref_empty
    lse_err = np.abs(lse[fin] - lse_ref[fin]) / np.maximum(1.0, np.abs(lse_ref[fin]))
    lse_max = float(lse_err.max()) if lse_err.size else 0.0
    if dtype == "f32":
        assert max_abs <= F32_MAX_ABS, f"{label}: fp32 max_abs {max_abs:.3e} > {F32_MAX_ABS}"
        assert lse_max <= F32_LSE_TOL, f"{label}: fp32 LSE rel err {lse_max:.3e}"
    else:
        mx, rl = (BF16_MAX_ABS, BF16_REL_L2) if dtype == "bf16" else (F16_MAX_ABS, F16_REL_L2)
        assert max_abs <= mx, f"{label}: {dtype} max_abs {max_abs:.3e} > {mx}"
        assert rel_l2 <= rl, f"{label}: {dtype} rel_l2 {rel_l2:.3e} > {rl}"
        assert lse_max <= BF16_LSE_TOL, f"{label}: {dtype} LSE rel err {lse_max:.3e}"
    return dict(max_abs=max_abs, rel_l2=rel_l2, lse_rel=lse_max)


def sample_rows(B, H, sq, skv, causal, n_random, seed):
    """Flat row ids covering first/last rows of every (b,h), the causal diagonal band, and random rows."""
    rng = np.random.default_rng(seed)
    rows = set()
    bh = B * H
    for h in range(bh):
        base = h * sq
        for i in (0, 1, sq // 2, sq - 2, sq - 1):
            if 0 <= i < sq:
                rows.add(base + i)
    rows.update(int(x) for x in rng.integers(0, bh * sq, size=n_random))
    if causal:
        off = skv - sq
        for i in range(max(0, -off - 2), min(sq, -off + 3)):
            rows.add(i)  # around the first row that sees a key, head 0
    return np.array(sorted(rows), dtype=np.int64)


def workload_case(name):
    w = gen.WORKLOADS[name]
    vals, bits = gen.make_inputs(w)
    return w, vals, bits


def metric_scale(w):
    return w.scale if w.scale is not None else 1.0 / math.sqrt(w.head_dim)
