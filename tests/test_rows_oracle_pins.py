"""Pins of the row-softmax oracle against facts it does not compute itself.

Closed forms (a constant row, a two-entry row), scipy's float64 softmax and
logsumexp on the admitted entries only, invariance under shifts far past the
range of exp, and the conventions the pages fix for masked and empty rows
(blocked entries exactly zero and never read, a row admitting nothing all
zeros). test_rows_oracle_mutations.py plants the plausible slips -- no max
subtraction, blocked entries in the max, a top-left causal mask, log2 for the
log-sum-exp, a uniform empty row -- and checks that each fails a pin here.
"""
import math

import numpy as np
import pytest
import scipy.special as sps

import oracle


def _rng(seed):
    return np.random.default_rng(seed)


def _allowed_prefix(i, rows, cols, causal):
    """Test-side bookkeeping of the bottom-right causal mask: admitted prefix length of row i."""
    if not causal:
        return cols
    return int(min(max(i + cols - rows + 1, 0), cols))


# ------------------------------------------------------------------ closed forms
@pytest.mark.parametrize("cols", [1, 2, 7, 64, 1000])
def test_constant_row_is_uniform_and_lse_is_c_plus_log_n(cols):
    c = _rng(cols).normal(size=(5, 1)).astype(np.float32) * 4
    x = np.repeat(c, cols, axis=1)
    p = oracle.softmax_rows(x)
    assert np.all(np.abs(p - 1.0 / cols) <= 1e-15)
    lse = oracle.logsumexp_rows(x)
    ref = np.array([float(v) + math.log(cols) for v in c[:, 0]])
    assert np.all(np.abs(lse - ref) <= 1e-12 * np.maximum(1, np.abs(ref)))


def test_two_entry_rows_are_logistic():
    ab = _rng(1).normal(size=(40, 2)).astype(np.float32) * 6
    p = oracle.softmax_rows(ab)
    for (a, b), (p0, p1) in zip(ab.astype(np.float64), p):
        assert abs(p0 - 1.0 / (1.0 + math.exp(b - a))) <= 1e-15
        assert abs(p1 - 1.0 / (1.0 + math.exp(a - b))) <= 1e-15


# ------------------------------------------------------------------ library routine
@pytest.mark.parametrize("rows,cols", [(3, 5), (17, 333), (4, 4096)])
def test_matches_scipy_softmax_and_logsumexp(rows, cols):
    x = (_rng(rows * cols).normal(size=(rows, cols)) * 5).astype(np.float32)
    x64 = x.astype(np.float64)
    assert np.abs(oracle.softmax_rows(x) - sps.softmax(x64, axis=1)).max() <= 1e-13
    assert np.abs(oracle.logsumexp_rows(x) - sps.logsumexp(x64, axis=1)).max() <= 1e-12


def test_rows_are_stochastic():
    x = (_rng(2).normal(size=(50, 777)) * 8).astype(np.float32)
    assert np.abs(oracle.softmax_rows(x).sum(axis=1) - 1.0).max() <= 1e-12


# ------------------------------------------------------------------ max subtraction
def test_shift_far_beyond_exp_range():
    """x on a 1/64 grid plus 2^13 is exact in fp32; exp(8192) overflows double."""
    x = (np.round(_rng(3).normal(size=(8, 300)) * 64) / 64).astype(np.float32)
    shifted = (x + np.float32(8192.0)).astype(np.float32)
    assert np.array_equal(shifted - np.float32(8192.0), x)
    p = oracle.softmax_rows(shifted)
    assert np.all(np.isfinite(p))
    assert np.abs(p - sps.softmax(x.astype(np.float64), axis=1)).max() <= 1e-13
    lse = oracle.logsumexp_rows(shifted)
    assert np.abs(lse - (sps.logsumexp(x.astype(np.float64), axis=1) + 8192.0)).max() <= 1e-9


# ------------------------------------------------------------------ hard mask
def test_masked_all_admitted_equals_scipy():
    x = (_rng(4).normal(size=(9, 130)) * 3).astype(np.float32)
    p = oracle.masked_softmax_rows(x, np.ones_like(x))
    assert np.abs(p - sps.softmax(x.astype(np.float64), axis=1)).max() <= 1e-13


def test_masked_blocked_entries_never_reach_the_arithmetic():
    """Blocked entries hold NaN, +inf and 1e30; the result is scipy's softmax over the admitted ones."""
    rng = _rng(5)
    x = (rng.normal(size=(12, 200)) * 4).astype(np.float32)
    mask = (rng.random(size=x.shape) < 0.4).astype(np.float32)
    mask[:, 0] = 1.0
    poison = np.array([np.nan, np.inf, 1e30], dtype=np.float32)
    xb = np.where(mask != 0, x, poison[rng.integers(0, 3, size=x.shape)]).astype(np.float32)
    p = oracle.masked_softmax_rows(xb, mask * rng.choice([1.0, -2.5, 7.0], size=x.shape).astype(np.float32))
    for i in range(x.shape[0]):
        adm = mask[i] != 0
        ref = np.zeros(x.shape[1])
        ref[adm] = sps.softmax(x[i, adm].astype(np.float64))
        assert np.all(p[i][~adm] == 0.0)
        assert np.abs(p[i] - ref).max() <= 1e-13


def test_masked_single_admitted_entry_is_one_hot():
    rng = _rng(6)
    x = (rng.normal(size=(6, 50)) * 10).astype(np.float32)
    mask = np.zeros_like(x)
    idx = rng.integers(0, 50, size=6)
    mask[np.arange(6), idx] = 1.0
    p = oracle.masked_softmax_rows(x, mask)
    ref = np.zeros_like(p)
    ref[np.arange(6), idx] = 1.0
    assert np.array_equal(p, ref)


def test_rows_admitting_nothing_are_zero():
    x = _rng(7).normal(size=(4, 33)).astype(np.float32)
    assert np.array_equal(oracle.masked_softmax_rows(x, np.zeros_like(x)), np.zeros(x.shape))
    neg = np.full((3, 10), -np.inf, dtype=np.float32)
    assert np.array_equal(oracle.softmax_rows(neg), np.zeros(neg.shape))
    assert np.all(np.isneginf(oracle.logsumexp_rows(neg)))
    empty = np.zeros((5, 0), dtype=np.float32)
    assert oracle.softmax_rows(empty).shape == (5, 0)
    assert np.all(np.isneginf(oracle.logsumexp_rows(empty)))


def test_negative_infinity_entries_weigh_zero():
    x = (_rng(8).normal(size=(5, 40)) * 2).astype(np.float32)
    x[:, ::3] = -np.inf
    p = oracle.softmax_rows(x)
    assert np.all(p[:, ::3] == 0.0)
    keep = np.ones(40, dtype=bool)
    keep[::3] = False
    assert np.abs(p[:, keep] - sps.softmax(x[:, keep].astype(np.float64), axis=1)).max() <= 1e-13
    assert np.abs(oracle.logsumexp_rows(x) - sps.logsumexp(x[:, keep].astype(np.float64), axis=1)).max() <= 1e-12


# ------------------------------------------------------------------ fused scale + causal
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("rows,cols", [(16, 16), (20, 7), (7, 20), (1, 9)])
@pytest.mark.parametrize("scale", [0.125, 1.0, -0.3, 0.0])
def test_scaled_causal_matches_scipy_on_the_admitted_prefix(rows, cols, causal, scale):
    x = (_rng(rows * 31 + cols).normal(size=(3, rows, cols)) * 4).astype(np.float32)
    p = oracle.scaled_causal_softmax(x, scale, causal)
    for b in range(3):
        for i in range(rows):
            hi = _allowed_prefix(i, rows, cols, causal)
            ref = np.zeros(cols)
            if hi > 0:
                ref[:hi] = sps.softmax(scale * x[b, i, :hi].astype(np.float64))
            assert np.abs(p[b, i] - ref).max() <= 1e-13, (b, i, hi)


def test_scaled_keeps_negative_infinity():
    x = np.zeros((1, 2, 4), dtype=np.float32)
    x[0, :, 1] = -np.inf
    for scale in (0.5, -0.5, 0.0):
        p = oracle.scaled_causal_softmax(x, scale, False)
        assert np.all(p[0, :, 1] == 0.0) and np.allclose(p[0, :, [0, 2, 3]], 1.0 / 3.0, atol=1e-15)


def test_rejects_bad_shapes():
    with pytest.raises(ValueError):
        oracle.softmax_rows(np.zeros(5, dtype=np.float32))
    with pytest.raises(ValueError):
        oracle.masked_softmax_rows(np.zeros((2, 3), np.float32), np.zeros((3, 2), np.float32))
    with pytest.raises(ValueError):
        oracle.scaled_causal_softmax(np.zeros((2, 3), np.float32), 1.0, True)


# ------------------------------------------------------------------ softmax backward
def _softmax_grid(rng, rows, cols):
    return (np.round(rng.uniform(-3, 3, size=(rows, cols)) * 64) / 64).astype(np.float32)


@pytest.mark.parametrize("scale", [1.0, 0.25, -0.5])
def test_softmax_backward_matches_finite_differences(scale):
    """d/dx of L = sum(dy * softmax(scale x)), by Richardson-extrapolated central differences of
    the forward oracle on inputs where the perturbations are exact in fp32, equals
    scale * y * (dy - sum y dy) with y = softmax(scale x)."""
    rng = np.random.default_rng(31)
    x = _softmax_grid(rng, 3, 6)
    dy = rng.normal(size=(3, 6))
    y = oracle.scaled_causal_softmax(x[None], scale, False)[0]

    def loss(xx):
        return float(np.sum(dy * oracle.scaled_causal_softmax(xx[None], scale, False)[0]))

    num = np.zeros_like(dy)
    for idx in np.ndindex(x.shape):
        est = []
        for h in (2.0 ** -8, 2.0 ** -9):
            xp, xm = x.copy(), x.copy()
            xp[idx] += h
            xm[idx] -= h
            est.append((loss(xp) - loss(xm)) / (2 * h))
        num[idx] = (4 * est[1] - est[0]) / 3
    got = oracle.softmax_rows_backward(y.astype(np.float32), dy.astype(np.float32), scale)
    # y and dy rounded to fp32 for the call: compare within that rounding
    assert np.abs(got - num).max() <= 1e-6 * max(1.0, np.abs(num).max())


def test_softmax_backward_matches_torch_float64_autograd():
    torch = pytest.importorskip("torch")
    rng = np.random.default_rng(32)
    x = rng.normal(size=(5, 40)).astype(np.float32)
    dy = rng.normal(size=(5, 40)).astype(np.float32)
    tx = torch.tensor(x, dtype=torch.float64, requires_grad=True)
    ty = torch.softmax(tx, dim=-1)
    (ty * torch.tensor(dy, dtype=torch.float64)).sum().backward()
    y32 = ty.detach().numpy().astype(np.float32)
    got = oracle.softmax_rows_backward(y32, dy)
    # the oracle sees y rounded to fp32: recompute torch's gradient from that y exactly
    yd, gd = y32.astype(np.float64), dy.astype(np.float64)
    assert np.abs(got - tx.grad.numpy()).max() <= 1e-6
    assert np.abs(got - yd * (gd - (yd * gd).sum(axis=1, keepdims=True))).max() <= 1e-15


def test_softmax_backward_closed_forms():
    rng = np.random.default_rng(33)
    y = oracle.softmax_rows(rng.normal(size=(4, 30)).astype(np.float32)).astype(np.float32)
    y = y / y.sum(axis=1, keepdims=True, dtype=np.float64).astype(np.float32)
    c = np.repeat(rng.normal(size=(4, 1)), 30, axis=1).astype(np.float32)
    # constant dy per row: dx = y * c * (1 - sum y), i.e. zero up to sum(y) - 1
    dx = oracle.softmax_rows_backward(y, c)
    s = y.astype(np.float64).sum(axis=1, keepdims=True)
    assert np.abs(dx - y * c * (1.0 - s)).max() <= 1e-15
    # one-hot y: every entry zero
    oh = np.zeros((3, 9), np.float32)
    oh[np.arange(3), [1, 4, 8]] = 1.0
    assert np.all(oracle.softmax_rows_backward(oh, rng.normal(size=(3, 9)).astype(np.float32)) == 0.0)
    # linear in the scale; entries with y = 0 (masked) stay 0
    g = rng.normal(size=(4, 30)).astype(np.float32)
    y[:, 5] = 0.0
    a1, a3 = oracle.softmax_rows_backward(y, g, 1.0), oracle.softmax_rows_backward(y, g, -3.0)
    assert np.abs(a3 + 3.0 * a1).max() <= 1e-15 and np.all(a1[:, 5] == 0.0)
