"""Pins of the masked attention-backward oracle against facts it does not compute itself.

Central finite differences of the masked forward oracle (Richardson-extrapolated, on inputs
whose perturbations are exact in fp32), torch's float64 autograd of a masked attention
written with torch ops on the CPU, and closed forms: a key no row admits gets no gradient;
rows that admit a single key have no softmax gradient (dS = 0), so dQ = dK = 0 and dV_j sums
the dO of the rows admitting j; a mask broadcast over heads equals the same mask expanded;
an all-ones mask is the unmasked backward. A planted mistake (the mask ignored) is caught
by test_planted_mask_mistake_is_caught.
"""
import numpy as np
import pytest

import oracle


def _grid(rng, shape, step=2.0 ** -6, span=2.0):
    """Values on a 2^-6 grid in [-span, span]: +-2^-8 and +-2^-9 perturbations stay exact in fp32."""
    return (np.round(rng.uniform(-span, span, size=shape) / step) * step).astype(np.float32)


def _mask(rng, shape, density, empty_row=None):
    m = (rng.uniform(size=shape) < density).astype(np.uint8)
    if empty_row is not None:
        m[..., empty_row, :] = 0
    return m


def _loss(q, k, v, g, mask, scale, causal):
    o, _ = oracle.attention_fwd_masked(q, k, v, mask, scale, causal)
    return float(np.sum(o * g.astype(np.float64)))


def _numeric_grad(which, q, k, v, g, mask, scale, causal):
    arrs = {"q": q, "k": k, "v": v}
    x = arrs[which]
    grad = np.zeros(x.shape)
    for idx in np.ndindex(x.shape):
        est = []
        for h in (2.0 ** -8, 2.0 ** -9):
            vals = []
            for sgn in (1.0, -1.0):
                y = x.copy()
                y[idx] = np.float32(x[idx] + sgn * h)
                a = dict(arrs)
                a[which] = y
                vals.append(_loss(a["q"], a["k"], a["v"], g, mask, scale, causal))
            est.append((vals[0] - vals[1]) / (2 * h))
        grad[idx] = (4 * est[1] - est[0]) / 3
    return grad


@pytest.mark.parametrize("causal,sq,skv", [(False, 5, 7), (True, 6, 8), (True, 7, 4)])
def test_matches_finite_differences_of_the_masked_forward(causal, sq, skv):
    rng = np.random.default_rng(40 + sq + skv)
    q, k, v = _grid(rng, (1, 2, sq, 4)), _grid(rng, (1, 2, skv, 4)), _grid(rng, (1, 2, skv, 4))
    g = _grid(rng, (1, 2, sq, 4))
    mask = _mask(rng, (1, 2, sq, skv), 0.6, empty_row=1)
    dq, dk, dv = oracle.attention_bwd_masked(q, k, v, g, mask, 0.75, causal)
    for name, ana in (("q", dq), ("k", dk), ("v", dv)):
        num = _numeric_grad(name, q, k, v, g, mask, 0.75, causal)
        assert np.abs(ana - num).max() <= 1e-8 * max(1.0, np.abs(num).max()), name


def _torch_reference(q, k, v, g, mask, scale, causal):
    torch = pytest.importorskip("torch")
    tq, tk, tv = (torch.tensor(x, dtype=torch.float64, requires_grad=True) for x in (q, k, v))
    s = scale * torch.matmul(tq, tk.transpose(-1, -2).contiguous())
    sq, skv = q.shape[2], k.shape[2]
    blocked = torch.tensor(np.broadcast_to(mask, s.shape) == 0)
    if causal:
        i = torch.arange(sq)[:, None]
        j = torch.arange(skv)[None, :]
        blocked = blocked | (j > i + (skv - sq))
    s = s.masked_fill(blocked, float("-inf"))
    p = torch.nan_to_num(torch.softmax(s, dim=-1), nan=0.0)  # rows that admit nothing
    o = torch.matmul(p, tv)
    (o * torch.tensor(g, dtype=torch.float64)).sum().backward()
    return tq.grad.numpy(), tk.grad.numpy(), tv.grad.numpy()


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("form", ["full", "per_head", "shared"])
def test_matches_torch_float64_autograd(form, causal):
    rng = np.random.default_rng(50 + causal)
    B, H, sq, skv, d = 2, 3, 23, 31, 16
    q, k, v, g = (rng.normal(size=s).astype(np.float32) for s in
                  ((B, H, sq, d), (B, H, skv, d), (B, H, skv, d), (B, H, sq, d)))
    shape = {"full": (B, H, sq, skv), "per_head": (1, H, sq, skv), "shared": (1, 1, sq, skv)}[form]
    mask = _mask(rng, shape, 0.5, empty_row=3)
    got = oracle.attention_bwd_masked(q, k, v, g, mask, 1.0 / np.sqrt(d), causal)
    ref = _torch_reference(q, k, v, g, mask, 1.0 / np.sqrt(d), causal)
    for a, b, n in zip(got, ref, "qkv"):
        assert np.abs(a - b).max() <= 1e-12 * max(1.0, np.abs(b).max()), n


def test_key_admitted_by_no_row_gets_no_gradient():
    rng = np.random.default_rng(60)
    q, k, v, g = (rng.normal(size=s).astype(np.float32) for s in ((1, 1, 8, 8), (1, 1, 9, 8), (1, 1, 9, 8), (1, 1, 8, 8)))
    mask = _mask(rng, (1, 1, 8, 9), 0.7)
    mask[..., 4] = 0  # key 4 is blocked for every row
    dq, dk, dv = oracle.attention_bwd_masked(q, k, v, g, mask, 0.4, False)
    assert np.all(dk[0, 0, 4] == 0.0) and np.all(dv[0, 0, 4] == 0.0)
    assert np.abs(dk).max() > 0 and np.abs(dv).max() > 0


def test_rows_with_one_admitted_key_have_no_softmax_gradient():
    """Each row admits exactly one key: P = 1 there, dS = 0, so dQ = dK = 0, and dV_j is the
    sum of dO over the rows admitting j (counted here without the oracle)."""
    rng = np.random.default_rng(61)
    sq, skv = 10, 6
    q, k, v, g = (rng.normal(size=s).astype(np.float32) for s in ((1, 1, sq, 8), (1, 1, skv, 8), (1, 1, skv, 8), (1, 1, sq, 8)))
    pick = rng.integers(0, skv, size=sq)
    mask = np.zeros((1, 1, sq, skv), np.uint8)
    mask[0, 0, np.arange(sq), pick] = 1
    dq, dk, dv = oracle.attention_bwd_masked(q, k, v, g, mask, 0.7, False)
    assert np.abs(dq).max() <= 1e-15 and np.abs(dk).max() <= 1e-15
    ref = np.zeros((skv, 8))
    for i in range(sq):
        ref[pick[i]] += g[0, 0, i].astype(np.float64)
    assert np.abs(dv[0, 0] - ref).max() <= 1e-13


def test_empty_rows_get_zero_dq():
    rng = np.random.default_rng(62)
    q, k, v, g = (rng.normal(size=s).astype(np.float32) for s in ((1, 2, 7, 8), (1, 2, 9, 8), (1, 2, 9, 8), (1, 2, 7, 8)))
    mask = _mask(rng, (1, 2, 7, 9), 0.5, empty_row=2)
    dq, _, _ = oracle.attention_bwd_masked(q, k, v, g, mask, 0.4, False)
    assert np.all(dq[:, :, 2] == 0.0) and np.abs(dq).max() > 0


def test_broadcast_equals_expanded_and_all_ones_equals_unmasked():
    rng = np.random.default_rng(63)
    B, H, sq, skv, d = 2, 2, 12, 15, 8
    q, k, v, g = (rng.normal(size=s).astype(np.float32) for s in ((B, H, sq, d), (B, H, skv, d), (B, H, skv, d), (B, H, sq, d)))
    m = _mask(rng, (1, H, sq, skv), 0.5)
    a = oracle.attention_bwd_masked(q, k, v, g, m, 0.3, True)
    b = oracle.attention_bwd_masked(q, k, v, g, np.broadcast_to(m, (B, H, sq, skv)), 0.3, True)
    assert all(np.array_equal(x, y) for x, y in zip(a, b))
    ones = np.ones((1, 1, sq, skv), np.uint8)
    c = oracle.attention_bwd_masked(q, k, v, g, ones, 0.3, True)
    e = oracle.attention_bwd(q, k, v, g, 0.3, True)
    assert all(np.abs(x - y).max() <= 1e-14 * max(1.0, np.abs(y).max()) for x, y in zip(c, e))


def test_bound_bounds_the_gradients():
    """The error scale is a sum of magnitudes, so it bounds each gradient (triangle inequality)."""
    rng = np.random.default_rng(64)
    q, k, v, g = (rng.normal(size=s).astype(np.float32) for s in ((1, 2, 11, 8), (1, 2, 13, 8), (1, 2, 13, 8), (1, 2, 11, 8)))
    mask = _mask(rng, (1, 2, 11, 13), 0.5, empty_row=0)
    grads = oracle.attention_bwd_masked(q, k, v, g, mask, 0.5, True)
    bounds = oracle.attention_bwd_masked_bound(q, k, v, g, mask, 0.5, True)
    for x, m in zip(grads, bounds):
        assert np.all(np.abs(x) <= m * (1 + 1e-12))
    assert np.all(bounds[0][:, :, 0] == 0.0)  # the empty row


def test_planted_mask_mistake_is_caught(tmp_path):
    path = oracle.build(force=True, out=str(tmp_path / "liboracle_mbwd.so"), defines=["MBWD_PLANT_IGNORE_MASK"])
    bad = oracle.load(path)
    saved = oracle._lib
    caught = []
    try:
        oracle._lib = bad
        for name, fn, args in (("finite_diff", test_matches_finite_differences_of_the_masked_forward, (True, 6, 8)),
                               ("torch", test_matches_torch_float64_autograd, ("shared", True)),
                               ("no_row", test_key_admitted_by_no_row_gets_no_gradient, ()),
                               ("one_key", test_rows_with_one_admitted_key_have_no_softmax_gradient, ())):
            try:
                with np.errstate(all="ignore"):
                    fn(*args)
            except (AssertionError, ValueError, FloatingPointError):
                caught.append(name)
    finally:
        oracle._lib = saved
    assert len(caught) >= 3, f"planted mask mistake caught only by {caught}"
