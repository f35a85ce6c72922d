"""Pins of the attention-backward oracle against facts it does not compute itself.

Central finite differences of the forward oracle (Richardson-extrapolated, on
inputs whose perturbations are exact in fp32), torch's float64 autograd of an
attention written with torch ops on the CPU, and closed forms: a zero upstream
gradient, value rows that are all equal (the softmax then has no effect, so
dQ = dK = 0), a query of zeros (uniform probabilities over the allowed
prefix), a single key, and rows with no allowed key.
test_bwd_oracle_mutations.py plants the plausible slips -- the D term
dropped, dK without the scale, dV weighted by dS instead of P, a top-left
causal mask -- and checks that each fails a pin here.
"""
import numpy as np
import pytest

import oracle


def _grid(rng, shape, step=2.0 ** -6, span=2.0):
    """Values on a 2^-6 grid in [-span, span]: +-2^-8 and +-2^-9 perturbations stay exact in fp32."""
    return (np.round(rng.uniform(-span, span, size=shape) / step) * step).astype(np.float32)


def _loss(q, k, v, g, scale, causal):
    o, _ = oracle.attention_fwd(q, k, v, scale, causal)
    return float(np.sum(o * g.astype(np.float64)))


def _numeric_grad(which, q, k, v, g, scale, causal):
    """Richardson-extrapolated central differences of L = sum(dO * O) for every element of `which`."""
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
                vals.append(_loss(a["q"], a["k"], a["v"], g, scale, causal))
            est.append((vals[0] - vals[1]) / (2 * h))
        grad[idx] = (4 * est[1] - est[0]) / 3
    return grad


@pytest.mark.parametrize("causal,sq,skv", [(False, 4, 6), (True, 5, 7), (True, 6, 3)])
def test_matches_finite_differences_of_the_forward(causal, sq, skv):
    rng = np.random.default_rng(10 + sq + skv)
    q, k, v = _grid(rng, (1, 2, sq, 4)), _grid(rng, (1, 2, skv, 4)), _grid(rng, (1, 2, skv, 4))
    g = _grid(rng, (1, 2, sq, 4))
    scale = 0.75
    dq, dk, dv = oracle.attention_bwd(q, k, v, g, scale, causal)
    for name, ana in (("q", dq), ("k", dk), ("v", dv)):
        num = _numeric_grad(name, q, k, v, g, scale, causal)
        assert np.abs(ana - num).max() <= 1e-8 * max(1.0, np.abs(num).max()), name


def _torch_reference(q, k, v, g, scale, causal):
    torch = pytest.importorskip("torch")
    tq, tk, tv = (torch.tensor(x, dtype=torch.float64, requires_grad=True) for x in (q, k, v))
    s = scale * torch.matmul(tq, tk.transpose(-1, -2).contiguous())
    sq, skv = q.shape[2], k.shape[2]
    if causal:
        i = torch.arange(sq)[:, None]
        j = torch.arange(skv)[None, :]
        blocked = j > i + (skv - sq)
        s = s.masked_fill(blocked, float("-inf"))
    p = torch.softmax(s, dim=-1)
    p = torch.nan_to_num(p, nan=0.0)  # rows with no allowed key
    o = torch.matmul(p, tv)
    (o * torch.tensor(g, dtype=torch.float64)).sum().backward()
    return tq.grad.numpy(), tk.grad.numpy(), tv.grad.numpy()


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("B,H,sq,skv,d", [(1, 2, 33, 47, 16), (2, 1, 64, 64, 64), (1, 1, 90, 20, 8)])
def test_matches_torch_float64_autograd(B, H, sq, skv, d, causal):
    rng = np.random.default_rng(B * 100 + sq + skv)
    q, k, v, g = (rng.normal(size=s).astype(np.float32) for s in
                  ((B, H, sq, d), (B, H, skv, d), (B, H, skv, d), (B, H, sq, d)))
    got = oracle.attention_bwd(q, k, v, g, 1.0 / np.sqrt(d), causal)
    ref = _torch_reference(q, k, v, g, 1.0 / np.sqrt(d), causal)
    for a, b, n in zip(got, ref, "qkv"):
        assert np.abs(a - b).max() <= 1e-12 * max(1.0, np.abs(b).max()), n


def test_zero_upstream_gradient_gives_zero():
    rng = np.random.default_rng(1)
    q, k, v = (rng.normal(size=(1, 2, 9, 8)).astype(np.float32) for _ in range(3))
    for grad in oracle.attention_bwd(q, k, v, np.zeros_like(q), 0.3, True):
        assert np.all(grad == 0.0)


def test_equal_value_rows_give_no_query_or_key_gradient():
    """With every v_j equal, O does not depend on P: dQ = dK = 0 and dV_j = sum_i P_ij dO_i."""
    rng = np.random.default_rng(2)
    q, k = rng.normal(size=(1, 1, 12, 8)).astype(np.float32), rng.normal(size=(1, 1, 10, 8)).astype(np.float32)
    v = np.repeat(rng.normal(size=(1, 1, 1, 8)).astype(np.float32), 10, axis=2)
    g = rng.normal(size=(1, 1, 12, 8)).astype(np.float32)
    dq, dk, dv = oracle.attention_bwd(q, k, v, g, 0.5, False)
    assert np.abs(dq).max() <= 1e-13 and np.abs(dk).max() <= 1e-13
    p = oracle.softmax_probs(q[0, 0], k[0, 0], 0.5, False)
    assert np.abs(dv[0, 0] - p.T @ g[0, 0].astype(np.float64)).max() <= 1e-13


@pytest.mark.parametrize("causal,sq,skv", [(False, 6, 9), (True, 6, 9), (True, 9, 6)])
def test_zero_query_gives_prefix_mean_weights(causal, sq, skv):
    """q = 0: P is uniform over each row's allowed prefix, so dV_j = sum over rows i admitting j
    of dO_i / hi(i), counted here without the oracle."""
    rng = np.random.default_rng(3 + sq)
    q = np.zeros((1, 1, sq, 4), np.float32)
    k, v = rng.normal(size=(1, 1, skv, 4)).astype(np.float32), rng.normal(size=(1, 1, skv, 4)).astype(np.float32)
    g = rng.normal(size=(1, 1, sq, 4)).astype(np.float32)
    _, _, dv = oracle.attention_bwd(q, k, v, g, 0.9, causal)
    ref = np.zeros((skv, 4))
    for i in range(sq):
        hi = skv if not causal else min(max(i + skv - sq + 1, 0), skv)
        for j in range(hi):
            ref[j] += g[0, 0, i].astype(np.float64) / hi
    assert np.abs(dv[0, 0] - ref).max() <= 1e-14


def test_single_key_has_no_softmax_gradient():
    rng = np.random.default_rng(4)
    q, g = rng.normal(size=(1, 2, 5, 8)).astype(np.float32), rng.normal(size=(1, 2, 5, 8)).astype(np.float32)
    k, v = rng.normal(size=(1, 2, 1, 8)).astype(np.float32), rng.normal(size=(1, 2, 1, 8)).astype(np.float32)
    dq, dk, dv = oracle.attention_bwd(q, k, v, g, 0.5, False)
    assert np.abs(dq).max() <= 1e-15 and np.abs(dk).max() <= 1e-15
    assert np.abs(dv[:, :, 0] - g.astype(np.float64).sum(axis=2)).max() <= 1e-12


def test_rows_without_keys_contribute_nothing():
    """Causal with sq > skv: the first sq - skv rows see no key. Their dQ is zero and changing
    their dO changes nothing else."""
    rng = np.random.default_rng(5)
    sq, skv = 8, 3
    q, g = rng.normal(size=(1, 1, sq, 4)).astype(np.float32), rng.normal(size=(1, 1, sq, 4)).astype(np.float32)
    k, v = rng.normal(size=(1, 1, skv, 4)).astype(np.float32), rng.normal(size=(1, 1, skv, 4)).astype(np.float32)
    dq, dk, dv = oracle.attention_bwd(q, k, v, g, 0.5, True)
    assert np.all(dq[:, :, : sq - skv] == 0.0)
    g2 = g.copy()
    g2[:, :, : sq - skv] = 1e6
    dq2, dk2, dv2 = oracle.attention_bwd(q, k, v, g2, 0.5, True)
    assert np.array_equal(dk, dk2) and np.array_equal(dv, dv2) and np.array_equal(dq, dq2)


def test_rejects_bad_arguments():
    lib = oracle.load()
    z = np.zeros(4, np.float64)
    f = np.zeros(4, np.float32)
    assert lib.oracle_attention_bwd(f.ctypes.data, f.ctypes.data, f.ctypes.data, f.ctypes.data,
                                    1, 1, 1, 1, 0, 1.0, 0, z.ctypes.data, z.ctypes.data,
                                    z.ctypes.data) == -1


# ------------------------------------------------------------------ error scale of the gradients
@pytest.mark.parametrize("causal,sq,skv", [(False, 13, 29), (True, 29, 13), (True, 20, 20)])
def test_bound_dominates_every_gradient(causal, sq, skv):
    """Triangle inequality: |dq| <= mq, |dk| <= mk, |dv| <= mv elementwise."""
    rng = np.random.default_rng(20 + sq)
    q, k, v, g = (rng.normal(size=s).astype(np.float32) for s in
                  ((2, 2, sq, 8), (2, 2, skv, 8), (2, 2, skv, 8), (2, 2, sq, 8)))
    grads = oracle.attention_bwd(q, k, v, g, -0.4, causal)
    bounds = oracle.attention_bwd_bound(q, k, v, g, -0.4, causal)
    for a, m in zip(grads, bounds):
        assert np.all(np.abs(a) <= m * (1 + 1e-12) + 1e-300)
        assert np.all(m >= 0)


def test_bound_zero_scale_closed_form():
    """scale = 0: P is uniform over each row's prefix of hi_i keys and a_ij = |lse_i| = log hi_i,
    so mv_j = sum over rows i admitting j of (1 + log hi_i) |dO_i| / hi_i, and mq = mk = 0."""
    rng = np.random.default_rng(21)
    sq, skv = 9, 6
    q, g = rng.normal(size=(1, 1, sq, 4)).astype(np.float32), rng.normal(size=(1, 1, sq, 4)).astype(np.float32)
    k, v = rng.normal(size=(1, 1, skv, 4)).astype(np.float32), rng.normal(size=(1, 1, skv, 4)).astype(np.float32)
    mq, mk, mv = oracle.attention_bwd_bound(q, k, v, g, 0.0, True)
    ref = np.zeros((skv, 4))
    for i in range(sq):
        hi = min(max(i + skv - sq + 1, 0), skv)
        for j in range(hi):
            ref[j] += (1.0 + np.log(hi)) * np.abs(g[0, 0, i].astype(np.float64)) / hi
    assert np.abs(mv[0, 0] - ref).max() <= 1e-14 * ref.max()
    assert np.all(mq == 0) and np.all(mk == 0)


def test_bound_single_key_closed_form():
    """One key: P = 1, lse_i = s_i = scale q_i.k, a_i = |scale| sum_c |q_ic k_c| + |s_i|, and with
    b_i = sum_c |dO_ic v_c| (= dPmag_i = Dmag_i / (1 + a_i)):
    mq_i = |scale| (1 + a_i) b_i (2 + a_i) |k|, mk = |scale| sum_i (1 + a_i) b_i (2 + a_i) |q_i|,
    mv = sum_i (1 + a_i) |dO_i|."""
    rng = np.random.default_rng(22)
    q, g = rng.normal(size=(1, 1, 6, 4)).astype(np.float32), rng.normal(size=(1, 1, 6, 4)).astype(np.float32)
    k, v = rng.normal(size=(1, 1, 1, 4)).astype(np.float32), rng.normal(size=(1, 1, 1, 4)).astype(np.float32)
    scale = -0.7
    mq, mk, mv = oracle.attention_bwd_bound(q, k, v, g, scale, False)
    q64, g64 = q[0, 0].astype(np.float64), g[0, 0].astype(np.float64)
    k64, v64 = k[0, 0, 0].astype(np.float64), v[0, 0, 0].astype(np.float64)
    s = scale * (q64 @ k64)
    a = abs(scale) * np.abs(q64 * k64[None, :]).sum(axis=1) + np.abs(s)
    b = np.abs(g64 * v64[None, :]).sum(axis=1)
    w = (1 + a) * (b + (1 + a) * b)
    assert np.allclose(mq[0, 0], abs(scale) * w[:, None] * np.abs(k64)[None, :], rtol=1e-13, atol=0)
    assert np.allclose(mk[0, 0, 0], abs(scale) * (w[:, None] * np.abs(q64)).sum(axis=0), rtol=1e-13, atol=0)
    assert np.allclose(mv[0, 0, 0], ((1 + a)[:, None] * np.abs(g64)).sum(axis=0), rtol=1e-13, atol=0)
def test_bound_zero_scale_and_rows_without_keys():
    rng = np.random.default_rng(23)
    q, g = rng.normal(size=(1, 1, 9, 4)).astype(np.float32), rng.normal(size=(1, 1, 9, 4)).astype(np.float32)
    k, v = rng.normal(size=(1, 1, 4, 4)).astype(np.float32), rng.normal(size=(1, 1, 4, 4)).astype(np.float32)
    mq, mk, mv = oracle.attention_bwd_bound(q, k, v, g, 0.0, False)
    assert np.all(mq == 0) and np.all(mk == 0) and np.all(mv > 0)
    mq, mk, _ = oracle.attention_bwd_bound(q, k, v, g, 0.5, True)
    assert np.all(mq[0, 0, :5] == 0) and np.all(mq[0, 0, 5:] > 0)
