"""Pins of the CPU oracle against facts it does not compute itself.

Each test ties the oracle to something independent of its own code: closed
forms derived by hand (tests/golden), special cases whose answer follows from
the mathematics (q = 0, one key, empty rows, a dominant key), invariances, a
brute-force textbook evaluation in extended precision, and a library routine
(torch's scaled_dot_product_attention in float64 on the CPU, scipy's
logsumexp). The set is chosen so that the plausible slips -- dropping or
dividing by the scale, a mask off by one or aligned top-left, swapped K and V,
a transposed product, log2 instead of ln, a missing max or normaliser, a wrong
empty-row value -- each fail at least one test (test_oracle_mutations.py
plants them and checks).
"""
import json
import math
import os

import numpy as np
import pytest

import gen
import oracle

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _bhsd(a):
    a = np.asarray(a, dtype=np.float32)
    return a.reshape((1, 1) + a.shape)


def _allowed(i, sq, skv, causal):
    """Independent restatement of the bottom-right mask for the tests' own bookkeeping."""
    if not causal:
        return skv
    return int(min(max(i + skv - sq + 1, 0), skv))


# ---------------------------------------------------------------- golden, by hand
def _golden_cases():
    with open(os.path.join(GOLDEN, "handworked_cases.json")) as f:
        return json.load(f)["cases"]


@pytest.mark.parametrize("case", _golden_cases(), ids=lambda c: c["name"])
def test_handworked_golden(case, orc=None):
    o, lse = oracle.attention_fwd(_bhsd(case["q"]), _bhsd(case["k"]), _bhsd(case["v"]),
                                  case["scale"], case["causal"], lib=orc)
    exp_o = np.array(case["o"], dtype=np.float64)
    exp_lse = np.array([-np.inf if x == "-inf" else x for x in case["lse"]], dtype=np.float64)
    np.testing.assert_allclose(o[0, 0], exp_o, rtol=1e-12, atol=1e-12)
    fin = np.isfinite(exp_lse)
    assert np.array_equal(np.isneginf(lse[0, 0]), ~fin)
    np.testing.assert_allclose(lse[0, 0][fin], exp_lse[fin], rtol=1e-12, atol=1e-12)
    # empty rows are +0.0 exactly
    for i in np.where(~fin)[0]:
        assert np.all(o[0, 0, i] == 0.0) and not np.any(np.signbit(o[0, 0, i]))


# ---------------------------------------------------------------- special cases
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("sq,skv", [(7, 7), (5, 13), (13, 5), (1, 9), (33, 33)])
def test_q_zero_gives_prefix_mean_of_v(sq, skv, causal):
    (q, k, v), _ = gen.random_case(11, (2, 3, sq, 8), (2, 3, skv, 8))
    q[:] = 0.0
    o, lse = oracle.attention_fwd(q, k, v, 0.37, causal)
    vl = v.astype(np.longdouble)
    csum = np.cumsum(vl, axis=2)
    for i in range(sq):
        hi = _allowed(i, sq, skv, causal)
        if hi == 0:
            assert np.all(o[:, :, i] == 0.0) and np.all(np.isneginf(lse[:, :, i]))
            continue
        mean = (csum[:, :, hi - 1] / hi).astype(np.float64)
        np.testing.assert_allclose(o[:, :, i], mean, rtol=1e-13, atol=1e-13)
        np.testing.assert_allclose(lse[:, :, i], math.log(hi), rtol=1e-14, atol=1e-14)


@pytest.mark.parametrize("sq", [1, 4, 9])
def test_single_key_returns_v_exactly(sq):
    (q, k, v), _ = gen.random_case(12, (2, 2, sq, 16), (2, 2, 1, 16))
    scale = 0.25
    o, lse = oracle.attention_fwd(q, k, v, scale, False)
    assert np.array_equal(o, np.broadcast_to(v.astype(np.float64), o.shape))
    dots = np.einsum("bhid,bhd->bhi", q.astype(np.float64), k[:, :, 0].astype(np.float64))
    np.testing.assert_allclose(lse, scale * dots, rtol=1e-13, atol=1e-13)
    # causal, bottom-right: only the last query row sees the key
    oc, lc = oracle.attention_fwd(q, k, v, scale, True)
    assert np.all(oc[:, :, : sq - 1] == 0.0) and np.all(np.isneginf(lc[:, :, : sq - 1]))
    assert np.array_equal(oc[:, :, sq - 1], v[:, :, 0].astype(np.float64))


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("sq,skv", [(16, 16), (6, 20), (20, 6)])
def test_probabilities_are_row_stochastic_and_masked(sq, skv, causal):
    (q, k, _), _ = gen.random_case(13, (1, 1, sq, 32), (1, 1, skv, 32), sigma_qk=2.0)
    p = oracle.softmax_probs(q[0, 0], k[0, 0], 0.3, causal)
    for i in range(sq):
        hi = _allowed(i, sq, skv, causal)
        assert np.all(p[i, hi:] == 0.0)
        if hi == 0:
            assert np.all(p[i] == 0.0)
        else:
            assert abs(p[i].sum() - 1.0) <= 1e-12
            assert np.all(p[i, :hi] > 0.0)


def test_fully_masked_rows_are_zero_even_with_nan_queries():
    sq, skv = 200, 64
    (q, k, v), _ = gen.random_case(14, (1, 2, sq, 16), (1, 2, skv, 16))
    q[:, :, : sq - skv] = np.nan  # these rows see no key; their content must not matter
    o, lse = oracle.attention_fwd(q, k, v, 0.25, True)
    assert np.all(o[:, :, : sq - skv] == 0.0) and not np.any(np.signbit(o[:, :, : sq - skv]))
    assert np.all(np.isneginf(lse[:, :, : sq - skv]))
    assert np.all(np.isfinite(o[:, :, sq - skv:]))


def test_no_keys_at_all():
    (q, _, _), _ = gen.random_case(15, (2, 3, 5, 8), (2, 3, 1, 8))
    k = np.zeros((2, 3, 0, 8), np.float32)
    for causal in (False, True):
        o, lse = oracle.attention_fwd(q, k, k, 0.5, causal)
        assert o.shape == (2, 3, 5, 8) and np.all(o == 0.0) and np.all(np.isneginf(lse))


def test_dominant_key_selects_its_value():
    (q, k, v), _ = gen.random_case(16, (1, 1, 4, 8), (1, 1, 12, 8))
    q[:] = 0.0
    q[..., 0] = 1.0
    k[..., 0] = 0.0
    k[0, 0, 5, 0] = 150.0  # score 150 above every other key at scale 1
    o, lse = oracle.attention_fwd(q, k, v, 1.0, False)
    np.testing.assert_allclose(o[0, 0], np.broadcast_to(v[0, 0, 5], (4, 8)), rtol=0, atol=1e-60)
    np.testing.assert_allclose(lse[0, 0], 150.0, rtol=1e-15)


# ---------------------------------------------------------------- brute force
def _brute_force(q, k, v, scale, causal):
    """Textbook softmax in long double, no max subtraction, full score matrix."""
    q = q.astype(np.longdouble)
    k = k.astype(np.longdouble)
    v = v.astype(np.longdouble)
    B, H, sq, d = q.shape
    skv = k.shape[2]
    o = np.zeros((B, H, sq, d), dtype=np.longdouble)
    lse = np.full((B, H, sq), -np.inf, dtype=np.longdouble)
    for b in range(B):
        for h in range(H):
            s = (q[b, h] @ k[b, h].T) * np.longdouble(scale)
            for i in range(sq):
                hi = _allowed(i, sq, skv, causal)
                if hi == 0:
                    continue
                e = np.exp(s[i, :hi])
                tot = e.sum()
                o[b, h, i] = (e[:, None] * v[b, h, :hi]).sum(axis=0) / tot
                lse[b, h, i] = np.log(tot)
    return o, lse


_GRID = [(B, H, sq, skv, d, c)
         for B in (1, 2) for H in (1, 3) for sq in (1, 2, 3, 5, 17) for skv in (0, 1, 2, 3, 7, 33)
         for d in (1, 2, 4, 8) for c in (False, True)]


@pytest.mark.parametrize("B,H,sq,skv,d,causal", _GRID[::3] + _GRID[1::7])
def test_brute_force_tiny_grid(B, H, sq, skv, d, causal):
    seed = 1000 + B * 7 + H * 31 + sq * 101 + skv * 1009 + d * 10007 + causal
    (q, k, v), _ = gen.random_case(seed, (B, H, sq, d), (B, H, skv, d))
    scale = 0.9 / math.sqrt(d)
    o, lse = oracle.attention_fwd(q, k, v, scale, causal)
    ob, lb = _brute_force(q, k, v, scale, causal)
    np.testing.assert_allclose(o, ob.astype(np.float64), rtol=1e-12, atol=1e-12)
    assert np.array_equal(np.isneginf(lse), np.isneginf(lb.astype(np.float64)))
    f = np.isfinite(lse)
    np.testing.assert_allclose(lse[f], lb.astype(np.float64)[f], rtol=1e-12, atol=1e-12)


# ---------------------------------------------------------------- library routine
def _bottom_right_mask(sq, skv):
    i = np.arange(sq)[:, None]
    j = np.arange(skv)[None, :]
    return j <= i + (skv - sq)


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("B,H,sq,skv,d", [(1, 2, 128, 128, 64), (2, 2, 96, 300, 128),
                                          (1, 3, 300, 96, 64), (2, 1, 257, 257, 128)])
def test_matches_torch_sdpa_float64(B, H, sq, skv, d, causal):
    torch = pytest.importorskip("torch")
    from scipy.special import logsumexp

    (q, k, v), _ = gen.random_case(17 + sq + skv, (B, H, sq, d), (B, H, skv, d), sigma_qk=1.5)
    scale = 1.0 / math.sqrt(d)
    o, lse = oracle.attention_fwd(q, k, v, scale, causal)
    tq, tk, tv = (torch.from_numpy(x.astype(np.float64)) for x in (q, k, v))
    mask = torch.from_numpy(_bottom_right_mask(sq, skv)) if causal else None
    ref = torch.nn.functional.scaled_dot_product_attention(tq, tk, tv, attn_mask=mask, scale=scale)
    ref = ref.numpy()
    rows_ok = np.array([_allowed(i, sq, skv, causal) > 0 for i in range(sq)])
    np.testing.assert_allclose(o[:, :, rows_ok], ref[:, :, rows_ok], rtol=1e-11, atol=1e-12)
    s = np.einsum("bhid,bhjd->bhij", q.astype(np.float64), k.astype(np.float64)) * scale
    if causal:
        s = np.where(_bottom_right_mask(sq, skv), s, -np.inf)
    with np.errstate(divide="ignore"):
        ref_lse = logsumexp(s, axis=-1)
    np.testing.assert_allclose(lse[:, :, rows_ok], ref_lse[:, :, rows_ok], rtol=1e-12, atol=1e-12)
    assert np.all(np.isneginf(lse[:, :, ~rows_ok]))


# ---------------------------------------------------------------- invariances
def test_key_shift_invariance_at_overflow_scale():
    """Adding one vector u to every key shifts each row's scores by scale*q.u: O is unchanged.

    The shift is ~200, beyond float32 exp's range, so only a max-subtracted
    evaluation stays finite in single precision; the oracle (double) must agree
    with the unshifted result and move LSE by exactly that amount.
    """
    (q, k, v), _ = gen.random_case(18, (1, 2, 24, 16), (1, 2, 40, 16))
    scale = 0.25
    u = np.zeros(16, np.float32)
    u[0] = 64.0
    q[..., 0] = np.abs(q[..., 0]) + 12.5  # scale * q0 * 64 >= 200
    k[..., 0] = 0.0  # so that k + u is exact in float32
    o0, l0 = oracle.attention_fwd(q, k, v, scale, True)
    o1, l1 = oracle.attention_fwd(q, (k + u).astype(np.float32), v, scale, True)
    shift = scale * (q.astype(np.float64) @ u.astype(np.float64))
    assert shift.min() >= 200.0
    np.testing.assert_allclose(o1, o0, rtol=1e-9, atol=1e-9)
    np.testing.assert_allclose(l1, l0 + shift, rtol=1e-12, atol=1e-9)


def test_scores_beyond_double_exp_range():
    """Scores near 1000 overflow exp even in double unless the row max is subtracted first."""
    (q, k, v), _ = gen.random_case(25, (1, 1, 6, 8), (1, 1, 9, 8))
    k[..., 0] = 0.0
    q[..., 0] = 1.0
    o0, l0 = oracle.attention_fwd(q, k, v, 1.0, False)
    k2 = k.copy()
    k2[..., 0] = 1000.0  # every score moves up by exactly 1000
    o1, l1 = oracle.attention_fwd(q, k2, v, 1.0, False)
    assert np.all(np.isfinite(o1))
    np.testing.assert_allclose(o1, o0, rtol=1e-9, atol=1e-9)
    np.testing.assert_allclose(l1, l0 + 1000.0, rtol=1e-13)


def test_joint_key_value_permutation_invariance():
    (q, k, v), _ = gen.random_case(19, (2, 2, 10, 8), (2, 2, 23, 8))
    perm = np.random.default_rng(3).permutation(23)
    o0, l0 = oracle.attention_fwd(q, k, v, 0.4, False)
    o1, l1 = oracle.attention_fwd(q, k[:, :, perm], v[:, :, perm], 0.4, False)
    np.testing.assert_allclose(o1, o0, rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(l1, l0, rtol=1e-13, atol=1e-13)


def test_query_rescale_against_scale():
    (q, k, v), _ = gen.random_case(20, (1, 2, 12, 8), (1, 2, 12, 8))
    o0, l0 = oracle.attention_fwd(q, k, v, 0.3, True)
    o1, l1 = oracle.attention_fwd((q * 4.0).astype(np.float32), k, v, 0.3 / 4.0, True)
    np.testing.assert_allclose(o1, o0, rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(l1, l0, rtol=1e-12, atol=1e-13)


def test_causal_single_query_equals_unmasked():
    (q, k, v), _ = gen.random_case(21, (2, 2, 1, 8), (2, 2, 17, 8))
    o0, l0 = oracle.attention_fwd(q, k, v, 0.3, False)
    o1, l1 = oracle.attention_fwd(q, k, v, 0.3, True)
    assert np.array_equal(o0, o1) and np.array_equal(l0, l1)


@pytest.mark.parametrize("sq", [1, 5, 17, 40])
def test_bottom_right_slicing(sq):
    """Causal O for the last sq queries equals the tail of the square causal problem."""
    skv = 40
    (qf, k, v), _ = gen.random_case(22, (1, 2, skv, 8), (1, 2, skv, 8))
    of, lf = oracle.attention_fwd(qf, k, v, 0.35, True)
    q = np.ascontiguousarray(qf[:, :, skv - sq:])
    o, l = oracle.attention_fwd(q, k, v, 0.35, True)
    assert np.array_equal(o, of[:, :, skv - sq:]) and np.array_equal(l, lf[:, :, skv - sq:])


def test_sampled_rows_match_full_run():
    (q, k, v), _ = gen.random_case(23, (2, 3, 33, 16), (2, 3, 41, 16))
    of, lf = oracle.attention_fwd(q, k, v, 0.2, True)
    rows = np.array([0, 5, 32, 33, 100, 197], dtype=np.int64)
    o, l = oracle.attention_fwd(q, k, v, 0.2, True, rows=rows)
    assert np.array_equal(o, of.reshape(-1, 16)[rows]) and np.array_equal(l, lf.reshape(-1)[rows])


def test_rejects_bad_arguments():
    (q, k, v), _ = gen.random_case(24, (1, 1, 4, 8), (1, 1, 4, 8))
    with pytest.raises(ValueError):
        oracle.attention_fwd(q, k, v, 0.5, False, rows=np.array([4], dtype=np.int64))
