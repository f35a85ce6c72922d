"""Pins of the masked attention-forward oracle against facts it does not compute itself.

scipy's float64 softmax and logsumexp over each row's admitted entries (numpy for the
products), the causal mask written as an explicit mask, a single admitted key, rows that
admit nothing, masked keys whose K and V are NaN, broadcasting of the mask, and a shift of
every score past exp's range. test_masked_oracle_mutations.py plants the plausible slips and
checks that each fails one of these.
"""
import numpy as np
import pytest

import oracle

sp = pytest.importorskip("scipy.special")


def _inputs(seed, B, H, sq, skv, d, sigma=1.0):
    rng = np.random.default_rng(seed)
    q = (rng.normal(size=(B, H, sq, d)) * sigma).astype(np.float32)
    k = (rng.normal(size=(B, H, skv, d)) * sigma).astype(np.float32)
    v = rng.normal(size=(B, H, skv, d)).astype(np.float32)
    return q, k, v


def _reference(q, k, v, mask, scale, causal):
    """numpy/scipy float64: softmax over the admitted entries of each row."""
    B, H, sq, d = q.shape
    skv = k.shape[2]
    m = np.broadcast_to(np.asarray(mask) != 0, (B, H, sq, skv))
    o = np.zeros((B, H, sq, d))
    lse = np.full((B, H, sq), -np.inf)
    for b in range(B):
        for h in range(H):
            s = scale * (q[b, h].astype(np.float64) @ k[b, h].astype(np.float64).T)
            for i in range(sq):
                adm = m[b, h, i].copy()
                if causal:
                    adm &= np.arange(skv) <= i + skv - sq
                if adm.any():
                    p = sp.softmax(s[i, adm])
                    o[b, h, i] = p @ v[b, h][adm].astype(np.float64)
                    lse[b, h, i] = sp.logsumexp(s[i, adm])
    return o, lse


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("density", [0.05, 0.5, 0.95])
def test_matches_scipy_on_the_admitted_entries(density, causal):
    q, k, v = _inputs(int(density * 100) + causal, 2, 2, 13, 17, 8)
    mask = np.random.default_rng(7).random((2, 2, 13, 17)) < density
    o, lse = oracle.attention_fwd_masked(q, k, v, mask, 0.4, causal)
    o_ref, lse_ref = _reference(q, k, v, mask, 0.4, causal)
    assert np.abs(o - o_ref).max() <= 1e-13
    fin = np.isfinite(lse_ref)
    assert np.array_equal(np.isfinite(lse), fin)
    assert np.abs(lse[fin] - lse_ref[fin]).max() <= 1e-13


@pytest.mark.parametrize("sq,skv", [(9, 9), (5, 11), (11, 5)])
def test_causal_pattern_as_a_mask_equals_the_causal_flag(sq, skv):
    q, k, v = _inputs(sq * 31 + skv, 1, 2, sq, skv, 4)
    pattern = (np.arange(skv)[None, :] <= np.arange(sq)[:, None] + skv - sq)[None, None]
    o1, l1 = oracle.attention_fwd_masked(q, k, v, pattern, 0.5, False)
    o2, l2 = oracle.attention_fwd(q, k, v, 0.5, True)
    assert np.array_equal(o1, o2) and np.array_equal(l1, l2)
    o3, l3 = oracle.attention_fwd_masked(q, k, v, np.ones((1, 1, sq, skv)), 0.5, True)
    assert np.array_equal(o3, o2) and np.array_equal(l3, l2)


def test_single_admitted_key_returns_its_value_row():
    q, k, v = _inputs(3, 1, 1, 6, 10, 8)
    mask = np.zeros((1, 1, 6, 10), bool)
    for i in range(6):
        mask[0, 0, i, (3 * i) % 10] = True
    o, lse = oracle.attention_fwd_masked(q, k, v, mask, 0.3, False)
    for i in range(6):
        j = (3 * i) % 10
        assert np.array_equal(o[0, 0, i], v[0, 0, j].astype(np.float64))
        s = 0.3 * float(np.dot(q[0, 0, i].astype(np.float64), k[0, 0, j].astype(np.float64)))
        assert abs(lse[0, 0, i] - s) <= 1e-14 * max(1.0, abs(s))


def test_rows_admitting_nothing_are_zero_and_masked_keys_are_never_read():
    q, k, v = _inputs(4, 1, 2, 7, 9, 4)
    mask = np.random.default_rng(4).random((1, 2, 7, 9)) < 0.4
    mask[0, 1, 2] = False
    mask[..., 5] = False           # key 5 admitted nowhere: its K and V may be anything
    k2, v2 = k.copy(), v.copy()
    k2[:, :, 5] = np.nan
    v2[:, :, 5] = np.inf
    o, lse = oracle.attention_fwd_masked(q, k2, v2, mask, 0.7, False)
    o_ref, lse_ref = oracle.attention_fwd_masked(q, k, v, mask, 0.7, False)
    assert np.array_equal(o, o_ref) and np.array_equal(lse, lse_ref)
    assert np.all(o[0, 1, 2] == 0.0) and lse[0, 1, 2] == -np.inf


def test_broadcast_mask_equals_the_repeated_mask():
    q, k, v = _inputs(5, 2, 3, 6, 8, 4)
    m = np.random.default_rng(5).random((1, 1, 6, 8)) < 0.6
    o1, l1 = oracle.attention_fwd_masked(q, k, v, m, 0.5, True)
    o2, l2 = oracle.attention_fwd_masked(q, k, v, np.repeat(np.repeat(m, 2, 0), 3, 1), 0.5, True)
    assert np.array_equal(o1, o2) and np.array_equal(l1, l2)
    mh = np.random.default_rng(6).random((1, 3, 6, 8)) < 0.6  # per head, shared by the batch
    o3, _ = oracle.attention_fwd_masked(q, k, v, mh, 0.5, False)
    o4, _ = oracle.attention_fwd_masked(q, k, v, np.repeat(mh, 2, 0), 0.5, False)
    assert np.array_equal(o3, o4)


def test_mask_and_causal_combine_by_and():
    q, k, v = _inputs(6, 1, 1, 8, 8, 4)
    m = np.random.default_rng(8).random((1, 1, 8, 8)) < 0.7
    both = m & (np.arange(8)[None, :] <= np.arange(8)[:, None])[None, None]
    o1, l1 = oracle.attention_fwd_masked(q, k, v, m, 0.5, True)
    o2, l2 = oracle.attention_fwd_masked(q, k, v, both, 0.5, False)
    assert np.array_equal(o1, o2) and np.array_equal(l1, l2)


def test_scores_beyond_the_exp_range():
    """Every admitted score shifted by ~1500: only a max-subtracted softmax stays finite."""
    q, k, v = _inputs(9, 1, 1, 5, 12, 4)
    q[..., 0] = 40.0
    k[..., 0] = 40.0
    mask = np.random.default_rng(9).random((1, 1, 5, 12)) < 0.5
    mask[..., 0] = True
    o, lse = oracle.attention_fwd_masked(q, k, v, mask, 1.0, False)
    o_ref, lse_ref = _reference(q, k, v, mask, 1.0, False)
    assert np.all(np.isfinite(o)) and lse.min() > 1000
    assert np.abs(o - o_ref).max() <= 1e-12


def test_rejects_bad_mask_shapes():
    q, k, v = _inputs(10, 1, 2, 4, 5, 4)
    with pytest.raises(ValueError):
        oracle.attention_fwd_masked(q, k, v, np.ones((4, 5), bool), 1.0, False)
    with pytest.raises(ValueError):
        oracle.attention_fwd_masked(q, k, v, np.ones((1, 3, 4, 5), bool), 1.0, False)
