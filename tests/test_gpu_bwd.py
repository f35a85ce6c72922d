"""HIP attention backward vs the oracle's gradients, element by element, through the C ABI.

The GPU backward consumes the GPU forward's O and LSE, as a training step
would; the oracle recomputes every gradient from Q, K, V and dO in double.
Small and ragged shapes compare every element; the full-size workloads
compare every element of a few whole (batch, head) slices (each gradient of a
head depends only on that head) plus properties that hold everywhere.
"""
import functools
import math

import numpy as np
import pytest

import gen
import helpers
import oracle
from helpers import empty_rows, workload_case

pytestmark = pytest.mark.gpu

# Parity bars for the fp32 gradients, with M the oracle's error scale of each element (the
# gradient's sum with every factor in magnitude and each probability weighted by the size of
# its exponent, oracle.attention_bwd_bound):
#  elementwise  |gpu - ref| <= GRAD_TAU * M  (an element whose M is 0 must be exactly 0);
#  per tensor   ||gpu - ref||_2 <= GRAD_REL_L2 * ||ref||_2 + GRAD_NOISE * ||M||_2, the second
#               term allowing the rounding noise of sums that cancel (about 2 ulp per term).
GRAD_TAU = 1e-5
GRAD_REL_L2 = 1e-5
GRAD_NOISE = 1e-7


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    torch = pytest.importorskip("torch")
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import scaled_masked_attention_amd as sma

    sma.library()  # fail loudly if the HIP library is missing


def _gpu_grads(q, k, v, g, scale, causal, ws_fill=None):
    """Forward then backward on the GPU; returns (dq, dk, dv) as float64 numpy arrays."""
    import torch

    import scaled_masked_attention_amd as sma

    tq, tk, tv, tg = (torch.from_numpy(np.ascontiguousarray(x)).to("cuda") for x in (q, k, v, g))
    o, lse = sma.attention_fwd(tq, tk, tv, scale=scale, causal=causal, return_lse=True)
    ws = None
    if ws_fill is not None:
        B, H, sq, d = q.shape
        n = sma.attention_bwd_workspace_bytes(sma.SMA_DTYPE_F32, B, H, sq, k.shape[2], d, causal)
        ws = torch.full((max(n, 4) // 4,), ws_fill, dtype=torch.float32, device="cuda")
    dq, dk, dv = sma.attention_bwd(tq, tk, tv, o, lse, tg, scale=scale, causal=causal, workspace=ws)
    torch.cuda.synchronize()
    return tuple(t.cpu().numpy().astype(np.float64) for t in (dq, dk, dv))


def check_grads(got, ref, bound, label):
    """Elementwise |got - ref| <= GRAD_TAU * bound for (dq, dk, dv); returns per-gradient stats."""
    stats = {}
    for name, a, b, m in zip(("dq", "dk", "dv"), got, ref, bound):
        assert a.shape == b.shape == m.shape, (label, name, a.shape, b.shape, m.shape)
        assert np.all(np.isfinite(a)), f"{label}: non-finite {name}"
        if not a.size:
            continue
        err = np.abs(a - b)
        zero = m == 0
        assert np.all(a[zero] == 0.0), f"{label}: {name} nonzero where every term is zero"
        ratio = np.where(zero, 0.0, err / np.where(zero, 1.0, m))
        worst = float(ratio.max())
        idx = np.unravel_index(int(ratio.argmax()), ratio.shape)
        assert worst <= GRAD_TAU, (f"{label}: {name} error {err[idx]:.3e} at {idx} is {worst:.3e} of its "
                                   f"scale {m[idx]:.3e} (bar {GRAD_TAU})")
        d2, r2, m2 = (float(np.linalg.norm(x)) for x in (a - b, b, m))
        bar2 = GRAD_REL_L2 * r2 + GRAD_NOISE * m2
        assert d2 <= bar2, f"{label}: {name} L2 error {d2:.3e} > {bar2:.3e} (||ref|| {r2:.3e}, ||M|| {m2:.3e})"
        helpers.bwd_regression("f32", worst / GRAD_TAU, d2 / bar2 if bar2 > 0 else 0.0, f"{label} {name}")
        stats[name] = dict(err_over_scale=worst, rel_l2=d2 / r2 if r2 > 0 else None,
                           max_abs=float(err.max()), max_ref=float(np.abs(b).max()))
    return stats


def _oracle(q, k, v, g, scale, causal):
    return (oracle.attention_bwd(q, k, v, g, scale, causal),
            oracle.attention_bwd_bound(q, k, v, g, scale, causal))


def _case(seed, B, H, sq, skv, d, sigma_qk=1.0, sigma_g=1.0):
    (q, k, v), _ = gen.random_case(seed, (B, H, sq, d), (B, H, skv, d), sigma_qk=sigma_qk)
    g = gen.upstream_grad(seed, (B, H, sq, d), sigma_g)
    return q, k, v, g


SHAPES = [  # (B, H, sq, skv): several blocks with ragged tails, cross shapes both ways
    (1, 2, 128, 128), (2, 3, 200, 200), (1, 2, 77, 300), (2, 1, 300, 77), (1, 1, 1, 1000),
    (1, 1, 1000, 1), (1, 1, 513, 513), (3, 2, 64, 96), (1, 4, 257, 1025),
]


@functools.lru_cache(maxsize=4)
def _small(shape, causal, d):
    B, H, sq, skv = shape
    q, k, v, g = _case(300 + sq + 7 * skv + d, B, H, sq, skv, d)
    scale = 1.0 / math.sqrt(d)
    return (q, k, v, g), scale, _oracle(q, k, v, g, scale, causal)


@pytest.mark.parametrize("d", [32, 64, 128])
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("shape", SHAPES, ids=lambda s: "x".join(map(str, s)))
def test_bwd_parity_small(shape, causal, d):
    (q, k, v, g), scale, (ref, bound) = _small(shape, causal, d)
    got = _gpu_grads(q, k, v, g, scale, causal)
    stats = check_grads(got, ref, bound, f"{shape} causal={causal} d={d}")
    print(f"{shape} causal={causal} d={d}: {stats}")


@pytest.mark.parametrize("d", [32, 64, 128])
def test_bwd_rows_without_keys(d):
    """Causal with sq > skv: the first sq - skv rows admit no key; their dq is exactly 0."""
    q, k, v, g = _case(41, 1, 2, 150, 60, d)
    scale = 1.0 / math.sqrt(d)
    got = _gpu_grads(q, k, v, g, scale, True)
    check_grads(got, *_oracle(q, k, v, g, scale, True), "rows without keys")
    er = empty_rows(150, 60, True)
    assert er.sum() == 90
    assert np.all(got[0][:, :, er] == 0.0)


@pytest.mark.parametrize("d", [32, 64, 128])
def test_bwd_no_keys_gives_zero_dq(d):
    q, _, _, g = _case(42, 2, 2, 70, 1, d)
    k = np.zeros((2, 2, 0, d), np.float32)
    dq, dk, dv = _gpu_grads(q, k, k, g, 0.3, False)
    assert dk.shape == (2, 2, 0, d) and dv.shape == (2, 2, 0, d)
    assert np.all(dq == 0.0) and not np.any(np.signbit(dq))


@pytest.mark.parametrize("d", [32, 64, 128])
def test_bwd_no_queries_gives_zero_dk_dv(d):
    _, k, v, _ = _case(43, 1, 3, 1, 90, d)
    q = np.zeros((1, 3, 0, d), np.float32)
    dq, dk, dv = _gpu_grads(q, k, v, q, 0.3, True)
    assert dq.shape == (1, 3, 0, d)
    assert np.all(dk == 0.0) and np.all(dv == 0.0)


@pytest.mark.parametrize("causal", [False, True])
def test_bwd_zero_upstream_gradient_is_exactly_zero(causal):
    q, k, v, _ = _case(44, 1, 2, 100, 130, 64)
    for grad in _gpu_grads(q, k, v, np.zeros_like(q), 0.125, causal):
        assert np.all(grad == 0.0)


@pytest.mark.parametrize("scale", [-0.2, 0.0, 0.4])
def test_bwd_scale_sign_and_zero(scale):
    """Negative and zero scales (zero: uniform P over each row's prefix, dq = dk = 0)."""
    q, k, v, g = _case(45, 1, 2, 96, 160, 128)
    got = _gpu_grads(q, k, v, g, scale, True)
    check_grads(got, *_oracle(q, k, v, g, scale, True), f"scale={scale}")
    if scale == 0.0:
        assert np.all(got[0] == 0.0) and np.all(got[1] == 0.0)


def test_bwd_sharp_softmax():
    """Large logits (sigma 3 on q and k, scale 0.25): P close to one-hot in many rows."""
    q, k, v, g = _case(46, 1, 2, 200, 200, 64, sigma_qk=3.0)
    got = _gpu_grads(q, k, v, g, 0.25, True)
    check_grads(got, *_oracle(q, k, v, g, 0.25, True), "sharp")


def test_bwd_is_deterministic_and_ignores_workspace_contents():
    q, k, v, g = _case(47, 2, 2, 300, 333, 128)
    a = _gpu_grads(q, k, v, g, 0.09, True, ws_fill=float("nan"))
    b = _gpu_grads(q, k, v, g, 0.09, True, ws_fill=12345.0)
    c = _gpu_grads(q, k, v, g, 0.09, True)
    for x, y, z in zip(a, b, c):
        assert np.array_equal(x, y) and np.array_equal(x, z)


def _workload_grads(name, heads):
    """GPU gradients of a whole workload, and the oracle's for the (b, h) slices `heads`."""
    w, vals, _ = workload_case(name)
    q, k, v = vals
    g = gen.upstream_grad(w.seed, w.q_shape)
    got = _gpu_grads(q, k, v, g, w.scale, w.causal)
    sl = []
    for b, h in heads:
        sl.append(((b, h), _oracle(q[b:b + 1, h:h + 1], k[b:b + 1, h:h + 1], v[b:b + 1, h:h + 1],
                                   g[b:b + 1, h:h + 1], w.scale, w.causal)))
    return w, got, sl


@pytest.mark.parametrize("name", ["f32_causal_b1h2_s128_d64", "f32_b4h8_s512_d64"])
def test_bwd_parity_small_workloads_full(name):
    w, vals, _ = workload_case(name)
    q, k, v = vals
    g = gen.upstream_grad(w.seed, w.q_shape)
    got = _gpu_grads(q, k, v, g, w.scale, w.causal)
    stats = check_grads(got, *_oracle(q, k, v, g, w.scale, w.causal), name)
    print(f"{name}: {stats}")


@pytest.mark.parametrize("name", ["f32_causal_b8h16_s2048_d128", "f32_cross_b2h32_q256_kv4096_d128",
                                  "f32_cross_causal_b2h32_q256_kv4096_d128"])
def test_bwd_parity_full_size_head_slices(name):
    w = gen.WORKLOADS[name]
    heads = [(0, 0), (w.batch - 1, w.heads - 1)]
    w, got, slices = _workload_grads(name, heads)
    for (b, h), (ref, bound) in slices:
        part = tuple(x[b:b + 1, h:h + 1] for x in got)
        stats = check_grads(part, ref, bound, f"{name} b={b} h={h}")
        print(f"{name} b={b} h={h}: {stats}")
    er = empty_rows(w.seq_q, w.seq_kv, w.causal)
    if er.any():
        assert np.all(got[0][:, :, er] == 0.0)
