"""bf16 attention backward (bf16 Q, K, V on 16-bit MFMA; fp32 O, dO, LSE and gradients)
against the oracle's gradients, element by element, through the C ABI.

The GPU backward consumes the GPU bf16 forward's O and LSE, as a training step would; the
oracle recomputes every gradient in double from the exact bf16 values of Q, K, V and the
fp32 dO.

Parity bar (derived): the kernels round three factors to bf16 (8 significant bits, unit
roundoff u = 2^-8): dO (for dP and dV), P (for dV) and dS (for dK and dQ). Each term of a
gradient then carries a relative error of at most about 2u (to first order) beyond the fp32
rounding, relative to the magnitudes the oracle's error scale M sums
(oracle.attention_bwd_bound: every factor in magnitude, |dP| and |D| bounded by dPmag and
Dmag, each P weighted by the size of its exponent). So elementwise
|gpu - ref| <= BF16_GRAD_TAU * M with BF16_GRAD_TAU = 2u = 2^-7, that bound; an element
whose M is 0 must be exactly 0. Per tensor, the roundings of independent terms add up like a
random walk, far below their sum of magnitudes: ||gpu - ref||_2 <= BF16_GRAD_L2 * ||M||_2
with BF16_GRAD_L2 = u/2.
"""
import functools
import math

import numpy as np
import pytest

import gen
import helpers
import oracle
from helpers import empty_rows, to_device, workload_case

pytestmark = pytest.mark.gpu

BF16_GRAD_TAU = 2.0**-7
BF16_GRAD_L2 = 2.0**-9


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    torch = pytest.importorskip("torch")
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import scaled_masked_attention_amd as sma

    sma.library()  # fail loudly if the HIP library is missing


def _gpu_grads(bits, g, scale, causal, ws_fill=None):
    """bf16 forward then backward on the GPU; returns (dq, dk, dv) as float64 numpy arrays."""
    import torch

    import scaled_masked_attention_amd as sma

    tq, tk, tv = to_device(None, bits, "bf16")
    tg = torch.from_numpy(np.ascontiguousarray(g)).to("cuda")
    o, lse = sma.attention_fwd(tq, tk, tv, scale=scale, causal=causal, return_lse=True)
    ws = None
    if ws_fill is not None:
        B, H, sq, d = tq.shape
        n = sma.attention_bwd_workspace_bytes(sma.SMA_DTYPE_BF16, B, H, sq, tk.shape[2], d, causal)
        ws = torch.full((max(n, 4) // 4,), ws_fill, dtype=torch.float32, device="cuda")
    dq, dk, dv = sma.attention_bwd(tq, tk, tv, o, lse, tg, scale=scale, causal=causal, workspace=ws)
    torch.cuda.synchronize()
    assert dq.dtype == dk.dtype == dv.dtype == torch.float32
    return tuple(t.cpu().numpy().astype(np.float64) for t in (dq, dk, dv))


def check_grads(got, ref, bound, label):
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
        assert worst <= BF16_GRAD_TAU, (f"{label}: {name} error {err[idx]:.3e} at {idx} is {worst:.3e} of "
                                        f"its scale {m[idx]:.3e} (bar {BF16_GRAD_TAU:.3e})")
        d2, r2, m2 = (float(np.linalg.norm(x)) for x in (a - b, b, m))
        assert d2 <= BF16_GRAD_L2 * m2, f"{label}: {name} L2 error {d2:.3e} > {BF16_GRAD_L2:.3e} * ||M|| {m2:.3e}"
        helpers.bwd_regression("bf16", worst / BF16_GRAD_TAU, d2 / (BF16_GRAD_L2 * m2) if m2 > 0 else 0.0,
                               f"{label} {name}")
        stats[name] = dict(err_over_scale=worst, l2_over_m=d2 / m2 if m2 > 0 else None,
                           rel_l2=d2 / r2 if r2 > 0 else None)
    return stats


def _case(seed, B, H, sq, skv, d, sigma_qk=1.0, sigma_g=1.0):
    (q, k, v), bits = gen.random_case(seed, (B, H, sq, d), (B, H, skv, d), sigma_qk=sigma_qk, dtype="bf16")
    g = gen.upstream_grad(seed, (B, H, sq, d), sigma_g)
    return (q, k, v), bits, g


def _oracle(q, k, v, g, scale, causal):
    return (oracle.attention_bwd(q, k, v, g, scale, causal),
            oracle.attention_bwd_bound(q, k, v, g, scale, causal))


SHAPES = [  # (B, H, sq, skv): several blocks with ragged tails, cross shapes both ways
    (1, 2, 128, 128), (2, 3, 200, 200), (1, 2, 77, 300), (2, 1, 300, 77), (1, 1, 1, 1000),
    (1, 1, 1000, 1), (1, 1, 513, 513), (3, 2, 64, 96), (1, 4, 257, 1025),
]


@functools.lru_cache(maxsize=4)
def _small(shape, causal, d):
    B, H, sq, skv = shape
    (q, k, v), bits, g = _case(700 + sq + 7 * skv + d, B, H, sq, skv, d)
    scale = 1.0 / math.sqrt(d)
    return bits, g, scale, _oracle(q, k, v, g, scale, causal)


@pytest.mark.parametrize("d", [32, 64, 128, 256])
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("shape", SHAPES, ids=lambda s: "x".join(map(str, s)))
def test_bwd_bf16_parity_small(shape, causal, d):
    bits, g, scale, (ref, bound) = _small(shape, causal, d)
    got = _gpu_grads(bits, g, scale, causal)
    print(shape, causal, d, check_grads(got, ref, bound, f"{shape} causal={causal} d={d}"))


@pytest.mark.parametrize("d", [32, 64, 128, 256])
def test_bwd_bf16_rows_without_keys(d):
    """Causal with more queries than keys: the first sq - skv rows admit nothing."""
    (q, k, v), bits, g = _case(801 + d, 1, 2, 150, 100, d)
    got = _gpu_grads(bits, g, 0.2, True)
    ref, bound = _oracle(q, k, v, g, 0.2, True)
    er = empty_rows(150, 100, True)
    assert np.all(got[0][:, :, er] == 0.0)
    check_grads(got, ref, bound, "empty rows")


@pytest.mark.parametrize("d", [32, 64, 128, 256])
def test_bwd_bf16_no_keys_and_no_queries(d):
    import torch

    import scaled_masked_attention_amd as sma

    tq = torch.randn(1, 2, 40, d, device="cuda").to(torch.bfloat16)
    tk = torch.empty(1, 2, 0, d, device="cuda", dtype=torch.bfloat16)
    o, lse = sma.attention_fwd(tq, tk, tk, return_lse=True)
    dq, dk, dv = sma.attention_bwd(tq, tk, tk, o, lse, torch.randn(1, 2, 40, d, device="cuda"))
    torch.cuda.synchronize()
    assert torch.all(dq == 0) and not torch.any(torch.signbit(dq)) and dk.numel() == dv.numel() == 0
    tq0 = torch.empty(1, 2, 0, d, device="cuda", dtype=torch.bfloat16)
    tk = torch.randn(1, 2, 50, d, device="cuda").to(torch.bfloat16)
    o0 = torch.empty(1, 2, 0, d, device="cuda")
    lse0 = torch.empty(1, 2, 0, device="cuda")
    dq, dk, dv = sma.attention_bwd(tq0, tk, tk, o0, lse0, o0)
    torch.cuda.synchronize()
    assert dq.numel() == 0 and torch.all(dk == 0) and torch.all(dv == 0)


@pytest.mark.parametrize("causal", [False, True])
def test_bwd_bf16_zero_upstream_gradient_is_exactly_zero(causal):
    (q, k, v), bits, g = _case(802, 1, 2, 100, 130, 64)
    got = _gpu_grads(bits, np.zeros_like(g), 0.125, causal)
    for t in got:
        assert np.all(t == 0.0)


@pytest.mark.parametrize("scale", [0.0, -0.15])
def test_bwd_bf16_scale_sign_and_zero(scale):
    (q, k, v), bits, g = _case(803, 1, 2, 96, 140, 128)
    got = _gpu_grads(bits, g, scale, True)
    ref, bound = _oracle(q, k, v, g, scale, True)
    check_grads(got, ref, bound, f"scale={scale}")


def test_bwd_bf16_sharp_softmax():
    (q, k, v), bits, g = _case(804, 1, 2, 130, 150, 128, sigma_qk=3.0)
    got = _gpu_grads(bits, g, 1.0 / math.sqrt(128), True)
    ref, bound = _oracle(q, k, v, g, 1.0 / math.sqrt(128), True)
    check_grads(got, ref, bound, "sharp")


def test_bwd_bf16_is_deterministic_and_ignores_workspace_contents():
    (q, k, v), bits, g = _case(805, 2, 2, 200, 230, 64)
    a = _gpu_grads(bits, g, 0.125, True)
    b = _gpu_grads(bits, g, 0.125, True, ws_fill=float("nan"))
    for x, y in zip(a, b):
        assert np.array_equal(x, y)


def test_bwd_bf16_matches_fp32_backward_on_bf16_values():
    """The same bf16-exact inputs through the fp32 backward: the two differ only by the
    bf16 roundings, inside the bar against the oracle for both."""
    import torch

    import scaled_masked_attention_amd as sma

    (q, k, v), bits, g = _case(806, 1, 3, 190, 210, 128)
    got16 = _gpu_grads(bits, g, 0.09, True)
    tq, tk, tv, tg = (torch.from_numpy(np.ascontiguousarray(x)).to("cuda") for x in (q, k, v, g))
    o, lse = sma.attention_fwd(tq, tk, tv, scale=0.09, causal=True, return_lse=True)
    got32 = tuple(t.cpu().numpy().astype(np.float64)
                  for t in sma.attention_bwd(tq, tk, tv, o, lse, tg, scale=0.09, causal=True))
    ref, bound = _oracle(q, k, v, g, 0.09, True)
    check_grads(got16, ref, bound, "bf16")
    check_grads(got32, ref, bound, "fp32")


def test_bwd_bf16_binding_checks():
    import torch

    import scaled_masked_attention_amd as sma

    q = torch.randn(1, 1, 8, 64, device="cuda").to(torch.bfloat16)
    o = torch.zeros(1, 1, 8, 64, device="cuda")
    lse = torch.zeros(1, 1, 8, device="cuda")
    with pytest.raises(ValueError):  # mixed input dtypes
        sma.attention_bwd(q, q.float(), q, o, lse, o)
    with pytest.raises(ValueError):  # bf16 and fp16 mixed
        sma.attention_bwd(q.half(), q, q, o, lse, o)
    with pytest.raises(ValueError):  # dO must be fp32
        sma.attention_bwd(q, q, q, o, lse, o.to(torch.bfloat16))


@pytest.mark.parametrize("name", ["bf16_causal_b1h32_s16384_d128", "bf16_causal_b1h32_s16384_d256"])
def test_bwd_bf16_full_size_exact_subproblems(name):
    """The full workload in one launch sequence; exact oracle values from sub-problems that
    bottom-right causal alignment keeps intact. The last T query rows with every key form a
    causal problem (Sq = T, Skv = S) whose row i' admits keys up to i' + S - T, as in the
    full one; it holds every query that admits a key >= S - T, so its oracle gives the
    exact dQ of those rows and dK, dV of those keys. A single row i with keys 0..i
    (unmasked) gives the exact dQ of row i."""
    import torch

    import scaled_masked_attention_amd as sma

    w, vals, bits = workload_case(name)
    assert w.causal and w.seq_q == w.seq_kv
    S, T = w.seq_q, 64
    g = gen.upstream_grad(w.seed, w.q_shape)
    tq, tk, tv = to_device(vals, bits, w.dtype)
    o, lse = sma.attention_fwd(tq, tk, tv, scale=w.scale, causal=True, return_lse=True)
    tg = torch.from_numpy(g).to("cuda")
    dq, dk, dv = sma.attention_bwd(tq, tk, tv, o, lse, tg, scale=w.scale, causal=True)
    torch.cuda.synchronize()
    dq, dk, dv = (t.cpu().numpy().astype(np.float64) for t in (dq, dk, dv))
    assert all(np.all(np.isfinite(t)) for t in (dq, dk, dv))
    q, k, v = vals
    for h in (0, w.heads - 1):
        sub = (slice(0, 1), slice(h, h + 1))
        last = sub + (slice(S - T, S),)
        ref, bound = _oracle(q[last], k[sub], v[sub], g[last], w.scale, True)
        got = (dq[last], dk[last], dv[last])
        ref = (ref[0], ref[1][:, :, S - T:], ref[2][:, :, S - T:])
        bound = (bound[0], bound[1][:, :, S - T:], bound[2][:, :, S - T:])
        print(name, h, "last rows/keys", check_grads(got, ref, bound, f"{name} head {h} last {T}"))
        for i in (0, 1, 777, S // 2):
            row = sub + (slice(i, i + 1),)
            keys = sub + (slice(0, i + 1),)
            (rq, _, _), (mq, _, _) = _oracle(q[row], k[keys], v[keys], g[row], w.scale, False)
            e = np.abs(dq[row] - rq)
            assert np.all(e <= BF16_GRAD_TAU * mq), (name, h, i, float((e / np.maximum(mq, 1e-300)).max()))
