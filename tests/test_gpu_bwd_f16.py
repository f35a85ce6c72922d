"""fp16 attention backward (fp16 Q, K, V on 16-bit MFMA; fp32 O, dO, LSE and gradients)
against the oracle's gradients, element by element, through the C ABI.

O and LSE come from the GPU fp32 forward on the same fp16-exact values (its error is a few
fp32 roundings), so the 16-bit roundings under test are the backward's own: dO, P and dS
rounded to fp16 (nearest even) for the products that take them.

Parity bar (derived from fp16's rounding model: 11 significant bits, unit roundoff
u = 2^-11 in the normal range; under 2^-14 the spacing is 2^-24, so a rounding there errs by
at most eta = 2^-25 in absolute terms):
  - The relative part is that of the bf16 backward with fp16's u: each term of a gradient
    carries at most about 2u relative to the magnitudes the oracle's error scale M sums,
    so |gpu - ref| <= 2u M = 2^-10 M, and per tensor ||gpu - ref||_2 <= (u/2) ||M||_2.
  - The absolute part bounds what underflow can add when every rounded factor is taken at
    its largest (P <= 1): over the admitted pairs (i, j),
      dV_jc: sum_i (|dO_ic| + 1)               (P rounded; dO rounded)
      dK_jc: |scale| sum_i |q_ic| (1 + |v_j|_1)  (dS rounded; dO rounded inside dP)
      dQ_ic: |scale| sum_j |k_jc| (1 + |v_j|_1)
    times eta; the tests allow twice that, 2^-24 A, computed here by brute force over the
    admitted pairs (independent of the oracle).
"""
import math

import numpy as np
import pytest

import gen
import helpers
import oracle
from helpers import to_device, workload_case

pytestmark = pytest.mark.gpu

F16_GRAD_TAU = 2.0**-10
F16_GRAD_L2 = 2.0**-12
F16_UNDERFLOW = 2.0**-24


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    torch = pytest.importorskip("torch")
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import scaled_masked_attention_amd as sma

    sma.library()  # fail loudly if the HIP library is missing


def _case(seed, B, H, sq, skv, d):
    (q, k, v), bits = gen.random_case(seed, (B, H, sq, d), (B, H, skv, d), dtype="f16")
    return (q, k, v), bits, gen.upstream_grad(seed, (B, H, sq, d))


def _gpu_grads(vals, bits, g, scale, causal, mask=None, layout="bhsd"):
    """fp32 forward on the fp16-exact values, then the fp16 backward; float64 numpy grads."""
    import torch

    import scaled_masked_attention_amd as sma

    q32, k32, v32, tg = (torch.from_numpy(np.ascontiguousarray(x)).to("cuda") for x in (*vals, g))
    tm = None if mask is None else torch.from_numpy(np.ascontiguousarray(mask)).to("cuda")
    o, lse = sma.attention_fwd(q32, k32, v32, scale=scale, causal=causal, return_lse=True, mask=tm)
    tq, tk, tv = to_device(None, bits, "f16")
    assert tq.dtype == torch.float16
    if layout == "bshd":
        tq, tk, tv, o, tg = (x.transpose(1, 2).contiguous() for x in (tq, tk, tv, o, tg))
    grads = sma.attention_bwd(tq, tk, tv, o, lse, tg, scale=scale, causal=causal, mask=tm, layout=layout)
    torch.cuda.synchronize()
    if layout == "bshd":
        grads = tuple(x.transpose(1, 2) for x in grads)
    assert all(x.dtype == torch.float32 for x in grads)
    return tuple(x.cpu().numpy().astype(np.float64) for x in grads)


def _admitted(sq, skv, causal, mask=None):
    """W[b, h, i, j] = 1 where row i admits key j (bottom-right causal bound and mask)."""
    w = np.ones((1, 1, sq, skv))
    if causal:
        i = np.arange(sq)[:, None]
        j = np.arange(skv)[None, :]
        w = w * (j <= i + (skv - sq))
    if mask is not None:
        w = w * (mask != 0)
    return w


def underflow_scale(q, k, v, g, scale, causal, mask=None):
    """The A of the module docstring, by brute force over the admitted pairs."""
    q, k, v, g = (np.abs(x.astype(np.float64)) for x in (q, k, v, g))
    w = np.broadcast_to(_admitted(q.shape[2], k.shape[2], causal, mask), q.shape[:2] + (q.shape[2], k.shape[2]))
    wt = np.swapaxes(w, -1, -2)
    v1 = 1.0 + v.sum(axis=-1, keepdims=True)
    a_v = wt @ (g + 1.0)
    a_k = abs(scale) * v1 * (wt @ q)
    a_q = abs(scale) * (w @ (k * v1))
    return a_q, a_k, a_v


def check_grads(got, ref, bound, under, label):
    for name, a, b, m, u in zip(("dq", "dk", "dv"), got, ref, bound, under):
        assert a.shape == b.shape == m.shape == u.shape, (label, name)
        assert np.all(np.isfinite(a)), f"{label}: non-finite {name}"
        if not a.size:
            continue
        err = np.abs(a - b)
        zero = m == 0
        assert np.all(a[zero] == 0.0), f"{label}: {name} nonzero where every term is zero"
        bar = F16_GRAD_TAU * m + F16_UNDERFLOW * u
        idx = np.unravel_index(int(np.argmax(err - bar)), err.shape)
        assert np.all(err <= bar), (f"{label}: {name} error {err[idx]:.3e} at {idx} over its bar {bar[idx]:.3e} "
                                    f"(M {m[idx]:.3e}, A {u[idx]:.3e})")
        d2 = float(np.linalg.norm(a - b))
        l2_bar = F16_GRAD_L2 * float(np.linalg.norm(m)) + F16_UNDERFLOW * float(np.linalg.norm(u))
        assert d2 <= l2_bar, f"{label}: {name} L2 error {d2:.3e} > {l2_bar:.3e}"
        pos = bar > 0
        frac = float((err[pos] / bar[pos]).max()) if pos.any() else 0.0
        helpers.bwd_regression("f16", frac, d2 / l2_bar if l2_bar > 0 else 0.0, f"{label} {name}")


SHAPES = [  # (B, H, sq, skv): several blocks with ragged tails, cross shapes both ways
    (1, 2, 128, 128), (2, 3, 200, 200), (1, 2, 77, 300), (2, 1, 300, 77), (1, 1, 1, 1000),
    (1, 1, 1000, 1), (1, 1, 513, 513), (3, 2, 64, 96), (1, 4, 257, 1025),
]


@pytest.mark.parametrize("d", [32, 64, 128, 256])
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("shape", SHAPES, ids=lambda s: "x".join(map(str, s)))
def test_bwd_f16_parity_small(shape, causal, d):
    B, H, sq, skv = shape
    vals, bits, g = _case(1700 + sq + 7 * skv + d, B, H, sq, skv, d)
    scale = 1.0 / math.sqrt(d)
    got = _gpu_grads(vals, bits, g, scale, causal)
    ref = oracle.attention_bwd(*vals, g, scale, causal)
    bound = oracle.attention_bwd_bound(*vals, g, scale, causal)
    check_grads(got, ref, bound, underflow_scale(*vals, g, scale, causal), f"{shape} causal={causal} d={d}")


@pytest.mark.parametrize("causal", [False, True])
def test_bwd_f16_with_a_hard_mask(causal):
    B, H, sq, skv, d = 2, 2, 150, 230, 128
    vals, bits, g = _case(1790 + causal, B, H, sq, skv, d)
    mask = (gen.uniform24(1791, np.arange(H * sq * skv, dtype=np.uint64)).reshape(1, H, sq, skv) < 0.5)
    mask = mask.astype(np.uint8)
    mask[..., 4, :] = 0  # a row that admits nothing
    got = _gpu_grads(vals, bits, g, 0.1, causal, mask=mask)
    ref = oracle.attention_bwd_masked(*vals, g, mask, 0.1, causal)
    bound = oracle.attention_bwd_masked_bound(*vals, g, mask, 0.1, causal)
    check_grads(got, ref, bound, underflow_scale(*vals, g, 0.1, causal, mask), f"masked causal={causal}")
    assert np.all(got[0][:, :, 4] == 0.0)


def test_bwd_f16_bshd_equals_bhsd():
    vals, bits, g = _case(1795, 2, 3, 150, 190, 64)
    a = _gpu_grads(vals, bits, g, 0.125, True)
    b = _gpu_grads(vals, bits, g, 0.125, True, layout="bshd")
    for x, y in zip(a, b):
        assert np.array_equal(x, y)


def test_bwd_f16_zero_upstream_gradient_is_exactly_zero():
    vals, bits, g = _case(1796, 1, 2, 140, 170, 128)
    got = _gpu_grads(vals, bits, np.zeros_like(g), 0.1, True)
    assert all(np.all(x == 0.0) for x in got)


def test_bwd_f16_differs_from_bf16_on_the_same_values():
    """Values exact in both types through both 16-bit backwards: the fp16 one lands at least
    twice as close to the oracle in L2 (its roundings are 8 times finer), so fp16 inputs run
    the fp16 MFMA and roundings, not the bf16 ones."""
    import torch

    import scaled_masked_attention_amd as sma

    (q, k, v), bits, g = _case(1797, 1, 2, 190, 210, 128)
    q, k, v = (gen.bf16_bits_to_f32(gen.f32_to_bf16_bits(x)) for x in (q, k, v))  # exact in bf16
    q, k, v = (np.where(np.abs(x) < 2.0**-14, np.float32(0), x) for x in (q, k, v))  # and in fp16
    assert all(np.array_equal(gen.f16_bits_to_f32(gen.f32_to_f16_bits(x)), x) for x in (q, k, v))
    q32, k32, v32, tg = (torch.from_numpy(np.ascontiguousarray(x)).to("cuda") for x in (q, k, v, g))
    o, lse = sma.attention_fwd(q32, k32, v32, scale=0.09, causal=True, return_lse=True)
    ref = oracle.attention_bwd(q, k, v, g, 0.09, True)
    errs = {}
    for dt in (torch.float16, torch.bfloat16):
        got = sma.attention_bwd(q32.to(dt), k32.to(dt), v32.to(dt), o, lse, tg, scale=0.09, causal=True)
        torch.cuda.synchronize()
        errs[dt] = [float(np.linalg.norm(x.cpu().numpy() - r)) for x, r in zip(got, ref)]
    for name, e16, e_b in zip(("dq", "dk", "dv"), errs[torch.float16], errs[torch.bfloat16]):
        assert e16 < e_b / 2, (name, e16, e_b)


def test_bwd_f16_full_size_exact_subproblems():
    """The 16384-token causal fp16 workload in one launch sequence; exact oracle values from
    the last 64 query rows with every key (a causal sub-problem that bottom-right alignment
    keeps intact: the exact dQ of those rows and dK, dV of keys >= S - 64)."""
    import torch

    import scaled_masked_attention_amd as sma

    w, vals, bits = workload_case("f16_causal_b1h32_s16384_d128")
    assert w.causal and w.seq_q == w.seq_kv and w.dtype == "f16"
    S, T = w.seq_q, 64
    g = gen.upstream_grad(w.seed, w.q_shape)
    q32, k32, v32, tg = (torch.from_numpy(np.ascontiguousarray(x)).to("cuda") for x in (*vals, g))
    o, lse = sma.attention_fwd(q32, k32, v32, scale=w.scale, causal=True, return_lse=True)
    del q32, k32, v32
    tq, tk, tv = to_device(None, bits, "f16")
    dq, dk, dv = sma.attention_bwd(tq, tk, tv, o, lse, tg, scale=w.scale, causal=True)
    torch.cuda.synchronize()
    dq, dk, dv = (t.cpu().numpy().astype(np.float64) for t in (dq, dk, dv))
    assert all(np.all(np.isfinite(t)) for t in (dq, dk, dv))
    q, k, v = vals
    for h in (0, w.heads - 1):
        sub = (slice(0, 1), slice(h, h + 1))
        last = sub + (slice(S - T, S),)
        args = (q[last], k[sub], v[sub], g[last], w.scale, True)
        ref, bound, under = oracle.attention_bwd(*args), oracle.attention_bwd_bound(*args), underflow_scale(*args)
        keep = lambda t: (t[0], t[1][:, :, S - T:], t[2][:, :, S - T:])  # noqa: E731
        check_grads((dq[last], dk[last], dv[last]), keep(ref), keep(bound), keep(under), f"head {h} last {T}")
