"""Row primitives on the GPU vs the CPU oracle, element by element, through the C ABI.

Shapes cover every mapping of a row: a wave per row (up to 4096 floats), a
workgroup per row (up to 16384), two streaming passes beyond, each with vector
(cols a multiple of 4, 16-byte aligned) and scalar loads.
"""
import numpy as np
import pytest

import oracle

pytestmark = pytest.mark.gpu

P_ABS = 2e-6        # probabilities in [0, 1]
LSE_TOL = 1e-5      # |d lse| <= LSE_TOL * max(1, |lse|)


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    torch = pytest.importorskip("torch")
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import scaled_masked_attention_amd as sma

    sma.library()


def _dev(a, offset=0):
    """Host array -> contiguous cuda float32 tensor, optionally starting `offset` floats into a buffer."""
    import torch

    a = np.ascontiguousarray(a, dtype=np.float32)
    if offset == 0:
        return torch.from_numpy(a).to("cuda")
    buf = torch.zeros(a.size + offset, dtype=torch.float32, device="cuda")
    buf[offset:] = torch.from_numpy(a.ravel()).to("cuda")
    return buf[offset:].view(a.shape)


def _host(t):
    import torch

    torch.cuda.synchronize()
    return t.cpu().numpy().astype(np.float64)


def _check_p(p, ref, label):
    assert p.shape == ref.shape
    assert np.all(np.isfinite(p)), label
    err = np.abs(p - ref)
    assert err.max(initial=0.0) <= P_ABS, f"{label}: max abs {err.max():.3e}"
    zero = ref == 0.0
    assert np.all(p[zero] == 0.0) and not np.any(np.signbit(p[zero])), f"{label}: nonzero blocked entries"


def _check_lse(l, ref, label):
    ninf = np.isneginf(ref)
    assert np.array_equal(np.isneginf(l), ninf), label
    fin = ~ninf
    err = np.abs(l[fin] - ref[fin]) / np.maximum(1.0, np.abs(ref[fin]))
    assert err.max(initial=0.0) <= LSE_TOL, f"{label}: lse rel {err.max():.3e}"


SHAPES = [(1, 1), (3, 5), (7, 64), (5, 65), (64, 1000), (33, 4096), (9, 4097), (4, 8192),
          (3, 16384), (2, 16385), (2, 40000), (1000, 128), (257, 12)]


def _x(rows, cols, seed, sigma=4.0):
    return (np.random.default_rng(seed).normal(size=(rows, cols)) * sigma).astype(np.float32)


@pytest.mark.parametrize("offset", [0, 1])
@pytest.mark.parametrize("shape", SHAPES, ids=lambda s: "x".join(map(str, s)))
def test_softmax_and_lse_rows(shape, offset):
    import scaled_masked_attention_amd as sma

    rows, cols = shape
    x = _x(rows, cols, rows * 7 + cols)
    tx = _dev(x, offset)
    _check_p(_host(sma.softmax_rows(tx)), oracle.softmax_rows(x), f"softmax {shape} +{offset}")
    _check_lse(_host(sma.logsumexp_rows(tx)), oracle.logsumexp_rows(x), f"lse {shape} +{offset}")


@pytest.mark.parametrize("offset", [0, 1])
@pytest.mark.parametrize("shape", SHAPES, ids=lambda s: "x".join(map(str, s)))
def test_masked_rows(shape, offset):
    import scaled_masked_attention_amd as sma

    rows, cols = shape
    rng = np.random.default_rng(rows + 3 * cols)
    x = _x(rows, cols, rows + 11 * cols)
    mask = (rng.random(size=x.shape) < 0.5).astype(np.float32) * rng.choice([1.0, -3.0], size=x.shape).astype(np.float32)
    mask[0] = 0.0                                   # a row admitting nothing
    if rows > 1:
        mask[1] = 0.0
        mask[1, rng.integers(0, cols)] = 2.0        # a one-hot row
    poison = np.array([np.nan, np.inf, -np.inf, 1e30], dtype=np.float32)
    xb = np.where(mask != 0, x, poison[rng.integers(0, 4, size=x.shape)]).astype(np.float32)
    p = _host(sma.masked_softmax_rows(_dev(xb, offset), _dev(mask, offset)))
    ref = oracle.masked_softmax_rows(xb, mask)
    _check_p(p, ref, f"masked {shape} +{offset}")
    assert np.all(p[0] == 0.0)


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("scale", [0.125, -0.3, 0.0])
@pytest.mark.parametrize("brc", [(2, 16, 16), (3, 200, 77), (2, 77, 200), (1, 1, 4096), (2, 40, 9000),
                                 (1, 5, 20000)], ids=lambda s: "x".join(map(str, s)))
def test_scaled_causal(brc, scale, causal):
    import scaled_masked_attention_amd as sma

    b, r, c = brc
    x = (np.random.default_rng(b * r + c).normal(size=brc) * 6).astype(np.float32)
    p = _host(sma.scaled_causal_softmax(_dev(x), scale, causal))
    _check_p(p, oracle.scaled_causal_softmax(x, scale, causal), f"scaled {brc} {scale} {causal}")


@pytest.mark.parametrize("cols", [40, 5000, 30000])
def test_negative_infinity_entries_and_rows(cols):
    import scaled_masked_attention_amd as sma

    x = _x(6, cols, cols)
    x[:, ::3] = -np.inf
    x[2] = -np.inf
    tx = _dev(x)
    p = _host(sma.softmax_rows(tx))
    _check_p(p, oracle.softmax_rows(x), "neg inf")
    assert np.all(p[2] == 0.0)
    lse = _host(sma.logsumexp_rows(tx))
    _check_lse(lse, oracle.logsumexp_rows(x), "neg inf lse")
    assert np.isneginf(lse[2])
    y = x.reshape(2, 3, cols)
    _check_p(_host(sma.scaled_causal_softmax(_dev(y), -0.5, True)),
             oracle.scaled_causal_softmax(y, -0.5, True), "neg inf scaled")


@pytest.mark.parametrize("cols", [300, 8192, 20000])
def test_shift_far_beyond_exp_range(cols):
    import scaled_masked_attention_amd as sma

    x = (np.round(np.random.default_rng(cols).normal(size=(5, cols)) * 64) / 64).astype(np.float32)
    shifted = (x + np.float32(8192.0)).astype(np.float32)
    t = _dev(shifted)
    _check_p(_host(sma.softmax_rows(t)), oracle.softmax_rows(shifted), "shift")
    _check_lse(_host(sma.logsumexp_rows(t)), oracle.logsumexp_rows(shifted), "shift lse")


@pytest.mark.parametrize("cols", [100, 4096, 20000])
def test_in_place(cols):
    import scaled_masked_attention_amd as sma

    x = _x(7, cols, 5 * cols)
    t = _dev(x)
    out = sma.softmax_rows(t, out=t)
    assert out.data_ptr() == t.data_ptr()
    _check_p(_host(t), oracle.softmax_rows(x), "in place")


# Softmax backward: dx = scale * y * (dy - sum_k y_k dy_k). The kernel's dot product runs in fp32
# over at most 72 terms in sequence (64 per lane, then an 8-level tree over the lanes), so its
# error is at most 72 * 2^-24 = 4.3e-6 of sum_k y_k |dy_k|; with the final products this gives
# |dx_j - ref_j| <= BWD_TOL * |scale| * y_j * (|dy_j| + sum_k y_k |dy_k|) with a factor of 2 to spare.
BWD_TOL = 1e-5


def _check_bwd(dx, y, dy, scale, label):
    ref = oracle.softmax_rows_backward(y, dy, scale)
    y64, dy64 = y.astype(np.float64), np.abs(dy.astype(np.float64))
    bound = BWD_TOL * abs(scale) * y64 * (dy64 + (y64 * dy64).sum(axis=1, keepdims=True))
    assert dx.shape == ref.shape and np.all(np.isfinite(dx)), label
    err = np.abs(dx - ref)
    worst = float(np.max(err - bound, initial=0.0))
    assert worst <= 0.0, f"{label}: error beyond the bound by {worst:.3e}"
    assert np.all(dx[y == 0] == 0.0), f"{label}: nonzero gradient where y = 0"


def _y_dy(rows, cols, seed, masked=False):
    x = _x(rows, cols, seed)
    if masked:
        m = (np.random.default_rng(seed + 1).random((rows, cols)) < 0.5).astype(np.float32)
        y = oracle.masked_softmax_rows(x, m).astype(np.float32)
    else:
        y = oracle.softmax_rows(x).astype(np.float32)
    dy = np.random.default_rng(seed + 2).normal(size=(rows, cols)).astype(np.float32)
    return y, dy


@pytest.mark.parametrize("scale", [1.0, 0.125, -0.5])
@pytest.mark.parametrize("offset", [0, 1])
@pytest.mark.parametrize("shape", SHAPES, ids=lambda s: "x".join(map(str, s)))
def test_softmax_rows_backward(shape, offset, scale):
    import scaled_masked_attention_amd as sma

    rows, cols = shape
    y, dy = _y_dy(rows, cols, 11 * rows + cols, masked=(rows + cols) % 2 == 1)
    dx = _host(sma.softmax_rows_backward(_dev(y, offset), _dev(dy, offset), scale=scale))
    _check_bwd(dx, y, dy, scale, f"bwd {shape} +{offset} scale={scale}")


@pytest.mark.parametrize("target", ["y", "dy"])
@pytest.mark.parametrize("cols", [100, 4096, 40000])
def test_softmax_rows_backward_in_place(cols, target):
    import scaled_masked_attention_amd as sma

    y, dy = _y_dy(5, cols, 3 * cols)
    ty, tg = _dev(y), _dev(dy)
    out = ty if target == "y" else tg
    r = sma.softmax_rows_backward(ty, tg, scale=0.3, out=out)
    assert r.data_ptr() == out.data_ptr()
    _check_bwd(_host(out), y, dy, 0.3, f"in place over {target}")


def test_softmax_rows_backward_closed_form_on_gpu():
    """A one-hot y gives dx = 0 (dy_j - dot vanishes where y_j = 1, y_k = 0 elsewhere), and a
    uniform y with dy = e_0 gives dx_j = scale * (delta_j0 - 1/n) / n."""
    import scaled_masked_attention_amd as sma

    n = 64
    y = np.zeros((3, n), dtype=np.float32)
    y[np.arange(3), [0, 17, 63]] = 1.0
    dy = np.random.default_rng(4).normal(size=(3, n)).astype(np.float32)
    assert np.all(_host(sma.softmax_rows_backward(_dev(y), _dev(dy))) == 0.0)
    yu = np.full((2, n), 1.0 / n, dtype=np.float32)  # 1/64 is exact in fp32
    e0 = np.zeros((2, n), dtype=np.float32)
    e0[:, 0] = 1.0
    dx = _host(sma.softmax_rows_backward(_dev(yu), _dev(e0), scale=2.0))
    expect = 2.0 * (np.eye(1, n).repeat(2, 0) - 1.0 / n) / n
    assert np.allclose(dx, expect, rtol=0, atol=1e-9)


def test_empty_shapes():
    import torch

    import scaled_masked_attention_amd as sma

    z = torch.zeros((4, 0), dtype=torch.float32, device="cuda")
    assert sma.softmax_rows(z).shape == (4, 0)
    lse = _host(sma.logsumexp_rows(z))
    assert lse.shape == (4,) and np.all(np.isneginf(lse))
    e = torch.zeros((0, 9), dtype=torch.float32, device="cuda")
    assert sma.softmax_rows(e).shape == (0, 9)
    assert sma.logsumexp_rows(e).shape == (0,)
    assert sma.scaled_causal_softmax(torch.zeros((0, 3, 3), device="cuda"), 1.0).shape == (0, 3, 3)
    assert sma.softmax_rows_backward(e, e).shape == (0, 9)
    assert sma.softmax_rows_backward(z, z).shape == (4, 0)


def test_binding_rejects():
    import torch

    import scaled_masked_attention_amd as sma

    x = torch.zeros((4, 8), dtype=torch.float32, device="cuda")
    with pytest.raises(ValueError):
        sma.softmax_rows(x.double())
    with pytest.raises(ValueError):
        sma.masked_softmax_rows(x, torch.zeros((4, 9), device="cuda"))
    with pytest.raises(sma.SMAError) as e:
        sma.scaled_causal_softmax(x.view(1, 4, 8), float("inf"))
    assert e.value.status == 2
    buf = torch.zeros(40, device="cuda")
    with pytest.raises(sma.SMAError) as e:
        sma.softmax_rows(buf[:32].view(4, 8), out=buf[4:36].view(4, 8))  # partial overlap
    assert e.value.status == 5
