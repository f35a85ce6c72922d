"""Attention backward with a hard mask, through the C ABI, against the masked-backward oracle.

The GPU backward takes the GPU masked forward's O and LSE, as a training step would. Masks
at two densities in every broadcast form, rows that admit nothing, causal and not, fp32
(bar 1e-5 of the oracle's error scale, as in test_gpu_bwd.py), bf16 inputs (bar 2^-7 of
it, as in test_gpu_bwd_bf16.py) and fp16 inputs (2^-10 of it plus the underflow term, as in
test_gpu_bwd_f16.py, from the fp32 forward's O and LSE). An all-ones mask must reproduce the unmasked backward bit
for bit, the [B,S,H,d] layout must equal [B,H,S,d] on transposed data bit for bit, and HIP-graph
replays of the backward (fp32, bf16 and fp16 inputs) must equal the eager call bit for bit.
"""
import numpy as np
import pytest

import gen
import helpers
import oracle
from helpers import to_device
from test_gpu_bwd_f16 import underflow_scale

pytestmark = pytest.mark.gpu

TAU = {"f32": 1e-5, "bf16": 2.0**-7, "f16": 2.0**-10}
L2 = {"f32": 1e-5, "bf16": 2.0**-9, "f16": 2.0**-12}
F16_UNDERFLOW = 2.0**-24  # fp16's absolute rounding floor, as derived in test_gpu_bwd_f16.py


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    torch = pytest.importorskip("torch")
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import scaled_masked_attention_amd as sma

    sma.library()


def _mask(seed, shape, density, empty_rows=()):
    m = gen.uniform24(seed, np.arange(int(np.prod(shape)), dtype=np.uint64)).reshape(shape) < density
    for r in empty_rows:
        m[..., r, :] = False
    return m.astype(np.uint8)


def _run(q, k, v, bits, g, mask, scale, causal, dtype, layout="bhsd"):
    import torch

    import scaled_masked_attention_amd as sma

    tq, tk, tv = to_device((q, k, v), bits, dtype)
    tg = torch.from_numpy(np.ascontiguousarray(g)).to("cuda")
    tm = torch.from_numpy(np.ascontiguousarray(mask)).to("cuda") if mask is not None else None
    # fp16: O and LSE from the fp32 forward on the same values, so that the fp16 bar (derived
    # for the backward's own roundings) applies; bf16 and fp32 take their own forward
    fwd_in = to_device((q, k, v), bits, "f32") if dtype == "f16" else (tq, tk, tv)
    o, lse = sma.attention_fwd(*fwd_in, scale=scale, causal=causal, return_lse=True, mask=tm)
    if layout == "bshd":
        tq, tk, tv, o, tg = (x.transpose(1, 2).contiguous() for x in (tq, tk, tv, o, tg))
    grads = sma.attention_bwd(tq, tk, tv, o, lse, tg, scale=scale, causal=causal, mask=tm, layout=layout)
    torch.cuda.synchronize()
    if layout == "bshd":
        grads = tuple(x.transpose(1, 2) for x in grads)
    return tuple(x.contiguous() for x in grads)


def _check(got, ref, bound, dtype, label, under=(0.0, 0.0, 0.0)):
    for name, t, b, m, u in zip(("dq", "dk", "dv"), got, ref, bound, under):
        a = t.cpu().numpy().astype(np.float64)
        assert np.all(np.isfinite(a)), f"{label}: non-finite {name}"
        err = np.abs(a - b)
        zero = m == 0
        assert np.all(a[zero] == 0.0), f"{label}: {name} nonzero where every term is zero"
        bar = TAU[dtype] * m + F16_UNDERFLOW * u
        assert np.all(err <= bar), f"{label}: {name} error beyond its bar"
        d2 = float(np.linalg.norm(a - b))
        l2_bar = (L2[dtype] * float(np.linalg.norm(m)) + 1e-5 * float(np.linalg.norm(b))
                  + F16_UNDERFLOW * float(np.linalg.norm(u)))
        assert d2 <= l2_bar, f"{label}: {name} L2 error"
        pos = bar > 0
        frac = float((err[pos] / bar[pos]).max()) if pos.any() else 0.0
        helpers.bwd_regression(dtype, frac, d2 / l2_bar if l2_bar > 0 else 0.0, f"{label} {name}")


FORMS = {"shared": (1, 1), "per_head": (1, "H"), "full": ("B", "H")}


# (the fp32 backward is not built for head dim 256)
@pytest.mark.parametrize("dtype,d", [(t, d) for t in ("f32", "bf16", "f16") for d in (32, 64, 128, 256) if not (t == "f32" and d == 256)])
@pytest.mark.parametrize("form", list(FORMS))
@pytest.mark.parametrize("density", [0.3, 0.9])
@pytest.mark.parametrize("causal", [False, True])
def test_masked_backward_parity(causal, d, density, form, dtype):
    B, H, sq, skv = 2, 2, 130, 177
    (q, k, v), bits = gen.random_case(1600 + d + int(density * 10), (B, H, sq, d), (B, H, skv, d), dtype=dtype)
    g = gen.upstream_grad(1601 + d, (B, H, sq, d))
    mb = B if FORMS[form][0] == "B" else 1
    mh = H if FORMS[form][1] == "H" else 1
    mask = _mask(1602 + causal, (mb, mh, sq, skv), density, empty_rows=(5, 6))
    scale = 1.0 / np.sqrt(d)
    got = _run(q, k, v, bits, g, mask, scale, causal, dtype)
    ref = oracle.attention_bwd_masked(q, k, v, g, mask, scale, causal)
    bound = oracle.attention_bwd_masked_bound(q, k, v, g, mask, scale, causal)
    under = underflow_scale(q, k, v, g, scale, causal, mask) if dtype == "f16" else (0.0, 0.0, 0.0)
    _check(got, ref, bound, dtype, f"{form} {density} {dtype}", under)
    assert np.all(got[0].cpu().numpy()[:, :, 5:7] == 0.0)  # rows that admit nothing


@pytest.mark.parametrize("dtype", ["f32", "bf16", "f16"])
@pytest.mark.parametrize("causal", [False, True])
def test_all_ones_mask_is_bitwise_the_unmasked_backward(dtype, causal):
    """Both calls take the same O and LSE (the unmasked forward's: with a mask the 16-bit
    forward at head dim 128 runs another kernel, whose O differs in its roundings), so only
    the backward's mask path is compared."""
    import torch

    import scaled_masked_attention_amd as sma

    (q, k, v), bits = gen.random_case(1610, (1, 3, 200, 128), (1, 3, 230, 128), dtype=dtype)
    g = gen.upstream_grad(1610, (1, 3, 200, 128))
    tq, tk, tv = to_device((q, k, v), bits, dtype)
    tg = torch.from_numpy(np.ascontiguousarray(g)).to("cuda")
    ones = torch.ones((1, 1, 200, 230), dtype=torch.uint8, device="cuda")
    o, lse = sma.attention_fwd(tq, tk, tv, scale=0.09, causal=causal, return_lse=True)
    a = sma.attention_bwd(tq, tk, tv, o, lse, tg, scale=0.09, causal=causal, mask=ones)
    b = sma.attention_bwd(tq, tk, tv, o, lse, tg, scale=0.09, causal=causal)
    torch.cuda.synchronize()
    for x, y in zip(a, b):
        assert torch.equal(x, y)


@pytest.mark.parametrize("dtype", ["f32", "bf16", "f16"])
def test_masked_backward_bshd_equals_bhsd(dtype):
    (q, k, v), bits = gen.random_case(1620, (2, 3, 150, 64), (2, 3, 190, 64), dtype=dtype)
    g = gen.upstream_grad(1620, (2, 3, 150, 64))
    mask = _mask(1621, (2, 1, 150, 190), 0.5, empty_rows=(0,))
    a = _run(q, k, v, bits, g, mask, 0.125, True, dtype)
    b = _run(q, k, v, bits, g, mask, 0.125, True, dtype, layout="bshd")
    for x, y in zip(a, b):
        assert np.array_equal(x.cpu().numpy(), y.cpu().numpy())


def test_masked_backward_binding_checks():
    import torch

    import scaled_masked_attention_amd as sma

    q = torch.randn(1, 2, 40, 64, device="cuda")
    k = torch.randn(1, 2, 50, 64, device="cuda")
    m = torch.ones(40, 50, dtype=torch.bool, device="cuda")
    o, lse = sma.attention_fwd(q, k, k, return_lse=True, mask=m)
    with pytest.raises(ValueError):
        sma.attention_bwd(q, k, k, o, lse, o, mask=torch.ones(40, 51, dtype=torch.bool, device="cuda"))
    with pytest.raises(ValueError):
        sma.attention_bwd(q, k, k, o, lse, o, mask=torch.ones(40, 50, device="cuda"))  # float mask


@pytest.mark.parametrize("masked", [False, True])
@pytest.mark.parametrize("dtype", ["f32", "bf16", "f16"])
def test_backward_hip_graph_replays_match_eager(dtype, masked):
    """The backward (with its mask packing when masked) captured in a HIP graph through torch,
    replayed several times with eager work and synchronizations between replays and the
    gradients refilled with NaN before each: every replay equals the eager result bitwise."""
    import torch

    import scaled_masked_attention_amd as sma

    (q, k, v), bits = gen.random_case(1630, (2, 2, 180, 64), (2, 2, 210, 64), dtype=dtype)
    g = gen.upstream_grad(1630, (2, 2, 180, 64))
    tq, tk, tv = to_device((q, k, v), bits, dtype)
    tg = torch.from_numpy(g).to("cuda")
    tm = torch.from_numpy(_mask(1631, (1, 2, 180, 210), 0.6, empty_rows=(3,))).to("cuda") if masked else None
    o, lse = sma.attention_fwd(tq, tk, tv, scale=0.12, causal=True, return_lse=True, mask=tm)
    in_dt = {"f32": sma.SMA_DTYPE_F32, "bf16": sma.SMA_DTYPE_BF16, "f16": sma.SMA_DTYPE_F16}[dtype]
    if masked:
        n = sma.library().sma_attention_bwd_masked_workspace_bytes(in_dt, 2, 2, 180, 210, 64, 1, 0, 1, 2)
    else:
        n = sma.attention_bwd_workspace_bytes(in_dt, 2, 2, 180, 210, 64, True)
    ws = torch.empty(n, dtype=torch.uint8, device="cuda")
    eager = sma.attention_bwd(tq, tk, tv, o, lse, tg, scale=0.12, causal=True, mask=tm, workspace=ws)
    torch.cuda.synchronize()
    eager = [t.clone() for t in eager]
    graph = torch.cuda.CUDAGraph()
    s = torch.cuda.Stream()
    with torch.cuda.stream(s):
        with torch.cuda.graph(graph, stream=s):
            grads = sma.attention_bwd(tq, tk, tv, o, lse, tg, scale=0.12, causal=True, mask=tm, workspace=ws,
                                      stream=torch.cuda.current_stream())
    for rep in range(4):
        for t in grads:
            t.fill_(float("nan"))
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        for name, a, b in zip(("dq", "dk", "dv"), grads, eager):
            assert torch.equal(a, b), f"replay {rep}: {name} differs"
        _ = (tg * 2).sum().item()  # eager work between replays
