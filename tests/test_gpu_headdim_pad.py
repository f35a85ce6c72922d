"""Head dims against each other, with no tolerance: a problem zero-padded to a larger head
dim must give the smaller problem's results exactly.

Zero-padding Q, K, V (and dO) from head dim d to 2d changes no score S = q.k, no
dP = dO.v and so no probability: the extra MFMA k-steps add exact zeros to the same fp32
sums, in the same order, so every rounding (the 16-bit P, dO and dS included) sees the same
fp32 number. Hence:
  - forward: O in dims 0..d-1 and the LSE equal the d problem's, and O is zero above;
  - backward, given O = 0 (so D = dO.O is exactly 0) and the same LSE: dQ, dK and dV in dims
    0..d-1 equal the d problem's and are zero above (Q, K and dO are zero there).
Each pair runs one kernel family at two head dims, whose tiles, register layouts and copy
splits differ with the head dim (and at 256 the 16-bit backward splits its dQ work by role
and forms its LDS addresses its own way), so each is pinned against the other. The forward
pairs force one unsplit plan on both calls. A fused product-and-round that rounds dS once
from the exact product, instead of from its fp32 value, fails the 16-bit backward pairs.
Comparisons are by value (+0 == -0).

Not paired, because their sums are not the same sums: the qblock forward kernels (fp32 and
16-bit), whose two lane halves hold the two halves of the head dim, so that one MFMA adds
dim x and dim x + d/2 together and zero-padding regroups the terms; and the fp32 backward
at 256, which is not built.
"""
import numpy as np
import pytest

import gen
from helpers import to_device

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    torch = pytest.importorskip("torch")
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import scaled_masked_attention_amd as sma

    sma.library()  # fail loudly if the HIP library is missing


SHAPES = [((1, 2, 300, 300), False), ((2, 1, 200, 333), False), ((1, 2, 333, 200), False),
          ((1, 2, 260, 290), True)]


def _pad(t, d):
    import torch

    return torch.nn.functional.pad(t, (0, d - t.shape[-1])).contiguous()


def _inputs(dtype, shape, d, causal, masked):
    import torch

    B, H, sq, skv = shape
    seed = 9100 + sq + 7 * skv + d + (1 if causal else 0) + {"f32": 0, "bf16": 2, "f16": 4}[dtype]
    vals, bits = gen.random_case(seed, (B, H, sq, d), (B, H, skv, d), dtype=dtype)
    tq, tk, tv = to_device(vals, bits, dtype)
    g = torch.from_numpy(np.ascontiguousarray(gen.upstream_grad(seed, (B, H, sq, d)))).to("cuda")
    tm = torch.from_numpy(gen.bernoulli_mask(seed, (1, H, sq, skv), 0.6)).to("cuda") if masked else None
    return tq, tk, tv, g, tm


def _equal(name, small, big, d):
    import torch

    assert torch.isfinite(small).all(), name
    head = big[..., :d]
    assert torch.equal(head, small), (f"{name}: dims 0..{d - 1} differ ({int((head != small).sum())} elements, "
                                      f"max {float((head - small).abs().max()):.3e})")
    assert (big[..., d:] == 0).all(), f"{name}: dims {d}.. not zero"


FWD_PAIRS = [("f32", "f32_ksplit", 32), ("f32", "f32_ksplit", 64)]


@pytest.mark.parametrize("dtype,kernel,d", FWD_PAIRS)
@pytest.mark.parametrize("causal", [True, False])
@pytest.mark.parametrize("shape,masked", SHAPES)
def test_forward_padded_head_dim(dtype, kernel, d, causal, shape, masked):
    import torch

    import scaled_masked_attention_amd as sma

    code = {v: k for k, v in sma.KERNEL_NAMES.items()}[kernel]
    tq, tk, tv, _, tm = _inputs(dtype, shape, d, causal, masked)
    scale = 1.0 / np.sqrt(d)
    o1, l1 = sma.attention_fwd(tq, tk, tv, scale=scale, causal=causal, return_lse=True, mask=tm,
                               kernel=code, nsplit=1)
    pq, pk, pv = (_pad(x, 2 * d) for x in (tq, tk, tv))
    o2, l2 = sma.attention_fwd(pq, pk, pv, scale=scale, causal=causal, return_lse=True, mask=tm,
                               kernel=code, nsplit=1)
    torch.cuda.synchronize()
    _equal("O", o1, o2, d)
    assert torch.equal(l1, l2), f"LSE differs ({int((l1 != l2).sum())} rows)"


BWD_PAIRS = [("f32", 32), ("f32", 64), ("bf16", 32), ("bf16", 64), ("bf16", 128),
             ("f16", 32), ("f16", 64), ("f16", 128)]


@pytest.mark.parametrize("dtype,d", BWD_PAIRS)
@pytest.mark.parametrize("causal", [True, False])
@pytest.mark.parametrize("shape,masked", SHAPES)
def test_backward_padded_head_dim(dtype, d, causal, shape, masked):
    import torch

    import scaled_masked_attention_amd as sma

    tq, tk, tv, g, tm = _inputs(dtype, shape, d, causal, masked)
    B, H, sq, _ = shape
    scale = 1.0 / np.sqrt(d)
    _, lse = sma.attention_fwd(tq, tk, tv, scale=scale, causal=causal, return_lse=True, mask=tm)
    o = torch.zeros((B, H, sq, d), dtype=torch.float32, device="cuda")
    small = sma.attention_bwd(tq, tk, tv, o, lse, g, scale=scale, causal=causal, mask=tm)
    pq, pk, pv, pg, po = (_pad(x, 2 * d) for x in (tq, tk, tv, g, o))
    big = sma.attention_bwd(pq, pk, pv, po, lse, pg, scale=scale, causal=causal, mask=tm)
    torch.cuda.synchronize()
    for name, a, b in zip(("dq", "dk", "dv"), small, big):
        _equal(name, a, b, d)
    # The problem is not degenerate: every gradient has nonzero entries.
    assert all(bool((x != 0).any()) for x in small)
