"""Head dims 128 and 256 of the 16-bit backward against each other, with no tolerance.

Zero-padding Q, K, V and dO from d = 128 to d = 256 changes no score S = q.k, no
dP = dO.v and so no P: the extra MFMA k-steps add exact zeros to the same fp32 sums. With
O = 0 given to both calls (D = dO.O is then exactly 0) and the same LSE, dS = P dP is the
same fp32 number in both, rounded once to the input type (nearest even). So the padded
problem's gradients must equal the d = 128 problem's in dims 0..127, and dQ, dK and dV
must be zero in dims 128..255, where K, Q and dO are zero.

The two head dims run different code: at d = 256 the dQ work is split by role between two
waves, and the dK/dV kernel forms its LDS addresses its own way. This pins each against the
other exactly, including every rounding of dO, P and dS (a fused product-and-round that
rounds dS once from the exact product, instead of from its fp32 value, fails it).
Comparisons are by value, so +0 and -0 count as equal.
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


def _pad(t, d):
    import torch

    return torch.nn.functional.pad(t, (0, d - t.shape[-1])).contiguous()


@pytest.mark.parametrize("dtype", ["bf16", "f16"])
@pytest.mark.parametrize("causal", [True, False])
@pytest.mark.parametrize("shape,masked", [((1, 2, 300, 300), False), ((2, 1, 200, 333), False),
                                          ((1, 2, 333, 200), False), ((1, 2, 260, 290), True)])
def test_padded_head_dim_256_equals_128(dtype, causal, shape, masked):
    import torch

    import scaled_masked_attention_amd as sma

    B, H, sq, skv = shape
    d = 128
    seed = 9100 + sq + 7 * skv + (1 if causal else 0) + (2 if dtype == "f16" else 0)
    _, bits = gen.random_case(seed, (B, H, sq, d), (B, H, skv, d), dtype=dtype)
    tq, tk, tv = to_device(None, bits, dtype)
    g = torch.from_numpy(np.ascontiguousarray(gen.upstream_grad(seed, (B, H, sq, d)))).to("cuda")
    tm = None
    if masked:
        tm = torch.from_numpy(gen.bernoulli_mask(seed, (1, H, sq, skv), 0.6)).to("cuda")
    scale = 1.0 / np.sqrt(d)
    _, lse = sma.attention_fwd(tq, tk, tv, scale=scale, causal=causal, return_lse=True, mask=tm)
    o = torch.zeros((B, H, sq, d), dtype=torch.float32, device="cuda")
    got128 = sma.attention_bwd(tq, tk, tv, o, lse, g, scale=scale, causal=causal, mask=tm)
    pq, pk, pv, pg, po = (_pad(x, 256) for x in (tq, tk, tv, g, o))
    got256 = sma.attention_bwd(pq, pk, pv, po, lse, pg, scale=scale, causal=causal, mask=tm)
    torch.cuda.synchronize()
    for name, a, b in zip(("dq", "dk", "dv"), got128, got256):
        assert torch.isfinite(a).all(), name
        assert torch.equal(b[..., :d], a), f"{name}: dims 0..127 differ from head dim 128 " \
            f"({int((b[..., :d] != a).sum())} elements, max {float((b[..., :d] - a).abs().max()):.3e})"
        assert (b[..., d:] == 0).all(), f"{name}: dims 128..255 not zero"
    # The padded problem is not degenerate: every gradient has nonzero entries.
    assert all(bool((x != 0).any()) for x in got128)
