"""Attention backward in the [B,S,H,d] layout, through the C ABI: the gradients must equal
those of the [B,H,S,d] backward on the same data, bit for bit (the kernels do the same
arithmetic through different strides), for fp32, bf16 and fp16 inputs, causal and not, on ragged
shapes. The [B,H,S,d] backward itself is checked against the oracle in test_gpu_bwd.py and
test_gpu_bwd_bf16.py.
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

    sma.library()


# (the fp32 backward is not built for head dim 256)
@pytest.mark.parametrize("dtype,d", [(t, d) for t in ("f32", "bf16", "f16") for d in (32, 64, 128, 256) if not (t == "f32" and d == 256)])
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("shape", [(2, 3, 130, 77), (1, 2, 200, 333), (2, 1, 257, 129)],
                         ids=lambda s: "x".join(map(str, s)))
def test_bshd_backward_equals_transposed_bhsd(shape, causal, d, dtype):
    import torch

    import scaled_masked_attention_amd as sma

    B, H, sq, skv = shape
    (q, k, v), bits = gen.random_case(1500 + sq + skv + d, (B, H, sq, d), (B, H, skv, d), dtype=dtype)
    g = gen.upstream_grad(1500 + sq, (B, H, sq, d))
    tq, tk, tv = to_device((q, k, v), bits, dtype)
    tg = torch.from_numpy(g).to("cuda")
    o, lse = sma.attention_fwd(tq, tk, tv, scale=0.11, causal=causal, return_lse=True)
    ref = sma.attention_bwd(tq, tk, tv, o, lse, tg, scale=0.11, causal=causal)
    t = [x.transpose(1, 2).contiguous() for x in (tq, tk, tv, o, tg)]
    got = sma.attention_bwd(t[0], t[1], t[2], t[3], lse, t[4], scale=0.11, causal=causal, layout="bshd")
    torch.cuda.synchronize()
    for name, a, b in zip(("dq", "dk", "dv"), got, ref):
        assert a.dtype == torch.float32 and a.shape == b.transpose(1, 2).shape, name
        assert torch.equal(a.transpose(1, 2), b), f"{name} differs between layouts"


def test_bshd_backward_binding_checks():
    import torch

    import scaled_masked_attention_amd as sma

    q = torch.randn(1, 8, 2, 64, device="cuda")  # [B, S, H, D]
    lse = torch.zeros(1, 2, 8, device="cuda")
    with pytest.raises(ValueError):
        sma.attention_bwd(q, q, q, q, lse, q, layout="bsdh")
    with pytest.raises(ValueError):  # lse must be [B, H, Sq]
        sma.attention_bwd(q, q, q, q, torch.zeros(1, 8, 2, device="cuda"), q, layout="bshd")
