"""The [B,S,H,d] layout through the C ABI: for every kernel and plan, the output on the
transposed inputs is bitwise the transposed output on [B,H,S,d] inputs (the arithmetic is
the same; only addresses differ), and it matches the oracle."""
import math

import numpy as np
import pytest

import gen
import oracle
from helpers import check_parity, to_device

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    torch = pytest.importorskip("torch")
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import scaled_masked_attention_amd as sma

    sma.library()


CASES = {  # name: (input dtype, kernel, key splits)
    "f32-qblock": ("f32", "F32_QBLOCK", 1),
    "f32-split3": ("f32", "F32_QBLOCK", 3),
    "f32-ksplit": ("f32", "F32_KSPLIT", 1),
    "bf16": ("bf16", "BF16_QBLOCK", 1),
    "bf16-split2": ("bf16", "BF16_QBLOCK", 2),
    "f16": ("f16", "BF16_QBLOCK", 1),
}


@pytest.mark.parametrize("out_dtype", ["f32", "bf16"])
@pytest.mark.parametrize("case", list(CASES))
@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("shape", [(2, 3, 200, 333), (1, 4, 300, 77)], ids=lambda s: "x".join(map(str, s)))
def test_bshd_equals_transposed_bhsd(shape, causal, d, case, out_dtype):
    import torch

    import scaled_masked_attention_amd as sma

    dtype, kern, nsplit = CASES[case]
    kw = dict(kernel=getattr(sma, "SMA_KERNEL_" + kern), nsplit=nsplit)
    odt = torch.float32 if out_dtype == "f32" else torch.bfloat16
    B, H, sq, skv = shape
    (q, k, v), bits = gen.random_case(900 + sq + skv + d, (B, H, sq, d), (B, H, skv, d),
                                      sigma_qk=1.0 if dtype == "f32" else 3.0, dtype=dtype)
    tq, tk, tv = to_device((q, k, v), bits, dtype)
    scale = 1.0 / math.sqrt(d)
    o1, l1 = sma.attention_fwd(tq, tk, tv, scale=scale, causal=causal, return_lse=True,
                               out_dtype=odt, **kw)
    sq_t, sk_t, sv_t = (t.transpose(1, 2).contiguous() for t in (tq, tk, tv))
    o2, l2 = sma.attention_fwd(sq_t, sk_t, sv_t, scale=scale, causal=causal, return_lse=True,
                               out_dtype=odt, layout="bshd", **kw)
    torch.cuda.synchronize()
    assert tuple(o2.shape) == (B, sq, H, d)
    assert torch.equal(o2.transpose(1, 2), o1), "BSHD result differs from transposed BHSD"
    assert torch.equal(l1, l2)
    if out_dtype == "f32":
        o_ref, lse_ref = oracle.attention_fwd(q, k, v, scale, causal)
        check_parity(o2.transpose(1, 2).cpu().numpy().astype(np.float64),
                     l2.cpu().numpy().astype(np.float64), o_ref, lse_ref, dtype, f"bshd {case}")


def test_bshd_automatic_plan_and_binding_checks():
    import torch

    import scaled_masked_attention_amd as sma

    (q, k, v), _ = gen.random_case(901, (2, 5, 130, 64), (2, 5, 260, 64))
    tq, tk, tv = (torch.from_numpy(x).to("cuda").transpose(1, 2).contiguous() for x in (q, k, v))
    o, lse = sma.attention_fwd(tq, tk, tv, scale=0.11, causal=True, return_lse=True, layout="bshd")
    torch.cuda.synchronize()
    o_ref, lse_ref = oracle.attention_fwd(q, k, v, 0.11, True)
    check_parity(o.transpose(1, 2).cpu().numpy().astype(np.float64), lse.cpu().numpy().astype(np.float64),
                 o_ref, lse_ref, "f32", "bshd auto")
    with pytest.raises(ValueError):
        sma.attention_fwd(tq, tk, tv, layout="sbhd")
    with pytest.raises(ValueError):  # k in the other layout: shapes disagree
        sma.attention_fwd(tq, tk.transpose(1, 2).contiguous(), tv, layout="bshd")
