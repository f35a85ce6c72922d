"""16-bit output (bf16 and fp16) of the attention forward, on every kernel and plan, through
the C ABI.

The 16-bit O must be the fp32 O of the same plan rounded to nearest even, bit for bit (both
sides take the rounding decision from the same fp32 value; numpy's float32 -> float16
conversion, pinned by textbook encodings in test_gen.py, rounds to nearest even), and it
must sit within the input dtype's parity bar of the oracle plus the rounding itself:
|O16 - O_ref| <= bar + u |O| elementwise, u = 2^-8 for bf16 and 2^-11 for fp16 (half an
ulp), plus 2^-25 for fp16's subnormal spacing. Rows without keys are +0.0 exactly.
"""
import math

import numpy as np
import pytest

import gen
import oracle
from helpers import BF16_MAX_ABS, F16_MAX_ABS, F32_MAX_ABS, empty_rows, to_device

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    torch = pytest.importorskip("torch")
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import scaled_masked_attention_amd as sma

    sma.library()


PLANS = {"auto": None, "qblock": ("qblock", 1), "split3": ("qblock", 3), "ksplit": ("ksplit", 1)}

# The in-workgroup key-split kernel is fp32 only: it is paired with fp32 inputs alone.
DTYPE_PLANS = [(dt, pl) for dt in ("f32", "bf16", "f16") for pl in PLANS if dt == "f32" or pl != "ksplit"]


def _plan_kwargs(plan, dtype):
    import scaled_masked_attention_amd as sma

    if PLANS[plan] is None:
        return {}
    kind, nsplit = PLANS[plan]
    if kind == "ksplit":
        assert dtype == "f32", "the in-workgroup key-split kernel is fp32 only"
        return dict(kernel=sma.SMA_KERNEL_F32_KSPLIT, nsplit=1)
    kern = sma.SMA_KERNEL_F32_QBLOCK if dtype == "f32" else sma.SMA_KERNEL_BF16_QBLOCK
    return dict(kernel=kern, nsplit=nsplit)


def _bits(t):
    import torch

    return t.view(torch.int16).cpu().numpy().view(np.uint16)


@pytest.mark.parametrize("dtype,plan", DTYPE_PLANS)
@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("shape", [(2, 3, 200, 200), (1, 2, 77, 300), (2, 1, 300, 77), (1, 4, 257, 1025)],
                         ids=lambda s: "x".join(map(str, s)))
def test_bf16_output_is_the_rounded_fp32_output(shape, causal, d, dtype, plan):
    import torch

    import scaled_masked_attention_amd as sma

    kw = _plan_kwargs(plan, dtype)
    B, H, sq, skv = shape
    (q, k, v), bits = gen.random_case(700 + sq + 3 * skv + d, (B, H, sq, d), (B, H, skv, d),
                                      sigma_qk=1.0 if dtype == "f32" else 3.0, dtype=dtype)
    tq, tk, tv = to_device((q, k, v), bits, dtype)
    scale = 1.0 / math.sqrt(d)
    o32, l32 = sma.attention_fwd(tq, tk, tv, scale=scale, causal=causal, return_lse=True, **kw)
    o16, l16 = sma.attention_fwd(tq, tk, tv, scale=scale, causal=causal, return_lse=True,
                                 out_dtype=torch.bfloat16, **kw)
    torch.cuda.synchronize()
    assert o16.dtype == torch.bfloat16
    f32 = o32.cpu().numpy()
    assert np.array_equal(_bits(o16), gen.f32_to_bf16_bits(f32)), "bf16 O is not RNE of the fp32 O"
    assert torch.equal(l16, l32), "LSE changed with the output dtype"
    o_ref, _ = oracle.attention_fwd(q, k, v, scale, causal)
    got = gen.bf16_bits_to_f32(_bits(o16)).astype(np.float64)
    bar = ({"f32": F32_MAX_ABS, "bf16": BF16_MAX_ABS, "f16": F16_MAX_ABS}[dtype]
           + 2.0 ** -8 * np.abs(f32.astype(np.float64)))
    assert np.all(np.abs(got - o_ref) <= bar)
    er = empty_rows(sq, skv, causal)
    if er.any():
        assert np.all(_bits(o16)[:, :, er] == 0)


def test_bf16_output_with_no_keys_is_positive_zero():
    import torch

    import scaled_masked_attention_amd as sma

    q = torch.randn(1, 2, 40, 64, device="cuda")
    k = torch.empty(1, 2, 0, 64, device="cuda")
    o, lse = sma.attention_fwd(q, k, k, causal=False, return_lse=True, out_dtype=torch.bfloat16)
    torch.cuda.synchronize()
    assert np.all(_bits(o) == 0) and torch.isneginf(lse).all()


@pytest.mark.parametrize("dtype,plan", DTYPE_PLANS)
@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("shape", [(2, 3, 200, 200), (1, 4, 257, 1025)], ids=lambda s: "x".join(map(str, s)))
def test_f16_output_is_the_rounded_fp32_output(shape, causal, d, dtype, plan):
    import torch

    import scaled_masked_attention_amd as sma

    kw = _plan_kwargs(plan, dtype)
    B, H, sq, skv = shape
    (q, k, v), bits = gen.random_case(720 + sq + 3 * skv + d, (B, H, sq, d), (B, H, skv, d),
                                      sigma_qk=1.0 if dtype == "f32" else 3.0, dtype=dtype)
    tq, tk, tv = to_device((q, k, v), bits, dtype)
    scale = 1.0 / math.sqrt(d)
    o32, l32 = sma.attention_fwd(tq, tk, tv, scale=scale, causal=causal, return_lse=True, **kw)
    o16, l16 = sma.attention_fwd(tq, tk, tv, scale=scale, causal=causal, return_lse=True,
                                 out_dtype=torch.float16, **kw)
    torch.cuda.synchronize()
    assert o16.dtype == torch.float16
    f32 = o32.cpu().numpy()
    assert np.array_equal(_bits(o16), f32.astype(np.float16).view(np.uint16)), "fp16 O is not RNE of the fp32 O"
    assert torch.equal(l16, l32), "LSE changed with the output dtype"
    o_ref, _ = oracle.attention_fwd(q, k, v, scale, causal)
    got = o16.float().cpu().numpy().astype(np.float64)
    bar = ({"f32": F32_MAX_ABS, "bf16": BF16_MAX_ABS, "f16": F16_MAX_ABS}[dtype]
           + 2.0 ** -11 * np.abs(f32.astype(np.float64)) + 2.0 ** -25)
    assert np.all(np.abs(got - o_ref) <= bar)
    er = empty_rows(sq, skv, causal)
    if er.any():
        assert np.all(_bits(o16)[:, :, er] == 0)


def test_f16_output_with_a_mask_and_bshd_layout():
    import torch

    import scaled_masked_attention_amd as sma

    (q, k, v), _ = gen.random_case(740, (2, 3, 100, 64), (2, 3, 150, 64))
    m = torch.from_numpy((gen.uniform24(741, np.arange(100 * 150, dtype=np.uint64)) < 0.4).reshape(100, 150)).to("cuda")
    tq, tk, tv = (torch.from_numpy(x).to("cuda").transpose(1, 2).contiguous() for x in (q, k, v))
    o32 = sma.attention_fwd(tq, tk, tv, scale=0.125, causal=True, mask=m, layout="bshd")
    o16 = sma.attention_fwd(tq, tk, tv, scale=0.125, causal=True, mask=m, layout="bshd", out_dtype=torch.float16)
    torch.cuda.synchronize()
    assert np.array_equal(_bits(o16), o32.cpu().numpy().astype(np.float16).view(np.uint16))

