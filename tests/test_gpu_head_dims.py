"""Head dims 32 and 256 through the C ABI, against the oracle: fp32 inputs on the 128-row fp32
kernel (with the split combine) and, at d = 32, on the in-workgroup key-split kernel; 16-bit
inputs on the 16-bit kernel.

Ragged shapes that span several query blocks and key tiles, causal and not, unsplit and split
across workgroups (forced and automatic), a hard mask, the bshd layout, bf16 output, rows
with no admitted key, and zero and negative scales.
"""
import functools
import math

import numpy as np
import pytest

import gen
import oracle
from helpers import check_parity, run_gpu, to_device

pytestmark = pytest.mark.gpu

HEAD_DIMS = [32, 256]


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    torch = pytest.importorskip("torch")
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import scaled_masked_attention_amd as sma

    sma.library()


def _qblock(nsplit):
    import scaled_masked_attention_amd as sma

    return dict(kernel=sma.SMA_KERNEL_F32_QBLOCK, nsplit=nsplit)


def _ksplit():
    import scaled_masked_attention_amd as sma

    return dict(kernel=sma.SMA_KERNEL_F32_KSPLIT, nsplit=1)


def _plans(d, nsplit):
    """The 128-row kernel unsplit and split nsplit ways, and at d = 32 the in-workgroup
    key-split kernel."""
    return [_qblock(1), _qblock(nsplit)] + ([_ksplit()] if d == 32 else [])


SHAPES = [(1, 2, 128, 128), (2, 3, 200, 200), (1, 2, 77, 300), (2, 1, 300, 77), (1, 1, 1, 1000),
          (1, 1, 513, 513), (1, 3, 257, 1025)]


@functools.lru_cache(maxsize=4)
def _case(shape, causal, d):
    B, H, sq, skv = shape
    (q, k, v), _ = gen.random_case(500 + sq + 7 * skv + d, (B, H, sq, d), (B, H, skv, d))
    scale = 1.0 / math.sqrt(d)
    return (q, k, v), scale, oracle.attention_fwd(q, k, v, scale, causal)


@pytest.mark.parametrize("plan", ["auto", "unsplit", "split3", "ksplit"])
@pytest.mark.parametrize("d", HEAD_DIMS)
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("shape", SHAPES, ids=lambda s: "x".join(map(str, s)))
def test_parity(shape, causal, d, plan):
    import scaled_masked_attention_amd as sma

    (q, k, v), scale, (o_ref, lse_ref) = _case(shape, causal, d)
    kw = {"auto": {}, "unsplit": _qblock(1), "split3": _qblock(3), "ksplit": _ksplit()}[plan]
    dev = to_device((q, k, v), None, "f32")
    if plan == "ksplit" and d == 256:  # its per-wave K/V slots would not fit LDS
        with pytest.raises(sma.SMAError) as e:
            run_gpu(*dev, scale, causal, **kw)
        assert e.value.status == sma.SMA_ERR_UNSUPPORTED
        return
    o, lse = run_gpu(*dev, scale, causal, **kw)
    check_parity(o, lse, o_ref, lse_ref, "f32", f"{shape} causal={causal} d={d} {plan}")


@pytest.mark.parametrize("d", HEAD_DIMS)
@pytest.mark.parametrize("causal", [False, True])
def test_automatic_split_matches_oracle_and_unsplit(d, causal):
    """Few query blocks and long rows: the planner splits keys across workgroups."""
    import torch

    import scaled_masked_attention_amd as sma

    B, H, sq, skv = 1, 2, 200, 3000
    (q, k, v), _ = gen.random_case(600 + d, (B, H, sq, d), (B, H, skv, d))
    assert sma.plan(sma.SMA_DTYPE_F32, B, H, sq, skv, d, causal).nsplit > 1
    dev = to_device((q, k, v), None, "f32")
    o_s, l_s = run_gpu(*dev, 0.07, causal)
    o_n, l_n = run_gpu(*dev, 0.07, causal, workspace=torch.empty(16, dtype=torch.uint8, device="cuda"))
    o_ref, lse_ref = oracle.attention_fwd(q, k, v, 0.07, causal)
    check_parity(o_s, l_s, o_ref, lse_ref, "f32", f"d={d} split")
    check_parity(o_n, l_n, o_ref, lse_ref, "f32", f"d={d} unsplit")


@pytest.mark.parametrize("nsplit", [1, 3, "ksplit"])
@pytest.mark.parametrize("form", ["shared", "full"])
@pytest.mark.parametrize("d", HEAD_DIMS)
@pytest.mark.parametrize("causal", [False, True])
def test_masked(causal, d, form, nsplit):
    if nsplit == "ksplit" and d == 256:
        pytest.skip("the in-workgroup key-split kernel is not built for head dim 256")
    import torch

    import scaled_masked_attention_amd as sma

    B, H, sq, skv = 2, 2, 300, 333
    (q, k, v), _ = gen.random_case(700 + d, (B, H, sq, d), (B, H, skv, d))
    shape = (1, 1, sq, skv) if form == "shared" else (B, H, sq, skv)
    n = int(np.prod(shape))
    mask = gen.uniform24(701 + causal, np.arange(n, dtype=np.uint64)).reshape(shape) < 0.5
    mask[..., 40:44, :] = False  # rows that admit nothing
    mask = mask.astype(np.uint8)
    tq, tk, tv = to_device((q, k, v), None, "f32")
    o, lse = sma.attention_fwd(tq, tk, tv, scale=0.1, causal=causal, return_lse=True,
                               mask=torch.from_numpy(mask).to("cuda"),
                               **(_ksplit() if nsplit == "ksplit" else _qblock(nsplit)))
    torch.cuda.synchronize()
    o_ref, lse_ref = oracle.attention_fwd_masked(q, k, v, mask, 0.1, causal)
    check_parity(o.cpu().numpy().astype(np.float64), lse.cpu().numpy().astype(np.float64), o_ref,
                 lse_ref, "f32", f"mask d={d} {form} nsplit={nsplit}")


@pytest.mark.parametrize("nsplit", [1, 3, "ksplit"])
@pytest.mark.parametrize("d", HEAD_DIMS)
def test_bshd_layout_and_bf16_output(d, nsplit):
    """bshd equals bhsd transposed, bit for bit; bf16 output is the fp32 output rounded to
    nearest even."""
    import torch

    import scaled_masked_attention_amd as sma

    B, H, sq, skv = 2, 3, 190, 230
    (q, k, v), _ = gen.random_case(800 + d, (B, H, sq, d), (B, H, skv, d))
    tq, tk, tv = to_device((q, k, v), None, "f32")
    if nsplit == "ksplit" and d == 256:
        pytest.skip("the in-workgroup key-split kernel is not built for head dim 256")
    kw = _ksplit() if nsplit == "ksplit" else _qblock(nsplit)
    o1, l1 = sma.attention_fwd(tq, tk, tv, scale=0.1, causal=True, return_lse=True, **kw)
    t2 = [x.transpose(1, 2).contiguous() for x in (tq, tk, tv)]
    o2, l2 = sma.attention_fwd(*t2, scale=0.1, causal=True, return_lse=True, layout="bshd", **kw)
    o3 = sma.attention_fwd(tq, tk, tv, scale=0.1, causal=True, out_dtype=torch.bfloat16, **kw)
    o4 = sma.attention_fwd(*t2, scale=0.1, causal=True, layout="bshd", out_dtype=torch.bfloat16, **kw)
    torch.cuda.synchronize()
    assert torch.equal(o2.transpose(1, 2), o1) and torch.equal(l1, l2)
    bits = gen.f32_to_bf16_bits(o1.cpu().numpy())
    assert np.array_equal(o3.view(torch.int16).cpu().numpy().view(np.uint16), bits)
    assert np.array_equal(o4.transpose(1, 2).contiguous().view(torch.int16).cpu().numpy()
                          .view(np.uint16), bits)
    o_ref, lse_ref = oracle.attention_fwd(q, k, v, 0.1, True)
    check_parity(o1.cpu().numpy().astype(np.float64), l1.cpu().numpy().astype(np.float64), o_ref,
                 lse_ref, "f32", f"d={d}")


@pytest.mark.parametrize("d", HEAD_DIMS)
def test_no_keys_and_rows_without_keys(d):
    import torch

    import scaled_masked_attention_amd as sma

    q = torch.randn(1, 2, 70, d, device="cuda")
    k = torch.empty(1, 2, 0, d, device="cuda")
    out = torch.full((1, 2, 70, d), float("nan"), device="cuda")
    for kw in _plans(d, 1)[1:]:
        out.fill_(float("nan"))
        o, lse = sma.attention_fwd(q, k, k, causal=False, return_lse=True, out=out, **kw)
        torch.cuda.synchronize()
        assert torch.all(o == 0) and not torch.any(torch.signbit(o)) and torch.all(torch.isneginf(lse))
    # causal with more queries than keys: the first sq - skv rows admit nothing
    (qn, kn, vn), _ = gen.random_case(900 + d, (1, 2, 150, d), (1, 2, 100, d))
    for kw in _plans(d, 2):
        o, lse = run_gpu(*to_device((qn, kn, vn), None, "f32"), 0.2, True, **kw)
        assert np.all(o[:, :, :50] == 0) and np.all(np.isneginf(lse[:, :, :50]))
        o_ref, lse_ref = oracle.attention_fwd(qn, kn, vn, 0.2, True)
        check_parity(o, lse, o_ref, lse_ref, "f32", f"d={d} {kw}")


@pytest.mark.parametrize("scale", [0.0, -0.3, 2.5])
@pytest.mark.parametrize("d", HEAD_DIMS)
def test_zero_negative_and_large_scale(d, scale):
    """Inputs are multiples of 1/2 in [-1, 1], so every dot product is exact in fp32 and the
    fp32 bar holds even where scale * |s| reaches the hundreds."""
    (q, k, v), _ = gen.random_case(1000 + d, (1, 2, 160, d), (1, 2, 200, d))
    q, k = ((np.clip(np.round(x * 2), -2, 2) / 2).astype(np.float32) for x in (q, k))
    for kw in _plans(d, 2):
        o, lse = run_gpu(*to_device((q, k, v), None, "f32"), scale, True, **kw)
        o_ref, lse_ref = oracle.attention_fwd(q, k, v, scale, True)
        check_parity(o, lse, o_ref, lse_ref, "f32", f"d={d} scale={scale} {kw}")


def test_large_scale_random_scores_within_rounding_bound():
    """N(0, 1) inputs at head dim 256 and scale 2.5. Each score is a dot product rounded in
    fp32, and exp turns its absolute error into a relative error of p. So O moves by about
    scale * u * sum_c |q_c k_c| * max|v| (u = 2^-24): about 1.4e-4 here, beyond the plain fp32
    bar. Bound used: 2e-5 plus twice that, with the largest sum over all (i, j)."""
    d, scale = 256, 2.5
    (q, k, v), _ = gen.random_case(1050, (1, 2, 160, d), (1, 2, 200, d))
    o, lse = run_gpu(*to_device((q, k, v), None, "f32"), scale, True, **_qblock(1))
    o_ref, lse_ref = oracle.attention_fwd(q, k, v, scale, True)
    absdot = np.einsum("bhic,bhjc->bhij", np.abs(q.astype(np.float64)), np.abs(k.astype(np.float64)))
    tol = 2e-5 + 2 * 2.0**-24 * scale * absdot.max() * np.abs(v).max()
    err = float(np.abs(o - o_ref).max())
    assert err <= tol, (err, tol)
    assert np.array_equal(np.isneginf(lse), np.isneginf(lse_ref))
    fin = np.isfinite(lse_ref)
    assert np.all(np.abs(lse[fin] - lse_ref[fin]) <= tol * np.maximum(1.0, np.abs(lse_ref[fin])))


@pytest.mark.parametrize("d", HEAD_DIMS)
def test_deterministic_bitwise(d):
    (q, k, v), _ = gen.random_case(1100 + d, (2, 2, 300, d), (2, 2, 400, d))
    dev = to_device((q, k, v), None, "f32")
    for kw in _plans(d, 3):
        a = run_gpu(*dev, 0.1, False, **kw)
        b = run_gpu(*dev, 0.1, False, **kw)
        assert np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1])


# ------------------------------------------------------------------ 16-bit inputs
# The 16-bit kernel at head dims 32 (8 waves, 64-key tiles, K and V copied by half the
# waves each) and 256 (4 waves of 32 rows, 32-key tiles).
def _k16(nsplit):
    import scaled_masked_attention_amd as sma

    return dict(kernel=sma.SMA_KERNEL_BF16_QBLOCK, nsplit=nsplit)


@functools.lru_cache(maxsize=4)
def _case16(shape, causal, d, dtype):
    B, H, sq, skv = shape
    (q, k, v), bits = gen.random_case(900 + sq + 7 * skv + d, (B, H, sq, d), (B, H, skv, d),
                                      sigma_qk=3.0, dtype=dtype)
    scale = 1.0 / math.sqrt(d)
    return (q, k, v), bits, scale, oracle.attention_fwd(q, k, v, scale, causal)


@pytest.mark.parametrize("plan", ["auto", "unsplit", "split3"])
@pytest.mark.parametrize("dtype", ["bf16", "f16"])
@pytest.mark.parametrize("d", HEAD_DIMS)
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("shape", SHAPES, ids=lambda s: "x".join(map(str, s)))
def test_parity_16bit(shape, causal, d, dtype, plan):
    (q, k, v), bits, scale, (o_ref, lse_ref) = _case16(shape, causal, d, dtype)
    kw = {} if plan == "auto" else _k16(1 if plan == "unsplit" else 3)
    o, lse = run_gpu(*to_device((q, k, v), bits, dtype), scale, causal, **kw)
    check_parity(o, lse, o_ref, lse_ref, dtype, f"{shape} causal={causal} d={d} {dtype} {plan}")


@pytest.mark.parametrize("dtype", ["bf16", "f16"])
@pytest.mark.parametrize("d", HEAD_DIMS)
def test_16bit_edge_cases(d, dtype):
    """No keys at all (O = +0, LSE = -inf); causal rows before the first key exactly zero with
    NaN queries; Q = 0 (the mean of V over the admitted keys); zero and negative scales."""
    import torch

    import scaled_masked_attention_amd as sma

    tdt = torch.bfloat16 if dtype == "bf16" else torch.float16
    q0 = torch.randn(1, 2, 70, d, device="cuda").to(tdt)
    k0 = torch.empty(1, 2, 0, d, device="cuda", dtype=tdt)
    o, lse = sma.attention_fwd(q0, k0, k0, return_lse=True)
    torch.cuda.synchronize()
    assert torch.all(o == 0) and not torch.any(torch.signbit(o)) and torch.all(torch.isneginf(lse))
    B, H, sq, skv = 1, 2, 300, 100
    (q, k, v), bits = gen.random_case(950 + d, (B, H, sq, d), (B, H, skv, d), sigma_qk=3.0, dtype=dtype)
    q = q.copy()
    qb = bits[0].copy()
    qb[:, :, : sq - skv] = 0x7FC0 if dtype == "bf16" else 0x7E00  # NaN in rows that see no key
    q[:, :, : sq - skv] = np.nan
    for scale, nsplit in ((1.0 / math.sqrt(d), 1), (0.0, 1), (-0.2, 3)):
        o, lse = run_gpu(*to_device((q, k, v), (qb, bits[1], bits[2]), dtype), scale, True,
                         **_k16(nsplit))
        assert np.all(o[:, :, : sq - skv] == 0.0) and np.all(np.isneginf(lse[:, :, : sq - skv]))
        qn = np.nan_to_num(q, nan=0.0)
        o_ref, lse_ref = oracle.attention_fwd(qn, k, v, scale, True)
        check_parity(o, lse, o_ref, lse_ref, dtype, f"d={d} {dtype} scale={scale}")
    zero = np.zeros((B, H, sq, d), np.float32)
    zbits = np.zeros((B, H, sq, d), np.uint16)
    o, lse = run_gpu(*to_device((zero, k, v), (zbits, bits[1], bits[2]), dtype), 0.3, False)
    o_ref, lse_ref = oracle.attention_fwd(zero, k, v, 0.3, False)
    check_parity(o, lse, o_ref, lse_ref, dtype, f"d={d} {dtype} Q=0")


@pytest.mark.parametrize("nsplit", [1, 2])
@pytest.mark.parametrize("d", HEAD_DIMS)
@pytest.mark.parametrize("causal", [False, True])
def test_16bit_masked(causal, d, nsplit):
    """A mask of whole 32x64 blocks admitting nothing, everything or a random half (every
    tile class of the 16-bit kernel), per (batch, head)."""
    import torch

    import scaled_masked_attention_amd as sma

    B, H, sq, skv = 2, 2, 300, 333
    (q, k, v), bits = gen.random_case(960 + d, (B, H, sq, d), (B, H, skv, d), sigma_qk=3.0,
                                      dtype="bf16")
    nrb, ntk = (sq + 31) // 32, (skv + 63) // 64
    kind = np.floor(gen.uniform24(961 + d, np.arange(B * H * nrb * ntk, dtype=np.uint64)) * 3
                    ).reshape(B, H, nrb, ntk)
    rnd = gen.uniform24(962 + d, np.arange(B * H * sq * skv, dtype=np.uint64)).reshape(B, H, sq, skv) < 0.5
    mask = np.zeros((B, H, sq, skv), bool)
    for r in range(nrb):
        for t in range(ntk):
            rs, ts = slice(32 * r, 32 * r + 32), slice(64 * t, 64 * t + 64)
            kk = kind[:, :, r, t][:, :, None, None]
            mask[:, :, rs, ts] = np.where(kk == 1, True, np.where(kk == 2, rnd[:, :, rs, ts], False))
    mask = mask.astype(np.uint8)
    tq, tk, tv = to_device((q, k, v), bits, "bf16")
    o, lse = sma.attention_fwd(tq, tk, tv, scale=0.1, causal=causal, return_lse=True,
                               mask=torch.from_numpy(mask).to("cuda"), **_k16(nsplit))
    torch.cuda.synchronize()
    o_ref, lse_ref = oracle.attention_fwd_masked(q, k, v, mask, 0.1, causal)
    check_parity(o.cpu().numpy().astype(np.float64), lse.cpu().numpy().astype(np.float64), o_ref,
                 lse_ref, "bf16", f"16-bit mask d={d} nsplit={nsplit}")


@pytest.mark.parametrize("d", HEAD_DIMS)
def test_16bit_bshd_layout_and_16bit_output(d):
    """bshd equals bhsd transposed, bit for bit; bf16 output is the fp32 output rounded."""
    import torch

    import scaled_masked_attention_amd as sma

    B, H, sq, skv = 2, 3, 190, 230
    (q, k, v), bits = gen.random_case(970 + d, (B, H, sq, d), (B, H, skv, d), sigma_qk=3.0,
                                      dtype="bf16")
    tq, tk, tv = to_device((q, k, v), bits, "bf16")
    o1, l1 = sma.attention_fwd(tq, tk, tv, scale=0.1, causal=True, return_lse=True)
    t2 = [x.transpose(1, 2).contiguous() for x in (tq, tk, tv)]
    o2, l2 = sma.attention_fwd(*t2, scale=0.1, causal=True, return_lse=True, layout="bshd")
    o3 = sma.attention_fwd(tq, tk, tv, scale=0.1, causal=True, out_dtype=torch.bfloat16)
    torch.cuda.synchronize()
    assert torch.equal(o2.transpose(1, 2), o1) and torch.equal(l1, l2)
    assert np.array_equal(o3.view(torch.int16).cpu().numpy().view(np.uint16),
                          gen.f32_to_bf16_bits(o1.cpu().numpy()))
