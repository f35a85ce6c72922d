"""HIP path vs the CPU oracle, element by element, through the C ABI.

Small and ragged shapes compare every output. The full-size workloads run in
the benchmark's launch configuration and compare every output against the
whole oracle run; sampled-row variants (and the 128-row fp32 kernel on the
fp32 workloads) run alongside.
"""
import functools
import math

import numpy as np
import pytest

import gen
import helpers
import oracle
from helpers import (check_parity, empty_rows, run_gpu, sample_rows, to_device, workload_case)

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    torch = pytest.importorskip("torch")
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import scaled_masked_attention_amd as sma

    sma.library()  # fail loudly if the HIP library is missing


def _case(seed, B, H, sq, skv, d, dtype, sigma_qk=1.0):
    return gen.random_case(seed, (B, H, sq, d), (B, H, skv, d), sigma_qk=sigma_qk, dtype=dtype)


SHAPES = [  # (B, H, sq, skv): several tiles with ragged tails, cross shapes both ways, one head
    (1, 2, 128, 128), (2, 3, 200, 200), (1, 2, 77, 300), (2, 1, 300, 77), (1, 1, 1, 1000),
    (1, 1, 1000, 1), (1, 1, 513, 513), (3, 2, 64, 96), (1, 4, 257, 1025),
]


# Forced plans: every kernel, unsplit and split across workgroups, on the same inputs.
PLANS = {"auto": None, "qblock": ("qblock", 1), "split3": ("qblock", 3), "ksplit": ("ksplit", 1)}

# The in-workgroup key-split kernel is fp32 only: it is paired with fp32 inputs alone.
DTYPE_PLANS = [(dt, pl) for dt in ("f32", "bf16", "f16") for pl in PLANS if dt == "f32" or pl != "ksplit"]


def plan_kwargs(plan, dtype):
    import scaled_masked_attention_amd as sma

    if PLANS[plan] is None:
        return {}
    kind, nsplit = PLANS[plan]
    if kind == "ksplit":
        assert dtype == "f32", "the in-workgroup key-split kernel is fp32 only"
        return dict(kernel=sma.SMA_KERNEL_F32_KSPLIT, nsplit=1)
    kern = sma.SMA_KERNEL_F32_QBLOCK if dtype == "f32" else sma.SMA_KERNEL_BF16_QBLOCK
    return dict(kernel=kern, nsplit=nsplit)


@functools.lru_cache(maxsize=8)
def _small_case(shape, causal, d, dtype):
    B, H, sq, skv = shape
    sig = 1.0 if dtype == "f32" else 3.0
    (q, k, v), bits = _case(100 + sq + 7 * skv + d, B, H, sq, skv, d, dtype, sigma_qk=sig)
    scale = 1.0 / math.sqrt(d)
    o_ref, lse_ref = oracle.attention_fwd(q, k, v, scale, causal)
    return (q, k, v), bits, scale, o_ref, lse_ref


@pytest.mark.parametrize("dtype,plan", DTYPE_PLANS)
@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("shape", SHAPES, ids=lambda s: "x".join(map(str, s)))
def test_parity_small(shape, causal, d, dtype, plan):
    kw = plan_kwargs(plan, dtype)
    vals, bits, scale, o_ref, lse_ref = _small_case(shape, causal, d, dtype)
    o, lse = run_gpu(*to_device(vals, bits, dtype), scale, causal, **kw)
    check_parity(o, lse, o_ref, lse_ref, dtype, f"{shape} causal={causal} d={d} {dtype} {plan}")


@pytest.mark.parametrize("name", ["f32_causal_b1h2_s128_d64", "f32_b4h8_s512_d64"])
def test_parity_small_workloads_full(name):
    w, vals, bits = workload_case(name)
    o, lse = run_gpu(*to_device(vals, bits, w.dtype), w.scale, w.causal)
    o_ref, lse_ref = _workload_oracle(name)
    check_parity(o, lse, o_ref, lse_ref, w.dtype, name)


@pytest.mark.parametrize("plan", ["qblock", "split3", "ksplit"])
@pytest.mark.parametrize("name", ["f32_causal_b1h2_s128_d64", "f32_b4h8_s512_d64"])
def test_parity_small_workloads_every_kernel(name, plan):
    w, vals, bits = workload_case(name)
    kw = plan_kwargs(plan, w.dtype)
    o, lse = run_gpu(*to_device(vals, bits, w.dtype), w.scale, w.causal, **kw)
    o_ref, lse_ref = _workload_oracle(name)
    check_parity(o, lse, o_ref, lse_ref, w.dtype, f"{name} {plan}")


@functools.lru_cache(maxsize=2)
def _workload_oracle(name):
    w, vals, _ = workload_case(name)
    return oracle.attention_fwd(*vals, w.scale, w.causal)


@pytest.mark.parametrize("name", ["f32_causal_b8h16_s2048_d128", "f32_cross_b2h32_q256_kv4096_d128",
                                  "f32_cross_causal_b2h32_q256_kv4096_d128"])
def test_parity_full_size_qblock_sampled(name):
    """The 128-row fp32 kernel (with its automatic key split) at full size; the automatic
    plan runs the in-workgroup key-split kernel on these shapes."""
    import scaled_masked_attention_amd as sma

    w, vals, bits = workload_case(name)
    kw = dict(kernel=sma.SMA_KERNEL_F32_QBLOCK, nsplit=0)
    o, lse = run_gpu(*to_device(vals, bits, w.dtype), w.scale, w.causal, **kw)
    rows = sample_rows(w.batch, w.heads, w.seq_q, w.seq_kv, w.causal, n_random=256, seed=8)
    o_ref, lse_ref = oracle.attention_fwd(*vals, w.scale, w.causal, rows=rows)
    check_parity(o.reshape(-1, w.head_dim)[rows], lse.reshape(-1)[rows], o_ref, lse_ref, w.dtype,
                 f"{name} qblock")


@pytest.mark.parametrize("name", ["f32_causal_b8h16_s2048_d128", "f32_cross_b2h32_q256_kv4096_d128",
                                  "f32_cross_causal_b2h32_q256_kv4096_d128", "bf16_causal_b1h32_s16384_d128",
                                  "f16_causal_b1h32_s16384_d128", "f32_causal_b8h16_s2048_d32",
                                  "f32_causal_b8h16_s2048_d256", "bf16_causal_b1h32_s16384_d32",
                                  "bf16_causal_b1h32_s16384_d256"])
def test_parity_full_size_sampled(name):
    w, vals, bits = workload_case(name)
    o, lse = run_gpu(*to_device(vals, bits, w.dtype), w.scale, w.causal)
    B, H, sq, skv = w.batch, w.heads, w.seq_q, w.seq_kv
    rows = sample_rows(B, H, sq, skv, w.causal, n_random=512 if w.dtype == "f32" else 192, seed=7)
    o_ref, lse_ref = oracle.attention_fwd(*vals, w.scale, w.causal, rows=rows)
    o_s = o.reshape(-1, w.head_dim)[rows]
    l_s = lse.reshape(-1)[rows]
    stats = check_parity(o_s, l_s, o_ref, lse_ref, w.dtype, name)
    print(f"{name}: {len(rows)} sampled rows {stats}")
    # Everywhere: finite, and rows that see no key are exactly zero.
    assert np.all(np.isfinite(o))
    er = empty_rows(sq, skv, w.causal)
    if er.any():
        assert np.all(o.reshape(B * H, sq, -1)[:, er] == 0.0)


@pytest.mark.parametrize("name", ["f32_causal_b8h16_s2048_d128", "f32_cross_b2h32_q256_kv4096_d128",
                                  "f32_cross_causal_b2h32_q256_kv4096_d128", "bf16_causal_b1h32_s16384_d128",
                                  "f16_causal_b1h32_s16384_d128", "f32_causal_b8h16_s2048_d32",
                                  "f32_causal_b8h16_s2048_d256", "bf16_causal_b1h32_s16384_d32",
                                  "bf16_causal_b1h32_s16384_d256"])
@pytest.mark.timeout(600)  # the whole oracle: about a minute per 16384-token workload at d = 128
def test_parity_full_size_whole(name):
    """The large workloads at full size in the benchmark's launch configuration (the
    library's own plan), every element of O and LSE against the whole oracle run: max-abs
    and, for 16-bit inputs, relative L2 over the whole O tensor."""
    w, vals, bits = workload_case(name)
    o, lse = run_gpu(*to_device(vals, bits, w.dtype), w.scale, w.causal)
    o_ref, lse_ref = oracle.attention_fwd(*vals, w.scale, w.causal)
    stats = check_parity(o, lse, o_ref, lse_ref, w.dtype, f"{name} whole")
    line = (f"{name}: all {o.size} outputs, max_abs {stats['max_abs']:.3e}, rel_l2 "
            f"{stats['rel_l2']:.3e}, lse_rel {stats['lse_rel']:.3e}")
    helpers.SUMMARY.append(line)
    print(line, flush=True)


# ------------------------------------------------------------------ edge cases
# Each edge case runs on every kernel: the fp32 128-row kernel (unsplit), the
# fp32 in-workgroup key-split kernel, and the 16-bit kernel with bf16 and fp16 inputs.
VARIANTS = ["f32-qblock", "f32-ksplit", "bf16", "f16"]


def variant_kwargs(variant):
    import scaled_masked_attention_amd as sma

    if variant == "f32-qblock":
        return "f32", dict(kernel=sma.SMA_KERNEL_F32_QBLOCK, nsplit=1)
    if variant == "f32-ksplit":
        return "f32", dict(kernel=sma.SMA_KERNEL_F32_KSPLIT, nsplit=1)
    return variant, dict(kernel=sma.SMA_KERNEL_BF16_QBLOCK, nsplit=1)


@pytest.mark.parametrize("variant", VARIANTS)
def test_no_keys_gives_zero_and_neg_inf(variant):
    dtype, kw = variant_kwargs(variant)
    import torch

    import scaled_masked_attention_amd as sma

    tdt = {"f32": torch.float32, "bf16": torch.bfloat16, "f16": torch.float16}[dtype]
    q = torch.randn(2, 3, 70, 128, device="cuda").to(tdt)
    k = torch.empty(2, 3, 0, 128, device="cuda", dtype=tdt)
    out = torch.full((2, 3, 70, 128), float("nan"), device="cuda")
    o, lse = sma.attention_fwd(q, k, k, causal=False, return_lse=True, out=out, **kw)
    torch.cuda.synchronize()
    assert torch.all(o == 0) and not torch.any(torch.signbit(o))
    assert torch.all(torch.isneginf(lse))


@pytest.mark.parametrize("variant", VARIANTS)
def test_fully_masked_rows_exact_zero_with_nan_queries(variant):
    dtype, kw = variant_kwargs(variant)
    sq, skv, d = 300, 100, 128
    (q, k, v), bits = _case(31, 1, 2, sq, skv, d, dtype)
    tq, tk, tv = to_device((q, k, v), bits, dtype)
    tq[:, :, : sq - skv] = float("nan")  # rows with no admitted key: content must not matter
    o, lse = run_gpu(tq, tk, tv, 0.1, True, **kw)
    assert np.all(o[:, :, : sq - skv] == 0.0) and not np.any(np.signbit(o[:, :, : sq - skv]))
    assert np.all(np.isneginf(lse[:, :, : sq - skv]))
    o_ref, lse_ref = oracle.attention_fwd(q, k, v, 0.1, True)
    check_parity(o, lse, o_ref, lse_ref, dtype, "masked rows")


@pytest.mark.parametrize("variant", VARIANTS)
@pytest.mark.parametrize("causal", [False, True])
def test_q_zero_is_prefix_mean(variant, causal):
    dtype, kw = variant_kwargs(variant)
    sq, skv, d = 150, 250, 64
    (q, k, v), bits = _case(32, 1, 2, sq, skv, d, dtype)
    q[:] = 0
    if bits is not None:
        bits = (np.zeros_like(bits[0]),) + bits[1:]
    o, lse = run_gpu(*to_device((q, k, v), bits, dtype), 0.3, causal, **kw)
    o_ref, lse_ref = oracle.attention_fwd(q, k, v, 0.3, causal)
    check_parity(o, lse, o_ref, lse_ref, dtype, "q=0")


@pytest.mark.parametrize("variant", VARIANTS)
def test_v_ones_gives_ones(variant):
    dtype, kw = variant_kwargs(variant)
    sq, skv, d = 260, 333, 128
    (q, k, v), bits = _case(33, 2, 2, sq, skv, d, dtype, sigma_qk=3.0)
    v[:] = 1.0
    if bits is not None:
        bits = bits[:2] + (gen.to_16bit(v, dtype)[1],)
    o, _ = run_gpu(*to_device((q, k, v), bits, dtype), 1.0 / math.sqrt(d), True, **kw)
    er = empty_rows(sq, skv, True)
    tol = {"f32": 2e-5, "bf16": 2 ** -8, "f16": 2 ** -11}[dtype]
    assert np.all(np.abs(o[:, :, ~er] - 1.0) <= tol)


@pytest.mark.parametrize("variant", VARIANTS)
def test_one_hot_v_extracts_probabilities(variant):
    """With V = I (Skv = d keys), O[i, c] = P[i, c]: the GPU's implicit P is read out."""
    dtype, kw = variant_kwargs(variant)
    sq, d = 96, 64
    (q, k, _), bits = _case(34, 1, 1, sq, d, d, dtype, sigma_qk=2.0)
    v = np.eye(d, dtype=np.float32).reshape(1, 1, d, d)
    if bits is not None:
        bits = bits[:2] + (gen.to_16bit(v, dtype)[1],)
    o, _ = run_gpu(*to_device((q, k, v), bits, dtype), 0.2, True, **kw)
    p = oracle.softmax_probs(q[0, 0], k[0, 0], 0.2, True)
    tol = {"f32": 2e-5, "bf16": 2e-2, "f16": 4e-3}[dtype]
    assert np.abs(o[0, 0] - p).max() <= tol


@pytest.mark.parametrize("variant", VARIANTS)
def test_key_shift_beyond_fp32_exp_range(variant):
    """Every score of a row shifted by ~181 (fp32 exp overflows past ~88.7): only a
    max-subtracted softmax stays finite. Inputs are multiples of 1/2 in [-1, 1]
    (exact in bf16 and fp32), so every dot product is exact in fp32 and the
    comparison isolates the softmax from dot-product rounding at |s| ~ 2000."""
    dtype, kw = variant_kwargs(variant)
    sq, skv, d = 130, 190, 128
    (q, k, v), _ = _case(35, 1, 2, sq, skv, d, "f32")
    q = (np.clip(np.round(q * 2), -2, 2) / 2).astype(np.float32)
    k = (np.clip(np.round(k * 2), -2, 2) / 2).astype(np.float32)
    q[..., 0] = 8.0
    k[..., 0] = 256.0  # scale * 8 * 256 = 181 added to every score of a row
    bits = None
    if dtype != "f32":
        pairs = [gen.to_16bit(x, dtype) for x in (q, k, v)]
        (q, k, v), bits = tuple(p[0] for p in pairs), tuple(p[1] for p in pairs)
    scale = 1.0 / math.sqrt(d)
    o, lse = run_gpu(*to_device((q, k, v), bits, dtype), scale, True, **kw)
    o_ref, lse_ref = oracle.attention_fwd(q, k, v, scale, True)
    assert lse_ref[np.isfinite(lse_ref)].min() > 150
    check_parity(o, lse, o_ref, lse_ref, dtype, "key shift")


@pytest.mark.parametrize("variant", VARIANTS)
@pytest.mark.parametrize("scale", [-0.09, 0.0, 0.7])
def test_negative_zero_and_large_scale(variant, scale):
    dtype, kw = variant_kwargs(variant)
    (q, k, v), bits = _case(36, 1, 2, 140, 170, 128, dtype)
    o, lse = run_gpu(*to_device((q, k, v), bits, dtype), scale, True, **kw)
    o_ref, lse_ref = oracle.attention_fwd(q, k, v, scale, True)
    check_parity(o, lse, o_ref, lse_ref, dtype, f"scale={scale}")


@pytest.mark.parametrize("variant", VARIANTS)
def test_causal_single_query_equals_unmasked(variant):
    dtype, kw = variant_kwargs(variant)
    (q, k, v), bits = _case(37, 2, 2, 1, 700, 128, dtype)
    dev = to_device((q, k, v), bits, dtype)
    o0, l0 = run_gpu(*dev, 0.1, False, **kw)
    o1, l1 = run_gpu(*dev, 0.1, True, **kw)
    assert np.array_equal(o0, o1) and np.array_equal(l0, l1)


@pytest.mark.parametrize("variant", VARIANTS)
def test_deterministic_bitwise(variant):
    dtype, kw = variant_kwargs(variant)
    (q, k, v), bits = _case(38, 2, 4, 333, 777, 128, dtype)
    dev = to_device((q, k, v), bits, dtype)
    o0, l0 = run_gpu(*dev, 0.1, True, **kw)
    o1, l1 = run_gpu(*dev, 0.1, True, **kw)
    assert np.array_equal(o0, o1) and np.array_equal(l0, l1)


@pytest.mark.parametrize("variant", VARIANTS)
def test_guard_bands_untouched_and_nan_prefill_overwritten(variant):
    dtype, kw = variant_kwargs(variant)
    import torch

    import scaled_masked_attention_amd as sma

    B, H, sq, skv, d = 1, 3, 190, 260, 128
    (q, k, v), bits = _case(39, B, H, sq, skv, d, dtype)
    tq, tk, tv = to_device((q, k, v), bits, dtype)
    n_o, n_l, pad = B * H * sq * d, B * H * sq, 1024
    big_o = torch.full((n_o + 2 * pad,), 12345.0, device="cuda")
    big_l = torch.full((n_l + 2 * pad,), 12345.0, device="cuda")
    o_view = big_o[pad: pad + n_o].view(B, H, sq, d)
    l_view = big_l[pad: pad + n_l].view(B, H, sq)
    o_view.fill_(float("nan"))
    l_view.fill_(float("nan"))
    sma.attention_fwd(tq, tk, tv, scale=0.1, causal=True, return_lse=True, out=o_view, lse=l_view,
                      **kw)
    torch.cuda.synchronize()
    assert torch.all(big_o[:pad] == 12345.0) and torch.all(big_o[pad + n_o:] == 12345.0)
    assert torch.all(big_l[:pad] == 12345.0) and torch.all(big_l[pad + n_l:] == 12345.0)
    assert not torch.any(torch.isnan(o_view)) and not torch.any(torch.isnan(l_view))
    o_ref, lse_ref = oracle.attention_fwd(q, k, v, 0.1, True)
    check_parity(o_view.cpu().numpy().astype(np.float64), l_view.cpu().numpy().astype(np.float64),
                 o_ref, lse_ref, dtype, "guard")


@pytest.mark.parametrize("dtype", ["f32", "bf16", "f16"])
def test_non_default_stream(dtype):
    import torch

    import scaled_masked_attention_amd as sma

    (q, k, v), bits = _case(40, 2, 2, 300, 300, 64, dtype)
    s = torch.cuda.Stream()
    with torch.cuda.stream(s):
        tq, tk, tv = to_device((q, k, v), bits, dtype)
        o, lse = sma.attention_fwd(tq, tk, tv, scale=0.125, causal=True, return_lse=True)
        o2 = o * 2.0  # ordered after the attention kernel on the same stream
    s.synchronize()
    o_ref, lse_ref = oracle.attention_fwd(q, k, v, 0.125, True)
    check_parity(o.cpu().numpy().astype(np.float64), lse.cpu().numpy().astype(np.float64), o_ref,
                 lse_ref, dtype, "stream")
    assert torch.equal(o2, o * 2.0)


def _segment_stream(torch, ptr):
    """The stream the caching allocator holds the block at `ptr` for."""
    for seg in torch.cuda.memory_snapshot():
        if seg["address"] <= ptr < seg["address"] + seg["total_size"]:
            return seg["stream"]
    raise AssertionError("pointer not in any allocator segment")


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_stream_argument_allocates_on_the_launch_stream(dtype):
    """With stream= other than the current stream, the outputs and the workspace (a forced key
    split, and a mask's packed bits) are allocated on the launch stream, so the caching
    allocator cannot hand the freed workspace to work queued on the current stream while the
    kernels still use it. The side stream is held back by a sleep while the current stream
    allocates and fills blocks of the workspace's size."""
    import torch

    import scaled_masked_attention_amd as sma

    (q, k, v), bits = _case(41, 2, 2, 300, 1100, 64, dtype)
    tq, tk, tv = to_device((q, k, v), bits, dtype)
    mask_np = gen.bernoulli_mask(41, (1, 1, 300, 1100), 0.7)
    tmask = torch.from_numpy(mask_np).to("cuda")
    kern = sma.SMA_KERNEL_F32_QBLOCK if dtype == "f32" else sma.SMA_KERNEL_BF16_QBLOCK
    torch.cuda.synchronize()
    s = torch.cuda.Stream()
    results = []
    for mask in (None, tmask):
        with torch.cuda.stream(s):
            torch.cuda._sleep(20_000_000)
        o, lse = sma.attention_fwd(tq, tk, tv, scale=0.125, causal=True, return_lse=True, stream=s,
                                   kernel=kern, nsplit=3, mask=mask)
        junk = [torch.full((1 << 20,), float("nan"), device="cuda") for _ in range(8)]
        assert _segment_stream(torch, o.data_ptr()) == s.cuda_stream
        assert _segment_stream(torch, lse.data_ptr()) == s.cuda_stream
        results.append((o, lse, junk))
    torch.cuda.synchronize()
    o_ref, lse_ref = oracle.attention_fwd(q, k, v, 0.125, True)
    m_ref, mlse_ref = oracle.attention_fwd_masked(q, k, v, mask_np, 0.125, True)
    for (o, lse, _), (r, lr), lab in zip(results, ((o_ref, lse_ref), (m_ref, mlse_ref)),
                                         ("split", "masked split")):
        check_parity(o.cpu().numpy().astype(np.float64), lse.cpu().numpy().astype(np.float64), r,
                     lr, dtype, f"side stream {lab}")


@pytest.mark.parametrize("dtype", ["f32", "bf16", "f16"])
@pytest.mark.parametrize("causal", [False, True])
def test_split_keys_path_matches_unsplit(dtype, causal):
    """A shape the planner splits across workgroups: with and without workspace."""
    import torch

    import scaled_masked_attention_amd as sma

    B, H, sq, skv, d = 1, 4, 200, 3000, 128
    (q, k, v), bits = _case(41, B, H, sq, skv, d, dtype)
    in_dt = {"f32": sma.SMA_DTYPE_F32, "bf16": sma.SMA_DTYPE_BF16, "f16": sma.SMA_DTYPE_F16}[dtype]
    assert sma.workspace_bytes(in_dt, B, H, sq, skv, d, causal) > 0
    dev = to_device((q, k, v), bits, dtype)
    o_s, l_s = run_gpu(*dev, 0.1, causal)
    tiny = torch.empty(16, dtype=torch.uint8, device="cuda")
    o_n, l_n = run_gpu(*dev, 0.1, causal, workspace=tiny)  # too small: no split
    o_ref, lse_ref = oracle.attention_fwd(q, k, v, 0.1, causal)
    check_parity(o_s, l_s, o_ref, lse_ref, dtype, "split")
    check_parity(o_n, l_n, o_ref, lse_ref, dtype, "unsplit")


def test_binding_rejects_bad_arguments():
    import torch

    import scaled_masked_attention_amd as sma

    q = torch.randn(1, 1, 8, 96, device="cuda")
    with pytest.raises(sma.SMAError) as e:
        sma.attention_fwd(q, q, q)
    assert e.value.status == 3  # head_dim 96 unsupported
    q = torch.randn(1, 1, 8, 64, device="cuda")
    with pytest.raises(sma.SMAError) as e:
        sma.attention_fwd(q, q, q, out=q)  # output aliases the inputs
    assert e.value.status == 5
    with pytest.raises(ValueError):
        sma.attention_fwd(q, q.half(), q)


@pytest.mark.parametrize("variant", VARIANTS)
def test_hip_graph_replays_match_eager(variant):
    """The call captured in a HIP graph (through torch), replayed several times with eager work
    and synchronizations between replays: every replay equals the eager result bitwise."""
    import torch

    import scaled_masked_attention_amd as sma

    dtype, kw = variant_kwargs(variant)
    (q, k, v), bits = _case(44, 2, 3, 300, 450, 64, dtype)
    tq, tk, tv = to_device((q, k, v), bits, dtype)
    out = torch.empty((2, 3, 300, 64), dtype=torch.float32, device="cuda")
    lse = torch.empty((2, 3, 300), dtype=torch.float32, device="cuda")
    sma.attention_fwd(tq, tk, tv, scale=0.1, causal=True, return_lse=True, out=out, lse=lse, **kw)
    torch.cuda.synchronize()
    o_eager, l_eager = out.clone(), lse.clone()
    g = torch.cuda.CUDAGraph()
    s = torch.cuda.Stream()
    with torch.cuda.stream(s):
        with torch.cuda.graph(g, stream=s):
            sma.attention_fwd(tq, tk, tv, scale=0.1, causal=True, return_lse=True, out=out, lse=lse,
                              stream=torch.cuda.current_stream(), **kw)
    for rep in range(4):
        out.fill_(float("nan"))
        lse.fill_(float("nan"))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out, o_eager) and torch.equal(lse, l_eager), f"replay {rep} differs"
        _ = (tq.float() * 2).sum().item()  # eager work between replays
    o_ref, lse_ref = oracle.attention_fwd(q, k, v, 0.1, True)
    check_parity(o_eager.cpu().numpy().astype(np.float64), l_eager.cpu().numpy().astype(np.float64),
                 o_ref, lse_ref, dtype, "graph")
