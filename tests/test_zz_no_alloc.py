"""sma_attention_fwd_noalloc through the C ABI (the forward for callers that cannot
allocate: its key-split partials go to the library's per-GPU device scratch).

Each case runs two calls in a row, the second on a smaller input, and compares
every output with sma_attention_fwd_ex given a torch workspace and the same
plan (the same kernels, so bitwise equal) and with the oracle at the parity
bars. A plan whose split does not fit the scratch is refused before launch."""
import gc
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

    sma.library()  # fail loudly if the HIP library is missing


def _run(noalloc, vals, bits, dtype, causal, kernel, nsplit, layout="bhsd"):
    """O and LSE (float64 numpy, [B,H,S,d] order) of one call: the no-allocation entry point, or
    sma_attention_fwd_ex with a workspace of the plan's size."""
    import torch

    import scaled_masked_attention_amd as sma

    tq, tk, tv = to_device(vals, bits, dtype)
    B, H, sq, d = tq.shape
    skv = tk.shape[2]
    if layout == "bshd":
        tq, tk, tv = (t.transpose(1, 2).contiguous() for t in (tq, tk, tv))
    in_dt = {"f32": sma.SMA_DTYPE_F32, "bf16": sma.SMA_DTYPE_BF16, "f16": sma.SMA_DTYPE_F16}[dtype]
    scale = 1.0 / math.sqrt(d)
    o = torch.full(tq.shape, float("nan"), dtype=torch.float32, device="cuda")
    lse = torch.full((B, H, sq), float("nan"), dtype=torch.float32, device="cuda")
    lay = sma.LAYOUTS[layout]
    pl = None
    if kernel is not None:
        pl = sma.plan(in_dt, B, H, sq, skv, d, causal, kernel, nsplit, layout=layout)
    s = torch.cuda.current_stream().cuda_stream
    torch.cuda.synchronize()
    if noalloc:
        # Python's collector could free an unrelated tensor left by an earlier test in the
        # middle of the call, which would read as a change: collect first, then hold it off.
        gc.collect()
        gc.disable()
        try:
            before = torch.cuda.memory_allocated()
            sma.attention_fwd_noalloc_raw(tq.data_ptr(), tk.data_ptr(), tv.data_ptr(), o.data_ptr(),
                                          lse.data_ptr(), in_dt, sma.SMA_DTYPE_F32, B, H, sq, skv, d,
                                          scale, causal, pl, s, layout=lay)
            assert torch.cuda.memory_allocated() == before
        finally:
            gc.enable()
    else:
        need = pl.workspace_bytes if pl is not None else sma.workspace_bytes(
            in_dt, B, H, sq, skv, d, causal, layout=layout)
        ws = torch.empty(max(need, 1), dtype=torch.uint8, device="cuda")
        sma.attention_fwd_ex_raw(tq.data_ptr(), tk.data_ptr(), tv.data_ptr(), o.data_ptr(),
                                 lse.data_ptr(), in_dt, sma.SMA_DTYPE_F32, B, H, sq, skv, d, scale,
                                 causal, ws.data_ptr(), need, pl, s, layout=lay)
    torch.cuda.synchronize()
    if layout == "bshd":
        o = o.transpose(1, 2)
    return o.cpu().numpy().astype(np.float64), lse.cpu().numpy().astype(np.float64), scale


def _kernel(name):
    import scaled_masked_attention_amd as sma

    return {None: None, "f32_qblock": sma.SMA_KERNEL_F32_QBLOCK,
            "bf16_qblock": sma.SMA_KERNEL_BF16_QBLOCK}[name]


# (dtype, causal, kernel, nsplit, layout, (B, H, Sq, Skv, d) of the first call, then the second)
CASES = [
    ("f32", True, "f32_qblock", 3, "bhsd", (2, 3, 300, 1500, 128), (1, 2, 70, 400, 64)),
    ("f32", False, None, 0, "bhsd", (1, 4, 200, 3000, 128), (1, 1, 50, 1000, 64)),
    ("bf16", True, "bf16_qblock", 4, "bhsd", (1, 3, 520, 2000, 128), (1, 1, 90, 700, 128)),
    ("f16", False, "bf16_qblock", 2, "bshd", (2, 2, 300, 900, 64), (1, 2, 33, 300, 64)),
    ("bf16", True, None, 0, "bhsd", (1, 2, 256, 8192, 128), (1, 1, 1, 2000, 128)),
]


@pytest.mark.parametrize("case", CASES, ids=lambda c: f"{c[0]}-{c[2] or 'auto'}-{c[3]}-{c[4]}")
def test_noalloc_matches_workspace_entry_point(case):
    import scaled_masked_attention_amd as sma

    dtype, causal, kname, nsplit, layout, first, second = case
    kernel = _kernel(kname)
    for seed, (B, H, sq, skv, d) in ((11, first), (12, second)):
        print(f"[noalloc] {dtype} causal={causal} {kname} nsplit={nsplit} {layout} "
              f"B={B} H={H} Sq={sq} Skv={skv} d={d}", flush=True)
        (q, k, v), bits = gen.random_case(seed, (B, H, sq, d), (B, H, skv, d),
                                          sigma_qk=1.0 if dtype == "f32" else 3.0, dtype=dtype)
        if kernel is not None or nsplit == 0:
            in_dt = {"f32": 0, "bf16": 1, "f16": 2}[dtype]
            pl = sma.plan(in_dt, B, H, sq, skv, d, causal, kernel if kernel is not None else -1,
                          nsplit, layout=layout)
            if seed == 11:
                assert pl.nsplit > 1, "the first call must exercise the scratch"
        o_n, l_n, scale = _run(True, (q, k, v), bits, dtype, causal, kernel, nsplit, layout)
        o_w, l_w, _ = _run(False, (q, k, v), bits, dtype, causal, kernel, nsplit, layout)
        assert np.array_equal(o_n, o_w) and np.array_equal(l_n, l_w), \
            "no-allocation result differs from the workspace entry point's"
        o_ref, lse_ref = oracle.attention_fwd(q, k, v, scale, causal)
        check_parity(o_n, l_n, o_ref, lse_ref, dtype, f"noalloc {case} seed {seed}")


def test_noalloc_refuses_a_split_beyond_the_scratch():
    """An explicit split whose partials exceed SMA_NOALLOC_SCRATCH_BYTES is SMA_ERR_SCRATCH,
    returned before anything is launched (the buffers are real, so nothing could fault)."""
    import torch

    import scaled_masked_attention_amd as sma

    B, H, sq, skv, d = 1, 32, 1024, 4096, 128
    pl = sma.plan(sma.SMA_DTYPE_F32, B, H, sq, skv, d, False, sma.SMA_KERNEL_F32_QBLOCK, 8)
    assert pl.workspace_bytes > sma.NOALLOC_SCRATCH_BYTES
    q = torch.zeros((B, H, sq, d), device="cuda")
    k = torch.zeros((B, H, skv, d), device="cuda")
    o = torch.full((B, H, sq, d), 7.0, device="cuda")
    s = torch.cuda.current_stream().cuda_stream
    with pytest.raises(sma.SMAError) as e:
        sma.attention_fwd_noalloc_raw(q.data_ptr(), k.data_ptr(), k.data_ptr(), o.data_ptr(), None,
                                      sma.SMA_DTYPE_F32, sma.SMA_DTYPE_F32, B, H, sq, skv, d, 0.1,
                                      False, pl, s)
    assert e.value.status == sma.SMA_ERR_SCRATCH
    torch.cuda.synchronize()
    assert torch.all(o == 7.0)  # nothing ran
    # the same call with the library's plan runs
    sma.attention_fwd_noalloc_raw(q.data_ptr(), k.data_ptr(), k.data_ptr(), o.data_ptr(), None,
                                  sma.SMA_DTYPE_F32, sma.SMA_DTYPE_F32, B, H, sq, skv, d, 0.1,
                                  False, None, s)
    torch.cuda.synchronize()
    assert torch.all(o == 0.0)
