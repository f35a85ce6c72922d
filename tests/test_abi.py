"""The C ABI on the CPU: the library loads, exports what include/sma.h declares,
and the host-only checks return the documented status for each bad argument.
No compute call is made here (there is no GPU)."""
import ctypes
import os
import re
import subprocess
import sys

import pytest

import scaled_masked_attention_amd as sma

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "sma.h")

OK, NULLP, INVAL, UNSUP, MISAL, ALIAS = 0, 1, 2, 3, 4, 5
F32, BF16, F16 = 0, 1, 2


def _declared_functions():
    text = open(HEADER).read()
    return sorted(set(re.findall(r"^\s*(?:const\s+)?\w+\s*\*?\s*(sma_\w+)\s*\(", text, re.M)))


def test_library_exports_every_declared_symbol():
    names = _declared_functions()
    assert {"sma_attention_fwd", "sma_attention_fwd_validate", "sma_attention_fwd_workspace_bytes",
            "sma_status_string", "sma_abi_version"} <= set(names)
    lib = ctypes.CDLL(sma.LIB_PATH)
    for n in names:
        assert hasattr(lib, n), f"{n} declared in sma.h but not exported"


def test_abi_version_and_status_strings():
    assert sma.abi_version() == 3
    for st in range(8):
        assert sma.status_string(st).startswith(sma.STATUS_NAMES[st])
    assert sma.status_string(99) == "unknown sma status"


# fake, aligned, non-overlapping device addresses (never dereferenced by validate)
Q, K, V, O, L, W = 0x10_0000_0000, 0x20_0000_0000, 0x30_0000_0000, 0x40_0000_0000, 0x50_0000_0000, 0x60_0000_0000


def _v(q=Q, k=K, v=V, o=O, lse=L, idt=F32, odt=F32, B=1, H=2, sq=128, skv=128, d=64, scale=0.125,
       causal=1, ws=None, wsb=0):
    return sma.validate(q, k, v, o, lse, idt, odt, B, H, sq, skv, d, scale, causal, ws, wsb)


def test_valid_calls():
    assert _v() == OK
    assert _v(odt=BF16) == OK and _v(odt=BF16, idt=BF16, d=128) == OK
    assert _v(idt=BF16, d=128) == OK
    assert _v(idt=F16, d=128) == OK and _v(idt=F16, odt=BF16, d=64) == OK
    assert _v(lse=None) == OK
    assert _v(scale=-1.0) == OK and _v(scale=0.0) == OK
    assert _v(d=32) == OK and _v(d=256) == OK and _v(d=256, odt=BF16) == OK  # fp32 inputs only


def test_null_pointers():
    assert _v(q=None) == NULLP
    assert _v(o=None) == NULLP
    assert _v(k=None) == NULLP
    assert _v(v=None) == NULLP
    assert _v(k=None, v=None, skv=0) == OK  # no keys: k and v are never read
    assert _v(q=None, o=None, k=None, v=None, sq=0) == OK  # nothing to do


def test_invalid_values():
    assert _v(d=0) == INVAL
    assert _v(idt=7) == INVAL
    assert _v(odt=-1) == INVAL
    assert _v(scale=float("nan")) == INVAL
    assert _v(scale=float("inf")) == INVAL
    assert _v(B=1 << 40, H=1 << 40) == INVAL  # size_t overflow


def test_unsupported():
    assert _v(d=96) == UNSUP and _v(d=16) == UNSUP and _v(d=512) == UNSUP
    for d in (32, 256):  # the 16-bit kernel is built for these head dims too
        assert _v(idt=BF16, d=d) == OK and _v(idt=F16, odt=BF16, d=d) == OK
    assert _v(odt=BF16, idt=BF16, d=96) == UNSUP
    assert _v(odt=F16) == OK and _v(odt=F16, idt=F16) == OK and _v(odt=F16, idt=BF16) == OK
    assert _v(idt=F16, d=128, skv=1 << 23) == UNSUP
    assert _v(sq=(1 << 30) + 1) == UNSUP
    assert _v(idt=BF16, d=128, skv=(1 << 23) - 256) == OK  # K/V of one head just under 2 GiB
    assert _v(idt=BF16, d=128, skv=1 << 23) == UNSUP
    assert _v(idt=F32, d=128, skv=1 << 23) == OK


def test_alignment():
    assert _v(q=Q + 4) == MISAL
    assert _v(k=K + 8) == MISAL
    assert _v(o=O + 2) == MISAL
    assert _v(lse=L + 2) == MISAL
    assert _v(lse=L + 4) == OK
    assert _v(ws=W + 8, wsb=4096) == MISAL


def test_aliasing():
    nq = 1 * 2 * 128 * 64 * 4
    assert _v(o=Q) == ALIAS
    assert _v(o=Q + nq) == OK  # adjacent, not overlapping
    assert _v(o=Q + nq - 16) == ALIAS
    assert _v(lse=O + 64) == ALIAS
    assert _v(lse=V) == ALIAS
    assert _v(ws=K, wsb=64) == ALIAS
    assert _v(ws=O + 16, wsb=64) == ALIAS
    assert _v(q=K) == OK  # inputs may share memory


def test_workspace_planner():
    small = dict(in_dtype=F32, batch=1, heads=4, seq_q=200, seq_kv=3000, head_dim=128)
    n = sma.workspace_bytes(causal=False, num_cus=256, **small)
    rows = 1 * 4 * 200
    assert n >= 2 * rows * (128 + 1) * 4  # at least two splits of O and LSE
    assert sma.workspace_bytes(F32, 2, 32, 256, 4096, 128, False, 256) == 0  # in-workgroup split
    assert sma.workspace_bytes(F32, 8, 16, 2048, 2048, 128, True, 256) == 0  # enough query blocks
    assert sma.workspace_bytes(BF16, 1, 32, 16384, 16384, 128, True, 256) == 0
    assert sma.workspace_bytes(F32, 1, 1, 100, 100, 64, True, 256) == 0  # too few keys to split
    assert sma.workspace_bytes(F32, 1, 1, 100, 4096, 96, True, 256) == 0  # invalid -> 0


def test_workspace_query_has_the_boundary_signature():
    """sma_attention_fwd_workspace_bytes takes exactly the shape arguments of the call (no CU
    count). Without a GPU here the planner assumes 256 CUs, so it equals the 256-CU plan."""
    lib = ctypes.CDLL(sma.LIB_PATH)
    f = lib.sma_attention_fwd_workspace_bytes
    sz = ctypes.c_size_t
    f.argtypes = [ctypes.c_int, sz, sz, sz, sz, sz, ctypes.c_int]
    f.restype = sz
    n = f(F32, 1, 4, 200, 3000, 128, 0)
    assert n > 0 and n == sma.plan(F32, 1, 4, 200, 3000, 128, False, num_cus=256).workspace_bytes
    assert f(F32, 1, 4, 200, 3000, 96, 0) == 0  # invalid head dim -> 0
    assert f(BF16, 1, 32, 16384, 16384, 128, 1) == 0


def test_plan_follows_the_layout():
    """Under [B,S,H,d] a head's rows are heads*head_dim apart, which moves the size limits:
    the plan and workspace queries take the layout, so they agree with the call."""
    # The 16-bit kernel reaches one head's K/V through 32-bit byte offsets: (seq_kv + 256)
    # rows of the row stride must stay below 2 GiB. 300000 keys at a stride of 32 heads x 128
    # dims (8 KiB per row in bf16) span 2.46e9 bytes under [B,S,H,d], 77 MB under [B,H,S,d].
    args = (BF16, 1, 32, 1024, 300000, 128, True)
    assert sma.plan(*args, num_cus=256).kernel == sma.SMA_KERNEL_BF16_QBLOCK
    with pytest.raises(sma.SMAError) as e:
        sma.plan(*args, num_cus=256, layout="bshd")
    assert e.value.status == UNSUP
    assert sma.workspace_bytes(*args, num_cus=256, layout="bshd") == 0
    # fp32: the in-workgroup key split needs its per-head span under 2 GiB; with the [B,S,H,d]
    # stride the automatic choice moves to the 128-row kernel, whose split needs a workspace
    a32 = (F32, 1, 64, 256, 140000, 64, False)
    p_bhsd = sma.plan(*a32, num_cus=256)
    p_bshd = sma.plan(*a32, num_cus=256, layout="bshd")
    assert p_bhsd.kernel == sma.SMA_KERNEL_F32_KSPLIT and p_bhsd.workspace_bytes == 0
    assert p_bshd.kernel == sma.SMA_KERNEL_F32_QBLOCK and p_bshd.nsplit > 1
    assert sma.workspace_bytes(*a32, num_cus=256, layout="bshd") == p_bshd.workspace_bytes > 0
    with pytest.raises(ValueError):
        sma.plan(*a32, layout="sbhd")


def test_product_path_fails_loudly_without_library(tmp_path):
    code = ("import scaled_masked_attention_amd as s; s.LIB_PATH = '/nonexistent/libsma.so'\n"
            "try:\n    s.library()\nexcept RuntimeError as e:\n    print('raised', e)\n")
    r = subprocess.run([sys.executable, "-c", code], cwd=ROOT, capture_output=True, text=True)
    assert "raised" in r.stdout and "missing" in r.stdout


def test_package_does_not_reference_the_oracle():
    pkg = os.path.join(ROOT, "scaled_masked_attention_amd")
    for dirpath, _, files in os.walk(pkg):
        for f in files:
            if f.endswith((".py", ".cpp", ".hip", ".h")):
                text = open(os.path.join(dirpath, f)).read()
                assert "oracle" not in text.lower(), f"{f} mentions the oracle"


def test_plan_auto_choices():
    P = sma.plan
    p = P(F32, 4, 8, 512, 512, 64, False, num_cus=256)  # 128-row blocks cannot fill 256 CUs
    assert (p.kernel, p.nsplit, p.workgroups, p.workspace_bytes) == (sma.SMA_KERNEL_F32_KSPLIT, 1, 512, 0)
    p = P(F32, 8, 16, 2048, 2048, 128, True, num_cus=256)  # 32-row blocks fill the GPU
    assert (p.kernel, p.nsplit, p.workgroups) == (sma.SMA_KERNEL_F32_KSPLIT, 1, 8 * 16 * 64)
    p = P(F32, 2, 32, 256, 4096, 128, False, num_cus=256)
    assert (p.kernel, p.nsplit, p.workgroups, p.workspace_bytes) == (sma.SMA_KERNEL_F32_KSPLIT, 1, 512, 0)
    p = P(F32, 1, 4, 200, 3000, 128, False, num_cus=256)  # few 32-row blocks, long rows
    assert p.kernel == sma.SMA_KERNEL_F32_QBLOCK and p.nsplit > 1
    assert p.workspace_bytes == sma.workspace_bytes(F32, 1, 4, 200, 3000, 128, False, 256)
    p = P(BF16, 1, 32, 16384, 16384, 128, True, num_cus=256)  # 512-row workgroups at d = 128
    assert (p.kernel, p.nsplit, p.workgroups) == (sma.SMA_KERNEL_BF16_QBLOCK, 1, 32 * 32)
    p = P(F16, 1, 32, 16384, 16384, 128, True, num_cus=256)
    assert (p.kernel, p.nsplit, p.workgroups) == (sma.SMA_KERNEL_BF16_QBLOCK, 1, 32 * 32)
    p = P(F32, 1, 1, 1, 4096, 64, False, num_cus=256)  # one query row, many keys
    assert p.kernel == sma.SMA_KERNEL_F32_QBLOCK and p.nsplit == 32
    # head dim 32 follows the 64/128 rule; 256 goes to the 128-row fp32 kernel, where one
    # workgroup fits a CU
    p = P(F32, 8, 16, 2048, 2048, 32, True, num_cus=256)
    assert (p.kernel, p.nsplit, p.workgroups) == (sma.SMA_KERNEL_F32_KSPLIT, 1, 8 * 16 * 64)
    p = P(F32, 1, 4, 256, 8192, 256, False, num_cus=256)  # 8 blocks: split to 32 per block
    assert (p.kernel, p.nsplit, p.workgroups) == (sma.SMA_KERNEL_F32_QBLOCK, 32, 8 * 32)
    assert p.workspace_bytes == sma.workspace_bytes(F32, 1, 4, 256, 8192, 256, False, 256)
    assert p.workspace_bytes >= 32 * 4 * 256 * 257 * 4
    p = P(F32, 1, 4, 256, 8192, 64, False, num_cus=256)  # two workgroups per CU at 64
    assert p.nsplit == 32 and P(F32, 1, 16, 256, 8192, 256, False, num_cus=256).nsplit == 8
    assert P(F32, 1, 16, 256, 8192, 64, False, num_cus=256).nsplit == 16


def test_plan_forced():
    P = sma.plan
    p = P(F32, 4, 8, 512, 512, 64, False, kernel=sma.SMA_KERNEL_F32_QBLOCK, nsplit=1, num_cus=256)
    assert (p.nsplit, p.workgroups, p.workspace_bytes) == (1, 4 * 8 * 4, 0)
    p = P(F32, 4, 8, 512, 512, 64, False, kernel=sma.SMA_KERNEL_F32_QBLOCK, nsplit=3, num_cus=256)
    rows = 4 * 8 * 512
    assert p.nsplit == 3 and p.workgroups == 3 * 4 * 8 * 4
    assert p.workspace_bytes >= 3 * rows * 65 * 4
    # a split is merged so that each keeps whole 32-key tiles: 100 keys -> at most 4 tiles
    p = P(F32, 1, 1, 10, 100, 64, False, kernel=sma.SMA_KERNEL_F32_QBLOCK, nsplit=32, num_cus=256)
    assert p.nsplit == 4
    p = P(F32, 1, 1, 10, 0, 64, False, kernel=sma.SMA_KERNEL_F32_QBLOCK, nsplit=8, num_cus=256)
    assert p.nsplit == 1 and p.workspace_bytes == 0
    p = P(F32, 3, 5, 100, 300, 128, True, kernel=sma.SMA_KERNEL_F32_KSPLIT, num_cus=256)
    assert (p.kernel, p.nsplit, p.workgroups) == (sma.SMA_KERNEL_F32_KSPLIT, 1, 15 * 4)


def test_plan_rejects():
    P = sma.plan
    with pytest.raises(sma.SMAError) as e:
        P(BF16, 1, 1, 8, 8, 64, False, kernel=sma.SMA_KERNEL_F32_QBLOCK)
    assert e.value.status == UNSUP
    with pytest.raises(sma.SMAError) as e:
        P(F32, 1, 1, 8, 8, 64, False, kernel=sma.SMA_KERNEL_BF16_QBLOCK)
    assert e.value.status == UNSUP
    with pytest.raises(sma.SMAError) as e:
        P(F32, 1, 1, 8, 8, 64, False, kernel=sma.SMA_KERNEL_F32_KSPLIT, nsplit=2)
    assert e.value.status == UNSUP
    for bad_kernel in (3, -2, 99):
        with pytest.raises(sma.SMAError) as e:
            P(F32, 1, 1, 8, 8, 64, False, kernel=bad_kernel)
        assert e.value.status == INVAL
    for bad_split in (-1, 33):
        with pytest.raises(sma.SMAError) as e:
            P(F32, 1, 1, 8, 8, 64, False, nsplit=bad_split)
        assert e.value.status == INVAL
    with pytest.raises(sma.SMAError) as e:
        P(F32, 1, 1, 8, 8, 96, False)
    assert e.value.status == UNSUP
    # every kernel is built for head dims 32 and 256, except ksplit for 256 (LDS)
    with pytest.raises(sma.SMAError) as e:
        P(F32, 1, 1, 8, 8, 256, False, kernel=sma.SMA_KERNEL_F32_KSPLIT)
    assert e.value.status == UNSUP
    assert P(F32, 1, 1, 8, 8, 32, False, kernel=sma.SMA_KERNEL_F32_KSPLIT).kernel == sma.SMA_KERNEL_F32_KSPLIT
    assert P(F32, 8, 16, 2048, 2048, 32, True, num_cus=256).kernel == sma.SMA_KERNEL_F32_KSPLIT
    assert P(F32, 8, 16, 2048, 2048, 256, True, num_cus=256).kernel == sma.SMA_KERNEL_F32_QBLOCK
    for d in (32, 256):
        assert P(F32, 1, 1, 8, 8, d, False, kernel=sma.SMA_KERNEL_F32_QBLOCK, nsplit=1).nsplit == 1
        assert P(BF16, 1, 1, 8, 8, d, False, kernel=sma.SMA_KERNEL_BF16_QBLOCK, nsplit=1).nsplit == 1
    # the 16-bit kernels' geometry: 256 rows and 64-key tiles at d = 32 and 64, 512 rows and
    # 32-key tiles at d = 128, 192 rows and 32-key tiles at d = 256
    K16 = sma.SMA_KERNEL_BF16_QBLOCK
    assert P(BF16, 1, 4, 1000, 1000, 32, True, kernel=K16, nsplit=1).workgroups == 4 * 4
    assert P(BF16, 1, 4, 1000, 1000, 64, True, kernel=K16, nsplit=1).workgroups == 4 * 4
    assert P(BF16, 1, 4, 1000, 1000, 128, True, kernel=K16, nsplit=1).workgroups == 4 * 2
    assert P(BF16, 1, 4, 1000, 1000, 256, True, kernel=K16, nsplit=1).workgroups == 4 * 6
    # a forced split at d = 128 rounds its key range to the 32-key tile
    p = P(BF16, 1, 1, 512, 1000, 128, False, kernel=K16, nsplit=3)
    assert p.nsplit == 3 and p.workgroups == 3
    p = P(F16, 1, 1, 128, 4096, 256, False, num_cus=256)  # one 128-row block: split in 32-key tiles
    assert p.nsplit == 32 and p.workspace_bytes >= 32 * 128 * 257 * 4
    lib = sma.library()
    assert lib.sma_attention_fwd_plan(F32, 1, 1, 8, 8, 64, 0, 0, -1, 0, 256, None) == NULLP
    assert lib.sma_attention_fwd_plan(F32, 1, 1, 8, 8, 64, 0, 2, -1, 0, 256, ctypes.byref(sma.Plan())) == INVAL


def _ex(plan, q=Q, o=O, idt=F32, ws=None, wsb=0, layout=0, H=2, skv=128):
    # Error paths only: every one returns before the library touches a device.
    return sma.library().sma_attention_fwd_ex(q, K, V, o, L, idt, F32, 1, H, 128, skv, 64, 0.125,
                                              1, layout, ws, wsb,
                                              ctypes.byref(plan) if plan else None, None, None, None)


def test_ex_rejects_bad_plans_before_launch():
    assert _ex(sma.Plan(kernel=sma.SMA_KERNEL_F32_QBLOCK, nsplit=0)) == INVAL
    assert _ex(sma.Plan(kernel=sma.SMA_KERNEL_F32_QBLOCK, nsplit=33)) == INVAL
    assert _ex(sma.Plan(kernel=7, nsplit=1)) == INVAL
    assert _ex(sma.Plan(kernel=sma.SMA_KERNEL_BF16_QBLOCK, nsplit=1)) == UNSUP
    assert _ex(sma.Plan(kernel=sma.SMA_KERNEL_F32_QBLOCK, nsplit=1), idt=BF16) == UNSUP
    assert _ex(sma.Plan(kernel=sma.SMA_KERNEL_F32_KSPLIT, nsplit=2)) == UNSUP
    assert _ex(sma.Plan(kernel=sma.SMA_KERNEL_F32_KSPLIT, nsplit=1), q=None) == NULLP
    assert _ex(None, o=Q) == ALIAS


def test_plan_ksplit_offset_limit():
    # (seq + 32) rows of d floats per head must stay within 2 GiB for the ksplit kernel
    ok = (1 << 31) // (4 * 128) - 32
    p = sma.plan(F32, 1, 1, 64, ok, 128, False, kernel=sma.SMA_KERNEL_F32_KSPLIT, num_cus=256)
    assert p.kernel == sma.SMA_KERNEL_F32_KSPLIT
    with pytest.raises(sma.SMAError) as e:
        sma.plan(F32, 1, 1, 64, ok + 1, 128, False, kernel=sma.SMA_KERNEL_F32_KSPLIT, num_cus=256)
    assert e.value.status == UNSUP
    with pytest.raises(sma.SMAError) as e:
        sma.plan(F32, 1, 1, ok + 1, 64, 128, False, kernel=sma.SMA_KERNEL_F32_KSPLIT, num_cus=256)
    assert e.value.status == UNSUP


def test_row_ops_host_checks():
    """Argument errors of the row primitives return before any HIP call."""
    lib = sma.library()
    X, Y, M = 0x10_0000_0000, 0x20_0000_0000, 0x30_0000_0000
    assert lib.sma_softmax_rows(None, None, 0, 5, None) == OK          # nothing to do
    assert lib.sma_softmax_rows(None, Y, 3, 5, None) == NULLP
    assert lib.sma_softmax_rows(X, None, 3, 5, None) == NULLP
    assert lib.sma_logsumexp_rows(X, None, 3, 0, None) == NULLP         # writes -inf per row
    assert lib.sma_softmax_rows(X + 2, Y, 3, 5, None) == MISAL
    assert lib.sma_softmax_rows(X, X + 4, 3, 5, None) == ALIAS          # partial overlap
    assert lib.sma_logsumexp_rows(X, X + 8, 3, 5, None) == ALIAS
    assert lib.sma_masked_softmax_rows(X, M, M, 3, 5, None) == ALIAS     # out over the mask
    assert lib.sma_masked_softmax_rows(X, None, Y, 3, 5, None) == NULLP
    assert lib.sma_scaled_causal_softmax(X, Y, 2, 3, 5, float("nan"), 1, None) == INVAL
    assert lib.sma_scaled_causal_softmax(X, Y, 1 << 40, 1 << 40, 5, 1.0, 1, None) == INVAL
    assert lib.sma_softmax_rows(X, Y, 1 << 40, 1 << 40, None) == INVAL
    assert lib.sma_softmax_rows(X, Y, 1, 1 << 31, None) == UNSUP
    assert lib.sma_softmax_rows(X, Y, 1 << 31, 1, None) == UNSUP


def test_softmax_backward_host_checks():
    """sma_softmax_rows_backward's argument errors return before any HIP call."""
    lib = sma.library()
    Y, G, D = 0x10_0000_0000, 0x20_0000_0000, 0x30_0000_0000
    f = lib.sma_softmax_rows_backward
    assert f(None, None, None, 0, 5, 1.0, None) == OK                   # nothing to do
    assert f(None, None, None, 4, 0, 1.0, None) == OK
    assert f(Y, G, None, 3, 5, 1.0, None) == NULLP
    assert f(None, G, D, 3, 5, 1.0, None) == NULLP
    assert f(Y, None, D, 3, 5, 1.0, None) == NULLP
    assert f(Y + 2, G, D, 3, 5, 1.0, None) == MISAL
    assert f(Y, G, D + 2, 3, 5, 1.0, None) == MISAL
    assert f(Y, G, Y + 4, 3, 5, 1.0, None) == ALIAS                    # partial overlap with y
    assert f(Y, G, G + 8, 3, 5, 1.0, None) == ALIAS                    # partial overlap with dy
    assert f(Y, G, D, 3, 5, float("nan"), None) == INVAL
    assert f(Y, G, D, 3, 5, float("inf"), None) == INVAL
    assert f(Y, G, D, 1 << 40, 1 << 40, 1.0, None) == INVAL
    assert f(Y, G, D, 1, 1 << 31, 1.0, None) == UNSUP
    assert f(Y, G, D, 1 << 31, 1, 1.0, None) == UNSUP


def test_backward_workspace_and_host_checks():
    """sma_attention_bwd's argument errors return before any HIP call."""
    lib = sma.library()
    assert sma.attention_bwd_workspace_bytes(F32, 2, 3, 100, 50, 64, True) == 2 * 3 * 4 * 256
    assert sma.attention_bwd_workspace_bytes(F32, 1, 1, 0, 50, 64, False) == 0
    assert sma.attention_bwd_workspace_bytes(F32, 1, 1, 33, 50, 96, False) == 0   # head_dim
    assert sma.attention_bwd_workspace_bytes(7, 1, 1, 33, 50, 64, False) == 0     # dtype
    # bf16 Q, K, V: the per-block lse2/D, then dO rounded to bf16 (256-byte aligned)
    assert sma.attention_bwd_workspace_bytes(BF16, 2, 3, 100, 50, 64, True) == 2 * 3 * 4 * 256 + 76800
    assert sma.attention_bwd_workspace_bytes(BF16, 1, 1, 33, 50, 64, False) == 2 * 256 + 4352
    # fp16 Q, K, V take the same layout, with dO rounded to fp16
    assert sma.attention_bwd_workspace_bytes(F16, 2, 3, 100, 50, 64, True) == 2 * 3 * 4 * 256 + 76800
    base = [0x10_0000_0000 * i for i in range(1, 11)]
    q, k, v, o, lse, g, dq, dk, dv, ws = base

    def call(q=q, k=k, v=v, o=o, lse=lse, g=g, dq=dq, dk=dk, dv=dv, idt=F32, B=1, H=2, sq=100,
             skv=70, d=64, scale=0.125, causal=1, ws=ws, wsb=1 << 20):
        return lib.sma_attention_bwd(q, k, v, o, lse, g, dq, dk, dv, idt, B, H, sq, skv, d, scale,
                                     causal, ws, wsb, None)

    assert call(B=0) == OK and call(sq=0, skv=0) == OK                       # nothing to do
    assert call(q=None, o=None, lse=None, g=None, dq=None, sq=0, skv=0, ws=None, wsb=0) == OK
    for name in ("q", "o", "lse", "g", "dq", "k", "v", "dk", "dv"):
        assert call(**{name: None}) == NULLP, name
    assert call(ws=None) == INVAL and call(wsb=8 * 256 - 1) == INVAL        # 2 heads x 4 blocks
    assert call(d=0) == INVAL and call(scale=float("inf")) == INVAL
    assert call(B=1 << 40, H=1 << 40) == INVAL
    assert call(d=96) == UNSUP and call(idt=7) == INVAL
    # 16-bit inputs take a larger workspace (the 16-bit copy of dO): the fp32 size is too small
    assert call(idt=BF16, wsb=8 * 256) == INVAL and call(idt=BF16, d=96) == UNSUP
    assert call(idt=F16, wsb=8 * 256) == INVAL and call(idt=F16, d=96) == UNSUP
    assert call(d=256) == UNSUP                                 # fp32: not built for head dim 256
    assert sma.attention_bwd_workspace_bytes(F32, 1, 1, 33, 50, 256, False) == 0
    assert sma.attention_bwd_workspace_bytes(BF16, 1, 1, 33, 50, 256, False) == 2 * 256 + 33 * 256 * 2  # 16-bit: built
    assert sma.attention_bwd_workspace_bytes(F16, 1, 1, 33, 50, 256, False) > 0
    assert sma.attention_bwd_workspace_bytes(F32, 1, 1, 33, 50, 32, False) == 2 * 256  # head dim 32
    assert call(sq=(1 << 23), d=64) == UNSUP                                 # 32-bit tile offsets
    assert call(q=q + 8) == MISAL and call(dk=dk + 4) == MISAL and call(lse=lse + 2) == MISAL
    assert call(ws=ws + 8) == MISAL
    assert call(dq=q) == ALIAS and call(dv=dk + 16) == ALIAS and call(ws=lse) == ALIAS
    assert call(dk=o + 64) == ALIAS and call(ws=dq + 256) == ALIAS


def test_backward_layout_host_checks():
    """sma_attention_bwd_layout: the layout code and the [B,S,H,d] 32-bit offset limit are
    checked before any HIP call."""
    lib = sma.library()
    base = [0x10_0000_0000 * i for i in range(1, 11)]
    q, k, v, o, lse, g, dq, dk, dv, ws = base

    def call(layout, H=2, sq=100, skv=70, d=64, idt=F32, wsb=1 << 30, dq=dq):
        return lib.sma_attention_bwd_layout(q, k, v, o, lse, g, dq, dk, dv, idt, 1, H, sq, skv, d,
                                            0.125, 1, layout, ws, wsb, None)

    assert call(7) == INVAL and call(-1) == INVAL
    # one head's rows are heads*d elements apart under [B,S,H,d]: 64 heads x 128 dims x 2^17
    # rows pass under [B,H,S,d] and exceed 2 GiB of offsets under [B,S,H,d]
    big = dict(H=64, sq=1 << 17, skv=64, d=128)
    assert call(sma.SMA_LAYOUT_BSHD, **big) == UNSUP
    assert call(sma.SMA_LAYOUT_BSHD, idt=F16, wsb=8 * 256) == INVAL and call(sma.SMA_LAYOUT_BSHD, d=96) == UNSUP
    assert call(sma.SMA_LAYOUT_BSHD, wsb=16) == INVAL  # workspace too small
    assert call(sma.SMA_LAYOUT_BSHD, dq=q) == ALIAS


def test_layout_argument_and_its_limits():
    """Layout codes other than BHSD/BSHD are invalid; under BSHD the 2 GiB offset limits apply to
    rows heads*head_dim apart, so the in-workgroup key-split kernel stops fitting at 1/heads
    the sequence length."""
    ks = sma.Plan(kernel=sma.SMA_KERNEL_F32_KSPLIT, nsplit=1)
    assert _ex(ks, layout=2) == INVAL and _ex(ks, layout=-1) == INVAL
    assert _ex(ks, layout=1, q=None) == NULLP  # valid layout: the next check fails
    # 64 heads x d 64 x 4 B = 16 KiB per row: (skv + 32) rows stay below 2 GiB up to skv = 131040
    assert _ex(ks, layout=1, H=64, skv=131041) == UNSUP
    lib = sma.library()
    b = [0x10_0000_0000 * i for i in range(1, 6)]
    assert lib.sma_attention_fwd_layout(b[0], b[1], b[2], b[3], b[4], F32, F32, 1, 2, 8, 8, 64, 0.1, 0,
                                        5, None, 0, None) == INVAL
    assert lib.sma_attention_fwd_layout(None, b[1], b[2], b[3], b[4], F32, F32, 1, 2, 8, 8, 64, 0.1, 0,
                                        1, None, 0, None) == NULLP


def test_masked_entry_point_host_checks():
    """Argument errors of sma_attention_fwd_masked return before any HIP call."""
    lib = sma.library()
    M, WS = 0x70_0000_0000, 0x60_0000_0000
    need = lib.sma_attention_fwd_masked_workspace_bytes(F32, 1, 2, 128, 100, 64, 1, 0, 1, 2)
    split = sma.workspace_bytes(F32, 1, 2, 128, 100, 64, 1)
    assert need == 2 * 128 * 4 * 4 + split  # 2 head slabs x 128 rows x ceil(100/32) words x 4 B
    assert lib.sma_attention_fwd_masked_workspace_bytes(F32, 1, 2, 128, 100, 64, 1, 0, 3, 1) == 0

    def call(mask=M, mb=1, mh=2, idt=F32, ws=WS, wsb=1 << 20, plan=None, o=O, skv=100, causal=1):
        return lib.sma_attention_fwd_masked(Q, K, V, o, L, mask, mb, mh, idt, F32, 1, 2, 128, skv, 64,
                                            0.125, causal, 0, ws, wsb,
                                            ctypes.byref(plan) if plan else None, None, None, None)

    assert call(mb=2) == INVAL and call(mh=3) == INVAL and call(mb=0, mh=0) == INVAL
    assert call(mask=None) == NULLP
    assert call(o=M - 64) == ALIAS                     # o runs into the mask bytes
    assert call(ws=M + 128, wsb=4096) == ALIAS         # workspace on top of the mask
    assert call(ws=None, wsb=0) == INVAL and call(wsb=2 * 128 * 4 * 4 - 1) == INVAL
    assert call(idt=BF16, plan=sma.Plan(kernel=sma.SMA_KERNEL_F32_QBLOCK, nsplit=1)) == UNSUP


def test_backward_masked_host_checks():
    """sma_attention_bwd_masked: mask broadcast sizes, a missing mask, aliasing with an
    output and a workspace without room for the packed mask fail before any HIP call."""
    lib = sma.library()
    base = [0x10_0000_0000 * i for i in range(1, 12)]
    q, k, v, o, lse, g, dq, dk, dv, ws, m = base
    plain = sma.attention_bwd_workspace_bytes(F32, 2, 3, 100, 70, 64, True)
    # 3 heads x 100 rows x 3 words (70 keys) x 4 bytes = 3600 -> 3840 after rounding to 256
    assert lib.sma_attention_bwd_masked_workspace_bytes(F32, 2, 3, 100, 70, 64, 1, 0, 1, 3) == plain + 3840
    assert lib.sma_attention_bwd_masked_workspace_bytes(F32, 2, 3, 100, 70, 64, 1, 0, 2, 2) == 0

    def call(mb=1, mh=3, mask=m, dq=dq, wsb=1 << 30):
        return lib.sma_attention_bwd_masked(q, k, v, o, lse, g, dq, dk, dv, mask, mb, mh, F32, 2, 3, 100,
                                            70, 64, 0.125, 1, 0, ws, wsb, None)

    assert call(mb=3) == INVAL and call(mh=2) == INVAL
    assert call(mask=None) == NULLP
    assert call(dq=m - 4096) == ALIAS  # dq (100 rows of 64 floats per head) runs into the mask
    assert call(wsb=plain) == INVAL     # no room for the packed mask

