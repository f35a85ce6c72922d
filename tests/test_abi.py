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
F32, BF16 = 0, 1


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
    assert sma.abi_version() == 1
    for st in range(7):
        assert sma.status_string(st).startswith(sma.STATUS_NAMES[st])
    assert sma.status_string(99) == "unknown sma status"


# fake, aligned, non-overlapping device addresses (never dereferenced by validate)
Q, K, V, O, L, W = 0x10_0000_0000, 0x20_0000_0000, 0x30_0000_0000, 0x40_0000_0000, 0x50_0000_0000, 0x60_0000_0000


def _v(q=Q, k=K, v=V, o=O, lse=L, idt=F32, odt=F32, B=1, H=2, sq=128, skv=128, d=64, scale=0.125,
       causal=1, ws=None, wsb=0):
    return sma.validate(q, k, v, o, lse, idt, odt, B, H, sq, skv, d, scale, causal, ws, wsb)


def test_valid_calls():
    assert _v() == OK
    assert _v(idt=BF16, d=128) == OK
    assert _v(lse=None) == OK
    assert _v(scale=-1.0) == OK and _v(scale=0.0) == OK


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
    assert _v(d=96) == UNSUP
    assert _v(d=256) == UNSUP
    assert _v(odt=BF16, idt=BF16, d=128) == UNSUP
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
    c4 = dict(in_dtype=F32, batch=2, heads=32, seq_q=256, seq_kv=4096, head_dim=128)
    n = sma.workspace_bytes(causal=False, num_cus=256, **c4)
    rows = 2 * 32 * 256
    assert n >= 2 * rows * (128 + 1) * 4  # at least two splits of O and LSE
    assert sma.workspace_bytes(F32, 8, 16, 2048, 2048, 128, True, 256) == 0  # enough query blocks
    assert sma.workspace_bytes(BF16, 1, 32, 16384, 16384, 128, True, 256) == 0
    assert sma.workspace_bytes(F32, 1, 1, 100, 100, 64, True, 256) == 0  # too few keys to split
    assert sma.workspace_bytes(F32, 1, 1, 100, 4096, 96, True, 256) == 0  # invalid -> 0


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
