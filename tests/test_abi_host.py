"""The C ABI on the host: the library loads, exports what the header
declares, and every argument error is reported before any device work
(CPU only; only the host-only validation entry points are called)."""

import ctypes
import os
import re

import pytest

from fp8_w8a8_block_amd import _lib

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "fp8w8a8.h")

OK, NULL, SHAPE, STRIDE, ALIGN, BLOCK, SCHEME, WORKSPACE = 0, 1, 2, 3, 4, 5, 6, 7
ALIAS = 10

# fake, well-aligned, non-overlapping addresses: validation never dereferences
X = 0x10_0000_0000
Q = 0x20_0000_0000
S = 0x30_0000_0000
WS = 0x40_0000_0000
O = 0x50_0000_0000


def header_functions():
    text = open(HEADER).read()
    return sorted(set(re.findall(r"\b(fp8_[a-z0-9_]+)\s*\(", text)))


def test_exports_every_declared_symbol():
    lib = _lib.lib()
    names = header_functions()
    assert len(names) == 12, names
    for n in names:
        assert hasattr(lib, n), n


def test_status_strings():
    for code in range(0, 11):
        s = _lib.status_str(code)
        assert s and s != "unknown status"
    assert _lib.status_str(99) == "unknown status"


def test_workspace_bytes():
    assert _lib.workspace_bytes(_lib.OP_QUANT_ACT, 16, 0, 4096, "block") == 0
    assert _lib.workspace_bytes(_lib.OP_QUANT_ACT, 16, 0, 4096, "tensor") == 4096
    assert _lib.workspace_bytes(_lib.OP_QUANT_WEIGHT, 4096, 0, 4096, "tensor") == 4096
    assert _lib.workspace_bytes(_lib.OP_GEMM, 16, 256, 4096, "tensor") == 0
    # fused decode linear needs none; other shapes hold codes + scales
    assert _lib.workspace_bytes(_lib.OP_LINEAR, 4, 11008, 4096, "block") == 0
    assert _lib.workspace_bytes(_lib.OP_LINEAR, 16, 11008, 4096, "block") >= 16 * 4096
    assert _lib.workspace_bytes(_lib.OP_LINEAR, 1, 256, 512, "block") == 0
    n = _lib.workspace_bytes(_lib.OP_LINEAR, 100, 256, 512, "block")
    assert n >= 100 * 512 + 4 * 100 * 4
    assert _lib.workspace_bytes(_lib.OP_LINEAR, 4, 256, 512, "tensor") >= 4 * 512 + 4 + 4096


def vq(x=X, M=16, K=512, ld_x=None, q=Q, ld_q=None, s=S, ld_s=None, mode=0, ws=None, ws_bytes=0):
    ld_x = K if ld_x is None else ld_x
    ld_q = K if ld_q is None else ld_q
    ld_s = K // 128 if ld_s is None else ld_s
    return _lib.lib().fp8_validate_quant_act(x, M, K, ld_x, q, ld_q, s, ld_s, mode, ws, ws_bytes)


def test_validate_quant_act():
    assert vq() == OK
    assert vq(M=0, x=None, q=None, s=None) == OK          # empty call
    assert vq(M=-1) == SHAPE
    assert vq(K=0) == SHAPE
    assert vq(K=100) == SHAPE
    assert vq(K=200) == SHAPE
    assert vq(x=None) == NULL
    assert vq(q=None) == NULL
    assert vq(s=None) == NULL
    assert vq(ld_x=256) == STRIDE
    assert vq(ld_q=256) == STRIDE
    assert vq(ld_s=3) == STRIDE
    assert vq(x=X + 2) == ALIGN
    assert vq(q=Q + 8) == ALIGN
    assert vq(s=S + 2) == ALIGN
    assert vq(ld_x=520) == OK
    assert vq(ld_x=516) == ALIGN
    assert vq(ld_q=520) == ALIGN
    assert vq(q=X + 1024) == ALIAS                        # codes inside x
    assert vq(s=Q + 64) == ALIAS
    assert vq(mode=7) == SCHEME
    # dynamic per-tensor needs its workspace
    assert vq(mode=1) == WORKSPACE
    assert vq(mode=1, ws=WS, ws_bytes=100) == WORKSPACE
    assert vq(mode=1, ws=WS, ws_bytes=4096) == OK
    assert vq(mode=1, ws=X, ws_bytes=4096) == ALIAS


def vw(w=X, N=256, K=512, q=Q, s=S, bn=128, bk=128, mode=0, ld_s=None, ws=None, ws_bytes=0):
    ld_s = K // 128 if ld_s is None else ld_s
    return _lib.lib().fp8_validate_quant_weight_block(w, N, K, K, q, K, s, ld_s, bn, bk, mode,
                                                      ws, ws_bytes)


def test_validate_quant_weight_block():
    assert vw() == OK
    # the block size must be two-dimensional 128 x 128
    assert vw(bn=0) == BLOCK
    assert vw(bk=64) == BLOCK
    assert vw(bn=128, bk=256) == BLOCK
    assert vw(N=200) == SHAPE
    assert vw(N=0) == OK
    assert vw(ld_s=1) == STRIDE
    assert vw(mode=1, ws=WS, ws_bytes=4096, bn=0, bk=0) == OK   # block dims unused
    assert vw(mode=1) == WORKSPACE


def vg(a=X, ld_a=None, sa=S, ld_as=None, w=Q, ld_w=None, sw=WS, ld_ws=None, out=O, ld_out=None,
       M=16, N=256, K=512, mode=0):
    ld_a = K if ld_a is None else ld_a
    ld_w = K if ld_w is None else ld_w
    ld_as = K // 128 if ld_as is None else ld_as
    ld_ws = K // 128 if ld_ws is None else ld_ws
    ld_out = N if ld_out is None else ld_out
    return _lib.lib().fp8_validate_block_gemm(a, ld_a, sa, ld_as, w, ld_w, sw, ld_ws, out, ld_out,
                                              M, N, K, mode)


def test_validate_block_gemm():
    assert vg() == OK
    assert vg(mode=1) == OK
    assert vg(M=0, a=None) == OK
    assert vg(M=1) == OK and vg(M=3) == OK                 # any M >= 1
    assert vg(N=100) == SHAPE
    assert vg(K=64) == SHAPE
    assert vg(N=0) == SHAPE
    assert vg(mode=7) == SCHEME
    assert vg(out=None) == NULL
    assert vg(sa=None) == NULL
    assert vg(ld_out=128) == STRIDE
    assert vg(ld_as=1) == STRIDE
    assert vg(ld_as=1, mode=1) == OK                       # per-tensor scales have no ld
    assert vg(out=O + 4) == ALIGN
    assert vg(ld_out=260) == ALIGN
    assert vg(out=X + 16) == ALIAS


def test_validate_row_mode():
    # per token / per channel: one scale per row at stride ld_s >= 1
    assert vq(mode=2, ld_s=1) == OK
    assert vq(mode=2, ld_s=3) == OK
    assert vq(mode=2, ld_s=0) == STRIDE
    assert vq(mode=2, ld_s=1, s=Q + 64) == ALIAS
    assert vw(mode=2, ld_s=1, bn=0, bk=0) == OK                 # block dims unused
    assert vw(mode=2, ld_s=0) == STRIDE
    # GEMM: per-row vectors, stride 0 = one value for all rows / columns
    assert vg(mode=2, ld_as=1, ld_ws=1) == OK
    assert vg(mode=2, ld_as=0, ld_ws=1) == OK
    assert vg(mode=2, ld_as=0, ld_ws=0) == OK
    assert vg(mode=2, ld_as=-1, ld_ws=1) == STRIDE
    assert vg(mode=2, ld_as=1, ld_ws=-2) == STRIDE
    assert vg(mode=2, ld_as=1, ld_ws=1, out=S + 16) == ALIAS     # out over the token scales
    assert _lib.workspace_bytes(_lib.OP_QUANT_ACT, 16, 0, 4096, "row") == 0
    assert _lib.workspace_bytes(_lib.OP_LINEAR, 16, 11008, 4096, "row") >= 16 * 4096 + 16 * 4


def vs(x=X, M=16, K=512, ld_x=None, q=Q, ld_q=None, s=S):
    ld_x = K if ld_x is None else ld_x
    ld_q = K if ld_q is None else ld_q
    return _lib.lib().fp8_validate_quant_act_static(x, M, K, ld_x, q, ld_q, s)


def test_validate_quant_act_static():
    assert vs() == OK
    assert vs(M=0, x=None, q=None, s=None) == OK
    assert vs(K=100) == SHAPE
    assert vs(s=None) == NULL
    assert vs(x=None) == NULL
    assert vs(ld_q=256) == STRIDE
    assert vs(s=S + 2) == ALIGN
    assert vs(q=X + 64) == ALIAS
    assert vs(s=Q + 16) == ALIAS                                # scale inside the codes


def test_binding_rejects_host_tensors():
    torch = pytest.importorskip("torch")
    x = torch.zeros((16, 512), dtype=torch.bfloat16)
    with pytest.raises(ValueError):
        _lib.quant_act(x)
