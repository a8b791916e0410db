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
    assert len(names) == 19, names
    for n in names:
        assert hasattr(lib, n), n


def header_signatures():
    """name -> (return type, [parameter types]) of every declaration in the
    header, with parameter names and const dropped."""
    text = re.sub(r"/\*.*?\*/|//[^\n]*", "", open(HEADER).read(), flags=re.S)
    sigs = {}
    for ret, name, params in re.findall(
            r"^\s*((?:const\s+)?[A-Za-z_][A-Za-z0-9_]*\s*\**)\s*(fp8_[a-z0-9_]+)\s*\(([^)]*)\)\s*;",
            text, flags=re.M):
        types = []
        for prm in params.split(","):
            prm = " ".join(prm.replace("const", " ").split())
            m = re.fullmatch(r"([A-Za-z_][A-Za-z0-9_]*)\s*(\**)\s*[A-Za-z_][A-Za-z0-9_]*", prm)
            assert m, (name, prm)
            types.append(m.group(1) + m.group(2))
        sigs[name] = (" ".join(ret.replace("const", " ").split()).replace(" *", "*"), types)
    return sigs


def test_binding_argument_types_match_the_header():
    # every ctypes signature the binding sets is the header's, parameter for
    # parameter: pointers as c_void_p, int64_t as c_int64, int and the status
    # enum as c_int, size_t as c_size_t
    c_of = {"int64_t": ctypes.c_int64, "int": ctypes.c_int, "size_t": ctypes.c_size_t,
            "fp8_status": ctypes.c_int}
    sigs = header_signatures()
    assert sorted(sigs) == header_functions()
    assert sorted(_lib._SIGS) == sorted(sigs)
    for name, (ret, params) in sigs.items():
        b_ret, b_args = _lib._SIGS[name]
        want_ret = ctypes.c_char_p if ret == "char*" else c_of[ret]
        assert b_ret is want_ret, (name, ret, b_ret)
        assert len(b_args) == len(params), (name, params, b_args)
        for i, (t, b) in enumerate(zip(params, b_args)):
            want = ctypes.c_void_p if t.endswith("*") else c_of[t]
            assert b is want, (name, i, t, b)


def test_status_strings():
    for code in range(0, 12):
        s = _lib.status_str(code)
        assert s and s != "unknown status"
    assert _lib.status_str(99) == "unknown status"


def test_workspace_bytes():
    assert _lib.workspace_bytes(_lib.OP_QUANT_ACT, 16, 0, 4096, "block") == 0
    assert _lib.workspace_bytes(_lib.OP_QUANT_ACT, 16, 0, 4096, "tensor") == 4096
    assert _lib.workspace_bytes(_lib.OP_QUANT_WEIGHT, 4096, 0, 4096, "tensor") == 4096
    assert _lib.workspace_bytes(_lib.OP_GEMM, 16, 256, 4096, "tensor") == 0
    # split K: 1024 x 4096 has 128 tiles of 128 x 256 (at most half of 256
    # CUs) and K / 128 = 112 is a multiple of 8: 64 KiB of slot words, then a
    # 16 KiB fp32 partial per (tile, wave); every scale form
    for mode in ("block", "tensor", "row"):
        assert _lib.workspace_bytes(_lib.OP_GEMM, 1024, 4096, 14336, mode) == 65536 + 128 * 8 * 16384
    assert _lib.workspace_bytes(_lib.OP_GEMM, 2048, 4096, 14336, "block") == 0   # 256 tiles
    assert _lib.workspace_bytes(_lib.OP_GEMM, 4096, 4096, 4096, "block") == 0    # 256 x 256 tiles
    assert _lib.workspace_bytes(_lib.OP_GEMM, 1024, 4096, 14208, "block") == 0   # 111 K blocks
    assert _lib.workspace_bytes(_lib.OP_GEMM, 64, 4096, 14336, "block") == 0     # decode shape
    lin = _lib.workspace_bytes(_lib.OP_LINEAR, 1024, 4096, 14336, "block")
    assert lin >= 1024 * 14336 + 1024 * 112 * 4 + 65536 + 128 * 8 * 16384
    lin2 = _lib.workspace_bytes(_lib.OP_LINEAR, 2048, 4096, 14336, "block")
    assert lin2 >= 2048 * 14336 + 2048 * 112 * 4
    # ... and both fit fp8_linear_noalloc's scratch (FP8_NOALLOC_SCRATCH_BYTES)
    with open(os.path.join(ROOT, "include", "fp8w8a8.h")) as f:
        m = re.search(r"#define FP8_NOALLOC_SCRATCH_BYTES \((\d+)u << (\d+)\)", f.read())
    assert max(lin, lin2) <= int(m.group(1)) << int(m.group(2))
    # fused decode linear needs none; other shapes hold codes + scales
    assert _lib.workspace_bytes(_lib.OP_LINEAR, 4, 11008, 4096, "block") == 0
    # up to 16 rows fuse while M * K <= 16384 and (N / 16) * M * K <= 2^21
    assert _lib.workspace_bytes(_lib.OP_LINEAR, 16, 256, 512, "block") == 0     # the tiny shape
    assert _lib.workspace_bytes(_lib.OP_LINEAR, 16, 2048, 1024, "block") == 0   # 2^21 exactly
    assert _lib.workspace_bytes(_lib.OP_LINEAR, 16, 2176, 1024, "block") > 0    # grid past 2^21
    assert _lib.workspace_bytes(_lib.OP_LINEAR, 16, 256, 1152, "block") > 0     # M * K past 16384
    assert _lib.workspace_bytes(_lib.OP_LINEAR, 17, 256, 512, "block") > 0
    assert _lib.workspace_bytes(_lib.OP_LINEAR, 16, 256, 512, "tensor") > 0     # block scales only
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


OFFS = 0xA0_0000_0000


def vgg(a=X, ld_a=None, sa=S, ld_as=None, w=Q, ld_w=None, sw=WS, ld_ws=None, off=OFFS, E=4,
        out=O, ld_out=None, M=40, N=256, K=512):
    ld_a = K if ld_a is None else ld_a
    ld_w = K if ld_w is None else ld_w
    ld_as = K // 128 if ld_as is None else ld_as
    ld_ws = K // 128 if ld_ws is None else ld_ws
    ld_out = N if ld_out is None else ld_out
    return _lib.lib().fp8_validate_grouped_gemm(a, ld_a, sa, ld_as, w, ld_w, sw, ld_ws, off, E,
                                                out, ld_out, M, N, K)


def test_validate_grouped_gemm():
    assert vgg() == OK
    assert vgg(M=0, a=None, sa=None) == OK                    # nothing to do
    assert vgg(E=0, w=None, sw=None, off=None) == OK
    assert vgg(E=-1) == SHAPE
    assert vgg(E=65536) == SHAPE
    assert vgg(K=128 * 129) == SHAPE                          # K <= 16384
    assert vgg(N=200) == SHAPE
    assert vgg(off=None) == NULL
    assert vgg(off=OFFS + 4) == ALIGN
    assert vgg(ld_ws=3) == STRIDE
    assert vgg(ld_out=128) == STRIDE
    assert vgg(ld_a=520) == ALIGN
    assert vgg(out=Q + 4 * 256 * 512 - 64) == ALIAS           # over the last expert's codes
    assert vgg(out=Q + 4 * 256 * 512) == OK                   # just past them
    assert vgg(out=OFFS - 16) == ALIAS                        # over the offsets


KC = 0x60_0000_0000
VC = 0x70_0000_0000
SL = 0x80_0000_0000
KS = 0x90_0000_0000
VS = 0x90_0000_0010


def vkw(k=X, ld_k=None, v=O, ld_v=None, sl=SL, T=37, H=8, D=128, kc=KC, vc=VC, nb=5, bs=16,
        ks=KS, vs=VS):
    ld_k = H * D if ld_k is None else ld_k
    ld_v = H * D if ld_v is None else ld_v
    return _lib.lib().fp8_validate_kv_cache_write(k, ld_k, v, ld_v, sl, T, H, D, kc, vc, nb, bs,
                                                  ks, vs)


def test_validate_kv_cache_write():
    assert vkw() == OK
    assert vkw(T=0, k=None, v=None, sl=None, kc=None, vc=None, ks=None, vs=None) == OK
    assert vkw(nb=0, kc=None, vc=None) == OK                    # nothing can be stored
    assert vkw(kc=None) == NULL
    assert vkw(ks=None) == NULL
    assert vkw(sl=None) == NULL
    assert vkw(T=-1) == SHAPE
    assert vkw(H=0) == SHAPE
    assert vkw(H=1, D=12) == SHAPE                              # H * D not a multiple of 8
    assert vkw(H=3, D=8) == OK
    assert vkw(bs=0) == SHAPE
    assert vkw(nb=-1) == SHAPE
    assert vkw(ld_k=1000) == STRIDE
    assert vkw(ld_k=1032) == OK                                 # tokens of a wider row
    assert vkw(ld_v=1028) == ALIGN
    assert vkw(k=X + 8) == ALIGN
    assert vkw(kc=KC + 8) == ALIGN
    assert vkw(sl=SL + 4) == ALIGN
    assert vkw(ks=KS + 2) == ALIGN
    assert vkw(vc=KC + 4096) == ALIAS                           # the two caches overlap
    assert vkw(kc=X + 2048) == ALIAS                            # cache over the keys
    assert vkw(sl=VC + 64) == ALIAS
    assert vkw(k=X, v=X) == OK                                  # inputs may coincide
    assert vkw(nb=1 << 31) == SHAPE


def vkr(c=KC, nb=5, bs=16, H=8, D=128, sl=SL, T=37, s=KS, out=O, ld_out=None):
    ld_out = H * D if ld_out is None else ld_out
    return _lib.lib().fp8_validate_kv_cache_read(c, nb, bs, H, D, sl, T, s, out, ld_out)


def test_validate_kv_cache_read():
    assert vkr() == OK
    assert vkr(T=0, c=None, sl=None, s=None, out=None) == OK
    assert vkr(nb=0, c=None) == OK                              # every token reads zeros
    assert vkr(out=None) == NULL
    assert vkr(s=None) == NULL
    assert vkr(D=4, H=1) == SHAPE
    assert vkr(ld_out=512) == STRIDE
    assert vkr(ld_out=1028) == ALIGN
    assert vkr(out=O + 2) == ALIGN
    assert vkr(c=KC + 8) == ALIGN
    assert vkr(out=KC + 1024) == ALIAS                          # output over the cache
    assert vkr(out=SL - 64) == ALIAS                            # output over the slots


def test_binding_rejects_host_tensors():
    torch = pytest.importorskip("torch")
    x = torch.zeros((16, 512), dtype=torch.bfloat16)
    with pytest.raises(ValueError):
        _lib.quant_act(x)


def test_binding_scale_vector_strides():
    torch = pytest.importorskip("torch")
    v = torch.zeros(12)
    assert _lib._vec_ld(v[:1], 5, "s") == 0                  # one value for all rows
    assert _lib._vec_ld(v[:5], 5, "s") == 1
    assert _lib._vec_ld(v[::2][:5], 5, "s") == 2
    m = torch.zeros((5, 3))
    assert _lib._vec_ld(m[:, 0], 5, "s") == 3                # a column of a matrix
    assert _lib._vec_ld(m[:, :1], 5, "s") == 3               # the same as [5, 1]
    assert _lib._vec_ld(torch.zeros((1, 5)), 5, "s") == 1
    with pytest.raises(ValueError):
        _lib._vec_ld(v[:4], 5, "s")                           # wrong count
    with pytest.raises(ValueError):
        _lib._vec_ld(torch.zeros((5, 2)), 10, "s")            # not a vector


def test_binding_rejects_host_scales_and_outputs():
    torch = pytest.importorskip("torch")
    dev = torch.device("cuda", 0)
    with pytest.raises(ValueError):
        _lib._device_tensor(torch.zeros(4), "s", torch.float32, dev)
    with pytest.raises(TypeError):
        _lib._device_tensor(torch.zeros(4, dtype=torch.float64), "s", torch.float32, dev)
    with pytest.raises(TypeError):
        _lib._device_tensor(None, "s", torch.float32, dev)


def test_leading_dimensions_are_bounded():
    # rows x ld beyond 2^56 elements is refused before any byte range is
    # formed (such a tensor cannot exist, and its range would overflow)
    huge = 1 << 62
    assert vq(ld_x=huge) == STRIDE
    assert vq(ld_q=huge) == STRIDE
    assert vq(ld_s=huge) == STRIDE
    assert vq(mode=2, ld_s=huge) == STRIDE
    assert vq(M=1 << 20, ld_x=1 << 37) == STRIDE          # 2^57 elements
    assert vq(M=2, ld_x=1 << 30) == OK                    # large but within bounds
    assert vg(ld_a=huge) == STRIDE
    assert vg(ld_w=huge) == STRIDE
    assert vg(ld_out=huge) == STRIDE
    assert vg(ld_as=huge) == STRIDE
    assert vg(ld_ws=huge) == STRIDE
    assert vg(ld_as=huge, mode=1) == OK                    # per-tensor scales have no ld
    assert vg(mode=2, ld_as=(1 << 31) - 1, ld_ws=1, M=(1 << 26)) == STRIDE
    assert vgg(ld_a=huge) == STRIDE
    assert vgg(ld_w=huge) == STRIDE
    assert vgg(ld_ws=huge) == STRIDE
    assert vkw(ld_k=huge) == STRIDE
    assert vkr(ld_out=huge) == STRIDE


def test_grids_beyond_32_bit_work_items_are_shapes():
    # every launch must stay below 2^32 work-items (the dispatch packet's
    # grid size is 32-bit): such calls are refused as shapes up front.
    # Fake tensors 2^44 bytes apart, so these sizes do not overlap.
    far = dict(x=1 << 44, q=2 << 44, s=3 << 44)
    assert vq(M=(1 << 24) - 1, K=4096, **far) == OK          # 256 threads per row: just fits
    assert vq(M=1 << 24, K=4096, **far) == SHAPE
    assert vq(M=1 << 25, K=512, **far) == OK                  # groups numbered across rows
    assert vq(M=1 << 30, K=512, **far) == SHAPE
    assert vq(M=(1 << 26) - 4, K=128, ld_s=1, mode=2, **far) == OK   # per row: 4 rows a group
    assert vq(M=1 << 26, K=128, ld_s=1, mode=2, **far) == SHAPE
    farw = dict(w=1 << 44, q=2 << 44, s=3 << 44)
    assert vw(N=1 << 20, K=1 << 17, **farw) == OK             # a workgroup per 128 x 128 block
    assert vw(N=1 << 20, K=1 << 18, **farw) == SHAPE
    farg = dict(a=1 << 44, w=2 << 44, out=3 << 44, sa=4 << 44, sw=5 << 44)
    assert vg(M=16, N=(1 << 27) - 128, K=128, **farg) == OK   # decode tile: 16 columns a group
    assert vg(M=16, N=1 << 27, K=128, **farg) == SHAPE
    assert vg(M=1 << 19, N=1 << 18, K=128, **farg) == OK      # tile grid of the large-M kernels
    assert vg(M=1 << 19, N=1 << 19, K=128, **farg) == SHAPE
    assert vgg(N=1 << 27, K=128) == SHAPE
    lib = _lib.lib()
    # fp8_e4m3_encode_f32 and fp8_linear validate before they touch a device
    assert lib.fp8_e4m3_encode_f32(X, 1 << 32, Q, None) == SHAPE
    assert lib.fp8_linear(X, 128, Q, 128, S, 1, O, 1 << 27, 1, 1 << 27, 128, 0, None, 0,
                          None) == SHAPE
