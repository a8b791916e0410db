"""ctypes binding of libfp8w8a8.so: argument marshalling only.

Every step of the computation runs in the library's HIP kernels; this module
turns torch tensors into device pointers, leading dimensions and the current
HIP stream, and turns nonzero status codes into ValueError (the same
convention as the eager configuration errors of "[vLLM] FP8", block
quantization).  There is no fallback: if the library is missing, importing
the binding raises.
"""

import ctypes
import os

import torch

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libfp8w8a8.so")

FP8_OK = 0
SCALE_BLOCK = 0
SCALE_TENSOR = 1
SCALE_ROW = 2
OP_QUANT_ACT = 0
OP_QUANT_WEIGHT = 1
OP_GEMM = 2
OP_LINEAR = 3

_MODES = {"block": SCALE_BLOCK, "tensor": SCALE_TENSOR, "row": SCALE_ROW}

_i64 = ctypes.c_int64
_int = ctypes.c_int
_vp = ctypes.c_void_p
_sz = ctypes.c_size_t

_SIGS = {
    "fp8_status_str": (ctypes.c_char_p, [_int]),
    "fp8_workspace_bytes": (_sz, [_int, _i64, _i64, _i64, _int]),
    "fp8_quant_act": (_int, [_vp, _i64, _i64, _i64, _vp, _i64, _vp, _i64, _int, _vp, _sz, _vp]),
    "fp8_quant_weight_block": (_int, [_vp, _i64, _i64, _i64, _vp, _i64, _vp, _i64, _int, _int,
                                      _int, _vp, _sz, _vp]),
    "fp8_block_gemm": (_int, [_vp, _i64, _vp, _i64, _vp, _i64, _vp, _i64, _vp, _i64, _i64, _i64,
                              _i64, _int, _vp, _sz, _vp]),
    "fp8_validate_quant_act": (_int, [_vp, _i64, _i64, _i64, _vp, _i64, _vp, _i64, _int, _vp,
                                      _sz]),
    "fp8_validate_quant_weight_block": (_int, [_vp, _i64, _i64, _i64, _vp, _i64, _vp, _i64, _int,
                                               _int, _int, _vp, _sz]),
    "fp8_validate_block_gemm": (_int, [_vp, _i64, _vp, _i64, _vp, _i64, _vp, _i64, _vp, _i64,
                                       _i64, _i64, _i64, _int]),
    "fp8_e4m3_encode_f32": (_int, [_vp, _i64, _vp, _vp]),
    "fp8_linear": (_int, [_vp, _i64, _vp, _i64, _vp, _i64, _vp, _i64, _i64, _i64, _i64, _int, _vp,
                          _sz, _vp]),
    "fp8_linear_noalloc": (_int, [_vp, _i64, _vp, _i64, _vp, _i64, _vp, _i64, _i64, _i64, _i64,
                                  _int, _vp]),
    "fp8_quant_act_static": (_int, [_vp, _i64, _i64, _i64, _vp, _i64, _vp, _vp]),
    "fp8_validate_quant_act_static": (_int, [_vp, _i64, _i64, _i64, _vp, _i64, _vp]),
    "fp8_grouped_gemm": (_int, [_vp, _i64, _vp, _i64, _vp, _i64, _vp, _i64, _vp, _i64, _vp, _i64,
                                _i64, _i64, _i64, _vp]),
    "fp8_validate_grouped_gemm": (_int, [_vp, _i64, _vp, _i64, _vp, _i64, _vp, _i64, _vp, _i64,
                                         _vp, _i64, _i64, _i64, _i64]),
    "fp8_kv_cache_write": (_int, [_vp, _i64, _vp, _i64, _vp, _i64, _i64, _i64, _vp, _vp, _i64,
                                  _i64, _vp, _vp, _vp]),
    "fp8_kv_cache_read": (_int, [_vp, _i64, _i64, _i64, _i64, _vp, _i64, _vp, _vp, _i64, _vp]),
    "fp8_validate_kv_cache_write": (_int, [_vp, _i64, _vp, _i64, _vp, _i64, _i64, _i64, _vp, _vp,
                                           _i64, _i64, _vp, _vp]),
    "fp8_validate_kv_cache_read": (_int, [_vp, _i64, _i64, _i64, _i64, _vp, _i64, _vp, _vp,
                                          _i64]),
}

_lib = None


def lib():
    """The loaded shared library (ctypes.CDLL) with argument types set."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError(
                f"{LIB_PATH} is missing: build it with `python -m fp8_w8a8_block_amd.build`")
        l = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in _SIGS.items():
            f = getattr(l, name)
            f.restype = res
            f.argtypes = args
        _lib = l
    return _lib


def status_str(code):
    return lib().fp8_status_str(int(code)).decode()


def _check(code):
    if code != FP8_OK:
        raise ValueError(f"fp8w8a8 status {code}: {status_str(code)}")


def _mode(scale_mode):
    if isinstance(scale_mode, str):
        if scale_mode not in _MODES:
            raise ValueError(f"unknown scale mode {scale_mode!r}")
        return _MODES[scale_mode]
    return int(scale_mode)


def _stream(t):
    return ctypes.c_void_p(torch.cuda.current_stream(t.device).cuda_stream)


def _rows(t, dtype, name):
    if t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if t.dim() != 2 or t.stride(1) != 1:
        raise ValueError(f"{name} must be a 2-D row-major tensor with unit column stride")
    if not t.is_cuda:
        raise ValueError(f"{name} must be a device tensor")
    # a single row's stride is arbitrary in torch; its leading dimension is its length
    return t.shape[0], t.shape[1], (t.stride(0) if t.shape[0] > 1 else t.shape[1])


def _ld(t):
    """Leading dimension of a 2-D scale tensor (one row: its length)."""
    if t.dim() != 2:
        return 1
    return t.stride(0) if t.shape[0] > 1 else t.shape[1]


def _vec_ld(t, n, name):
    """Element stride of a row-mode scale vector of n entries (1-D, or 2-D
    with one dimension of size 1), or 0 for a single value shared by all."""
    if t.numel() == 1:
        return 0
    if t.numel() != n:
        raise ValueError(f"{name} must hold {n} scales or one, got {t.numel()}")
    if t.dim() == 1:
        return t.stride(0)
    if t.dim() == 2 and 1 in t.shape:
        return t.stride(0) if t.shape[1] == 1 else t.stride(1)
    raise ValueError(f"{name} must be a vector")


def _device_tensor(t, name, dtype, device, shape=None):
    """Check a caller-supplied tensor before its pointer goes to a kernel:
    type, dtype, device and (if given) exact shape."""
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a tensor")
    if t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if not t.is_cuda or t.device != device:
        raise ValueError(f"{name} must be a tensor on {device}")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} must have shape {tuple(shape)}, got {tuple(t.shape)}")
    return t


def _scale_matrix(t, name, rows, cols, device):
    """Block-scale matrix [rows, cols] with unit column stride -> its leading dimension."""
    _device_tensor(t, name, torch.float32, device, (rows, cols))
    if cols > 1 and t.stride(1) != 1:
        raise ValueError(f"{name} must have unit column stride")
    return _ld(t)


def _workspace(ws, device):
    if ws is None:
        return None, 0
    _device_tensor(ws, "workspace", torch.uint8, device)
    if not ws.is_contiguous():
        raise ValueError("workspace must be contiguous")
    return ws.data_ptr(), ws.numel()


def workspace_bytes(op, M, N, K, scale_mode):
    return int(lib().fp8_workspace_bytes(int(op), int(M), int(N), int(K), _mode(scale_mode)))


def quant_act(x, scale_mode="block", workspace=None, q=None, scales=None):
    """Dynamic activation quantization of bf16 x [M, K] -> (codes uint8 [M, K], scales fp32).

    Block mode gives scales [M, K/128]; row (per-token) mode [M]; tensor mode
    a 1-element tensor.
    """
    mode = _mode(scale_mode)
    M, K, ld_x = _rows(x, torch.bfloat16, "x")
    with torch.cuda.device(x.device):
        if q is None:
            q = torch.empty((M, K), dtype=torch.uint8, device=x.device)
        _device_tensor(q, "q", torch.uint8, x.device, (M, K))
        ld_q = _rows(q, torch.uint8, "q")[2]
        shape = (M, K // 128) if mode == SCALE_BLOCK else (M,) if mode == SCALE_ROW else (1,)
        if scales is None:
            scales = torch.empty(shape, dtype=torch.float32, device=x.device)
        if mode == SCALE_BLOCK:
            ld_s = _scale_matrix(scales, "scales", M, K // 128, x.device)
        else:
            _device_tensor(scales, "scales", torch.float32, x.device, shape)
            ld_s = scales.stride(0) if mode == SCALE_ROW else 1
        nws = workspace_bytes(OP_QUANT_ACT, M, 0, K, mode)
        if nws and workspace is None:
            workspace = torch.empty(nws, dtype=torch.uint8, device=x.device)
        ws_ptr, ws_len = _workspace(workspace, x.device)
        _check(lib().fp8_quant_act(x.data_ptr(), M, K, ld_x, q.data_ptr(), ld_q,
                                   scales.data_ptr(), ld_s, mode, ws_ptr, ws_len, _stream(x)))
    return q, scales


def quant_weight_block(w, scale_mode="block", block_n=128, block_k=128, workspace=None):
    """Weight quantization of bf16 w [N, K] -> (codes uint8 [N, K], scales fp32).

    Block mode gives scales [N/128, K/128]; row (per-channel) mode [N];
    tensor mode a 1-element tensor.
    """
    mode = _mode(scale_mode)
    N, K, ld_w = _rows(w, torch.bfloat16, "w")
    with torch.cuda.device(w.device):
        q = torch.empty((N, K), dtype=torch.uint8, device=w.device)
        if mode == SCALE_BLOCK:
            scales = torch.empty((max(N // 128, 0), K // 128), dtype=torch.float32, device=w.device)
            ld_s = _ld(scales)
        elif mode == SCALE_ROW:
            scales = torch.empty((N,), dtype=torch.float32, device=w.device)
            ld_s = 1
        else:
            scales = torch.empty((1,), dtype=torch.float32, device=w.device)
            ld_s = 1
        nws = workspace_bytes(OP_QUANT_WEIGHT, N, 0, K, mode)
        if nws and workspace is None:
            workspace = torch.empty(nws, dtype=torch.uint8, device=w.device)
        ws_ptr, ws_len = _workspace(workspace, w.device)
        _check(lib().fp8_quant_weight_block(w.data_ptr(), N, K, ld_w, q.data_ptr(), K,
                                            scales.data_ptr(), ld_s, int(block_n), int(block_k),
                                            mode, ws_ptr, ws_len, _stream(w)))
    return q, scales


def block_gemm(a_q, a_s, w_q, w_s, scale_mode="block", out=None, workspace=None, split=True):
    """out[M, N] bf16 = A . W^T from FP8 codes and their scales.

    Shapes that split K in two (fp8_workspace_bytes(FP8_OP_GEMM) > 0) get a
    workspace (allocated here unless given); split=False passes none, so the
    call runs unsplit."""
    mode = _mode(scale_mode)
    M, K, ld_a = _rows(a_q, torch.uint8, "a_q")
    N, K2, ld_w = _rows(w_q, torch.uint8, "w_q")
    if K2 != K:
        raise ValueError(f"K mismatch: a_q has {K}, w_q has {K2}")
    _device_tensor(w_q, "w_q", torch.uint8, a_q.device)
    for t, nm in ((a_s, "a_s"), (w_s, "w_s")):
        _device_tensor(t, nm, torch.float32, a_q.device)
    if mode == SCALE_ROW:
        ld_as, ld_ws = _vec_ld(a_s, M, "a_s"), _vec_ld(w_s, N, "w_s")
    elif mode == SCALE_BLOCK:
        ld_as = _scale_matrix(a_s, "a_s", M, K // 128, a_q.device)
        ld_ws = _scale_matrix(w_s, "w_s", N // 128, K // 128, a_q.device)
    else:
        if a_s.numel() != 1 or w_s.numel() != 1:
            raise ValueError("per-tensor scales are one value each")
        ld_as, ld_ws = 1, 1
    with torch.cuda.device(a_q.device):
        if out is None:
            out = torch.empty((M, N), dtype=torch.bfloat16, device=a_q.device)
        _device_tensor(out, "out", torch.bfloat16, a_q.device, (M, N))
        ld_out = _rows(out, torch.bfloat16, "out")[2]
        ws_ptr, ws_len = None, 0
        if split:
            nws = workspace_bytes(OP_GEMM, M, N, K, mode)
            if nws and workspace is None:
                workspace = torch.empty(nws, dtype=torch.uint8, device=a_q.device)
            if workspace is not None:
                ws_ptr, ws_len = _workspace(workspace, a_q.device)
        _check(lib().fp8_block_gemm(a_q.data_ptr(), ld_a, a_s.data_ptr(), ld_as, w_q.data_ptr(),
                                    ld_w, w_s.data_ptr(), ld_ws, out.data_ptr(), ld_out,
                                    M, N, K, mode, ws_ptr, ws_len, _stream(a_q)))
    return out


def linear(x, w_q, w_s, scale_mode="block", out=None, workspace=None):
    """One W8A8 linear call in one library call: out = GEMM(quant_act(x), W).

    Bit-identical to quant_act followed by block_gemm.  Block-scaled calls
    with few rows run fused (no workspace: workspace_bytes(OP_LINEAR) is 0);
    otherwise a workspace is used (allocated here unless given).  Row mode: per-token activation scales, per-channel
    weight scales w_s [N] (or one value).
    """
    mode = _mode(scale_mode)
    M, K, ld_x = _rows(x, torch.bfloat16, "x")
    N, K2, ld_w = _rows(w_q, torch.uint8, "w_q")
    if K2 != K:
        raise ValueError(f"K mismatch: x has {K}, w_q has {K2}")
    _device_tensor(w_q, "w_q", torch.uint8, x.device)
    _device_tensor(w_s, "w_s", torch.float32, x.device)
    if mode == SCALE_ROW:
        ld_ws = _vec_ld(w_s, N, "w_s")
    elif mode == SCALE_BLOCK:
        ld_ws = _scale_matrix(w_s, "w_s", N // 128, K // 128, x.device)
    else:
        if w_s.numel() != 1:
            raise ValueError("a per-tensor weight scale is one value")
        ld_ws = 1
    with torch.cuda.device(x.device):
        if out is None:
            out = torch.empty((M, N), dtype=torch.bfloat16, device=x.device)
        _device_tensor(out, "out", torch.bfloat16, x.device, (M, N))
        ld_out = _rows(out, torch.bfloat16, "out")[2]
        nws = workspace_bytes(OP_LINEAR, M, N, K, mode)
        if nws and workspace is None:
            workspace = torch.empty(nws, dtype=torch.uint8, device=x.device)
        ws_ptr, ws_len = _workspace(workspace, x.device)
        _check(lib().fp8_linear(x.data_ptr(), ld_x, w_q.data_ptr(), ld_w, w_s.data_ptr(), ld_ws,
                                out.data_ptr(), ld_out, M, N, K, mode, ws_ptr, ws_len, _stream(x)))
    return out


def linear_noalloc(x, w_q, w_s, out, scale_mode="block"):
    """fp8_linear_noalloc: the linear call with the library's own per-device
    scratch instead of a workspace (for callers that cannot allocate; the
    caller passes the output).  Bit-identical to linear()."""
    mode = _mode(scale_mode)
    M, K, ld_x = _rows(x, torch.bfloat16, "x")
    N, K2, ld_w = _rows(w_q, torch.uint8, "w_q")
    if K2 != K:
        raise ValueError(f"K mismatch: x has {K}, w_q has {K2}")
    _device_tensor(w_q, "w_q", torch.uint8, x.device)
    _device_tensor(w_s, "w_s", torch.float32, x.device)
    if mode == SCALE_ROW:
        ld_ws = _vec_ld(w_s, N, "w_s")
    elif mode == SCALE_BLOCK:
        ld_ws = _scale_matrix(w_s, "w_s", N // 128, K // 128, x.device)
    else:
        if w_s.numel() != 1:
            raise ValueError("a per-tensor weight scale is one value")
        ld_ws = 1
    _device_tensor(out, "out", torch.bfloat16, x.device, (M, N))
    ld_out = _rows(out, torch.bfloat16, "out")[2]
    with torch.cuda.device(x.device):
        _check(lib().fp8_linear_noalloc(x.data_ptr(), ld_x, w_q.data_ptr(), ld_w, w_s.data_ptr(),
                                        ld_ws, out.data_ptr(), ld_out, M, N, K, mode, _stream(x)))
    return out


def quant_act_static(x, scale, q=None):
    """Static activation quantization of bf16 x [M, K] with a calibrated
    scale (a 1-element float32 device tensor) -> codes uint8 [M, K]."""
    M, K, ld_x = _rows(x, torch.bfloat16, "x")
    _scalar_scale(scale, "scale")
    _device_tensor(scale, "scale", torch.float32, x.device)
    with torch.cuda.device(x.device):
        if q is None:
            q = torch.empty((M, K), dtype=torch.uint8, device=x.device)
        _device_tensor(q, "q", torch.uint8, x.device, (M, K))
        ld_q = _rows(q, torch.uint8, "q")[2]
        _check(lib().fp8_quant_act_static(x.data_ptr(), M, K, ld_x, q.data_ptr(), ld_q,
                                          scale.data_ptr(), _stream(x)))
    return q


def grouped_gemm(a_q, a_s, w_q, w_s, expert_offsets, out=None):
    """MoE grouped block-scaled GEMM: rows expert_offsets[e] .. [e+1] of the
    codes a_q [M, K] (scales a_s [M, K/128]) against expert e of w_q
    [E, N, K] (scales w_s [E, N/128, K/128]) -> bf16 [M, N].  Rows in no
    expert's range are left as they were in ``out`` (uninitialized when
    ``out`` is None)."""
    M, K, ld_a = _rows(a_q, torch.uint8, "a_q")
    if w_q.dtype != torch.uint8 or w_q.dim() != 3 or not w_q.is_cuda:
        raise ValueError("w_q must be a uint8 [E, N, K] device tensor")
    E, N, Kw = w_q.shape
    if Kw != K:
        raise ValueError("w_q and a_q disagree on K")
    if w_q.stride(2) != 1 or w_q.stride(0) != N * w_q.stride(1):
        raise ValueError("w_q experts must be stacked rows: strides (N * ld_w, ld_w, 1)")
    ld_w = w_q.stride(1) if N > 1 else K
    _device_tensor(w_q, "w_q", torch.uint8, a_q.device)
    _device_tensor(w_s, "w_s", torch.float32, a_q.device, (E, N // 128, K // 128))
    if w_s.stride(2) != 1 or w_s.stride(0) != (N // 128) * w_s.stride(1):
        raise ValueError("w_s must be a float32 [E, N/128, K/128] device tensor, experts stacked")
    ld_as = _scale_matrix(a_s, "a_s", M, K // 128, a_q.device)
    ld_ws = w_s.stride(1) if N // 128 > 1 else w_s.shape[2]
    _device_tensor(expert_offsets, "expert_offsets", torch.int64, a_q.device, (E + 1,))
    offs = expert_offsets.contiguous()
    with torch.cuda.device(a_q.device):
        if out is None:
            out = torch.empty((M, N), dtype=torch.bfloat16, device=a_q.device)
        _device_tensor(out, "out", torch.bfloat16, a_q.device, (M, N))
        ld_out = _rows(out, torch.bfloat16, "out")[2]
        _check(lib().fp8_grouped_gemm(a_q.data_ptr(), ld_a, a_s.data_ptr(), ld_as,
                                      w_q.data_ptr(), ld_w, w_s.data_ptr(), ld_ws,
                                      offs.data_ptr(), E, out.data_ptr(), ld_out,
                                      M, N, K, _stream(a_q)))
    return out


def _scalar_scale(t, name):
    if t.dtype != torch.float32 or not t.is_cuda or t.numel() != 1:
        raise TypeError(f"{name} must be a 1-element float32 device tensor")


def _tokens(t, name):
    """[T, H, D] bf16 with each token's H * D values contiguous -> (T, H, D, ld)."""
    if t.dtype != torch.bfloat16:
        raise TypeError(f"{name} must be bfloat16, got {t.dtype}")
    if t.dim() != 3 or t.stride(2) != 1 or t.stride(1) != t.shape[2]:
        raise ValueError(f"{name} must be [T, H, D] with contiguous heads")
    if not t.is_cuda:
        raise ValueError(f"{name} must be a device tensor")
    T, H, D = t.shape
    return T, H, D, (t.stride(0) if T > 1 else H * D)


def _cache(c, name):
    if c.dtype != torch.uint8 or c.dim() != 4 or not c.is_contiguous() or not c.is_cuda:
        raise ValueError(f"{name} must be a contiguous uint8 [blocks, block_size, H, D] device "
                         "tensor")
    return c.shape


def _slots(s, T):
    if s.dtype != torch.int64 or s.dim() != 1 or s.shape[0] != T or not s.is_cuda:
        raise ValueError("slots must be a 1-D int64 device tensor with one entry per token")
    return s.contiguous()


def kv_cache_write(key, value, slot_mapping, key_cache, value_cache, k_scale, v_scale):
    """Store bf16 key / value [T, H, D] as E4M3 codes into the paged caches
    [blocks, block_size, H, D] at slot_mapping[t] (in place; negative or
    out-of-range slots are skipped)."""
    T, H, D, ld_k = _tokens(key, "key")
    Tv, Hv, Dv, ld_v = _tokens(value, "value")
    if (Tv, Hv, Dv) != (T, H, D):
        raise ValueError("key and value shapes differ")
    nb, bs, Hc, Dc = _cache(key_cache, "key_cache")
    if tuple(value_cache.shape) != (nb, bs, Hc, Dc) or (Hc, Dc) != (H, D):
        raise ValueError("cache shapes do not match the tokens")
    _cache(value_cache, "value_cache")
    _scalar_scale(k_scale, "k_scale")
    _scalar_scale(v_scale, "v_scale")
    slots = _slots(slot_mapping, T)
    with torch.cuda.device(key.device):
        _check(lib().fp8_kv_cache_write(key.data_ptr(), ld_k, value.data_ptr(), ld_v,
                                        slots.data_ptr(), T, H, D, key_cache.data_ptr(),
                                        value_cache.data_ptr(), nb, bs, k_scale.data_ptr(),
                                        v_scale.data_ptr(), _stream(key)))


def kv_cache_read(cache, slots, scale, out=None):
    """Gather cache[slots] and restore to bf16 [T, H, D] (out-of-range slots
    read zeros)."""
    nb, bs, H, D = _cache(cache, "cache")
    _scalar_scale(scale, "scale")
    T = slots.shape[0] if slots.dim() == 1 else -1
    slots = _slots(slots, T)
    with torch.cuda.device(cache.device):
        if out is None:
            out = torch.empty((T, H, D), dtype=torch.bfloat16, device=cache.device)
        To, Ho, Do, ld_o = _tokens(out, "out")
        if (To, Ho, Do) != (T, H, D):
            raise ValueError("out must be [T, H, D]")
        _check(lib().fp8_kv_cache_read(cache.data_ptr(), nb, bs, H, D, slots.data_ptr(), T,
                                       scale.data_ptr(), out.data_ptr(), ld_o, _stream(cache)))
    return out


def encode_f32(x):
    """E4M3 codes of fp32 values with the device encoder (saturating, RNE)."""
    if x.dtype != torch.float32 or not x.is_cuda or not x.is_contiguous():
        raise TypeError("x must be a contiguous float32 device tensor")
    with torch.cuda.device(x.device):
        codes = torch.empty(x.shape, dtype=torch.uint8, device=x.device)
        _check(lib().fp8_e4m3_encode_f32(x.data_ptr(), x.numel(), codes.data_ptr(), _stream(x)))
    return codes
