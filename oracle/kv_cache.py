"""FP8 KV-cache codec (oracle).

TEST INFRASTRUCTURE ONLY -- not part of the product path.

What the pages describe: the KV cache is a separate quantization target from
the weights; with an fp8 KV dtype the keys and values are stored as E4M3
instead of 16 bits, halving the cache ("FP8 Quantization", D.4; "[vLLM] FP8",
KV cache quantization and "why this design" item 4).  Each of K and V has a
scale: the default is 1.0, which clips outliers, or a calibrated one baked
into the checkpoint; one paged-attention block holds 16 tokens; outside an
FP8 attention backend the stored codes are only a storage format, restored
to 16 bits inside the attention kernel ("Quantization guide for serving:
FP8, AWQ, GPTQ", KV-cache FP8 section).

What is computed here:
    write:  cache[slot(t), h, d] = E4M3( fp32(x[t, h, d]) / scale )
            (the static quantizer of oracle.quant: IEEE quotient, RNE,
            saturating), for every token t whose slot is in range; other
            cache entries are left as they were.
    read:   out[t, h, d] = bf16_RNE( fp32(dec(cache[slot(t), h, d])) * scale )
            for slots in range; tokens with an out-of-range slot read zeros.

Readings (the pages give no formula): the stored code is x / scale, the
restored value code * scale (the dequantized value of oracle.quant); slot =
block * block_size + offset in a cache laid out [blocks, block_size, heads,
head_dim]; a negative slot marks a token that is not stored (padding); the
restore multiplies in fp32 and rounds once to bf16; a NaN product (a NaN
code, or a NaN / infinite scale) restores to the quiet bf16 NaN carrying the
sign of the stored code, so the sign never depends on how a NaN propagates.
"""

import numpy as np

from . import e4m3, quant


def kv_write_ref(x_bits, slots, cache, scale):
    """Scatter E4M3(x / scale) into a copy of ``cache``.

    x_bits: uint16 [T, H, D] bf16; slots: int64 [T]; cache: uint8
    [blocks, block_size, H, D].  Returns the new cache.
    """
    x_bits = np.asarray(x_bits, dtype=np.uint16)
    T, H, D = x_bits.shape
    out = np.array(cache, dtype=np.uint8, copy=True)
    nb, bs = out.shape[0], out.shape[1]
    assert out.shape[2:] == (H, D)
    codes = quant.quant_static_ref(x_bits.reshape(T, H * D), scale).reshape(T, H, D)
    for t in range(T):
        s = int(slots[t])
        if 0 <= s < nb * bs:
            out[s // bs, s % bs] = codes[t]
    return out


def bf16_rne_bits(f32):
    """fp32 -> bf16 bit patterns, round to nearest even; NaN -> quiet NaN with its sign."""
    f = np.asarray(f32, dtype=np.float32)
    b = f.view(np.uint32).astype(np.uint64)
    r = ((b + np.uint64(0x7FFF) + ((b >> np.uint64(16)) & np.uint64(1))) >> np.uint64(16))
    r = r.astype(np.uint16)
    nan = np.isnan(f)
    sign = (f.view(np.uint32) >> np.uint32(16)).astype(np.uint16) & np.uint16(0x8000)
    return np.where(nan, sign | np.uint16(0x7FC0), r).astype(np.uint16)


def kv_read_ref(cache, slots, scale):
    """Gather and restore: bf16 bits [T, H, D] of dec(cache[slot]) * scale."""
    cache = np.asarray(cache, dtype=np.uint8)
    nb, bs, H, D = cache.shape
    T = len(slots)
    out = np.zeros((T, H, D), dtype=np.uint16)
    s32 = np.float32(np.asarray(scale, dtype=np.float32).reshape(-1)[0])
    for t in range(T):
        s = int(slots[t])
        if 0 <= s < nb * bs:
            codes = cache[s // bs, s % bs]
            v = e4m3.decode(codes).astype(np.float32)
            with np.errstate(over="ignore", invalid="ignore"):
                prod = (v * s32).astype(np.float32)
            r = bf16_rne_bits(prod)
            code_sign = (codes.astype(np.uint16) & np.uint16(0x80)) << np.uint16(8)
            out[t] = np.where(np.isnan(prod), code_sign | np.uint16(0x7FC0), r)
    return out
