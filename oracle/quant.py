"""FP8 quantizers (oracle): dynamic 1x128 activations, 128x128 weights,
per-tensor and per-row (per token / per output channel); static per-tensor.

TEST INFRASTRUCTURE ONLY -- not part of the product path.

What is computed, per scaling group G (a 1x128 slice of an activation row, a
128x128 block of the weight, one whole row, or the whole tensor):

    amax = max_{x in G} |x|                       exact (bf16 -> fp32 widening)
    s    = fp32(amax) / fp32(448)                 IEEE fp32, round to nearest
    q    = fp32(x) / s                            IEEE fp32, round to nearest
    code = E4M3 encode of q                        RNE, saturating (oracle.e4m3)

Sources:
  * Activation scales are computed at run time, per call, from the data
    ("FP8 Quantization", sections C and D.2); the block path only accepts a
    dynamic activation scheme ("[vLLM] FP8", block quantization).
  * Scaling strategies: dynamic 128-group, dynamic per-tensor, dynamic
    per-token, static 128-block and static per-tensor are listed side by
    side; per-tensor uses one scale for the whole tensor, block-128 keeps one
    per block; "static" scales come from calibration beforehand, "dynamic"
    ones are computed at run time ("[vLLM] FP8", scaling strategies).
  * Weights pre-quantized with one scale per output channel are the
    recommended checkpoint form ("FP8 Quantization", the llm-compressor
    path); per-channel scales sit between per-tensor and per-group
    ("fp8-serving-slower-than-bf16", granularity).
  * Weight blocks are two-dimensional, 128x128, with an independent scale
    each so that an outlier only affects its own block ("[vLLM] FP8", block
    quantization and "why this design" item 2; "FP8 Quantization", D.1
    gives block size 128).
  * 448 is the largest E4M3 magnitude ("[vLLM] FP8", format table).

Readings (the pages give the scale only as "scale"; see oracle.e4m3 for the
format readings):
  * Per token = one group per activation row, per channel = one group per
    weight row (W is [N, K], row n feeds output column n): the same per-row
    quantizer serves both.
  * Static quantization applies the same quotient and encoding with a given
    scale; a zero scale follows IEEE division (x/0 saturates, 0/0 is NaN).
  * scale = amax / 448 maps the group's largest magnitude onto the largest
    code; dequantized value = code value * scale.
  * The quotient is a true fp32 division x / s, not x * (1/s).
  * An all-zero group gets s = 0 and every code is the zero of x's sign.
  * Arithmetic is IEEE with subnormals (numpy on the host keeps them).
"""

import numpy as np

from . import e4m3

GROUP = 128
FP8_MAX = np.float32(448.0)


def bf16_bits_to_f32(bits):
    """Widen raw bf16 bit patterns (uint16) to float32 exactly."""
    b = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
    return b.view(np.float32)


def _quantize_group_values(x, amax):
    """Codes and scale for values ``x`` (float32) sharing one ``amax``.

    ``amax`` broadcasts against ``x``.  Returns (codes uint8, scale float32).
    """
    amax = np.asarray(amax, dtype=np.float32)
    with np.errstate(divide="ignore", invalid="ignore"):
        s = (amax / FP8_MAX).astype(np.float32)
        q = (x / s).astype(np.float32)
    # all-zero group: every x is +-0; keep its sign, code is +-0.
    q = np.where(s == 0, x, q).astype(np.float32)
    return e4m3.encode(q), s


def quant_act_ref(a_bits):
    """1x128 dynamic activation quantization.

    a_bits: uint16 [M, K] bf16 bit patterns, K % 128 == 0.
    Returns codes uint8 [M, K] and scales float32 [M, K/128] (row-major).
    """
    a_bits = np.asarray(a_bits, dtype=np.uint16)
    M, K = a_bits.shape
    assert K % GROUP == 0
    x = bf16_bits_to_f32(a_bits).reshape(M, K // GROUP, GROUP)
    amax = np.max(np.abs(x), axis=2, keepdims=True)
    codes, s = _quantize_group_values(x, amax)
    return codes.reshape(M, K), s.reshape(M, K // GROUP)


def quant_weight_block_ref(w_bits, block_n=GROUP, block_k=GROUP):
    """128x128 block weight quantization.

    w_bits: uint16 [N, K] bf16 bit patterns, N % 128 == K % 128 == 0.
    Returns codes uint8 [N, K] and scales float32 [N/128, K/128].
    """
    w_bits = np.asarray(w_bits, dtype=np.uint16)
    N, K = w_bits.shape
    assert N % block_n == 0 and K % block_k == 0
    x = bf16_bits_to_f32(w_bits).reshape(N // block_n, block_n, K // block_k, block_k)
    amax = np.max(np.abs(x), axis=(1, 3), keepdims=True)
    codes, s = _quantize_group_values(x, amax)
    return codes.reshape(N, K), s.reshape(N // block_n, K // block_k)


def quant_tensor_ref(bits):
    """Per-tensor dynamic quantization: one amax, one scale for the tensor.

    bits: uint16 [R, C] bf16 bit patterns.  Returns codes uint8 [R, C] and
    the scale as a float32 array of shape (1,).
    """
    x = bf16_bits_to_f32(np.asarray(bits, dtype=np.uint16))
    amax = np.max(np.abs(x)) if x.size else np.float32(0)
    codes, s = _quantize_group_values(x, amax)
    return codes, np.asarray(s, dtype=np.float32).reshape(1)


def quant_tensor_with_amax_ref(bits, amax):
    """Per-tensor quantization of a slice of a tensor whose amax is known.

    Used to check sampled rows of a large tensor: the whole-tensor amax is
    computed by the caller over all of it, the codes here for ``bits`` only.
    """
    x = bf16_bits_to_f32(np.asarray(bits, dtype=np.uint16))
    codes, s = _quantize_group_values(x, np.float32(amax))
    return codes, np.asarray(s, dtype=np.float32).reshape(1)


def tensor_amax_ref(bits):
    """max |x| over a bf16 tensor, as float32 (exact)."""
    x = bf16_bits_to_f32(np.asarray(bits, dtype=np.uint16))
    return np.float32(np.max(np.abs(x))) if x.size else np.float32(0)


def quant_rows_ref(bits):
    """Dynamic per-row quantization: one amax and one scale per row.

    bits: uint16 [R, C] bf16 bit patterns.  Returns codes uint8 [R, C] and
    scales float32 [R].  Per token for activations, per output channel for
    weights ("[vLLM] FP8", scaling strategies: dynamic per-token; "FP8
    Quantization": channel-wise weight scales).
    """
    x = bf16_bits_to_f32(np.asarray(bits, dtype=np.uint16))
    R, C = x.shape
    if C == 0:
        return np.zeros((R, 0), dtype=np.uint8), np.zeros(R, dtype=np.float32)
    amax = np.max(np.abs(x), axis=1, keepdims=True)
    codes, s = _quantize_group_values(x, amax)
    return codes, s.reshape(R)


def quant_static_ref(bits, scale):
    """Static quantization with a calibrated scale: code = E4M3(fp32(x) / scale).

    ("[vLLM] FP8", scaling strategies: static per-tensor, scale computed in
    advance.)  bits: uint16 array of bf16 bit patterns; scale: one float32.
    Returns codes uint8 of the same shape.
    """
    x = bf16_bits_to_f32(np.asarray(bits, dtype=np.uint16))
    s = np.float32(np.asarray(scale, dtype=np.float32).reshape(-1)[0])
    with np.errstate(divide="ignore", invalid="ignore", over="ignore"):
        q = (x / s).astype(np.float32)
    return e4m3.encode(q)
