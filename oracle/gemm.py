"""fp64 reference GEMM on the FP8 operands (oracle).

TEST INFRASTRUCTURE ONLY -- not part of the product path.

The W8A8 linear layer multiplies FP8 activations by FP8 weights with a wide
accumulator ("FP8 and FP4: Throughput Needs Scaling", kernel-caveat card:
low-bit operands into the matrix unit, high-precision accumulation; "FP8
Quantization", section C: weights and activations both lowered).  With
block scales ("[vLLM] FP8", block quantization: one scale per 128x128
weight block; 1x128 dynamic activation groups from the scaling-strategy
list) the value of out[m, n] is

    out[m, n] = sum_kb  sa[m, kb] * sw[n // 128, kb] * C_kb[m, n]
    C_kb[m, n] = sum_{k in block kb}  dec(qa[m, k]) * dec(qw[n, k])

with W stored [N, K] (out = A . W^T).  Per-tensor scales give
out = sA * sW * sum_k dec(qa[m, k]) * dec(qw[n, k]); per-row scales (one per
token, one per output channel; "[vLLM] FP8", scaling strategies, and "FP8
Quantization", channel-wise weights) give
out[m, n] = sA[m] * sW[n] * sum_k dec(qa[m, k]) * dec(qw[n, k]).

Exactness: every decoded code is a multiple of 2**-9 with magnitude <= 448,
so each product is a multiple of 2**-18 below 2**18 and a 128-term block sum
fits in 43 bits: C_kb is exact in fp64 whatever the summation order (a BLAS
matmul serves as the summation step).  A full-K per-tensor sum up to
K = 2**15 needs at most 51 bits and is exact as well.  The only rounding is
the fp64 scale-and-add, about 1e-16 relative.
"""

import numpy as np

from . import e4m3

GROUP = 128


def gemm_block_ref_rows(a_codes, a_scales, w_codes, w_scale_rows):
    """Block-scaled reference where each W row carries its own scale row.

    a_codes: uint8 [M, K]; a_scales: float32 [M, K/128]
    w_codes: uint8 [N, K]; w_scale_rows: float32 [N, K/128] (the scale of
    the 128x128 block that row n falls in, repeated per row).
    Returns float64 [M, N].
    """
    a_codes = np.asarray(a_codes, dtype=np.uint8)
    w_codes = np.asarray(w_codes, dtype=np.uint8)
    M, K = a_codes.shape
    N, K2 = w_codes.shape
    assert K == K2 and K % GROUP == 0
    KB = K // GROUP
    a = e4m3.decode(a_codes)
    w = e4m3.decode(w_codes)
    sa = np.asarray(a_scales, dtype=np.float64).reshape(M, KB)
    sw = np.asarray(w_scale_rows, dtype=np.float64).reshape(N, KB)
    out = np.zeros((M, N), dtype=np.float64)
    for kb in range(KB):
        ks = slice(kb * GROUP, (kb + 1) * GROUP)
        c_kb = a[:, ks] @ w[:, ks].T                     # exact block sum
        out += (sa[:, kb:kb + 1] * sw[None, :, kb]) * c_kb
    return out


def gemm_block_ref(a_codes, a_scales, w_codes, w_scales):
    """Block-scaled reference with W scales given per 128x128 block [N/128, K/128]."""
    w_scales = np.asarray(w_scales, dtype=np.float32)
    return gemm_block_ref_rows(a_codes, a_scales, w_codes,
                               np.repeat(w_scales, GROUP, axis=0))


def gemm_tensor_ref(a_codes, a_scale, w_codes, w_scale):
    """Per-tensor-scaled reference: sA * sW * (dec(A) . dec(W)^T), float64 [M, N]."""
    a = e4m3.decode(np.asarray(a_codes, dtype=np.uint8))
    w = e4m3.decode(np.asarray(w_codes, dtype=np.uint8))
    sa = float(np.asarray(a_scale, dtype=np.float32).reshape(-1)[0])
    sw = float(np.asarray(w_scale, dtype=np.float32).reshape(-1)[0])
    return (sa * sw) * (a @ w.T)


def gemm_rows_ref(a_codes, a_row_scales, w_codes, w_row_scales):
    """Per-row-scaled reference, float64 [M, N].

    a_row_scales: float32, M values (one per activation row) or one value
    for all rows; w_row_scales: float32, N values (one per weight row, i.e.
    per output column) or one value.  out[m, n] = sa[m] * sw[n] * S[m, n],
    S the exact full-K sum of decoded products.
    """
    a = e4m3.decode(np.asarray(a_codes, dtype=np.uint8))
    w = e4m3.decode(np.asarray(w_codes, dtype=np.uint8))
    M, N = a.shape[0], w.shape[0]
    sa = np.asarray(a_row_scales, dtype=np.float32).astype(np.float64).reshape(-1)
    sw = np.asarray(w_row_scales, dtype=np.float32).astype(np.float64).reshape(-1)
    sa = np.broadcast_to(sa, (M,)) if sa.size == 1 else sa
    sw = np.broadcast_to(sw, (N,)) if sw.size == 1 else sw
    assert sa.shape == (M,) and sw.shape == (N,)
    return (sa[:, None] * sw[None, :]) * (a @ w.T)
