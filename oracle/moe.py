"""FP8 block-scaled MoE grouped GEMM (oracle).

TEST INFRASTRUCTURE ONLY -- not part of the product path.

What the pages describe: a fused mixture-of-experts layer gets an FP8
method of its own next to the linear one -- expert weights either quantized
offline and loaded as FP8, or quantized at load time ("[vLLM] FP8", the
config's dispatch and its table of methods); expert routing is named as a
bottleneck FP8 does not remove ("FP8 Quantization", section E); the experts
of an MoE are small matrices, and FP8-trained MoE weights ship as the
original checkpoint ("Quantization guide for serving: FP8, AWQ, GPTQ",
closing section).

What is computed (contiguous grouped layout): the rows of A are grouped by
expert, rows off[e] <= r < off[e + 1] going to expert e, and each expert has
its own block-quantized weight W_e [N, K] with 128 x 128 block scales:

    out[r, n] = sum_kb  sa[r, kb] * sw_e[n // 128, kb] * C_kb[r, n]
    C_kb[r, n] = sum_{k in block kb}  dec(qa[r, k]) * dec(qw_e[n, k])

i.e. the block-scaled GEMM of oracle.gemm applied to each expert's rows with
that expert's weight.  Readings (the pages give no MoE formula): the grouped
GEMM is the per-expert block GEMM; routing, the gate activation and the
weighted combine are separate steps and not part of it; the caller groups
the rows (tokens permuted by expert); rows outside every segment are not
produced (NaN here).
"""

import numpy as np

from . import gemm


def grouped_gemm_ref(a_codes, a_scales, w_codes, w_scales, offsets):
    """Grouped block-scaled GEMM, float64 [M, N] (NaN rows: in no segment).

    a_codes uint8 [M, K]; a_scales float32 [M, K/128];
    w_codes uint8 [E, N, K]; w_scales float32 [E, N/128, K/128];
    offsets int [E + 1], nondecreasing, offsets[0] >= 0, offsets[E] <= M.
    """
    a_codes = np.asarray(a_codes, dtype=np.uint8)
    w_codes = np.asarray(w_codes, dtype=np.uint8)
    M = a_codes.shape[0]
    E, N = w_codes.shape[0], w_codes.shape[1]
    off = [int(v) for v in offsets]
    assert len(off) == E + 1 and off[0] >= 0 and off[-1] <= M
    assert all(off[e] <= off[e + 1] for e in range(E))
    out = np.full((M, N), np.nan, dtype=np.float64)
    for e in range(E):
        lo, hi = off[e], off[e + 1]
        if hi > lo:
            out[lo:hi] = gemm.gemm_block_ref(a_codes[lo:hi], np.asarray(a_scales)[lo:hi],
                                             w_codes[e], np.asarray(w_scales)[e])
    return out
