"""The device E4M3 encoder on every one of the 2^32 fp32 bit patterns (needs a gfx950 GPU).

The oracle's encoder (round to nearest, ties to the even code, saturating at
448, NaN to the NaN code, sign or-ed in) is a non-decreasing step function
of |x|, and the bit patterns of non-negative floats are ordered like their
values.  So the oracle's code of any pattern is fixed by 126 thresholds:
threshold c (1 <= c <= 126) is the smallest non-negative pattern the oracle
encodes to c or above, found here by binary search with the oracle itself
(a step function is checked at each threshold and its predecessor).  The
expected code of pattern p is then the number of thresholds <= (p & 0x7fffffff),
0x7F above the infinity pattern, with p's sign bit or-ed in; torch's
searchsorted evaluates that count on the device, chunk by chunk, beside the
HIP encoder's output (fp8_e4m3_encode_f32).
"""

import sys

import numpy as np
import pytest
import torch

from oracle import e4m3

pytestmark = pytest.mark.gpu

if torch.cuda.is_available():
    import fp8_w8a8_block_amd as fp8

INF_BITS = 0x7F800000


def oracle_code(bits):
    return int(e4m3.encode(np.array([bits], dtype=np.uint32).view(np.float32))[0])


def thresholds():
    """Smallest non-negative fp32 pattern the oracle encodes to >= c, c = 1..126."""
    out = []
    for c in range(1, 127):
        lo, hi = 0, INF_BITS                     # oracle_code(INF_BITS) = 126 >= c
        while lo < hi:
            mid = (lo + hi) // 2
            if oracle_code(mid) >= c:
                hi = mid
            else:
                lo = mid + 1
        assert oracle_code(lo) == c and oracle_code(lo - 1) == c - 1, c
        out.append(lo)
    return out


def test_encoder_every_fp32_pattern():
    thr = thresholds()
    assert all(a < b for a, b in zip(thr, thr[1:]))
    t = torch.tensor(thr, dtype=torch.int64, device="cuda")
    chunk = 1 << 28
    for start in range(0, 1 << 32, chunk):
        p = torch.arange(start, start + chunk, dtype=torch.int64, device="cuda")
        x = p.to(torch.int32).view(torch.float32)          # wraps to the same 32 bits
        got = fp8.encode_f32(x)
        mag = p & 0x7FFFFFFF
        want = torch.searchsorted(t, mag, right=True)
        want = torch.where(mag > INF_BITS, torch.full_like(want, 0x7F), want)
        want = (want | ((p >> 31) << 7)).to(torch.uint8)
        same = torch.equal(got, want)
        if not same:
            i = int(torch.nonzero(got != want)[0, 0])
            raise AssertionError(f"pattern {start + i:#010x}: device {int(got[i]):#04x} "
                                 f"oracle {int(want[i]):#04x}")
        if start % (1 << 30) == 0:
            print(f"patterns from {start:#010x}: equal", flush=True)
            sys.stdout.flush()
        del p, x, got, mag, want
    torch.cuda.synchronize()
