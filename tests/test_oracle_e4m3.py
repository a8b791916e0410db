"""Pins for the oracle's E4M3 codec (CPU only).

Each test fixes the codec against something other than its own code: the
pages' printed format table, closed forms of the format, an independent
library decoder (torch.float8_e4m3fn), brute force nearest-value search and
the hand-worked midpoint example under tests/golden/.
"""

import json
import math
import os

import numpy as np
import pytest
import torch

from oracle import e4m3


def test_census():
    t = e4m3.decode_table()
    nan = np.isnan(t)
    assert sorted(np.nonzero(nan)[0].tolist()) == [0x7F, 0xFF]
    zeros = np.nonzero((t == 0) & ~nan)[0].tolist()
    assert sorted(zeros) == [0x00, 0x80]
    finite_nonzero = (~nan) & (t != 0)
    assert finite_nonzero.sum() == 252
    assert (finite_nonzero[:128]).sum() == 126 and (finite_nonzero[128:]).sum() == 126
    assert np.signbit(t[0x80]) and not np.signbit(t[0x00])


def test_printed_format_table(golden_dir):
    """The three printed maxima pin the bias / reserved-exponent reading."""
    g = json.load(open(os.path.join(golden_dir, "format_table.json")))
    for f in g["formats"]:
        assert e4m3.closed_form_max(f["exp_bits"], f["man_bits"], f["ieee_reserved_top"]) == f["max"]
    # the IEEE-style reading of E4M3 would give 240, not the printed 448
    assert e4m3.closed_form_max(4, 3, True) == 240.0
    t = e4m3.decode_table()
    assert t[0x7E] == 448.0 and t[0xFE] == -448.0
    assert np.nanmax(t) == 448.0 and np.nanmin(t) == -448.0


def test_anchor_values():
    t = e4m3.decode_table()
    assert t[0x01] == 2.0 ** -9
    assert t[0x07] == 7 * 2.0 ** -9
    assert t[0x08] == 2.0 ** -6
    assert t[0x38] == 1.0
    assert t[0x77] == 240.0
    assert t[0x78] == 256.0
    assert t[0x7D] == 416.0


def test_decode_matches_library_table():
    """torch.float8_e4m3fn is an independent implementation of the same format."""
    codes = torch.arange(256, dtype=torch.int32).to(torch.uint8)
    lib = codes.view(torch.float8_e4m3fn).to(torch.float64).numpy()
    ours = e4m3.decode_table()
    both_nan = np.isnan(lib) & np.isnan(ours)
    assert np.all(both_nan | (lib == ours))
    assert np.array_equal(np.signbit(lib[~both_nan]), np.signbit(ours[~both_nan]))


def test_bitfield_reinterpretation():
    """Normal codes equal the float32 built from the same fields with bias 7."""
    t = e4m3.decode_table()
    for c in range(256):
        s, e, m = c >> 7, (c >> 3) & 15, c & 7
        if e == 0 or (e == 15 and m == 7):
            continue
        bits = (s << 31) | ((e - 7 + 127) << 23) | (m << 20)
        v = np.array([bits], dtype=np.uint32).view(np.float32)[0]
        assert float(v) == t[c]


def test_order_is_code_order():
    t = e4m3.decode_table()
    pos = t[:0x7F]
    assert np.all(np.diff(pos) > 0)


def test_round_trip_all_codes():
    t = e4m3.decode_table()
    codes = np.array([c for c in range(256) if c not in (0x7F, 0xFF)], dtype=np.uint8)
    assert np.array_equal(e4m3.encode(t[codes]), codes)
    assert np.array_equal(e4m3.encode(t[codes].astype(np.float32)), codes)


def test_midpoints_tie_to_even():
    t = e4m3.decode_table()
    n = 0
    for c in range(0x7E):
        mid = (t[c] + t[c + 1]) / 2
        even = c if c % 2 == 0 else c + 1
        assert e4m3.encode(np.array([mid]))[0] == even
        assert e4m3.encode(np.array([-mid]))[0] == even | 0x80
        # just off the midpoint goes to the nearer neighbour
        assert e4m3.encode(np.array([np.nextafter(mid, -np.inf)]))[0] == c
        assert e4m3.encode(np.array([np.nextafter(mid, np.inf)]))[0] == c + 1
        n += 1
    assert n == 126


def test_saturation_and_nan():
    enc = lambda v: int(e4m3.encode(np.array([v], dtype=np.float64))[0])
    assert enc(448.0) == 0x7E
    assert enc(449.0) == 0x7E
    assert enc(464.0) == 0x7E
    assert enc(1e30) == 0x7E
    assert enc(math.inf) == 0x7E
    assert enc(-math.inf) == 0xFE
    assert enc(-500.0) == 0xFE
    assert enc(math.nan) == 0x7F
    assert enc(-math.nan) == 0xFF
    assert enc(0.0) == 0x00 and enc(-0.0) == 0x80
    assert enc(-1e-30) == 0x80


def _brute_encode(v):
    """Nearest finite value by full scan, ties to even code (pure Python)."""
    t = e4m3.decode_table()
    a = min(abs(v), 448.0)
    best, bestd = None, None
    for c in range(0x7F):
        d = abs(t[c] - a)
        if best is None or d < bestd or (d == bestd and c % 2 == 0):
            best, bestd = c, d
    return best | (0x80 if math.copysign(1.0, v) < 0 else 0)


def test_brute_force_random():
    rng = np.random.default_rng(7)
    # log-uniform magnitudes across and beyond the code range, float32 values
    mags = np.exp(rng.uniform(np.log(2.0 ** -12), np.log(600.0), 3000)).astype(np.float32)
    vals = mags * np.where(rng.integers(0, 2, mags.size) == 1, -1, 1).astype(np.float32)
    ours = e4m3.encode(vals)
    for v, c in zip(vals.tolist(), ours.tolist()):
        assert c == _brute_encode(v), v


def test_library_encoder_in_range():
    """torch's float -> float8_e4m3fn cast rounds to nearest even; agree in range."""
    rng = np.random.default_rng(8)
    v = (rng.standard_normal(200000) * 50).astype(np.float32)
    v = np.clip(v, -448, 448)
    lib = torch.from_numpy(v).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(lib, e4m3.encode(v))


def test_monotone_and_half_ulp():
    rng = np.random.default_rng(9)
    x = np.sort(np.exp(rng.uniform(np.log(2.0 ** -11), np.log(448.0), 100000)))
    c = e4m3.encode(x)
    assert np.all(np.diff(c.astype(np.int64)) >= 0)
    d = e4m3.decode(c)
    # spacing at the decoded value's binade: 2**-9 below 2**-6, else value/8 floor
    _, e = np.frexp(np.maximum(np.abs(d), np.abs(x)))
    ulp = np.where(np.maximum(np.abs(d), np.abs(x)) < 2.0 ** -6, 2.0 ** -9, np.ldexp(1.0, e - 4))
    assert np.all(np.abs(d - x) <= ulp / 2)


def test_worked_group_codes(golden_dir):
    g = json.load(open(os.path.join(golden_dir, "e4m3_worked_group.json")))
    xs = np.array([c["x"] for c in g["cases"]], dtype=np.float64)
    want = np.array([int(c["code"], 16) for c in g["cases"]], dtype=np.uint8)
    assert np.array_equal(e4m3.encode(xs), want)
