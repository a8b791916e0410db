"""Pins for the oracle's dynamic quantizers (CPU only).

Pinned by: the hand-worked amax=448 group (tests/golden), the amax invariant
over every positive finite bf16 amax, power-of-two and sign metamorphic
relations, the format's error bound, and an independent pure-Python
brute-force quantizer on small tensors (fp64 division rounded once to fp32,
which equals the fp32 quotient because 53 >= 2*24 + 2).
"""

import json
import math
import os

import numpy as np
import pytest

from oracle import e4m3, quant
from workloads import synth


def f32_bits_to_bf16(vals):
    return synth.f32_to_bf16_bits(np.asarray(vals, dtype=np.float32))


def test_worked_group(golden_dir):
    g = json.load(open(os.path.join(golden_dir, "e4m3_worked_group.json")))
    xs = [c["x"] for c in g["cases"]]
    want = [int(c["code"], 16) for c in g["cases"]]
    row = np.zeros(128, dtype=np.float32)
    row[: len(xs)] = xs
    bits = f32_bits_to_bf16(row)[None, :]
    assert np.array_equal(quant.bf16_bits_to_f32(bits)[0, : len(xs)], np.array(xs, dtype=np.float32))
    codes, s = quant.quant_act_ref(bits)
    assert s.shape == (1, 1) and s[0, 0] == np.float32(g["scale"])
    assert codes[0, : len(xs)].tolist() == want
    assert np.all(codes[0, len(xs):] == 0)


def _brute_group(vals_f32):
    """Independent per-group quantizer in pure Python floats."""
    amax = max(abs(float(v)) for v in vals_f32)
    s = float(np.float32(amax / 448.0))           # fp64 divide, one rounding to fp32
    out = []
    for v in vals_f32:
        v = float(v)
        if s == 0.0:
            q = v
        else:
            q = float(np.float32(v / s))
        # nearest by scan, ties to even
        t = e4m3.decode_table()
        a = min(abs(q), 448.0)
        best, bd = 0, None
        for c in range(0x7F):
            d = abs(t[c] - a)
            if bd is None or d < bd or (d == bd and c % 2 == 0):
                best, bd = c, d
        out.append(best | (0x80 if math.copysign(1.0, q) < 0 else 0))
    return out, np.float32(s)


def test_act_brute_force_small():
    rng = np.random.default_rng(11)
    x = rng.standard_normal((3, 256)).astype(np.float32) * np.float32(3)
    x[0, 5] = 70.0
    x[1, 128:256] = 0.0
    x[1, 130] = -0.0
    bits = f32_bits_to_bf16(x)
    codes, s = quant.quant_act_ref(bits)
    xf = quant.bf16_bits_to_f32(bits)
    for m in range(3):
        for g in range(2):
            want, ws = _brute_group(xf[m, g * 128:(g + 1) * 128])
            assert codes[m, g * 128:(g + 1) * 128].tolist() == want
            assert s[m, g] == ws


def test_weight_brute_force_small():
    rng = np.random.default_rng(12)
    w = rng.standard_normal((128, 256)).astype(np.float32) * np.float32(0.02)
    w[3, 200] = 1.5
    bits = f32_bits_to_bf16(w)
    codes, s = quant.quant_weight_block_ref(bits)
    assert s.shape == (1, 2)
    wf = quant.bf16_bits_to_f32(bits)
    for kb in range(2):
        blk = wf[:, kb * 128:(kb + 1) * 128]
        want, ws = _brute_group(blk.reshape(-1))
        assert s[0, kb] == ws
        assert codes[:, kb * 128:(kb + 1) * 128].reshape(-1).tolist() == want


def test_tensor_brute_force_small():
    rng = np.random.default_rng(13)
    x = (rng.standard_normal((4, 128)) * 2).astype(np.float32)
    bits = f32_bits_to_bf16(x)
    codes, s = quant.quant_tensor_ref(bits)
    want, ws = _brute_group(quant.bf16_bits_to_f32(bits).reshape(-1))
    assert s[0] == ws
    assert codes.reshape(-1).tolist() == want


def test_amax_invariant_all_bf16_amax():
    """Every group's amax element lands on +-448's code, for every bf16 amax."""
    bits = synth.edge_activations()["all_amax"]
    codes, s = quant.quant_act_ref(bits)
    x = quant.bf16_bits_to_f32(bits)
    G = x.reshape(-1, 128)
    C = codes.reshape(-1, 128)
    S = s.reshape(-1)
    amax = np.abs(G).max(axis=1)
    nz = amax > 0
    assert np.all(S[~nz] == 0)
    assert np.all(S[nz] > 0)                      # no scale underflows to 0
    at_max = np.abs(G) == amax[:, None]
    assert np.all(((C & 0x7F) == 0x7E)[at_max & nz[:, None]])
    # amax / s stays inside 448 * (1 +- 2**-23) for normal s, and near 448 for subnormal s
    r = amax[nz].astype(np.float64) / S[nz].astype(np.float64)
    normal = S[nz] >= np.float32(2.0 ** -126)
    assert np.all(np.abs(r[normal] / 448.0 - 1) <= 2.0 ** -23)
    assert np.all((r[~normal] > 447.0) & (r[~normal] < 449.0))
    assert (~normal).sum() > 1000


def test_power_of_two_metamorphic():
    rng = np.random.default_rng(14)
    x = rng.standard_normal((8, 512)).astype(np.float32)
    bits = f32_bits_to_bf16(x)
    c0, s0 = quant.quant_act_ref(bits)
    for j in (-20, -3, 1, 7, 30):
        xs = quant.bf16_bits_to_f32(bits) * np.float32(2.0 ** j)
        c1, s1 = quant.quant_act_ref(f32_bits_to_bf16(xs))
        assert np.array_equal(c0, c1)
        assert np.array_equal(s1, (s0 * np.float32(2.0 ** j)).astype(np.float32))


def test_sign_symmetry():
    rng = np.random.default_rng(15)
    bits = f32_bits_to_bf16(rng.standard_normal((4, 384)).astype(np.float32))
    c0, s0 = quant.quant_act_ref(bits)
    c1, s1 = quant.quant_act_ref(bits ^ np.uint16(0x8000))
    assert np.array_equal(c1, c0 ^ np.uint8(0x80))
    assert np.array_equal(s0, s1)


def test_error_bound():
    rng = np.random.default_rng(16)
    x = rng.standard_normal((16, 1024)).astype(np.float32)
    x[:, 7] *= 50
    bits = f32_bits_to_bf16(x)
    codes, s = quant.quant_act_ref(bits)
    xf = quant.bf16_bits_to_f32(bits).astype(np.float64)
    sd = np.repeat(s.astype(np.float64), 128, axis=1)
    d = e4m3.decode(codes) * sd
    err = np.abs(xf - d)
    normal_code = (codes & 0x78) != 0
    slack = 2.0 ** -23 * np.abs(xf) + 1e-300
    assert np.all(err[normal_code] <= 2.0 ** -4 * np.abs(xf[normal_code]) + slack[normal_code])
    assert np.all(err[~normal_code] <= 2.0 ** -10 * sd[~normal_code] * (1 + 2.0 ** -20) + slack[~normal_code])


def test_zero_groups_and_sign_of_zero():
    e = synth.edge_activations()
    c, s = quant.quant_act_ref(e["zeros"])
    assert np.all(c == 0) and np.all(s == 0)
    c, s = quant.quant_act_ref(e["negzero"])
    assert np.all(c == 0x80) and np.all(s == 0)


def test_block_independence():
    rng = np.random.default_rng(17)
    w = (rng.standard_normal((256, 384)) * 0.02).astype(np.float32)
    b0 = f32_bits_to_bf16(w)
    c0, s0 = quant.quant_weight_block_ref(b0)
    w2 = w.copy()
    w2[130, 300] = 5.0                                  # block (1, 2)
    c1, s1 = quant.quant_weight_block_ref(f32_bits_to_bf16(w2))
    changed = s0 != s1
    assert changed.sum() == 1 and changed[1, 2]
    diff = (c0 != c1).reshape(2, 128, 3, 128).any(axis=(1, 3))
    assert diff.sum() == 1 and diff[1, 2]


def test_tensor_with_amax_matches_full():
    rng = np.random.default_rng(18)
    bits = f32_bits_to_bf16(rng.standard_normal((64, 256)).astype(np.float32))
    c, s = quant.quant_tensor_ref(bits)
    amax = quant.tensor_amax_ref(bits)
    c2, s2 = quant.quant_tensor_with_amax_ref(bits[10:20], amax)
    assert np.array_equal(c2, c[10:20]) and s2[0] == s[0]


def test_true_division_adversarial(golden_dir):
    """Pairs where x * (1/s) and x / s give different codes (tests/golden)."""
    pairs = json.load(open(os.path.join(golden_dir, "div_adversarial.json")))["pairs_amax_bits_x_bits"]
    rows = np.zeros((len(pairs), 128), dtype=np.uint16)
    for i, (ab, xb) in enumerate(pairs):
        rows[i, 0] = ab
        rows[i, 1] = xb
    codes, s = quant.quant_act_ref(rows)
    xf = quant.bf16_bits_to_f32(rows)
    for i in range(len(pairs)):
        want, ws = _brute_group(xf[i, :2])
        assert s[i, 0] == ws
        assert codes[i, :2].tolist() == want, pairs[i]


def test_rows_brute_force_small():
    # per-row quantization: each row is its own group (brute force per row)
    rng = np.random.default_rng(14)
    x = (rng.standard_normal((5, 384)) * 1.5).astype(np.float32)
    x[1, 17] = 99.0
    x[3, :] = 0.0
    x[3, 5] = -0.0
    bits = f32_bits_to_bf16(x)
    codes, s = quant.quant_rows_ref(bits)
    assert codes.shape == (5, 384) and s.shape == (5,)
    xf = quant.bf16_bits_to_f32(bits)
    for r in range(5):
        want, ws = _brute_group(xf[r])
        assert s[r] == ws
        assert codes[r].tolist() == want


def test_rows_special_cases_reduce_to_pinned_quantizers():
    rng = np.random.default_rng(15)
    x = f32_bits_to_bf16((rng.standard_normal((6, 128)) * 3).astype(np.float32))
    # K = 128: one row is one 1x128 group
    c_rows, s_rows = quant.quant_rows_ref(x)
    c_act, s_act = quant.quant_act_ref(x)
    assert np.array_equal(c_rows, c_act) and np.array_equal(s_rows, s_act[:, 0])
    # one row: the whole tensor
    y = f32_bits_to_bf16((rng.standard_normal((1, 640)) * 0.1).astype(np.float32))
    c1, s1 = quant.quant_rows_ref(y)
    c2, s2 = quant.quant_tensor_ref(y)
    assert np.array_equal(c1, c2) and s1[0] == s2[0]


def test_static_equals_dynamic_at_the_dynamic_scale():
    rng = np.random.default_rng(16)
    x = f32_bits_to_bf16((rng.standard_normal((7, 256)) * 2).astype(np.float32))
    c_dyn, s_dyn = quant.quant_tensor_ref(x)
    assert np.array_equal(quant.quant_static_ref(x, s_dyn), c_dyn)


def test_static_brute_force_and_saturation():
    rng = np.random.default_rng(17)
    xf = (rng.standard_normal(300) * 4).astype(np.float32)
    bits = f32_bits_to_bf16(xf)
    xf = quant.bf16_bits_to_f32(bits)
    s = np.float32(0.0123)           # values up to ~16 / 0.0123 = 1300: many saturate
    got = quant.quant_static_ref(bits, s)
    t = e4m3.decode_table()
    for v, c in zip(xf.tolist(), got.tolist()):
        q = float(np.float32(v / float(s)))          # fp64 divide rounded once to fp32
        a = min(abs(q), 448.0)
        best, bd = 0, None
        for k in range(0x7F):
            d = abs(t[k] - a)
            if bd is None or d < bd or (d == bd and k % 2 == 0):
                best, bd = k, d
        assert c == (best | (0x80 if math.copysign(1.0, q) < 0 else 0))
    assert np.any(got & 0x7F == 0x7E)                 # some saturated to 448
