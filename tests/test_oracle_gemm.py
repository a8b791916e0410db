"""Pins for the oracle's fp64 GEMM and tolerance check (CPU only).

Pinned by: exact rational brute force (Fractions) on tiny shapes with M != N
so that a transposed operand or a wrong scale index fails; closed forms
(all-ones codes, identity blocks); a dequantize-then-single-matmul
cross-check; and the tolerance checker against torch's bf16 rounding and a
planted error.
"""

from fractions import Fraction

import numpy as np
import torch

from oracle import e4m3, gemm, tolerance


def _random_operands(rng, M, N, K):
    ok = np.array([c for c in range(256) if c not in (0x7F, 0xFF)], dtype=np.uint8)
    a = rng.choice(ok, size=(M, K))
    w = rng.choice(ok, size=(N, K))
    sa = (rng.uniform(0.1, 3.0, (M, K // 128))).astype(np.float32)
    sw = (rng.uniform(0.001, 0.2, (N // 128, K // 128))).astype(np.float32)
    return a, sa, w, sw


def _exact(a, sa, w, sw):
    t = e4m3.decode_table()
    M, K = a.shape
    N = w.shape[0]
    F = [Fraction(float(v)) if np.isfinite(v) else None for v in t]
    out = [[Fraction(0)] * N for _ in range(M)]
    mag = np.zeros((M, N))
    for m in range(M):
        for n in range(N):
            acc = Fraction(0)
            for kb in range(K // 128):
                blk = sum(F[a[m, k]] * F[w[n, k]] for k in range(kb * 128, (kb + 1) * 128))
                term = Fraction(float(sa[m, kb])) * Fraction(float(sw[n // 128, kb])) * blk
                acc += term
                mag[m, n] += abs(float(term))
            out[m][n] = acc
    return out, mag


def test_exact_brute_force_block():
    rng = np.random.default_rng(21)
    a, sa, w, sw = _random_operands(rng, 3, 256, 256)
    ref = gemm.gemm_block_ref(a, sa, w, sw)
    assert ref.shape == (3, 256)
    ex, mag = _exact(a, sa, w, sw)
    for m in range(3):
        for n in range(256):
            e = float(ex[m][n])
            # two fp64 roundings per K-block (the scale product is exact)
            assert abs(ref[m, n] - e) <= 4 * 2.0 ** -53 * mag[m, n]


def test_exact_brute_force_tensor():
    rng = np.random.default_rng(22)
    a, _, w, _ = _random_operands(rng, 2, 128, 384)
    sa = np.array([0.37], dtype=np.float32)
    sw = np.array([0.0041], dtype=np.float32)
    ref = gemm.gemm_tensor_ref(a, sa, w, sw)
    t = e4m3.decode_table()
    for m in range(2):
        for n in range(0, 128, 7):
            s = sum(Fraction(float(t[a[m, k]])) * Fraction(float(t[w[n, k]])) for k in range(384))
            e = float(Fraction(float(sa[0])) * Fraction(float(sw[0])) * s)
            assert abs(ref[m, n] - e) <= 2 * np.spacing(abs(e) + 1e-300)


def test_dequantize_then_single_matmul():
    rng = np.random.default_rng(23)
    a, sa, w, sw = _random_operands(rng, 17, 384, 512)
    ref = gemm.gemm_block_ref(a, sa, w, sw)
    ad = e4m3.decode(a) * np.repeat(sa.astype(np.float64), 128, axis=1)
    wd = e4m3.decode(w) * np.repeat(np.repeat(sw.astype(np.float64), 128, axis=0), 128, axis=1)
    alt = ad @ wd.T
    scale = np.abs(ad) @ np.abs(wd).T
    assert np.all(np.abs(ref - alt) <= 1e-13 * scale + 1e-300)


def test_closed_form_all_ones():
    M, N, K = 4, 256, 384
    a = np.full((M, K), 0x38, dtype=np.uint8)
    w = np.full((N, K), 0x38, dtype=np.uint8)
    rng = np.random.default_rng(24)
    sa = rng.uniform(0.5, 2, (M, K // 128)).astype(np.float32)
    sw = rng.uniform(0.5, 2, (N // 128, K // 128)).astype(np.float32)
    ref = gemm.gemm_block_ref(a, sa, w, sw)
    for m in range(M):
        for n in range(N):
            want = sum(128.0 * float(sa[m, kb]) * float(sw[n // 128, kb]) for kb in range(K // 128))
            assert abs(ref[m, n] - want) <= 1e-12 * abs(want)


def test_closed_form_identity_blocks():
    rng = np.random.default_rng(25)
    K = 256
    a, sa, _, _ = _random_operands(rng, 5, 128, K)
    w = np.zeros((K, K), dtype=np.uint8)
    w[np.arange(K), np.arange(K)] = 0x38
    sw = np.ones((K // 128, K // 128), dtype=np.float32)
    ref = gemm.gemm_block_ref(a, sa, w, sw)
    deq = e4m3.decode(a) * np.repeat(sa.astype(np.float64), 128, axis=1)
    assert np.array_equal(ref, deq)


def test_orientation_and_scale_index():
    """A planted transpose or wrong W-scale row index changes the result."""
    rng = np.random.default_rng(26)
    a, sa, w, sw = _random_operands(rng, 2, 256, 256)
    ref = gemm.gemm_block_ref(a, sa, w, sw)
    wrong_scale = gemm.gemm_block_ref(a, sa, w, sw[::-1])
    assert not np.allclose(ref, wrong_scale)
    t = e4m3.decode_table()
    m, n = 1, 200
    direct = sum(float(sa[m, kb]) * float(sw[n // 128, kb]) *
                 sum(t[a[m, k]] * t[w[n, k]] for k in range(kb * 128, kb * 128 + 128))
                 for kb in range(2))
    assert abs(ref[m, n] - direct) <= 1e-12 * abs(direct)


def test_bf16_rne_matches_torch():
    rng = np.random.default_rng(27)
    v = (rng.standard_normal(100000) * np.exp(rng.uniform(-20, 20, 100000))).astype(np.float32)
    lib = torch.from_numpy(v).to(torch.bfloat16).to(torch.float64).numpy()
    assert np.array_equal(tolerance.bf16_rne(v.astype(np.float64)), lib)


def test_tolerance_gate_and_floor():
    rng = np.random.default_rng(28)
    ref = rng.standard_normal((64, 64)) * 3
    rounded = tolerance.bf16_rne(ref)
    bits = torch.from_numpy(rounded.astype(np.float32)).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    r = tolerance.check(bits, ref)
    assert r["ok"] and r["frac_equal_rne"] == 1.0
    assert r["maxabs_over_rms"] == r["floor_maxabs_over_rms"]
    # planted error: one output off by 5% of rms fails the elementwise gate
    bad = rounded.copy()
    bad[3, 4] += 0.05 * tolerance.rms(ref) + 4 * tolerance.bf16_ulp(bad[3, 4])
    bbits = torch.from_numpy(bad.astype(np.float32)).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert not tolerance.check(bbits, ref)["ok"]
    # a uniformly scaled output fails the Frobenius bound
    sc = tolerance.bf16_rne(ref * 1.01)
    sbits = torch.from_numpy(sc.astype(np.float32)).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert not tolerance.check(sbits, ref)["frob_ok"]


def test_exact_brute_force_rows():
    # per-token x per-channel scales; M != N so a swapped scale vector fails
    rng = np.random.default_rng(23)
    a, _, w, _ = _random_operands(rng, 3, 128, 256)
    sa = rng.uniform(0.1, 2.0, 3).astype(np.float32)
    sw = rng.uniform(0.001, 0.1, 128).astype(np.float32)
    ref = gemm.gemm_rows_ref(a, sa, w, sw)
    assert ref.shape == (3, 128)
    t = e4m3.decode_table()
    for m in range(3):
        for n in range(0, 128, 5):
            s = sum(Fraction(float(t[a[m, k]])) * Fraction(float(t[w[n, k]])) for k in range(256))
            e = float(Fraction(float(sa[m])) * Fraction(float(sw[n])) * s)
            assert abs(ref[m, n] - e) <= 2 * np.spacing(abs(e) + 1e-300)


def test_rows_broadcast_is_per_tensor():
    rng = np.random.default_rng(24)
    a, _, w, _ = _random_operands(rng, 4, 256, 384)
    sa = np.array([0.25], dtype=np.float32)
    sw = np.array([0.0625], dtype=np.float32)
    assert np.array_equal(gemm.gemm_rows_ref(a, sa, w, sw), gemm.gemm_tensor_ref(a, sa, w, sw))
