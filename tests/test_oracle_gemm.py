"""Pins for the oracle's fp64 GEMM and tolerance check (CPU only).

Pinned by: exact rational brute force (Fractions) on tiny shapes with M != N
so that a transposed operand or a wrong scale index fails; closed forms
(all-ones codes, identity blocks); a dequantize-then-single-matmul
cross-check; and the tolerance checker against torch's bf16 rounding, torch's
bf16 nextafter (ulp distance), fp32 accumulations simulated in several orders
(the accumulation bound), and planted errors (5% of rms, a 1% scale, 2 ulps
on a large output, a near-zero output beyond its bound).
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


def _bits_of(values):
    return torch.from_numpy(np.asarray(values, dtype=np.float32)).to(torch.bfloat16).view(
        torch.int16).numpy().view(np.uint16)


def test_tolerance_gate_and_floor():
    rng = np.random.default_rng(28)
    ref = rng.standard_normal((64, 64)) * 3
    rounded = tolerance.bf16_rne(ref)
    bits = _bits_of(rounded)
    r = tolerance.check(bits, ref, 0.0)
    assert r["ok"] and r["frac_equal_rne"] == 1.0 and r["max_ulp"] == 0
    assert r["maxabs_over_rms"] == r["floor_maxabs_over_rms"]
    # planted error: one output off by 5% of rms fails the elementwise gate
    bad = rounded.copy()
    bad[3, 4] += 0.05 * tolerance.rms(ref) + 4 * tolerance.bf16_ulp(bad[3, 4])
    assert not tolerance.check(_bits_of(bad), ref, 0.0)["ok"]
    # a uniformly scaled output fails the Frobenius bound
    sc = tolerance.bf16_rne(ref * 1.01)
    assert not tolerance.check(_bits_of(sc), ref, 0.0)["frob_ok"]


def test_ulp_distance_counts_bf16_steps():
    # consecutive bf16 values (torch.nextafter in bf16) are one step apart,
    # across binade edges, subnormals and zero; +0 and -0 are the same point
    rng = np.random.default_rng(31)
    v = (rng.standard_normal(20000) * np.exp(rng.uniform(-85, 80, 20000))).astype(np.float32)
    v = np.concatenate([v, [1.0, 2.0, -2.0, 2.0 ** -126, 2.0 ** -133, 0.0, -0.0]]).astype(np.float32)
    t = torch.from_numpy(v).to(torch.bfloat16)
    up = torch.nextafter(t, torch.full_like(t, float("inf")))
    up2 = torch.nextafter(up, torch.full_like(t, float("inf")))
    ref = t.to(torch.float64).numpy()
    assert np.all(tolerance.ulp_distance(up.view(torch.int16).numpy().view(np.uint16), ref) == 1)
    assert np.all(tolerance.ulp_distance(up2.view(torch.int16).numpy().view(np.uint16), ref) == 2)
    z = np.array([0x0000, 0x8000, 0x0001, 0x8001], dtype=np.uint16)
    assert tolerance.ulp_distance(z, np.zeros(4)).tolist() == [0, 0, 1, 1]
    assert tolerance.ulp_distance(np.array([0x0001], dtype=np.uint16),
                                  np.array([-(2.0 ** -133)])).tolist() == [2]


def test_abs_reference_is_sum_of_magnitudes():
    # T (the reference on absolute codes and scales) equals the brute-force
    # sum of |scale * product| that _exact accumulates beside the exact value
    rng = np.random.default_rng(32)
    a, sa, w, sw = _random_operands(rng, 3, 256, 256)
    sa[0, 1] = -sa[0, 1]
    T = gemm.gemm_block_ref(tolerance.abs_codes(a), np.abs(sa), tolerance.abs_codes(w), np.abs(sw))
    _, mag = _exact(a, sa, w, sw)
    # mag sums |sa sw blk| per block; T sums |sa sw| sum|products| >= it
    assert np.all(T >= mag * (1 - 1e-12))
    t = e4m3.decode_table()
    for m, n in ((0, 0), (2, 255), (1, 130)):
        direct = sum(abs(float(sa[m, k // 128]) * float(sw[n // 128, k // 128]) *
                         t[a[m, k]] * t[w[n, k]]) for k in range(256))
        assert abs(T[m, n] - direct) <= 1e-12 * direct


def _fp32_block_gemm(a, sa, w, sw, order_rng):
    """One fp32 accumulation of the block-scaled GEMM: each 128-term block
    sum in a random order in float32, scale product in float32, fold with a
    float32 multiply-add rounded once (computed in float64, then rounded)."""
    t = e4m3.decode_table()
    M, K = a.shape
    N = w.shape[0]
    out = np.zeros((M, N), dtype=np.float32)
    for kb in range(K // 128):
        ks = np.arange(kb * 128, kb * 128 + 128)
        P = np.zeros((M, N), dtype=np.float32)
        for k in order_rng.permutation(ks):
            P = (P + (t[a[:, k]][:, None] * t[w[:, k]][None, :]).astype(np.float32)).astype(np.float32)
        s = (sa[:, kb][:, None] * np.repeat(sw[:, kb], 128)[None, :]).astype(np.float32)
        out = (s.astype(np.float64) * P.astype(np.float64) + out.astype(np.float64)).astype(np.float32)
    return out


def test_accumulation_bound_holds_for_fp32_sums():
    # fp32 accumulations in several orders stay inside B; the bound is at
    # least the error they make (a dropped factor or a 2**-24 unit for a
    # truncating unit would not be conservative, the simulated sums are RNE)
    rng = np.random.default_rng(33)
    a, sa, w, sw = _random_operands(rng, 4, 128, 512)
    ref = gemm.gemm_block_ref(a, sa, w, sw)
    T = gemm.gemm_block_ref(tolerance.abs_codes(a), np.abs(sa), tolerance.abs_codes(w), np.abs(sw))
    B = tolerance.accumulation_bound(T, 512, "block")
    for seed in range(3):
        acc = _fp32_block_gemm(a, sa, w, sw, np.random.default_rng(seed)).astype(np.float64)
        assert np.all(np.abs(acc - ref) <= B)
        out = _bits_of(acc)
        r = tolerance.check(out, ref, B)
        assert r["ok"], r
        assert r["max_ulp_where_clause_holds"] <= 1
    assert tolerance.fp32_roundings(512, "block") == 128 + 4 + 16
    assert tolerance.fp32_roundings(512, "tensor") == 512 + 2 + 16


def test_neighbour_clause_catches_two_ulp_error():
    # a 2-ulp error on an output of about 0.8 rms (far from the cancellation
    # floor) passes the rounding-aware max-abs gate and the Frobenius bound,
    # and fails the neighbour clause; 1 ulp passes
    rng = np.random.default_rng(34)
    a, sa, w, sw = _random_operands(rng, 8, 256, 512)
    ref = gemm.gemm_block_ref(a, sa, w, sw)
    T = gemm.gemm_block_ref(tolerance.abs_codes(a), np.abs(sa), tolerance.abs_codes(w), np.abs(sw))
    B = tolerance.accumulation_bound(T, 512, "block")
    good = _bits_of(tolerance.bf16_rne(ref))
    i = np.unravel_index(np.argmin(np.abs(np.abs(ref) - 0.8 * tolerance.rms(ref))), ref.shape)
    assert B[i] < 0.25 * tolerance.bf16_ulp(ref[i])
    key = tolerance.bf16_order_key(good[i])
    # ref[i] is further than B from every rounding midpoint, so even a 1-ulp
    # move is beyond what fp32 accumulation can do (item 4 catches it); the
    # neighbour clause alone allows 1 ulp and rejects 2
    gap = np.abs(np.abs(ref[i]) - (np.abs(tolerance.bf16_rne(ref[i])) +
                                   0.5 * tolerance.bf16_ulp(ref[i])))
    assert gap > B[i]
    for steps, neighbour_ok in ((1, True), (2, False), (-2, False)):
        bad = good.copy()
        k = int(key) + steps
        bad[i] = np.uint16(k) if k >= 0 else np.uint16(0x8000 | -k)
        r = tolerance.check(bad, ref, B)
        assert r["elementwise_gate_ok"] and r["frob_ok"], r
        assert r["max_ulp"] == abs(steps)
        assert r["neighbour_gate_ok"] == neighbour_ok, (steps, r)
        assert not r["ok"]
    # the exemption is confined to outputs near the cancellation floor
    r = tolerance.check(good, ref, B)
    assert r["n_clause_exempt"] < 0.5 * ref.size
    exempt = B > 0.25 * tolerance.bf16_ulp(ref)
    assert np.all(np.abs(ref[exempt]) < np.abs(ref).max() / 4)


def test_accumulation_gate_catches_error_near_zero():
    # an output whose reference is near zero may be several ulps from
    # bf16_RNE(ref), but not further from ref than B + half an ulp
    ref = np.array([[1e-6, 3.0]])
    B = np.array([[4e-6, 1e-5]])
    ok_bits = _bits_of([[1e-6 + 3e-6, 3.0]])
    r = tolerance.check(ok_bits, ref, B)
    assert r["ok"] and r["max_ulp"] > 1 and r["n_clause_exempt"] == 1
    bad_bits = _bits_of([[1e-6 + 9e-6, 3.0]])
    r = tolerance.check(bad_bits, ref, B)
    assert not r["accumulation_gate_ok"] and not r["ok"]


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
