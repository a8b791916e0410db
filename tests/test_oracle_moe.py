"""Pins for the grouped (MoE) GEMM oracle (CPU only).

Pinned by: an exact computation on a tiny case with an empty expert and an
uncovered row (integer dot products of the codes times 2^9 and exact
rational scales, independent of the oracle's fp64 matrix products); the
permutation law (relabelling experts and moving their row segments with
them permutes the output rows the same way); the reduction to one big block
GEMM when every expert holds the same weight; and weights that differ by
expert (a segment multiplied by the wrong expert shows up at once)."""

from fractions import Fraction

import numpy as np

from oracle import e4m3, gemm, moe


def _codes(rng, shape):
    c = rng.integers(0, 256, shape).astype(np.uint8)
    c[(c & 0x7F) == 0x7F] = 0x30                       # no NaN codes
    return c


def _exact(a, sa, w, sw, offsets):
    """Exact values as Fractions: dec * 2^9 are integers, scales are exact binary fractions."""
    dec_a = np.rint(e4m3.decode(a) * 512).astype(np.int64)
    E = w.shape[0]
    M, K = a.shape
    N = w.shape[1]
    KB = K // 128
    out = {}
    for e in range(E):
        dec_w = np.rint(e4m3.decode(w[e]) * 512).astype(np.int64)
        for r in range(int(offsets[e]), int(offsets[e + 1])):
            for n in range(N):
                acc = Fraction(0)
                for kb in range(KB):
                    ks = slice(kb * 128, (kb + 1) * 128)
                    c = int(np.dot(dec_a[r, ks], dec_w[n, ks]))      # exact, < 2^43
                    acc += Fraction(float(sa[r, kb])) * Fraction(float(sw[e, n // 128, kb])) * c
                out[(r, n)] = acc / (512 * 512)
    return out


def test_exact_tiny_with_empty_expert_and_uncovered_row():
    rng = np.random.default_rng(51)
    E, M, N, K = 3, 6, 128, 256
    offsets = [0, 2, 2, 5]                              # expert 1 empty, row 5 in no segment
    a = _codes(rng, (M, K))
    w = _codes(rng, (E, N, K))
    sa = rng.uniform(0.001, 0.02, (M, K // 128)).astype(np.float32)
    sw = rng.uniform(0.0005, 0.01, (E, N // 128, K // 128)).astype(np.float32)
    got = moe.grouped_gemm_ref(a, sa, w, sw, offsets)
    ex = _exact(a, sa, w, sw, offsets)
    for (r, n), v in ex.items():
        assert abs(got[r, n] - float(v)) <= 1e-13 * abs(float(v)) + 1e-300, (r, n)
    assert np.isnan(got[5]).all()
    assert len(ex) == 5 * N


def test_permuting_experts_permutes_rows():
    rng = np.random.default_rng(52)
    E, N, K = 4, 256, 384
    sizes = [3, 0, 5, 2]
    off = np.concatenate([[0], np.cumsum(sizes)])
    M = int(off[-1])
    a = _codes(rng, (M, K))
    sa = rng.uniform(0.001, 0.02, (M, K // 128)).astype(np.float32)
    w = _codes(rng, (E, N, K))
    sw = rng.uniform(0.0005, 0.01, (E, N // 128, K // 128)).astype(np.float32)
    base = moe.grouped_gemm_ref(a, sa, w, sw, off)
    perm = [2, 0, 3, 1]                                 # new expert j is old expert perm[j]
    rows = np.concatenate([np.arange(off[p], off[p + 1]) for p in perm]).astype(np.int64)
    off2 = np.concatenate([[0], np.cumsum([sizes[p] for p in perm])])
    got = moe.grouped_gemm_ref(a[rows], sa[rows], w[perm], sw[perm], off2)
    assert np.array_equal(got, base[rows])


def test_shared_weight_is_one_block_gemm():
    rng = np.random.default_rng(53)
    E, M, N, K = 5, 23, 256, 256
    a = _codes(rng, (M, K))
    sa = rng.uniform(0.001, 0.02, (M, K // 128)).astype(np.float32)
    w1 = _codes(rng, (N, K))
    sw1 = rng.uniform(0.0005, 0.01, (N // 128, K // 128)).astype(np.float32)
    off = [0, 4, 4, 11, 20, 23]
    got = moe.grouped_gemm_ref(a, sa, np.stack([w1] * E), np.stack([sw1] * E), off)
    assert np.array_equal(got, gemm.gemm_block_ref(a, sa, w1, sw1))


def test_each_segment_uses_its_own_expert():
    rng = np.random.default_rng(54)
    E, N, K = 3, 128, 128
    off = [0, 1, 2, 3]
    a = _codes(rng, (3, K))
    sa = np.ones((3, 1), dtype=np.float32)
    w1 = _codes(rng, (N, K))
    w = np.stack([w1] * E)
    sw = np.array([1.0, 2.0, 4.0], dtype=np.float32).reshape(E, 1, 1)   # expert e scaled by 2^e
    got = moe.grouped_gemm_ref(a, sa, w, sw, off)
    one = gemm.gemm_block_ref(a, sa, w1, np.ones((1, 1), np.float32))
    for e in range(E):
        assert np.array_equal(got[e], one[e] * 2.0 ** e)
