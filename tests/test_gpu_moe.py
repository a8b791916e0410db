"""Parity of the grouped (MoE) block-scaled GEMM with the oracle (needs a gfx950 GPU).

fp8_grouped_gemm through the C ABI against oracle.moe.grouped_gemm_ref on
the same FP8 operands (quantized by the oracle on the host), through the
tolerance gate of the block GEMM: both kernel paths (the decode tile for a
few rows per expert, including its 16-row chunk loop, and the grouped
hand-scheduled kernel in both tile shapes: 128-row tiles while experts
average at most 512 rows, 256-row tiles above), empty experts, rows in no
expert's range left untouched, ragged segments crossing 128- and 256-row tiles,
clamped offsets, an activation stride past 32-bit buffer offsets, bit-identity with fp8_block_gemm for a single expert, and
sampled rows of the two full MoE workloads.
"""

import sys

import numpy as np
import pytest
import torch

from oracle import moe, quant, tolerance  # noqa: F401

import oracle_refs
from workloads import synth

pytestmark = pytest.mark.gpu

if torch.cuda.is_available():
    import fp8_w8a8_block_amd as fp8

SENTINEL = 0x7E00          # a bf16 NaN the kernels never produce


def log(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def dev(a):
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


def host_u16(t):
    return t.view(torch.int16).cpu().numpy().view(np.uint16)


def operands(seed, E, N, K, M):
    """Oracle-quantized activations [M, K] and expert weights [E, N, K]."""
    rng = np.random.default_rng(seed)
    a_bits = synth.f32_to_bf16_bits(rng.standard_normal((M, K), dtype=np.float32))
    aq, as_ = quant.quant_act_ref(a_bits)
    wq = np.empty((E, N, K), dtype=np.uint8)
    ws = np.empty((E, N // 128, K // 128), dtype=np.float32)
    for e in range(E):
        w_bits = synth.f32_to_bf16_bits(
            rng.standard_normal((N, K), dtype=np.float32) * np.float32(0.02 * (1 + e)))
        wq[e], ws[e] = quant.quant_weight_block_ref(w_bits)
    return aq, as_, wq, ws


def run_grouped(aq, as_, wq, ws, offsets):
    M, N = aq.shape[0], wq.shape[1]
    out = torch.full((M, N), SENTINEL, dtype=torch.int16, device="cuda").view(torch.bfloat16)
    fp8.grouped_gemm(dev(aq), dev(as_), dev(wq), dev(ws), dev(np.asarray(offsets, np.int64)),
                     out=out)
    torch.cuda.synchronize()
    return host_u16(out)


def check(got, aq, as_, wq, ws, offsets, what):
    d = oracle_refs.grouped(aq, as_, wq, ws, offsets)
    covered = ~np.isnan(d["ref"][:, 0])
    r = oracle_refs.check(got[covered], oracle_refs.select(d, np.flatnonzero(covered)))
    log(what, {k: (round(v, 6) if isinstance(v, float) else v) for k, v in r.items()})
    assert r["ok"], (what, r)
    assert (got[~covered] == SENTINEL).all(), f"{what}: rows in no segment were written"


# (E, N, K, segment sizes, uncovered rows before, after); the path follows
# from M against 32 rows per expert and from K / 128 % 4
CASES = {
    "decode_small": (5, 256, 512, [3, 0, 17, 1, 40], 2, 3),
    "decode_chunks": (8, 256, 512, [100, 0, 0, 0, 0, 0, 0, 5], 0, 0),
    "decode_k640": (2, 256, 640, [150, 90], 1, 0),
    "asm_128row": (3, 512, 1024, [300, 0, 530], 5, 7),
    "asm_k512_edges": (4, 384, 512, [255, 256, 257, 1], 0, 2),
    # the longest K of a grouped call (128 K blocks) on both paths
    "decode_k16384": (3, 256, 16384, [5, 20, 0], 1, 0),
    "asm_k16384": (2, 256, 16384, [300, 100], 0, 0),
}


@pytest.mark.parametrize("case", list(CASES))
def test_grouped_small(case):
    E, N, K, sizes, lead, tail = CASES[case]
    M = lead + sum(sizes) + tail
    offsets = lead + np.concatenate([[0], np.cumsum(sizes)])
    log("grouped", case, dict(E=E, N=N, K=K, M=M, offsets=offsets.tolist()))
    aq, as_, wq, ws = operands(61, E, N, K, M)
    got = run_grouped(aq, as_, wq, ws, offsets)
    check(got, aq, as_, wq, ws, offsets, case)


def test_grouped_w8_sampled():
    # 3000 rows per expert on average: the 256 x 256 shape; rows sampled at
    # segment and tile edges
    E, N, K = 4, 1920, 1024                   # N % 256 = 128: a half-empty last tile
    sizes = [4000, 3000, 0, 5000]
    lead, tail = 3, 4
    M = lead + sum(sizes) + tail
    offsets = lead + np.concatenate([[0], np.cumsum(sizes)])
    log("grouped w8", dict(M=M, offsets=offsets.tolist()))
    aq, as_, wq, ws = operands(62, E, N, K, M)
    got = run_grouped(aq, as_, wq, ws, offsets)
    rows = set(range(lead)) | set(range(M - tail, M))
    for e in range(E):
        lo, hi = int(offsets[e]), int(offsets[e + 1])
        for r in (lo, lo + 1, lo + 255, lo + 256, lo + 257, hi - 2, hi - 1):
            if lo <= r < hi:
                rows.add(r)
    rng = np.random.default_rng(63)
    rows |= set(rng.choice(M, 40, replace=False).tolist())
    rows = np.array(sorted(rows))
    # the oracle on the sampled rows: each row keeps its expert
    expert = np.searchsorted(offsets, rows, side="right") - 1
    inside = (rows >= offsets[0]) & (rows < offsets[-1])
    sub_off = np.concatenate([[0], np.cumsum([np.sum(inside & (expert == e)) for e in range(E)])])
    order = rows[inside]
    r = oracle_refs.check(got[order], oracle_refs.grouped(aq[order], as_[order], wq, ws, sub_off))
    log("grouped w8 sampled", r)
    assert r["ok"], r
    assert (got[rows[~inside]] == SENTINEL).all()


def test_single_expert_bit_identical_to_block_gemm():
    E, M, N, K = 1, 1000, 1024, 1024
    aq, as_, wq, ws = operands(64, E, N, K, M)
    got = run_grouped(aq, as_, wq, ws, [0, M])
    # the grouped kernel never splits K: compare with the unsplit dense call
    plain = fp8.block_gemm(dev(aq), dev(as_), dev(wq[0]), dev(ws[0]), split=False)
    torch.cuda.synchronize()
    assert np.array_equal(got, host_u16(plain))
    # and a decode-path segment (at most 16 rows) equals the decode GEMM
    got16 = run_grouped(aq[:13], as_[:13], np.stack([wq[0], wq[0]]), np.stack([ws[0], ws[0]]),
                        [0, 5, 13])
    plain16 = fp8.block_gemm(dev(aq[5:13]), dev(as_[5:13]), dev(wq[0]), dev(ws[0]))
    torch.cuda.synchronize()
    assert np.array_equal(got16[5:13], host_u16(plain16))


def test_wide_activation_stride_uses_the_decode_tile():
    # 200 rows over 2 experts would take the grouped hand-scheduled kernel;
    # an activation stride past its 32-bit buffer offsets sends the call to
    # the grouped decode tile, which has no such limit
    E, N, K, M = 2, 256, 512, 200
    aq, as_, wq, ws = operands(67, E, N, K, M)
    offsets = [0, 120, 200]
    ld_a = (1 << 23) + 16
    a_big = torch.zeros((M, ld_a), dtype=torch.uint8, device="cuda")
    a_big[:, :K] = torch.from_numpy(aq).cuda()
    out = torch.full((M, N), SENTINEL, dtype=torch.int16, device="cuda").view(torch.bfloat16)
    fp8.grouped_gemm(a_big[:, :K], dev(as_), dev(wq), dev(ws), dev(np.asarray(offsets, np.int64)),
                     out=out)
    torch.cuda.synchronize()
    check(host_u16(out), aq, as_, wq, ws, offsets, "wide activation stride")
    del a_big
    torch.cuda.empty_cache()


def test_offsets_are_clamped():
    E, N, K, M = 3, 256, 512, 50
    aq, as_, wq, ws = operands(65, E, N, K, M)
    got = run_grouped(aq, as_, wq, ws, [-5, 10, 10, 1000])
    check(got, aq, as_, wq, ws, [0, 10, 10, 50], "clamped")


@pytest.mark.parametrize("name", ["moe_decode", "moe_prefill"])
def test_full_workload_sampled(name):
    c = synth.MOE_CONFIGS[name]
    E, N, K = c["experts_local"], c["N"], c["K"]
    rows, offsets = synth.make_moe_routing(c["cfg"], c["tokens"], c["top_k"], c["experts_total"], E)
    M = len(rows)
    log("moe workload", name, dict(M=M, E=E, N=N, K=K))
    tok = synth.make_moe_tokens(c["cfg"], c["tokens"], K, c["n_outliers"], c["outlier_mult"])
    a_bits = tok[rows]
    aq, as_ = quant.quant_act_ref(a_bits)
    # every expert's weight quantized on the device for the call; the three
    # sampled experts' weights quantized again by the oracle for the check
    wq = torch.empty((E, N, K), dtype=torch.uint8, device="cuda")
    ws = torch.empty((E, N // 128, K // 128), dtype=torch.float32, device="cuda")
    counts = np.diff(offsets)
    picks = [int(np.argmax(counts)), int(np.argmin(np.where(counts > 0, counts, 1 << 30))),
             int(np.flatnonzero(counts > 0)[len(np.flatnonzero(counts > 0)) // 2])]
    ref_w = {}
    for e in range(E):
        w_bits = synth.make_moe_weight(c["cfg"], e, N, K, c["w_std"])
        q, s = fp8.quant_weight_block(dev(w_bits.view(np.int16)).view(torch.bfloat16))
        wq[e].copy_(q)
        ws[e].copy_(s)
        if e in picks:
            ref_w[e] = quant.quant_weight_block_ref(w_bits)
    out = torch.full((M, N), SENTINEL, dtype=torch.int16, device="cuda").view(torch.bfloat16)
    fp8.grouped_gemm(dev(aq), dev(as_), wq, ws, dev(offsets), out=out)
    torch.cuda.synchronize()
    got = host_u16(out)
    rng = np.random.default_rng(66)
    for e in picks:
        lo, hi = int(offsets[e]), int(offsets[e + 1])
        sample = np.unique(np.concatenate([[lo, hi - 1], rng.integers(lo, hi, 6)]))
        r = oracle_refs.check(got[sample], oracle_refs.grouped(
            aq[sample], as_[sample], ref_w[e][0][None], ref_w[e][1][None], [0, len(sample)]))
        log(name, "expert", e, "rows", hi - lo, r)
        assert r["ok"], (name, e, r)
    assert not (got == SENTINEL).any(), "every row belongs to an expert here"
