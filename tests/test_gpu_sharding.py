"""The column-parallel sharding of the linear layer, on one GPU (needs a gfx950 GPU).

Split along N on multiples of the 128-wide weight blocks, every GPU quantizes
the same activation and multiplies it by its slice of the weight codes and
block scales; the output columns of the shards are disjoint.  That is a
valid way to shard the layer because a shard's output is exactly the
matching columns of the unsharded output: the quantizer's codes and scales
depend on the activation alone, and every output column is one fixed
sequence of per-K-block products and folds, however the columns are tiled.

Here the decode weight (11008 x 4096, 86 weight blocks) is cut as eight GPUs
would take it (11, 11, 11, 11, 11, 11, 10, 10 blocks).  Decode batches go
through fp8_linear shard by shard (the fused kernel, and the two-launch path
at 16 rows) and must give the full call's columns bit for bit.  A prefill
batch goes through the block GEMM on codes quantized once, unsplit: the
hand-scheduled kernel's tile grid differs between the full call and the
shards, but each column's arithmetic does not, so again bit for bit.  (A
shard small enough to split K in two sums its two halves at the end, a
different order: the same value up to fp32 rounding, checked through the
tolerance gate below.)  The first GPU's share is also checked against the
oracle through the GEMM tolerance gate, through fp8_linear as a caller
would run it.  Slices of the token rows (data parallelism) likewise give the
full call's rows bit for bit.
"""

import sys

import numpy as np
import pytest
import torch

from oracle import quant

import oracle_refs
from workloads import synth

pytestmark = pytest.mark.gpu

if torch.cuda.is_available():
    import fp8_w8a8_block_amd as fp8

BLOCKS = [11, 11, 11, 11, 11, 11, 10, 10]          # 86 weight blocks over 8 GPUs


def log(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def dev_bf16(bits):
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).cuda().view(torch.bfloat16)


def host_u16(t):
    return t.view(torch.int16).cpu().numpy().view(np.uint16)


def shard_bounds():
    assert sum(BLOCKS) * 128 == 11008
    edges = np.cumsum([0] + BLOCKS) * 128
    return list(zip(edges[:-1], edges[1:]))


@pytest.fixture(scope="module")
def decode_weight():
    d = synth.make_config("decode", M=16)
    w = d["W"]
    wq, ws = fp8.quant_weight_block(dev_bf16(w))
    torch.cuda.synchronize()
    return w, wq, ws


def shard(wq, ws, lo, hi):
    """A shard's own contiguous weight codes and block scales."""
    return wq[lo:hi].contiguous(), ws[lo // 128:hi // 128].contiguous()


@pytest.mark.parametrize("M", [1, 4, 16])
def test_decode_shards_equal_the_full_call(M, decode_weight):
    w, wq, ws = decode_weight
    rng = np.random.default_rng([M, 77])
    a = synth.f32_to_bf16_bits(rng.standard_normal((M, 4096)).astype(np.float32))
    x = dev_bf16(a)
    full = host_u16(fp8.linear(x, wq, ws))
    for lo, hi in shard_bounds():
        log(f"decode shard M={M} columns {lo}..{hi}")
        got = host_u16(fp8.linear(x, *shard(wq, ws, lo, hi)))
        assert np.array_equal(got, full[:, lo:hi]), f"M={M} shard {lo}..{hi}"


def test_prefill_shards_equal_the_full_call(decode_weight):
    w, wq, ws = decode_weight
    M = 300
    rng = np.random.default_rng([M, 77])
    a = synth.f32_to_bf16_bits(rng.standard_normal((M, 4096)).astype(np.float32))
    aq, as_ = fp8.quant_act(dev_bf16(a))
    full = host_u16(fp8.block_gemm(aq, as_, wq, ws, split=False))
    for lo, hi in shard_bounds():
        log(f"prefill shard M={M} columns {lo}..{hi}")
        got = host_u16(fp8.block_gemm(aq, as_, *shard(wq, ws, lo, hi), split=False))
        assert np.array_equal(got, full[:, lo:hi]), f"M={M} shard {lo}..{hi}"


@pytest.mark.parametrize("M,parts", [(16, 4), (300, 3)])
def test_row_slices_equal_the_full_call(M, parts, decode_weight):
    # token rows (data parallel): rows are independent, scales are per row,
    # so a slice of the batch gives the full call's rows bit for bit -- at
    # M = 16 the slices of 4 rows take the fused kernel and the full call the
    # two-launch path; at M = 300 both run the unsplit block GEMM
    w, wq, ws = decode_weight
    rng = np.random.default_rng([M, 79])
    a = synth.f32_to_bf16_bits(rng.standard_normal((M, 4096)).astype(np.float32))
    step = M // parts
    if M <= 16:
        full = host_u16(fp8.linear(dev_bf16(a), wq, ws))
        part = lambda lo, hi: host_u16(fp8.linear(dev_bf16(a[lo:hi]), wq, ws))
    else:
        full = host_u16(fp8.block_gemm(*fp8.quant_act(dev_bf16(a)), wq, ws, split=False))
        part = lambda lo, hi: host_u16(fp8.block_gemm(*fp8.quant_act(dev_bf16(a[lo:hi])), wq, ws,
                                                      split=False))
    for lo in range(0, M, step):
        hi = min(lo + step, M)
        log(f"row slice M={M} rows {lo}..{hi}")
        assert np.array_equal(part(lo, hi), full[lo:hi]), f"M={M} rows {lo}..{hi}"


@pytest.mark.parametrize("M", [4, 300])
def test_one_gpu_share_against_the_oracle(M, decode_weight):
    # the first GPU's share: N = 1408, K = 4096
    w, wq, ws = decode_weight
    rng = np.random.default_rng([M, 78])
    a = synth.f32_to_bf16_bits(rng.standard_normal((M, 4096)).astype(np.float32))
    lo, hi = shard_bounds()[0]
    got = host_u16(fp8.linear(dev_bf16(a), *shard(wq, ws, lo, hi)))
    aq, as_ = quant.quant_act_ref(a)
    wq_r, ws_r = quant.quant_weight_block_ref(w[lo:hi])
    r = oracle_refs.check(got, oracle_refs.block(aq, as_, wq_r, ws_r))
    log(f"share M={M}", {k: (round(v, 6) if isinstance(v, float) else v) for k, v in r.items()})
    assert r["ok"], r
