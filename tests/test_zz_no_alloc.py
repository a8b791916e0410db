"""fp8_linear_noalloc: the linear call for callers that cannot allocate
(needs a gfx950 GPU).  Through the C ABI, its output equals fp8_linear's bit
for bit on two calls in a row -- the second with a smaller input, so stale
scratch contents from the first call would show -- in every scale mode and on
the fused path; a call needing more than the scratch is refused up front."""

import numpy as np
import pytest
import torch

from workloads import synth

pytestmark = pytest.mark.gpu

if torch.cuda.is_available():
    import fp8_w8a8_block_amd as fp8


def dev_bf16(bits):
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).cuda().view(torch.bfloat16)


def operands(seed, M, N, K, mode):
    rng = np.random.default_rng(seed)
    a = synth.f32_to_bf16_bits((rng.standard_normal((M, K)) * 2).astype(np.float32))
    w = synth.f32_to_bf16_bits((rng.standard_normal((N, K)) * 0.05).astype(np.float32))
    wq, ws = fp8.quant_weight_block(dev_bf16(w), mode)
    return dev_bf16(a), wq, ws


@pytest.mark.parametrize("mode,shapes", [
    ("block", [(300, 384, 640), (100, 384, 640)]),        # quantizer + GEMM through scratch
    ("block", [(16, 11008, 4096), (9, 11008, 4096)]),     # decode batch above the fused limit
    ("tensor", [(257, 256, 1024), (3, 256, 1024)]),       # per-tensor partials in scratch
    ("row", [(64, 512, 512), (17, 512, 512)]),
    ("block", [(4, 512, 1024), (1, 512, 1024)]),          # fused path: no scratch
    ("block", [(16, 256, 512), (9, 256, 512)]),           # fused up to 16 rows on small shapes
    ("block", [(512, 1024, 4096), (300, 512, 2048)]),     # GEMM split in K: its slots in scratch
    ("tensor", [(512, 1024, 4096), (300, 512, 2048)]),    # the same with one scale per tensor
])
def test_noalloc_matches_linear(mode, shapes):
    for i, (M, N, K) in enumerate(shapes):
        x, wq, ws = operands([M, N, K, i], M, N, K, mode)
        want = fp8.linear(x, wq, ws, mode)
        out = torch.full((M, N), float("nan"), dtype=torch.bfloat16, device="cuda")
        got = fp8.linear_noalloc(x, wq, ws, out, mode)
        torch.cuda.synchronize()
        assert got.data_ptr() == out.data_ptr()
        assert torch.equal(got.view(torch.int16), want.view(torch.int16)), (mode, M, N, K)


def test_noalloc_refuses_calls_beyond_its_scratch():
    # 16384 x 4096 block activations need 64 MiB of codes plus scales: more
    # than the 64 MiB scratch; refused before anything is enqueued
    M, N, K = 16384, 256, 4096
    x = torch.zeros((M, K), dtype=torch.bfloat16, device="cuda")
    wq = torch.zeros((N, K), dtype=torch.uint8, device="cuda")
    ws = torch.ones((N // 128, K // 128), dtype=torch.float32, device="cuda")
    out = torch.full((M, N), 7.0, dtype=torch.bfloat16, device="cuda")
    assert fp8.workspace_bytes(3, M, N, K, "block") > (64 << 20)
    with pytest.raises(ValueError, match="scratch"):
        fp8.linear_noalloc(x, wq, ws, out)
    torch.cuda.synchronize()
    assert bool((out == 7.0).all())
