"""Parity of the other scaling granularities with the oracle (needs a gfx950 GPU).

Dynamic per-token activation scales and per-channel weight scales
(FP8_SCALE_ROW), static per-tensor activation quantization
(fp8_quant_act_static) and the per-row-scaled GEMM, all through the C ABI.
Codes and scales bit-exact against oracle.quant.quant_rows_ref /
quant_static_ref; GEMM outputs through the oracle's tolerance gate against
oracle.gemm.gemm_rows_ref on every kernel path (decode, mid-size tile,
hand-scheduled prefill in both tile shapes, C++ prefill for K % 512 != 0).
"""

import json
import os
import sys

import numpy as np
import pytest
import torch

from oracle import gemm, quant, tolerance  # noqa: F401

import oracle_refs
from workloads import synth

pytestmark = pytest.mark.gpu

if torch.cuda.is_available():
    import fp8_w8a8_block_amd as fp8

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def log(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def dev_bf16(bits):
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).cuda().view(torch.bfloat16)


def host_u16(t):
    return t.view(torch.int16).cpu().numpy().view(np.uint16)


def assert_equal_codes(got, want, what):
    if not np.array_equal(got, want):
        bad = np.argwhere(got != want)
        i = tuple(bad[0])
        raise AssertionError(f"{what}: {len(bad)} mismatches, first at {i}: "
                             f"got {got[i]:#04x} want {want[i]:#04x}")


def assert_equal_scales(got, want, what):
    g = np.asarray(got, dtype=np.float32).view(np.uint32)
    w = np.asarray(want, dtype=np.float32).view(np.uint32)
    if not np.array_equal(g, w):
        i = tuple(np.argwhere(g != w)[0])
        raise AssertionError(f"{what}: scale mismatch at {i}: got {got[i]!r} want {want[i]!r}")


def check_out(out_bits, refd, what):
    r = oracle_refs.check(out_bits, refd)
    log(what, {k: (round(v, 6) if isinstance(v, float) else v) for k, v in r.items()})
    assert r["ok"], (what, r)


# ---------------------------------------------------------------------------
# dynamic per-row quantization (per token / per output channel)

@pytest.mark.parametrize("name,M", [("tiny", None), ("decode", 1), ("decode", 16), ("prefill", None)])
def test_quant_rows_activations(name, M):
    d = synth.make_config(name, M=M)
    log("quant rows act", name, d["A"].shape)
    q, s = fp8.quant_act(dev_bf16(d["A"]), "row")
    torch.cuda.synchronize()
    wq, ws = quant.quant_rows_ref(d["A"])
    assert_equal_scales(s.cpu().numpy(), ws, f"{name} token scales")
    assert_equal_codes(q.cpu().numpy(), wq, f"{name} codes")


@pytest.mark.parametrize("case", ["zeros", "negzero", "tiny", "huge", "mixed", "single", "ragged_m",
                                  "all_amax"])
def test_quant_rows_edges(case):
    bits = synth.edge_activations()[case]
    q, s = fp8.quant_act(dev_bf16(bits), "row")
    torch.cuda.synchronize()
    wq, ws = quant.quant_rows_ref(bits)
    assert_equal_scales(s.cpu().numpy(), ws, f"{case} scales")
    assert_equal_codes(q.cpu().numpy(), wq, f"{case} codes")


@pytest.mark.parametrize("name", ["decode", "mlp_down"])
def test_quant_rows_weights_per_channel(name):
    d = synth.make_config(name)
    log("quant rows weight", name, d["W"].shape)
    q, s = fp8.quant_weight_block(dev_bf16(d["W"]), "row")
    torch.cuda.synchronize()
    wq, ws = quant.quant_rows_ref(d["W"])
    assert_equal_scales(s.cpu().numpy(), ws, f"{name} channel scales")
    assert_equal_codes(q.cpu().numpy(), wq, f"{name} codes")


def test_quant_rows_long_rows_and_strides():
    # K = 32768 (64 chunks per lane), a padded row stride and a strided scale vector
    rng = np.random.default_rng(91)
    a = synth.f32_to_bf16_bits((rng.standard_normal((5, 32768)) * 3).astype(np.float32))
    x = torch.zeros((5, 32768 + 64), dtype=torch.bfloat16, device="cuda")
    x[:, :32768] = dev_bf16(a)
    q = torch.zeros((5, 32768 + 16), dtype=torch.uint8, device="cuda")
    s = torch.full((5, 3), -1.0, dtype=torch.float32, device="cuda")
    fp8.quant_act(x[:, :32768], "row", q=q[:, :32768], scales=s[:, 0])
    torch.cuda.synchronize()
    wq, ws = quant.quant_rows_ref(a)
    assert_equal_codes(q[:, :32768].cpu().numpy(), wq, "codes")
    assert_equal_scales(s[:, 0].cpu().numpy(), ws, "scales")
    assert torch.all(s[:, 1:] == -1.0) and torch.all(q[:, 32768:] == 0)


# ---------------------------------------------------------------------------
# static quantization

def _static(bits, scale):
    sc = torch.tensor([scale], dtype=torch.float32, device="cuda")
    q = fp8.quant_act_static(dev_bf16(bits), sc)
    torch.cuda.synchronize()
    return q.cpu().numpy()


def test_static_at_the_dynamic_scale_equals_dynamic():
    d = synth.make_config("prefill")
    _, s = quant.quant_tensor_ref(d["A"][:512])
    got = _static(d["A"][:512], s[0])
    assert_equal_codes(got, quant.quant_static_ref(d["A"][:512], s), "codes")


@pytest.mark.parametrize("scale", [0.0123, 1.0, 3.0e-30, 7.5e-39, 6.0e30, 0.0, float("inf"),
                                   float("nan")])
def test_static_scales(scale):
    # saturating, subnormal, huge, zero, infinite and NaN scales: IEEE quotients
    edges = synth.edge_activations()
    bits = np.concatenate([edges["mixed"], edges["tiny"], edges["huge"], edges["zeros"],
                           edges["negzero"]], axis=0)
    got = _static(bits, np.float32(scale))
    assert_equal_codes(got, quant.quant_static_ref(bits, np.float32(scale)), f"scale {scale}")


# scales at the edges of the one-reciprocal quotient path: smallest and
# largest normal, an all-ones mantissa, negative, and seeded mantissas
# across the exponent range
_EDGE_SCALES = [2.0 ** -126, 3.4028234663852886e38, 1.9999998807907104, -0.37, -2.0 ** -126,
                448.0, 1.0 / 448.0] + [float(v) for v in np.float32(
                    np.random.default_rng(41).uniform(1, 2, 8) *
                    2.0 ** np.random.default_rng(42).integers(-120, 120, 8))]


@pytest.mark.parametrize("scale", _EDGE_SCALES)
def test_static_every_bf16_pattern(scale):
    # all 65536 bf16 inputs, shuffled so NaN and infinite inputs share
    # 8-value chunks with ordinary ones
    allb = np.random.default_rng(43).permutation(65536).astype(np.uint16).reshape(64, 1024)
    s = np.float32(scale)
    assert_equal_codes(_static(allb, s), quant.quant_static_ref(allb, s), f"scale {scale!r}")


def test_static_division_adversarial():
    # the adversarial (amax, x) pairs with s = fp32(amax) / 448 as the static scale
    pairs = json.load(open(os.path.join(GOLDEN, "div_adversarial.json")))["pairs_amax_bits_x_bits"]
    for ab, xb in pairs[:64]:
        amax = quant.bf16_bits_to_f32(np.array([ab], dtype=np.uint16))[0]
        s = np.float32(amax / np.float32(448))
        row = np.zeros((1, 128), dtype=np.uint16)
        row[0, 0], row[0, 1] = ab, xb
        assert_equal_codes(_static(row, s), quant.quant_static_ref(row, s), f"pair {ab:#x},{xb:#x}")


# ---------------------------------------------------------------------------
# GEMM with per-row scales

def run_rows(a_bits, w_bits, a_kind="row", w_kind="row"):
    """GPU: per-token (or static per-tensor) A, per-channel (or per-tensor) W, GEMM in row mode."""
    x, wd = dev_bf16(a_bits), dev_bf16(w_bits)
    if w_kind == "row":
        wq, ws = fp8.quant_weight_block(wd, "row")
    else:
        wq, ws = fp8.quant_weight_block(wd, "tensor")
    if a_kind == "row":
        aq, as_ = fp8.quant_act(x, "row")
    else:                                    # static per-tensor with the oracle's scale
        _, s = quant.quant_tensor_ref(a_bits)
        as_ = torch.tensor(s, dtype=torch.float32, device="cuda")
        aq = fp8.quant_act_static(x, as_)
    out = fp8.block_gemm(aq, as_, wq, ws, "row")
    torch.cuda.synchronize()
    return host_u16(out)


def oracle_rows(a_bits, w_bits, a_kind="row", w_kind="row"):
    if a_kind == "row":
        aq, sa = quant.quant_rows_ref(a_bits)
    else:
        _, sa = quant.quant_tensor_ref(a_bits)
        aq = quant.quant_static_ref(a_bits, sa)
    if w_kind == "row":
        wq, sw = quant.quant_rows_ref(w_bits)
    else:
        wq, sw = quant.quant_tensor_ref(w_bits)
    return oracle_refs.rows(aq, sa, wq, sw)


@pytest.mark.parametrize("M", [1, 4, 16])
def test_gemm_rows_decode(M):
    d = synth.make_config("decode", M=M)
    log("gemm rows decode", M)
    check_out(run_rows(d["A"], d["W"]), oracle_rows(d["A"], d["W"]), f"decode M={M}")


@pytest.mark.parametrize("M,N,K", [(40, 384, 640), (300, 384, 512), (2000, 4224, 1024),
                                   (300, 384, 640), (129, 256, 2048)])
def test_gemm_rows_paths(M, N, K):
    # mid-size tile kernel, hand-scheduled prefill 128x256 and 256x256 tiles,
    # C++ prefill (K % 512 != 0); ragged M and N
    rng = np.random.default_rng([M, N, K, 5])
    a = synth.f32_to_bf16_bits(rng.standard_normal((M, K)).astype(np.float32))
    a[::7] = synth.f32_to_bf16_bits((rng.standard_normal((len(a[::7]), K)) * 40).astype(np.float32))
    w = synth.f32_to_bf16_bits((rng.standard_normal((N, K)) * 0.05).astype(np.float32))
    log("gemm rows", M, N, K)
    check_out(run_rows(a, w), oracle_rows(a, w), f"rows {M}x{N}x{K}")


@pytest.mark.parametrize("M,N,K", [(4, 11008, 4096), (300, 384, 512), (2000, 4224, 1024)])
def test_gemm_rows_broadcast(M, N, K):
    # static per-tensor activations x per-channel weights (a_s stride 0), and
    # per-token activations x a per-tensor weight (w_s stride 0)
    rng = np.random.default_rng([M, N, K, 6])
    a = synth.f32_to_bf16_bits(rng.standard_normal((M, K)).astype(np.float32))
    w = synth.f32_to_bf16_bits((rng.standard_normal((N, K)) * 0.05).astype(np.float32))
    check_out(run_rows(a, w, "static", "row"), oracle_rows(a, w, "static", "row"),
              f"static x channel {M}x{N}x{K}")
    check_out(run_rows(a, w, "row", "tensor"), oracle_rows(a, w, "row", "tensor"),
              f"token x tensor {M}x{N}x{K}")


def test_gemm_rows_prefill_sampled():
    d = synth.make_config("prefill")
    log("gemm rows prefill sampled")
    out = run_rows(d["A"], d["W"])
    rng = np.random.default_rng(45)
    rows = np.sort(rng.choice(d["M"], 64, replace=False))
    cols = np.sort(rng.choice(d["N"], 1024, replace=False))
    aq, sa = quant.quant_rows_ref(d["A"][rows])          # per row: rows are independent
    wq, sw = quant.quant_rows_ref(d["W"][cols])
    check_out(out[np.ix_(rows, cols)], oracle_refs.rows(aq, sa, wq, sw), "prefill rows sampled")


@pytest.mark.parametrize("M,N,K", [(16, 256, 512), (300, 384, 512), (2000, 4224, 1024)])
def test_tensor_mode_is_row_mode_with_single_scales(M, N, K):
    # FP8_SCALE_TENSOR and FP8_SCALE_ROW with one-element scales run the same
    # arithmetic: identical bits
    rng = np.random.default_rng([M, N, K, 7])
    x = dev_bf16(synth.f32_to_bf16_bits(rng.standard_normal((M, K)).astype(np.float32)))
    wd = dev_bf16(synth.f32_to_bf16_bits((rng.standard_normal((N, K)) * 0.05).astype(np.float32)))
    wq, ws = fp8.quant_weight_block(wd, "tensor")
    aq, as_ = fp8.quant_act(x, "tensor")
    o1 = fp8.block_gemm(aq, as_, wq, ws, "tensor")
    o2 = fp8.block_gemm(aq, as_, wq, ws, "row")
    torch.cuda.synchronize()
    assert torch.equal(o1.view(torch.int16), o2.view(torch.int16))


# ---------------------------------------------------------------------------
# linear in row mode

@pytest.mark.parametrize("M", [1, 4, 16, 300])
def test_linear_rows_matches_two_calls(M):
    rng = np.random.default_rng([M, 8])
    K, N = 1024, 768
    x = dev_bf16(synth.f32_to_bf16_bits(rng.standard_normal((M, K)).astype(np.float32)))
    wd = dev_bf16(synth.f32_to_bf16_bits((rng.standard_normal((N, K)) * 0.05).astype(np.float32)))
    wq, ws = fp8.quant_weight_block(wd, "row")
    aq, as_ = fp8.quant_act(x, "row")
    want = fp8.block_gemm(aq, as_, wq, ws, "row")
    got = fp8.linear(x, wq, ws, "row")
    torch.cuda.synchronize()
    assert torch.equal(got.view(torch.int16), want.view(torch.int16))


def test_linear_rows_decode_vs_oracle():
    d = synth.make_config("decode", M=4)
    wq, ws = fp8.quant_weight_block(dev_bf16(d["W"]), "row")
    out = fp8.linear(dev_bf16(d["A"]), wq, ws, "row")
    torch.cuda.synchronize()
    check_out(host_u16(out), oracle_rows(d["A"], d["W"]), "linear rows decode M=4")
