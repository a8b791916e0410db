"""Parity of the HIP path with the CPU oracle (needs a gfx950 GPU).

Every call goes through the C ABI (libfp8w8a8.so via the ctypes binding).
Inputs are the seeded workloads; expected values come from oracle/ only.
Codes and scales must be bit-exact; the GEMM must pass the oracle's
tolerance gate (elementwise 1e-2 * rms(ref) + half a bf16 ulp, Frobenius
<= 4e-3, the accumulation bound and the bf16-neighbour clause).
Codes and scales are compared in full on every workload.  GEMM outputs are
compared in full on every workload except the 8192 x 28672 x 8192 one, where
stratified full rows and full columns cover every output tile of the launch.
"""

import sys

import numpy as np
import pytest
import torch

from oracle import e4m3, gemm, quant, tolerance  # noqa: F401

import oracle_refs
from workloads import synth

pytestmark = pytest.mark.gpu

if torch.cuda.is_available():
    import fp8_w8a8_block_amd as fp8


def log(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def dev_bf16(bits):
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).cuda().view(torch.bfloat16)


def host_u16(t):
    return t.view(torch.int16).cpu().numpy().view(np.uint16)


def gpu_quant_act(bits, mode="block"):
    q, s = fp8.quant_act(dev_bf16(bits), mode)
    torch.cuda.synchronize()
    return q.cpu().numpy(), s.cpu().numpy()


def gpu_quant_weight(bits, mode="block"):
    q, s = fp8.quant_weight_block(dev_bf16(bits), mode)
    torch.cuda.synchronize()
    return q.cpu().numpy(), s.cpu().numpy()


def assert_codes_equal(got, want, what):
    if not np.array_equal(got, want):
        bad = np.argwhere(got != want)
        i = tuple(bad[0])
        raise AssertionError(f"{what}: {len(bad)} code mismatches, first at {i}: "
                             f"got {got[i]:#04x} want {want[i]:#04x}")


def assert_scales_equal(got, want, what):
    g = np.asarray(got, dtype=np.float32).view(np.uint32)
    w = np.asarray(want, dtype=np.float32).view(np.uint32)
    if not np.array_equal(g, w):
        bad = np.argwhere(g != w)
        i = tuple(bad[0])
        raise AssertionError(f"{what}: {len(bad)} scale mismatches, first at {i}: "
                             f"got {got[i]!r} want {want[i]!r}")


# ---------------------------------------------------------------------------
# element encoder

def test_encoder_targeted_values():
    t = e4m3.decode_table()
    pos = t[:0x7F]
    mids = (pos[:-1] + pos[1:]) / 2
    vals = [pos, mids]
    for ulps in (1, 2, 3):
        f = mids.astype(np.float32)
        up = f.copy()
        dn = f.copy()
        for _ in range(ulps):
            up = np.nextafter(up, np.float32(np.inf))
            dn = np.nextafter(dn, np.float32(-np.inf))
        vals += [up.astype(np.float64), dn.astype(np.float64)]
    rng = np.random.default_rng(41)
    vals.append(np.exp(rng.uniform(np.log(1e-45), np.log(1e3), 200000)))
    vals.append(np.array([448.0, 448.00003, 455.9, 463.99997, 464.0, 464.00003, 500.0, 1e30,
                          np.inf, 2.0 ** -10, 2.0 ** -149, 0.0]))
    v = np.concatenate(vals).astype(np.float32)
    v = np.concatenate([v, -v, np.array([np.nan, -np.nan], dtype=np.float32)])
    got = fp8.encode_f32(torch.from_numpy(v).cuda()).cpu().numpy()
    assert_codes_equal(got, e4m3.encode(v), "encoder")


# ---------------------------------------------------------------------------
# activation quantizer

@pytest.mark.parametrize("case", ["zeros", "negzero", "tiny", "huge", "mixed", "single",
                                  "ragged_m", "all_amax"])
def test_quant_act_edge_cases(case):
    bits = synth.edge_activations()[case]
    log("quant_act edge", case, bits.shape)
    q, s = gpu_quant_act(bits)
    wq, ws = quant.quant_act_ref(bits)
    assert_scales_equal(s, ws, f"scales[{case}]")
    assert_codes_equal(q, wq, f"codes[{case}]")


def test_quant_act_worked_group():
    import json, os
    g = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "e4m3_worked_group.json")))
    row = np.zeros(128, dtype=np.float32)
    row[:len(g["cases"])] = [c["x"] for c in g["cases"]]
    bits = synth.f32_to_bf16_bits(row)[None, :]
    q, s = gpu_quant_act(bits)
    assert s[0, 0] == 1.0
    assert q[0, :len(g["cases"])].tolist() == [int(c["code"], 16) for c in g["cases"]]


def test_quant_act_division_adversarial():
    import json, os
    pairs = json.load(open(os.path.join(os.path.dirname(__file__), "golden",
                                        "div_adversarial.json")))["pairs_amax_bits_x_bits"]
    rows = np.zeros((len(pairs), 128), dtype=np.uint16)
    for i, (ab, xb) in enumerate(pairs):
        rows[i, 0], rows[i, 1] = ab, xb
    q, s = gpu_quant_act(rows)
    wq, ws = quant.quant_act_ref(rows)
    assert_scales_equal(s, ws, "scales")
    assert_codes_equal(q, wq, "codes")


@pytest.mark.parametrize("name,M", [("tiny", None), ("decode", 1), ("decode", 4), ("decode", 16),
                                    ("prefill", None), ("mlp_down", None)])
def test_quant_act_configs_full(name, M):
    c = synth.CONFIGS[name]
    M = c["M"] if M is None else M
    ch = synth.outlier_channels(c["cfg"], c["K"], c["n_outliers"])
    bits = synth.make_activation(c["cfg"], M, c["K"], c["a_kind"], c["a_std"], ch, c["outlier_mult"])
    log("quant_act", name, bits.shape)
    q, s = gpu_quant_act(bits)
    wq, ws = quant.quant_act_ref(bits)
    assert_scales_equal(s, ws, f"scales[{name}]")
    assert_codes_equal(q, wq, f"codes[{name}]")


def test_quant_act_large_full():
    # every code and scale of the 8192 x 8192 activation (oracle in row chunks)
    d, wq, ws, _, _ = oracle_refs.workload("large")
    log("quant_act large", d["A"].shape)
    q, s = gpu_quant_act(d["A"])
    assert_scales_equal(s, ws, "scales[large]")
    assert_codes_equal(q, wq, "codes[large]")


def test_quant_act_strided_and_ragged():
    rng = np.random.default_rng(43)
    bits = synth.f32_to_bf16_bits(rng.standard_normal((37, 1024)).astype(np.float32))
    big = np.zeros((37, 1024 + 64), dtype=np.uint16)
    big[:, :1024] = bits
    x = dev_bf16(big)[:, :1024]                     # ld_x = 1088
    qbuf = torch.zeros((37, 1024 + 32), dtype=torch.uint8, device="cuda")
    sbuf = torch.zeros((37, 11), dtype=torch.float32, device="cuda")
    q, s = fp8.quant_act(x, "block", q=qbuf[:, :1024], scales=sbuf[:, :8])
    torch.cuda.synchronize()
    wq, ws = quant.quant_act_ref(bits)
    assert_codes_equal(qbuf[:, :1024].cpu().numpy(), wq, "codes")
    assert_scales_equal(sbuf[:, :8].cpu().numpy(), ws, "scales")
    assert np.all(qbuf[:, 1024:].cpu().numpy() == 0)     # padding untouched
    assert np.all(sbuf[:, 8:].cpu().numpy() == 0)


@pytest.mark.parametrize("M,K", [(3, 1 << 20), (100003, 128)])
def test_quant_act_extreme_shapes(M, K):
    # a 2^20-element row (256 workgroups per row) and 100003 one-group rows
    # (groups numbered across rows); codes and scales bit-exact
    rng = np.random.default_rng([M, K])
    bits = synth.f32_to_bf16_bits((rng.standard_normal((M, K)) * 3).astype(np.float32))
    log("quant extreme", (M, K))
    q, s = gpu_quant_act(bits)
    wq, ws = quant.quant_act_ref(bits)
    assert_codes_equal(q, wq, f"codes {M}x{K}")
    assert_scales_equal(s, ws, f"scales {M}x{K}")


def test_quant_act_empty():
    x = torch.empty((0, 512), dtype=torch.bfloat16, device="cuda")
    q, s = fp8.quant_act(x)
    assert q.shape == (0, 512) and s.shape == (0, 4)


# ---------------------------------------------------------------------------
# weight quantizer

@pytest.mark.parametrize("name", ["tiny", "decode", "prefill", "mlp_down"])
def test_quant_weight_configs_full(name):
    c = synth.CONFIGS[name]
    bits = synth.make_weight(c["cfg"], c["N"], c["K"], c["w_std"])
    log("quant_weight", name, bits.shape)
    q, s = gpu_quant_weight(bits)
    wq, ws = quant.quant_weight_block_ref(bits)
    assert_scales_equal(s, ws, f"wscales[{name}]")
    assert_codes_equal(q, wq, f"wcodes[{name}]")


def test_quant_weight_large_full():
    # all 224 block rows of the 28672 x 8192 weight
    d, _, _, wq, ws = oracle_refs.workload("large")
    log("quant_weight large", d["W"].shape)
    q, s = gpu_quant_weight(d["W"])
    assert_scales_equal(s, ws, "wscales[large]")
    assert_codes_equal(q, wq, "wcodes[large]")


def test_quant_weight_edge_blocks():
    e = synth.edge_activations()
    # build a 256 x 512 weight from edge rows: zero blocks, tiny blocks, huge blocks
    w = np.zeros((256, 512), dtype=np.uint16)
    w[0:2] = e["tiny"][:2]
    w[128:130] = e["huge"]
    w[200, 300] = 0x8000
    q, s = gpu_quant_weight(w)
    wq, ws = quant.quant_weight_block_ref(w)
    assert_scales_equal(s, ws, "wscales")
    assert_codes_equal(q, wq, "wcodes")


# ---------------------------------------------------------------------------
# per-tensor quantization (MLP down-projection variant)

def test_quant_tensor_mlp_down():
    c = synth.CONFIGS["mlp_down"]
    ch = synth.outlier_channels(c["cfg"], c["K"], c["n_outliers"])
    a = synth.make_activation(c["cfg"], c["M"], c["K"], c["a_kind"], c["a_std"], ch, c["outlier_mult"])
    w = synth.make_weight(c["cfg"], c["N"], c["K"], c["w_std"])
    qa, sa = gpu_quant_act(a, "tensor")
    wqa, wsa = quant.quant_tensor_ref(a)
    assert_scales_equal(sa, wsa, "tensor scale A")
    assert_codes_equal(qa, wqa, "tensor codes A")
    qw, sw = gpu_quant_weight(w, "tensor")
    wqw, wsw = quant.quant_tensor_ref(w)
    assert_scales_equal(sw, wsw, "tensor scale W")
    assert_codes_equal(qw, wqw, "tensor codes W")


def test_quant_tensor_edges():
    for case in ("zeros", "negzero", "tiny", "ragged_m"):
        bits = synth.edge_activations()[case]
        q, s = gpu_quant_act(bits, "tensor")
        wq, ws = quant.quant_tensor_ref(bits)
        assert_scales_equal(s, ws, f"tensor scale {case}")
        assert_codes_equal(q, wq, f"tensor codes {case}")


# ---------------------------------------------------------------------------
# GEMM

def run_gemm(a_bits, w_bits, mode="block", split=True):
    """GPU: quantize A and W, then GEMM (split in K where the shape allows it,
    unless split is False).  Returns out bits (uint16 [M, N])."""
    x = dev_bf16(a_bits)
    wd = dev_bf16(w_bits)
    wq, ws = fp8.quant_weight_block(wd, mode)
    aq, as_ = fp8.quant_act(x, mode)
    out = fp8.block_gemm(aq, as_, wq, ws, mode, split=split)
    torch.cuda.synchronize()
    return host_u16(out)


def oracle_gemm(a_bits, w_bits, mode="block"):
    """The oracle's reference dict (oracle_refs) on the oracle's own codes."""
    if mode == "block":
        aq, as_ = quant.quant_act_ref(a_bits)
        wq, ws = quant.quant_weight_block_ref(w_bits)
        return oracle_refs.block(aq, as_, wq, ws)
    aq, as_ = quant.quant_tensor_ref(a_bits)
    wq, ws = quant.quant_tensor_ref(w_bits)
    return oracle_refs.tensor(aq, as_, wq, ws)


def check_out(out_bits, refd, what):
    r = oracle_refs.check(out_bits, refd)
    log(what, {k: (round(v, 6) if isinstance(v, float) else v) for k, v in r.items()})
    assert r["ok"], (what, r)
    return r


@pytest.mark.parametrize("K", [32768, 33280])
def test_gemm_longest_k(K):
    # K = 32768 fills the hand-scheduled kernel's weight-scale table (256 K
    # blocks), split in K and unsplit; one more 512 goes to the C++ prefill
    # kernel
    M, N = 300, 256
    rng = np.random.default_rng(K)
    a_bits = synth.f32_to_bf16_bits(rng.standard_normal((M, K), dtype=np.float32))
    w_bits = synth.f32_to_bf16_bits(rng.standard_normal((N, K), dtype=np.float32) * np.float32(0.02))
    log("gemm longest K", (M, N, K))
    ref = oracle_gemm(a_bits, w_bits)
    check_out(run_gemm(a_bits, w_bits), ref, f"K={K}")
    check_out(run_gemm(a_bits, w_bits, split=False), ref, f"K={K} unsplit")


def test_gemm_longest_k_256_tiles_sampled():
    # the 256 x 256 tile shape at K = 32768 (both rows of the weight-scale
    # table): the device quantizes for the call, the oracle re-quantizes the
    # sampled activation rows and weight blocks for the check
    M, N, K = 2304, 4096, 32768
    rng = np.random.default_rng(72)
    a_bits = synth.f32_to_bf16_bits(rng.standard_normal((M, K), dtype=np.float32))
    w_bits = synth.f32_to_bf16_bits(rng.standard_normal((N, K), dtype=np.float32) * np.float32(0.02))
    log("gemm longest K, 256x256 tiles", (M, N, K))
    out = run_gemm(a_bits, w_bits)
    rows = np.array([0, 1, 255, 256, 1000, 2047, 2048, M - 1])
    blocks = [0, 17, 31]                               # weight blocks of 128 rows
    cols = np.concatenate([np.arange(b * 128, b * 128 + 128) for b in blocks])
    aq, as_ = quant.quant_act_ref(a_bits[rows])
    wq, ws = quant.quant_weight_block_ref(w_bits[cols])
    check_out(np.ascontiguousarray(out[rows][:, cols]), oracle_refs.block(aq, as_, wq, ws),
              "K=32768 256x256 sampled")


@pytest.mark.parametrize("which", ["wide_a", "wide_out"])
def test_gemm_strides_beyond_32bit_offsets(which):
    # leading dimensions past the hand-scheduled kernel's 32-bit buffer
    # offsets: an activation stride of 2^23 + 16 codes sends M > 64 to the
    # 128 x 128 tile kernel, an output stride of 2^22 + 64 to the C++ prefill
    # kernel; both against the oracle
    M, N, K = 100, 256, 512
    rng = np.random.default_rng(71)
    a_bits = synth.f32_to_bf16_bits(rng.standard_normal((M, K), dtype=np.float32))
    w_bits = synth.f32_to_bf16_bits(rng.standard_normal((N, K), dtype=np.float32) * np.float32(0.02))
    aq, as_ = quant.quant_act_ref(a_bits)
    wq, ws = quant.quant_weight_block_ref(w_bits)
    ld_a = (1 << 23) + 16 if which == "wide_a" else K
    ld_o = (1 << 22) + 64 if which == "wide_out" else N
    log("gemm wide strides", which, dict(ld_a=ld_a, ld_out=ld_o))
    a_big = torch.zeros((M, ld_a), dtype=torch.uint8, device="cuda")
    a_big[:, :K] = torch.from_numpy(aq).cuda()
    o_big = torch.full((M, ld_o), 0x7E00, dtype=torch.int16, device="cuda")
    out = o_big.view(torch.bfloat16)[:, :N]
    fp8.block_gemm(a_big[:, :K], torch.from_numpy(as_).cuda(), torch.from_numpy(wq).cuda(),
                   torch.from_numpy(ws).cuda(), out=out)
    torch.cuda.synchronize()
    check_out(host_u16(out), oracle_refs.block(aq, as_, wq, ws), f"wide strides {which}")
    if which == "wide_out":
        assert (o_big[:, N:N + 64] == 0x7E00).all().item()      # nothing past the row written
    del a_big, o_big
    torch.cuda.empty_cache()


@pytest.mark.parametrize("M", [1, 4, 16])
def test_gemm_decode_full(M):
    d = synth.make_config("decode", M=M)
    log("gemm decode", M)
    out = run_gemm(d["A"], d["W"])
    check_out(out, oracle_gemm(d["A"], d["W"]), f"decode M={M}")


def test_gemm_tiny_full():
    d = synth.make_config("tiny")
    out = run_gemm(d["A"], d["W"])
    check_out(out, oracle_gemm(d["A"], d["W"]), "tiny")


@pytest.mark.parametrize("M,N,K", [(1, 128, 128), (3, 256, 384), (17, 384, 640), (40, 256, 512),
                                   (64, 512, 1024), (100, 256, 1024), (129, 512, 512),
                                   (300, 384, 640), (256, 256, 2304),
                                   # one K block past 64 rows; one 128-wide N tile on both
                                   # large-M kernels
                                   (65, 128, 128), (300, 128, 512), (70, 128, 2176),
                                   # K / 128 = 128: the decode tile's longest K (both forms);
                                   # K / 128 > 128: the 128 x 128 tile kernel
                                   (5, 256, 16384), (40, 256, 16384),
                                   (10, 256, 16512), (40, 256, 16512)])
def test_gemm_ragged_full(M, N, K):
    rng = np.random.default_rng([M, N, K])
    a = synth.f32_to_bf16_bits(rng.standard_normal((M, K)).astype(np.float32))
    w = synth.f32_to_bf16_bits((rng.standard_normal((N, K)) * 0.05).astype(np.float32))
    log("gemm ragged", M, N, K)
    out = run_gemm(a, w)
    check_out(out, oracle_gemm(a, w), f"ragged {M}x{N}x{K}")
    out_t = run_gemm(a, w, "tensor")
    check_out(out_t, oracle_gemm(a, w, "tensor"), f"ragged tensor {M}x{N}x{K}")


def test_gemm_prefill_full():
    # every output of the 4096^3 GEMM in the launch configuration the bench
    # times, against the oracle on its own codes
    d, aq, as_, wq, ws = oracle_refs.workload("prefill")
    log("gemm prefill full", (d["M"], d["N"], d["K"]))
    out = run_gemm(d["A"], d["W"])
    check_out(out, oracle_refs.block(aq, as_, wq, ws), "prefill full")


def test_gemm_mlp_down_full():
    d, aq, as_, wq, ws = oracle_refs.workload("mlp_down")
    log("gemm mlp_down full", (d["M"], d["N"], d["K"]))
    out = run_gemm(d["A"], d["W"])
    check_out(out, oracle_refs.block(aq, as_, wq, ws), "mlp_down full")


def test_gemm_mlp_down_tensor_full():
    d = oracle_refs.workload("mlp_down")[0]
    log("gemm mlp_down tensor full", (d["M"], d["N"], d["K"]))
    out = run_gemm(d["A"], d["W"], "tensor")
    a_amax = quant.tensor_amax_ref(d["A"])
    w_amax = quant.tensor_amax_ref(d["W"])
    aq, as_ = oracle_refs.parallel_rows(lambda b: quant.quant_tensor_with_amax_ref(b, a_amax),
                                        d["A"], 256)
    wq, ws = oracle_refs.parallel_rows(lambda b: quant.quant_tensor_with_amax_ref(b, w_amax),
                                       d["W"], 512)
    check_out(out, oracle_refs.tensor(aq, as_[:1], wq, ws[:1]), "mlp_down tensor full")


def stratified(extent, tile, per_tile, seed):
    """``per_tile`` indices in every ``tile``-wide tile of [0, extent): the
    offsets within the tile cycle through every residue mod 16 and through
    both halves of the tile, so every fragment row position and wave row of
    the launch is sampled."""
    rng = np.random.default_rng(seed)
    out = []
    for t in range(-(-extent // tile)):
        for j in range(per_tile):
            k = t * per_tile + j
            off = (k % 16) + 16 * int(rng.integers(0, tile // 16))
            off = (off % (tile // 2)) + (tile // 2) * (k % 2)
            if t * tile + off < extent:
                out.append(t * tile + off)
    return np.unique(np.array(out))


def test_gemm_large_stratified():
    # 8192 x 28672 x 8192: two rows in every 256-row M tile compared on all
    # 28672 columns, and two columns in every 256-wide N tile compared on all
    # 8192 rows, so every output tile of the full launch is checked
    d, aq, as_, wq, ws = oracle_refs.workload("large")
    log("gemm large", (d["M"], d["N"], d["K"]))
    out = run_gemm(d["A"], d["W"])
    rows = stratified(d["M"], 256, 2, 45)
    cols = stratified(d["N"], 256, 2, 46)
    assert len(rows) == 64 and len(cols) == 224
    assert sorted(set(rows % 16)) == list(range(16)) and sorted(set(cols % 16)) == list(range(16))
    for lo in range(0, d["N"], 4096):                  # full rows, in column chunks
        sl = np.arange(lo, min(lo + 4096, d["N"]))
        check_out(np.ascontiguousarray(out[np.ix_(rows, sl)]),
                  oracle_refs.block_cols(aq[rows], as_[rows], wq, ws, sl, 1 << 28),
                  f"large rows x cols {lo}..")
    for lo in range(0, d["M"], 2048):                  # full columns, in row chunks
        rs = np.arange(lo, lo + 2048)
        check_out(np.ascontiguousarray(out[np.ix_(rs, cols)]),
                  oracle_refs.block_cols(aq[rs], as_[rs], wq, ws, cols, 1 << 28),
                  f"large rows {lo}.. x cols")


# ---------------------------------------------------------------------------
# split K: shapes whose 128 x 256 tiles would fill at most half of the CUs
# run as two workgroups per tile, each over half of the K blocks, when the
# call has the workspace (scales constant along K are applied to the sum of
# the two halves)

def _split_case(M, N, K, mode, seed):
    rng = np.random.default_rng(seed)
    a = synth.f32_to_bf16_bits((rng.standard_normal((M, K)) * 2).astype(np.float32))
    w = synth.f32_to_bf16_bits((rng.standard_normal((N, K)) * 0.03).astype(np.float32))
    qmode = "row" if mode == "row" else mode
    wq, ws = fp8.quant_weight_block(dev_bf16(w), qmode)
    aq, as_ = fp8.quant_act(dev_bf16(a), qmode)
    return a, w, aq, as_, wq, ws


def _oracle_mode(a, w, mode):
    if mode == "row":
        aq, sa = quant.quant_rows_ref(a)
        wq, sw = quant.quant_rows_ref(w)
        return oracle_refs.rows(aq, sa, wq, sw)
    return oracle_gemm(a, w, mode)


@pytest.mark.parametrize("M,N,K,mode", [(512, 512, 2048, "block"), (300, 384, 1024, "block"),
                                        (65, 256, 1024, "block"), (257, 1024, 3072, "block"),
                                        (1000, 640, 2048, "block"), (1024, 2048, 8192, "block"),
                                        (512, 512, 2048, "tensor"), (1000, 640, 2048, "tensor"),
                                        (300, 384, 1024, "row"), (1024, 2048, 8192, "row")])
def test_gemm_split_k(M, N, K, mode):
    # both forms against the oracle; the split form again with a workspace
    # full of garbage (counters are cleared by the call) and once more
    # reusing that workspace: the same bits every time
    nws = fp8.workspace_bytes(fp8._lib.OP_GEMM, M, N, K, mode)
    assert nws > 0, (M, N, K)
    a, w, aq, as_, wq, ws = _split_case(M, N, K, mode, [M, N, K, 3])
    log("gemm split K", (M, N, K, mode), nws)
    out_split = host_u16(fp8.block_gemm(aq, as_, wq, ws, mode))
    out_plain = host_u16(fp8.block_gemm(aq, as_, wq, ws, mode, split=False))
    junk = torch.full((nws,), 0xA5, dtype=torch.uint8, device="cuda")
    out_junk = host_u16(fp8.block_gemm(aq, as_, wq, ws, mode, workspace=junk))
    out_again = host_u16(fp8.block_gemm(aq, as_, wq, ws, mode, workspace=junk))
    torch.cuda.synchronize()
    assert np.array_equal(out_split, out_junk) and np.array_equal(out_split, out_again)
    ref = _oracle_mode(a, w, mode)
    check_out(out_split, ref, f"split {mode} {M}x{N}x{K}")
    check_out(out_plain, ref, f"unsplit {mode} {M}x{N}x{K}")


def test_gemm_split_k_small_workspace_runs_unsplit():
    M, N, K = 300, 512, 2048
    nws = fp8.workspace_bytes(fp8._lib.OP_GEMM, M, N, K, "block")
    a, w, aq, as_, wq, ws = _split_case(M, N, K, "block", 17)
    short = torch.zeros((nws - 256,), dtype=torch.uint8, device="cuda")
    out_short = host_u16(fp8.block_gemm(aq, as_, wq, ws, "block", workspace=short))
    out_plain = host_u16(fp8.block_gemm(aq, as_, wq, ws, "block", split=False))
    assert np.array_equal(out_short, out_plain)
    assert torch.all(short == 0)                 # an unused workspace is not touched


@pytest.mark.parametrize("mode", ["block", "tensor", "row"])
def test_linear_split_k_matches_two_calls(mode):
    # fp8_linear's workspace holds the GEMM's split-K bytes: the result equals
    # quant_act followed by block_gemm with its workspace
    M, N, K = 512, 1024, 4096
    rng = np.random.default_rng(71)
    a = synth.f32_to_bf16_bits(rng.standard_normal((M, K)).astype(np.float32))
    w = synth.f32_to_bf16_bits((rng.standard_normal((N, K)) * 0.02).astype(np.float32))
    nws = fp8.workspace_bytes(fp8._lib.OP_GEMM, M, N, K, mode)
    assert nws > 0 and fp8.workspace_bytes(fp8._lib.OP_LINEAR, M, N, K, mode) >= M * K + nws
    wq, ws = fp8.quant_weight_block(dev_bf16(w), mode)
    x = dev_bf16(a)
    got = host_u16(fp8.linear(x, wq, ws, mode))
    assert np.array_equal(got, _two_call(x, wq, ws, mode))
    check_out(got, _oracle_mode(a, w, mode), f"linear split K {mode}")


def test_split_k_replays_from_a_hip_graph():
    # the split launch clears its words with a kernel, not a memset node, so
    # it can be captured: three replays of a captured fp8_block_gemm and of a
    # captured fp8_linear, with eager work and synchronizations between them,
    # each equal to the eager result bit for bit
    M, N, K = 512, 1024, 4096
    rng = np.random.default_rng(83)
    a = synth.f32_to_bf16_bits(rng.standard_normal((M, K)).astype(np.float32))
    w = synth.f32_to_bf16_bits((rng.standard_normal((N, K)) * 0.02).astype(np.float32))
    wq, ws = fp8.quant_weight_block(dev_bf16(w))
    x = dev_bf16(a)
    aq, as_ = fp8.quant_act(x)
    gws = torch.empty(fp8.workspace_bytes(fp8._lib.OP_GEMM, M, N, K, "block"), dtype=torch.uint8,
                      device="cuda")
    lws = torch.empty(fp8.workspace_bytes(fp8._lib.OP_LINEAR, M, N, K, "block"), dtype=torch.uint8,
                      device="cuda")
    assert gws.numel() > 0
    want_g = host_u16(fp8.block_gemm(aq, as_, wq, ws, workspace=gws))
    want_l = host_u16(fp8.linear(x, wq, ws, workspace=lws))
    out_g = torch.empty((M, N), dtype=torch.bfloat16, device="cuda")
    out_l = torch.empty((M, N), dtype=torch.bfloat16, device="cuda")
    stream = torch.cuda.Stream()
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph, stream=stream):
        fp8.block_gemm(aq, as_, wq, ws, out=out_g, workspace=gws)
        fp8.linear(x, wq, ws, out=out_l, workspace=lws)
    for r in range(3):
        out_g.zero_()
        out_l.zero_()
        gws.fill_(0xA5)                       # garbage in the words between replays
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        assert np.array_equal(host_u16(out_g), want_g), r
        assert np.array_equal(host_u16(out_l), want_l), r
        fp8.block_gemm(aq, as_, wq, ws, workspace=gws)      # eager work between replays
    check_out(want_l, oracle_gemm(a, w), "split K from a graph")


def test_gemm_small_integers_exact():
    """Codes are small integers, unit scales: every partial is exact, so the
    bf16 output must equal the exact result bit for bit."""
    rng = np.random.default_rng(45)
    M, N, K = 40, 256, 256
    # codes of small integers (exactly representable), unit scales; every
    # partial and final sum is an integer of magnitude <= 256, exact in bf16
    ints = rng.integers(-3, 4, size=(M, K)).astype(np.float64)
    intw = rng.integers(-1, 2, size=(N, K)).astype(np.float64)
    aq = e4m3.encode(ints)
    wq = e4m3.encode(intw)
    exact = ints @ intw.T
    assert np.all(np.abs(exact) <= 256)
    a_s = torch.ones((M, K // 128), dtype=torch.float32, device="cuda")
    w_s = torch.ones((N // 128, K // 128), dtype=torch.float32, device="cuda")
    out = fp8.block_gemm(torch.from_numpy(aq).cuda(), a_s, torch.from_numpy(wq).cuda(), w_s)
    got = tolerance.bf16_bits_to_f64(host_u16(out))
    assert np.array_equal(got, exact)
    M1 = 5
    out1 = fp8.block_gemm(torch.from_numpy(aq[:M1]).cuda(), a_s[:M1], torch.from_numpy(wq).cuda(), w_s)
    assert np.array_equal(tolerance.bf16_bits_to_f64(host_u16(out1)), exact[:M1])


def test_gemm_determinism():
    d = synth.make_config("tiny")
    o1 = run_gemm(d["A"], d["W"])
    o2 = run_gemm(d["A"], d["W"])
    assert np.array_equal(o1, o2)
    e = synth.make_config("decode", M=16)
    x = dev_bf16(e["A"])
    wq, ws = fp8.quant_weight_block(dev_bf16(e["W"]))
    outs = [host_u16(fp8.linear(x, wq, ws)) for _ in range(3)]
    assert all(np.array_equal(outs[0], o) for o in outs[1:])


def test_gemm_empty_and_errors():
    wq = torch.zeros((256, 512), dtype=torch.uint8, device="cuda")
    ws = torch.ones((2, 4), dtype=torch.float32, device="cuda")
    aq = torch.zeros((0, 512), dtype=torch.uint8, device="cuda")
    as_ = torch.ones((0, 4), dtype=torch.float32, device="cuda")
    out = fp8.block_gemm(aq, as_, wq, ws)
    assert out.shape == (0, 256)
    with pytest.raises(ValueError):
        fp8.block_gemm(torch.zeros((4, 500), dtype=torch.uint8, device="cuda"),
                       torch.ones((4, 4), dtype=torch.float32, device="cuda"),
                       torch.zeros((256, 500), dtype=torch.uint8, device="cuda"), ws)
    with pytest.raises(ValueError):
        fp8.quant_weight_block(torch.zeros((256, 512), dtype=torch.bfloat16, device="cuda"),
                               block_n=64)


# ---------------------------------------------------------------------------
# one-call linear (fused decode path and workspace path)

def _two_call(x, wq, ws, mode):
    aq, as_ = fp8.quant_act(x, mode)
    return host_u16(fp8.block_gemm(aq, as_, wq, ws, mode))


@pytest.mark.parametrize("K", [512, 4096, 16384])
def test_linear_fused_matches_two_calls(K):
    """The fused decode path is bit-identical to quant_act + block_gemm."""
    rng = np.random.default_rng([K, 7])
    N = 512
    w = synth.f32_to_bf16_bits((rng.standard_normal((N, K)) * 0.02).astype(np.float32))
    wq, ws = fp8.quant_weight_block(dev_bf16(w))
    for M in (1, 2, 3, 4, 5, 7, 8, 9, 12, 15, 16):
        a = synth.f32_to_bf16_bits(rng.standard_normal((M, K)).astype(np.float32))
        a[:, 3] = synth.f32_to_bf16_bits(np.full(M, 60.0, dtype=np.float32))
        x = dev_bf16(a)
        got = host_u16(fp8.linear(x, wq, ws))
        want = _two_call(x, wq, ws, "block")
        assert np.array_equal(got, want), f"M={M} K={K}"


@pytest.mark.parametrize("M", [1, 4, 16])
def test_linear_decode_vs_oracle(M):
    d = synth.make_config("decode", M=M)
    wq, ws = fp8.quant_weight_block(dev_bf16(d["W"]))
    out = host_u16(fp8.linear(dev_bf16(d["A"]), wq, ws))
    check_out(out, oracle_gemm(d["A"], d["W"]), f"linear decode M={M}")


@pytest.mark.parametrize("M,mode", [(17, "block"), (100, "block"), (300, "block"), (3, "tensor"),
                                    (100, "tensor")])
def test_linear_workspace_path(M, mode):
    rng = np.random.default_rng([M, 8])
    N, K = 384, 640
    a = synth.f32_to_bf16_bits(rng.standard_normal((M, K)).astype(np.float32))
    w = synth.f32_to_bf16_bits((rng.standard_normal((N, K)) * 0.05).astype(np.float32))
    wq, ws = fp8.quant_weight_block(dev_bf16(w), mode)
    x = dev_bf16(a)
    got = host_u16(fp8.linear(x, wq, ws, mode))
    assert np.array_equal(got, _two_call(x, wq, ws, mode))
    check_out(got, oracle_gemm(a, w, mode), f"linear {mode} M={M}")


def test_binding_checks_caller_tensors():
    # outputs and scales handed in by the caller are checked before any launch
    x = torch.zeros((16, 512), dtype=torch.bfloat16, device="cuda")
    with pytest.raises(ValueError):
        fp8.quant_act(x, q=torch.empty((8, 512), dtype=torch.uint8, device="cuda"))
    with pytest.raises(ValueError):
        fp8.quant_act(x, scales=torch.empty((16, 3), dtype=torch.float32, device="cuda"))
    with pytest.raises(ValueError):
        fp8.quant_act(x, scales=torch.empty((16, 4), dtype=torch.float32))     # host memory
    aq, as_ = fp8.quant_act(x)
    wq = torch.zeros((256, 512), dtype=torch.uint8, device="cuda")
    ws = torch.ones((2, 4), dtype=torch.float32, device="cuda")
    with pytest.raises(ValueError):
        fp8.block_gemm(aq, as_, wq, ws, out=torch.empty((16, 128), dtype=torch.bfloat16,
                                                        device="cuda"))
    with pytest.raises(ValueError):
        fp8.block_gemm(aq, as_[:8], wq, ws)
    with pytest.raises(ValueError):
        fp8.block_gemm(aq, as_, wq, ws[:1])
    with pytest.raises(ValueError):
        fp8.linear(x, wq, ws.cpu())
    with pytest.raises(ValueError):
        fp8.grouped_gemm(aq, as_, wq[None], ws[None],
                         torch.tensor([0, 16], device="cuda"), out=torch.empty(
                             (16, 256), dtype=torch.bfloat16))
    torch.cuda.synchronize()


def test_linear_errors():
    x = torch.zeros((100, 512), dtype=torch.bfloat16, device="cuda")
    wq = torch.zeros((256, 512), dtype=torch.uint8, device="cuda")
    ws = torch.ones((2, 4), dtype=torch.float32, device="cuda")
    small = torch.empty(16, dtype=torch.uint8, device="cuda")
    with pytest.raises(ValueError):
        fp8.linear(x, wq, ws, workspace=small)          # workspace too small
    with pytest.raises(ValueError):
        fp8.linear(x[:, :500], wq[:, :500], ws)          # K not a multiple of 128
    assert fp8.linear(x[:0], wq, ws).shape == (0, 256)
