"""The shared input generator: bf16 rounding, determinism, shapes (CPU only)."""

import numpy as np
import torch

from workloads import synth


def test_bf16_rounding_matches_torch():
    rng = np.random.default_rng(31)
    v = (rng.standard_normal(200000) * np.exp(rng.uniform(-30, 30, 200000))).astype(np.float32)
    lib = torch.from_numpy(v).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(synth.f32_to_bf16_bits(v), lib)


def test_deterministic_and_shapes():
    a = synth.make_config("tiny")
    b = synth.make_config("tiny")
    assert np.array_equal(a["A"], b["A"]) and np.array_equal(a["W"], b["W"])
    assert a["A"].shape == (16, 512) and a["W"].shape == (256, 512)
    assert len(a["channels"]) == 2


def test_outlier_channels():
    ch = synth.outlier_channels(2, 4096)
    assert len(ch) == 4 and len(set(ch.tolist())) == 4
    assert len(synth.outlier_channels(5, 8192)) == 8
    d1 = synth.make_config("decode", M=4)
    x = synth.bf16_bits_to_f32_input(d1["A"])
    colmax = np.abs(x).max(axis=0)
    assert np.all(colmax[d1["channels"]] > 20)


def test_decode_rows_share_channels():
    c1 = synth.make_config("decode", M=1)["channels"]
    c16 = synth.make_config("decode", M=16)["channels"]
    assert np.array_equal(c1, c16)


def test_edge_cases_shapes():
    e = synth.edge_activations()
    for k, v in e.items():
        assert v.dtype == np.uint16 and v.shape[1] % 128 == 0, k
    x = synth.bf16_bits_to_f32_input(e["all_amax"]).reshape(-1, 128)
    amax = np.abs(x).max(axis=1)
    assert len(np.unique(amax[amax > 0])) == 32639


def test_kv_slots_are_paged_and_distinct():
    d = synth.make_kv(6, 300, 2, 16, block_size=16, num_blocks=64, n_seqs=7, pad_frac=0.1)
    assert d["key"].shape == d["value"].shape == (300, 2, 16)
    s = d["slots"]
    live = s[s >= 0]
    assert 0 < (s < 0).sum() < 60
    assert len(np.unique(live)) == len(live) and live.max() < 64 * 16
    # without padding every token has a slot and consecutive tokens of a
    # sequence sit at consecutive offsets of one block
    d = synth.make_kv(6, 64, 1, 8, block_size=16, num_blocks=8, n_seqs=2)
    s = d["slots"]
    assert (s >= 0).all()
    for seq in (s[:32], s[32:]):
        assert (seq[:16] // 16 == seq[0] // 16).all() and (seq[:16] % 16 == np.arange(16)).all()
    assert np.array_equal(synth.make_kv(6, 64, 1, 8, 16, 8, 2)["key"], d["key"])
