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
