"""Pins for the FP8 KV-cache codec oracle (CPU only).

Pinned by: the write is the pinned static quantizer placed by slot (checked
element by element against a direct loop over blocks and offsets, with
padding and out-of-range slots left untouched); round trips that the format
makes exact (E4M3-representable values times a power-of-two scale come back
bit-exact); saturation at 448 * scale with the default scale 1.0; and the
fp32 -> bf16 rounding against torch's."""

import numpy as np
import torch

from oracle import e4m3, kv_cache, quant
from workloads import synth


def _bits(a):
    return synth.f32_to_bf16_bits(np.asarray(a, dtype=np.float32))


def test_write_places_static_codes_by_slot():
    rng = np.random.default_rng(31)
    T, H, D, nb, bs = 6, 2, 16, 3, 4
    x = _bits(rng.standard_normal((T, H, D)) * 3)
    slots = np.array([5, -1, 0, 11, 12, 7], dtype=np.int64)      # -1 padding, 12 past the end
    cache0 = rng.integers(0, 255, (nb, bs, H, D), dtype=np.uint8)
    s = np.float32(0.05)
    got = kv_cache.kv_write_ref(x, slots, cache0, s)
    want = cache0.copy()
    for t in range(T):
        sl = int(slots[t])
        if sl < 0 or sl >= nb * bs:
            continue
        blk, off = divmod(sl, bs)
        for h in range(H):
            want[blk, off, h] = quant.quant_static_ref(x[t, h][None, :], s)[0]
    assert np.array_equal(got, want)
    assert np.array_equal(got[0, 1], cache0[0, 1])                 # untouched slots stay


def test_round_trip_exact_on_representable_values():
    # every finite E4M3 magnitude times a power-of-two scale survives write + read
    t = e4m3.decode_table()
    vals = t[np.isfinite(t)]
    for scale in (1.0, 0.25, 8.0):
        x = (vals * scale).astype(np.float32)
        x = x[: (len(x) // 16) * 16].reshape(-1, 1, 16)
        bits = _bits(x)
        assert np.array_equal(quant.bf16_bits_to_f32(bits), x)   # exact in bf16
        T = bits.shape[0]
        cache = kv_cache.kv_write_ref(bits, np.arange(T), np.zeros((T, 1, 1, 16), np.uint8),
                                      np.float32(scale))
        back = kv_cache.kv_read_ref(cache, np.arange(T), np.float32(scale))
        assert np.array_equal(back, bits)


def test_default_scale_saturates_outliers():
    x = _bits([[[1000.0, -600.0, 448.0, 500.0, 0.5, -0.0, 3.0, 1e-6]]])
    cache = kv_cache.kv_write_ref(x, np.array([0]), np.zeros((1, 1, 1, 8), np.uint8),
                                  np.float32(1.0))
    assert cache[0, 0, 0].tolist() == [0x7E, 0xFE, 0x7E, 0x7E, 0x30, 0x80, 0x44, 0x00]
    back = kv_cache.kv_read_ref(cache, np.array([0, -1]), np.float32(1.0))
    assert quant.bf16_bits_to_f32(back[0, 0]).tolist() == [448, -448, 448, 448, 0.5, -0.0, 3.0, 0.0]
    assert np.all(back[1] == 0)                                    # padding token reads zeros


def test_bf16_rounding_matches_torch():
    rng = np.random.default_rng(32)
    f = (rng.standard_normal(10000) * 100).astype(np.float32)
    want = torch.from_numpy(f).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(kv_cache.bf16_rne_bits(f), want)
    nan = kv_cache.bf16_rne_bits(np.array([np.nan, -np.nan], dtype=np.float32))
    assert nan.tolist() == [0x7FC0, 0xFFC0]


def test_nan_restores_with_the_code_sign():
    # 0x7F / 0xFF are the E4M3 NaN codes; a zero code times an infinite scale
    # and any code times a NaN scale are NaN products too: each restores to
    # the quiet bf16 NaN carrying the stored code's sign bit
    cache = np.array([0x7F, 0xFF, 0x00, 0x80, 0x01, 0x81, 0x38, 0xB8],
                     dtype=np.uint8).reshape(1, 1, 1, 8)
    one = kv_cache.kv_read_ref(cache, np.array([0]), np.float32(1.0))[0, 0]
    assert one.tolist()[:2] == [0x7FC0, 0xFFC0]
    assert one.tolist()[2:] == [0x0000, 0x8000, 0x3B00, 0xBB00, 0x3F80, 0xBF80]  # 2^-9, 1.0
    inf = kv_cache.kv_read_ref(cache, np.array([0]), np.float32(np.inf))[0, 0]
    assert inf.tolist() == [0x7FC0, 0xFFC0, 0x7FC0, 0xFFC0, 0x7F80, 0xFF80, 0x7F80, 0xFF80]
    nan = kv_cache.kv_read_ref(cache, np.array([0]), np.float32(np.nan))[0, 0]
    assert nan.tolist() == [0x7FC0, 0xFFC0] * 4
