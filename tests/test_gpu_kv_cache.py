"""Parity of the FP8 KV-cache codec with the oracle (needs a gfx950 GPU).

fp8_kv_cache_write (static E4M3 quantization scattered by slot into a paged
[blocks, block_size, H, D] cache) and fp8_kv_cache_read (gather + restore to
bf16), through the C ABI, bit-exact against oracle.kv_cache: whole caches on
small paged layouts (padding, out-of-range slots, odd head sizes, strided
token rows, untouched slots keeping their bytes), every bf16 input pattern,
every stored code under ordinary and degenerate scales, and sampled tokens
of the full 65536-token, 1 GiB-per-cache workload.
"""

import sys

import numpy as np
import pytest
import torch

from oracle import kv_cache, quant
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


def dev_scale(v):
    return torch.tensor([v], dtype=torch.float32, device="cuda")


def assert_same(got, want, what):
    if not np.array_equal(got, want):
        bad = np.argwhere(got != want)
        i = tuple(bad[0])
        raise AssertionError(f"{what}: {len(bad)} mismatches, first at {i}: "
                             f"got {int(got[i]):#06x} want {int(want[i]):#06x}")


def amax_scale(bits):
    f = quant.bf16_bits_to_f32(bits)
    return np.float32(np.abs(f).max() / np.float32(448.0))


# (T, H, D, num_blocks, block_size, n_seqs, pad_frac, row_stride_factor)
CASES = {
    "heads8_d128": (37, 8, 128, 5, 16, 3, 0.15, 1),
    "odd_heads": (53, 3, 40, 8, 7, 4, 0.0, 1),
    "one_chunk": (5, 1, 8, 1, 16, 1, 0.0, 1),
    "qkv_rows": (70, 4, 64, 6, 16, 5, 0.1, 3),       # K and V are slices of a [T, 3 * H * D] row
    "many_tokens": (1500, 2, 128, 120, 16, 9, 0.05, 1),
}


@pytest.mark.parametrize("case", list(CASES))
def test_write_whole_cache(case):
    T, H, D, nb, bs, ns, pad, f = CASES[case]
    log("kv write", case, (T, H, D, nb, bs))
    d = synth.make_kv(7, T, H, D, bs, nb, ns, pad_frac=pad)
    slots = d["slots"].copy()
    if T > 4:
        slots[1] = nb * bs                               # one past the end: not stored
        slots[3] = nb * bs + 1000
    rng = np.random.default_rng(8)
    k0 = rng.integers(0, 256, (nb, bs, H, D), dtype=np.uint8)
    v0 = rng.integers(0, 256, (nb, bs, H, D), dtype=np.uint8)
    ks, vs = amax_scale(d["key"]), np.float32(1.0)       # calibrated keys, default values
    if f == 1:
        key, value = dev_bf16(d["key"]), dev_bf16(d["value"])
    else:
        hd = H * D
        row = np.zeros((T, f * hd), dtype=np.uint16)
        row[:, hd:2 * hd] = d["key"].reshape(T, hd)
        row[:, 2 * hd:] = d["value"].reshape(T, hd)
        big = dev_bf16(row)
        key = big[:, hd:2 * hd].view(T, H, D)
        value = big[:, 2 * hd:].view(T, H, D)
        assert key.stride(0) == f * hd
    kc = torch.from_numpy(k0).cuda()
    vc = torch.from_numpy(v0).cuda()
    fp8.kv_cache_write(key, value, torch.from_numpy(slots).cuda(), kc, vc, dev_scale(ks),
                       dev_scale(vs))
    torch.cuda.synchronize()
    assert_same(kc.cpu().numpy(), kv_cache.kv_write_ref(d["key"], slots, k0, ks), case + " keys")
    assert_same(vc.cpu().numpy(), kv_cache.kv_write_ref(d["value"], slots, v0, vs),
                case + " values")


@pytest.mark.parametrize("scale", [1.0, 0.0123, 1e-38, 0.0, float("inf"), float("nan"), -0.5,
                                   2.0 ** -126, 3.4028234663852886e38, 1.9999998807907104])
def test_write_every_bf16_pattern(scale):
    log("kv write all bf16, scale", scale)
    # every bf16 input, shuffled so NaN and infinite inputs share 8-value
    # chunks with ordinary ones
    allb = np.random.default_rng(44).permutation(65536).astype(np.uint16).reshape(64, 1, 1024)
    x = np.ascontiguousarray(allb)
    y = np.ascontiguousarray(allb[::-1])
    slots = np.arange(64, dtype=np.int64)[::-1].copy()
    kc = torch.zeros((4, 16, 1, 1024), dtype=torch.uint8, device="cuda")
    vc = torch.zeros_like(kc)
    s = np.float32(scale)
    fp8.kv_cache_write(dev_bf16(x), dev_bf16(y), torch.from_numpy(slots).cuda(), kc, vc,
                       dev_scale(s), dev_scale(np.float32(2.0)))
    torch.cuda.synchronize()
    z = np.zeros((4, 16, 1, 1024), dtype=np.uint8)
    assert_same(kc.cpu().numpy(), kv_cache.kv_write_ref(x, slots, z, s), f"keys at {scale}")
    assert_same(vc.cpu().numpy(), kv_cache.kv_write_ref(y, slots, z, np.float32(2.0)), "values")


@pytest.mark.parametrize("scale", [1.0, 0.37, 2.0 ** -10, 1e30, 3.0e38, -2.0, 0.0,
                                   float("inf"), float("nan"), 1e-40])
def test_read_every_code(scale):
    log("kv read all codes, scale", scale)
    cache = np.arange(256, dtype=np.uint8).reshape(2, 1, 1, 128)
    slots = np.array([0, 1, -1, 2, 1, 0, -7], dtype=np.int64)   # repeats and out-of-range
    s = np.float32(scale)
    out = fp8.kv_cache_read(torch.from_numpy(cache).cuda(), torch.from_numpy(slots).cuda(),
                            dev_scale(s))
    torch.cuda.synchronize()
    assert out.shape == (7, 1, 128)
    assert_same(host_u16(out), kv_cache.kv_read_ref(cache, slots, s), f"restore at {scale}")


def test_read_strided_output_and_odd_heads():
    T, H, D, nb, bs = 41, 3, 24, 6, 9
    rng = np.random.default_rng(9)
    cache = rng.integers(0, 256, (nb, bs, H, D), dtype=np.uint8)
    slots = rng.integers(-3, nb * bs + 3, T).astype(np.int64)
    s = np.float32(0.0421)
    wide = torch.full((T, 2 * H * D), -1.0, dtype=torch.bfloat16, device="cuda")
    out = wide[:, H * D:].view(T, H, D)
    fp8.kv_cache_read(torch.from_numpy(cache).cuda(), torch.from_numpy(slots).cuda(),
                      dev_scale(s), out=out)
    torch.cuda.synchronize()
    got = host_u16(wide)
    assert_same(got[:, H * D:].reshape(T, H, D), kv_cache.kv_read_ref(cache, slots, s), "restore")
    assert (got[:, :H * D] == 0xBF80).all()                      # the other half untouched


def test_empty_and_zero_capacity():
    H, D = 2, 16
    e = torch.empty((0, H, D), dtype=torch.bfloat16, device="cuda")
    kc = torch.full((2, 4, H, D), 7, dtype=torch.uint8, device="cuda")
    vc = torch.full((2, 4, H, D), 9, dtype=torch.uint8, device="cuda")
    one = dev_scale(1.0)
    no_slots = torch.empty((0,), dtype=torch.int64, device="cuda")
    fp8.kv_cache_write(e, e, no_slots, kc, vc, one, one)
    assert fp8.kv_cache_read(kc, no_slots, one).shape == (0, H, D)
    # a cache with no blocks: nothing is stored, every token reads zeros
    x = dev_bf16(synth.make_kv(7, 6, H, D, 4, 2, 1)["key"])
    z = torch.empty((0, 4, H, D), dtype=torch.uint8, device="cuda")
    sl = torch.arange(6, dtype=torch.int64, device="cuda")
    fp8.kv_cache_write(x, x, sl, z, z.clone(), one, one)
    out = fp8.kv_cache_read(z, sl, one)
    torch.cuda.synchronize()
    assert (host_u16(out) == 0).all()
    assert (kc == 7).all().item() and (vc == 9).all().item()


def test_full_workload_sampled():
    c = synth.KV_CONFIG
    T, H, D, bs, nb = c["T"], c["H"], c["D"], c["block_size"], c["num_blocks"]
    log("kv full workload", (T, H, D, nb, bs))
    d = synth.make_kv(c["cfg"], T, H, D, bs, nb, c["n_seqs"], c["key_outlier_dims"],
                      c["key_outlier_mult"], c["pad_frac"])
    kc = torch.full((nb, bs, H, D), 0x5A, dtype=torch.uint8, device="cuda")
    vc = torch.full((nb, bs, H, D), 0x5A, dtype=torch.uint8, device="cuda")
    ks, vs = amax_scale(d["key"]), np.float32(1.0)
    slots = torch.from_numpy(d["slots"]).cuda()
    fp8.kv_cache_write(dev_bf16(d["key"]), dev_bf16(d["value"]), slots, kc, vc, dev_scale(ks),
                       dev_scale(vs))
    kout = fp8.kv_cache_read(kc, slots, dev_scale(ks))
    vout = fp8.kv_cache_read(vc, slots, dev_scale(vs))
    torch.cuda.synchronize()
    rng = np.random.default_rng(10)
    sample = np.unique(np.concatenate([[0, T - 1], rng.choice(T, 62, replace=False)]))
    sl = d["slots"][sample]
    kc_flat = kc.view(nb * bs, H, D)
    vc_flat = vc.view(nb * bs, H, D)
    idx = torch.from_numpy(sl).cuda()
    for name, x, cache, out, s in (("keys", d["key"], kc_flat, kout, ks),
                                   ("values", d["value"], vc_flat, vout, vs)):
        want = np.zeros((len(sample), 1, H, D), dtype=np.uint8)
        want = kv_cache.kv_write_ref(x[sample], np.arange(len(sample)), want, s)
        assert_same(cache[idx].cpu().numpy(), want[:, 0], name + " codes")
        back = kv_cache.kv_read_ref(want, np.arange(len(sample)), s)
        assert_same(host_u16(out[torch.from_numpy(sample).cuda()]), back, name + " restored")
    # slots no token names keep their bytes
    used = np.zeros(nb * bs, dtype=bool)
    used[d["slots"][d["slots"] >= 0]] = True
    free = np.flatnonzero(~used)
    pick = torch.from_numpy(rng.choice(free, 256, replace=False)).cuda()
    assert (kc_flat[pick] == 0x5A).all().item() and (vc_flat[pick] == 0x5A).all().item()
