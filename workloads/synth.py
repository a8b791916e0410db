"""Seeded synthetic bf16 inputs for the five W8A8 workloads and the edge cases.

This module holds no quantization or GEMM arithmetic; both the GPU path and
the oracle receive the same bf16 bit patterns from here.

Recipe (shapes and distributions of the workloads):
  * numpy PCG64 ``default_rng`` seeded with ``[cfg, stream, ...]``:
    W <- [cfg, 0], A <- [cfg, 1, M], outlier channels <- [cfg, 2].
  * Normal draws in float32 (``standard_normal(dtype=float32)``), times the
    standard deviation in float32, rounded to bf16 (round to nearest even).
    "N(0, s)" reads s as the standard deviation.
  * Outlier channels: round(0.001 * K) distinct columns of A (2 for the tiny
    case), drawn without replacement, multiplied by the factor (50, or 100
    for the large case) in float32 before the bf16 rounding; the decode rows
    M in {1, 4, 16} share the channels.
  * The MLP down-projection input is x * sigmoid(x), x ~ N(0, 2), computed in
    float64 before the bf16 rounding (a SiLU-like heavy right tail).
  * KV cache (``make_kv``), seeded ``[cfg, 3, T]``: keys N(0, 1) with a few
    head-dimension channels (the same ones in every head) multiplied by an
    outlier factor, values N(0, 1), both [T, H, D] bf16; T tokens split
    evenly over n_seqs sequences, each sequence's tokens filling its own
    blocks in order, the blocks drawn without replacement from the whole
    pool (a paged cache whose blocks are scattered); a seed-chosen fraction
    of tokens gets slot -1 (padding).
  * MoE (``make_moe``), seeded ``[cfg, 4]`` for routing, ``[cfg, 5]`` for the
    token activations (N(0, 1) with outlier channels as above) and
    ``[cfg, 6, e]`` for expert e's weight (N(0, w_std)): every token picks
    top_k distinct experts of experts_total, without replacement, with
    probabilities proportional to a lognormal popularity (sigma 0.6, drawn
    once: some experts hot, some cold); the experts 0 .. experts_local - 1
    are this GPU's shard, and their (token, expert) pairs, grouped by expert
    and ordered by token within an expert, are the rows of the grouped GEMM.
"""

import numpy as np

__all__ = [
    "CONFIGS", "f32_to_bf16_bits", "bf16_bits_to_f32_input", "make_weight",
    "make_activation", "make_config", "outlier_channels", "edge_activations", "KV_CONFIG",
    "make_kv", "MOE_CONFIGS", "make_moe_routing", "make_moe_tokens", "make_moe_weight",
]


def f32_to_bf16_bits(x):
    """float32 -> bf16 bit patterns, round to nearest even (finite inputs)."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    lsb = (u >> np.uint32(16)) & np.uint32(1)
    r = (u + np.uint32(0x7FFF) + lsb) >> np.uint32(16)
    return r.astype(np.uint16)


def bf16_bits_to_f32_input(bits):
    """bf16 bit patterns -> float32 (exact widening), for building inputs."""
    return (np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


# name -> shape and distribution parameters
CONFIGS = {
    "tiny":     dict(cfg=1, M=16,   K=512,   N=256,   a_kind="normal", a_std=1.0, w_std=0.02,
                     n_outliers=2, outlier_mult=50.0),
    "decode":   dict(cfg=2, M=16,   K=4096,  N=11008, a_kind="normal", a_std=1.0, w_std=0.02,
                     n_outliers=None, outlier_mult=50.0, decode_m=(1, 4, 16)),
    "prefill":  dict(cfg=3, M=4096, K=4096,  N=4096,  a_kind="normal", a_std=1.0, w_std=0.02,
                     n_outliers=None, outlier_mult=50.0),
    "mlp_down": dict(cfg=4, M=2048, K=14336, N=4096,  a_kind="silu",   a_std=2.0, w_std=0.015,
                     n_outliers=0, outlier_mult=1.0),
    "large":    dict(cfg=5, M=8192, K=8192,  N=28672, a_kind="normal", a_std=1.0, w_std=0.01,
                     n_outliers=None, outlier_mult=100.0),
}


# paged FP8 KV cache: 8 KV heads of 128 (a grouped-query 8B-class model),
# 16-token blocks, a 1 GiB pool per cache, 64 sequences of 1024 tokens
KV_CONFIG = dict(cfg=6, T=65536, H=8, D=128, block_size=16, num_blocks=65536, n_seqs=64,
                 key_outlier_dims=4, key_outlier_mult=20.0, pad_frac=0.0)


def make_kv(cfg, T, H, D, block_size, num_blocks, n_seqs, key_outlier_dims=4,
            key_outlier_mult=20.0, pad_frac=0.0):
    """Return dict(key=bits [T,H,D], value=bits [T,H,D], slots=int64 [T])."""
    rng = np.random.default_rng([cfg, 3, T])
    key = rng.standard_normal((T, H, D), dtype=np.float32)
    if key_outlier_dims:
        dims = rng.choice(D, size=min(key_outlier_dims, D), replace=False)
        key[:, :, dims] *= np.float32(key_outlier_mult)
    value = rng.standard_normal((T, H, D), dtype=np.float32)
    lens = np.full(n_seqs, T // n_seqs, dtype=np.int64)
    lens[: T % n_seqs] += 1
    need = int(sum(-(-int(n) // block_size) for n in lens))
    if need > num_blocks:
        raise ValueError(f"{need} blocks needed, pool has {num_blocks}")
    pool = rng.permutation(num_blocks)[:need]
    slots = np.empty(T, dtype=np.int64)
    t = b = 0
    for n in lens:
        i = np.arange(n)
        blk = pool[b + i // block_size]
        slots[t:t + n] = blk * block_size + i % block_size
        t += int(n)
        b += -(-int(n) // block_size)
    if pad_frac > 0:
        slots[rng.random(T) < pad_frac] = -1
    return dict(key=f32_to_bf16_bits(key), value=f32_to_bf16_bits(value), slots=slots)


# MoE layer, one GPU's expert shard: 256 experts of hidden 7168, the gate and
# up projections fused (N = 2 * 2048), top-8 routing, 32 experts per GPU
# (expert parallelism over 8 GPUs); a decode batch and a prefill chunk
MOE_CONFIGS = {
    "moe_decode":  dict(cfg=7, tokens=256,  top_k=8, experts_total=256, experts_local=32,
                        K=7168, N=4096, w_std=0.02, n_outliers=None, outlier_mult=20.0),
    "moe_prefill": dict(cfg=8, tokens=8192, top_k=8, experts_total=256, experts_local=32,
                        K=7168, N=4096, w_std=0.02, n_outliers=None, outlier_mult=20.0),
}


def make_moe_routing(cfg, tokens, top_k, experts_total, experts_local):
    """Routing of one batch: (token index of each row [M], offsets [E_local + 1])."""
    rng = np.random.default_rng([cfg, 4])
    logp = rng.standard_normal(experts_total) * 0.6
    # Gumbel-top-k: top_k distinct experts per token, P(e) proportional to exp(logp[e])
    g = logp[None, :] - np.log(-np.log(rng.random((tokens, experts_total))))
    choice = np.argpartition(-g, top_k - 1, axis=1)[:, :top_k]
    rows, counts = [], []
    for e in range(experts_local):
        tok = np.flatnonzero((choice == e).any(axis=1))
        rows.append(tok)
        counts.append(len(tok))
    offsets = np.concatenate([[0], np.cumsum(counts)]).astype(np.int64)
    return np.concatenate(rows).astype(np.int64), offsets


def make_moe_tokens(cfg, tokens, K, n_outliers=None, mult=20.0):
    """Token activations bf16 bits [tokens, K] ~ N(0, 1), outlier channels times mult."""
    rng = np.random.default_rng([cfg, 5])
    x = rng.standard_normal((tokens, K), dtype=np.float32)
    ch = outlier_channels(cfg, K, n_outliers)
    if len(ch):
        x[:, ch] *= np.float32(mult)
    return f32_to_bf16_bits(x)


def make_moe_weight(cfg, e, N, K, std):
    """Expert e's weight, bf16 bits [N, K] ~ N(0, std)."""
    rng = np.random.default_rng([cfg, 6, e])
    return f32_to_bf16_bits(rng.standard_normal((N, K), dtype=np.float32) * np.float32(std))


def outlier_channels(cfg, K, n_outliers=None):
    """Seed-chosen outlier columns: round(0.001*K) of them unless given."""
    n = int(round(0.001 * K)) if n_outliers is None else int(n_outliers)
    if n == 0:
        return np.zeros(0, dtype=np.int64)
    rng = np.random.default_rng([cfg, 2])
    return np.sort(rng.choice(K, size=n, replace=False)).astype(np.int64)


def make_weight(cfg, N, K, std, row_chunk=2048):
    """W bf16 bits [N, K] ~ N(0, std), drawn in row chunks to bound memory."""
    rng = np.random.default_rng([cfg, 0])
    out = np.empty((N, K), dtype=np.uint16)
    sd = np.float32(std)
    for r0 in range(0, N, row_chunk):
        r1 = min(N, r0 + row_chunk)
        x = rng.standard_normal((r1 - r0, K), dtype=np.float32) * sd
        out[r0:r1] = f32_to_bf16_bits(x)
    return out


def make_activation(cfg, M, K, kind, std, channels, mult):
    """A bf16 bits [M, K]; outlier channels multiplied before the bf16 rounding."""
    rng = np.random.default_rng([cfg, 1, M])
    if kind == "normal":
        x = rng.standard_normal((M, K), dtype=np.float32) * np.float32(std)
    elif kind == "silu":
        z = rng.standard_normal((M, K)) * float(std)
        x = (z / (1.0 + np.exp(-z))).astype(np.float32)
    else:
        raise ValueError(kind)
    if len(channels):
        x[:, channels] *= np.float32(mult)
    return f32_to_bf16_bits(x)


def make_config(name, M=None):
    """Return dict(A=bits [M,K], W=bits [N,K], M, K, N, channels, cfg)."""
    c = CONFIGS[name]
    M = c["M"] if M is None else int(M)
    K, N = c["K"], c["N"]
    ch = outlier_channels(c["cfg"], K, c["n_outliers"])
    A = make_activation(c["cfg"], M, K, c["a_kind"], c["a_std"], ch, c["outlier_mult"])
    W = make_weight(c["cfg"], N, K, c["w_std"])
    return dict(A=A, W=W, M=M, K=K, N=N, channels=ch, cfg=c["cfg"], name=name)


def edge_activations():
    """Named edge-case activation tensors (bf16 bits), each a few groups wide.

    zeros / negzero: all-zero groups with +0 and -0; tiny: groups whose amax
    is a bf16 subnormal or near the smallest normal (subnormal scales);
    huge: amax near the bf16 maximum; mixed: zero groups next to normal ones;
    single: one nonzero element per group; ragged_m: 3 rows (odd M).
    """
    rng = np.random.default_rng([99, 1])
    K = 512
    cases = {}
    cases["zeros"] = np.zeros((2, K), dtype=np.uint16)
    cases["negzero"] = np.full((2, K), 0x8000, dtype=np.uint16)
    # tiny magnitudes: random bf16 subnormals (exponent field 0) and small normals
    t = rng.integers(1, 0x80, size=(4, K), dtype=np.uint16)            # subnormal bf16
    t |= (rng.integers(0, 2, size=(4, K), dtype=np.uint16) << np.uint16(15))
    t[2:] = rng.integers(0x0080, 0x0400, size=(2, K), dtype=np.uint16)  # 2^-126..~1e-37
    cases["tiny"] = t
    h = rng.integers(0x7E00, 0x7F7F, size=(2, K), dtype=np.uint16)     # ~1e37..3.4e38
    h |= (rng.integers(0, 2, size=(2, K), dtype=np.uint16) << np.uint16(15))
    cases["huge"] = h
    m = f32_to_bf16_bits(rng.standard_normal((4, K), dtype=np.float32))
    m[0, :128] = 0
    m[1, 128:256] = 0x8000
    m[2, 256:384] = f32_to_bf16_bits(rng.standard_normal(128, dtype=np.float32) * np.float32(1e-30))
    cases["mixed"] = m
    s = np.zeros((2, K), dtype=np.uint16)
    for g in range(K // 128):
        s[0, g * 128 + int(rng.integers(0, 128))] = f32_to_bf16_bits(
            np.array([rng.standard_normal()], dtype=np.float32))[0]
        s[1, g * 128 + int(rng.integers(0, 128))] = 0xBF80           # -1.0
    cases["single"] = s
    cases["ragged_m"] = f32_to_bf16_bits(rng.standard_normal((3, K), dtype=np.float32) * np.float32(3.0))
    # every positive finite bf16 value as a group's amax, with random bf16
    # values below it in the group: covers all scale binades incl. subnormal s
    allpos = np.arange(1, 0x7F80, dtype=np.uint16)                      # 32639 values
    G = allpos.size
    body = rng.integers(0, 0x7F80, size=(G, 128), dtype=np.uint16)
    body = np.minimum(body, allpos[:, None])                            # |x| <= amax in bits order
    body[:, int(0)] = allpos
    body |= (rng.integers(0, 2, size=(G, 128), dtype=np.uint16) << np.uint16(15))
    perm = rng.permuted(np.tile(np.arange(128), (G, 1)), axis=1)
    body = np.take_along_axis(body, perm, axis=1)
    pad = (-G) % 4
    body = np.concatenate([body, np.zeros((pad, 128), dtype=np.uint16)])
    cases["all_amax"] = body.reshape(-1, 512)
    return cases
