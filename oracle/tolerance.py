"""Tolerance check of a bf16 GEMM output against the fp64 reference (oracle).

TEST INFRASTRUCTURE ONLY -- not part of the product path.

Stated bar: max|out - ref| <= 1e-2 * rms(ref) and ||out - ref||_F / ||ref||_F
<= 4e-3, with ref the fp64 reference on the same FP8 operands.

Reading (the bar as written sits below bf16's own rounding floor): an output
in the binade [2**e, 2**(e+1)) carries up to 2**(e-8) of pure output
rounding, which exceeds 1e-2 * rms(ref) as soon as |ref| passes about
2.56 * rms(ref) -- so even a correctly rounded bf16(ref) can fail the literal
max-abs bound.  The check therefore

  1. reports the literal max-abs ratio and the same ratio for bf16_RNE(ref)
     (the floor any bf16 output has);
  2. gates elementwise on |out - ref| <= 1e-2 * rms(ref) + ulp/2, where ulp
     is the bf16 spacing at max(|out|, |ref|) -- the literal bound plus the
     unavoidable output rounding;
  3. gates on the literal Frobenius bound, never relaxed;
  4. gates elementwise on |out - ref| <= B + ulp(out)/2, where B bounds the
     error any fp32 accumulation of the same sum can make (below);
  5. gates on "out equals bf16_RNE(ref) or one of its two bf16 neighbours"
     wherever B <= ulp(ref)/4, and reports the largest ulp distance of out
     from bf16_RNE(ref) over all outputs.

The accumulation bound B.  The kernels multiply FP8 codes exactly (a product
of two E4M3 values has at most 8 significant bits), add them up in fp32 and
fold in the scales in fp32.  Write T[m, n] for the same reference computed on
absolute values: T = sum_kb |sa * sw| * sum_{k in kb} |dec(qa) * dec(qw)|
(block scales; |sa * sw| * sum_k |dec * dec| for scales constant along K).
Every partial sum any summation order forms is bounded by T, so each fp32
rounding (relative error at most 2**-23, which also covers truncation) adds
at most 2**-23 * T, and an accumulation with at most n roundings stays within
n * 2**-23 * T of the exact value (to first order; a 2**-10 relative margin
covers the rest).  The count n is taken as small as the structure of the
arithmetic allows without trusting the matrix unit's internal order:

  * block scales: one 128-term block sum restarts from zero for each K block
    (at most 127 roundings, however the unit orders them, each bounded by
    that block's share of T, so 127 * 2**-23 * T over all blocks), the scale
    products sa * sw (one rounding per block, 2**-23 * T over all blocks),
    one rounding per K block for the fold into the accumulator (each bounded
    by 2**-23 * T), and at most 16 more for sums of partial accumulators:
    n = 128 + K / 128 + 16;
  * scales constant along K: the K products may be chained into one
    accumulator (at most K roundings), then the scale product and the final
    multiply (two more), and the same 16 partial-sum roundings:
    n = K + 2 + 16.

Where B <= ulp(ref)/4 (a quarter of the bf16 spacing at |ref|, i.e. half the
spacing of the binade below), the interval between the fp32 accumulator and
ref holds at most one rounding midpoint of the bf16 grid, so a correctly
rounded output is bf16_RNE(ref) or its neighbour: the clause is exact there,
and only outputs with |ref| this close to the cancellation floor are exempt
from it (they are still held to item 4).
"""

import numpy as np

MAXABS_REL = 1e-2
FROB_REL = 4e-3
U_FP32 = 2.0 ** -23             # relative size of one fp32 rounding (RNE or truncation)
GROUP = 128
EXTRA_ROUNDINGS = 16            # sums of partial accumulators (split K across waves)


def bf16_bits_to_f64(bits):
    b = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
    return b.view(np.float32).astype(np.float64)


def bf16_ulp(v):
    """Spacing of the bf16 grid at |v| (8 significant bits; subnormal step 2**-133)."""
    a = np.abs(np.asarray(v, dtype=np.float64))
    _, e = np.frexp(a)                       # a = f * 2**e, f in [0.5, 1)
    ulp = np.ldexp(1.0, e - 8)
    return np.where(a < 2.0 ** -126, 2.0 ** -133, ulp)


def bf16_rne(v):
    """Round float64 values to the nearest bf16 value, ties to even (finite range)."""
    v = np.asarray(v, dtype=np.float64)
    q = bf16_ulp(v)
    return np.rint(v / q) * q                # rint rounds half to even


def bf16_value_bits(v):
    """Bit patterns (uint16) of float64 values that are already bf16 values."""
    f = np.asarray(v, dtype=np.float64).astype(np.float32)
    return (f.view(np.uint32) >> np.uint32(16)).astype(np.uint16)


def bf16_order_key(bits):
    """Integer key of bf16 bit patterns that orders them like their values,
    with consecutive finite values one apart (+0 and -0 both map to 0)."""
    b = np.asarray(bits, dtype=np.uint16).astype(np.int32)
    mag = b & 0x7FFF
    return np.where(b & 0x8000, -mag, mag)


def ulp_distance(out_bits, ref):
    """Number of bf16 grid steps between out and bf16_RNE(ref)."""
    want = bf16_value_bits(bf16_rne(ref))
    return np.abs(bf16_order_key(out_bits) - bf16_order_key(want))


def rms(ref):
    ref = np.asarray(ref, dtype=np.float64)
    return float(np.sqrt(np.mean(ref * ref))) if ref.size else 0.0


def abs_codes(codes):
    """E4M3 codes with the sign bit cleared: dec(abs_codes(c)) == |dec(c)|."""
    return np.asarray(codes, dtype=np.uint8) & np.uint8(0x7F)


def fp32_roundings(K, mode):
    """Upper bound on the fp32 roundings in one output's accumulation (see
    the module docstring): ``mode`` "block" (scales per 128-wide K block) or
    "tensor" / "row" (scales constant along K)."""
    if mode == "block":
        return 128 + K // GROUP + EXTRA_ROUNDINGS
    return K + 2 + EXTRA_ROUNDINGS


def accumulation_bound(abs_ref, K, mode):
    """B = n * 2**-23 * T (1 + 2**-10), T the reference on absolute values."""
    n = fp32_roundings(K, mode)
    return n * U_FP32 * (1.0 + 2.0 ** -10) * np.abs(np.asarray(abs_ref, dtype=np.float64))


def check(out_bits, ref, bound):
    """Compare bf16 output bits with the fp64 reference.

    ``bound`` is the accumulation bound B (``accumulation_bound``), an array
    of ref's shape or a scalar.  Returns a dict with the literal metrics, the
    bf16 floor, the gates of the module docstring and the ulp-distance
    report; ``ok`` is items 2 to 5 together.
    """
    out = bf16_bits_to_f64(out_bits)
    ref = np.asarray(ref, dtype=np.float64)
    assert out.shape == ref.shape
    B = np.broadcast_to(np.asarray(bound, dtype=np.float64), ref.shape)
    r = rms(ref)
    err = np.abs(out - ref)
    ref_norm = float(np.linalg.norm(ref))
    frob = float(np.linalg.norm(out - ref)) / ref_norm if ref_norm > 0 else float(np.linalg.norm(out))
    rounded = bf16_rne(ref)
    floor_abs = np.abs(rounded - ref)
    bound2 = MAXABS_REL * r + 0.5 * bf16_ulp(np.maximum(np.abs(out), np.abs(ref)))
    gate_elem = bool(np.all(err <= bound2)) if ref.size else True
    gate_acc = bool(np.all(err <= B + 0.5 * bf16_ulp(out))) if ref.size else True
    dist = ulp_distance(out_bits, ref)
    clause = B <= 0.25 * bf16_ulp(ref)           # where the neighbour clause is exact
    n_beyond = int(np.sum(dist > 1))
    n_beyond_covered = int(np.sum((dist > 1) & clause))
    denom = r if r > 0 else 1.0
    res = {
        "rms_ref": r,
        "maxabs_over_rms": float(err.max() / denom) if ref.size else 0.0,
        "floor_maxabs_over_rms": float(floor_abs.max() / denom) if ref.size else 0.0,
        "literal_maxabs_ok": bool(err.max() <= MAXABS_REL * r) if ref.size else True,
        "frob_rel": frob,
        "frob_ok": frob <= FROB_REL,
        "elementwise_gate_ok": gate_elem,
        "accumulation_gate_ok": gate_acc,
        "n_over_literal": int(np.sum(err > MAXABS_REL * r)),
        "frac_equal_rne": float(np.mean(out == rounded)) if ref.size else 1.0,
        "max_ulp": int(dist.max()) if ref.size else 0,
        "n_beyond_1ulp": n_beyond,
        "max_ulp_where_clause_holds": int(dist[clause].max()) if np.any(clause) else 0,
        "n_clause_exempt": int(np.sum(~clause)),
        "neighbour_gate_ok": n_beyond_covered == 0,
    }
    res["ok"] = bool(res["elementwise_gate_ok"] and res["frob_ok"] and res["accumulation_gate_ok"]
                     and res["neighbour_gate_ok"])
    return res
