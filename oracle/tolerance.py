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
  3. gates on the literal Frobenius bound, never relaxed.
"""

import numpy as np

MAXABS_REL = 1e-2
FROB_REL = 4e-3


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


def rms(ref):
    ref = np.asarray(ref, dtype=np.float64)
    return float(np.sqrt(np.mean(ref * ref))) if ref.size else 0.0


def check(out_bits, ref):
    """Compare bf16 output bits with the fp64 reference.

    Returns a dict with the literal metrics, the bf16 floor, the
    rounding-aware gate and the share of outputs that equal bf16_RNE(ref).
    ``ok`` is the gate (items 2 and 3 of the module docstring).
    """
    out = bf16_bits_to_f64(out_bits)
    ref = np.asarray(ref, dtype=np.float64)
    assert out.shape == ref.shape
    r = rms(ref)
    err = np.abs(out - ref)
    ref_norm = float(np.linalg.norm(ref))
    frob = float(np.linalg.norm(out - ref)) / ref_norm if ref_norm > 0 else float(np.linalg.norm(out))
    rounded = bf16_rne(ref)
    floor_abs = np.abs(rounded - ref)
    bound = MAXABS_REL * r + 0.5 * bf16_ulp(np.maximum(np.abs(out), np.abs(ref)))
    gate_elem = bool(np.all(err <= bound)) if ref.size else True
    denom = r if r > 0 else 1.0
    res = {
        "rms_ref": r,
        "maxabs_over_rms": float(err.max() / denom) if ref.size else 0.0,
        "floor_maxabs_over_rms": float(floor_abs.max() / denom) if ref.size else 0.0,
        "literal_maxabs_ok": bool(err.max() <= MAXABS_REL * r) if ref.size else True,
        "frob_rel": frob,
        "frob_ok": frob <= FROB_REL,
        "elementwise_gate_ok": gate_elem,
        "n_over_literal": int(np.sum(err > MAXABS_REL * r)),
        "frac_equal_rne": float(np.mean(out == rounded)) if ref.size else 1.0,
    }
    res["ok"] = bool(res["elementwise_gate_ok"] and res["frob_ok"])
    return res
