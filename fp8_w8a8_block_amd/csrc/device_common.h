// Device helpers shared by the gfx950 kernels: bf16 unpacking, 16-lane DPP
// reductions, the exact quotient x / s and the E4M3 element encoder.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace fp8k {

constexpr int kGroup = 128;          // K-group / block edge
constexpr float kE4M3Max = 448.0f;   // largest E4M3 magnitude

// ---- bf16 -> fp32 (exact widening of the two halves of a dword) ----------
__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

// Largest |bf16| of the two halves, as the bit pattern of a non-negative
// fp32.  Bit patterns of non-negative floats order like the values.
__device__ __forceinline__ uint32_t bf16x2_absmax_bits(uint32_t w) {
  uint32_t lo = (w << 16) & 0x7fff0000u;
  uint32_t hi = w & 0x7fff0000u;
  return lo > hi ? lo : hi;
}

// ---- 16-lane (one DPP row) max of non-negative values given as bits -------
// row_ror:n rotates inside each row of 16 lanes; after rotations by 8, 4, 2
// and 1 every lane holds the maximum of its row.
__device__ __forceinline__ uint32_t row16_max(uint32_t v) {
  uint32_t t;
  t = (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x128, 0xf, 0xf, false);  // row_ror:8
  v = v > t ? v : t;
  t = (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x124, 0xf, 0xf, false);  // row_ror:4
  v = v > t ? v : t;
  t = (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x122, 0xf, 0xf, false);  // row_ror:2
  v = v > t ? v : t;
  t = (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x121, 0xf, 0xf, false);  // row_ror:1
  v = v > t ? v : t;
  return v;
}

// Max over the whole 64-lane wave (result valid in every lane).
__device__ __forceinline__ uint32_t wave_max(uint32_t v) {
  v = row16_max(v);
  // combine the four rows: lanes read row r^1 and r^2 through ds_swizzle-free
  // readlane of one lane per row (uniform result)
  uint32_t r0 = __builtin_amdgcn_readlane(v, 0);
  uint32_t r1 = __builtin_amdgcn_readlane(v, 16);
  uint32_t r2 = __builtin_amdgcn_readlane(v, 32);
  uint32_t r3 = __builtin_amdgcn_readlane(v, 48);
  uint32_t a = r0 > r1 ? r0 : r1;
  uint32_t b = r2 > r3 ? r2 : r3;
  return a > b ? a : b;
}

// ---- per-group divisor set-up --------------------------------------------
// For a group with largest magnitude amax the scale is s = fp32(amax) / 448
// (IEEE division).  The quotient x / s is then formed as x' / s' with
// s' = s * 2^k in [1, 2) and x' = x * 2^k: the same real quotient, so the
// same fp32 rounding.  r = fp32(1 / s') seeds a one-step correction
//   q0 = x' r ;  e = fma(-q0, s', x') (exact) ;  q = fma(e, r, q0)
// which equals the correctly rounded fp32 quotient for every (amax, x) pair
// of bf16 inputs with |x| <= amax; that is checked exhaustively on the host
// by the test suite.  An all-zero group (amax = 0) gets s = 0 and k = 0,
// s' = r = 1, so its codes are the signed zeros of x.
struct GroupDivisor {
  float s;    // the scale written out
  float sp;   // s' in [1, 2)
  float r;    // fp32(1 / s')
  int k;      // exponent shift applied to |x|
};

__device__ __forceinline__ GroupDivisor make_divisor(float amax) {
  GroupDivisor d;
  d.s = amax / kE4M3Max;
  if (d.s == 0.0f) {
    d.sp = 1.0f;
    d.r = 1.0f;
    d.k = 0;
  } else {
    int e = __builtin_amdgcn_frexp_expf(d.s);          // s = f * 2^e, f in [0.5, 1)
    d.k = 1 - e;
    d.sp = __builtin_ldexpf(d.s, d.k);
    d.r = 1.0f / d.sp;
  }
  return d;
}

// |x| / s correctly rounded to fp32, for |x| <= amax of the group.
__device__ __forceinline__ float quotient_abs(float x, const GroupDivisor& d) {
  float xa = __builtin_ldexpf(__builtin_fabsf(x), d.k);
  float q0 = xa * d.r;
  float e = __builtin_fmaf(-q0, d.sp, xa);
  return __builtin_fmaf(e, d.r, q0);
}

// ---- E4M3 encoding --------------------------------------------------------
// Four non-negative quotients q0..q3 (each <= 464, no NaN) to four magnitude
// codes in one dword, byte i = code of q_i.  The gfx950 conversion rounds to
// nearest even in the OCP E4M3 format; 448 <= q < 464 rounds to 448.
__device__ __forceinline__ uint32_t e4m3_pack4_mag(float q0, float q1, float q2, float q3) {
  int w = __builtin_amdgcn_cvt_pk_fp8_f32(q0, q1, 0, false);
  w = __builtin_amdgcn_cvt_pk_fp8_f32(q2, q3, w, true);
  return (uint32_t)w;
}

// Sign bits of four bf16 values held in two dwords (d0 = x1:x0, d1 = x3:x2),
// placed at bit 7 of bytes 0..3.  v_perm picks the high byte of each bf16.
__device__ __forceinline__ uint32_t bf16x4_signs(uint32_t d0, uint32_t d1) {
  return __builtin_amdgcn_perm(d1, d0, 0x07050301u) & 0x80808080u;
}

// Full element encoder for arbitrary fp32 (saturating, NaN aware).
__device__ __forceinline__ uint8_t e4m3_encode_one(float x) {
  uint32_t bits = __float_as_uint(x);
  uint32_t sign = (bits >> 24) & 0x80u;
  if (x != x) return (uint8_t)(0x7fu | sign);
  float a = __builtin_fminf(__builtin_fabsf(x), kE4M3Max);
  int w = __builtin_amdgcn_cvt_pk_fp8_f32(a, 0.0f, 0, false);
  return (uint8_t)((w & 0xff) | sign);
}

// Quantize the 8 bf16 values a lane holds (uint4) with the group divisor;
// returns the 8 codes as a uint2 (byte i = element i).
__device__ __forceinline__ uint2 quant8(const uint4 v, const GroupDivisor& d) {
  uint32_t c0 = e4m3_pack4_mag(quotient_abs(bf16_lo(v.x), d), quotient_abs(bf16_hi(v.x), d),
                               quotient_abs(bf16_lo(v.y), d), quotient_abs(bf16_hi(v.y), d));
  uint32_t c1 = e4m3_pack4_mag(quotient_abs(bf16_lo(v.z), d), quotient_abs(bf16_hi(v.z), d),
                               quotient_abs(bf16_lo(v.w), d), quotient_abs(bf16_hi(v.w), d));
  c0 |= bf16x4_signs(v.x, v.y);
  c1 |= bf16x4_signs(v.z, v.w);
  return make_uint2(c0, c1);
}

// ---- division by a static scale ------------------------------------------
// A static scale s holds for a whole launch (calibrated activation scales,
// KV-cache scales).  For a normal finite s the quotient x / s is formed with
// the steps of the group divisor above: s' = |s| * 2^k in [1, 2),
// r = fp32(1 / s') once, then per element x' = |x| * 2^k, q0 = x' r,
// e = fma(-q0, s', x'), q = fma(e, r, q0).  An exhaustive host check in the
// test suite (every fp32 mantissa of s' against every bf16 mantissa of x',
// across the range where the E4M3 code depends on the quotient) shows q is
// the IEEE quotient bit for bit.  Outside that range the code is the zero
// code (x' underflows: the quotient is below 2^-126) or saturates (x'
// overflows, or x is infinite: q turns NaN and is clamped to 448).  A zero,
// subnormal, infinite or NaN scale divides directly, and so does any chunk
// holding a NaN input (its code keeps the input's sign, as a division does).
struct StaticDivisor {
  float s;        // the scale (direct-division path)
  float sp;       // s' in [1, 2)
  float r;        // fp32(1 / s')
  int k;          // exponent shift applied to |x|
  uint32_t sign;  // sign of s at bit 7 of every byte
  bool fast;      // s normal and finite
};

__device__ __forceinline__ StaticDivisor make_static_divisor(float s) {
  StaticDivisor d;
  d.s = s;
  const float a = __builtin_fabsf(s);
  d.fast = a >= 0x1p-126f && a <= 0x1.fffffep127f;    // false for NaN
  d.sign = (__float_as_uint(s) >> 31) * 0x80808080u;
  d.k = 0;
  d.sp = 1.0f;
  d.r = 1.0f;
  if (d.fast) {
    const int e = __builtin_amdgcn_frexp_expf(a);       // a = f * 2^e, f in [0.5, 1)
    d.k = 1 - e;
    d.sp = __builtin_ldexpf(a, d.k);
    d.r = 1.0f / d.sp;
  }
  return d;
}

// |x| / |s| for the fast path, clamped to 448 (NaN from an overflowed x' too)
__device__ __forceinline__ float static_quotient_abs(float x, const StaticDivisor& d) {
  const float xa = __builtin_ldexpf(__builtin_fabsf(x), d.k);
  const float q0 = xa * d.r;
  const float e = __builtin_fmaf(-q0, d.sp, xa);
  const float q = __builtin_fmaf(e, d.r, q0);
  return q < kE4M3Max ? q : kE4M3Max;
}

// Nonzero iff one of the two bf16 halves of w is a NaN (|h| > 0x7f80).
__device__ __forceinline__ uint32_t bf16x2_nan(uint32_t w) {
  return ((w & 0x7fff7fffu) + 0x007f007fu) & 0x80008000u;
}

// E4M3 codes of 8 bf16 values divided by a static scale (byte i = element i),
// equal to E4M3(fp32(x) / s) with an IEEE division.
__device__ __forceinline__ uint2 quant8_static(const uint4 v, const StaticDivisor& d) {
  const uint32_t nan = bf16x2_nan(v.x) | bf16x2_nan(v.y) | bf16x2_nan(v.z) | bf16x2_nan(v.w);
  if (!d.fast || nan) {
    const uint32_t w[4] = {v.x, v.y, v.z, v.w};
    uint32_t o[2] = {0u, 0u};
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const float xe = (e & 1) ? bf16_hi(w[e >> 1]) : bf16_lo(w[e >> 1]);
      o[e >> 2] |= (uint32_t)e4m3_encode_one(xe / d.s) << (8 * (e & 3));
    }
    return make_uint2(o[0], o[1]);
  }
  uint32_t c0 = e4m3_pack4_mag(static_quotient_abs(bf16_lo(v.x), d),
                               static_quotient_abs(bf16_hi(v.x), d),
                               static_quotient_abs(bf16_lo(v.y), d),
                               static_quotient_abs(bf16_hi(v.y), d));
  uint32_t c1 = e4m3_pack4_mag(static_quotient_abs(bf16_lo(v.z), d),
                               static_quotient_abs(bf16_hi(v.z), d),
                               static_quotient_abs(bf16_lo(v.w), d),
                               static_quotient_abs(bf16_hi(v.w), d));
  c0 |= bf16x4_signs(v.x, v.y) ^ d.sign;
  c1 |= bf16x4_signs(v.z, v.w) ^ d.sign;
  return make_uint2(c0, c1);
}

// Largest |x| of 8 bf16 values, as fp32 bits.
__device__ __forceinline__ uint32_t absmax8_bits(const uint4 v) {
  uint32_t a = bf16x2_absmax_bits(v.x);
  uint32_t b = bf16x2_absmax_bits(v.y);
  uint32_t c = bf16x2_absmax_bits(v.z);
  uint32_t e = bf16x2_absmax_bits(v.w);
  a = a > b ? a : b;
  c = c > e ? c : e;
  return a > c ? a : c;
}

// ---- fp32 -> bf16 round to nearest even (finite values) ------------------
__device__ __forceinline__ uint32_t f32_to_bf16_rne(float f) {
  uint32_t u = __float_as_uint(f);
  u += 0x7fffu + ((u >> 16) & 1u);
  return u >> 16;
}

}  // namespace fp8k
