// FP8 KV-cache codec for gfx950: scatter keys and values into a paged E4M3
// cache, and gather them back to bf16.
//
// The pages treat the KV cache as its own quantization target: with an fp8
// KV dtype keys and values are stored as E4M3 instead of 16 bits, halving the
// cache ("FP8 Quantization", D.4; "[vLLM] FP8", KV cache quantization), each
// with its own scale (default 1.0, which clips outliers, or calibrated); a
// paged block holds 16 tokens, and outside an FP8 attention backend the codes
// are restored to 16 bits inside the attention kernel ("Quantization guide
// for serving: FP8, AWQ, GPTQ", KV-cache FP8 section).  Here:
//   write: cache[slot(t)][h][d] = E4M3(x[t][h][d] / scale)   (the IEEE
//          quotient, formed exactly with one reciprocal per thread; round to
//          nearest even, saturating; tokens whose slot is negative or past
//          the cache are not stored)
//   read:  out[t][h][d] = bf16_RNE(dec(cache[slot(t)][h][d]) * scale) in fp32,
//          a NaN product giving the quiet NaN with the code's sign; tokens
//          whose slot is out of range read zeros.
// Both are streaming kernels over 8-value chunks (16 bytes of bf16, 8 of
// codes), ordered token-major so a wave covers contiguous bytes of
// consecutive tokens; a write item carries the key and the value chunk of
// one (token, chunk) pair, which share one slot.
#include "device_common.h"
#include "launch.h"

namespace fp8k {

namespace {

// fp32 -> bf16 round to nearest even; a NaN becomes the quiet NaN carrying
// the sign of the stored code (bit 7 of `code`), whatever NaN the multiply made
__device__ __forceinline__ uint32_t bf16_rne_nan(float f, uint32_t code) {
  if (f != f) return 0x7fc0u | ((code & 0x80u) << 8);
  return f32_to_bf16_rne(f);
}

// bf16 of 8 codes times sc
__device__ __forceinline__ uint4 decode8(const uint2 q, float sc) {
  const uint32_t qw[2] = {q.x, q.y};
  uint32_t h[4];
#pragma unroll
  for (int w = 0; w < 2; ++w) {
    // the hardware decodes two E4M3 bytes at a time, exactly, to fp32:
    // bytes 0-1 of the dword, then bytes 2-3
    const auto lo = __builtin_amdgcn_cvt_pk_f32_fp8((int)qw[w], false);
    const auto hi = __builtin_amdgcn_cvt_pk_f32_fp8((int)qw[w], true);
    const uint32_t b = qw[w];
    h[2 * w] = bf16_rne_nan(lo[0] * sc, b) | (bf16_rne_nan(lo[1] * sc, b >> 8) << 16);
    h[2 * w + 1] = bf16_rne_nan(hi[0] * sc, b >> 16) | (bf16_rne_nan(hi[1] * sc, b >> 24) << 16);
  }
  return make_uint4(h[0], h[1], h[2], h[3]);
}

constexpr int kWriteUnroll = 2;   // items per thread per pass (each: K and V chunks)
constexpr int kReadUnroll = 4;

// Item i = (token t, chunk c) of T * cpt; a thread takes items i, i + G, ...
// (G = threads in the grid), U of them per pass with every load issued
// before the first use, so each wave keeps several 16-byte loads in flight
// instead of waiting on the slot and then on the data.  Idx is uint32_t
// when every index fits (cheaper division), else uint64_t.
template <typename Idx>
__global__ __launch_bounds__(256) void kv_write_kernel(
    const uint16_t* __restrict__ k, int64_t ld_k, const uint16_t* __restrict__ v, int64_t ld_v,
    const int64_t* __restrict__ slots, Idx T, uint32_t cpt, uint8_t* __restrict__ kc,
    uint8_t* __restrict__ vc, int64_t capacity, const float* __restrict__ k_scale,
    const float* __restrict__ v_scale) {
  constexpr int U = kWriteUnroll;
  const Idx n = T * cpt;
  const Idx G = (Idx)gridDim.x * 256u;
  const StaticDivisor ks = make_static_divisor(k_scale[0]);
  const StaticDivisor vs = make_static_divisor(v_scale[0]);
  for (Idx i0 = (Idx)blockIdx.x * 256u + threadIdx.x; i0 < n; i0 += U * G) {
    Idx t[U], c[U];
    bool live[U];
    int64_t slot[U];
    uint4 xk[U], xv[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const Idx i = i0 + u * G;
      live[u] = i < n;
      t[u] = live[u] ? i / cpt : 0;
      c[u] = live[u] ? i - t[u] * cpt : 0;
      slot[u] = slots[t[u]];
      xk[u] = *reinterpret_cast<const uint4*>(k + (uint64_t)t[u] * ld_k + (uint64_t)c[u] * 8u);
      xv[u] = *reinterpret_cast<const uint4*>(v + (uint64_t)t[u] * ld_v + (uint64_t)c[u] * 8u);
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      if (!live[u] || slot[u] < 0 || slot[u] >= capacity) continue;
      const uint64_t off = (uint64_t)slot[u] * cpt * 8u + (uint64_t)c[u] * 8u;
      *reinterpret_cast<uint2*>(kc + off) = quant8_static(xk[u], ks);
      *reinterpret_cast<uint2*>(vc + off) = quant8_static(xv[u], vs);
    }
  }
}

template <typename Idx>
__global__ __launch_bounds__(256) void kv_read_kernel(
    const uint8_t* __restrict__ cache, int64_t capacity, uint32_t cpt,
    const int64_t* __restrict__ slots, Idx T, const float* __restrict__ scale,
    uint16_t* __restrict__ out, int64_t ld_out) {
  constexpr int U = kReadUnroll;
  const Idx n = T * cpt;
  const Idx G = (Idx)gridDim.x * 256u;
  const float sc = scale[0];
  for (Idx i0 = (Idx)blockIdx.x * 256u + threadIdx.x; i0 < n; i0 += U * G) {
    Idx t[U], c[U];
    bool live[U], hit[U];
    int64_t slot[U];
    uint2 q[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const Idx i = i0 + u * G;
      live[u] = i < n;
      t[u] = live[u] ? i / cpt : 0;
      c[u] = live[u] ? i - t[u] * cpt : 0;
      slot[u] = slots[t[u]];
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      hit[u] = live[u] && slot[u] >= 0 && slot[u] < capacity;
      q[u] = hit[u] ? *reinterpret_cast<const uint2*>(cache + (uint64_t)slot[u] * cpt * 8u +
                                                      (uint64_t)c[u] * 8u)
                    : make_uint2(0u, 0u);
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      if (!live[u]) continue;
      const uint4 r = hit[u] ? decode8(q[u], sc) : make_uint4(0u, 0u, 0u, 0u);
      *reinterpret_cast<uint4*>(out + (uint64_t)t[u] * ld_out + (uint64_t)c[u] * 8u) = r;
    }
  }
}

uint32_t stream_grid(uint64_t items, int unroll) {
  const uint64_t want = (items + 256 * unroll - 1) / (256 * unroll);
  return (uint32_t)(want < 8192 ? (want ? want : 1) : 8192);
}

// 32-bit item indices when i0 + U * G cannot wrap
bool narrow(uint64_t items, int unroll) {
  return items + (uint64_t)unroll * 8192ull * 256ull < (1ull << 32);
}

}  // namespace

hipError_t launch_kv_write(const uint16_t* k, int64_t ld_k, const uint16_t* v, int64_t ld_v,
                           const int64_t* slots, int64_t T, int64_t HD, uint8_t* kc, uint8_t* vc,
                           int64_t capacity, const float* k_scale, const float* v_scale,
                           hipStream_t st) {
  const uint32_t cpt = (uint32_t)(HD / 8);
  const uint64_t items = (uint64_t)T * cpt;
  const dim3 grid(stream_grid(items, kWriteUnroll));
  if (narrow(items, kWriteUnroll))
    hipLaunchKernelGGL(kv_write_kernel<uint32_t>, grid, dim3(256), 0, st, k, ld_k, v, ld_v, slots,
                       (uint32_t)T, cpt, kc, vc, capacity, k_scale, v_scale);
  else
    hipLaunchKernelGGL(kv_write_kernel<uint64_t>, grid, dim3(256), 0, st, k, ld_k, v, ld_v, slots,
                       (uint64_t)T, cpt, kc, vc, capacity, k_scale, v_scale);
  return hipGetLastError();
}

hipError_t launch_kv_read(const uint8_t* cache, int64_t capacity, int64_t HD, const int64_t* slots,
                          int64_t T, const float* scale, uint16_t* out, int64_t ld_out,
                          hipStream_t st) {
  const uint32_t cpt = (uint32_t)(HD / 8);
  const uint64_t items = (uint64_t)T * cpt;
  const dim3 grid(stream_grid(items, kReadUnroll));
  if (narrow(items, kReadUnroll))
    hipLaunchKernelGGL(kv_read_kernel<uint32_t>, grid, dim3(256), 0, st, cache, capacity, cpt,
                       slots, (uint32_t)T, scale, out, ld_out);
  else
    hipLaunchKernelGGL(kv_read_kernel<uint64_t>, grid, dim3(256), 0, st, cache, capacity, cpt,
                       slots, (uint64_t)T, scale, out, ld_out);
  return hipGetLastError();
}

}  // namespace fp8k
