// Measurement references for bench.py (helpers, not part of the W8A8 path;
// built into their own libhbmprobe.so): an HBM streaming read and a
// matrix-unit-only FP8 chain.
//
// A plain streaming read: workgroup b reads the contiguous slab
// [b * per, (b + 1) * per) of 16-byte words, four loads in flight per
// thread, folds them with XOR and stores one word per thread, so the loads
// cannot be dropped.  Its GB/s over a buffer larger than the Infinity Cache
// is what the memory system delivers to a read-only kernel, the ceiling the
// HBM-bound kernels are read against.
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {

__global__ __launch_bounds__(256) void hbm_read_kernel(const uint4* __restrict__ src, uint64_t n16,
                                                       uint32_t* __restrict__ out) {
  const uint64_t per = (n16 + gridDim.x - 1) / gridDim.x;
  const uint64_t lo = (uint64_t)blockIdx.x * per;
  const uint64_t hi = lo + per < n16 ? lo + per : n16;
  uint32_t acc = 0;
  for (uint64_t i = lo + threadIdx.x; i < hi; i += 4 * 256) {
    uint4 v[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const uint64_t k = i + (uint64_t)j * 256;
      v[j] = k < hi ? src[k] : make_uint4(0, 0, 0, 0);
    }
#pragma unroll
    for (int j = 0; j < 4; ++j) acc ^= v[j].x ^ v[j].y ^ v[j].z ^ v[j].w;
  }
  out[(uint64_t)blockIdx.x * 256 + threadIdx.x] = acc;
}

typedef int v8i_t __attribute__((ext_vector_type(8)));
typedef float v4f_t __attribute__((ext_vector_type(4)));

// The matrix unit alone: every wave keeps four activation and four weight
// fragments of E4M3 codes in registers (read once from `codes`, 32 bytes per
// lane each) and runs `iters` rounds of 16 v_mfma_f32_16x16x128_f8f6f4, one
// per (activation, weight) pair, into 16 independent accumulators, so
// consecutive instructions never wait on each other and every operand
// changes from one instruction to the next, as in a GEMM's K loop.  The
// accumulators are folded into one word per thread and stored, so nothing
// can be dropped.  FLOP = grid * 512 / 64 * iters * 16 * 2 * 16 * 16 * 128.
__global__ __launch_bounds__(512) void mfma_chain_kernel(const uint8_t* __restrict__ codes,
                                                         int iters, uint32_t* __restrict__ out) {
  const uint32_t lane = threadIdx.x & 63u;
  const uint32_t wave = (blockIdx.x * 8u + (threadIdx.x >> 6)) & 63u;
  // 64 waves' worth of distinct fragments: 8 KiB per wave of the 512 KiB
  const v8i_t* src = reinterpret_cast<const v8i_t*>(codes + (size_t)wave * 16384u);
  v8i_t a[4], b[4];
#pragma unroll
  for (int f = 0; f < 4; ++f) {
    a[f] = src[f * 64 + lane];
    b[f] = src[(4 + f) * 64 + lane];
  }
  v4f_t acc[16];
#pragma unroll
  for (int k = 0; k < 16; ++k) acc[k] = v4f_t{0.f, 0.f, 0.f, 0.f};
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int k = 0; k < 16; ++k)
      acc[k] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a[k & 3], b[k >> 2], acc[k], 0, 0,
                                                                0, 0, 0, 0);
  }
  uint32_t h = 0;
#pragma unroll
  for (int k = 0; k < 16; ++k)
    h ^= __float_as_uint(acc[k].x) ^ __float_as_uint(acc[k].y) ^ __float_as_uint(acc[k].z) ^
         __float_as_uint(acc[k].w);
  out[(size_t)blockIdx.x * 512u + threadIdx.x] = h;
}

}  // namespace

// codes: device buffer of 1 MiB of E4M3 codes (16-byte aligned); out: device
// buffer of grid * 512 words.  Returns 0, or the launch's hipError_t.
extern "C" int mfma_chain_probe(const void* codes, int iters, uint32_t* out, int grid,
                                void* stream) {
  if (!codes || !out || grid <= 0 || iters <= 0 || ((uintptr_t)codes & 15u) != 0)
    return (int)hipErrorInvalidValue;
  hipLaunchKernelGGL(mfma_chain_kernel, dim3((uint32_t)grid), dim3(512), 0, (hipStream_t)stream,
                     (const uint8_t*)codes, iters, out);
  return (int)hipGetLastError();
}

// src: device buffer of `bytes` bytes (a multiple of 16, 16-byte aligned);
// out: device buffer of grid * 256 words.  Returns 0, or the launch's
// hipError_t.
extern "C" int hbm_read_probe(const void* src, uint64_t bytes, uint32_t* out, int grid,
                              void* stream) {
  if (!src || !out || grid <= 0 || bytes % 16 != 0) return (int)hipErrorInvalidValue;
  hipLaunchKernelGGL(hbm_read_kernel, dim3((uint32_t)grid), dim3(256), 0, (hipStream_t)stream,
                     (const uint4*)src, bytes / 16, out);
  return (int)hipGetLastError();
}
