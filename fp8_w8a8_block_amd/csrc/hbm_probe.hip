// HBM read reference for bench.py (a measurement helper, not part of the
// W8A8 path; built into its own libhbmprobe.so).
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

}  // namespace

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
