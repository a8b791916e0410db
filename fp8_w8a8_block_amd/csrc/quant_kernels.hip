// Dynamic FP8 quantizers for gfx950: 1x128 activation groups, 128x128
// weight blocks, whole-tensor scales, and the bare element encoder.
//
// Rule per group G ("[vLLM] FP8", block quantization and scaling strategies;
// "FP8 Quantization", D.2 for run-time activation scales):
//   amax = max |x| over G,  s = fp32(amax) / 448,  code = E4M3(x / s)
// with the quotient correctly rounded in fp32 and the encoding rounded to
// nearest even, saturating (format: "[vLLM] FP8" format table).
//
// The path is HBM-bound: 2 bytes read and 1 + 4/128 bytes written per
// element.  Loads are 16 bytes per lane, 16 lanes per 128-group, so a wave
// reads four consecutive 256-byte groups; the group max is a 16-lane DPP
// reduction with no LDS traffic.
#include "device_common.h"
#include "launch.h"


namespace fp8k {

namespace {

// ---------------------------------------------------------------------------
// 1x128 activation groups.  Block = 256 threads = 16 groups per slot; each
// thread handles GPT groups (GPT loads in flight).  The grid is one run of
// blocks per row: blockIdx.x = row * blocks_per_row + block_in_row.
template <int GPT>
__global__ __launch_bounds__(256) void quant_act_block_kernel(
    const uint16_t* __restrict__ x, int64_t ld_x, uint8_t* __restrict__ q, int64_t ld_q,
    float* __restrict__ s, int64_t ld_s, uint32_t groups_per_row, uint32_t blocks_per_row,
    uint32_t* __restrict__ zero, uint32_t zero_n) {
  if (blockIdx.x == 0)
    for (uint32_t i = threadIdx.x; i < zero_n; i += 256) zero[i] = 0u;
  const uint32_t row = blockIdx.x / blocks_per_row;
  const uint32_t blk = blockIdx.x - row * blocks_per_row;
  const uint32_t lane16 = threadIdx.x & 15u;
  const uint32_t slot = threadIdx.x >> 4;
  const uint16_t* xrow = x + (int64_t)row * ld_x;
  uint8_t* qrow = q + (int64_t)row * ld_q;

  uint4 v[GPT];
  bool ok[GPT];
#pragma unroll
  for (int j = 0; j < GPT; ++j) {
    uint32_t g = (blk * GPT + j) * 16u + slot;
    ok[j] = g < groups_per_row;
    v[j] = ok[j] ? *reinterpret_cast<const uint4*>(xrow + (int64_t)g * kGroup + lane16 * 8u)
                 : make_uint4(0, 0, 0, 0);
  }
#pragma unroll
  for (int j = 0; j < GPT; ++j) {
    uint32_t g = (blk * GPT + j) * 16u + slot;
    uint32_t amax = row16_max(absmax8_bits(v[j]));
    GroupDivisor d = make_divisor(__uint_as_float(amax));
    uint2 c = quant8(v[j], d);
    if (ok[j]) {
      *reinterpret_cast<uint2*>(qrow + (int64_t)g * kGroup + lane16 * 8u) = c;
      if (lane16 == 0) s[(int64_t)row * ld_s + g] = d.s;
    }
  }
}

// The same groups numbered across rows (group f = row * groups_per_row +
// g), so a workgroup's 16 GPT groups run on into the next row instead of
// leaving lanes idle when a row has fewer groups.  f < 2^32 (the caller
// checks).
template <int GPT>
__global__ __launch_bounds__(256) void quant_act_flat_kernel(
    const uint16_t* __restrict__ x, int64_t ld_x, uint8_t* __restrict__ q, int64_t ld_q,
    float* __restrict__ s, int64_t ld_s, uint32_t groups_per_row, uint32_t total_groups,
    uint32_t* __restrict__ zero, uint32_t zero_n) {
  if (blockIdx.x == 0)
    for (uint32_t i = threadIdx.x; i < zero_n; i += 256) zero[i] = 0u;
  const uint32_t lane16 = threadIdx.x & 15u;
  const uint32_t slot = threadIdx.x >> 4;
  uint4 v[GPT];
  uint32_t row[GPT], g[GPT];
  bool ok[GPT];
#pragma unroll
  for (int j = 0; j < GPT; ++j) {
    const uint32_t f = (blockIdx.x * GPT + j) * 16u + slot;
    ok[j] = f < total_groups;
    row[j] = ok[j] ? f / groups_per_row : 0u;
    g[j] = ok[j] ? f - row[j] * groups_per_row : 0u;
    v[j] = ok[j] ? *reinterpret_cast<const uint4*>(x + (int64_t)row[j] * ld_x +
                                                   (int64_t)g[j] * kGroup + lane16 * 8u)
                 : make_uint4(0, 0, 0, 0);
  }
#pragma unroll
  for (int j = 0; j < GPT; ++j) {
    const uint32_t amax = row16_max(absmax8_bits(v[j]));
    const GroupDivisor d = make_divisor(__uint_as_float(amax));
    const uint2 c = quant8(v[j], d);
    if (ok[j]) {
      *reinterpret_cast<uint2*>(q + (int64_t)row[j] * ld_q + (int64_t)g[j] * kGroup +
                                lane16 * 8u) = c;
      if (lane16 == 0) s[(int64_t)row[j] * ld_s + g[j]] = d.s;
    }
  }
}

// ---------------------------------------------------------------------------
// 128x128 weight blocks: one 256-thread workgroup per block.  Thread t owns
// the 16-byte column chunk t % 16 of rows t/16 + 16 i, i = 0..7 (64 values
// held in registers between the max and the encode).
__global__ __launch_bounds__(256) void quant_weight_block_kernel(
    const uint16_t* __restrict__ w, int64_t ld_w, uint8_t* __restrict__ q, int64_t ld_q,
    float* __restrict__ s, int64_t ld_s, uint32_t kblocks) {
  __shared__ uint32_t wave_amax[4];
  const uint32_t nb = blockIdx.x / kblocks;
  const uint32_t kb = blockIdx.x - nb * kblocks;
  const uint32_t chunk = threadIdx.x & 15u;
  const uint32_t r0 = threadIdx.x >> 4;
  const uint16_t* base = w + (int64_t)nb * kGroup * ld_w + (int64_t)kb * kGroup + chunk * 8u;
  uint4 v[8];
#pragma unroll
  for (int i = 0; i < 8; ++i)
    v[i] = *reinterpret_cast<const uint4*>(base + (int64_t)(r0 + 16 * i) * ld_w);
  uint32_t m = 0;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    uint32_t t = absmax8_bits(v[i]);
    m = m > t ? m : t;
  }
  m = wave_max(m);
  if ((threadIdx.x & 63u) == 0) wave_amax[threadIdx.x >> 6] = m;
  __syncthreads();
  uint32_t a = wave_amax[0] > wave_amax[1] ? wave_amax[0] : wave_amax[1];
  uint32_t b = wave_amax[2] > wave_amax[3] ? wave_amax[2] : wave_amax[3];
  m = a > b ? a : b;
  GroupDivisor d = make_divisor(__uint_as_float(m));
  uint8_t* qbase = q + (int64_t)nb * kGroup * ld_q + (int64_t)kb * kGroup + chunk * 8u;
#pragma unroll
  for (int i = 0; i < 8; ++i)
    *reinterpret_cast<uint2*>(qbase + (int64_t)(r0 + 16 * i) * ld_q) = quant8(v[i], d);
  if (threadIdx.x == 0) s[(int64_t)nb * ld_s + kb] = d.s;
}

// ---------------------------------------------------------------------------
// Whole-tensor scale, two passes.  The tensor is [R, C] with C % 128 == 0,
// walked as 16-byte chunks (8 values); chunk i is row i / (C/8).
// Pass 1: each workgroup writes the max over its grid-stride share.
__global__ __launch_bounds__(256) void absmax_partial_kernel(
    const uint16_t* __restrict__ x, int64_t ld_x, uint32_t chunks_per_row, uint64_t nchunks,
    uint32_t* __restrict__ partials) {
  __shared__ uint32_t wave_amax[4];
  uint32_t m = 0;
  for (uint64_t i = (uint64_t)blockIdx.x * 256u + threadIdx.x; i < nchunks;
       i += (uint64_t)gridDim.x * 256u) {
    uint64_t row = i / chunks_per_row;
    uint64_t c = i - row * chunks_per_row;
    uint4 v = *reinterpret_cast<const uint4*>(x + row * ld_x + c * 8u);
    uint32_t t = absmax8_bits(v);
    m = m > t ? m : t;
  }
  m = wave_max(m);
  if ((threadIdx.x & 63u) == 0) wave_amax[threadIdx.x >> 6] = m;
  __syncthreads();
  if (threadIdx.x == 0) {
    uint32_t a = wave_amax[0] > wave_amax[1] ? wave_amax[0] : wave_amax[1];
    uint32_t b = wave_amax[2] > wave_amax[3] ? wave_amax[2] : wave_amax[3];
    partials[blockIdx.x] = a > b ? a : b;
  }
}

// Pass 2: every workgroup folds the partials into the tensor amax, then
// encodes its grid-stride share; workgroup 0 writes the scale.
__global__ __launch_bounds__(256) void quant_tensor_kernel(
    const uint16_t* __restrict__ x, int64_t ld_x, uint8_t* __restrict__ q, int64_t ld_q,
    float* __restrict__ s, uint32_t chunks_per_row, uint64_t nchunks,
    const uint32_t* __restrict__ partials, uint32_t npartials) {
  __shared__ uint32_t wave_amax[4];
  uint32_t m = 0;
  for (uint32_t i = threadIdx.x; i < npartials; i += 256u) {
    uint32_t t = partials[i];
    m = m > t ? m : t;
  }
  m = wave_max(m);
  if ((threadIdx.x & 63u) == 0) wave_amax[threadIdx.x >> 6] = m;
  __syncthreads();
  uint32_t a = wave_amax[0] > wave_amax[1] ? wave_amax[0] : wave_amax[1];
  uint32_t b = wave_amax[2] > wave_amax[3] ? wave_amax[2] : wave_amax[3];
  m = a > b ? a : b;
  GroupDivisor d = make_divisor(__uint_as_float(m));
  if (blockIdx.x == 0 && threadIdx.x == 0) s[0] = d.s;
  for (uint64_t i = (uint64_t)blockIdx.x * 256u + threadIdx.x; i < nchunks;
       i += (uint64_t)gridDim.x * 256u) {
    uint64_t row = i / chunks_per_row;
    uint64_t c = i - row * chunks_per_row;
    uint4 v = *reinterpret_cast<const uint4*>(x + row * ld_x + c * 8u);
    *reinterpret_cast<uint2*>(q + row * ld_q + c * 8u) = quant8(v, d);
  }
}

// ---------------------------------------------------------------------------
// Dynamic per-row quantization: one scale per row -- per token for
// activations, per output channel for weights ("[vLLM] FP8", scaling
// strategies: dynamic per-token; "FP8 Quantization": channel-wise weight
// scales).  One wave per row, four rows per workgroup: the wave reads the
// row as 16-byte chunks (lane i takes chunks i, i + 64, ...; coalesced), folds
// the amax with a wave reduction, then re-reads the row (from L1/L2) and
// encodes it with the same divisor and encoder as the 1x128 quantizer.
__global__ __launch_bounds__(256) void quant_rows_kernel(
    const uint16_t* __restrict__ x, int64_t R, int64_t ld_x, uint32_t chunks,
    uint8_t* __restrict__ q, int64_t ld_q, float* __restrict__ s, int64_t ld_s) {
  const int64_t row = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (row >= R) return;                                   // wave-uniform
  const uint32_t lane = threadIdx.x & 63u;
  const uint16_t* xr = x + row * ld_x;
  uint32_t m = 0;
  for (uint32_t c = lane; c < chunks; c += 64u) {
    const uint32_t t = absmax8_bits(*reinterpret_cast<const uint4*>(xr + c * 8u));
    m = m > t ? m : t;
  }
  m = wave_max(m);
  const GroupDivisor d = make_divisor(__uint_as_float(m));
  if (lane == 0) s[row * ld_s] = d.s;
  uint8_t* qr = q + row * ld_q;
  for (uint32_t c = lane; c < chunks; c += 64u)
    *reinterpret_cast<uint2*>(qr + c * 8u) = quant8(*reinterpret_cast<const uint4*>(xr + c * 8u), d);
}

// ---------------------------------------------------------------------------
// Static quantization with a calibrated scale held in device memory
// ("[vLLM] FP8", scaling strategies: static per-tensor): code = E4M3(x / s)
// with the IEEE fp32 quotient, formed by the static-divisor steps (one
// reciprocal per thread and one FMA correction per element, exact for every
// normal scale; other scales divide directly), saturating and NaN-aware.
// Grid-stride over 16-byte chunks.
__global__ __launch_bounds__(256) void quant_static_kernel(
    const uint16_t* __restrict__ x, int64_t ld_x, uint8_t* __restrict__ q, int64_t ld_q,
    const float* __restrict__ scale, uint32_t chunks_per_row, uint64_t nchunks) {
  const StaticDivisor d = make_static_divisor(scale[0]);
  for (uint64_t i = (uint64_t)blockIdx.x * 256u + threadIdx.x; i < nchunks;
       i += (uint64_t)gridDim.x * 256u) {
    const uint64_t row = i / chunks_per_row;
    const uint64_t c = i - row * chunks_per_row;
    const uint4 v = *reinterpret_cast<const uint4*>(x + row * ld_x + c * 8u);
    *reinterpret_cast<uint2*>(q + row * ld_q + c * 8u) = quant8_static(v, d);
  }
}

// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void encode_f32_kernel(const float* __restrict__ x, uint64_t n,
                                                         uint8_t* __restrict__ codes) {
  uint64_t i = (uint64_t)blockIdx.x * 256u + threadIdx.x;
  if (i < n) codes[i] = e4m3_encode_one(x[i]);
}

}  // namespace

// the flattened 1x128 kernel serves rows narrower than a workgroup's
// 16 GPT groups when its grid fits a dispatch
constexpr uint32_t kActGPT = 2;
constexpr uint32_t kActGroupsPerWG = 16u * kActGPT;

static bool act_flat(uint64_t groups, uint64_t total) {
  return groups < kActGroupsPerWG &&
         (total + kActGroupsPerWG - 1) / kActGroupsPerWG * 256u < kMaxGridItems;
}

uint64_t quant_act_block_items(int64_t M, int64_t K) {
  const uint64_t groups = (uint64_t)(K / kGroup), total = (uint64_t)M * groups;
  if (act_flat(groups, total)) return (total + kActGroupsPerWG - 1) / kActGroupsPerWG * 256u;
  return (groups + kActGroupsPerWG - 1) / kActGroupsPerWG * (uint64_t)M * 256u;
}

uint64_t quant_weight_block_items(int64_t N, int64_t K) {
  return (uint64_t)(N / kGroup) * (uint64_t)(K / kGroup) * 256u;
}

uint64_t quant_rows_items(int64_t R) { return ((uint64_t)R + 3) / 4 * 256u; }

uint64_t encode_items(int64_t n) { return ((uint64_t)n + 255) / 256 * 256u; }

hipError_t launch_quant_act_block(const uint16_t* x, int64_t M, int64_t K, int64_t ld_x,
                                  uint8_t* q, int64_t ld_q, float* s, int64_t ld_s,
                                  hipStream_t st, uint32_t* zero, uint32_t zero_n) {
  constexpr int GPT = kActGPT;
  const uint32_t groups = (uint32_t)(K / kGroup);
  const uint64_t total = (uint64_t)M * groups;
  // rows narrower than a workgroup's 16 GPT groups: number the groups across
  // rows so no lane idles (measured at K = 512, M = 4096: 4.8 -> 3.5 us);
  // wider rows keep one run of workgroups per row, which measured faster
  if (act_flat(groups, total)) {
    const uint64_t grid = (total + 16u * GPT - 1) / (16u * GPT);
    hipLaunchKernelGGL(quant_act_flat_kernel<GPT>, dim3((uint32_t)grid), dim3(256), 0, st, x,
                       ld_x, q, ld_q, s, ld_s, groups, (uint32_t)total, zero, zero_n);
    return hipGetLastError();
  }
  const uint32_t per_block = 16u * GPT;
  const uint32_t bpr = (groups + per_block - 1) / per_block;
  const uint64_t grid = (uint64_t)bpr * (uint64_t)M;
  hipLaunchKernelGGL(quant_act_block_kernel<GPT>, dim3((uint32_t)grid), dim3(256), 0, st, x,
                     ld_x, q, ld_q, s, ld_s, groups, bpr, zero, zero_n);
  return hipGetLastError();
}

hipError_t launch_quant_weight_block(const uint16_t* w, int64_t N, int64_t K, int64_t ld_w,
                                     uint8_t* q, int64_t ld_q, float* s, int64_t ld_s,
                                     hipStream_t st) {
  const uint32_t kb = (uint32_t)(K / kGroup);
  const uint64_t grid = (uint64_t)(N / kGroup) * kb;
  hipLaunchKernelGGL(quant_weight_block_kernel, dim3((uint32_t)grid), dim3(256), 0, st, w, ld_w,
                     q, ld_q, s, ld_s, kb);
  return hipGetLastError();
}

hipError_t launch_quant_tensor(const uint16_t* x, int64_t R, int64_t C, int64_t ld_x,
                               uint8_t* q, int64_t ld_q, float* s, uint32_t* partials,
                               hipStream_t st) {
  const uint32_t cpr = (uint32_t)(C / 8);
  const uint64_t nchunks = (uint64_t)R * cpr;
  uint64_t want = (nchunks + 255) / 256;
  const uint32_t p1 = (uint32_t)(want < (uint64_t)kTensorPartials ? want : kTensorPartials);
  hipLaunchKernelGGL(absmax_partial_kernel, dim3(p1), dim3(256), 0, st, x, ld_x, cpr, nchunks,
                     partials);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  // second pass: enough workgroups to cover the chip several times over
  uint64_t want2 = (nchunks + 255) / 256;
  const uint32_t p2 = (uint32_t)(want2 < 8192 ? want2 : 8192);
  hipLaunchKernelGGL(quant_tensor_kernel, dim3(p2), dim3(256), 0, st, x, ld_x, q, ld_q, s, cpr,
                     nchunks, partials, p1);
  return hipGetLastError();
}

hipError_t launch_quant_rows(const uint16_t* x, int64_t R, int64_t K, int64_t ld_x, uint8_t* q,
                             int64_t ld_q, float* s, int64_t ld_s, hipStream_t st) {
  const uint64_t grid = ((uint64_t)R + 3) / 4;
  hipLaunchKernelGGL(quant_rows_kernel, dim3((uint32_t)grid), dim3(256), 0, st, x, R, ld_x,
                     (uint32_t)(K / 8), q, ld_q, s, ld_s);
  return hipGetLastError();
}

hipError_t launch_quant_static(const uint16_t* x, int64_t R, int64_t K, int64_t ld_x, uint8_t* q,
                               int64_t ld_q, const float* scale, hipStream_t st) {
  const uint32_t cpr = (uint32_t)(K / 8);
  const uint64_t nchunks = (uint64_t)R * cpr;
  const uint64_t want = (nchunks + 255) / 256;
  const uint32_t grid = (uint32_t)(want < 8192 ? want : 8192);
  hipLaunchKernelGGL(quant_static_kernel, dim3(grid), dim3(256), 0, st, x, ld_x, q, ld_q, scale,
                     cpr, nchunks);
  return hipGetLastError();
}

hipError_t launch_encode_f32(const float* x, int64_t n, uint8_t* codes, hipStream_t st) {
  const uint64_t grid = ((uint64_t)n + 255) / 256;
  hipLaunchKernelGGL(encode_f32_kernel, dim3((uint32_t)grid), dim3(256), 0, st, x, (uint64_t)n,
                     codes);
  return hipGetLastError();
}

}  // namespace fp8k
