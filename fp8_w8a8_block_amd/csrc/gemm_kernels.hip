// Block-scaled FP8 x FP8 GEMM for gfx950: out[M, N] = A[M, K] . W[N, K]^T.
//
// Per 128-wide K block kb the matrix unit forms the fp32 partial
//   P_kb[m, n] = sum_{k in kb} dec(a[m, k]) * dec(w[n, k])
// with one v_mfma_f32_16x16x128_f8f6f4 per 16x16 output tile (E4M3 x E4M3),
// and the VALU folds it into the fp32 accumulator with both scales:
//   acc[m, n] += (sa[m, kb] * sw[n / 128, kb]) * P_kb[m, n]
// The epilogue rounds acc to bf16 (nearest even).  This follows "FP8 and
// FP4: Throughput Needs Scaling", kernel-caveat card (FP8 operands straight
// into the matrix unit, wide accumulation) and "[vLLM] FP8", block
// quantization (one scale per 128x128 weight block, 1x128 dynamic
// activation groups).  With per-tensor scales the matrix unit accumulates
// over all of K and the single product sa * sw is applied at the end.
//
// MFMA operand layout used here: lane l supplies row (l % 16) of its
// operand and the 32 bytes [32 (l / 16), 32 (l / 16) + 32) of the 128-byte
// K block.  A and B use the same assignment, so every k pairs a[m, k] with
// w[n, k] whatever order the unit walks the 32 bytes in.  The 16x16 fp32
// result sits in lane n + 16 (m / 4), register m % 4.
#include "device_common.h"
#include "launch.h"

namespace fp8k {

namespace {

typedef int v8i __attribute__((ext_vector_type(8)));
typedef float v4f __attribute__((ext_vector_type(4)));

__device__ __forceinline__ v4f mfma_fp8(const v8i& a, const v8i& b, const v4f& c) {
  // cbsz = blgp = 0: both operands E4M3; zero scale operands select the
  // unscaled instruction.
  return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, c, 0, 0, 0, 0, 0, 0);
}

__device__ __forceinline__ v8i load32(const uint8_t* p) {
  const uint4* q = reinterpret_cast<const uint4*>(p);
  uint4 x = q[0];
  uint4 y = q[1];
  v8i r;
  r[0] = (int)x.x; r[1] = (int)x.y; r[2] = (int)x.z; r[3] = (int)x.w;
  r[4] = (int)y.x; r[5] = (int)y.y; r[6] = (int)y.z; r[7] = (int)y.w;
  return r;
}

__device__ __forceinline__ v8i zero8() {
  v8i r;
#pragma unroll
  for (int i = 0; i < 8; ++i) r[i] = 0;
  return r;
}

// ---------------------------------------------------------------------------
// Decode shape (M <= 16): HBM-bound on the weight.  One workgroup per 16
// output columns; its KSPLIT waves take interleaved K blocks, keep UNROLL
// blocks of W loads in flight, and reduce their 16x16 partial sums in LDS.
template <int KSPLIT, int UNROLL, bool PER_TENSOR>
__global__ __launch_bounds__(64 * KSPLIT) void gemm_decode_kernel(
    const uint8_t* __restrict__ a, int64_t ld_a, const float* __restrict__ sa, int64_t ld_sa,
    const uint8_t* __restrict__ w, int64_t ld_w, const float* __restrict__ sw, int64_t ld_sw,
    uint16_t* __restrict__ out, int64_t ld_out, int M, int KB) {
  __shared__ float red[KSPLIT][4][64];
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int r16 = lane & 15;
  const int kg = lane >> 4;
  const int64_t n0 = (int64_t)blockIdx.x * 16;
  const int nb = (int)(n0 >> 7);
  const uint8_t* wp = w + (n0 + r16) * ld_w + kg * 32;
  const bool arow = r16 < M;
  const uint8_t* ap = a + (int64_t)(arow ? r16 : 0) * ld_a + kg * 32;

  // rows of the output this lane accumulates: m = 4 kg + i
  bool mrow[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) mrow[i] = (4 * kg + i) < M;

  v4f acc = {0.f, 0.f, 0.f, 0.f};
  for (int kb0 = wave; kb0 < KB; kb0 += KSPLIT * UNROLL) {
    v8i bw[UNROLL], av[UNROLL];
#pragma unroll
    for (int u = 0; u < UNROLL; ++u) {
      const int kb = kb0 + u * KSPLIT;
      bw[u] = kb < KB ? load32(wp + (int64_t)kb * 128) : zero8();
    }
#pragma unroll
    for (int u = 0; u < UNROLL; ++u) {
      const int kb = kb0 + u * KSPLIT;
      av[u] = (arow && kb < KB) ? load32(ap + (int64_t)kb * 128) : zero8();
    }
#pragma unroll
    for (int u = 0; u < UNROLL; ++u) {
      const int kb = kb0 + u * KSPLIT;
      if (PER_TENSOR) {
        acc = mfma_fp8(av[u], bw[u], acc);
      } else {
        v4f p = mfma_fp8(av[u], bw[u], v4f{0.f, 0.f, 0.f, 0.f});
        if (kb < KB) {
          const float s_w = sw[(int64_t)nb * ld_sw + kb];
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const float s_a = mrow[i] ? sa[(int64_t)(4 * kg + i) * ld_sa + kb] : 0.f;
            acc[i] = __builtin_fmaf(s_a * s_w, p[i], acc[i]);
          }
        }
      }
    }
  }
#pragma unroll
  for (int i = 0; i < 4; ++i) red[wave][i][lane] = acc[i];
  __syncthreads();
  if (wave == 0) {
    const float st = PER_TENSOR ? sa[0] * sw[0] : 1.0f;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      float v = 0.f;
#pragma unroll
      for (int s = 0; s < KSPLIT; ++s) v += red[s][i][lane];
      if (PER_TENSOR) v *= st;
      const int m = 4 * kg + i;
      if (m < M) out[(int64_t)m * ld_out + n0 + r16] = (uint16_t)f32_to_bf16_rne(v);
    }
  }
}

// ---------------------------------------------------------------------------
// General shape: 128x128 output tile per 256-thread workgroup, 2x2 waves of
// 64x64 (4x4 MFMA tiles).  Each K block of A and W (128 rows x 128 bytes
// each) is staged through LDS with rows padded to 144 bytes, which spreads
// the 16 rows a ds_read_b128 phase touches over distinct banks.
constexpr int kBM = 128;
constexpr int kBN = 128;
constexpr int kLdsRow = 144;

template <bool PER_TENSOR>
__global__ __launch_bounds__(256) void gemm_tile_kernel(
    const uint8_t* __restrict__ a, int64_t ld_a, const float* __restrict__ sa, int64_t ld_sa,
    const uint8_t* __restrict__ w, int64_t ld_w, const float* __restrict__ sw, int64_t ld_sw,
    uint16_t* __restrict__ out, int64_t ld_out, int M, int KB, int tiles_n) {
  __shared__ __attribute__((aligned(16))) uint8_t lds_a[kBM * kLdsRow];
  __shared__ __attribute__((aligned(16))) uint8_t lds_w[kBN * kLdsRow];
  __shared__ float lds_sa[kBM];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int wm = wave >> 1;
  const int wn = wave & 1;
  const int r16 = lane & 15;
  const int kg = lane >> 4;
  const int tm = blockIdx.x / tiles_n;
  const int tn = blockIdx.x - tm * tiles_n;
  const int64_t m0 = (int64_t)tm * kBM;
  const int64_t n0 = (int64_t)tn * kBN;
  const int nb = (int)(n0 >> 7);

  // global -> LDS copy assignment: 8 threads per 128-byte row, 32 rows/pass
  const int crow = tid >> 3;
  const int cchunk = tid & 7;

  v4f acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = v4f{0.f, 0.f, 0.f, 0.f};

  for (int kb = 0; kb < KB; ++kb) {
    uint4 ra[4], rw[4];
#pragma unroll
    for (int p = 0; p < 4; ++p) {
      // rows past M read the last valid row and are zeroed after the load,
      // so every load is unconditional and in bounds
      const int r = crow + 32 * p;
      const int64_t gm = m0 + r;
      const int64_t gmc = gm < M ? gm : (int64_t)M - 1;
      ra[p] = *reinterpret_cast<const uint4*>(a + gmc * ld_a + (int64_t)kb * 128 + cchunk * 16);
      rw[p] = *reinterpret_cast<const uint4*>(w + (n0 + r) * ld_w + (int64_t)kb * 128 + cchunk * 16);
    }
#pragma unroll
    for (int p = 0; p < 4; ++p) {
      if (m0 + crow + 32 * p >= M) ra[p] = make_uint4(0, 0, 0, 0);
    }
    float s_a_ld = 0.f;
    if (!PER_TENSOR && tid < kBM) {
      const int64_t gm = m0 + tid;
      s_a_ld = gm < M ? sa[gm * ld_sa + kb] : 0.f;
    }
    __syncthreads();  // previous block's LDS reads are done
#pragma unroll
    for (int p = 0; p < 4; ++p) {
      const int r = crow + 32 * p;
      *reinterpret_cast<uint4*>(lds_a + r * kLdsRow + cchunk * 16) = ra[p];
      *reinterpret_cast<uint4*>(lds_w + r * kLdsRow + cchunk * 16) = rw[p];
    }
    if (!PER_TENSOR && tid < kBM) lds_sa[tid] = s_a_ld;
    __syncthreads();

    v8i fa[4], fb[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) fa[i] = load32(lds_a + (wm * 64 + i * 16 + r16) * kLdsRow + kg * 32);
#pragma unroll
    for (int j = 0; j < 4; ++j) fb[j] = load32(lds_w + (wn * 64 + j * 16 + r16) * kLdsRow + kg * 32);

    if (PER_TENSOR) {
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = mfma_fp8(fa[i], fb[j], acc[i][j]);
    } else {
      const float s_w = sw[(int64_t)nb * ld_sw + kb];
      float s_c[4][4];
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int r = 0; r < 4; ++r) s_c[i][r] = lds_sa[wm * 64 + i * 16 + 4 * kg + r] * s_w;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          v4f p = mfma_fp8(fa[i], fb[j], v4f{0.f, 0.f, 0.f, 0.f});
#pragma unroll
          for (int r = 0; r < 4; ++r) acc[i][j][r] = __builtin_fmaf(s_c[i][r], p[r], acc[i][j][r]);
        }
      }
    }
  }

  const float st = PER_TENSOR ? sa[0] * sw[0] : 1.0f;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int64_t gm = m0 + wm * 64 + i * 16 + 4 * kg + r;
      if (gm < M) {
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          float v = acc[i][j][r];
          if (PER_TENSOR) v *= st;
          out[gm * ld_out + n0 + wn * 64 + j * 16 + r16] = (uint16_t)f32_to_bf16_rne(v);
        }
      }
    }
  }
}

}  // namespace

hipError_t launch_gemm(const uint8_t* a, int64_t ld_a, const float* sa, int64_t ld_sa,
                       const uint8_t* w, int64_t ld_w, const float* sw, int64_t ld_sw,
                       uint16_t* out, int64_t ld_out, int64_t M, int64_t N, int64_t K,
                       bool per_tensor, hipStream_t st) {
  const int KB = (int)(K / 128);
  if (M <= 16) {
    constexpr int KSPLIT = 8, UNROLL = 4;
    dim3 grid((uint32_t)(N / 16));
    if (per_tensor)
      hipLaunchKernelGGL((gemm_decode_kernel<KSPLIT, UNROLL, true>), grid, dim3(64 * KSPLIT), 0, st,
                         a, ld_a, sa, ld_sa, w, ld_w, sw, ld_sw, out, ld_out, (int)M, KB);
    else
      hipLaunchKernelGGL((gemm_decode_kernel<KSPLIT, UNROLL, false>), grid, dim3(64 * KSPLIT), 0,
                         st, a, ld_a, sa, ld_sa, w, ld_w, sw, ld_sw, out, ld_out, (int)M, KB);
    return hipGetLastError();
  }
  const int tiles_m = (int)((M + kBM - 1) / kBM);
  const int tiles_n = (int)(N / kBN);
  dim3 grid((uint32_t)tiles_m * (uint32_t)tiles_n);
  if (per_tensor)
    hipLaunchKernelGGL(gemm_tile_kernel<true>, grid, dim3(256), 0, st, a, ld_a, sa, ld_sa, w, ld_w,
                       sw, ld_sw, out, ld_out, (int)M, KB, tiles_n);
  else
    hipLaunchKernelGGL(gemm_tile_kernel<false>, grid, dim3(256), 0, st, a, ld_a, sa, ld_sa, w, ld_w,
                       sw, ld_sw, out, ld_out, (int)M, KB, tiles_n);
  return hipGetLastError();
}

}  // namespace fp8k
