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
#include <atomic>
#include <type_traits>

#include "device_common.h"
#include "launch.h"

namespace fp8k {

namespace {

typedef int v8i __attribute__((ext_vector_type(8)));

// the decode path stages all activation scales of a call in LDS
constexpr int kDecodeMaxKB = 128;             // K <= 16384

// decode split: waves per workgroup and K blocks per wave batch
#ifndef FP8_DECODE_KSPLIT
#define FP8_DECODE_KSPLIT 8
#endif
#ifndef FP8_DECODE_KBW
#define FP8_DECODE_KBW 1
#endif
// largest M the decode tile serves (16-row chunks above 16)
#ifndef FP8_DECODE_MAX_M
#define FP8_DECODE_MAX_M 64
#endif
// prefill: the hand-scheduled K loop (prefill_asm.inc) instead of the C++ one
#ifndef FP8_PREFILL_ASM
#define FP8_PREFILL_ASM 1
#endif
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

// LDS swizzle of 128-byte operand rows: the 16-byte chunk c of row r is
// stored at chunk position c ^ swz(r).  A fragment read touches 16 rows at
// one logical chunk per ds_read_b128; with this swizzle the 16 rows land on
// 16 distinct 16-byte bank groups of a 256-byte bank row, and any 8
// consecutive rows on 8 distinct groups of a 128-byte bank row, so the read
// is conflict free whether the LDS serves it 16 or 8 lanes at a time.
__device__ __forceinline__ int swz(int r) { return ((r >> 1) & 7) ^ ((r & 1) << 2); }

__device__ __forceinline__ v8i zero8() {
  v8i r;
#pragma unroll
  for (int i = 0; i < 8; ++i) r[i] = 0;
  return r;
}

// ---------------------------------------------------------------------------
// Decode shape (M <= 16): HBM-bound on the weight (one byte per weight
// element, read once).  A workgroup owns 16 output columns; its KSPLIT
// waves each own a contiguous run of K blocks, processed in batches of KBW.
//
// Operands never go through registers on their way in: each wave streams
// its weight fragments (16 rows x 128 bytes per K block) and the matching
// activation fragments into private LDS buffers with global_load_lds_dwordx4,
// lane-linear, so every load instruction covers eight whole 128-byte rows.
// (Loading the MFMA layout straight from memory makes each instruction
// touch 16 rows x 64 bytes, which streams far below the HBM rate.)  Within
// a row the eight 16-byte chunks are stored XOR-swizzled by swz(row), so the
// fragment reads hit distinct banks.  While the MFMAs of batch b run, the loads of batch b+1
// are in flight.  Activation rows >= M are not copied (the lanes that would
// copy them are switched off; M = 1 moves 128 bytes per K block instead of
// 2 KiB) and are zeroed in registers.  The waves' 16x16 partial sums are
// reduced in LDS.
//
// Dynamic LDS: KSPLIT * KBW * 4 KiB operand buffers, then the reduction
// buffer (KSPLIT * 1 KiB), then the activation scales (16 * KB floats; in
// the loop-free form already multiplied by the tile's weight scales).
constexpr int kFrag = 2048;                   // 16 rows x 128 bytes

template <int KSPLIT, int KBW>
constexpr size_t decode_lds_bytes(int KB, bool kconst) {
  return (size_t)KSPLIT * KBW * 2 * kFrag + (size_t)KSPLIT * 4 * 64 * sizeof(float) +
         (kconst ? 0 : (size_t)16 * KB * sizeof(float));
}

// One 16-column output tile of at most 16 rows (1 <= M <= 16), columns
// n0 .. n0 + 15; the whole workgroup takes part (it holds barriers).
// WSTAGE: the weight scales are folded into the staged activation scales up
// front, so the K loop reads no scale from memory (the same fp32 product,
// bit for bit); the chunked and grouped forms, which sit at their register
// limit, read the weight scale in the loop.
template <int KSPLIT, int KBW, bool KCONST, bool WSTAGE = false>
__device__ __forceinline__ void decode_tile(
    uint8_t* lds, const uint8_t* __restrict__ a, int64_t ld_a, const float* __restrict__ sa,
    int64_t ld_sa, const uint8_t* __restrict__ w, int64_t ld_w, const float* __restrict__ sw,
    int64_t ld_sw, uint16_t* __restrict__ out, int64_t ld_out, int M, int KB, int64_t n0) {
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int r16 = lane & 15;
  const int kg = lane >> 4;
  const bool arow = r16 < M;

  uint8_t* wbuf = lds + (size_t)wave * (KBW * 2 * kFrag);     // this wave's W fragments
  uint8_t* abuf = wbuf + KBW * kFrag;                          // and A fragments
  float* red = reinterpret_cast<float*>(lds + (size_t)KSPLIT * KBW * 2 * kFrag);
  float* s_as = red + KSPLIT * 4 * 64;

  // load slot s = 64 j + lane holds row s / 8 at stored chunk s % 8, which is
  // source chunk (s % 8) ^ swz(row)
  const int drow = lane >> 3;
  const int dchunk0 = (lane & 7) ^ swz(drow);
  const int dchunk1 = (lane & 7) ^ swz(8 + drow);
  const uint8_t* wsrc0 = w + (n0 + drow) * ld_w + dchunk0 * 16;
  const uint8_t* wsrc1 = w + (n0 + 8 + drow) * ld_w + dchunk1 * 16;
  const uint8_t* asrc0 = a + (int64_t)min(drow, M - 1) * ld_a + dchunk0 * 16;
  const uint8_t* asrc1 = a + (int64_t)min(8 + drow, M - 1) * ld_a + dchunk1 * 16;
  // fragment reads: row r16, source chunks 2 kg and 2 kg + 1
  const int rd0 = r16 * 128 + (((2 * kg) ^ swz(r16)) * 16);
  const int rd1 = r16 * 128 + (((2 * kg + 1) ^ swz(r16)) * 16);

  const int per = (KB + KSPLIT - 1) / KSPLIT;
  const int kb_lo = wave * per;
  const int kb_hi = min(KB, kb_lo + per);

  auto dma = [&](const uint8_t* src, uint8_t* dst) {
    __builtin_amdgcn_global_load_lds((const void*)src,
                                     (__attribute__((address_space(3))) void*)dst, 16, 0, 0);
  };
  auto issue = [&](int kb0) {
#pragma unroll
    for (int u = 0; u < KBW; ++u) {
      const int kb = kb0 + u;
      if (kb < kb_hi) {                               // wave-uniform
        const int64_t off = (int64_t)kb * 128;
        dma(wsrc0 + off, wbuf + u * kFrag);
        dma(wsrc1 + off, wbuf + u * kFrag + 1024);
        // activation rows >= M are never copied: their fragment lanes are
        // zeroed in registers, whatever the LDS holds
        if (drow < M) dma(asrc0 + off, abuf + u * kFrag);
        if (8 + drow < M) dma(asrc1 + off, abuf + u * kFrag + 1024);
      }
    }
  };
  auto frag = [&](const uint8_t* buf) {
    const uint4 x = *reinterpret_cast<const uint4*>(buf + rd0);
    const uint4 y = *reinterpret_cast<const uint4*>(buf + rd1);
    v8i r;
    r[0] = (int)x.x; r[1] = (int)x.y; r[2] = (int)x.z; r[3] = (int)x.w;
    r[4] = (int)y.x; r[5] = (int)y.y; r[6] = (int)y.z; r[7] = (int)y.w;
    return r;
  };

  if (kb_lo < kb_hi) issue(kb_lo);
  if (!KCONST) {
    // s_as[kb * 16 + m] = sa[m, kb] (rows >= M read 0), times sw[n0 / 128, kb]
    // when WSTAGE; queued behind the first batch's loads
    const float* __restrict__ swr = sw + (int64_t)(n0 >> 7) * ld_sw;
    for (int i = threadIdx.x; i < KB * 16; i += 64 * KSPLIT) {
      const int m = i & 15;
      const int kb = i >> 4;
      if (WSTAGE)
        s_as[i] = m < M ? sa[(int64_t)m * ld_sa + kb] * swr[kb] : 0.f;
      else
        s_as[i] = m < M ? sa[(int64_t)m * ld_sa + kb] : 0.f;
    }
  }
  __syncthreads();

  v4f acc = {0.f, 0.f, 0.f, 0.f};
  for (int kb0 = kb_lo; kb0 < kb_hi; kb0 += KBW) {    // wave-uniform; no barrier inside
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    v8i av[KBW], bw[KBW];
#pragma unroll
    for (int u = 0; u < KBW; ++u) {
      av[u] = frag(abuf + u * kFrag);
      bw[u] = frag(wbuf + u * kFrag);
    }
    // this batch's combined scales, read before the next batch's LDS writes
    // are queued (LDS reads are ordered behind those)
    float sc[KBW][4];
#pragma unroll
    for (int u = 0; u < KBW; ++u) {
      const int kb = kb0 + u;
      const int kbc = min(kb, kb_hi - 1);
      const float s_w = KCONST || WSTAGE ? 0.f : sw[(int64_t)(n0 >> 7) * ld_sw + kbc];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float s_a = KCONST ? 0.f : s_as[kbc * 16 + 4 * kg + i];
        sc[u][i] = kb < kb_hi ? (WSTAGE ? s_a : s_a * s_w) : 0.f;
      }
    }
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
    if (kb0 + KBW < kb_hi) issue(kb0 + KBW);
#pragma unroll
    for (int u = 0; u < KBW; ++u) {
      const bool ok = arow && (kb0 + u < kb_hi);
#pragma unroll
      for (int e = 0; e < 8; ++e) av[u][e] = ok ? av[u][e] : 0;
      if (KCONST) {
        acc = mfma_fp8(av[u], bw[u], acc);
      } else {
        v4f p = mfma_fp8(av[u], bw[u], v4f{0.f, 0.f, 0.f, 0.f});
#pragma unroll
        for (int i = 0; i < 4; ++i) acc[i] = __builtin_fmaf(sc[u][i], p[i], acc[i]);
      }
    }
  }
#pragma unroll
  for (int i = 0; i < 4; ++i) red[(wave * 4 + i) * 64 + lane] = acc[i];
  __syncthreads();
  if (wave == 0) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      float v = 0.f;
#pragma unroll
      for (int s2 = 0; s2 < KSPLIT; ++s2) v += red[(s2 * 4 + i) * 64 + lane];
      const int m = 4 * kg + i;
      if (m < M) {
        if (KCONST) v *= sa[(int64_t)m * ld_sa] * sw[(n0 + r16) * ld_sw];
        out[(int64_t)m * ld_out + n0 + r16] = (uint16_t)f32_to_bf16_rne(v);
      }
    }
  }
}

// CHUNKED (16 < M): rows go through the tile 16 at a time, each chunk
// streaming the workgroup's weight strip again, which keeps every CU busy
// for the mid-size batches the 256-row prefill tiles would leave mostly
// empty.  M <= 16 uses the loop-free form: the loop raised the register
// count to 86 (two workgroups per CU instead of three; 9.9 -> 12.3 us at
// M = 1).  Six waves per SIMD are requested for both forms, so that three
// 8-wave workgroups fit on a CU.
template <int KSPLIT, int KBW, bool KCONST, bool CHUNKED>
__global__ __launch_bounds__(64 * KSPLIT) __attribute__((amdgpu_waves_per_eu(6, 8)))
void gemm_decode_kernel(
    const uint8_t* __restrict__ a, int64_t ld_a, const float* __restrict__ sa, int64_t ld_sa,
    const uint8_t* __restrict__ w, int64_t ld_w, const float* __restrict__ sw, int64_t ld_sw,
    uint16_t* __restrict__ out, int64_t ld_out, int M, int KB) {
  extern __shared__ __attribute__((aligned(16))) uint8_t lds[];
  if (!CHUNKED) {
    decode_tile<KSPLIT, KBW, KCONST, true>(lds, a, ld_a, sa, ld_sa, w, ld_w, sw, ld_sw, out,
                                           ld_out, M, KB, (int64_t)blockIdx.x * 16);
    return;
  }
  for (int r = 0; r < M; r += 16) {
    if (r > 0) __syncthreads();                       // LDS reuse across row chunks
    decode_tile<KSPLIT, KBW, KCONST>(lds, a + (int64_t)r * ld_a, ld_a,
                                     sa + (int64_t)r * ld_sa, ld_sa,
                                     w, ld_w, sw, ld_sw, out + (int64_t)r * ld_out, ld_out,
                                     M - r < 16 ? M - r : 16, KB, (int64_t)blockIdx.x * 16);
  }
}

// Clamped row range of expert e in a grouped call: offsets are read as
// given, then clamped to 0 <= lo <= hi <= M, so no offsets can send an
// access outside the M rows.
__device__ __forceinline__ void expert_rows(const int64_t* __restrict__ offsets, int e, int64_t M,
                                            int64_t& lo, int64_t& hi) {
  int64_t a = offsets[e], b = offsets[e + 1];
  lo = a < 0 ? 0 : (a > M ? M : a);
  hi = b < lo ? lo : (b > M ? M : b);
}

// Grouped (MoE) GEMM for few rows per expert: workgroup (x, e) computes
// columns 16 x .. 16 x + 15 of expert e's rows, 16 rows at a time with the
// decode tile, weight W + e * w_es, scales sw + e * sw_es.  An expert with no
// rows costs one offsets read.  Six waves per SIMD keep three workgroups on a
// CU, as for the chunked decode kernel.
template <int KSPLIT, int KBW>
__global__ __launch_bounds__(64 * KSPLIT) __attribute__((amdgpu_waves_per_eu(6, 8)))
void gemm_grouped_decode_kernel(
    const uint8_t* __restrict__ a, int64_t ld_a, const float* __restrict__ sa, int64_t ld_sa,
    const uint8_t* __restrict__ w, int64_t ld_w, int64_t w_es, const float* __restrict__ sw,
    int64_t ld_sw, int64_t sw_es, uint16_t* __restrict__ out, int64_t ld_out,
    const int64_t* __restrict__ offsets, int64_t M, int KB) {
  extern __shared__ __attribute__((aligned(16))) uint8_t lds[];
  const int e = blockIdx.y;
  int64_t lo, hi;
  expert_rows(offsets, e, M, lo, hi);
  const uint8_t* we = w + (int64_t)e * w_es;
  const float* swe = sw + (int64_t)e * sw_es;
  for (int64_t r = lo; r < hi; r += 16) {
    if (r > lo) __syncthreads();                      // LDS reuse across row chunks
    const int m = (int)(hi - r < 16 ? hi - r : 16);
    decode_tile<KSPLIT, KBW, false>(lds, a + r * ld_a, ld_a, sa + r * ld_sa, ld_sa, we, ld_w, swe,
                                    ld_sw, out + r * ld_out, ld_out, m, KB,
                                    (int64_t)blockIdx.x * 16);
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

template <bool KCONST>
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
    if (!KCONST && tid < kBM) {
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
    if (!KCONST && tid < kBM) lds_sa[tid] = s_a_ld;
    __syncthreads();

    v8i fa[4], fb[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) fa[i] = load32(lds_a + (wm * 64 + i * 16 + r16) * kLdsRow + kg * 32);
#pragma unroll
    for (int j = 0; j < 4; ++j) fb[j] = load32(lds_w + (wn * 64 + j * 16 + r16) * kLdsRow + kg * 32);

    if (KCONST) {
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

#pragma unroll
  for (int i = 0; i < 4; ++i) {
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int64_t gm = m0 + wm * 64 + i * 16 + 4 * kg + r;
      if (gm < M) {
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const int64_t gn = n0 + wn * 64 + j * 16 + r16;
          float v = acc[i][j][r];
          if (KCONST) v *= sa[gm * ld_sa] * sw[gn * ld_sw];
          out[gm * ld_out + gn] = (uint16_t)f32_to_bf16_rne(v);
        }
      }
    }
  }
}

// ---------------------------------------------------------------------------
// Prefill shape (large M): MFMA-bound.  Workgroup tile 256 (M) x 256 (N),
// eight waves in a 2 x 4 grid, each computing 128 x 64 outputs.  One K step
// is one 128-wide scale block.
//
// The matrix unit computes the transposed tile: its first operand is a
// 16-row weight fragment, its second a 16-row activation fragment, so lane
// l holds output column (token row) m = l % 16 and four consecutive weight
// rows n = 4 (l / 16) + r.  Each lane then needs a single activation scale
// per 16-row activation fragment (the weight scale is uniform: a wave's 64
// columns lie in one 128-row weight block), and its four outputs are four
// adjacent bf16 values of one output row, written with one 8-byte store.
//
// Both operand tiles of a K block (256 rows of 128 bytes each) are copied
// into LDS by buffer_load_dwordx4 ... lds, lane-linear (one instruction =
// eight whole rows) with the chunks of a row XOR-swizzled by swz(row).  The
// buffer descriptors start at the tile's first row and K block and end at
// the operand's last row: rows past M (or past N in a half-filled last
// tile) fall outside, read as zero and are never stored.  LDS holds two
// stages: the copy of block kb + 1 is in flight while block kb is
// multiplied.  The activation scales of block kb + 1 travel through
// registers into LDS, multiplied by the two weight-block scales of the
// tile and laid out so that a lane's eight scales are 32 contiguous bytes.
// Per K block a wave holds its 4 weight fragments and streams its 8
// activation fragments, software-pipelined: the 4 MFMAs of fragment i run
// in the matrix pipe while the VALU folds the partials of fragment i - 1
// into the accumulators with sa[m, kb] * sw[n / 128, kb].  Per-tensor
// scales accumulate in the matrix unit and scale once at the end.
//
// Tiles are visited in groups of kGroupM tile-rows, and consecutive
// workgroup ids -- which the dispatcher spreads over the 8 XCDs -- are
// remapped so that each XCD works on a compact block of tiles and shares
// their A and B panels in its own L2.
constexpr int kPM = 256, kPN = 256;           // workgroup tile
constexpr int kPWavesM = 2, kPWavesN = 4;
constexpr int kPWM = kPM / kPWavesM;          // 128 token rows per wave
constexpr int kPWN = kPN / kPWavesN;          // 64 weight rows per wave
constexpr int kPMF = kPWM / 16;               // 8 activation fragments
constexpr int kPNF = kPWN / 16;               // 4 weight fragments
constexpr int kPThreads = 64 * kPWavesM * kPWavesN;
constexpr int kPWaves = kPThreads / 64;
constexpr int kCopies = kPM / 8 / kPWaves;   // copy instructions per wave per operand
constexpr int kGroupM = 4;
constexpr int64_t kPrefillMaxLd = ((int64_t)1 << 31) / kPM;   // 32-bit buffer offsets
constexpr uint32_t kRawBufferWord3 = 0x00020000u;             // raw byte buffer, gfx9

__device__ __forceinline__ __amdgpu_buffer_rsrc_t raw_buffer(const void* base, int64_t bytes) {
  const int64_t n = bytes < 0 ? 0 : (bytes > 0x7fffffff ? 0x7fffffff : bytes);
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)n,
                                           (int)kRawBufferWord3);
}

// position of the scale of tile row t (weight block blk) in the staged array:
// [blk][wave row wm][row within fragment j][fragment mf]
__device__ __forceinline__ int sc_index(int blk, int t) {
  const int wm = t / kPWM, mf = (t % kPWM) / 16, j = t % 16;
  return ((blk * kPWavesM + wm) * 16 + j) * kPMF + mf;
}

template <bool KCONST>
__global__ __launch_bounds__(kPThreads) void gemm_prefill_kernel(
    const uint8_t* __restrict__ a, int64_t ld_a, const float* __restrict__ sa, int64_t ld_sa,
    const uint8_t* __restrict__ w, int64_t ld_w, const float* __restrict__ sw, int64_t ld_sw,
    uint16_t* __restrict__ out, int64_t ld_out, int M, int N, int KB, int tiles_m, int tiles_n) {
  __shared__ __attribute__((aligned(16))) uint8_t a_lds0[kPM * 128];
  __shared__ __attribute__((aligned(16))) uint8_t a_lds1[kPM * 128];
  __shared__ __attribute__((aligned(16))) uint8_t b_lds0[kPN * 128];
  __shared__ __attribute__((aligned(16))) uint8_t b_lds1[kPN * 128];
  __shared__ __attribute__((aligned(16))) float sc_lds0[2 * kPM];
  __shared__ __attribute__((aligned(16))) float sc_lds1[2 * kPM];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave / kPWavesN;
  const int wn = wave % kPWavesN;
  const int r16 = lane & 15;
  const int kg = lane >> 4;

  // workgroup id -> tile: XCD-contiguous ranges, then grouped row-major
  const int tiles = tiles_m * tiles_n;
  int lin = blockIdx.x;
  if (tiles % 8 == 0) lin = (lin % 8) * (tiles / 8) + lin / 8;
  const int group = lin / (kGroupM * tiles_n);
  const int first_m = group * kGroupM;
  const int gsize = min(tiles_m - first_m, kGroupM);
  const int tm = first_m + (lin % (kGroupM * tiles_n)) % gsize;
  const int tn = (lin % (kGroupM * tiles_n)) / gsize;
  const int64_t m0 = (int64_t)tm * kPM;
  const int64_t n0 = (int64_t)tn * kPN;

  // copy assignment: instruction t of this wave covers tile rows 8 j .. 8 j + 7
  // with j = wave + 8 t; slot (row, stored chunk lane & 7) holds source chunk
  // (lane & 7) ^ swz(row), and row & 15 = 8 (j & 1) + crow with j & 1 = wave & 1
  const int crow = lane >> 3;
  const int cchunk = (lane & 7) ^ swz(8 * (wave & 1) + crow);
  const uint8_t* a_tile = a + m0 * ld_a;
  const uint8_t* w_tile = w + n0 * ld_w;
  const int64_t a_bytes = ((int64_t)M - m0) * ld_a;
  const int64_t w_bytes = ((int64_t)N - n0) * ld_w;
  // copy instruction t (0 .. kCopies-1) of both operands for K block kb: tile
  // rows 8 j + crow with j = wave + 8 t.  The uniform part of the offset
  // (64 t rows and the K block) goes into the descriptor base, so every copy
  // uses the same per-lane offset; the descriptor still ends at the last row.
  const int a_lane_off = (8 * wave + crow) * (int)ld_a + cchunk * 16;
  const int w_lane_off = (8 * wave + crow) * (int)ld_w + cchunk * 16;
  auto issue_part = [&](int kb, int t, uint8_t* adst, uint8_t* bdst) {
    const int j = wave + t * kPWaves;
    const int64_t a_off = (int64_t)kb * 128 + (int64_t)t * 8 * kPWaves * ld_a;
    const int64_t w_off = (int64_t)kb * 128 + (int64_t)t * 8 * kPWaves * ld_w;
    const __amdgpu_buffer_rsrc_t ra = raw_buffer(a_tile + a_off, a_bytes - a_off);
    const __amdgpu_buffer_rsrc_t rb = raw_buffer(w_tile + w_off, w_bytes - w_off);
    __builtin_amdgcn_raw_ptr_buffer_load_lds(
        ra, (__attribute__((address_space(3))) void*)(adst + j * 1024), 16, a_lane_off, 0, 0, 0);
    __builtin_amdgcn_raw_ptr_buffer_load_lds(
        rb, (__attribute__((address_space(3))) void*)(bdst + j * 1024), 16, w_lane_off, 0, 0, 0);
  };
  auto issue = [&](int kb, uint8_t* adst, uint8_t* bdst) {
#pragma unroll
    for (int t = 0; t < kCopies; ++t) issue_part(kb, t, adst, bdst);
  };
  // activation scale of tile row tid (threads 0 .. 255), 0 past M
  const bool sa_thread = !KCONST && tid < kPM;
  const float* sa_row = sa + min<int64_t>(m0 + tid, (int64_t)M - 1) * ld_sa;
  const bool sa_valid = m0 + tid < M;
  const int nb0 = (int)(n0 >> 7);
  const int nb1 = min(nb0 + 1, N / 128 - 1);
  const int sc_w0 = sc_index(0, tid & (kPM - 1));
  const int sc_w1 = sc_index(1, tid & (kPM - 1));
  auto load_sa = [&](int kb) { return sa_valid ? sa_row[kb] : 0.f; };

  // fragment read offsets within a 16-row group: row r16, chunks 2 kg and
  // 2 kg + 1 (group bases are multiples of 16, so swz(row) = swz(r16))
  const int rd0 = r16 * 128 + (((2 * kg) ^ swz(r16)) * 16);
  const int rd1 = r16 * 128 + (((2 * kg + 1) ^ swz(r16)) * 16);
  auto frag = [&](const uint8_t* base) {
    const uint4 x = *reinterpret_cast<const uint4*>(base + rd0);
    const uint4 y = *reinterpret_cast<const uint4*>(base + rd1);
    v8i r;
    r[0] = (int)x.x; r[1] = (int)x.y; r[2] = (int)x.z; r[3] = (int)x.w;
    r[4] = (int)y.x; r[5] = (int)y.y; r[6] = (int)y.z; r[7] = (int)y.w;
    return r;
  };
  // this lane's eight scales: weight block of the wave's columns, its token row
  const int sc_rd = (((wn * kPWN) >> 7) * kPWavesM + wm) * 16 * kPMF + r16 * kPMF;

  // acc[nf][mf]: weight rows 16 nf + 4 kg + r, token row 16 mf + r16
  v4f acc[kPNF][kPMF];
#pragma unroll
  for (int i = 0; i < kPNF; ++i)
#pragma unroll
    for (int j = 0; j < kPMF; ++j) acc[i][j] = v4f{0.f, 0.f, 0.f, 0.f};

  // One K block: wait for its copy, publish its scales, then queue the next
  // block into the other stage and multiply this one.  The two stages are
  // distinct LDS arrays named statically in each call, so the compiler can
  // tell the fragment reads of this stage from the copy into the other one
  // and does not wait for that copy before reading.
  float sa_next = 0.f;
  auto step = [&](int kb, const uint8_t* a_cur, const uint8_t* b_cur, float* sc_cur,
                  uint8_t* a_nxt, uint8_t* b_nxt) {
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    if (sa_thread) {
      sc_cur[sc_w0] = sa_next * sw[(int64_t)nb0 * ld_sw + kb];
      sc_cur[sc_w1] = sa_next * sw[(int64_t)nb1 * ld_sw + kb];
    }
    __syncthreads();                 // block kb is in LDS; block kb - 1 is consumed
    if (kb + 1 < KB) {
      issue(kb + 1, a_nxt, b_nxt);
      if (sa_thread) sa_next = load_sa(kb + 1);
    }
    const uint8_t* at = a_cur + (wm * kPWM) * 128;
    const uint8_t* bt = b_cur + (wn * kPWN) * 128;
    v8i fw[kPNF];
#pragma unroll
    for (int i = 0; i < kPNF; ++i) fw[i] = frag(bt + i * 16 * 128);
    if (KCONST) {
      v8i fa = frag(at);
#pragma unroll
      for (int j = 0; j < kPMF; ++j) {
        const v8i fa_next = j + 1 < kPMF ? frag(at + (j + 1) * 16 * 128) : fa;
#pragma unroll
        for (int i = 0; i < kPNF; ++i) acc[i][j] = mfma_fp8(fw[i], fa, acc[i][j]);
        fa = fa_next;
      }
    } else {
      const float4 s_lo = *reinterpret_cast<const float4*>(sc_cur + sc_rd);
      const float4 s_hi = *reinterpret_cast<const float4*>(sc_cur + sc_rd + 4);
      const float sc[kPMF] = {s_lo.x, s_lo.y, s_lo.z, s_lo.w, s_hi.x, s_hi.y, s_hi.z, s_hi.w};
      v8i fa = frag(at);
      v4f pp[kPNF];
#pragma unroll
      for (int j = 0; j < kPMF; ++j) {
        const v8i fa_next = j + 1 < kPMF ? frag(at + (j + 1) * 16 * 128) : fa;
        v4f pc[kPNF];
#pragma unroll
        for (int i = 0; i < kPNF; ++i) pc[i] = mfma_fp8(fw[i], fa, v4f{0.f, 0.f, 0.f, 0.f});
        if (j > 0) {
#pragma unroll
          for (int i = 0; i < kPNF; ++i)
#pragma unroll
            for (int r = 0; r < 4; ++r)
              acc[i][j - 1][r] = __builtin_fmaf(sc[j - 1], pp[i][r], acc[i][j - 1][r]);
        }
#pragma unroll
        for (int i = 0; i < kPNF; ++i) pp[i] = pc[i];
        fa = fa_next;
      }
#pragma unroll
      for (int i = 0; i < kPNF; ++i)
#pragma unroll
        for (int r = 0; r < 4; ++r)
          acc[i][kPMF - 1][r] = __builtin_fmaf(sc[kPMF - 1], pp[i][r], acc[i][kPMF - 1][r]);
    }
  };

  issue(0, a_lds0, b_lds0);
  if (sa_thread) sa_next = load_sa(0);
  for (int kb = 0; kb < KB; kb += 2) {
    step(kb, a_lds0, b_lds0, sc_lds0, a_lds1, b_lds1);
    if (kb + 1 < KB) step(kb + 1, a_lds1, b_lds1, sc_lds1, a_lds0, b_lds0);   // KB is uniform
  }

  // epilogue: lane writes 4 adjacent bf16 of token row m per weight fragment
#pragma unroll
  for (int j = 0; j < kPMF; ++j) {
    const int64_t gm = m0 + wm * kPWM + j * 16 + r16;
    if (gm < M) {
#pragma unroll
      for (int i = 0; i < kPNF; ++i) {
        const int64_t gn = n0 + wn * kPWN + i * 16 + 4 * kg;
        if (gn < N) {
          float v[4];
#pragma unroll
          for (int r = 0; r < 4; ++r)
            v[r] = KCONST ? acc[i][j][r] * (sa[gm * ld_sa] * sw[(gn + r) * ld_sw]) : acc[i][j][r];
          const uint2 packed = make_uint2(f32_to_bf16_rne(v[0]) | (f32_to_bf16_rne(v[1]) << 16),
                                          f32_to_bf16_rne(v[2]) | (f32_to_bf16_rne(v[3]) << 16));
          *reinterpret_cast<uint2*>(out + gm * ld_out + gn) = packed;
        }
      }
    }
  }
}

// ---------------------------------------------------------------------------
// Prefill shape, hand-scheduled: the MFMA roles of gemm_prefill_kernel
// (its 256 x 256 tile and wave grid, or 128 x 256 tiles of 8 waves of
// 64 x 64), with the K loop as generated gfx950 assembly (prefill_asm.inc,
// written by gen_prefill_asm.py).  C++ below only sets up the operands; the
// assembly issues every copy, fragment read, MFMA and scale fold in a fixed
// order:
//
//  * one K step = 4 MFMA slots per activation fragment of the wave (32 for
//    128 x 64 wave tiles, 16 for 64 x 64); the activation fragment of slot
//    group j + 1 is read while group j multiplies, each partial product is
//    folded four MFMAs after it was issued (six partial-product slots in
//    rotation);
//  * the weight fragments are double-buffered in registers, so the next
//    step's fragments are read as soon as its copy is visible, and the
//    barrier that releases a stage sits before the last fragment group's
//    MFMAs rather than after them (the matrix unit does not drain on it);
//  * the copies of K block kb + S (and its activation scales) go out one per
//    slot after that barrier, S the number of LDS stages (2 for 256 x 256
//    tiles, 3 for 128 x 256 tiles, whose copies get two K steps to land);
//    each barrier waits only for the copies of the next block.  The block
//    index is clamped to the last block, so no copy ever addresses past the
//    operands' K extent.
//
// Activation scales travel by DMA too, four K blocks at a time: every fourth
// step waves 0 .. tm / 64 - 1 copy sa[m0 + row, g .. g + 3] (16 bytes per
// row, one row per lane) into one of two group buffers; per step each lane
// gathers its fragments' scales with ds_read2 pairs.  (One float per row per
// step costs a cache line per row per step.)  The K loop therefore runs on K
// blocks in multiples of four (K % 512 == 0); other K take the C++ kernel.
// The tile's weight blocks' scales for every K block are copied into an LDS
// table once.  Per step the lane
// multiplies its activation scales by its weight block's scale
// (fp32), then folds acc = fma(scale, partial, acc): the arithmetic of the
// C++ kernel, operation for operation.
//
// Buffer descriptors carry the row range of each copy (rows >= M or >= N read
// as zero); the K offset is a scalar offset within the row.  The bf16 output
// is staged through LDS (after a final barrier frees the stages) so every
// store writes 16 contiguous bytes of a row; the stores go through a
// descriptor that ends at row M, and a wave whose 64 columns start at or
// past N skips its stores.
#include "prefill_asm.inc"

// Workgroup shapes of the generated loop, by tag (gen_prefill_asm.py): nw
// waves on a tm x tn tile, tn / 64 waves along N, each wave 64 columns and
// tm / (nw / (tn / 64)) rows; its LDS layout: `stages` activation stages (tm
// rows x 128 B), `stages` weight stages (tn rows x 128 B), two
// activation-scale group buffers, the weight-scale table.
//   W8:  256 x 256, 8 waves of 128 x 64, two stages;
//   W8M: 128 x 256, 8 waves of 64 x 64, three stages (and the split-K form).
constexpr int kPfKbGroup = FP8_PREFILL_KB_GROUP;   // K blocks per activation-scale copy
constexpr int kPrefillMaxKB = 256;            // weight-scale table rows: K <= 32768

#define FP8_PF_SHAPE(TAG)                                                                       \
  struct Pf##TAG {                                                                              \
    static constexpr int nw = FP8_PREFILL_##TAG##_WAVES, tm = FP8_PREFILL_##TAG##_TM,           \
                         tn = FP8_PREFILL_##TAG##_TN, stages = FP8_PREFILL_##TAG##_STAGES,      \
                         unit = FP8_PREFILL_##TAG##_LDS_UNIT,                                   \
                         bytes = FP8_PREFILL_##TAG##_LDS_BYTES, w = FP8_PREFILL_##TAG##_LDS_W,  \
                         sa = FP8_PREFILL_##TAG##_LDS_SA,                                       \
                         sa_group = FP8_PREFILL_##TAG##_LDS_SA_GROUP_BYTES,                     \
                         sw = FP8_PREFILL_##TAG##_LDS_SW;                                       \
  };
FP8_PF_SHAPE(W8)
FP8_PF_SHAPE(W8M)
#undef FP8_PF_SHAPE

template <class L>
constexpr bool pf_layout_ok() {
  return L::unit >= 1024 && L::unit % 16 == 0 &&           // 8 rows of 128 B, then a pad
         L::tn % 64 == 0 && L::nw % (L::tn / 64) == 0 &&    // whole 64-column waves
         L::tm % (16 * (L::nw / (L::tn / 64))) == 0 &&      // whole 16-row fragments
         L::nw % 2 == 0 && L::nw >= 4 &&                    // copy rows, scale-table waves
         L::tm % 64 == 0 && L::tm / 64 <= L::nw &&          // activation-scale copy waves
         L::tn <= 32 * L::nw && L::tn <= 256 &&             // weight-scale table rows
         L::w == L::stages * (L::tm / 8) * L::unit &&       // activation stages first
         L::sa == L::w + L::stages * (L::tn / 8) * L::unit &&   // then the weight stages
         L::sa_group == L::tm * kPfKbGroup * 4 &&           // a group: 4 K blocks of tm rows
         L::sw == L::sa + 2 * L::sa_group &&                // two groups, then the table
         L::bytes == L::sw + 2 * kPrefillMaxKB * 4 &&       // which ends the layout
         L::bytes <= 160 * 1024;                            // LDS of one CU
}
static_assert(pf_layout_ok<PfW8>() && pf_layout_ok<PfW8M>(), "LDS layout of the generated loop");

// tiles of an M x N output in shape S
template <class S>
int64_t pf_tiles(int64_t M, int64_t N) {
  return ((M + S::tm - 1) / S::tm) * ((N + S::tn - 1) / S::tn);
}

typedef int v4i __attribute__((ext_vector_type(4)));

// pair-preserving swizzle: chunk pairs (2c, 2c + 1) stay adjacent, so the two
// 16-byte halves of a lane's fragment are 16 bytes apart in LDS; any eight
// consecutive rows still land on eight distinct 16-byte bank groups.  The
// LDS serves 16 lanes per cycle over 64 four-byte banks, and a fragment read
// spans 16 rows: the pad after every 8 rows (the layout's unit is 1 KiB plus
// 16 bytes) moves rows 8-15 one bank group along, so the 16 rows meet 16
// distinct groups and the read takes one pass instead of two.
__device__ __forceinline__ int swz_pair(int r) { return 2 * ((r >> 1) & 3); }

// Workspace of a split-K launch (two W8M workgroups per 128 x 256 tile, each
// half of the K blocks), one slot per (tile, wave): four 32-bit words at
// 16 slot (arrival counter, ready flag, the XCD records of the two halves),
// zeroed before every launch, and from kSplitWordsBytes on the fp32
// partials, 16 KiB per slot (64 x 64 accumulators, lane-major), which need
// no initial value.
constexpr uint32_t kSplitPartBytes = FP8_PREFILL_SPLIT_PART_BYTES;
constexpr uint32_t kSplitWordsBytes = FP8_PREFILL_SPLIT_WORDS_BYTES;
static_assert(kSplitPartBytes == PfW8M::tm / (PfW8M::nw / (PfW8M::tn / 64)) * 64 * 4,
              "one wave's accumulators per slot");
constexpr uint64_t kSplitMaxSlots = kSplitWordsBytes / 16;
struct SplitLayout {
  uint64_t slots, total;
  __host__ __device__ SplitLayout(int64_t tiles, int nw) {
    slots = (uint64_t)tiles * (uint64_t)nw;
    total = kSplitWordsBytes + slots * kSplitPartBytes;
  }
};

// the scalar operands of the assembly must sit in SGPRs: every one passes
// through readfirstlane (the values are wave-uniform by construction)
__device__ __forceinline__ int pf_uni(int x) { return __builtin_amdgcn_readfirstlane(x); }
__device__ __forceinline__ uint32_t pf_uni(uint32_t x) {
  return (uint32_t)__builtin_amdgcn_readfirstlane((int)x);
}

// raw buffer descriptor over [base, base + bytes), bytes clamped to [0, 2^31 - 1]
__device__ __forceinline__ v4i pf_desc(const void* base, int64_t bytes) {
  const uint64_t b = (uint64_t)(uintptr_t)base;
  const int64_t n = bytes < 0 ? 0 : (bytes > 0x7fffffff ? 0x7fffffff : bytes);
  v4i d;
  d[0] = pf_uni((int)(uint32_t)b);
  d[1] = pf_uni((int)((uint32_t)(b >> 32) & 0xffffu));
  d[2] = pf_uni((int)n);
  d[3] = (int)kRawBufferWord3;
  return d;
}

// Grouped (MoE) tile lookup.  Tile numbers run expert by expert; within
// expert e (t_e = ceil(rows_e / rows) M tiles) the M tile varies fastest, so
// the t_e tiles that read one weight slab (same expert, same N tile) are
// neighbours: they land on one XCD together and share the slab in its L2.
// Every wave runs the same scan (64 experts per step, a wave prefix sum of
// t_e * tiles_n), so the result is uniform over the workgroup.  Returns
// false when the tile lies past the last expert's tiles.
__device__ __forceinline__ bool grouped_tile(const int64_t* __restrict__ offsets, int E,
                                             int64_t M, int tile, int tiles_n, int rows, int& e_out,
                                             int& tm_out, int& tn_out, int64_t& lo_out,
                                             int64_t& hi_out) {
  const int lane = threadIdx.x & 63;
  // 64-bit counts: even offsets that overlap cannot wrap them
  long long base = 0;                            // tiles of the experts before this chunk
  for (int c = 0; c < E; c += 64) {
    const int e = c + lane;
    long long t = 0;
    if (e < E) {
      int64_t lo, hi;
      expert_rows(offsets, e, M, lo, hi);
      t = (hi - lo + rows - 1) / rows * tiles_n;
    }
    long long incl = t;
#pragma unroll
    for (int d = 1; d < 64; d <<= 1) {
      const long long v = __shfl_up(incl, d, 64);
      if (lane >= d) incl += v;
    }
    const long long excl = incl - t;
    const unsigned long long own = __ballot(t > 0 && tile >= base + excl && tile < base + incl);
    if (own) {
      const int l = __ffsll((long long)own) - 1;
      const int e_own = __builtin_amdgcn_readfirstlane(c + l);
      const long long local = (long long)tile - base - __shfl(excl, l, 64);
      int64_t lo, hi;
      expert_rows(offsets, e_own, M, lo, hi);
      const long long te = (hi - lo + rows - 1) / rows;
      // 0 <= local < te * tiles_n by construction; checked anyway
      if (te <= 0 || local < 0 || local >= te * tiles_n) return false;
      e_out = e_own;
      tm_out = __builtin_amdgcn_readfirstlane((int)(local % te));
      tn_out = __builtin_amdgcn_readfirstlane((int)(local / te));
      lo_out = lo;
      hi_out = hi;
      return true;
    }
    base += __shfl(incl, 63, 64);
  }
  return false;
}

// S: the workgroup shape (PfW8, PfW8M).  W8 is the default; W8M serves grids
// whose 256 x 256 tiles would leave CUs idle.
// nsplit = 1 (W8M only, E = 0): two workgroups per tile, consecutive after the
// XCD remap, each over half of the K blocks (the launch passes that half as
// KB); the generated epilogue hands the first half's fp32 accumulators to the
// second through the workspace ws (SplitLayout) before the bf16 stores.
// E > 0: the grouped (MoE) form, chosen at run time so the K loop's code
// exists once per variant.  The grid enumerates the tiles of all experts
// (rounded up to a multiple of 8; workgroups past the last tile exit at
// once), consecutive numbers on one XCD; each workgroup finds its expert and
// tile and then runs the plain kernel on that expert's rows (A, scales and
// output rebased to the expert's first row, M = its row count) and weight
// (w + e * w_es, sw + e * sw_es).  The range-checked descriptors end at the expert's last row,
// so the next expert's rows are neither read nor written.
template <bool KCONST, class S>
__global__ __launch_bounds__(64 * S::nw) void gemm_prefill_asm_kernel(
    const uint8_t* __restrict__ a, int64_t ld_a, const float* __restrict__ sa, int64_t ld_sa,
    const uint8_t* __restrict__ w, int64_t ld_w, const float* __restrict__ sw, int64_t ld_sw,
    uint16_t* __restrict__ out, int64_t ld_out, int64_t M_all, int N, int KB, int tiles_m,
    int tiles_n, const int64_t* __restrict__ offsets, int E, int64_t w_es, int64_t sw_es,
    uint8_t* __restrict__ ws, int nsplit) {
  using Lay = S;
  constexpr int NW = S::nw;
  constexpr int kTM = S::tm, kTN = S::tn;      // tile height and width
  constexpr int kWN = kTN / kPWN;              // waves along N
  constexpr int kWR = kTM / (NW / kWN);        // rows per wave
  constexpr int kSaWaves = kTM / 64;           // waves that copy activation scales
  __shared__ __attribute__((aligned(1024))) uint8_t lds[Lay::bytes];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave / kWN;
  const int wn = wave % kWN;
  const int r16 = lane & 15;
  const int kg = lane >> 4;

  int tm, tn, split = 0, tile = 0;
  int M = (int)M_all;
  if (E > 0) {
    // gridDim.x is a multiple of 8: consecutive tiles share an XCD
    const int G = (int)gridDim.x;
    const int lin = (int)(blockIdx.x % 8) * (G / 8) + (int)(blockIdx.x / 8);
    int e;
    int64_t lo, hi;
    if (!grouped_tile(offsets, E, M_all, lin, tiles_n, kTM, e, tm, tn, lo, hi)) return;
    a += lo * ld_a;
    sa += lo * ld_sa;
    out += lo * ld_out;
    w += (int64_t)e * w_es;
    sw += (int64_t)e * sw_es;
    M = (int)(hi - lo);
  } else {
    // workgroup id -> tile, as gemm_prefill_kernel; with a split K the two
    // halves of a tile are consecutive after the remap (one XCD, one L2)
    const int G = (int)gridDim.x;
    int lin = blockIdx.x;
    if (G % 8 == 0) lin = (lin % 8) * (G / 8) + lin / 8;
    if (nsplit) {
      split = lin & 1;
      lin >>= 1;
    }
    tile = lin;
    const int group = lin / (kGroupM * tiles_n);
    const int first_m = group * kGroupM;
    const int gsize = min(tiles_m - first_m, kGroupM);
    tm = first_m + (lin % (kGroupM * tiles_n)) % gsize;
    tn = (lin % (kGroupM * tiles_n)) / gsize;
  }
  // split K: this workgroup takes K blocks kb0 .. kb0 + KB - 1 of its tile
  // (the launch passes half of them as KB); operand and scale bases move to
  // kb0 and every descriptor still ends where the whole matrix does
  const int kb0 = split * KB;
  const int64_t ksh = (int64_t)kb0 * 128;
  a += ksh;
  w += ksh;
  if (!KCONST) {
    sa += kb0;
    sw += kb0;
  }
  const int64_t m0 = (int64_t)tm * kTM;
  const int64_t n0 = (int64_t)tn * kTN;

  const uint32_t lds0 = (uint32_t)(uintptr_t)lds;

  // copies: wave w, copy t covers tile rows 8 (w + NW t) + (lane >> 3); lane
  // stores 16-byte chunk (lane & 7) of the row, which holds source chunk
  // (lane & 7) ^ swz_pair(row % 16), row % 16 = 8 (w & 1) + (lane >> 3).  The
  // descriptors end at row M (N); copy t adds t * rs to the lane offset.
  const int crow = lane >> 3;
  const int cchunk = (lane & 7) ^ swz_pair(8 * (wave & 1) + crow);
  const uint32_t offA = (uint32_t)((8 * wave + crow) * ld_a + cchunk * 16);
  const uint32_t offW = (uint32_t)((8 * wave + crow) * ld_w + cchunk * 16);
  const v4i dA = pf_desc(a + m0 * ld_a, ((int64_t)M - m0) * ld_a - ksh);
  const v4i dW = pf_desc(w + n0 * ld_w, ((int64_t)N - n0) * ld_w - ksh);
  const uint32_t rsA = pf_uni((uint32_t)(NW * 8 * ld_a));
  const uint32_t rsW = pf_uni((uint32_t)(NW * 8 * ld_w));
  // operand rows sit in units of 8 (Lay::unit bytes: 1 KiB and a pad); copy
  // t of this wave fills unit wave + NW t
  const uint32_t wave1k = pf_uni(lds0 + (uint32_t)(wave * Lay::unit));

  // fragment reads: row r16 of the wave's 16-row group, stored chunk
  // (2 kg) ^ swz_pair(r16) and the next one
  const int p0 = (2 * kg) ^ swz_pair(r16);
  const int rd_row = (r16 >> 3) * Lay::unit + (r16 & 7) * 128 + p0 * 16;
  const uint32_t rdA = lds0 + (uint32_t)(wm * (kWR / 8) * Lay::unit + rd_row);
  const uint32_t rdW = lds0 + (uint32_t)(Lay::w + wn * (kPWN / 8) * Lay::unit + rd_row);

  // activation scales, copied by waves 0 .. tm / 64 - 1 every four K blocks:
  // lane r = 64 wave + lane copies the 16 bytes sa[m0 + r, g .. g + 3] to 16 r
  // of a group buffer, so the scale of tile row r for block g + u sits at
  // 16 r + 4 u; lane r16 of wave row wm reads rows kWR wm + 16 j + r16,
  // fragments 0-3 from scL and 4-7 (if the wave has them) from scH (1 KiB
  // above)
  const uint32_t offSa = (uint32_t)((64 * (wave % kSaWaves) + lane) * ld_sa * 4);
  const v4i dSa = pf_desc(sa + m0 * ld_sa, (((int64_t)M - m0) * ld_sa - kb0) * 4);
  const int wsa = pf_uni(wave < kSaWaves ? 1 : 0);
  const uint32_t sam0 = pf_uni(lds0 + (uint32_t)(Lay::sa + (wave % kSaWaves) * 1024));
  const uint32_t scL0 = lds0 + (uint32_t)(Lay::sa + (wm * kWR + r16) * 16);
  const uint32_t scH0 = scL0 + 4u * 16u * 16u;
  const uint32_t scL1 = scL0 + (uint32_t)Lay::sa_group;
  const uint32_t scH1 = scH0 + (uint32_t)Lay::sa_group;

  // weight-scale table [2][kPrefillMaxKB]: wave w copies row w / 4, blocks
  // 64 (w % 4) + lane; the descriptor ends at the last weight block's last
  // K block, entries past it read zero and are never used
  const int nb0 = (int)(n0 >> 7);
  const uint32_t offSw = (uint32_t)(((wave >> 2) * ld_sw + 64 * (wave & 3) + lane) * 4);
  const v4i dSw = pf_desc(sw + (int64_t)nb0 * ld_sw, (((int64_t)(N / 128) - nb0 - 1) * ld_sw + KB) * 4);
  const uint32_t swm0 = pf_uni(lds0 + (uint32_t)(Lay::sw + wave * 256));
  uint32_t swrd = lds0 + (uint32_t)(Lay::sw + ((wn * kPWN) >> 7) * kPrefillMaxKB * 4);

  // output: bf16 rows from m0, columns from n0; the epilogue derives its
  // lane offsets from the lane id
  const v4i dOut = pf_desc(out + m0 * ld_out + n0, ((int64_t)M - m0) * ld_out * 2 - n0 * 2);
  const uint32_t ldo16 = pf_uni((uint32_t)(16 * ld_out * 2));
  const int colok = pf_uni((n0 + wn * kPWN < N) ? 1 : 0);
  // scales constant along K: row scale sa[m * ld_sa], column scale
  // sw[n * ld_sw] (strides 0: one scale each); the lane's rows are
  // kWR wm + 16 j + r16, its columns 64 wn + 16 i + 4 kg + r
  const v4i dSaR = pf_desc(sa + m0 * ld_sa, (((int64_t)M - m0 - 1) * ld_sa + 1) * 4);
  const v4i dSwR = pf_desc(sw + n0 * ld_sw, (((int64_t)N - n0 - 1) * ld_sw + 1) * 4);
  const uint32_t offSaR = (uint32_t)((wm * kWR + r16) * ld_sa * 4);
  const uint32_t offSwR = (uint32_t)((wn * kPWN + 4 * kg) * ld_sw * 4);
  const uint32_t sjA = pf_uni((uint32_t)(16 * ld_sa * 4));
  const uint32_t siW = pf_uni((uint32_t)(16 * ld_sw * 4));
  const uint32_t srW = pf_uni((uint32_t)(ld_sw * 4));
  const int kb = pf_uni(KB);
  const int kbm1 = pf_uni(KB - 1);
  const int kbm4 = pf_uni(KB - kPfKbGroup);
  const int wave_s = pf_uni(wave);
  const uint32_t ldsb = pf_uni(lds0);

  // split-K hand-over slots of this wave: its fp32 partial, arrival counter
  // and ready flag (SplitLayout)
  const SplitLayout spl(tiles_m * tiles_n, NW);
  const uint32_t slot = (uint32_t)(tile * NW + wave);
  const v4i dWs = pf_desc(ws, nsplit ? (int64_t)spl.total : 0);
  const uint32_t wsPart = pf_uni(kSplitWordsBytes + slot * kSplitPartBytes);
  // 1 | half << 8 for a split launch (the generated code reads the XCD)
  const uint32_t xinfo = pf_uni(nsplit ? 1u | ((uint32_t)split << 8) : 0u);

#define FP8_PF_COMMON_OPERANDS                                                                  \
  [rdA] "v"(rdA), [rdW] "v"(rdW), [offA] "v"(offA), [offW] "v"(offW), [dA] "s"(dA),            \
      [dW] "s"(dW), [rsA] "s"(rsA), [rsW] "s"(rsW), [dOut] "s"(dOut), [wave1k] "s"(wave1k),     \
      [kb] "s"(kb), [kbm1] "s"(kbm1), [ldo16] "s"(ldo16), [colok] "s"(colok),                  \
      [wave] "s"(wave_s), [ldsb] "s"(ldsb)
#define FP8_PF_KCONST_OPERANDS                                                                  \
  [offSaR] "v"(offSaR), [offSwR] "v"(offSwR), [dSaR] "s"(dSaR), [dSwR] "s"(dSwR),               \
      [sjA] "s"(sjA), [siW] "s"(siW), [srW] "s"(srW)
#define FP8_PF_SPLIT_OPERANDS                                                                   \
  [dWs] "s"(dWs), [wsPart] "s"(wsPart), [xinfo] "s"(xinfo)
#define FP8_PF_BLOCK_OPERANDS                                                                   \
  [offSa] "v"(offSa), [scL0] "v"(scL0), [scH0] "v"(scH0), [scL1] "v"(scL1), [scH1] "v"(scH1),  \
      [offSw] "v"(offSw), [dSa] "s"(dSa), [dSw] "s"(dSw), [sam0] "s"(sam0), [wsa] "s"(wsa),     \
      [swm0] "s"(swm0), [kbm4] "s"(kbm4)
  // the shapes with four activation fragments per wave read no scH
#define FP8_PF_BLOCK4_OPERANDS                                                                  \
  [offSa] "v"(offSa), [scL0] "v"(scL0), [scL1] "v"(scL1), [offSw] "v"(offSw), [dSa] "s"(dSa),   \
      [dSw] "s"(dSw), [sam0] "s"(sam0), [wsa] "s"(wsa), [swm0] "s"(swm0), [kbm4] "s"(kbm4)
#define FP8_PF_ASM(TEXT, ...) \
  asm volatile(TEXT : [swrd] "+v"(swrd) : __VA_ARGS__ : FP8_PREFILL_ASM_CLOBBERS)
  if constexpr (KCONST) {
    if constexpr (std::is_same<S, PfW8>::value)
      FP8_PF_ASM(FP8_PREFILL_ASM_TENSOR_W8, FP8_PF_COMMON_OPERANDS, FP8_PF_KCONST_OPERANDS);
    else if constexpr (std::is_same<S, PfW8M>::value)
      FP8_PF_ASM(FP8_PREFILL_ASM_TENSOR_W8M, FP8_PF_COMMON_OPERANDS, FP8_PF_KCONST_OPERANDS,
                 FP8_PF_SPLIT_OPERANDS);
    else
      static_assert(sizeof(S) == 0, "no generated loop for this shape");
  } else {
    if constexpr (std::is_same<S, PfW8>::value)
      FP8_PF_ASM(FP8_PREFILL_ASM_BLOCK_W8, FP8_PF_COMMON_OPERANDS, FP8_PF_BLOCK_OPERANDS);
    else if constexpr (std::is_same<S, PfW8M>::value)
      FP8_PF_ASM(FP8_PREFILL_ASM_BLOCK_W8M, FP8_PF_COMMON_OPERANDS, FP8_PF_BLOCK4_OPERANDS,
                 FP8_PF_SPLIT_OPERANDS);
    else
      static_assert(sizeof(S) == 0, "no generated loop for this shape");
  }
#undef FP8_PF_ASM
#undef FP8_PF_BLOCK4_OPERANDS
#undef FP8_PF_COMMON_OPERANDS
#undef FP8_PF_KCONST_OPERANDS
#undef FP8_PF_BLOCK_OPERANDS
#undef FP8_PF_SPLIT_OPERANDS
}

// zeroes n 32-bit words (the split-K slot words), one per thread, without a
// memset node, so the launch sequence stays capturable
__global__ __launch_bounds__(256) void zero_words_kernel(uint32_t* __restrict__ p, int64_t n) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i < n) p[i] = 0u;
}

// ws != nullptr: split K in two (W8M only; ws holds SplitLayout's bytes for
// this grid and KB is a multiple of 8)
template <class S>
hipError_t launch_prefill_asm(const uint8_t* a, int64_t ld_a, const float* sa, int64_t ld_sa,
                              const uint8_t* w, int64_t ld_w, const float* sw, int64_t ld_sw,
                              uint16_t* out, int64_t ld_out, int64_t M, int64_t N, int KB,
                              bool kconst, uint8_t* ws, hipStream_t st, bool words_zero = false) {
  const int tiles_m = (int)((M + S::tm - 1) / S::tm);
  const int tiles_n = (int)((N + S::tn - 1) / S::tn);
  const int nsplit = ws ? 1 : 0;
  if (nsplit && !std::is_same<S, PfW8M>::value) return hipErrorInvalidValue;
  dim3 grid((uint32_t)tiles_m * (uint32_t)tiles_n * (nsplit ? 2u : 1u));
  if (nsplit) {
    const SplitLayout spl((int64_t)tiles_m * tiles_n, S::nw);
    const int64_t words = (int64_t)spl.slots * 4;
    const int64_t blocks = (words + 255) / 256;
    if (!words_zero)
      hipLaunchKernelGGL(zero_words_kernel, dim3((uint32_t)blocks), dim3(256), 0, st,
                         (uint32_t*)ws, words);
    KB /= 2;
  }
  if (kconst)
    hipLaunchKernelGGL((gemm_prefill_asm_kernel<true, S>), grid, dim3(64 * S::nw), 0, st, a,
                       ld_a, sa, ld_sa, w, ld_w, sw, ld_sw, out, ld_out, M, (int)N, KB, tiles_m,
                       tiles_n, nullptr, 0, (int64_t)0, (int64_t)0, ws, nsplit);
  else
    hipLaunchKernelGGL((gemm_prefill_asm_kernel<false, S>), grid, dim3(64 * S::nw), 0, st, a,
                       ld_a, sa, ld_sa, w, ld_w, sw, ld_sw, out, ld_out, M, (int)N, KB, tiles_m,
                       tiles_n, nullptr, 0, (int64_t)0, (int64_t)0, ws, nsplit);
  return hipGetLastError();
}

// Grouped launch: at most floor((M + (tm - 1) E) / tm) M tiles over all
// experts (each expert's last tile may be partial), times the N tiles,
// rounded up to a multiple of 8.
template <class S>
hipError_t launch_prefill_asm_grouped(const uint8_t* a, int64_t ld_a, const float* sa,
                                      int64_t ld_sa, const uint8_t* w, int64_t ld_w, int64_t w_es,
                                      const float* sw, int64_t ld_sw, int64_t sw_es,
                                      uint16_t* out, int64_t ld_out, const int64_t* offsets,
                                      int64_t E, int64_t M, int64_t N, int KB, hipStream_t st) {
  const int64_t tiles_m = (M + (S::tm - 1) * E) / S::tm;
  const int64_t tiles_n = (N + S::tn - 1) / S::tn;
  const int64_t g = (tiles_m * tiles_n + 7) / 8 * 8;
  if (g == 0) return hipSuccess;
  hipLaunchKernelGGL((gemm_prefill_asm_kernel<false, S>), dim3((uint32_t)g), dim3(64 * S::nw),
                     0, st, a, ld_a, sa, ld_sa, w, ld_w, sw, ld_sw, out, ld_out, M, (int)N, KB,
                     (int)tiles_m, (int)tiles_n, offsets, (int)E, w_es, sw_es, nullptr, 0);
  return hipGetLastError();
}

// compute units of the current device (looked up once per device; every
// thread that races on the first lookup stores the same value)
std::atomic<int> g_device_cus[64];

int device_cus() {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
  int n = g_device_cus[dev].load(std::memory_order_relaxed);
  if (n == 0) {
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0)
      n = 256;
    g_device_cus[dev].store(n, std::memory_order_relaxed);
  }
  return n;
}

// ---------------------------------------------------------------------------
// Fused decode linear (M <= 16): the decode GEMM above with the dynamic 1x128
// activation quantization done inside it, one launch per call.  Each wave
// quantizes the groups of its own K blocks just in time: the bf16 loads of
// block kb are issued with its weight copy.  (The compiler waits for every
// load in flight before the bf16 values are used, since it does not order
// ordinary loads against LDS copies, so the quantization follows the copy's
// arrival; staging the bf16 rows by LDS copy to overlap the two was no
// faster.)  Quantization uses the same lane
// layout and device functions as quant_act_block_kernel (16 lanes x 8 values
// per group, 16-lane DPP max), so the codes and scales are bit-identical to
// fp8_quant_act's; the MFMA, fold and reduction order equal the decode
// GEMM's, so the output is bit-identical to quantizing and then calling the
// GEMM.  Codes land in the wave's LDS A fragment (swizzled like the copies);
// rows >= M stay zero, as do their scales.
//
// Dynamic LDS per wave: W fragment (2 KiB), A fragment (2 KiB), 16 scales;
// then the reduction buffer (KSPLIT * 1 KiB).
template <int KSPLIT>
constexpr size_t linear_decode_lds_bytes() {
  return (size_t)KSPLIT * (2 * kFrag + 64) + (size_t)KSPLIT * 4 * 64 * sizeof(float);
}

template <int KSPLIT>
__global__ __launch_bounds__(64 * KSPLIT) void linear_decode_kernel(
    const uint16_t* __restrict__ x, int64_t ld_x, const uint8_t* __restrict__ w, int64_t ld_w,
    const float* __restrict__ sw, int64_t ld_sw, uint16_t* __restrict__ out, int64_t ld_out,
    int M, int KB) {
  extern __shared__ __attribute__((aligned(16))) uint8_t lds[];
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int r16 = lane & 15;
  const int kg = lane >> 4;
  const int64_t n0 = (int64_t)blockIdx.x * 16;
  const bool arow = r16 < M;

  uint8_t* wbuf = lds + (size_t)wave * (2 * kFrag + 64);
  uint8_t* abuf = wbuf + kFrag;
  float* sbuf = reinterpret_cast<float*>(abuf + kFrag);
  float* red = reinterpret_cast<float*>(lds + (size_t)KSPLIT * (2 * kFrag + 64));

  // rows >= M of the A fragment and their scales stay zero
  for (int i = lane; i < kFrag / 16; i += 64)
    reinterpret_cast<uint4*>(abuf)[i] = make_uint4(0, 0, 0, 0);
  if (lane < 16) sbuf[lane] = 0.f;

  // weight copy slots and fragment reads as in gemm_decode_kernel
  const int drow = lane >> 3;
  const uint8_t* wsrc0 = w + (n0 + drow) * ld_w + ((lane & 7) ^ swz(drow)) * 16;
  const uint8_t* wsrc1 = w + (n0 + 8 + drow) * ld_w + ((lane & 7) ^ swz(8 + drow)) * 16;
  const int rd0 = r16 * 128 + (((2 * kg) ^ swz(r16)) * 16);
  const int rd1 = r16 * 128 + (((2 * kg + 1) ^ swz(r16)) * 16);

  // quantization: pass p covers rows 4 p + (lane >> 4); lane & 15 holds 8
  // values of the row's 128-group.  Rows past M in a pass read row M - 1 and
  // are not written.
  const int q_row = lane >> 4;
  const int q_l16 = lane & 15;
  const int npass = (M + 3) >> 2;                     // uniform, 1..4

  const int per = (KB + KSPLIT - 1) / KSPLIT;
  const int kb_lo = wave * per;
  const int kb_hi = min(KB, kb_lo + per);

  uint4 xv[4];
  auto issue = [&](int kb) {
#pragma unroll
    for (int p = 0; p < 4; ++p) {
      if (p < npass) {
        const int m = min(4 * p + q_row, M - 1);
        xv[p] = *reinterpret_cast<const uint4*>(x + (int64_t)m * ld_x + (int64_t)kb * 128 + q_l16 * 8);
      }
    }
    const int64_t off = (int64_t)kb * 128;
    __builtin_amdgcn_global_load_lds((const void*)(wsrc0 + off),
                                     (__attribute__((address_space(3))) void*)wbuf, 16, 0, 0);
    __builtin_amdgcn_global_load_lds((const void*)(wsrc1 + off),
                                     (__attribute__((address_space(3))) void*)(wbuf + 1024), 16, 0, 0);
  };
  auto frag = [&](const uint8_t* buf) {
    const uint4 a0 = *reinterpret_cast<const uint4*>(buf + rd0);
    const uint4 a1 = *reinterpret_cast<const uint4*>(buf + rd1);
    v8i r;
    r[0] = (int)a0.x; r[1] = (int)a0.y; r[2] = (int)a0.z; r[3] = (int)a0.w;
    r[4] = (int)a1.x; r[5] = (int)a1.y; r[6] = (int)a1.z; r[7] = (int)a1.w;
    return r;
  };

  v4f acc = {0.f, 0.f, 0.f, 0.f};
  if (kb_lo < kb_hi) issue(kb_lo);
  for (int kb = kb_lo; kb < kb_hi; ++kb) {            // wave-uniform; no barrier inside
    // the activation loads of block kb went out before its two weight copies
    // (the compiler adds the wait for those too before the values are used)
    asm volatile("s_waitcnt vmcnt(2)" ::: "memory");
#pragma unroll
    for (int p = 0; p < 4; ++p) {
      if (p < npass) {
        const uint32_t amax = row16_max(absmax8_bits(xv[p]));
        const GroupDivisor d = make_divisor(__uint_as_float(amax));
        const uint2 c = quant8(xv[p], d);
        const int m = 4 * p + q_row;
        if (m < M) {
          *reinterpret_cast<uint2*>(abuf + m * 128 + (((q_l16 >> 1) ^ swz(m)) * 16) +
                                    (q_l16 & 1) * 8) = c;
          if (q_l16 == 0) sbuf[m] = d.s;
        }
      }
    }
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");  // the weight fragment has landed
    v8i av = frag(abuf);
    const v8i bw = frag(wbuf);
    const float s_w = sw[(int64_t)(n0 >> 7) * ld_sw + kb];
    float sc[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) sc[i] = sbuf[4 * kg + i] * s_w;
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
    if (kb + 1 < kb_hi) issue(kb + 1);
#pragma unroll
    for (int e = 0; e < 8; ++e) av[e] = arow ? av[e] : 0;
    const v4f p = mfma_fp8(av, bw, v4f{0.f, 0.f, 0.f, 0.f});
#pragma unroll
    for (int i = 0; i < 4; ++i) acc[i] = __builtin_fmaf(sc[i], p[i], acc[i]);
  }
#pragma unroll
  for (int i = 0; i < 4; ++i) red[(wave * 4 + i) * 64 + lane] = acc[i];
  __syncthreads();
  if (wave == 0) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      float v = 0.f;
#pragma unroll
      for (int s2 = 0; s2 < KSPLIT; ++s2) v += red[(s2 * 4 + i) * 64 + lane];
      const int m = 4 * kg + i;
      if (m < M) out[(int64_t)m * ld_out + n0 + r16] = (uint16_t)f32_to_bf16_rne(v);
    }
  }
}

}  // namespace

hipError_t launch_linear_decode(const uint16_t* x, int64_t ld_x, const uint8_t* w, int64_t ld_w,
                                const float* sw, int64_t ld_sw, uint16_t* out, int64_t ld_out,
                                int64_t M, int64_t N, int64_t K, hipStream_t st) {
  // the same split as the decode GEMM, so the two paths agree bit for bit
  constexpr int KSPLIT = FP8_DECODE_KSPLIT;
  dim3 grid((uint32_t)(N / 16));
  hipLaunchKernelGGL((linear_decode_kernel<KSPLIT>), grid, dim3(64 * KSPLIT),
                     linear_decode_lds_bytes<KSPLIT>(), st, x, ld_x, w, ld_w, sw, ld_sw, out,
                     ld_out, (int)M, (int)(K / 128));
  return hipGetLastError();
}

// Every workgroup of the fused kernel quantizes all M rows over its K range,
// so the fused launch pays M * K quantizations per wave group and N / 16
// times that over the grid.  Up to 4 rows it beats the separate quantizer
// launch at any width (measured on MI355X at N = 11008, K = 4096); up to 16
// rows only while both counts stay small: per call, replayed from a graph,
// 16 x 256 x 512 took 3.9 against 5.1 us and 16 x 512 x 1024 4.5 against
// 5.3 us, while 16 x 1024 x 4096 took 9.5 against 7.0 us and 8 x 4096 x 4096
// 7.3 against 7.1 us.
constexpr int64_t kFusedMaxM = 4;
constexpr int64_t kFusedWideMaxM = 16;           // rows of the fused kernel's A fragment
constexpr int64_t kFusedWideMaxMK = 16384;       // M * K
constexpr int64_t kFusedWideMaxGridMK = 1 << 21; // (N / 16) * M * K

bool linear_decode_supported(int64_t M, int64_t N, int64_t K) {
  if (M < 1 || K / 128 > kDecodeMaxKB) return false;
  if (M <= kFusedMaxM) return true;
  return M <= kFusedWideMaxM && M * K <= kFusedWideMaxMK &&
         (N / 16) * M * K <= kFusedWideMaxGridMK;
}

// Work-items of the grid a GEMM launches: the decode tile (16 columns per
// 64 * KSPLIT-thread workgroup) up to 64 rows, otherwise at most the
// 128 x 128 tile kernel's (256 threads per 128 x 128 tile), which bounds the
// prefill kernels' 256 x 256 and 128 x 256 tiles too (a split-K launch has
// at most as many workgroups as the device has CUs).
uint64_t gemm_items(int64_t M, int64_t N, int64_t K) {
  if (M <= FP8_DECODE_MAX_M && K / 128 <= kDecodeMaxKB)
    return (uint64_t)(N / 16) * 64u * FP8_DECODE_KSPLIT;
  return (uint64_t)((M + kBM - 1) / kBM) * (uint64_t)(N / kBN) * 256u;
}

uint64_t linear_decode_items(int64_t N) { return (uint64_t)(N / 16) * 64u * FP8_DECODE_KSPLIT; }

// The grouped call's decode-tile path (grid x: 16 columns per workgroup);
// the grouped prefill path is taken only when its own grid fits.
uint64_t grouped_items(int64_t N) { return (uint64_t)(N / 16) * 64u * FP8_DECODE_KSPLIT; }

// The hand-scheduled prefill kernel takes the call (strides within its
// 32-bit offsets, K a multiple of 4 blocks).
bool prefill_asm_ok(int64_t M, int64_t KB, bool kconst, int64_t ld_a, int64_t ld_sa,
                    int64_t ld_w, int64_t ld_sw, int64_t ld_out) {
  return FP8_PREFILL_ASM && M > 64 && KB % kPfKbGroup == 0 && KB <= kPrefillMaxKB &&
         (!kconst || ld_sw < kPrefillMaxLd / 4) && ld_a < kPrefillMaxLd &&
         ld_w < kPrefillMaxLd && ld_out < kPrefillMaxLd / 2 && ld_sa < kPrefillMaxLd / 4 &&
         ld_sw < kPrefillMaxLd;
}

// Calls whose 128 x 256 tiles would occupy at most half of the CUs: K split
// in two (each half a multiple of 4 blocks) when a workspace is given.  0
// when the call does not split.  Scales constant along K are applied after
// the hand-over, to the sum of the two halves.
size_t gemm_split_bytes(int64_t M, int64_t N, int64_t K) {
  const int64_t KB = K / 128;
  if (!FP8_PREFILL_ASM || M <= 64 || KB % (2 * kPfKbGroup) != 0 || KB > kPrefillMaxKB)
    return 0;
  if (M <= FP8_DECODE_MAX_M && KB <= kDecodeMaxKB) return 0;
  const int64_t tiles = pf_tiles<PfW8M>(M, N);
  if (2 * tiles > device_cus() || (uint64_t)tiles * PfW8M::nw > kSplitMaxSlots) return 0;
  return (size_t)SplitLayout(tiles, PfW8M::nw).total;
}

uint32_t gemm_split_words(int64_t M, int64_t N, int64_t K) {
  if (!gemm_split_bytes(M, N, K)) return 0;
  return (uint32_t)(SplitLayout(pf_tiles<PfW8M>(M, N), PfW8M::nw).slots * 4);
}

hipError_t launch_gemm(const uint8_t* a, int64_t ld_a, const float* sa, int64_t ld_sa,
                       const uint8_t* w, int64_t ld_w, const float* sw, int64_t ld_sw,
                       uint16_t* out, int64_t ld_out, int64_t M, int64_t N, int64_t K,
                       bool kconst, void* ws, size_t ws_bytes, hipStream_t st, bool words_zero) {
  const int KB = (int)(K / 128);
  if (M <= FP8_DECODE_MAX_M && KB <= kDecodeMaxKB) {
    constexpr int KSPLIT = FP8_DECODE_KSPLIT, KBW = FP8_DECODE_KBW;
    dim3 grid((uint32_t)(N / 16));
    const size_t lds = decode_lds_bytes<KSPLIT, KBW>(KB, kconst);
    const dim3 block(64 * KSPLIT);
    if (M <= 16) {
      if (kconst)
        hipLaunchKernelGGL((gemm_decode_kernel<KSPLIT, KBW, true, false>), grid, block, lds, st,
                           a, ld_a, sa, ld_sa, w, ld_w, sw, ld_sw, out, ld_out, (int)M, KB);
      else
        hipLaunchKernelGGL((gemm_decode_kernel<KSPLIT, KBW, false, false>), grid, block, lds, st,
                           a, ld_a, sa, ld_sa, w, ld_w, sw, ld_sw, out, ld_out, (int)M, KB);
    } else {
      if (kconst)
        hipLaunchKernelGGL((gemm_decode_kernel<KSPLIT, KBW, true, true>), grid, block, lds, st,
                           a, ld_a, sa, ld_sa, w, ld_w, sw, ld_sw, out, ld_out, (int)M, KB);
      else
        hipLaunchKernelGGL((gemm_decode_kernel<KSPLIT, KBW, false, true>), grid, block, lds, st,
                           a, ld_a, sa, ld_sa, w, ld_w, sw, ld_sw, out, ld_out, (int)M, KB);
    }
    return hipGetLastError();
  }
  if (prefill_asm_ok(M, KB, kconst, ld_a, ld_sa, ld_w, ld_sw, ld_out)) {
    // 256 x 256 tiles unless they would occupy at most half of the CUs: then
    // 128 x 256 tiles (three LDS stages), with K split in two over twice the
    // workgroups when those too would occupy at most half of the CUs and the
    // caller gave the workspace
    if (2 * pf_tiles<PfW8>(M, N) > device_cus())
      return launch_prefill_asm<PfW8>(a, ld_a, sa, ld_sa, w, ld_w, sw, ld_sw, out, ld_out, M, N,
                                      KB, kconst, nullptr, st);
    const size_t need = gemm_split_bytes(M, N, K);
    if (need && ws && ws_bytes >= need)
      return launch_prefill_asm<PfW8M>(a, ld_a, sa, ld_sa, w, ld_w, sw, ld_sw, out, ld_out, M, N,
                                       KB, kconst, (uint8_t*)ws, st, words_zero);
    return launch_prefill_asm<PfW8M>(a, ld_a, sa, ld_sa, w, ld_w, sw, ld_sw, out, ld_out, M, N, KB,
                                     kconst, nullptr, st);
  }
  if (M > 64 && ld_a < kPrefillMaxLd && ld_w < kPrefillMaxLd) {
    const int tiles_m = (int)((M + kPM - 1) / kPM);
    const int tiles_n = (int)((N + kPN - 1) / kPN);
    dim3 grid((uint32_t)tiles_m * (uint32_t)tiles_n);
    if (kconst)
      hipLaunchKernelGGL(gemm_prefill_kernel<true>, grid, dim3(kPThreads), 0, st, a, ld_a, sa,
                         ld_sa, w, ld_w, sw, ld_sw, out, ld_out, (int)M, (int)N, KB, tiles_m,
                         tiles_n);
    else
      hipLaunchKernelGGL(gemm_prefill_kernel<false>, grid, dim3(kPThreads), 0, st, a, ld_a, sa,
                         ld_sa, w, ld_w, sw, ld_sw, out, ld_out, (int)M, (int)N, KB, tiles_m,
                         tiles_n);
    return hipGetLastError();
  }
  const int tiles_m = (int)((M + kBM - 1) / kBM);
  const int tiles_n = (int)(N / kBN);
  dim3 grid((uint32_t)tiles_m * (uint32_t)tiles_n);
  if (kconst)
    hipLaunchKernelGGL(gemm_tile_kernel<true>, grid, dim3(256), 0, st, a, ld_a, sa, ld_sa, w, ld_w,
                       sw, ld_sw, out, ld_out, (int)M, KB, tiles_n);
  else
    hipLaunchKernelGGL(gemm_tile_kernel<false>, grid, dim3(256), 0, st, a, ld_a, sa, ld_sa, w, ld_w,
                       sw, ld_sw, out, ld_out, (int)M, KB, tiles_n);
  return hipGetLastError();
}

// Grouped (MoE) block-scaled GEMM.  A few rows per expert on average: the
// decode tile per (16 columns, expert); otherwise the grouped form of the
// hand-scheduled prefill kernel.
#ifndef FP8_GROUPED_DECODE_MAX_AVG
#define FP8_GROUPED_DECODE_MAX_AVG 32
#endif

static_assert(kGroupedMaxKB <= kDecodeMaxKB, "grouped calls must fit the decode tile");

bool grouped_prefill_ok(int64_t M, int64_t E, int64_t N, int64_t K, int64_t ld_a, int64_t ld_w,
                        int64_t ld_sa, int64_t ld_sw, int64_t ld_out) {
  const int64_t KB = K / 128;
  // grid: at most (M + (tm - 1) E) / tm M tiles times the N tiles of either
  // tile shape, rounded up to a multiple of 8 workgroups
  const uint64_t tn = (uint64_t)((N + 255) / 256);
  const uint64_t t8 = (uint64_t)((M + (PfW8::tm - 1) * E) / PfW8::tm);
  const uint64_t tM = (uint64_t)((M + (PfW8M::tm - 1) * E) / PfW8M::tm);
  const uint64_t g8 = (t8 * tn + 7) / 8 * 8 * 512u;
  const uint64_t gM = (tM * tn + 7) / 8 * 8 * 512u;
  return FP8_PREFILL_ASM && M > FP8_GROUPED_DECODE_MAX_AVG * E && KB % kPfKbGroup == 0 &&
         KB <= kPrefillMaxKB && ld_a < kPrefillMaxLd && ld_w < kPrefillMaxLd &&
         ld_out < kPrefillMaxLd / 2 && ld_sa < kPrefillMaxLd / 4 && ld_sw < kPrefillMaxLd &&
         g8 < kMaxGridItems && gM < kMaxGridItems;
}

hipError_t launch_grouped_gemm(const uint8_t* a, int64_t ld_a, const float* sa, int64_t ld_sa,
                               const uint8_t* w, int64_t ld_w, const float* sw, int64_t ld_sw,
                               uint16_t* out, int64_t ld_out, const int64_t* offsets, int64_t E,
                               int64_t M, int64_t N, int64_t K, hipStream_t st) {
  const int KB = (int)(K / 128);
  const int64_t w_es = N * ld_w;                   // expert strides
  const int64_t sw_es = (N / 128) * ld_sw;
  if (grouped_prefill_ok(M, E, N, K, ld_a, ld_w, ld_sa, ld_sw, ld_out)) {
    // 128-row tiles while the experts average at most 512 rows: they waste
    // fewer padded rows, and their three LDS stages keep more weight bytes
    // in flight
    if (M <= 512 * E)
      return launch_prefill_asm_grouped<PfW8M>(a, ld_a, sa, ld_sa, w, ld_w, w_es, sw, ld_sw,
                                               sw_es, out, ld_out, offsets, E, M, N, KB, st);
    return launch_prefill_asm_grouped<PfW8>(a, ld_a, sa, ld_sa, w, ld_w, w_es, sw, ld_sw, sw_es,
                                            out, ld_out, offsets, E, M, N, KB, st);
  }
  constexpr int KSPLIT = FP8_DECODE_KSPLIT, KBW = FP8_DECODE_KBW;
  dim3 grid((uint32_t)(N / 16), (uint32_t)E);
  const size_t lds = decode_lds_bytes<KSPLIT, KBW>(KB, false);
  hipLaunchKernelGGL((gemm_grouped_decode_kernel<KSPLIT, KBW>), grid, dim3(64 * KSPLIT), lds, st,
                     a, ld_a, sa, ld_sa, w, ld_w, w_es, sw, ld_sw, sw_es, out, ld_out, offsets, M,
                     KB);
  return hipGetLastError();
}

}  // namespace fp8k
