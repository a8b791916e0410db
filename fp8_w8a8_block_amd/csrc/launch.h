// Internal launchers behind the C ABI.  Arguments are already validated by
// the ABI layer (abi.hip); each launcher only enqueues kernels on `st` and
// returns hipGetLastError() of the launch.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace fp8k {

// workspace of the per-tensor quantizer: one partial amax per workgroup of
// the first pass
constexpr int kTensorPartials = 1024;

// Work-items of the largest grid a call launches.  A dispatch packet holds
// the grid size in work-items as a 32-bit value, so every launch must stay
// below 2^32; the ABI rejects larger calls as shapes before anything is
// enqueued.  (The per-tensor, static and KV-cache kernels stride over their
// data with at most 8192 workgroups and never come near the limit.)
constexpr uint64_t kMaxGridItems = (uint64_t)1 << 32;
uint64_t quant_act_block_items(int64_t M, int64_t K);
uint64_t quant_weight_block_items(int64_t N, int64_t K);
uint64_t quant_rows_items(int64_t R);
uint64_t encode_items(int64_t n);
uint64_t gemm_items(int64_t M, int64_t N, int64_t K);
uint64_t grouped_items(int64_t N);
uint64_t linear_decode_items(int64_t N);

// zero / zero_n: words the launch also sets to 0 (the next GEMM's split-K
// slot words, so that GEMM needs no clearing launch of its own)
hipError_t launch_quant_act_block(const uint16_t* x, int64_t M, int64_t K, int64_t ld_x,
                                  uint8_t* q, int64_t ld_q, float* s, int64_t ld_s,
                                  hipStream_t st, uint32_t* zero = nullptr, uint32_t zero_n = 0);
hipError_t launch_quant_weight_block(const uint16_t* w, int64_t N, int64_t K, int64_t ld_w,
                                     uint8_t* q, int64_t ld_q, float* s, int64_t ld_s,
                                     hipStream_t st);
hipError_t launch_quant_tensor(const uint16_t* x, int64_t R, int64_t C, int64_t ld_x,
                               uint8_t* q, int64_t ld_q, float* s, uint32_t* partials,
                               hipStream_t st);
hipError_t launch_quant_rows(const uint16_t* x, int64_t R, int64_t K, int64_t ld_x, uint8_t* q,
                             int64_t ld_q, float* s, int64_t ld_s, hipStream_t st);
hipError_t launch_quant_static(const uint16_t* x, int64_t R, int64_t K, int64_t ld_x, uint8_t* q,
                               int64_t ld_q, const float* scale, hipStream_t st);
hipError_t launch_encode_f32(const float* x, int64_t n, uint8_t* codes, hipStream_t st);

// out = A . W^T.  kconst = false: block scales sa[m * ld_sa + kb],
// sw[(n / 128) * ld_sw + kb].  kconst = true: scales constant along K,
// out[m, n] = (sa[m * ld_sa] * sw[n * ld_sw]) * acc; ld_sa = ld_sw = 0 is the
// per-tensor case.  ws: device workspace of ws_bytes (may be null); a call
// for which gemm_split_bytes is nonzero splits K in two when ws_bytes is at
// least that (16-byte aligned, contents not needed), else runs unsplit.
// words_zero: the split-K slot words (the first gemm_split_words 32-bit
// words of ws) are already 0, so the launch skips clearing them.
hipError_t launch_gemm(const uint8_t* a, int64_t ld_a, const float* sa, int64_t ld_sa,
                       const uint8_t* w, int64_t ld_w, const float* sw, int64_t ld_sw,
                       uint16_t* out, int64_t ld_out, int64_t M, int64_t N, int64_t K,
                       bool kconst, void* ws, size_t ws_bytes, hipStream_t st,
                       bool words_zero = false);
// Workspace bytes of launch_gemm's split-K path on the current device for
// this shape, any scale form (0: the call never splits), and how many 32-bit
// words at its start must be 0 when the launch begins.
size_t gemm_split_bytes(int64_t M, int64_t N, int64_t K);
uint32_t gemm_split_words(int64_t M, int64_t N, int64_t K);

// Fused decode linear: dynamic 1x128 quantization of x inside the decode GEMM
// (block scales).  Dispatched for K <= 16384 and 1 <= M <= 4, or M <= 16
// with M * K <= 16384 and (N / 16) * M * K <= 2^21; the result is
// bit-identical to launch_quant_act_block followed by launch_gemm.
bool linear_decode_supported(int64_t M, int64_t N, int64_t K);
hipError_t launch_linear_decode(const uint16_t* x, int64_t ld_x, const uint8_t* w, int64_t ld_w,
                                const float* sw, int64_t ld_sw, uint16_t* out, int64_t ld_out,
                                int64_t M, int64_t N, int64_t K, hipStream_t st);

// largest K / 128 of a grouped call (its decode-tile path stages the
// activation scales of a row chunk in LDS)
constexpr int kGroupedMaxKB = 128;

// Grouped (MoE) block-scaled GEMM: rows offsets[e] .. offsets[e + 1] of A
// (clamped to [0, M]) against expert e's weight w + e * N * ld_w with scales
// sw + e * (N / 128) * ld_sw.  E >= 1; K <= 16384 (decode-tile path).
hipError_t launch_grouped_gemm(const uint8_t* a, int64_t ld_a, const float* sa, int64_t ld_sa,
                               const uint8_t* w, int64_t ld_w, const float* sw, int64_t ld_sw,
                               uint16_t* out, int64_t ld_out, const int64_t* offsets, int64_t E,
                               int64_t M, int64_t N, int64_t K, hipStream_t st);

// FP8 KV-cache codec: HD = heads * head_dim values per token (multiple of 8),
// capacity = blocks * block_size slots; out-of-range slots are skipped on
// write and read as zeros.
hipError_t launch_kv_write(const uint16_t* k, int64_t ld_k, const uint16_t* v, int64_t ld_v,
                           const int64_t* slots, int64_t T, int64_t HD, uint8_t* kc, uint8_t* vc,
                           int64_t capacity, const float* k_scale, const float* v_scale,
                           hipStream_t st);
hipError_t launch_kv_read(const uint8_t* cache, int64_t capacity, int64_t HD, const int64_t* slots,
                          int64_t T, const float* scale, uint16_t* out, int64_t ld_out,
                          hipStream_t st);

}  // namespace fp8k
