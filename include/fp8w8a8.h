/*
 * fp8w8a8.h -- C ABI of the FP8 W8A8 block-scaled linear layer for gfx950.
 *
 * What the library computes (the passages each call follows are named on
 * the call):
 *   1. dynamic activation quantization: per token, per 128-element group,
 *      scale = amax / 448, codes = E4M3(x / scale) rounded to nearest even
 *      and saturating;
 *   2. 128x128 block quantization of the weight (the same rule per block);
 *   3. the block-scaled FP8 x FP8 GEMM out = A . W^T with fp32 accumulation,
 *      the two scales applied once per 128-wide K block, bf16 output.
 *
 * Conventions shared by every call
 *   - Tensor pointers are DEVICE pointers owned by the caller.  The library
 *     never allocates, frees or synchronizes; it enqueues kernels on
 *     `stream` (a hipStream_t; NULL is the default stream) and returns.
 *   - bf16 tensors are raw uint16 bit patterns, FP8 tensors raw uint8 OCP
 *     E4M3 codes (bias 7, max 448, NaN = S.1111.111, no infinity), scales
 *     fp32.  Matrices are row-major with an explicit leading dimension in
 *     elements (ld >= row length).
 *   - Argument errors are detected on the host and returned before anything
 *     is enqueued; a failed launch returns FP8_ERR_LAUNCH.  On error no
 *     output is written.
 *   - Inputs and outputs must not overlap (FP8_ERR_ALIAS).
 *   - M = 0 is a valid empty call (nothing is enqueued).  K and N must be
 *     positive multiples of 128.
 *   - Alignment: base pointers of bf16 and FP8 tensors 16-byte aligned,
 *     scale pointers 4-byte aligned; ld of bf16 tensors a multiple of 8,
 *     of FP8 tensors a multiple of 16 (FP8_ERR_ALIGN).
 *   - Calls are thread-safe; the only global state is a per-device cache of
 *     the architecture check (and fp8_linear_noalloc's scratch, see there).
 *     Calls on one stream are ordered; calls on different streams that
 *     write the same buffers race (caller's duty).
 *   - The dynamic quantizers (scales derived from the data) assume finite
 *     bf16 inputs: a NaN or infinity in a group makes its scale non-finite.
 *     The static-scale calls (fp8_quant_act_static, fp8_kv_cache_write)
 *     define NaN and infinity per element.
 *
 * Page references: "[vLLM] FP8" = blog.secrett2633.cloud/opensource/vllm/fp8;
 * "FP8 Quantization" = zzong2006.github.io fp8-quantization;
 * "FP8 and FP4: Throughput Needs Scaling" = llm-engineer.pages.dev card.
 */
#ifndef FP8W8A8_H
#define FP8W8A8_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  FP8_OK = 0,
  FP8_ERR_NULL = 1,       /* a required pointer is NULL */
  FP8_ERR_SHAPE = 2,      /* K or N not a positive multiple of 128, M < 0, a KV-cache
                             shape out of range, or too large */
  FP8_ERR_STRIDE = 3,     /* a leading dimension is smaller than the row length, or
                             rows x leading dimension exceeds 2^56 elements */
  FP8_ERR_ALIGN = 4,      /* pointer or leading-dimension alignment */
  FP8_ERR_BLOCK = 5,      /* weight block size other than 128 x 128 */
  FP8_ERR_SCHEME = 6,     /* unsupported scale mode / scheme combination */
  FP8_ERR_WORKSPACE = 7,  /* workspace missing or smaller than fp8_workspace_bytes() */
  FP8_ERR_DEVICE = 8,     /* current device is not gfx950, or no device */
  FP8_ERR_LAUNCH = 9,     /* the kernel launch failed */
  FP8_ERR_ALIAS = 10,     /* an output overlaps an input or another output */
  FP8_ERR_SCRATCH = 11    /* fp8_linear_noalloc: the call needs more than its scratch */
} fp8_status;

/* Scale modes.
 * FP8_SCALE_BLOCK : activations 1x128 per row, weights 128x128 blocks
 *                   (the dynamic 128-group and static 128-block schemes of
 *                   "[vLLM] FP8", scaling strategies).
 * FP8_SCALE_TENSOR: one scale for the whole tensor, computed dynamically from
 *                   the tensor's amax (the dynamic per-tensor scheme).
 * FP8_SCALE_ROW   : one scale per row -- per token for activations (the
 *                   dynamic per-token scheme), per output channel for
 *                   weights (channel-wise weight scales, "FP8 Quantization",
 *                   the pre-quantized checkpoint path).  In the GEMM each
 *                   scale vector may also be a single value (stride 0), so a
 *                   static or dynamic per-tensor activation scale combines
 *                   with per-channel weights, and per-token activations with
 *                   a per-tensor weight. */
enum { FP8_SCALE_BLOCK = 0, FP8_SCALE_TENSOR = 1, FP8_SCALE_ROW = 2 };

/* Operation ids for fp8_workspace_bytes(). */
enum { FP8_OP_QUANT_ACT = 0, FP8_OP_QUANT_WEIGHT = 1, FP8_OP_GEMM = 2, FP8_OP_LINEAR = 3 };

/* Human-readable text of a status code (static storage, never NULL). */
const char* fp8_status_str(fp8_status s);

/* Bytes of device workspace a call needs (0 if none).  For op
 * FP8_OP_QUANT_ACT the shape is (M, K); for FP8_OP_QUANT_WEIGHT it is (N, K)
 * passed as (rows = M argument, K); FP8_OP_LINEAR takes (M, N, K) and needs
 * none on its fused path.  FP8_OP_GEMM takes (M, N, K): the bytes with which
 * fp8_block_gemm splits K in two on the current device (nonzero only for
 * shapes with M > 64 whose 128 x 256 output tiles would occupy at most half
 * of the device's compute units and whose K is a multiple of 1024, in every
 * scale mode); the call works without them. */
size_t fp8_workspace_bytes(int op, int64_t M, int64_t N, int64_t K, int scale_mode);

/* fp8_quant_act -- dynamic activation quantization.
 * Follows "FP8 Quantization" sections C and D.2 (activation scales computed
 * at run time per call) and "[vLLM] FP8", block quantization (the block path
 * takes only a dynamic activation scheme) and scaling strategies (dynamic
 * 128-group, dynamic per-tensor, dynamic per-token).
 *   x      [M, K] bf16, ld_x elements per row                      (input)
 *   q      [M, K] E4M3 codes, ld_q bytes per row                    (output)
 *   scales FP8_SCALE_BLOCK : [M, K/128] fp32, ld_s >= K/128         (output)
 *          FP8_SCALE_TENSOR: scales[0], one fp32                    (output)
 *          FP8_SCALE_ROW   : scales[m * ld_s], M fp32, ld_s >= 1    (output)
 *   For each group G (1x128 slice of a row, a whole row, or the tensor):
 *     amax = max |x|, s = fp32(amax) / 448 (IEEE round to nearest),
 *     code = E4M3_RNE_saturating(fp32(x) / s), the quotient correctly
 *     rounded; an all-zero group gets s = 0 and codes +-0 by x's sign.
 *   workspace: FP8_SCALE_TENSOR needs fp8_workspace_bytes(FP8_OP_QUANT_ACT,
 *     M, 0, K, FP8_SCALE_TENSOR) bytes of device memory (4-byte aligned,
 *     contents need not be initialized); the other modes need none. */
fp8_status fp8_quant_act(const uint16_t* x, int64_t M, int64_t K, int64_t ld_x,
                         uint8_t* q, int64_t ld_q, float* scales, int64_t ld_s,
                         int scale_mode, void* workspace, size_t ws_bytes, void* stream);

/* fp8_quant_weight_block -- weight quantization, done once, offline.
 * Follows "[vLLM] FP8", block quantization (two-dimensional 128x128 blocks,
 * one scale each; block mode needs a pre-quantized checkpoint, which this
 * call produces) and "why this design" item 2 (an outlier stays inside its
 * block); "FP8 Quantization" D.1 (block size 128).
 *   w      [N, K] bf16, ld_w elements per row                      (input)
 *   q      [N, K] E4M3 codes, ld_q bytes per row                    (output)
 *   scales FP8_SCALE_BLOCK : [N/128, K/128] fp32, ld_s >= K/128     (output)
 *          FP8_SCALE_TENSOR: scales[0]                               (output)
 *          FP8_SCALE_ROW   : scales[n * ld_s], one per output channel (output)
 *   block_n, block_k: must both be 128 in FP8_SCALE_BLOCK mode (the block
 *   size has two dimensions; other sizes give FP8_ERR_BLOCK); ignored in the
 *   other modes.
 *   Same per-group rule as fp8_quant_act with G = one 128x128 block, one
 *   weight row, or the tensor.  workspace as for fp8_quant_act with M = N. */
fp8_status fp8_quant_weight_block(const uint16_t* w, int64_t N, int64_t K, int64_t ld_w,
                                  uint8_t* q, int64_t ld_q, float* scales, int64_t ld_s,
                                  int block_n, int block_k, int scale_mode,
                                  void* workspace, size_t ws_bytes, void* stream);

/* fp8_block_gemm -- out = A . W^T on FP8 operands.
 * Follows "FP8 and FP4: Throughput Needs Scaling", kernel-caveat card (FP8
 * operands straight into the matrix unit, wide accumulation) and "[vLLM]
 * FP8", block quantization (128x128 weight blocks) with the dynamic
 * 128-group activation scheme.
 *   a_q [M, K] codes (ld_a), a_s scales (ld_as), w_q [N, K] codes (ld_w),
 *   w_s scales (ld_ws), out [M, N] bf16 (ld_out).
 *   FP8_SCALE_BLOCK : a_s [M, K/128], w_s [N/128, K/128] and
 *     out[m,n] = bf16_RNE( sum_kb a_s[m,kb] * w_s[n/128,kb] *
 *                          sum_{k in kb} dec(a_q[m,k]) * dec(w_q[n,k]) )
 *     accumulated in fp32.
 *   FP8_SCALE_TENSOR: a_s[0], w_s[0]; out = bf16(a_s * w_s * sum_k ...).
 *   FP8_SCALE_ROW   : a_s[m * ld_as] (per token), w_s[n * ld_ws] (per output
 *     channel), ld_as, ld_ws >= 0 (0: one value for all rows / columns);
 *     out[m,n] = bf16_RNE( (a_s[m] * w_s[n]) * sum_k dec(a_q) * dec(w_q) ),
 *     the scale product in fp32, the sum accumulated in fp32.
 *   Mixing a per-tensor activation scale with block weights (or the reverse)
 *   is not a mode (FP8_ERR_SCHEME).
 *   workspace (optional, may be NULL): with at least
 *   fp8_workspace_bytes(FP8_OP_GEMM, M, N, K, scale_mode) bytes (16-byte
 *   aligned, apart from every tensor of the call, contents not needed and
 *   not read afterwards) a shape for which that is nonzero runs as two
 *   workgroups per output tile, each over half of the K blocks, and adds the
 *   two fp32 partial sums before rounding to bf16 -- the same arithmetic
 *   with the K-block sum split in two, so the result can differ from the
 *   unsplit call's in the last bits.  A smaller or NULL workspace runs the
 *   call unsplit.  The result of a given call does not depend on timing. */
fp8_status fp8_block_gemm(const uint8_t* a_q, int64_t ld_a, const float* a_s, int64_t ld_as,
                          const uint8_t* w_q, int64_t ld_w, const float* w_s, int64_t ld_ws,
                          uint16_t* out, int64_t ld_out, int64_t M, int64_t N, int64_t K,
                          int scale_mode, void* workspace, size_t ws_bytes, void* stream);

/* fp8_linear -- one W8A8 linear call: dynamic activation quantization of x
 * followed by the FP8 GEMM against pre-quantized weights.  The pages describe
 * the two as one runtime step: activation scales computed per call ("FP8
 * Quantization" §D.2, and "fp8-serving-slower-than-bf16" on per-step scale
 * overhead) feeding the FP8 matrix unit ("FP8 and FP4: Throughput Needs
 * Scaling", kernel-caveat card).
 *   x [M, K] bf16 (ld_x), w_q / w_s as for fp8_block_gemm, out [M, N] bf16.
 *   The result is bit-identical to fp8_quant_act (same scale_mode) followed
 *   by fp8_block_gemm.
 *   FP8_SCALE_ROW quantizes x per token (dynamic) and takes per-channel
 *   (or, with ld_ws = 0, per-tensor) weight scales w_s[n * ld_ws].
 *   FP8_SCALE_BLOCK with K <= 16384 and either 1 <= M <= 4, or M <= 16
 *   with M * K <= 16384 and (N / 16) * M * K <= 2^21, runs as one fused
 *   launch (quantization inside the decode GEMM) and needs no workspace
 *   (fp8_workspace_bytes(FP8_OP_LINEAR, ...) is 0 exactly for these).
 *   Any other call quantizes into the workspace and then multiplies; it
 *   needs fp8_workspace_bytes(FP8_OP_LINEAR, M, N, K, scale_mode) bytes of
 *   device memory (16-byte aligned, not initialized, not read afterwards),
 *   which include the GEMM's split-K bytes (fp8_block_gemm) when the shape
 *   splits: the result equals fp8_quant_act followed by fp8_block_gemm
 *   given that workspace. */
fp8_status fp8_linear(const uint16_t* x, int64_t ld_x, const uint8_t* w_q, int64_t ld_w,
                      const float* w_s, int64_t ld_ws, uint16_t* out, int64_t ld_out,
                      int64_t M, int64_t N, int64_t K, int scale_mode, void* workspace,
                      size_t ws_bytes, void* stream);

/* fp8_linear_noalloc -- fp8_linear for callers that cannot allocate device
 * memory: code under HIP graph capture, tight serving loops, harnesses that
 * forbid hipMalloc.  Same arguments, arithmetic and result as fp8_linear,
 * bit for bit, without the workspace: the unfused path (every call but the
 * fused ones above) keeps its activation codes, scales and
 * per-tensor partials in a scratch buffer of FP8_NOALLOC_SCRATCH_BYTES that
 * the library holds on every device it runs on, from the first call on that
 * device until the process ends (a static device array; its address is
 * looked up once per device, nothing is allocated).  A call whose workspace
 * (fp8_workspace_bytes(FP8_OP_LINEAR, M, N, K, scale_mode)) exceeds it
 * returns FP8_ERR_SCRATCH before anything is enqueued.
 *   Every call on one device shares that device's buffer, which keeps the
 *   last call's contents: calls that can overlap on one device (different
 *   streams, or threads without ordering) race and are the caller's to
 *   order.  No byte of it needs to start at any value (each call writes
 *   everything it reads). */
#define FP8_NOALLOC_SCRATCH_BYTES (64u << 20)
fp8_status fp8_linear_noalloc(const uint16_t* x, int64_t ld_x, const uint8_t* w_q, int64_t ld_w,
                              const float* w_s, int64_t ld_ws, uint16_t* out, int64_t ld_out,
                              int64_t M, int64_t N, int64_t K, int scale_mode, void* stream);

/* fp8_quant_act_static -- static activation quantization with a scale
 * calibrated beforehand ("[vLLM] FP8", scaling strategies: static
 * per-tensor; static scales come from calibration data, dynamic ones are
 * computed at run time).
 *   x      [M, K] bf16, ld_x elements per row                      (input)
 *   q      [M, K] E4M3 codes, ld_q bytes per row                    (output)
 *   scale  one fp32 in device memory, read by the kernel            (input)
 *   code = E4M3_RNE_saturating(fp32(x) / scale), the quotient an IEEE fp32
 *   division (a zero scale gives x / 0: saturated codes, NaN for 0 / 0).
 *   The codes pair with a_s = scale in fp8_block_gemm (FP8_SCALE_TENSOR, or
 *   FP8_SCALE_ROW with ld_as = 0 against per-channel weights).  No workspace. */
fp8_status fp8_quant_act_static(const uint16_t* x, int64_t M, int64_t K, int64_t ld_x,
                                uint8_t* q, int64_t ld_q, const float* scale, void* stream);

/* fp8_grouped_gemm -- block-scaled FP8 grouped GEMM for a mixture-of-experts
 * layer: each expert's rows of A against that expert's FP8 weight.  A fused
 * MoE layer gets its own FP8 method, with expert weights quantized offline
 * or at load ("[vLLM] FP8", the config's dispatch and its table of methods);
 * the experts are small matrices ("Quantization guide for serving: FP8,
 * AWQ, GPTQ", closing section).
 *   a_q, a_s       [M, K] codes (ld_a) and [M, K/128] scales (ld_as) of the
 *                  activations, rows grouped by expert (as fp8_quant_act
 *                  makes them, block mode)                             (input)
 *   w_q, w_s       E experts stacked: codes [E, N, K] (row stride ld_w,
 *                  expert e at w_q + e * N * ld_w) and 128 x 128 block scales
 *                  [E, N/128, K/128] (row stride ld_ws, expert e at
 *                  w_s + e * (N/128) * ld_ws)                          (input)
 *   expert_offsets [E + 1] int64 in device memory: expert e owns rows
 *                  expert_offsets[e] .. expert_offsets[e + 1] - 1      (input)
 *   out            [M, N] bf16 (ld_out)                                (output)
 *   out[r, n] = bf16_RNE( sum_kb a_s[r, kb] * w_s[e][n/128, kb] *
 *                         sum_{k in kb} dec(a_q[r, k]) * dec(w_q[e][n, k]) )
 *   for every row r of expert e, the same arithmetic as fp8_block_gemm.
 *   The offsets should be nondecreasing with expert_offsets[0] >= 0 and
 *   expert_offsets[E] <= M; the device clamps each range to [0, M], so other
 *   offsets give unspecified rows but no access outside the tensors.  Rows
 *   in no expert's range are not written.  1 <= E <= 65535, K <= 16384;
 *   alignment as for fp8_block_gemm.  E == 0 or M == 0 does nothing.  No
 *   workspace; the routing that groups the rows is the caller's. */
fp8_status fp8_grouped_gemm(const uint8_t* a_q, int64_t ld_a, const float* a_s, int64_t ld_as,
                            const uint8_t* w_q, int64_t ld_w, const float* w_s, int64_t ld_ws,
                            const int64_t* expert_offsets, int64_t E, uint16_t* out,
                            int64_t ld_out, int64_t M, int64_t N, int64_t K, void* stream);

/* fp8_kv_cache_write -- quantize one step's keys and values into a paged
 * FP8 KV cache.  With an fp8 KV-cache dtype keys and values are stored as
 * E4M3, halving the cache, each with its own scale: 1.0 by default (large
 * values clip) or calibrated ("FP8 Quantization", D.4; "[vLLM] FP8", KV
 * cache quantization; "Quantization guide for serving: FP8, AWQ, GPTQ",
 * KV-cache FP8 section).
 *   key, value    [T, H, D] bf16; the H * D values of a token are
 *                 contiguous, tokens ld_key / ld_value elements apart  (input)
 *   slot_mapping  [T] int64: the cache slot of each token,
 *                 slot = block * block_size + offset                   (input)
 *   key_cache, value_cache  [num_blocks, block_size, H, D] E4M3 codes,
 *                 contiguous; only the slots named are written    (in/out)
 *   k_scale, v_scale  one fp32 each in device memory                   (input)
 *   cache[slot(t)][h][d] = E4M3_RNE_saturating(fp32(x[t][h][d]) / scale),
 *   the quotient an IEEE fp32 division (as fp8_quant_act_static).  A token
 *   whose slot is negative (padding) or >= num_blocks * block_size is not
 *   stored; two tokens with one slot leave either token's codes.
 *   H * D a multiple of 8; key, value and the caches 16-byte aligned, ld_key
 *   and ld_value multiples of 8.  The caches may be NULL when
 *   num_blocks == 0.  T == 0 does nothing.  No workspace. */
fp8_status fp8_kv_cache_write(const uint16_t* key, int64_t ld_key, const uint16_t* value,
                              int64_t ld_value, const int64_t* slot_mapping, int64_t T,
                              int64_t H, int64_t D, uint8_t* key_cache, uint8_t* value_cache,
                              int64_t num_blocks, int64_t block_size, const float* k_scale,
                              const float* v_scale, void* stream);

/* fp8_kv_cache_read -- gather tokens from a paged FP8 cache (either one)
 * and restore them to bf16, as an attention backend without FP8 support
 * does before it reads the cache ("Quantization guide for serving: FP8,
 * AWQ, GPTQ", KV-cache FP8 section).
 *   cache   [num_blocks, block_size, H, D] E4M3 codes, contiguous       (input)
 *   slots   [T] int64 cache slots                                       (input)
 *   scale   one fp32 in device memory: the scale the codes were written
 *           with                                                        (input)
 *   out     [T, H, D] bf16, tokens ld_out elements apart               (output)
 *   out[t][h][d] = bf16_RNE(fp32(decode(code)) * scale), one fp32 multiply
 *   and one rounding; a NaN result is the quiet bf16 NaN with the code's
 *   sign.  A token whose slot is out of range reads zeros.  Alignment as for
 *   fp8_kv_cache_write; no workspace. */
fp8_status fp8_kv_cache_read(const uint8_t* cache, int64_t num_blocks, int64_t block_size,
                             int64_t H, int64_t D, const int64_t* slots, int64_t T,
                             const float* scale, uint16_t* out, int64_t ld_out, void* stream);

/* Host-only validation: the argument checks of the calls above, in the
 * same order, without touching any device (no device check, no launch). */
fp8_status fp8_validate_quant_act(const uint16_t* x, int64_t M, int64_t K, int64_t ld_x,
                                  const uint8_t* q, int64_t ld_q, const float* scales,
                                  int64_t ld_s, int scale_mode, const void* workspace,
                                  size_t ws_bytes);
fp8_status fp8_validate_quant_weight_block(const uint16_t* w, int64_t N, int64_t K,
                                           int64_t ld_w, const uint8_t* q, int64_t ld_q,
                                           const float* scales, int64_t ld_s, int block_n,
                                           int block_k, int scale_mode,
                                           const void* workspace, size_t ws_bytes);
fp8_status fp8_validate_block_gemm(const uint8_t* a_q, int64_t ld_a, const float* a_s,
                                   int64_t ld_as, const uint8_t* w_q, int64_t ld_w,
                                   const float* w_s, int64_t ld_ws, const uint16_t* out,
                                   int64_t ld_out, int64_t M, int64_t N, int64_t K,
                                   int scale_mode);
fp8_status fp8_validate_quant_act_static(const uint16_t* x, int64_t M, int64_t K, int64_t ld_x,
                                         const uint8_t* q, int64_t ld_q, const float* scale);
fp8_status fp8_validate_grouped_gemm(const uint8_t* a_q, int64_t ld_a, const float* a_s,
                                     int64_t ld_as, const uint8_t* w_q, int64_t ld_w,
                                     const float* w_s, int64_t ld_ws,
                                     const int64_t* expert_offsets, int64_t E, const uint16_t* out,
                                     int64_t ld_out, int64_t M, int64_t N, int64_t K);
fp8_status fp8_validate_kv_cache_write(const uint16_t* key, int64_t ld_key,
                                       const uint16_t* value, int64_t ld_value,
                                       const int64_t* slot_mapping, int64_t T, int64_t H,
                                       int64_t D, const uint8_t* key_cache,
                                       const uint8_t* value_cache, int64_t num_blocks,
                                       int64_t block_size, const float* k_scale,
                                       const float* v_scale);
fp8_status fp8_validate_kv_cache_read(const uint8_t* cache, int64_t num_blocks,
                                      int64_t block_size, int64_t H, int64_t D,
                                      const int64_t* slots, int64_t T, const float* scale,
                                      const uint16_t* out, int64_t ld_out);

/* fp8_e4m3_encode_f32 -- the device element encoder on its own.
 * codes[i] = E4M3 of x[i]: round to nearest even, magnitudes above 448 and
 * infinities saturate to 448, NaN gives the NaN code with x's sign, the sign
 * of zero is kept.  Format as in "[vLLM] FP8" format table.  Exposed so the
 * device conversion can be checked value by value.  x: n fp32 (4-byte
 * aligned), codes: n bytes; n >= 0. */
fp8_status fp8_e4m3_encode_f32(const float* x, int64_t n, uint8_t* codes, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* FP8W8A8_H */
