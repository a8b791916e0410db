// C ABI of the FP8 W8A8 library: argument validation, device check, and
// dispatch to the launchers.  Validation mirrors the eager configuration
// checks of "[vLLM] FP8", block quantization (block mode needs pre-quantized
// weights, a two-dimensional block size, and a dynamic activation scheme),
// turned into status codes returned before anything is enqueued.
#include <atomic>
#include <cstring>

#include "fp8w8a8.h"
#include "launch.h"

namespace {

constexpr int64_t kMaxDim = (int64_t)1 << 31;        // any single extent
constexpr int64_t kMaxElems = (int64_t)1 << 40;      // rows * cols of one tensor
constexpr int64_t kMaxSpan = (int64_t)1 << 56;       // rows * ld of one tensor (elements)

// rows rows at leading dimension ld span at most kMaxSpan elements, so every
// byte range below is computed without overflow
bool span_ok(int64_t rows, int64_t ld) {
  return ld >= 0 && ld <= kMaxSpan && (rows <= 1 || ld <= kMaxSpan / rows);
}

bool aligned(const void* p, uintptr_t a) { return ((uintptr_t)p & (a - 1)) == 0; }

// Byte range [lo, hi) of a row-major matrix.
struct Range {
  uintptr_t lo, hi;
};
Range range_of(const void* p, int64_t rows, int64_t cols, int64_t ld, int64_t elem) {
  uintptr_t lo = (uintptr_t)p;
  if (rows <= 0 || cols <= 0) return {lo, lo};
  uintptr_t hi = lo + (uintptr_t)(((rows - 1) * ld + cols) * elem);
  return {lo, hi};
}
bool overlap(Range a, Range b) { return a.lo < b.hi && b.lo < a.hi; }

bool shape_ok_kn(int64_t K) { return K > 0 && K % 128 == 0 && K < kMaxDim; }

bool mode_ok(int scale_mode) {
  return scale_mode == FP8_SCALE_BLOCK || scale_mode == FP8_SCALE_TENSOR ||
         scale_mode == FP8_SCALE_ROW;
}

// Work-items of the quantizer's grid for R rows of K (per-tensor mode
// strides over the data with a bounded grid).
uint64_t quant_items(int64_t R, int64_t K, int scale_mode, bool rows_blocked) {
  if (R <= 0) return 0;
  if (scale_mode == FP8_SCALE_BLOCK)
    return rows_blocked ? fp8k::quant_weight_block_items(R, K) : fp8k::quant_act_block_items(R, K);
  if (scale_mode == FP8_SCALE_ROW) return fp8k::quant_rows_items(R);
  return 0;
}

fp8_status validate_quant(const uint16_t* x, int64_t R, int64_t K, int64_t ld_x,
                          const uint8_t* q, int64_t ld_q, const float* scales, int64_t ld_s,
                          int scale_mode, const void* ws, size_t ws_bytes, bool rows_blocked) {
  if (!mode_ok(scale_mode)) return FP8_ERR_SCHEME;
  if (R < 0 || R >= kMaxDim || !shape_ok_kn(K)) return FP8_ERR_SHAPE;
  if (rows_blocked && scale_mode == FP8_SCALE_BLOCK && R % 128 != 0) return FP8_ERR_SHAPE;
  if (R > 0 && R * K > kMaxElems) return FP8_ERR_SHAPE;
  if (quant_items(R, K, scale_mode, rows_blocked) >= fp8k::kMaxGridItems) return FP8_ERR_SHAPE;
  if (R == 0) return FP8_OK;
  if (!x || !q || !scales) return FP8_ERR_NULL;
  const int64_t groups = K / 128;
  if (ld_x < K || ld_q < K) return FP8_ERR_STRIDE;
  if (scale_mode == FP8_SCALE_BLOCK && ld_s < groups) return FP8_ERR_STRIDE;
  if (scale_mode == FP8_SCALE_ROW && ld_s < 1) return FP8_ERR_STRIDE;
  const int64_t srows = scale_mode == FP8_SCALE_BLOCK ? (rows_blocked ? R / 128 : R)
                        : scale_mode == FP8_SCALE_ROW ? R : 1;
  if (!span_ok(R, ld_x) || !span_ok(R, ld_q) ||
      (scale_mode != FP8_SCALE_TENSOR && !span_ok(srows, ld_s)))
    return FP8_ERR_STRIDE;
  if (!aligned(x, 16) || !aligned(q, 16) || !aligned(scales, 4)) return FP8_ERR_ALIGN;
  if (ld_x % 8 != 0 || ld_q % 16 != 0) return FP8_ERR_ALIGN;
  const int64_t scols = scale_mode == FP8_SCALE_BLOCK ? groups : 1;
  const int64_t sld = scale_mode == FP8_SCALE_TENSOR ? 1 : ld_s;
  Range rx = range_of(x, R, K, ld_x, 2), rq = range_of(q, R, K, ld_q, 1);
  Range rs = range_of(scales, srows, scols, sld, 4);
  if (overlap(rx, rq) || overlap(rx, rs) || overlap(rq, rs)) return FP8_ERR_ALIAS;
  if (scale_mode == FP8_SCALE_TENSOR) {
    const size_t need = (size_t)fp8k::kTensorPartials * sizeof(uint32_t);
    if (!ws || ws_bytes < need || !aligned(ws, 4)) return FP8_ERR_WORKSPACE;
    Range rw = {(uintptr_t)ws, (uintptr_t)ws + need};
    if (overlap(rw, rx) || overlap(rw, rq) || overlap(rw, rs)) return FP8_ERR_ALIAS;
  }
  return FP8_OK;
}

// Scale vectors of the row mode: n entries at stride ld (ld = 0: one entry).
Range row_scales(const float* p, int64_t n, int64_t ld) {
  return ld == 0 ? range_of(p, 1, 1, 1, 4) : range_of(p, n, 1, ld, 4);
}

fp8_status validate_gemm(const uint8_t* a_q, int64_t ld_a, const float* a_s, int64_t ld_as,
                         const uint8_t* w_q, int64_t ld_w, const float* w_s, int64_t ld_ws,
                         const uint16_t* out, int64_t ld_out, int64_t M, int64_t N, int64_t K,
                         int scale_mode) {
  if (!mode_ok(scale_mode)) return FP8_ERR_SCHEME;
  if (M < 0 || M >= kMaxDim || !shape_ok_kn(K) || !shape_ok_kn(N)) return FP8_ERR_SHAPE;
  if (M * K > kMaxElems || N * K > kMaxElems || M * N > kMaxElems) return FP8_ERR_SHAPE;
  if (M > 0 && fp8k::gemm_items(M, N, K) >= fp8k::kMaxGridItems) return FP8_ERR_SHAPE;
  if (M == 0) return FP8_OK;
  if (!a_q || !a_s || !w_q || !w_s || !out) return FP8_ERR_NULL;
  const int64_t KB = K / 128;
  if (ld_a < K || ld_w < K || ld_out < N) return FP8_ERR_STRIDE;
  if (scale_mode == FP8_SCALE_BLOCK && (ld_as < KB || ld_ws < KB)) return FP8_ERR_STRIDE;
  if (scale_mode == FP8_SCALE_ROW && (ld_as < 0 || ld_ws < 0 || ld_as >= kMaxDim ||
                                      ld_ws >= kMaxDim))
    return FP8_ERR_STRIDE;
  if (!span_ok(M, ld_a) || !span_ok(N, ld_w) || !span_ok(M, ld_out)) return FP8_ERR_STRIDE;
  if (scale_mode == FP8_SCALE_BLOCK && (!span_ok(M, ld_as) || !span_ok(N / 128, ld_ws)))
    return FP8_ERR_STRIDE;
  if (scale_mode == FP8_SCALE_ROW && (!span_ok(M, ld_as) || !span_ok(N, ld_ws)))
    return FP8_ERR_STRIDE;
  if (!aligned(a_q, 16) || !aligned(w_q, 16) || !aligned(out, 16)) return FP8_ERR_ALIGN;
  if (!aligned(a_s, 4) || !aligned(w_s, 4)) return FP8_ERR_ALIGN;
  if (ld_a % 16 != 0 || ld_w % 16 != 0 || ld_out % 8 != 0) return FP8_ERR_ALIGN;
  Range ro = range_of(out, M, N, ld_out, 2);
  Range ra = range_of(a_q, M, K, ld_a, 1), rw = range_of(w_q, N, K, ld_w, 1);
  Range ras = scale_mode == FP8_SCALE_BLOCK ? range_of(a_s, M, KB, ld_as, 4)
              : scale_mode == FP8_SCALE_ROW ? row_scales(a_s, M, ld_as)
                                            : range_of(a_s, 1, 1, 1, 4);
  Range rws = scale_mode == FP8_SCALE_BLOCK ? range_of(w_s, N / 128, KB, ld_ws, 4)
              : scale_mode == FP8_SCALE_ROW ? row_scales(w_s, N, ld_ws)
                                            : range_of(w_s, 1, 1, 1, 4);
  if (overlap(ro, ra) || overlap(ro, rw) || overlap(ro, ras) || overlap(ro, rws)) return FP8_ERR_ALIAS;
  return FP8_OK;
}

// Per-device cache of "is this a gfx950": 0 unknown, 1 yes, 2 no.
constexpr int kMaxDevices = 64;
std::atomic<int> g_arch_ok[kMaxDevices];

fp8_status check_device() {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return FP8_ERR_DEVICE;
  int state = g_arch_ok[dev].load(std::memory_order_relaxed);
  if (state == 0) {
    hipDeviceProp_t prop;
    if (hipGetDeviceProperties(&prop, dev) != hipSuccess) return FP8_ERR_DEVICE;
    state = std::strncmp(prop.gcnArchName, "gfx950", 6) == 0 ? 1 : 2;
    g_arch_ok[dev].store(state, std::memory_order_relaxed);
  }
  return state == 1 ? FP8_OK : FP8_ERR_DEVICE;
}

fp8_status launched(hipError_t e) { return e == hipSuccess ? FP8_OK : FP8_ERR_LAUNCH; }

// Workspace of the unfused fp8_linear path: activation codes [M, ld = K
// rounded up to 16], then the scales (block: [M, K/128]; row: [M]; tensor:
// one float), then the per-tensor partials.  Every piece starts 256-byte
// aligned.
struct LinearLayout {
  size_t codes, scales, partials, gemm, gemm_bytes, total;
  int64_t ld_q;
};
size_t align256(size_t v) { return (v + 255) & ~(size_t)255; }
LinearLayout linear_layout(int64_t M, int64_t N, int64_t K, int scale_mode) {
  LinearLayout l;
  l.ld_q = (K + 15) / 16 * 16;
  l.codes = 0;
  l.scales = align256((size_t)M * (size_t)l.ld_q);
  const size_t nscales = scale_mode == FP8_SCALE_BLOCK ? (size_t)M * (size_t)(K / 128)
                         : scale_mode == FP8_SCALE_ROW  ? (size_t)M
                                                        : 1;
  l.partials = align256(l.scales + nscales * sizeof(float));
  l.gemm = scale_mode == FP8_SCALE_TENSOR
               ? align256(l.partials + (size_t)fp8k::kTensorPartials * sizeof(uint32_t))
               : l.partials;
  // the GEMM's split-K workspace, when the shape splits
  l.gemm_bytes = fp8k::gemm_split_bytes(M, N, K);
  l.total = l.gemm + l.gemm_bytes;
  return l;
}

// Work-items of the largest grid fp8_linear launches: the fused decode
// kernel, or the quantizer and then the GEMM.
uint64_t linear_items(int64_t M, int64_t N, int64_t K, int scale_mode) {
  if (scale_mode == FP8_SCALE_BLOCK && fp8k::linear_decode_supported(M, N, K))
    return fp8k::linear_decode_items(N);
  const uint64_t q = quant_items(M, K, scale_mode, false), g = fp8k::gemm_items(M, N, K);
  return q > g ? q : g;
}

}  // namespace

extern "C" {

const char* fp8_status_str(fp8_status s) {
  switch (s) {
    case FP8_OK: return "ok";
    case FP8_ERR_NULL: return "a required pointer is NULL";
    case FP8_ERR_SHAPE: return "bad shape: K and N must be positive multiples of 128, M >= 0";
    case FP8_ERR_STRIDE: return "leading dimension smaller than the row length, or too large";
    case FP8_ERR_ALIGN: return "misaligned pointer or leading dimension";
    case FP8_ERR_BLOCK: return "the weight block size must have two dimensions, 128 x 128";
    case FP8_ERR_SCHEME: return "unsupported scale mode: block mode supports only dynamic activation scales";
    case FP8_ERR_WORKSPACE: return "workspace missing or too small";
    case FP8_ERR_DEVICE: return "no gfx950 device is current";
    case FP8_ERR_LAUNCH: return "kernel launch failed";
    case FP8_ERR_ALIAS: return "an output overlaps another tensor";
    case FP8_ERR_SCRATCH:
      return "the call needs more scratch than the allocation-free entry point holds "
             "(FP8_NOALLOC_SCRATCH_BYTES)";
  }
  return "unknown status";
}

size_t fp8_workspace_bytes(int op, int64_t M, int64_t N, int64_t K, int scale_mode) {
  if (op == FP8_OP_GEMM) {
    if (!mode_ok(scale_mode) || M <= 0 || M >= kMaxDim || !shape_ok_kn(K) || !shape_ok_kn(N))
      return 0;
    return fp8k::gemm_split_bytes(M, N, K);
  }
  if ((op == FP8_OP_QUANT_ACT || op == FP8_OP_QUANT_WEIGHT) && scale_mode == FP8_SCALE_TENSOR)
    return (size_t)fp8k::kTensorPartials * sizeof(uint32_t);
  if (op == FP8_OP_LINEAR) {
    if (scale_mode == FP8_SCALE_BLOCK && fp8k::linear_decode_supported(M, N, K)) return 0;
    if (M <= 0 || K <= 0) return 0;
    return linear_layout(M, N, K, scale_mode).total;
  }
  return 0;
}

fp8_status fp8_validate_quant_act(const uint16_t* x, int64_t M, int64_t K, int64_t ld_x,
                                  const uint8_t* q, int64_t ld_q, const float* scales,
                                  int64_t ld_s, int scale_mode, const void* workspace,
                                  size_t ws_bytes) {
  return validate_quant(x, M, K, ld_x, q, ld_q, scales, ld_s, scale_mode, workspace, ws_bytes,
                        false);
}

fp8_status fp8_validate_quant_weight_block(const uint16_t* w, int64_t N, int64_t K,
                                           int64_t ld_w, const uint8_t* q, int64_t ld_q,
                                           const float* scales, int64_t ld_s, int block_n,
                                           int block_k, int scale_mode,
                                           const void* workspace, size_t ws_bytes) {
  if (scale_mode == FP8_SCALE_BLOCK && (block_n != 128 || block_k != 128)) return FP8_ERR_BLOCK;
  return validate_quant(w, N, K, ld_w, q, ld_q, scales, ld_s, scale_mode, workspace, ws_bytes,
                        true);
}

fp8_status fp8_validate_block_gemm(const uint8_t* a_q, int64_t ld_a, const float* a_s,
                                   int64_t ld_as, const uint8_t* w_q, int64_t ld_w,
                                   const float* w_s, int64_t ld_ws, const uint16_t* out,
                                   int64_t ld_out, int64_t M, int64_t N, int64_t K,
                                   int scale_mode) {
  return validate_gemm(a_q, ld_a, a_s, ld_as, w_q, ld_w, w_s, ld_ws, out, ld_out, M, N, K,
                       scale_mode);
}

fp8_status fp8_quant_act(const uint16_t* x, int64_t M, int64_t K, int64_t ld_x, uint8_t* q,
                         int64_t ld_q, float* scales, int64_t ld_s, int scale_mode,
                         void* workspace, size_t ws_bytes, void* stream) {
  fp8_status st = validate_quant(x, M, K, ld_x, q, ld_q, scales, ld_s, scale_mode, workspace,
                                 ws_bytes, false);
  if (st != FP8_OK || M == 0) return st;
  if ((st = check_device()) != FP8_OK) return st;
  hipStream_t s = (hipStream_t)stream;
  if (scale_mode == FP8_SCALE_BLOCK)
    return launched(fp8k::launch_quant_act_block(x, M, K, ld_x, q, ld_q, scales, ld_s, s));
  if (scale_mode == FP8_SCALE_ROW)
    return launched(fp8k::launch_quant_rows(x, M, K, ld_x, q, ld_q, scales, ld_s, s));
  return launched(fp8k::launch_quant_tensor(x, M, K, ld_x, q, ld_q, scales,
                                            (uint32_t*)workspace, s));
}

fp8_status fp8_quant_weight_block(const uint16_t* w, int64_t N, int64_t K, int64_t ld_w,
                                  uint8_t* q, int64_t ld_q, float* scales, int64_t ld_s,
                                  int block_n, int block_k, int scale_mode, void* workspace,
                                  size_t ws_bytes, void* stream) {
  fp8_status st = fp8_validate_quant_weight_block(w, N, K, ld_w, q, ld_q, scales, ld_s, block_n,
                                                  block_k, scale_mode, workspace, ws_bytes);
  if (st != FP8_OK || N == 0) return st;
  if ((st = check_device()) != FP8_OK) return st;
  hipStream_t s = (hipStream_t)stream;
  if (scale_mode == FP8_SCALE_BLOCK)
    return launched(fp8k::launch_quant_weight_block(w, N, K, ld_w, q, ld_q, scales, ld_s, s));
  if (scale_mode == FP8_SCALE_ROW)
    return launched(fp8k::launch_quant_rows(w, N, K, ld_w, q, ld_q, scales, ld_s, s));
  return launched(fp8k::launch_quant_tensor(w, N, K, ld_w, q, ld_q, scales,
                                            (uint32_t*)workspace, s));
}

fp8_status fp8_block_gemm(const uint8_t* a_q, int64_t ld_a, const float* a_s, int64_t ld_as,
                          const uint8_t* w_q, int64_t ld_w, const float* w_s, int64_t ld_ws,
                          uint16_t* out, int64_t ld_out, int64_t M, int64_t N, int64_t K,
                          int scale_mode, void* workspace, size_t ws_bytes, void* stream) {
  fp8_status st = validate_gemm(a_q, ld_a, a_s, ld_as, w_q, ld_w, w_s, ld_ws, out, ld_out, M, N,
                                K, scale_mode);
  if (st != FP8_OK || M == 0) return st;
  // the workspace is optional; one that is used must be aligned and apart
  // from every tensor of the call
  size_t need = 0;
  if (workspace && ws_bytes > 0 &&
      (need = fp8k::gemm_split_bytes(M, N, K)) > 0 &&
      ws_bytes >= need) {
    if (!aligned(workspace, 16)) return FP8_ERR_ALIGN;
    const int64_t KB = K / 128;
    Range r = {(uintptr_t)workspace, (uintptr_t)workspace + need};
    Range ras = scale_mode == FP8_SCALE_BLOCK ? range_of(a_s, M, KB, ld_as, 4)
                : scale_mode == FP8_SCALE_ROW ? row_scales(a_s, M, ld_as)
                                              : range_of(a_s, 1, 1, 1, 4);
    Range rws = scale_mode == FP8_SCALE_BLOCK ? range_of(w_s, N / 128, KB, ld_ws, 4)
                : scale_mode == FP8_SCALE_ROW ? row_scales(w_s, N, ld_ws)
                                              : range_of(w_s, 1, 1, 1, 4);
    if (overlap(r, range_of(out, M, N, ld_out, 2)) || overlap(r, range_of(a_q, M, K, ld_a, 1)) ||
        overlap(r, range_of(w_q, N, K, ld_w, 1)) || overlap(r, ras) || overlap(r, rws))
      return FP8_ERR_ALIAS;
  } else {
    workspace = nullptr;
    ws_bytes = 0;
  }
  if ((st = check_device()) != FP8_OK) return st;
  const bool kconst = scale_mode != FP8_SCALE_BLOCK;
  const bool tensor = scale_mode == FP8_SCALE_TENSOR;
  return launched(fp8k::launch_gemm(a_q, ld_a, a_s, tensor ? 0 : ld_as, w_q, ld_w, w_s,
                                    tensor ? 0 : ld_ws, out, ld_out, M, N, K, kconst, workspace,
                                    ws_bytes, (hipStream_t)stream));
}

}  // extern "C"

namespace {

// Argument checks of fp8_linear and fp8_linear_noalloc (everything but the
// workspace).  Sets fused (one launch, no workspace) and the workspace
// layout of the unfused path.
fp8_status validate_linear(const uint16_t* x, int64_t ld_x, const uint8_t* w_q, int64_t ld_w,
                           const float* w_s, int64_t ld_ws, const uint16_t* out, int64_t ld_out,
                           int64_t M, int64_t N, int64_t K, int scale_mode, bool& fused,
                           LinearLayout& lay) {
  if (!mode_ok(scale_mode)) return FP8_ERR_SCHEME;
  if (M < 0 || M >= kMaxDim || !shape_ok_kn(K) || !shape_ok_kn(N)) return FP8_ERR_SHAPE;
  if (M * K > kMaxElems || N * K > kMaxElems || M * N > kMaxElems) return FP8_ERR_SHAPE;
  if (M > 0 && linear_items(M, N, K, scale_mode) >= fp8k::kMaxGridItems) return FP8_ERR_SHAPE;
  if (M == 0) return FP8_OK;
  if (!x || !w_q || !w_s || !out) return FP8_ERR_NULL;
  const int64_t KB = K / 128;
  if (ld_x < K || ld_w < K || ld_out < N) return FP8_ERR_STRIDE;
  if (scale_mode == FP8_SCALE_BLOCK && ld_ws < KB) return FP8_ERR_STRIDE;
  if (scale_mode == FP8_SCALE_ROW && (ld_ws < 0 || ld_ws >= kMaxDim)) return FP8_ERR_STRIDE;
  if (!span_ok(M, ld_x) || !span_ok(N, ld_w) || !span_ok(M, ld_out)) return FP8_ERR_STRIDE;
  if (scale_mode == FP8_SCALE_BLOCK && !span_ok(N / 128, ld_ws)) return FP8_ERR_STRIDE;
  if (scale_mode == FP8_SCALE_ROW && !span_ok(N, ld_ws)) return FP8_ERR_STRIDE;
  if (!aligned(x, 16) || !aligned(w_q, 16) || !aligned(out, 16) || !aligned(w_s, 4))
    return FP8_ERR_ALIGN;
  if (ld_x % 8 != 0 || ld_w % 16 != 0 || ld_out % 8 != 0) return FP8_ERR_ALIGN;
  Range ro = range_of(out, M, N, ld_out, 2);
  Range rx = range_of(x, M, K, ld_x, 2), rw = range_of(w_q, N, K, ld_w, 1);
  Range rws = scale_mode == FP8_SCALE_BLOCK ? range_of(w_s, N / 128, KB, ld_ws, 4)
              : scale_mode == FP8_SCALE_ROW ? row_scales(w_s, N, ld_ws)
                                            : range_of(w_s, 1, 1, 1, 4);
  if (overlap(ro, rx) || overlap(ro, rw) || overlap(ro, rws)) return FP8_ERR_ALIAS;
  fused = scale_mode == FP8_SCALE_BLOCK && fp8k::linear_decode_supported(M, N, K);
  lay = linear_layout(M, N, K, scale_mode);
  return FP8_OK;
}

// The workspace of an unfused call must not overlap its tensors.
bool linear_workspace_clear(const uint16_t* x, int64_t ld_x, const uint8_t* w_q, int64_t ld_w,
                            const float* w_s, int64_t ld_ws, const uint16_t* out, int64_t ld_out,
                            int64_t M, int64_t N, int64_t K, int scale_mode, const void* ws,
                            size_t bytes) {
  const int64_t KB = K / 128;
  Range rws = scale_mode == FP8_SCALE_BLOCK ? range_of(w_s, N / 128, KB, ld_ws, 4)
              : scale_mode == FP8_SCALE_ROW ? row_scales(w_s, N, ld_ws)
                                            : range_of(w_s, 1, 1, 1, 4);
  Range r = {(uintptr_t)ws, (uintptr_t)ws + bytes};
  return !overlap(r, range_of(out, M, N, ld_out, 2)) && !overlap(r, range_of(x, M, K, ld_x, 2)) &&
         !overlap(r, range_of(w_q, N, K, ld_w, 1)) && !overlap(r, rws);
}

// Enqueue a validated linear call: the fused decode kernel, or the quantizer
// into the workspace (activation codes, scales, per-tensor partials) and the
// GEMM.
fp8_status run_linear(const uint16_t* x, int64_t ld_x, const uint8_t* w_q, int64_t ld_w,
                      const float* w_s, int64_t ld_ws, uint16_t* out, int64_t ld_out, int64_t M,
                      int64_t N, int64_t K, int scale_mode, bool fused, const LinearLayout& lay,
                      void* workspace, hipStream_t s) {
  if (fused)
    return launched(fp8k::launch_linear_decode(x, ld_x, w_q, ld_w, w_s, ld_ws, out, ld_out, M, N,
                                               K, s));
  const int64_t KB = K / 128;
  uint8_t* ws8 = (uint8_t*)workspace;
  uint8_t* q = ws8 + lay.codes;
  float* sa = (float*)(ws8 + lay.scales);
  hipError_t e;
  // block scales: the quantizer also clears the GEMM's split-K slot words
  const uint32_t nzero =
      scale_mode == FP8_SCALE_BLOCK && lay.gemm_bytes ? fp8k::gemm_split_words(M, N, K) : 0;
  if (scale_mode == FP8_SCALE_BLOCK)
    e = fp8k::launch_quant_act_block(x, M, K, ld_x, q, lay.ld_q, sa, KB, s,
                                     (uint32_t*)(ws8 + lay.gemm), nzero);
  else if (scale_mode == FP8_SCALE_ROW)
    e = fp8k::launch_quant_rows(x, M, K, ld_x, q, lay.ld_q, sa, 1, s);
  else
    e = fp8k::launch_quant_tensor(x, M, K, ld_x, q, lay.ld_q, sa, (uint32_t*)(ws8 + lay.partials),
                                  s);
  if (e != hipSuccess) return FP8_ERR_LAUNCH;
  const int64_t lsa = scale_mode == FP8_SCALE_BLOCK ? KB : scale_mode == FP8_SCALE_ROW ? 1 : 0;
  const int64_t lsw = scale_mode == FP8_SCALE_TENSOR ? 0 : ld_ws;
  return launched(fp8k::launch_gemm(q, lay.ld_q, sa, lsa, w_q, ld_w, w_s, lsw, out, ld_out, M, N,
                                    K, scale_mode != FP8_SCALE_BLOCK, ws8 + lay.gemm,
                                    lay.gemm_bytes, s, nzero > 0));
}

// Scratch of fp8_linear_noalloc: a file-scope device array, one copy per
// device, held until the process ends.  In host code `scratch` names a
// host-side stand-in, not device memory: its device address is looked up
// once per device with hipGetSymbolAddress (no allocation) and only that
// address is handed to kernels.
__device__ __align__(256) uint8_t scratch[FP8_NOALLOC_SCRATCH_BYTES];
std::atomic<void*> g_scratch[kMaxDevices];

fp8_status device_scratch(void** ptr) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return FP8_ERR_DEVICE;
  void* p = g_scratch[dev].load(std::memory_order_acquire);
  if (!p) {
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return FP8_ERR_DEVICE;
    g_scratch[dev].store(p, std::memory_order_release);   // racing threads store the same address
  }
  *ptr = p;
  return FP8_OK;
}

}  // namespace

extern "C" {

fp8_status fp8_linear(const uint16_t* x, int64_t ld_x, const uint8_t* w_q, int64_t ld_w,
                      const float* w_s, int64_t ld_ws, uint16_t* out, int64_t ld_out,
                      int64_t M, int64_t N, int64_t K, int scale_mode, void* workspace,
                      size_t ws_bytes, void* stream) {
  bool fused = false;
  LinearLayout lay{};
  fp8_status st = validate_linear(x, ld_x, w_q, ld_w, w_s, ld_ws, out, ld_out, M, N, K,
                                  scale_mode, fused, lay);
  if (st != FP8_OK || M == 0) return st;
  if (!fused) {
    if (!workspace || ws_bytes < lay.total || !aligned(workspace, 16)) return FP8_ERR_WORKSPACE;
    if (!linear_workspace_clear(x, ld_x, w_q, ld_w, w_s, ld_ws, out, ld_out, M, N, K, scale_mode,
                                workspace, lay.total))
      return FP8_ERR_ALIAS;
  }
  if ((st = check_device()) != FP8_OK) return st;
  return run_linear(x, ld_x, w_q, ld_w, w_s, ld_ws, out, ld_out, M, N, K, scale_mode, fused, lay,
                    workspace, (hipStream_t)stream);
}

fp8_status fp8_linear_noalloc(const uint16_t* x, int64_t ld_x, const uint8_t* w_q, int64_t ld_w,
                              const float* w_s, int64_t ld_ws, uint16_t* out, int64_t ld_out,
                              int64_t M, int64_t N, int64_t K, int scale_mode, void* stream) {
  bool fused = false;
  LinearLayout lay{};
  fp8_status st = validate_linear(x, ld_x, w_q, ld_w, w_s, ld_ws, out, ld_out, M, N, K,
                                  scale_mode, fused, lay);
  if (st != FP8_OK || M == 0) return st;
  if (!fused && lay.total > (size_t)FP8_NOALLOC_SCRATCH_BYTES) return FP8_ERR_SCRATCH;
  if ((st = check_device()) != FP8_OK) return st;
  void* ws = nullptr;
  if (!fused && (st = device_scratch(&ws)) != FP8_OK) return st;
  return run_linear(x, ld_x, w_q, ld_w, w_s, ld_ws, out, ld_out, M, N, K, scale_mode, fused, lay,
                    ws, (hipStream_t)stream);
}

fp8_status fp8_validate_quant_act_static(const uint16_t* x, int64_t M, int64_t K, int64_t ld_x,
                                         const uint8_t* q, int64_t ld_q, const float* scale) {
  if (M < 0 || M >= kMaxDim || !shape_ok_kn(K)) return FP8_ERR_SHAPE;
  if (M > 0 && M * K > kMaxElems) return FP8_ERR_SHAPE;
  if (M == 0) return FP8_OK;
  if (!x || !q || !scale) return FP8_ERR_NULL;
  if (ld_x < K || ld_q < K) return FP8_ERR_STRIDE;
  if (!span_ok(M, ld_x) || !span_ok(M, ld_q)) return FP8_ERR_STRIDE;
  if (!aligned(x, 16) || !aligned(q, 16) || !aligned(scale, 4)) return FP8_ERR_ALIGN;
  if (ld_x % 8 != 0 || ld_q % 16 != 0) return FP8_ERR_ALIGN;
  Range rx = range_of(x, M, K, ld_x, 2), rq = range_of(q, M, K, ld_q, 1);
  Range rs = range_of(scale, 1, 1, 1, 4);
  if (overlap(rx, rq) || overlap(rq, rs)) return FP8_ERR_ALIAS;
  return FP8_OK;
}

fp8_status fp8_quant_act_static(const uint16_t* x, int64_t M, int64_t K, int64_t ld_x, uint8_t* q,
                                int64_t ld_q, const float* scale, void* stream) {
  fp8_status st = fp8_validate_quant_act_static(x, M, K, ld_x, q, ld_q, scale);
  if (st != FP8_OK || M == 0) return st;
  if ((st = check_device()) != FP8_OK) return st;
  return launched(fp8k::launch_quant_static(x, M, K, ld_x, q, ld_q, scale, (hipStream_t)stream));
}

// ---- grouped (MoE) GEMM ---------------------------------------------------

fp8_status fp8_validate_grouped_gemm(const uint8_t* a_q, int64_t ld_a, const float* a_s,
                                     int64_t ld_as, const uint8_t* w_q, int64_t ld_w,
                                     const float* w_s, int64_t ld_ws,
                                     const int64_t* expert_offsets, int64_t E, const uint16_t* out,
                                     int64_t ld_out, int64_t M, int64_t N, int64_t K) {
  if (E < 0 || E > 65535) return FP8_ERR_SHAPE;
  if (M < 0 || M >= kMaxDim || !shape_ok_kn(K) || !shape_ok_kn(N)) return FP8_ERR_SHAPE;
  if (K / 128 > fp8k::kGroupedMaxKB) return FP8_ERR_SHAPE;
  if (fp8k::grouped_items(N) >= fp8k::kMaxGridItems) return FP8_ERR_SHAPE;
  if (M * K > kMaxElems || M * N > kMaxElems || N * K > kMaxElems / (E > 0 ? E : 1))
    return FP8_ERR_SHAPE;
  if (M == 0 || E == 0) return FP8_OK;
  if (!a_q || !a_s || !w_q || !w_s || !out || !expert_offsets) return FP8_ERR_NULL;
  const int64_t KB = K / 128;
  if (ld_a < K || ld_w < K || ld_out < N || ld_as < KB || ld_ws < KB) return FP8_ERR_STRIDE;
  if (!span_ok(M, ld_a) || !span_ok(M, ld_as) || !span_ok(M, ld_out) || !span_ok(E * N, ld_w) ||
      !span_ok(E * (N / 128), ld_ws))
    return FP8_ERR_STRIDE;
  if (!aligned(a_q, 16) || !aligned(w_q, 16) || !aligned(out, 16)) return FP8_ERR_ALIGN;
  if (!aligned(a_s, 4) || !aligned(w_s, 4) || !aligned(expert_offsets, 8)) return FP8_ERR_ALIGN;
  if (ld_a % 16 != 0 || ld_w % 16 != 0 || ld_out % 8 != 0) return FP8_ERR_ALIGN;
  const Range ro = range_of(out, M, N, ld_out, 2);
  const Range ins[] = {range_of(a_q, M, K, ld_a, 1), range_of(a_s, M, KB, ld_as, 4),
                       range_of(w_q, E * N, K, ld_w, 1), range_of(w_s, E * (N / 128), KB, ld_ws, 4),
                       range_of(expert_offsets, 1, E + 1, E + 1, 8)};
  for (const Range& r : ins)
    if (overlap(ro, r)) return FP8_ERR_ALIAS;
  return FP8_OK;
}

fp8_status fp8_grouped_gemm(const uint8_t* a_q, int64_t ld_a, const float* a_s, int64_t ld_as,
                            const uint8_t* w_q, int64_t ld_w, const float* w_s, int64_t ld_ws,
                            const int64_t* expert_offsets, int64_t E, uint16_t* out,
                            int64_t ld_out, int64_t M, int64_t N, int64_t K, void* stream) {
  fp8_status st = fp8_validate_grouped_gemm(a_q, ld_a, a_s, ld_as, w_q, ld_w, w_s, ld_ws,
                                            expert_offsets, E, out, ld_out, M, N, K);
  if (st != FP8_OK || M == 0 || E == 0) return st;
  if ((st = check_device()) != FP8_OK) return st;
  return launched(fp8k::launch_grouped_gemm(a_q, ld_a, a_s, ld_as, w_q, ld_w, w_s, ld_ws, out,
                                            ld_out, expert_offsets, E, M, N, K,
                                            (hipStream_t)stream));
}

// ---- FP8 KV-cache codec --------------------------------------------------

namespace {

// Common shape checks: H * D values per token (a multiple of 8), a cache of
// num_blocks * block_size slots.
fp8_status kv_shape(int64_t T, int64_t H, int64_t D, int64_t num_blocks, int64_t block_size) {
  if (T < 0 || T >= kMaxDim || H <= 0 || D <= 0 || H >= kMaxDim || D >= kMaxDim)
    return FP8_ERR_SHAPE;
  if (num_blocks < 0 || num_blocks >= kMaxDim || block_size <= 0 || block_size >= kMaxDim)
    return FP8_ERR_SHAPE;
  const int64_t hd = H * D;
  if (hd >= kMaxDim || hd % 8 != 0) return FP8_ERR_SHAPE;
  if (num_blocks * block_size > kMaxElems / hd || T > kMaxElems / hd) return FP8_ERR_SHAPE;
  return FP8_OK;
}

}  // namespace

fp8_status fp8_validate_kv_cache_write(const uint16_t* key, int64_t ld_key,
                                       const uint16_t* value, int64_t ld_value,
                                       const int64_t* slot_mapping, int64_t T, int64_t H,
                                       int64_t D, const uint8_t* key_cache,
                                       const uint8_t* value_cache, int64_t num_blocks,
                                       int64_t block_size, const float* k_scale,
                                       const float* v_scale) {
  fp8_status st = kv_shape(T, H, D, num_blocks, block_size);
  if (st != FP8_OK || T == 0) return st;
  const int64_t hd = H * D, cap = num_blocks * block_size;
  if (!key || !value || !slot_mapping || !k_scale || !v_scale) return FP8_ERR_NULL;
  if (cap > 0 && (!key_cache || !value_cache)) return FP8_ERR_NULL;
  if (ld_key < hd || ld_value < hd) return FP8_ERR_STRIDE;
  if (!span_ok(T, ld_key) || !span_ok(T, ld_value)) return FP8_ERR_STRIDE;
  if (!aligned(key, 16) || !aligned(value, 16) || !aligned(slot_mapping, 8) ||
      !aligned(key_cache, 16) || !aligned(value_cache, 16) || !aligned(k_scale, 4) ||
      !aligned(v_scale, 4))
    return FP8_ERR_ALIGN;
  if (ld_key % 8 != 0 || ld_value % 8 != 0) return FP8_ERR_ALIGN;
  const Range ins[] = {range_of(key, T, hd, ld_key, 2), range_of(value, T, hd, ld_value, 2),
                       range_of(slot_mapping, 1, T, T, 8), range_of(k_scale, 1, 1, 1, 4),
                       range_of(v_scale, 1, 1, 1, 4)};
  const Range kc = range_of(key_cache, cap, hd, hd, 1), vc = range_of(value_cache, cap, hd, hd, 1);
  if (overlap(kc, vc)) return FP8_ERR_ALIAS;
  for (const Range& r : ins)
    if (overlap(r, kc) || overlap(r, vc)) return FP8_ERR_ALIAS;
  return FP8_OK;
}

fp8_status fp8_kv_cache_write(const uint16_t* key, int64_t ld_key, const uint16_t* value,
                              int64_t ld_value, const int64_t* slot_mapping, int64_t T, int64_t H,
                              int64_t D, uint8_t* key_cache, uint8_t* value_cache,
                              int64_t num_blocks, int64_t block_size, const float* k_scale,
                              const float* v_scale, void* stream) {
  fp8_status st = fp8_validate_kv_cache_write(key, ld_key, value, ld_value, slot_mapping, T, H, D,
                                              key_cache, value_cache, num_blocks, block_size,
                                              k_scale, v_scale);
  if (st != FP8_OK || T == 0) return st;
  if ((st = check_device()) != FP8_OK) return st;
  return launched(fp8k::launch_kv_write(key, ld_key, value, ld_value, slot_mapping, T, H * D,
                                        key_cache, value_cache, num_blocks * block_size, k_scale,
                                        v_scale, (hipStream_t)stream));
}

fp8_status fp8_validate_kv_cache_read(const uint8_t* cache, int64_t num_blocks,
                                      int64_t block_size, int64_t H, int64_t D,
                                      const int64_t* slots, int64_t T, const float* scale,
                                      const uint16_t* out, int64_t ld_out) {
  fp8_status st = kv_shape(T, H, D, num_blocks, block_size);
  if (st != FP8_OK || T == 0) return st;
  const int64_t hd = H * D, cap = num_blocks * block_size;
  if (!slots || !scale || !out) return FP8_ERR_NULL;
  if (cap > 0 && !cache) return FP8_ERR_NULL;
  if (ld_out < hd || !span_ok(T, ld_out)) return FP8_ERR_STRIDE;
  if (!aligned(cache, 16) || !aligned(slots, 8) || !aligned(scale, 4) || !aligned(out, 16))
    return FP8_ERR_ALIGN;
  if (ld_out % 8 != 0) return FP8_ERR_ALIGN;
  const Range ro = range_of(out, T, hd, ld_out, 2);
  if (overlap(ro, range_of(cache, cap, hd, hd, 1)) || overlap(ro, range_of(slots, 1, T, T, 8)) ||
      overlap(ro, range_of(scale, 1, 1, 1, 4)))
    return FP8_ERR_ALIAS;
  return FP8_OK;
}

fp8_status fp8_kv_cache_read(const uint8_t* cache, int64_t num_blocks, int64_t block_size,
                             int64_t H, int64_t D, const int64_t* slots, int64_t T,
                             const float* scale, uint16_t* out, int64_t ld_out, void* stream) {
  fp8_status st = fp8_validate_kv_cache_read(cache, num_blocks, block_size, H, D, slots, T, scale,
                                             out, ld_out);
  if (st != FP8_OK || T == 0) return st;
  if ((st = check_device()) != FP8_OK) return st;
  return launched(fp8k::launch_kv_read(cache, num_blocks * block_size, H * D, slots, T, scale, out,
                                       ld_out, (hipStream_t)stream));
}

fp8_status fp8_e4m3_encode_f32(const float* x, int64_t n, uint8_t* codes, void* stream) {
  if (n < 0 || n > kMaxElems || fp8k::encode_items(n) >= fp8k::kMaxGridItems)
    return FP8_ERR_SHAPE;
  if (n == 0) return FP8_OK;
  if (!x || !codes) return FP8_ERR_NULL;
  if (!aligned(x, 4)) return FP8_ERR_ALIGN;
  if (overlap(range_of(x, 1, n, n, 4), range_of(codes, 1, n, n, 1))) return FP8_ERR_ALIAS;
  fp8_status st = check_device();
  if (st != FP8_OK) return st;
  return launched(fp8k::launch_encode_f32(x, n, codes, (hipStream_t)stream));
}

}  // extern "C"
