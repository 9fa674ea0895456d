// capi.hip -- the C ABI of libhdq (declared in include/hdq.h).
//
// Validates every argument before anything is enqueued, carves the caller's
// workspace, and enqueues the kernels on the caller's stream.  No allocation,
// no synchronisation, no global state.
#include "hdq.h"
#include "hdq_internal.h"

#include <hip/hip_runtime.h>

#include <mutex>

// Fixed scratch of the allocation-free entry points: one copy per GPU, held
// until the process ends.  In host code `scratch` names a host-side stand-in,
// never the device memory: kernels and copies get the address that
// hipGetSymbolAddress returns for the current device (noalloc_scratch below).
static __device__ __align__(256) unsigned char scratch[HDQ_NOALLOC_SCRATCH_BYTES];

namespace {

using namespace hdq;

constexpr size_t kAlign = 256;
size_t align_up(size_t v) { return (v + kAlign - 1) / kAlign * kAlign; }

bool valid_block(int32_t hb) { return hb >= 1 && hb <= 128 && (hb & (hb - 1)) == 0; }

// Shape rules shared by the quantizers: cols a multiple of 8 (16-byte rows of
// bf16 chunks) and of the Hadamard block and of the format's scale block.
int check_quant_shape(int64_t rows, int64_t cols, int32_t hb, int32_t fmt) {
  if (rows <= 0 || cols <= 0 || rows > 0x7fffffff || !valid_block(hb)) return HDQ_ERR_SHAPE;
  if (cols % 8 != 0 || cols % hb != 0) return HDQ_ERR_SHAPE;
  if ((fmt == HDQ_FMT_NVFP4 || fmt == HDQ_FMT_NVFP4_P2) && cols % 16 != 0) return HDQ_ERR_SHAPE;
  if (fmt == HDQ_FMT_NVFP4_MX && cols % 32 != 0) return HDQ_ERR_SHAPE;
  return HDQ_OK;
}

bool valid_fmt(int32_t fmt) { return fmt >= HDQ_FMT_INT8_ROW && fmt <= HDQ_FMT_NVFP4_P2; }
bool is_fp4(int32_t fmt) {
  return fmt == HDQ_FMT_NVFP4 || fmt == HDQ_FMT_NVFP4_MX || fmt == HDQ_FMT_NVFP4_P2;
}

// The NVFP4 GEMM for the weights' format: FP4 MFMA (one pass per 32
// elements for MX, two for per-16 powers of two) or exact bf16 MFMA.
using Fp4Gemm = hipError_t (*)(const uint8_t*, const uint8_t*, const float*, const uint8_t*,
                               const uint8_t*, const float*, void*, int, int64_t, int64_t, int64_t,
                               const int32_t*, int32_t, hipStream_t);
Fp4Gemm fp4_gemm_for(int32_t fmt) {
  return fmt == HDQ_FMT_NVFP4_MX ? launch_gemm_nvfp4_mx
       : fmt == HDQ_FMT_NVFP4_P2 ? launch_gemm_nvfp4_p2 : launch_gemm_nvfp4_bf16;
}

// Bytes of one quantized activation tensor [M, K] in `fmt` (codes and scales).
size_t qtensor_bytes(int64_t M, int64_t K, int32_t fmt) {
  if (fmt == HDQ_FMT_INT8_ROW) return align_up((size_t)(M * K)) + align_up((size_t)M * 4);
  if (is_fp4(fmt)) return align_up((size_t)(M * K / 2)) + align_up((size_t)(M * K / 16)) + kAlign;
  return 0;
}

// Scratch of hdq_dq_linear: the core GEMM's fp32 [cubes, N]; on the combine
// route (shapes the fused core-add GEMM does not take) also the difference
// GEMM's fp32 [tokens, N] after it.
size_t dq_linear_ws(int64_t tokens, int64_t cubes, int64_t N, int64_t K, int32_t fmt) {
  size_t b = align_up((size_t)cubes * (size_t)N * 4);
  if (!fp4_core_add_applies(fmt, tokens, N, K)) b += align_up((size_t)tokens * (size_t)N * 4);
  return b;
}

// Scratch of the NVFP4 tensor-amax pre-pass: the stats partials + one float.
size_t amax_prepass_bytes() { return align_up(kStatsPartialBytes) + kAlign; }

int hip_status(hipError_t e) { return e == hipSuccess ? HDQ_OK : HDQ_ERR_HIP; }

// Device address of `scratch` on the current device, looked up once per
// device (with that device current) and kept; null if HIP reports an error.
void* noalloc_scratch() {
  constexpr int kMaxDevices = 64;
  static std::mutex mu;
  static void* ptr[kMaxDevices] = {};
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return nullptr;
  std::lock_guard<std::mutex> lock(mu);
  if (ptr[dev] == nullptr) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || p == nullptr) return nullptr;
    ptr[dev] = p;
  }
  return ptr[dev];
}

// Checks a quantized tensor's descriptor against a [rows, cols] operand.
int check_qtensor(const hdq_qtensor& q, int32_t fmt, int64_t rows, int64_t cols) {
  if (q.fmt != fmt) return HDQ_ERR_UNSUPPORTED;
  if (q.rows != rows || q.cols != cols) return HDQ_ERR_SHAPE;
  if (!valid_block(q.had_block)) return HDQ_ERR_SHAPE;
  if (q.codes == nullptr) return HDQ_ERR_INVALID;
  if ((fmt == HDQ_FMT_INT8_ROW || fmt == HDQ_FMT_INT4_ROW) && q.row_scale == nullptr) return HDQ_ERR_INVALID;
  if (is_fp4(fmt) && (q.blk_scale == nullptr || q.tensor_scale == nullptr)) return HDQ_ERR_INVALID;
  return HDQ_OK;
}

// Enqueues rotation + quantization of x into q (fields already filled).
// amax: NVFP4 rotated amax (device) or null; scratch holds the pre-pass
// space when amax is null.
hipError_t enqueue_quantize(const void* x, const hdq_qtensor& q, const float* amax, uint8_t* scratch,
                            const int32_t* gate, int32_t want, hipStream_t s) {
  const uint16_t* xb = static_cast<const uint16_t*>(x);
  if (q.fmt == HDQ_FMT_INT8_ROW || q.fmt == HDQ_FMT_INT4_ROW)
    return launch_quant_int_rows(xb, q.rows, q.cols, q.had_block, q.fmt, q.codes, q.row_scale, gate,
                                 want, s);
  if (amax == nullptr) {
    double* partials = reinterpret_cast<double*>(scratch);
    float* slot = reinterpret_cast<float*>(scratch + align_up(kStatsPartialBytes));
    hipError_t e = launch_stats(nullptr, nullptr, 0, xb, q.rows * q.cols, q.had_block, 0.0f, 0.0f,
                                nullptr, nullptr, slot, partials, gate, want, s);
    if (e != hipSuccess) return e;
    amax = slot;
  }
  return launch_quant_nvfp4(xb, q.rows, q.cols, q.had_block, q.fmt, amax, static_cast<uint8_t*>(q.codes),
                            q.blk_scale, q.tensor_scale, gate, want, s, static_cast<uint16_t*>(q.dec));
}

// Which decoded bf16 copies the plain-NVFP4 GEMM reads: both operands'
// (kNvfp4Decoded), the activations' only (kNvfp4XDecoded), or none (0),
// as given and as the pipelined bf16 body takes the shape (the one-launch
// kernel's shape rule implies both).
int decoded_mode(int32_t fmt, const hdq_qtensor& xq, const hdq_qtensor& wq, int64_t M, int64_t N, int64_t K) {
  if (fmt != HDQ_FMT_NVFP4 || xq.dec == nullptr) return 0;
  if (wq.dec != nullptr) return nvfp4_decoded_applies(M, N, K) ? kNvfp4Decoded : 0;
  return nvfp4_xdecoded_applies(M, N, K) ? kNvfp4XDecoded : 0;
}

// The plain-NVFP4 GEMM from decoded activations (and weights, mode
// kNvfp4Decoded).
hipError_t launch_decoded_gemm(int mode, const hdq_qtensor& xq, const hdq_qtensor& wq, void* y, int32_t y_dtype,
                               int64_t M, int64_t N, int64_t K, const int32_t* gate, hipStream_t s) {
  if (mode == kNvfp4Decoded)
    return launch_gemm_nvfp4_decoded(static_cast<const uint16_t*>(xq.dec), xq.tensor_scale,
                                     static_cast<const uint16_t*>(wq.dec), wq.tensor_scale, y, y_dtype, M, N, K,
                                     gate, HDQ_PREC_NVFP4, s);
  return launch_gemm_nvfp4_xdecoded(static_cast<const uint16_t*>(xq.dec), xq.tensor_scale,
                                    static_cast<const uint8_t*>(wq.codes), wq.blk_scale, wq.tensor_scale, y,
                                    y_dtype, M, N, K, gate, HDQ_PREC_NVFP4, s);
}

}  // namespace

extern "C" {

const char* hdq_status_string(int status) {
  switch (status) {
    case HDQ_OK: return "ok";
    case HDQ_ERR_INVALID: return "invalid argument (null pointer, bad enum or descriptor field)";
    case HDQ_ERR_SHAPE: return "bad shape (size, alignment or Hadamard block)";
    case HDQ_ERR_UNSUPPORTED: return "unsupported precision / format / output dtype combination";
    case HDQ_ERR_HIP: return "HIP launch error";
    case HDQ_ERR_WORKSPACE: return "workspace missing or too small";
    case HDQ_ERR_TOO_LARGE: return "input too large for the allocation-free call's fixed scratch";
    default: return "unknown status";
  }
}

int hdq_version(void) { return 10000; }

size_t hdq_workspace_bytes(int32_t op, int64_t M, int64_t K, int64_t N, int32_t fmt) {
  if (M <= 0 || K <= 0) return 0;
  switch (op) {
    case HDQ_OP_SELECT:
      return align_up(kStatsPartialBytes);
    case HDQ_OP_QUANTIZE:
      if (!valid_fmt(fmt)) return 0;
      return is_fp4(fmt) ? amax_prepass_bytes() : 0;
    case HDQ_OP_SELECT_Q8: {
      // one statistics partial per row (or the two-pass route's partials)
      const size_t per_row = (size_t)(M > 0 ? M : 0) * 6 * sizeof(double);
      return align_up(per_row > kStatsPartialBytes ? per_row : kStatsPartialBytes);
    }
    case HDQ_OP_DQ_QUANTIZE:
      return 256;
    case HDQ_OP_DQ_LINEAR:  // M = tokens, K = cubes
      if (N <= 0) return 0;
      return align_up((size_t)M * (size_t)N * 4) + align_up((size_t)K * (size_t)N * 4);
    case HDQ_OP_LINEAR: {
      (void)N;
      size_t b = qtensor_bytes(M, K, HDQ_FMT_INT8_ROW);
      if (is_fp4(fmt)) b += qtensor_bytes(M, K, fmt) + amax_prepass_bytes();
      return b;
    }
    default:
      return 0;
  }
}

int hdq_select_precision(const void* prev_in, const void* prev_out, int64_t prev_numel,
                         const void* cur_in, int64_t rows, int64_t cols, int32_t had_block,
                         float delta_thresh, float ratio_thresh, int32_t* decision_dev,
                         float* stats_dev, void* ws, size_t ws_bytes, void* stream) {
  if (cur_in == nullptr || decision_dev == nullptr || stats_dev == nullptr) return HDQ_ERR_INVALID;
  if ((prev_in == nullptr) != (prev_out == nullptr)) return HDQ_ERR_INVALID;
  if (rows <= 0 || cols <= 0) return HDQ_ERR_SHAPE;
  if (prev_in != nullptr && prev_numel <= 0) return HDQ_ERR_SHAPE;
  if (had_block != 0 && (!valid_block(had_block) || cols % had_block != 0 || cols % 8 != 0))
    return HDQ_ERR_SHAPE;
  if (ws == nullptr || ws_bytes < align_up(kStatsPartialBytes)) return HDQ_ERR_WORKSPACE;
  hipStream_t s = static_cast<hipStream_t>(stream);
  return hip_status(launch_stats(static_cast<const uint16_t*>(prev_in),
                                 static_cast<const uint16_t*>(prev_out), prev_numel,
                                 static_cast<const uint16_t*>(cur_in), rows * cols, had_block,
                                 delta_thresh, ratio_thresh, decision_dev, stats_dev, nullptr,
                                 static_cast<double*>(ws), nullptr, 0, s));
}

int hdq_delta_sums(const void* prev_in, const void* prev_out, int64_t numel, double* sums_dev,
                   void* ws, size_t ws_bytes, void* stream) {
  if (prev_in == nullptr || prev_out == nullptr || sums_dev == nullptr) return HDQ_ERR_INVALID;
  if (numel <= 0) return HDQ_ERR_SHAPE;
  if (ws == nullptr || ws_bytes < align_up(kStatsPartialBytes)) return HDQ_ERR_WORKSPACE;
  hipStream_t s = static_cast<hipStream_t>(stream);
  return hip_status(launch_stats(static_cast<const uint16_t*>(prev_in),
                                 static_cast<const uint16_t*>(prev_out), numel, nullptr, 0, 0, 0.0f,
                                 0.0f, nullptr, nullptr, nullptr, static_cast<double*>(ws), nullptr, 0,
                                 s, nullptr, sums_dev));
}

int hdq_select_precision_sums(const double* delta_sums_dev, int64_t delta_parts, const void* cur_in,
                              int64_t rows, int64_t cols, int32_t had_block, float delta_thresh,
                              float ratio_thresh, int32_t* decision_dev, float* stats_dev, void* ws,
                              size_t ws_bytes, void* stream) {
  if (cur_in == nullptr || decision_dev == nullptr || stats_dev == nullptr) return HDQ_ERR_INVALID;
  if (rows <= 0 || cols <= 0) return HDQ_ERR_SHAPE;
  if (delta_sums_dev != nullptr && (delta_parts < 1 || delta_parts > 0x7fffffff)) return HDQ_ERR_SHAPE;
  if (had_block != 0 && (!valid_block(had_block) || cols % had_block != 0 || cols % 8 != 0))
    return HDQ_ERR_SHAPE;
  if (ws == nullptr || ws_bytes < align_up(kStatsPartialBytes)) return HDQ_ERR_WORKSPACE;
  hipStream_t s = static_cast<hipStream_t>(stream);
  return hip_status(launch_stats(nullptr, nullptr, 0, static_cast<const uint16_t*>(cur_in),
                                 rows * cols, had_block, delta_thresh, ratio_thresh, decision_dev,
                                 stats_dev, nullptr, static_cast<double*>(ws), nullptr, 0, s,
                                 delta_sums_dev, nullptr, delta_parts));
}

}  // extern "C"

namespace {

// Argument checks of hdq_select_quantize_int8 (everything but the workspace).
int check_select_q8(const double* delta_sums_dev, int64_t delta_parts, const void* cur_in, int64_t rows,
                    int64_t cols, int32_t had_block, const int32_t* decision_dev, const float* stats_dev,
                    const hdq_qtensor* xq8) {
  if (cur_in == nullptr || decision_dev == nullptr || stats_dev == nullptr || xq8 == nullptr)
    return HDQ_ERR_INVALID;
  if (delta_sums_dev != nullptr && (delta_parts < 1 || delta_parts > 0x7fffffff)) return HDQ_ERR_SHAPE;
  if (xq8->codes == nullptr || xq8->row_scale == nullptr) return HDQ_ERR_INVALID;
  if (had_block == 0) return HDQ_ERR_SHAPE;
  int st = check_quant_shape(rows, cols, had_block, HDQ_FMT_INT8_ROW);
  if (st != HDQ_OK) return st;
  if (cols % 8 != 0) return HDQ_ERR_SHAPE;
  return HDQ_OK;
}

// Enqueues the fused selection + INT8 quantization (arguments checked; ws
// holds the per-row partials).
int enqueue_select_q8(const double* delta_sums_dev, int64_t delta_parts, const void* cur_in, int64_t rows,
                      int64_t cols, int32_t had_block, float delta_thresh, float ratio_thresh,
                      int32_t* decision_dev, float* stats_dev, hdq_qtensor* xq8, void* ws, hipStream_t s) {
  xq8->fmt = HDQ_FMT_INT8_ROW;
  xq8->had_block = had_block;
  xq8->rows = rows;
  xq8->cols = cols;
  const uint16_t* xb = static_cast<const uint16_t*>(cur_in);
  double* part = static_cast<double*>(ws);
  if (cols <= 16384) {
    // per-row partials, struct-of-arrays: sums, magnitude bits, rotated maxima
    uint32_t* pbits = reinterpret_cast<uint32_t*>(part + rows);
    float* ptmax = reinterpret_cast<float*>(pbits + rows);
    hipError_t e = launch_quant_int8_stats(xb, rows, cols, had_block, xq8->codes, xq8->row_scale, part,
                                           pbits, ptmax, s);
    if (e != hipSuccess) return HDQ_ERR_HIP;
    return hip_status(launch_stats_finalize_rows(part, pbits, ptmax, rows, rows * cols, had_block,
                                                 delta_thresh, ratio_thresh, decision_dev, stats_dev,
                                                 delta_sums_dev, delta_parts, s));
  }
  // rows too long to keep in registers: the two passes separately
  hipError_t e = launch_stats(nullptr, nullptr, 0, xb, rows * cols, had_block, delta_thresh, ratio_thresh,
                              decision_dev, stats_dev, nullptr, part, nullptr, 0, s, delta_sums_dev,
                              nullptr, delta_parts);
  if (e != hipSuccess) return HDQ_ERR_HIP;
  return hip_status(launch_quant_int_rows(xb, rows, cols, had_block, HDQ_FMT_INT8_ROW, xq8->codes,
                                          xq8->row_scale, nullptr, 0, s));
}

}  // namespace

extern "C" {

int hdq_select_quantize_int8(const double* delta_sums_dev, int64_t delta_parts, const void* cur_in,
                             int64_t rows, int64_t cols, int32_t had_block, float delta_thresh,
                             float ratio_thresh, int32_t* decision_dev, float* stats_dev,
                             hdq_qtensor* xq8, void* ws, size_t ws_bytes, void* stream) {
  int st = check_select_q8(delta_sums_dev, delta_parts, cur_in, rows, cols, had_block, decision_dev, stats_dev,
                           xq8);
  if (st != HDQ_OK) return st;
  if (ws == nullptr || ws_bytes < hdq_workspace_bytes(HDQ_OP_SELECT_Q8, rows, cols, 0, 0))
    return HDQ_ERR_WORKSPACE;
  return enqueue_select_q8(delta_sums_dev, delta_parts, cur_in, rows, cols, had_block, delta_thresh,
                           ratio_thresh, decision_dev, stats_dev, xq8, ws, static_cast<hipStream_t>(stream));
}

int hdq_select_quantize_int8_noalloc(const double* delta_sums_dev, int64_t delta_parts, const void* cur_in,
                                     int64_t rows, int64_t cols, int32_t had_block, float delta_thresh,
                                     float ratio_thresh, int32_t* decision_dev, float* stats_dev,
                                     hdq_qtensor* xq8, void* stream) {
  int st = check_select_q8(delta_sums_dev, delta_parts, cur_in, rows, cols, had_block, decision_dev, stats_dev,
                           xq8);
  if (st != HDQ_OK) return st;
  if (hdq_workspace_bytes(HDQ_OP_SELECT_Q8, rows, cols, 0, 0) > HDQ_NOALLOC_SCRATCH_BYTES)
    return HDQ_ERR_TOO_LARGE;
  void* ws = noalloc_scratch();
  if (ws == nullptr) return HDQ_ERR_HIP;
  return enqueue_select_q8(delta_sums_dev, delta_parts, cur_in, rows, cols, had_block, delta_thresh,
                           ratio_thresh, decision_dev, stats_dev, xq8, ws, static_cast<hipStream_t>(stream));
}

int hdq_tdc_decide(const double* sums_dev, const int64_t* parts_offsets_dev, const int32_t* state_dev,
                   float* c_dev, float* acc_dev, int32_t* skip_dev, int64_t n, float tau_skip,
                   float tau_acc, void* stream) {
  if (sums_dev == nullptr || state_dev == nullptr || c_dev == nullptr || acc_dev == nullptr ||
      skip_dev == nullptr)
    return HDQ_ERR_INVALID;
  if (n <= 0 || n > 0x7fffffff) return HDQ_ERR_SHAPE;
  return hip_status(launch_tdc_decide(sums_dev, parts_offsets_dev, state_dev, c_dev, acc_dev, skip_dev, n,
                                      tau_skip, tau_acc, static_cast<hipStream_t>(stream)));
}

int hdq_linear_dispatch(const int32_t* decision_dev, const void* x, const hdq_qtensor* xq8,
                        const hdq_qtensor* xq4, int64_t M, int64_t K, const hdq_weights* w, void* y,
                        int32_t y_dtype, void* stream) {
  if (decision_dev == nullptr || x == nullptr || xq8 == nullptr || xq4 == nullptr || w == nullptr ||
      y == nullptr)
    return HDQ_ERR_INVALID;
  if (y_dtype != HDQ_DTYPE_F32 && y_dtype != HDQ_DTYPE_BF16) return HDQ_ERR_UNSUPPORTED;
  if (M <= 0 || K <= 0 || w->N <= 0 || M > 0x7fffffff || K > 0x7fffffff || w->N > 0x7fffffff)
    return HDQ_ERR_SHAPE;
  if (w->K != K) return HDQ_ERR_SHAPE;
  const int64_t N = w->N;
  const int32_t f = w->w_fp4.fmt;
  int st;
  if ((st = check_qtensor(w->w_int4, HDQ_FMT_INT4_ROW, N, K)) != HDQ_OK) return st;
  if ((st = check_qtensor(*xq8, HDQ_FMT_INT8_ROW, M, K)) != HDQ_OK) return st;
  if (!is_fp4(f)) return HDQ_ERR_UNSUPPORTED;
  if ((st = check_qtensor(w->w_fp4, f, N, K)) != HDQ_OK) return st;
  if ((st = check_qtensor(*xq4, f, M, K)) != HDQ_OK) return st;
  if (w->w_bf16 == nullptr) return HDQ_ERR_INVALID;
  if (K % 32 != 0 || xq8->had_block != w->w_int4.had_block || xq4->had_block != w->w_fp4.had_block)
    return HDQ_ERR_SHAPE;
  hipStream_t s = static_cast<hipStream_t>(stream);
  const uint16_t* xb = static_cast<const uint16_t*>(x);
  const uint16_t* wb = static_cast<const uint16_t*>(w->w_bf16);
  const int dm = decoded_mode(f, *xq4, w->w_fp4, M, N, K);
  hipError_t e = launch_gemm_dispatch(
      decision_dev, static_cast<const int8_t*>(xq8->codes), xq8->row_scale,
      static_cast<const uint8_t*>(w->w_int4.codes), w->w_int4.row_scale,
      static_cast<const uint8_t*>(dm ? xq4->dec : xq4->codes), xq4->blk_scale, xq4->tensor_scale,
      static_cast<const uint8_t*>(dm == kNvfp4Decoded ? w->w_fp4.dec : w->w_fp4.codes), w->w_fp4.blk_scale,
      w->w_fp4.tensor_scale, dm ? dm : f, xb, wb, y, y_dtype, M, N, K, s);
  if (e == hipSuccess) return HDQ_OK;
  if (e != hipErrorNotSupported) return HDQ_ERR_HIP;
  // shapes the pipelined bodies do not take: the three gated GEMMs
  if (launch_gemm_i8i4(static_cast<const int8_t*>(xq8->codes), xq8->row_scale,
                       static_cast<const uint8_t*>(w->w_int4.codes), w->w_int4.row_scale, y, y_dtype,
                       M, N, K, decision_dev, HDQ_PREC_INT8, s) != hipSuccess)
    return HDQ_ERR_HIP;
  if (dm) {
    if (launch_decoded_gemm(dm, *xq4, w->w_fp4, y, y_dtype, M, N, K, decision_dev, s) != hipSuccess)
      return HDQ_ERR_HIP;
  } else if (fp4_gemm_for(f)(static_cast<const uint8_t*>(xq4->codes), xq4->blk_scale, xq4->tensor_scale,
                             static_cast<const uint8_t*>(w->w_fp4.codes), w->w_fp4.blk_scale,
                             w->w_fp4.tensor_scale, y, y_dtype, M, N, K, decision_dev, HDQ_PREC_NVFP4,
                             s) != hipSuccess) {
    return HDQ_ERR_HIP;
  }
  return hip_status(launch_gemm_bf16(xb, wb, y, y_dtype, M, N, K, decision_dev, HDQ_PREC_BF16, s));
}

static_assert(HDQ_DELTA_CHUNK == kDeltaChunk && HDQ_DELTA_MAX_SLICES == kDeltaMaxSlices,
              "the header's chunk size and slice count are the kernel's");

int hdq_linear_dispatch_delta(const int32_t* decision_dev, const void* x, const hdq_qtensor* xq8,
                              const hdq_qtensor* xq4, int64_t M, int64_t K, const hdq_weights* w,
                              void* y, int32_t y_dtype, const hdq_delta_slice* slices,
                              int32_t nslices, uint32_t* queue_dev, void* stream) {
  if (nslices < 0 || nslices > HDQ_DELTA_MAX_SLICES) return HDQ_ERR_SHAPE;
  if (nslices > 0 && (slices == nullptr || queue_dev == nullptr)) return HDQ_ERR_INVALID;
  DeltaWork dw{};
  dw.queue = queue_dev;
  for (int i = 0; i < nslices; ++i) {
    const hdq_delta_slice& q = slices[i];
    if (q.prev_in == nullptr || q.prev_out == nullptr || q.partials == nullptr) return HDQ_ERR_INVALID;
    if (q.numel <= 0 || q.numel % 8 != 0 || q.numel > ((int64_t)1 << 40)) return HDQ_ERR_SHAPE;
    if ((reinterpret_cast<uintptr_t>(q.prev_in) | reinterpret_cast<uintptr_t>(q.prev_out)) % 16 != 0)
      return HDQ_ERR_SHAPE;
    const int64_t nchunks = (q.numel + HDQ_DELTA_CHUNK - 1) / HDQ_DELTA_CHUNK;
    if (q.chunk_begin < 0 || q.chunk_end > nchunks || q.chunk_begin > q.chunk_end) return HDQ_ERR_SHAPE;
    dw.s[i] = DeltaSlice{static_cast<const uint16_t*>(q.prev_in), static_cast<const uint16_t*>(q.prev_out),
                         q.numel, q.chunk_begin, q.chunk_end, q.partials};
    dw.total += q.chunk_end - q.chunk_begin;
  }
  dw.n = nslices;
  if (dw.total > 0x7fffffff) return HDQ_ERR_SHAPE;
  // one workgroup per CU: the pipelined bodies' LDS admits no second one
  int dev = 0, cus = 256;
  if (hipGetDevice(&dev) != hipSuccess ||
      hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus < 1)
    cus = 256;
  dw.delta_wgs = (int)(dw.total < cus ? dw.total : cus);
  if (decision_dev == nullptr || x == nullptr || xq8 == nullptr || xq4 == nullptr || w == nullptr ||
      y == nullptr)
    return HDQ_ERR_INVALID;
  if (y_dtype != HDQ_DTYPE_F32 && y_dtype != HDQ_DTYPE_BF16) return HDQ_ERR_UNSUPPORTED;
  if (M <= 0 || K <= 0 || w->N <= 0 || M > 0x7fffffff || K > 0x7fffffff || w->N > 0x7fffffff)
    return HDQ_ERR_SHAPE;
  if (w->K != K) return HDQ_ERR_SHAPE;
  const int64_t N = w->N;
  const int32_t f = w->w_fp4.fmt;
  int st;
  if ((st = check_qtensor(w->w_int4, HDQ_FMT_INT4_ROW, N, K)) != HDQ_OK) return st;
  if ((st = check_qtensor(*xq8, HDQ_FMT_INT8_ROW, M, K)) != HDQ_OK) return st;
  if (!is_fp4(f)) return HDQ_ERR_UNSUPPORTED;
  if ((st = check_qtensor(w->w_fp4, f, N, K)) != HDQ_OK) return st;
  if ((st = check_qtensor(*xq4, f, M, K)) != HDQ_OK) return st;
  if (w->w_bf16 == nullptr) return HDQ_ERR_INVALID;
  if (xq8->had_block != w->w_int4.had_block || xq4->had_block != w->w_fp4.had_block) return HDQ_ERR_SHAPE;
  // the one-launch kernel only (the difference runs on its extra workgroups)
  if (K % 256 != 0 || M * 2 * K >= (1ll << 31) || N * 2 * K >= (1ll << 31)) return HDQ_ERR_SHAPE;
  hipStream_t s = static_cast<hipStream_t>(stream);
  const int dm = decoded_mode(f, *xq4, w->w_fp4, M, N, K);
  return hip_status(launch_gemm_dispatch(
      decision_dev, static_cast<const int8_t*>(xq8->codes), xq8->row_scale,
      static_cast<const uint8_t*>(w->w_int4.codes), w->w_int4.row_scale,
      static_cast<const uint8_t*>(dm ? xq4->dec : xq4->codes), xq4->blk_scale, xq4->tensor_scale,
      static_cast<const uint8_t*>(dm == kNvfp4Decoded ? w->w_fp4.dec : w->w_fp4.codes), w->w_fp4.blk_scale,
      w->w_fp4.tensor_scale, dm ? dm : f, static_cast<const uint16_t*>(x),
      static_cast<const uint16_t*>(w->w_bf16), y, y_dtype, M, N, K, s, &dw));
}

// ---- DeltaQuant ----------------------------------------------------------
static bool dq_grid(const hdq_dq_grid* g, DqGrid& d) {
  if (g == nullptr || g->frames <= 0 || g->height <= 0 || g->width <= 0 || g->cube_f <= 0 || g->cube_h <= 0 ||
      g->cube_w <= 0 || g->frames * g->height * g->width > 0x7fffffff ||
      (int64_t)g->cube_f * g->cube_h * g->cube_w > kDqMaxCube)
    return false;
  d.F = (int)g->frames;
  d.H = (int)g->height;
  d.W = (int)g->width;
  d.cf = g->cube_f;
  d.ch = g->cube_h;
  d.cw = g->cube_w;
  d.nF = (d.F + d.cf - 1) / d.cf;
  d.nH = (d.H + d.ch - 1) / d.ch;
  d.nW = (d.W + d.cw - 1) / d.cw;
  return true;
}

int64_t hdq_dq_cubes(const hdq_dq_grid* g) {
  DqGrid d;
  if (!dq_grid(g, d)) return -1;
  return (int64_t)d.nF * d.nH * d.nW;
}

int hdq_dq_quantize(const void* x, int64_t K, const hdq_dq_grid* g, int32_t fmt, uint8_t* core_codes,
                    float* core_scale, void* core_bf16, hdq_qtensor* delta, void* ws, size_t ws_bytes,
                    void* stream) {
  if (x == nullptr || core_codes == nullptr || core_scale == nullptr || delta == nullptr) return HDQ_ERR_INVALID;
  if (!is_fp4(fmt)) return HDQ_ERR_UNSUPPORTED;
  DqGrid d;
  if (!dq_grid(g, d)) return HDQ_ERR_SHAPE;
  const int64_t M = (int64_t)d.F * d.H * d.W;
  if (K <= 0 || K % 32 != 0 || K > 32768 || M * K / 8 >= (1ll << 31)) return HDQ_ERR_SHAPE;
  if (delta->fmt != fmt || delta->had_block != 1 || delta->rows != M || delta->cols != K) return HDQ_ERR_SHAPE;
  if (delta->codes == nullptr || delta->blk_scale == nullptr || delta->tensor_scale == nullptr)
    return HDQ_ERR_INVALID;
  if (ws == nullptr || ws_bytes < 256) return HDQ_ERR_WORKSPACE;
  return hip_status(launch_dq_quantize(static_cast<const uint16_t*>(x), K, d, fmt, core_codes, core_scale,
                                       static_cast<uint16_t*>(core_bf16), static_cast<uint32_t*>(ws),
                                       static_cast<uint8_t*>(delta->codes), delta->blk_scale,
                                       delta->tensor_scale, static_cast<hipStream_t>(stream)));
}

int hdq_dq_decode_weights(const hdq_qtensor* w_fp4, void* w_dec, void* stream) {
  if (w_fp4 == nullptr || w_dec == nullptr) return HDQ_ERR_INVALID;
  if (!is_fp4(w_fp4->fmt)) return HDQ_ERR_UNSUPPORTED;
  int st;
  if ((st = check_qtensor(*w_fp4, w_fp4->fmt, w_fp4->rows, w_fp4->cols)) != HDQ_OK) return st;
  if (w_fp4->cols % 16 != 0) return HDQ_ERR_SHAPE;
  return hip_status(launch_dq_decode_w(static_cast<const uint8_t*>(w_fp4->codes), w_fp4->blk_scale, w_fp4->rows,
                                       w_fp4->cols, static_cast<uint16_t*>(w_dec), static_cast<hipStream_t>(stream)));
}

size_t hdq_dq_linear_workspace_bytes(const hdq_dq_grid* g, int64_t K, int64_t N, int32_t fmt) {
  DqGrid d;
  if (!dq_grid(g, d) || K <= 0 || N <= 0 || !is_fp4(fmt)) return 0;
  const int64_t M = (int64_t)d.F * d.H * d.W, C = (int64_t)d.nF * d.nH * d.nW;
  return dq_linear_ws(M, C, N, K, fmt);
}

int hdq_dq_linear(const hdq_dq_grid* g, const uint8_t* core_codes, const void* core_bf16, const float* core_scale,
                  const hdq_qtensor* delta, const hdq_qtensor* w_fp4, const void* w_dec, void* y, int32_t y_dtype,
                  void* ws, size_t ws_bytes, void* stream) {
  if (core_scale == nullptr || delta == nullptr || w_fp4 == nullptr || y == nullptr) return HDQ_ERR_INVALID;
  if (y_dtype != HDQ_DTYPE_F32 && y_dtype != HDQ_DTYPE_BF16) return HDQ_ERR_UNSUPPORTED;
  DqGrid d;
  if (!dq_grid(g, d)) return HDQ_ERR_SHAPE;
  const int64_t M = (int64_t)d.F * d.H * d.W, C = (int64_t)d.nF * d.nH * d.nW;
  const int64_t K = delta->cols, N = w_fp4->rows;
  if (!is_fp4(delta->fmt) || w_fp4->fmt != delta->fmt) return HDQ_ERR_UNSUPPORTED;
  int st;
  if ((st = check_qtensor(*delta, delta->fmt, M, K)) != HDQ_OK) return st;
  if ((st = check_qtensor(*w_fp4, delta->fmt, N, K)) != HDQ_OK) return st;
  if (delta->had_block != 1 || w_fp4->had_block != 1 || K % 32 != 0 || N % 4 != 0 || N > 0x7fffffff)
    return HDQ_ERR_SHAPE;
  // the core GEMM: FP8 codes x FP4 weights when the weights' block scales are
  // powers of two, else the bf16 code values x the decoded weights
  const bool fp8_core = dq_core_fp8_applies(delta->fmt, C, N, K);
  if (fp8_core ? core_codes == nullptr : (core_bf16 == nullptr || w_dec == nullptr)) return HDQ_ERR_INVALID;
  if (ws == nullptr || ws_bytes < dq_linear_ws(M, C, N, K, delta->fmt)) return HDQ_ERR_WORKSPACE;
  hipStream_t s = static_cast<hipStream_t>(stream);
  // the core GEMM's output first; the combine route's difference output after it
  float* yc = static_cast<float*>(ws);
  float* yd = reinterpret_cast<float*>(static_cast<uint8_t*>(ws) + align_up((size_t)C * (size_t)N * 4));
  // the core GEMM, then (MX and P2 formats, K % 256 == 0) the difference GEMM
  // with the broadcast core term added in its epilogue
  const hipError_t ce =
      fp8_core ? launch_gemm_dq_core(core_codes, static_cast<const uint8_t*>(w_fp4->codes), w_fp4->blk_scale,
                                     delta->fmt, yc, C, N, K, s)
               : launch_gemm_bf16(static_cast<const uint16_t*>(core_bf16), static_cast<const uint16_t*>(w_dec), yc,
                                  HDQ_DTYPE_F32, C, N, K, nullptr, HDQ_PREC_BF16, s);
  if (ce != hipSuccess) return HDQ_ERR_HIP;
  const CoreAdd add{yc, core_scale, w_fp4->tensor_scale, d};
  const hipError_t fe = launch_gemm_fp4_core_add(
      static_cast<const uint8_t*>(delta->codes), delta->blk_scale, delta->tensor_scale,
      static_cast<const uint8_t*>(w_fp4->codes), w_fp4->blk_scale, w_fp4->tensor_scale, delta->fmt, add, y, y_dtype,
      M, N, K, s);
  if (fe == hipSuccess) return HDQ_OK;
  // the workspace was sized for the fused route when it applies: never fall
  // back to the combine route (whose fp32 output would not fit) there
  if (fe != hipErrorNotSupported || fp4_core_add_applies(delta->fmt, M, N, K)) return HDQ_ERR_HIP;
  if (fp4_gemm_for(delta->fmt)(static_cast<const uint8_t*>(delta->codes), delta->blk_scale, delta->tensor_scale,
                               static_cast<const uint8_t*>(w_fp4->codes), w_fp4->blk_scale, w_fp4->tensor_scale,
                               yd, HDQ_DTYPE_F32, M, N, K, nullptr, HDQ_PREC_NVFP4, s) != hipSuccess)
    return HDQ_ERR_HIP;
  return hip_status(launch_dq_combine(yd, yc, core_scale, w_fp4->tensor_scale, d, N, y, y_dtype, s));
}

int hdq_quantize(const void* x, int64_t rows, int64_t cols, int32_t had_block, int32_t fmt,
                 const float* tensor_amax, const int32_t* decision_dev, hdq_qtensor* out,
                 void* ws, size_t ws_bytes, void* stream) {
  if (x == nullptr || out == nullptr || !valid_fmt(fmt)) return HDQ_ERR_INVALID;
  if (decision_dev != nullptr && fmt == HDQ_FMT_INT4_ROW) return HDQ_ERR_UNSUPPORTED;
  int st = check_quant_shape(rows, cols, had_block, fmt);
  if (st != HDQ_OK) return st;
  hdq_qtensor q = *out;
  q.fmt = fmt;
  q.had_block = had_block;
  q.rows = rows;
  q.cols = cols;
  if ((st = check_qtensor(q, fmt, rows, cols)) != HDQ_OK) return st;
  if (is_fp4(fmt) && tensor_amax == nullptr &&
      (ws == nullptr || ws_bytes < amax_prepass_bytes()))
    return HDQ_ERR_WORKSPACE;
  *out = q;
  const int32_t want = is_fp4(fmt) ? HDQ_PREC_NVFP4 : HDQ_PREC_INT8;
  return hip_status(enqueue_quantize(x, q, is_fp4(fmt) ? tensor_amax : nullptr,
                                     static_cast<uint8_t*>(ws), decision_dev, want,
                                     static_cast<hipStream_t>(stream)));
}

int hdq_linear(int32_t precision, const int32_t* decision_dev, const void* x,
               const hdq_qtensor* xq, const float* x_amax, int64_t M, int64_t K,
               const hdq_weights* w, void* y, int32_t y_dtype, void* ws, size_t ws_bytes,
               void* stream) {
  if (w == nullptr || y == nullptr) return HDQ_ERR_INVALID;
  if (precision < -1 || precision > HDQ_PREC_BF16) return HDQ_ERR_INVALID;
  if (y_dtype < HDQ_DTYPE_F32 || y_dtype > HDQ_DTYPE_I32) return HDQ_ERR_INVALID;
  if (precision == -1 && (decision_dev == nullptr || xq != nullptr)) return HDQ_ERR_INVALID;
  if (precision == HDQ_PREC_BF16 && xq != nullptr) return HDQ_ERR_UNSUPPORTED;
  if (M <= 0 || K <= 0 || w->N <= 0 || M > 0x7fffffff || K > 0x7fffffff || w->N > 0x7fffffff)
    return HDQ_ERR_SHAPE;
  if (w->K != K) return HDQ_ERR_SHAPE;
  const int64_t N = w->N;
  const bool run_int8 = precision == HDQ_PREC_INT8 || precision == -1;
  const bool run_fp4 = precision == HDQ_PREC_NVFP4 || precision == -1;
  const bool run_bf16 = precision == HDQ_PREC_BF16 || precision == -1;
  if (y_dtype == HDQ_DTYPE_I32 && (run_fp4 || run_bf16)) return HDQ_ERR_UNSUPPORTED;
  if (xq == nullptr && x == nullptr) return HDQ_ERR_INVALID;
  int st;
  // Weights and activation descriptors for every path that may run.
  if (run_int8) {
    if ((st = check_qtensor(w->w_int4, HDQ_FMT_INT4_ROW, N, K)) != HDQ_OK) return st;
    if (K % 32 != 0 || K % w->w_int4.had_block != 0) return HDQ_ERR_SHAPE;
    if (xq != nullptr) {
      if ((st = check_qtensor(*xq, HDQ_FMT_INT8_ROW, M, K)) != HDQ_OK) return st;
      if (xq->had_block != w->w_int4.had_block) return HDQ_ERR_SHAPE;
    }
  }
  if (run_fp4) {
    const int32_t f = w->w_fp4.fmt;
    if (!is_fp4(f)) return HDQ_ERR_UNSUPPORTED;
    if ((st = check_qtensor(w->w_fp4, f, N, K)) != HDQ_OK) return st;
    if (K % 32 != 0 || K % w->w_fp4.had_block != 0) return HDQ_ERR_SHAPE;
    if (xq != nullptr) {
      if ((st = check_qtensor(*xq, f, M, K)) != HDQ_OK) return st;
      if (xq->had_block != w->w_fp4.had_block) return HDQ_ERR_SHAPE;
    }
  }
  if (run_bf16) {
    if (w->w_bf16 == nullptr || x == nullptr) return HDQ_ERR_INVALID;
    if (K % 8 != 0) return HDQ_ERR_SHAPE;
  }
  if (run_int8 && run_fp4 && w->w_int4.had_block != w->w_fp4.had_block) return HDQ_ERR_SHAPE;
  // Workspace.
  size_t need = 0;
  if (xq == nullptr) {
    if (run_int8) need += qtensor_bytes(M, K, HDQ_FMT_INT8_ROW);
    if (run_fp4) need += qtensor_bytes(M, K, w->w_fp4.fmt) + (x_amax ? 0 : amax_prepass_bytes());
  }
  if (need > 0 && (ws == nullptr || ws_bytes < need)) return HDQ_ERR_WORKSPACE;

  hipStream_t s = static_cast<hipStream_t>(stream);
  const int32_t* gate = decision_dev;  // -1: selects the path; fixed P: run only if P
  uint8_t* cursor = static_cast<uint8_t*>(ws);
  hipError_t e;
  if (run_int8) {
    hdq_qtensor q;
    if (xq != nullptr) {
      q = *xq;
    } else {
      q.fmt = HDQ_FMT_INT8_ROW;
      q.had_block = w->w_int4.had_block;
      q.rows = M;
      q.cols = K;
      q.codes = cursor;
      q.row_scale = reinterpret_cast<float*>(cursor + align_up((size_t)(M * K)));
      q.blk_scale = nullptr;
      q.tensor_scale = nullptr;
      q.dec = nullptr;
      cursor += qtensor_bytes(M, K, HDQ_FMT_INT8_ROW);
      if ((st = check_quant_shape(M, K, q.had_block, q.fmt)) != HDQ_OK) return st;
      if ((e = enqueue_quantize(x, q, nullptr, nullptr, gate, HDQ_PREC_INT8, s)) != hipSuccess)
        return HDQ_ERR_HIP;
    }
    e = launch_gemm_i8i4(static_cast<const int8_t*>(q.codes), q.row_scale,
                         static_cast<const uint8_t*>(w->w_int4.codes), w->w_int4.row_scale, y,
                         y_dtype, M, N, K, gate, HDQ_PREC_INT8, s);
    if (e != hipSuccess) return HDQ_ERR_HIP;
  }
  if (run_fp4) {
    const int32_t f = w->w_fp4.fmt;
    hdq_qtensor q;
    if (xq != nullptr) {
      q = *xq;
    } else {
      q.fmt = f;
      q.had_block = w->w_fp4.had_block;
      q.rows = M;
      q.cols = K;
      q.codes = cursor;
      q.blk_scale = cursor + align_up((size_t)(M * K / 2));
      q.tensor_scale = reinterpret_cast<float*>(q.blk_scale + align_up((size_t)(M * K / 16)));
      q.row_scale = nullptr;
      q.dec = nullptr;
      cursor += qtensor_bytes(M, K, f);
      uint8_t* pre = nullptr;
      if (x_amax == nullptr) {
        pre = cursor;
        cursor += amax_prepass_bytes();
      }
      if ((st = check_quant_shape(M, K, q.had_block, q.fmt)) != HDQ_OK) return st;
      if ((e = enqueue_quantize(x, q, x_amax, pre, gate, HDQ_PREC_NVFP4, s)) != hipSuccess)
        return HDQ_ERR_HIP;
    }
    const uint8_t* xc = static_cast<const uint8_t*>(q.codes);
    const uint8_t* wc = static_cast<const uint8_t*>(w->w_fp4.codes);
    if (const int dm = decoded_mode(f, q, w->w_fp4, M, N, K))
      e = launch_decoded_gemm(dm, q, w->w_fp4, y, y_dtype, M, N, K, gate, s);
    else
      e = fp4_gemm_for(f)(xc, q.blk_scale, q.tensor_scale, wc, w->w_fp4.blk_scale, w->w_fp4.tensor_scale,
                          y, y_dtype, M, N, K, gate, HDQ_PREC_NVFP4, s);
    if (e != hipSuccess) return HDQ_ERR_HIP;
  }
  if (run_bf16) {
    e = launch_gemm_bf16(static_cast<const uint16_t*>(x), static_cast<const uint16_t*>(w->w_bf16), y,
                         y_dtype, M, N, K, gate, HDQ_PREC_BF16, s);
    if (e != hipSuccess) return HDQ_ERR_HIP;
  }
  return HDQ_OK;
}

}  // extern "C"
