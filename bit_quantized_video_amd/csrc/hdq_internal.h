// hdq_internal.h -- host-side launchers of the libhdq kernels (internal).
//
// Each launcher enqueues on `stream` and returns hipGetLastError().  Shapes
// and pointers are validated by the C-ABI layer (capi.hip) before any
// launcher runs; the launchers only check what a launch geometry needs.
#pragma once

#include <hip/hip_runtime.h>

#include <atomic>
#include <stddef.h>
#include <stdint.h>

namespace hdq {

// Raises a kernel's dynamic LDS limit to `bytes` once per device (the
// attribute is set on the first launch on each device, not on every launch).
template <auto KERNEL>
hipError_t set_dynamic_lds_once(size_t bytes) {
  static std::atomic<uint64_t> done{0};  // one bit per device index below 64
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) dev = 0;
  const uint64_t bit = (dev >= 0 && dev < 64) ? (1ull << dev) : 0ull;
  if (bit != 0 && (done.load(std::memory_order_acquire) & bit)) return hipSuccess;
  const hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(KERNEL),
                                           hipFuncAttributeMaxDynamicSharedMemorySize, (int)bytes);
  if (e == hipSuccess && bit != 0) done.fetch_or(bit, std::memory_order_release);
  return e;
}


// Difference sums run by extra workgroups of a GEMM launch (gemm_dispatch.hip).
// A slice is the chunk range [c0, c1) of one pair of previous-step tensors;
// chunk c covers elements [c * kDeltaChunk, (c + 1) * kDeltaChunk) and its
// {sum |out - in|, sum |in|} go to parts[2c], parts[2c + 1].
constexpr int64_t kDeltaChunk = 65536;
constexpr int kDeltaMaxSlices = 4;
struct DeltaSlice {
  const uint16_t* in;
  const uint16_t* out;
  int64_t numel;
  int64_t c0, c1;
  double* parts;
};
struct DeltaWork {
  DeltaSlice s[kDeltaMaxSlices];
  int n;               // slices
  int64_t total;       // chunks over all slices
  uint32_t* queue;     // {next chunk, workgroups done}: zero on entry and on exit
  int delta_wgs;       // workgroups after the GEMM's
};

enum QFmt : int { kInt8Row = 0, kInt4Row = 1, kNvfp4 = 2, kNvfp4Mx = 3, kNvfp4P2 = 4 };
// The one-launch GEMM's NVFP4 body for plain NVFP4 operands given decoded to
// bf16 (not a tensor format).
constexpr int kNvfp4Decoded = 16;
// ... with only the activations decoded (the weights' codes decoded in the GEMM).
constexpr int kNvfp4XDecoded = 17;
enum Prec : int { kPrecNvfp4 = 0, kPrecInt8 = 1, kPrecBf16 = 2 };
enum OutDtype : int { kOutF32 = 0, kOutBf16 = 1, kOutI32 = 2 };

// fl32(1/sqrt(hb)): 2^-k/2 exactly for even log2(hb), otherwise the float
// nearest 1/sqrt(hb).
float hadamard_scale(int hb);

// Grid of a persistent GEMM whose workgroups fill a CU each: `tiles` when
// that is at most the workgroups it may use, else that number -- the
// current device's CU count rounded down to a multiple of 8, less 16 CUs
// left free for other streams (HDQ_GEMM_FREE_CUS) -- and the workgroups
// loop over tiles.
int64_t persistent_grid(int64_t tiles);

// ---- quantize (quant.hip) ----
// INT8 / INT4 per-row: codes int8 [rows, cols] or packed uint8 [rows, cols/2],
// row_scale fp32 [rows].
hipError_t launch_quant_int_rows(const uint16_t* x, int64_t rows, int64_t cols, int hb, int fmt,
                                 void* codes, float* row_scale, const int32_t* decision,
                                 int32_t want, hipStream_t s);
// NVFP4 / NVFP4_MX: codes uint8 [rows, cols/2], blk_scale uint8 [rows, cols/16],
// tensor_scale fp32 [1]; amax = device fp32[1] rotated tensor amax; dec:
// null, or bf16 [rows, cols] for the codes' exact values.
hipError_t launch_quant_nvfp4(const uint16_t* x, int64_t rows, int64_t cols, int hb, int fmt,
                              const float* amax, uint8_t* codes, uint8_t* blk_scale,
                              float* tensor_scale, const int32_t* decision, int32_t want,
                              hipStream_t s, uint16_t* dec = nullptr);

// ---- statistics (stats.hip) ----
constexpr int kStatsMaxBlocks = 1024;
constexpr size_t kStatsPartialBytes = (size_t)kStatsMaxBlocks * 6 * sizeof(double);
// Partial sums over prev_in/prev_out (may be null) and cur (may be null with
// cur_numel 0), then a one-block finalize that writes the five statistics,
// the decision and/or the rotated amax (any output pointer may be null).
// delta_sums_out (double[2]): write only the difference sums.  delta_sums_in
// (double[2 * delta_parts]): take the difference sums from there (history
// present), the pairs summed in order.
hipError_t launch_stats(const uint16_t* prev_in, const uint16_t* prev_out, int64_t prev_numel,
                        const uint16_t* cur, int64_t cur_numel, int hb, float delta_thresh,
                        float ratio_thresh, int32_t* decision, float* stats, float* amax_out,
                        double* partials, const int32_t* gate, int32_t want, hipStream_t s,
                        const double* delta_sums_in = nullptr, double* delta_sums_out = nullptr,
                        int64_t delta_parts = 1);

// The finalize over one partial per row, struct-of-arrays: psum = sum |x|,
// pbits = max bf16 magnitude bits, ptmax = max |rotated x| (scaled).
// Temporal delta cache skip rule over n modules.
// parts_off (device int64 [n + 1]) or null: module i's change sums are the
// pairs [parts_off[i], parts_off[i + 1]) of sums, else sums[i].
hipError_t launch_tdc_decide(const double* sums, const int64_t* parts_off, const int32_t* state, float* c,
                             float* acc, int32_t* skip, int64_t n, float tau_skip, float tau_acc,
                             hipStream_t s);
hipError_t launch_stats_finalize_rows(const double* psum, const uint32_t* pbits, const float* ptmax,
                                      int64_t rows, int64_t cur_numel, int hb, float delta_thresh,
                                      float ratio_thresh, int32_t* decision, float* stats,
                                      const double* delta_sums_in, int64_t delta_parts, hipStream_t s);
// INT8 per-row quantization that also writes those per-row partials;
// cols <= 16384.
hipError_t launch_quant_int8_stats(const uint16_t* x, int64_t rows, int64_t cols, int hb, void* codes,
                                   float* row_scale, double* psum, uint32_t* pbits, float* ptmax,
                                   hipStream_t s);

// ---- GEMMs ----
// INT8 activations [M, K] x INT4 weights packed [N, K/2]: y = (acc*sx)*sw.
hipError_t launch_gemm_i8i4(const int8_t* x, const float* sx, const uint8_t* w4, const float* sw,
                            void* y, int out_dtype, int64_t M, int64_t N, int64_t K,
                            const int32_t* decision, int32_t want, hipStream_t s);
// NVFP4 x NVFP4 decoded exactly to bf16 on the fly, bf16 MFMA.
hipError_t launch_gemm_nvfp4_bf16(const uint8_t* xc, const uint8_t* xs, const float* xts,
                                  const uint8_t* wc, const uint8_t* ws, const float* wts,
                                  void* y, int out_dtype, int64_t M, int64_t N, int64_t K,
                                  const int32_t* decision, int32_t want, hipStream_t s);
// The same product from operands decoded exactly to bf16 beforehand (xd, wd:
// bf16 [M, K], [N, K]): the bf16 GEMM body with the tensor scales.  Only
// where the pipelined bf16 body takes the shape (nvfp4_decoded_applies; it
// then runs the exact NVFP4 kernel's MFMAs in its order): otherwise
// hipErrorNotSupported.
bool nvfp4_decoded_applies(int64_t M, int64_t N, int64_t K);
// Only the activations decoded beforehand (xd: bf16 [M, K]); the weights'
// codes are decoded in the GEMM as the exact kernel does.  Pipelined shapes
// only (nvfp4_xdecoded_applies), else hipErrorNotSupported.
bool nvfp4_xdecoded_applies(int64_t M, int64_t N, int64_t K);
hipError_t launch_gemm_nvfp4_xdecoded(const uint16_t* xd, const float* xts, const uint8_t* wc,
                                      const uint8_t* ws, const float* wts, void* y, int out_dtype, int64_t M,
                                      int64_t N, int64_t K, const int32_t* decision, int32_t want, hipStream_t s);
hipError_t launch_gemm_nvfp4_decoded(const uint16_t* xd, const float* xts, const uint16_t* wd,
                                     const float* wts, void* y, int out_dtype, int64_t M, int64_t N,
                                     int64_t K, const int32_t* decision, int32_t want, hipStream_t s);
// MX-compatible NVFP4 on the block-scaled FP4 MFMA.
hipError_t launch_gemm_nvfp4_mx(const uint8_t* xc, const uint8_t* xs, const float* xts,
                                const uint8_t* wc, const uint8_t* ws, const float* wts,
                                void* y, int out_dtype, int64_t M, int64_t N, int64_t K,
                                const int32_t* decision, int32_t want, hipStream_t s);
// NVFP4 with a power-of-two scale per 16-block: the FP4 MFMA in two passes.
hipError_t launch_gemm_nvfp4_p2(const uint8_t* xc, const uint8_t* xs, const float* xts,
                                const uint8_t* wc, const uint8_t* ws, const float* wts,
                                void* y, int out_dtype, int64_t M, int64_t N, int64_t K,
                                const int32_t* decision, int32_t want, hipStream_t s);
// One launch running the GEMM the device decision names (INT8, NVFP4 -- on
// the FP4 MFMA when fp4_mx, else decoded to bf16 -- or bf16); every path's
// operands must be given.  hipErrorNotSupported when a shape does not fit
// the pipelined bodies (callers then launch the three gated GEMMs).
hipError_t launch_gemm_dispatch(const int32_t* decision, const int8_t* x8, const float* sx,
                                const uint8_t* w4, const float* sw, const uint8_t* xc,
                                const uint8_t* xsc, const float* xts, const uint8_t* wc,
                                const uint8_t* wsc, const float* wts, int fp4_fmt,
                                const uint16_t* xb, const uint16_t* wb, void* y, int out_dtype,
                                int64_t M, int64_t N, int64_t K, hipStream_t s,
                                const struct DeltaWork* delta = nullptr);
// DeltaQuant cube-delta quantization: the token grid (frame outermost), the
// cube size and the cube grid.
struct DqGrid {
  int F, H, W, cf, ch, cw, nF, nH, nW;
};
constexpr int kDqMaxCube = 256;  // tokens per cube (one per thread of a workgroup)
// Cube of token m.
__device__ __forceinline__ int dq_cube(int m, const DqGrid& g) {
  const int hw = g.H * g.W, f = m / hw, r = m - f * hw, h = r / g.W, w = r - h * g.W;
  return ((f / g.cf) * g.nH + h / g.ch) * g.nW + w / g.cw;
}
// The broadcast core term an NVFP4 GEMM adds to its output:
// y[m, n] += fl32(fl32(yc[cube(m), n] * cs[cube(m)]) * wts[0]).
struct CoreAdd {
  const float* yc;
  const float* cs;
  const float* wts;
  DqGrid g;
};
// Core tokens (codes, scales, optional bf16 code values) and the differences
// in NVFP4 format fmt; damax_bits: device uint32 scratch.
hipError_t launch_dq_quantize(const uint16_t* x, int64_t K, const DqGrid& g, int fmt, uint8_t* ccodes,
                              float* cscale, uint16_t* core_bf16, uint32_t* damax_bits, uint8_t* codes,
                              uint8_t* blk_scale, float* tensor_scale, hipStream_t s);
// NVFP4 weights [N, K] to bf16 E2M1 x block-scale values.
hipError_t launch_dq_decode_w(const uint8_t* codes, const uint8_t* blk, int64_t N, int64_t K, uint16_t* out,
                              hipStream_t s);
// Whether launch_gemm_fp4_core_add takes a shape: the pipelined FP4 body
// (MX or per-16 power-of-two format, K % 256 == 0, 32-bit operand offsets)
// with N % 4 == 0.
inline bool fp4_core_add_applies(int fmt, int64_t M, int64_t N, int64_t K) {
  return (fmt == kNvfp4Mx || fmt == kNvfp4P2) && K % 256 == 0 && M * K / 2 < (1ll << 31) &&
         N * K / 2 < (1ll << 31) && N % 4 == 0;
}
// Whether launch_gemm_dq_core takes a shape: weights with power-of-two
// block scales (MX or per-16 format), K % 128 == 0, 32-bit operand offsets.
inline bool dq_core_fp8_applies(int fmt, int64_t C, int64_t N, int64_t K) {
  return (fmt == kNvfp4Mx || fmt == kNvfp4P2) && K % 128 == 0 && C * K < (1ll << 31) && N * K / 2 < (1ll << 31);
}
// DeltaQuant's core GEMM: yc [C, N] fp32 = E4M3 core codes [C, K] times the
// NVFP4 weights' E2M1 codes with their power-of-two block scales (tensor
// scale left out), on the FP8 x FP4 scaled MFMA; hipErrorNotSupported for
// shapes dq_core_fp8_applies rejects.
hipError_t launch_gemm_dq_core(const uint8_t* core, const uint8_t* wc, const uint8_t* ws, int fmt, float* yc,
                               int64_t C, int64_t N, int64_t K, hipStream_t s);
// NVFP4-MX / P2 GEMM (pipelined shapes: K % 256 == 0) whose output also
// gets the broadcast core term; hipErrorNotSupported for other shapes.
hipError_t launch_gemm_fp4_core_add(const uint8_t* xc, const uint8_t* xs, const float* xts, const uint8_t* wc,
                                    const uint8_t* ws, const float* wts, int fmt, const CoreAdd& add, void* y,
                                    int out_dtype, int64_t M, int64_t N, int64_t K, hipStream_t s);
// y = yd + (yc of the token's cube) x s_c x s_tw (N a multiple of 4).
hipError_t launch_dq_combine(const float* yd, const float* yc, const float* cscale, const float* wts,
                             const DqGrid& g, int64_t N, void* y, int out_dtype, hipStream_t s);
// bf16 x bf16 (full-precision fallback).
hipError_t launch_gemm_bf16(const uint16_t* x, const uint16_t* w, void* y, int out_dtype,
                            int64_t M, int64_t N, int64_t K, const int32_t* decision,
                            int32_t want, hipStream_t s);

}  // namespace hdq
