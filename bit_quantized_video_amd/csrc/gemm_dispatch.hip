// gemm_dispatch.hip -- the quantized linear's GEMM in one launch for whichever
// precision the device-side decision names (gfx950).
//
// The selection of 6Bit-Diffusion (summary on vetunion.cn, sections one and
// three) picks INT8, NVFP4 or full precision per layer and step.  With the
// decision on the device, enqueuing one gated kernel per precision costs two
// launches that only read the decision and exit; each must still wait for a
// whole CU's worth of resources.  This kernel reads the decision once and
// runs the one pipelined GEMM body it names, so a layer call launches one
// GEMM.  The bodies are the gated kernels' own (gemm_*_pipe.h), so results
// are bit-identical to them.  Registers and LDS are the largest body's.
#include "gemm_bf16_pipe.h"
#include "gemm_fp4_pipe.h"
#include "gemm_i8_pipe.h"
#include "hdq_device.h"
#include "hdq_internal.h"

namespace hdq {

// FP4: the NVFP4 weights' format (kNvfp4: the exact bf16-MFMA body; kNvfp4Mx,
// kNvfp4P2: the FP4 MFMA body, one or two passes).
template <int OUT, int FP4>
__global__ __launch_bounds__(512) void k_gemm_dispatch(
    const int32_t* __restrict__ decision, const int8_t* __restrict__ x8, const float* __restrict__ sx,
    const uint8_t* __restrict__ w4, const float* __restrict__ sw, const uint8_t* __restrict__ xc,
    const uint8_t* __restrict__ xsc, const float* __restrict__ xts, const uint8_t* __restrict__ wc,
    const uint8_t* __restrict__ wsc, const float* __restrict__ wts, const uint16_t* __restrict__ xb,
    const uint16_t* __restrict__ wb, void* __restrict__ Y, int M, int N, int K) {
  const int32_t d = __builtin_amdgcn_readfirstlane(*decision);  // uniform: a scalar branch
  if (d == kPrecInt8) {
    gemm_i8i4_pipe_body<2, 4, 4, 2, OUT>(x8, sx, w4, sw, Y, M, N, K);
  } else if (d == kPrecNvfp4) {
    if constexpr (FP4 != kNvfp4)
      gemm_fp4mx_pipe_body<OUT, FP4 == kNvfp4P2>(xc, xsc, xts, wc, wsc, wts, Y, M, N, K);
    else
      gemm_bf16_pipe_body<kSrcNvfp4, OUT>(xc, xsc, xts, wc, wsc, wts, Y, M, N, K);
  } else if (d == kPrecBf16) {
    gemm_bf16_pipe_body<kSrcBf16, OUT>(xb, nullptr, nullptr, wb, nullptr, nullptr, Y, M, N, K);
  }
}

template <int OUT, int FP4>
static hipError_t launch_dispatch_t(const int32_t* decision, const int8_t* x8, const float* sx,
                                    const uint8_t* w4, const float* sw, const uint8_t* xc,
                                    const uint8_t* xsc, const float* xts, const uint8_t* wc,
                                    const uint8_t* wsc, const float* wts, const uint16_t* xb,
                                    const uint16_t* wb, void* y, int64_t M, int64_t N, int64_t K,
                                    hipStream_t s) {
  // Dynamic LDS: the largest body's (INT8: three 48 KB stages; FP4: two
  // 68 or 72 KB stages; bf16: a 256 x 256 bf16 output tile of 528-byte rows).
  constexpr size_t fp4_lds = (size_t)fp4_pipe_lds<FP4 == kNvfp4P2>();
  constexpr size_t i8_lds = (size_t)I8Cfg<2, 4, 4, 2>::LDS;
  constexpr size_t lds0 = fp4_lds > kBf16PipeLds ? fp4_lds : kBf16PipeLds;
  constexpr size_t lds = i8_lds > lds0 ? i8_lds : lds0;
  auto kern = k_gemm_dispatch<OUT, FP4>;
  hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(kern),
                                     hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
  if (e != hipSuccess) return e;
  const int64_t tiles = ((M + 255) / 256) * ((N + 255) / 256);
  hipLaunchKernelGGL(kern, dim3((unsigned)persistent_grid(tiles)), dim3(512), lds, s, decision, x8, sx,
                     w4, sw, xc, xsc, xts, wc, wsc, wts, xb, wb, y, (int)M, (int)N, (int)K);
  return hipGetLastError();
}

hipError_t launch_gemm_dispatch(const int32_t* decision, const int8_t* x8, const float* sx,
                                const uint8_t* w4, const float* sw, const uint8_t* xc,
                                const uint8_t* xsc, const float* xts, const uint8_t* wc,
                                const uint8_t* wsc, const float* wts, int fp4_fmt,
                                const uint16_t* xb, const uint16_t* wb, void* y, int out_dtype,
                                int64_t M, int64_t N, int64_t K, hipStream_t s) {
  // Every body's pipelined kernel must apply: K a multiple of each stage's
  // depth (256 covers them all) and 32-bit buffer offsets (bf16 rows are the
  // widest, 2 K bytes).
  if (K % 256 != 0 || M * 2 * K >= (1ll << 31) || N * 2 * K >= (1ll << 31)) return hipErrorNotSupported;
  if (out_dtype != kOutF32 && out_dtype != kOutBf16) return hipErrorNotSupported;
#define HDQ_DISPATCH(O, F) \
  return launch_dispatch_t<O, F>(decision, x8, sx, w4, sw, xc, xsc, xts, wc, wsc, wts, xb, wb, y, M, N, K, s)
  if (out_dtype == kOutBf16) {
    if (fp4_fmt == kNvfp4Mx) HDQ_DISPATCH(kOutBf16, kNvfp4Mx);
    if (fp4_fmt == kNvfp4P2) HDQ_DISPATCH(kOutBf16, kNvfp4P2);
    HDQ_DISPATCH(kOutBf16, kNvfp4);
  }
  if (fp4_fmt == kNvfp4Mx) HDQ_DISPATCH(kOutF32, kNvfp4Mx);
  if (fp4_fmt == kNvfp4P2) HDQ_DISPATCH(kOutF32, kNvfp4P2);
  HDQ_DISPATCH(kOutF32, kNvfp4);
#undef HDQ_DISPATCH
}

}  // namespace hdq
