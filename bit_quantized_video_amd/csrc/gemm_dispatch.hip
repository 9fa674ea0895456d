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
//
// Optionally the launch also computes difference statistics (summary on
// vetunion.cn, section one: the previous step's input/output difference)
// for later layer calls, on workgroups appended after the GEMM's persistent
// ones.  While the GEMM runs they hold the CUs the GEMM leaves free; as its
// workgroups retire, the waiting ones take their CUs.  They claim chunks
// from a queue, so the chunks left when the GEMM ends run on the whole GPU,
// inside this launch rather than beside the memory-bound passes that follow.
#include "gemm_bf16_pipe.h"
#include "gemm_fp4_pipe.h"
#include "gemm_i8_pipe.h"
#include "hdq_device.h"
#include "hdq_internal.h"

namespace hdq {

// One difference workgroup (512 threads): claims chunks until the queue is
// empty; per chunk, {sum |out - in|, sum |in|} in a fixed order (float over
// each 8 elements, double across a thread's vectors, then a fixed tree), so
// a chunk's partials do not depend on which workgroup ran it.  The last
// workgroup to finish resets the queue.  (Each workgroup's last claim
// returned before it counts itself done, so no claim follows the reset.)
__device__ __forceinline__ void delta_workgroup(const DeltaWork& dw, uint8_t* smem) {
  constexpr int T = 512, U = 8;  // threads; 16-byte vectors per thread and pass
  constexpr int64_t VPC = kDeltaChunk / 8;  // vectors per chunk
  static_assert(VPC == 2 * U * T, "two passes of U vectors per thread cover a chunk");
  int64_t* s_claim = reinterpret_cast<int64_t*>(smem);
  double* s_red = reinterpret_cast<double*>(smem + 64);
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  // The loop's exit must be a scalar (uniform) branch: with a per-lane exit
  // test the compiler may split the loop so that lane 0's claim sits outside
  // the part holding the barriers, and the other lanes spin on a stale claim.
  const int wv = __builtin_amdgcn_readfirstlane(wave);
  for (;;) {
    if (wv == 0) {
      uint32_t v = 0u;
      if (lane == 0) v = atomicAdd(&dw.queue[0], 1u);
      v = __builtin_amdgcn_readfirstlane(v);
      if (lane == 0) *s_claim = (int64_t)v;
    }
    __syncthreads();
    const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)*s_claim);
    __syncthreads();
    int64_t q = (int64_t)lo;
    if (q >= dw.total) break;
    int si = 0;
    while (si + 1 < dw.n && q >= dw.s[si].c1 - dw.s[si].c0) {
      q -= dw.s[si].c1 - dw.s[si].c0;
      ++si;
    }
    si = __builtin_amdgcn_readfirstlane(si);
    const DeltaSlice sl = dw.s[si];
    const int64_t c = sl.c0 + q;
    const int64_t v0 = c * VPC, v1 = min(v0 + VPC, sl.numel >> 3);
    const uint4* a4 = reinterpret_cast<const uint4*>(sl.in);
    const uint4* o4 = reinterpret_cast<const uint4*>(sl.out);
    double diff = 0.0, base = 0.0;
#pragma unroll
    for (int pass = 0; pass < 2; ++pass) {
      uint4 ra[U], ro[U];
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const int64_t v = v0 + (int64_t)(pass * U + u) * T + tid;
        ra[u] = v < v1 ? a4[v] : make_uint4(0u, 0u, 0u, 0u);
        ro[u] = v < v1 ? o4[v] : make_uint4(0u, 0u, 0u, 0u);
      }
#pragma unroll
      for (int u = 0; u < U; ++u) {
        float a[8], o[8];
        bf16x8_to_f32(ra[u], a);
        bf16x8_to_f32(ro[u], o);
        float d8 = 0.0f, b8 = 0.0f;
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          d8 += fabsf(o[i] - a[i]);
          b8 += fabsf(a[i]);
        }
        diff += d8;
        base += b8;
      }
    }
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) {
      diff += __shfl_xor(diff, o);
      base += __shfl_xor(base, o);
    }
    if (lane == 0) {
      s_red[2 * wave] = diff;
      s_red[2 * wave + 1] = base;
    }
    __syncthreads();
    if (tid == 0) {
      double d = s_red[0], b = s_red[1];
      for (int w = 1; w < T / 64; ++w) {
        d += s_red[2 * w];
        b += s_red[2 * w + 1];
      }
      sl.parts[2 * c] = d;
      sl.parts[2 * c + 1] = b;
    }
  }
  if (tid == 0 && atomicAdd(&dw.queue[1], 1u) == (uint32_t)dw.delta_wgs - 1u) {
    atomicExch(&dw.queue[0], 0u);
    atomicExch(&dw.queue[1], 0u);
  }
}

// FP4: the NVFP4 weights' format (kNvfp4: the exact bf16-MFMA body; kNvfp4Mx,
// kNvfp4P2: the FP4 MFMA body, one or two passes; kNvfp4Decoded: the bf16
// body on operands decoded beforehand, xc and wc then pointing at bf16;
// kNvfp4XDecoded: xc points at the activations' bf16 values, W is codes).
template <int OUT, int FP4>
__global__ __launch_bounds__(512) void k_gemm_dispatch(
    const int32_t* __restrict__ decision, const int8_t* __restrict__ x8, const float* __restrict__ sx,
    const uint8_t* __restrict__ w4, const float* __restrict__ sw, const uint8_t* __restrict__ xc,
    const uint8_t* __restrict__ xsc, const float* __restrict__ xts, const uint8_t* __restrict__ wc,
    const uint8_t* __restrict__ wsc, const float* __restrict__ wts, const uint16_t* __restrict__ xb,
    const uint16_t* __restrict__ wb, void* __restrict__ Y, int M, int N, int K, int gemm_wgs,
    const DeltaWork delta) {
  if ((int)blockIdx.x >= gemm_wgs) {
    extern __shared__ __attribute__((aligned(1024))) uint8_t dsmem[];
    delta_workgroup(delta, dsmem);
    return;
  }
  const int32_t d = __builtin_amdgcn_readfirstlane(*decision);  // uniform: a scalar branch
  if (d == kPrecInt8) {
    gemm_i8i4_pipe_body<2, 4, 4, 2, OUT>(x8, sx, w4, sw, Y, M, N, K, gemm_wgs);
  } else if (d == kPrecNvfp4) {
    if constexpr (FP4 == kNvfp4)
      gemm_bf16_pipe_body<kSrcNvfp4, OUT>(xc, xsc, xts, wc, wsc, wts, Y, M, N, K, gemm_wgs);
    else if constexpr (FP4 == kNvfp4Decoded)
      gemm_bf16_pipe_body<kSrcBf16, OUT>(xc, nullptr, xts, wc, nullptr, wts, Y, M, N, K, gemm_wgs);
    else if constexpr (FP4 == kNvfp4XDecoded)
      gemm_bf16_pipe_body<kSrcNvfp4X, OUT>(xc, nullptr, xts, wc, wsc, wts, Y, M, N, K, gemm_wgs);
    else
      gemm_fp4mx_pipe_body<OUT, FP4 == kNvfp4P2>(xc, xsc, xts, wc, wsc, wts, Y, M, N, K, gemm_wgs);
  } else if (d == kPrecBf16) {
    gemm_bf16_pipe_body<kSrcBf16, OUT>(xb, nullptr, nullptr, wb, nullptr, nullptr, Y, M, N, K, gemm_wgs);
  }
}

template <int OUT, int FP4>
static hipError_t launch_dispatch_t(const int32_t* decision, const int8_t* x8, const float* sx,
                                    const uint8_t* w4, const float* sw, const uint8_t* xc,
                                    const uint8_t* xsc, const float* xts, const uint8_t* wc,
                                    const uint8_t* wsc, const float* wts, const uint16_t* xb,
                                    const uint16_t* wb, void* y, int64_t M, int64_t N, int64_t K,
                                    hipStream_t s, const DeltaWork* delta) {
  // Dynamic LDS: the largest body's (INT8: three 48 KB stages; FP4: two
  // 68 or 72 KB stages; bf16: a 256 x 256 bf16 output tile of 528-byte rows).
  constexpr size_t fp4_lds = (size_t)fp4_pipe_lds<FP4 == kNvfp4P2>();
  constexpr size_t i8_lds = (size_t)I8Cfg<2, 4, 4, 2>::LDS;
  constexpr size_t lds0 = fp4_lds > kBf16PipeLds ? fp4_lds : kBf16PipeLds;
  constexpr size_t lds = i8_lds > lds0 ? i8_lds : lds0;
  auto kern = k_gemm_dispatch<OUT, FP4>;
  hipError_t e = set_dynamic_lds_once<k_gemm_dispatch<OUT, FP4>>(lds);
  if (e != hipSuccess) return e;
  const int64_t tiles = ((M + 255) / 256) * ((N + 255) / 256);
  const int gemm_wgs = (int)persistent_grid(tiles);
  DeltaWork dw{};
  if (delta != nullptr && delta->total > 0) dw = *delta;
  const unsigned grid = (unsigned)gemm_wgs + (unsigned)(dw.total > 0 ? dw.delta_wgs : 0);
  hipLaunchKernelGGL(kern, dim3(grid), dim3(512), lds, s, decision, x8, sx, w4, sw, xc, xsc, xts, wc,
                     wsc, wts, xb, wb, y, (int)M, (int)N, (int)K, gemm_wgs, dw);
  return hipGetLastError();
}

hipError_t launch_gemm_dispatch(const int32_t* decision, const int8_t* x8, const float* sx,
                                const uint8_t* w4, const float* sw, const uint8_t* xc,
                                const uint8_t* xsc, const float* xts, const uint8_t* wc,
                                const uint8_t* wsc, const float* wts, int fp4_fmt,
                                const uint16_t* xb, const uint16_t* wb, void* y, int out_dtype,
                                int64_t M, int64_t N, int64_t K, hipStream_t s, const DeltaWork* delta) {
  // Every body's pipelined kernel must apply: K a multiple of each stage's
  // depth (256 covers them all) and 32-bit buffer offsets (bf16 rows are the
  // widest, 2 K bytes).
  if (K % 256 != 0 || M * 2 * K >= (1ll << 31) || N * 2 * K >= (1ll << 31)) return hipErrorNotSupported;
  if (out_dtype != kOutF32 && out_dtype != kOutBf16) return hipErrorNotSupported;
#define HDQ_DISPATCH(O, F) \
  return launch_dispatch_t<O, F>(decision, x8, sx, w4, sw, xc, xsc, xts, wc, wsc, wts, xb, wb, y, M, N, K, s, delta)
  if (out_dtype == kOutBf16) {
    if (fp4_fmt == kNvfp4Mx) HDQ_DISPATCH(kOutBf16, kNvfp4Mx);
    if (fp4_fmt == kNvfp4P2) HDQ_DISPATCH(kOutBf16, kNvfp4P2);
    if (fp4_fmt == kNvfp4Decoded) HDQ_DISPATCH(kOutBf16, kNvfp4Decoded);
    if (fp4_fmt == kNvfp4XDecoded) HDQ_DISPATCH(kOutBf16, kNvfp4XDecoded);
    HDQ_DISPATCH(kOutBf16, kNvfp4);
  }
  if (fp4_fmt == kNvfp4Mx) HDQ_DISPATCH(kOutF32, kNvfp4Mx);
  if (fp4_fmt == kNvfp4P2) HDQ_DISPATCH(kOutF32, kNvfp4P2);
  if (fp4_fmt == kNvfp4Decoded) HDQ_DISPATCH(kOutF32, kNvfp4Decoded);
  if (fp4_fmt == kNvfp4XDecoded) HDQ_DISPATCH(kOutF32, kNvfp4XDecoded);
  HDQ_DISPATCH(kOutF32, kNvfp4);
#undef HDQ_DISPATCH
}

}  // namespace hdq
