// gemm_bf16.hip -- GEMMs on gfx950 bf16 MFMA: exact NVFP4 and the bf16
// full-precision fallback.
//
// * NVFP4 x NVFP4 (summary on vetunion.cn, section one: NVFP4 activations for
//   stable steps; 4-bit weights).  NVFP4 carries one E4M3 scale per 16
//   elements; gfx950's block-scaled FP4 MFMA takes one power-of-two scale per
//   32, so an arbitrary NVFP4 tensor cannot run on it exactly.  Instead every
//   element is decoded while it is staged into LDS: e2m1(code) * E4M3(scale)
//   has at most 2 + 4 significant bits and fits bf16 exactly, so the bf16
//   MFMA (float32 accumulation) computes
//       y = s_tx * s_tw * sum_k (e2m1 E)_x (e2m1 E)_w
//   with the products exact; only the float32 accumulation rounds.
// * bf16 x bf16 on the unrotated operands: the full-precision path that the
//   summary's section three (purified delta refresh) falls back to.
//
// v_mfma_f32_32x32x16_bf16 with the instruction's A operand on the weights
// and B on the activations.  Two kernels, as in gemm_i8.hip: a pipelined one
// for K % 64 == 0 (256 x 256 tiles, 8 waves, see below) and a fallback for
// any K % 32 == 0 (256 x 128 tiles, 4 waves of 128 x 64, K advancing 32
// elements per double-buffered stage).
#include "gemm_bf16_pipe.h"
#include "hdq_device.h"
#include "hdq_internal.h"

namespace hdq {

template <int SRC, int ROWS>
struct Stager {
  // Staged per thread per stage (32 K elements of ROWS rows).
  static constexpr int UNITS = SRC == kSrcBf16 ? ROWS * 4 / 256   // 16-byte bf16 chunks
                                               : ROWS * 2 / 256;  // 16-element NVFP4 units
  static_assert(UNITS >= 1, "tile too small");
  uint4 raw[UNITS];
  uint32_t sc[SRC == kSrcNvfp4 ? UNITS : 1];

  __device__ __forceinline__ void load(const void* data, const uint8_t* scales, int row0, int nrows,
                                       int K, int k0, int tid) {
#pragma unroll
    for (int p = 0; p < UNITS; ++p) {
      if constexpr (SRC == kSrcBf16) {
        const int q = tid + 256 * p, r = q >> 2, c = q & 3;
        const int row = row0 + r, k = k0 + 8 * c;
        raw[p] = (row < nrows && k < K)
                     ? *reinterpret_cast<const uint4*>(reinterpret_cast<const uint16_t*>(data) +
                                                       (int64_t)row * K + k)
                     : make_uint4(0u, 0u, 0u, 0u);
      } else {
        const int q = tid + 256 * p, r = q >> 1, c = q & 1;
        const int row = row0 + r, k = k0 + 16 * c;
        if (row < nrows && k < K) {
          const uint2 v = *reinterpret_cast<const uint2*>(reinterpret_cast<const uint8_t*>(data) +
                                                          (int64_t)row * (K >> 1) + (k >> 1));
          raw[p] = make_uint4(v.x, v.y, 0u, 0u);
          sc[p] = scales[(int64_t)row * (K >> 4) + (k >> 4)];
        } else {
          raw[p] = make_uint4(0u, 0u, 0u, 0u);
          sc[p] = 0u;
        }
      }
    }
  }
  __device__ __forceinline__ void store(uint8_t* lds, int tid) const {
#pragma unroll
    for (int p = 0; p < UNITS; ++p) {
      if constexpr (SRC == kSrcBf16) {
        const int q = tid + 256 * p, r = q >> 2, c = q & 3;
        *reinterpret_cast<uint4*>(lds + lds_off64(r, c)) = raw[p];
      } else {
        const int q = tid + 256 * p, r = q >> 1, c = q & 1;
        uint4 lo, hi;
        decode_nvfp4x16(make_uint2(raw[p].x, raw[p].y), sc[p], lo, hi);
        *reinterpret_cast<uint4*>(lds + lds_off64(r, 2 * c)) = lo;
        *reinterpret_cast<uint4*>(lds + lds_off64(r, 2 * c + 1)) = hi;
      }
    }
  }
};

template <int SRC, int WM, int WN>
__global__ __launch_bounds__(256) void k_gemm_bf16mfma(
    const void* __restrict__ X, const uint8_t* __restrict__ xs, const float* __restrict__ xts,
    const void* __restrict__ W, const uint8_t* __restrict__ ws, const float* __restrict__ wts,
    void* __restrict__ Y, int out_dtype, int M, int N, int K, const int32_t* __restrict__ decision,
    int32_t want) {
  if (decision != nullptr && *decision != want) return;
  constexpr int BM = 64 * WM, BN = 64 * WN, BK = 32;
  __shared__ __attribute__((aligned(16))) uint8_t lds[2][(BM + BN) * 64];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave & 1, wn = wave >> 1;
  const int tiles_m = (M + BM - 1) / BM, tiles_n = (N + BN - 1) / BN;
  int tm, tn;
  xcd_tile(tiles_m, tiles_n, tm, tn);
  const int m0 = tm * BM, n0 = tn * BN;

  Stager<SRC, BM> sx;
  Stager<SRC, BN> sw;
  v16f acc[WN][WM];
#pragma unroll
  for (int j = 0; j < WN; ++j)
#pragma unroll
    for (int i = 0; i < WM; ++i)
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[j][i][e] = 0.0f;

  const int nk = (K + BK - 1) / BK;
  sx.load(X, xs, m0, M, K, 0, tid);
  sw.load(W, ws, n0, N, K, 0, tid);
  sx.store(lds[0], tid);
  sw.store(lds[0] + BM * 64, tid);
  __syncthreads();
  for (int kt = 0; kt < nk; ++kt) {
    if (kt + 1 < nk) {
      sx.load(X, xs, m0, M, K, (kt + 1) * BK, tid);
      sw.load(W, ws, n0, N, K, (kt + 1) * BK, tid);
    }
    const uint8_t* lx = lds[kt & 1];
    const uint8_t* lw = lds[kt & 1] + BM * 64;
#pragma unroll
    for (int ks = 0; ks < BK / 16; ++ks) {
      const int c = 2 * ks + (lane >> 5);
      v8bf xf[WM], wf[WN];
#pragma unroll
      for (int i = 0; i < WM; ++i)
        xf[i] = *reinterpret_cast<const v8bf*>(lx + lds_off64(wm * WM * 32 + i * 32 + (lane & 31), c));
#pragma unroll
      for (int j = 0; j < WN; ++j)
        wf[j] = *reinterpret_cast<const v8bf*>(lw + lds_off64(wn * WN * 32 + j * 32 + (lane & 31), c));
#pragma unroll
      for (int j = 0; j < WN; ++j)
#pragma unroll
        for (int i = 0; i < WM; ++i)
          acc[j][i] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(wf[j], xf[i], acc[j][i], 0, 0, 0);
    }
    if (kt + 1 < nk) {
      sx.store(lds[(kt + 1) & 1], tid);
      sw.store(lds[(kt + 1) & 1] + BM * 64, tid);
    }
    __syncthreads();
  }

  const float scale = (SRC == kSrcNvfp4 || xts != nullptr) ? (*xts) * (*wts) : 1.0f;
  const bool vec = (N & 3) == 0;
#pragma unroll
  for (int i = 0; i < WM; ++i) {
    const int m = m0 + wm * WM * 32 + i * 32 + (lane & 31);
    if (m >= M) continue;
#pragma unroll
    for (int j = 0; j < WN; ++j) {
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int n = n0 + wn * WN * 32 + j * 32 + 8 * g + 4 * (lane >> 5);
        if (n >= N) continue;
        float y[4];
#pragma unroll
        for (int r = 0; r < 4; ++r) y[r] = acc[j][i][4 * g + r] * scale;
        const int64_t off = (int64_t)m * N + n;
        if (out_dtype == kOutF32) {
          float* yp = reinterpret_cast<float*>(Y) + off;
          if (vec && n + 3 < N)
            *reinterpret_cast<float4*>(yp) = make_float4(y[0], y[1], y[2], y[3]);
          else
            for (int r = 0; r < 4 && n + r < N; ++r) yp[r] = y[r];
        } else {
          uint16_t* yp = reinterpret_cast<uint16_t*>(Y) + off;
          if (vec && n + 3 < N)
            *reinterpret_cast<uint2*>(yp) = make_uint2(pack_bf16x2(y[0], y[1]), pack_bf16x2(y[2], y[3]));
          else
            for (int r = 0; r < 4 && n + r < N; ++r) yp[r] = __builtin_bit_cast(uint16_t, (__bf16)y[r]);
        }
      }
    }
  }
}

// The gated kernel around the pipelined body (gemm_bf16_pipe.h).
template <int SRC, int OUT>
__global__ __launch_bounds__(512) void k_gemm_bf16_pipe(
    const void* __restrict__ X, const uint8_t* __restrict__ xsc, const float* __restrict__ xts,
    const void* __restrict__ W, const uint8_t* __restrict__ wsc, const float* __restrict__ wts,
    void* __restrict__ Y, int M, int N, int K, const int32_t* __restrict__ decision, int32_t want) {
  if (decision != nullptr && *decision != want) return;
  gemm_bf16_pipe_body<SRC, OUT>(X, xsc, xts, W, wsc, wts, Y, M, N, K);
}

template <int SRC, int OUT>
static hipError_t launch_bf16_pipe(const void* x, const uint8_t* xs, const float* xts, const void* w,
                                   const uint8_t* ws, const float* wts, void* y, int64_t M, int64_t N,
                                   int64_t K, const int32_t* decision, int32_t want, hipStream_t s) {
  constexpr size_t lds = kBf16PipeLds;
  auto kern = k_gemm_bf16_pipe<SRC, OUT>;
  hipError_t e = set_dynamic_lds_once<k_gemm_bf16_pipe<SRC, OUT>>(lds);
  if (e != hipSuccess) return e;
  const int64_t tiles = ((M + 255) / 256) * ((N + 255) / 256);
  hipLaunchKernelGGL(kern, dim3((unsigned)persistent_grid(tiles)), dim3(512), lds, s, x, xs, xts, w, ws,
                     wts, y, (int)M, (int)N, (int)K, decision, want);
  return hipGetLastError();
}

// The pipelined kernel needs K % 64 == 0 and 32-bit buffer offsets.
template <int SRC>
static bool pipe_ok(int64_t M, int64_t N, int64_t K) {
  const int64_t row = SRC == kSrcBf16 ? 2 * K : K / 2;
  return K % 64 == 0 && M * row < (1ll << 31) && N * row < (1ll << 31);
}

template <int SRC>
static hipError_t launch_bf16mfma(const void* x, const uint8_t* xs, const float* xts, const void* w,
                                  const uint8_t* ws, const float* wts, void* y, int out_dtype,
                                  int64_t M, int64_t N, int64_t K, const int32_t* decision,
                                  int32_t want, hipStream_t s) {
  if (pipe_ok<SRC>(M, N, K)) {
    if (out_dtype == kOutF32)
      return launch_bf16_pipe<SRC, kOutF32>(x, xs, xts, w, ws, wts, y, M, N, K, decision, want, s);
    return launch_bf16_pipe<SRC, kOutBf16>(x, xs, xts, w, ws, wts, y, M, N, K, decision, want, s);
  }
  constexpr int WM = 4, WN = 2;
  constexpr int BM = 64 * WM, BN = 64 * WN;
  const int64_t tiles = ((M + BM - 1) / BM) * ((N + BN - 1) / BN);
  hipLaunchKernelGGL((k_gemm_bf16mfma<SRC, WM, WN>), dim3((unsigned)tiles), dim3(256), 0, s, x, xs,
                     xts, w, ws, wts, y, out_dtype, (int)M, (int)N, (int)K, decision, want);
  return hipGetLastError();
}

hipError_t launch_gemm_nvfp4_bf16(const uint8_t* xc, const uint8_t* xs, const float* xts,
                                  const uint8_t* wc, const uint8_t* ws, const float* wts,
                                  void* y, int out_dtype, int64_t M, int64_t N, int64_t K,
                                  const int32_t* decision, int32_t want, hipStream_t s) {
  return launch_bf16mfma<kSrcNvfp4>(xc, xs, xts, wc, ws, wts, y, out_dtype, M, N, K, decision, want, s);
}

bool nvfp4_decoded_applies(int64_t M, int64_t N, int64_t K) { return pipe_ok<kSrcBf16>(M, N, K); }
bool nvfp4_xdecoded_applies(int64_t M, int64_t N, int64_t K) {
  return K % 64 == 0 && M * 2 * K < (1ll << 31) && N * (K / 2) < (1ll << 31);
}

hipError_t launch_gemm_nvfp4_xdecoded(const uint16_t* xd, const float* xts, const uint8_t* wc,
                                      const uint8_t* ws, const float* wts, void* y, int out_dtype, int64_t M,
                                      int64_t N, int64_t K, const int32_t* decision, int32_t want, hipStream_t s) {
  if (!nvfp4_xdecoded_applies(M, N, K)) return hipErrorNotSupported;
  if (out_dtype == kOutF32)
    return launch_bf16_pipe<kSrcNvfp4X, kOutF32>(xd, nullptr, xts, wc, ws, wts, y, M, N, K, decision, want, s);
  return launch_bf16_pipe<kSrcNvfp4X, kOutBf16>(xd, nullptr, xts, wc, ws, wts, y, M, N, K, decision, want, s);
}

hipError_t launch_gemm_nvfp4_decoded(const uint16_t* xd, const float* xts, const uint16_t* wd,
                                     const float* wts, void* y, int out_dtype, int64_t M, int64_t N,
                                     int64_t K, const int32_t* decision, int32_t want, hipStream_t s) {
  if (!nvfp4_decoded_applies(M, N, K)) return hipErrorNotSupported;
  return launch_bf16mfma<kSrcBf16>(xd, nullptr, xts, wd, nullptr, wts, y, out_dtype, M, N, K, decision, want, s);
}

hipError_t launch_gemm_bf16(const uint16_t* x, const uint16_t* w, void* y, int out_dtype,
                            int64_t M, int64_t N, int64_t K, const int32_t* decision,
                            int32_t want, hipStream_t s) {
  return launch_bf16mfma<kSrcBf16>(x, nullptr, nullptr, w, nullptr, nullptr, y, out_dtype, M, N, K,
                                   decision, want, s);
}

}  // namespace hdq
