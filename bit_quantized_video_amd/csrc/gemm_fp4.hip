// gemm_fp4.hip -- MX-compatible NVFP4 on gfx950's block-scaled FP4 MFMA.
//
// NVFP4 (the low-precision activation format of 6Bit-Diffusion, summary on
// vetunion.cn, section one) scales every 16 elements by an E4M3 value;
// v_mfma_scale_f32_32x32x64_f8f6f4 scales every 32 elements of a row by an
// E8M0 power of two.  When the quantizer restricts each aligned pair of
// 16-blocks to one shared power-of-two scale (format NVFP4_MX), the NVFP4
// bytes are exactly representable on the instruction: the kernel reconciles
// the two layouts by reading one E4M3 byte per 32 elements and re-encoding
// it as E8M0 (2^e -> e + 127) while staging, and applies the two fp32 tensor
// scales in the epilogue:
//     y = s_tx * s_tw * sum_32-blocks 2^(ex + ew) sum_k e2m1_x e2m1_w.
// Every product and block sum is exact; only the float32 accumulation rounds.
//
// Two kernels: a pipelined, persistent one (the INT8 kernel's structure, see
// below) for K % 256 == 0, and a simple double-buffered one for any
// K % 32 == 0.  In both the per-row E8M0 bytes of a stage sit in LDS next to
// the codes.
#include "gemm_fp4_pipe.h"
#include "hdq_device.h"
#include "hdq_internal.h"

#include <type_traits>

namespace hdq {

template <int ROWS>
struct Fp4Stager {
  static constexpr int CH = ROWS * 4 / 256;  // 16-byte code chunks per thread
  static_assert(CH >= 1 && ROWS <= 256, "tile shape");
  uint4 raw[CH];
  uint32_t sc;  // this thread's row: 4 E8M0 bytes (threads < ROWS)

  __device__ __forceinline__ void load(const uint8_t* codes, const uint8_t* scales, int row0,
                                       int nrows, int K, int k0, int tid) {
#pragma unroll
    for (int p = 0; p < CH; ++p) {
      const int q = tid + 256 * p, r = q >> 2, c = q & 3;
      const int row = row0 + r, k = k0 + 32 * c;
      raw[p] = (row < nrows && k < K)
                   ? *reinterpret_cast<const uint4*>(codes + (int64_t)row * (K >> 1) + (k >> 1))
                   : make_uint4(0u, 0u, 0u, 0u);
    }
    sc = 0u;
    if (tid < ROWS) {
      const int row = row0 + tid;
      if (row < nrows) {
        const uint8_t* sp = scales + (int64_t)row * (K >> 4) + (k0 >> 4);
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          const int k = k0 + 32 * g;
          const uint32_t b = (k < K) ? sp[2 * g] : 0u;
          sc |= e4m3_pow2_to_e8m0(b) << (8 * g);
        }
      }
    }
  }
  __device__ __forceinline__ void store(uint8_t* lds_codes, uint32_t* lds_sc, int tid) const {
#pragma unroll
    for (int p = 0; p < CH; ++p) {
      const int q = tid + 256 * p, r = q >> 2, c = q & 3;
      *reinterpret_cast<uint4*>(lds_codes + lds_off64(r, c)) = raw[p];
    }
    if (tid < ROWS) lds_sc[tid] = sc;
  }
};

template <int WM, int WN>
__global__ __launch_bounds__(256) void k_gemm_fp4mx(
    const uint8_t* __restrict__ xc, const uint8_t* __restrict__ xs, const float* __restrict__ xts,
    const uint8_t* __restrict__ wc, const uint8_t* __restrict__ ws, const float* __restrict__ wts,
    void* __restrict__ Y, int out_dtype, int M, int N, int K, const int32_t* __restrict__ decision,
    int32_t want) {
  if (decision != nullptr && *decision != want) return;
  constexpr int BM = 64 * WM, BN = 64 * WN, BK = 128;
  __shared__ __attribute__((aligned(16))) uint8_t lds[2][(BM + BN) * 64];
  __shared__ uint32_t lsc[2][BM + BN];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave & 1, wn = wave >> 1;
  const int tiles_m = (M + BM - 1) / BM, tiles_n = (N + BN - 1) / BN;
  int tm, tn;
  xcd_tile(tiles_m, tiles_n, tm, tn);
  const int m0 = tm * BM, n0 = tn * BN;

  Fp4Stager<BM> sx;
  Fp4Stager<BN> sw;
  v16f acc[WN][WM];
#pragma unroll
  for (int j = 0; j < WN; ++j)
#pragma unroll
    for (int i = 0; i < WM; ++i)
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[j][i][e] = 0.0f;

  const int nk = (K + BK - 1) / BK;
  sx.load(xc, xs, m0, M, K, 0, tid);
  sw.load(wc, ws, n0, N, K, 0, tid);
  sx.store(lds[0], lsc[0], tid);
  sw.store(lds[0] + BM * 64, lsc[0] + BM, tid);
  __syncthreads();
  for (int kt = 0; kt < nk; ++kt) {
    if (kt + 1 < nk) {
      sx.load(xc, xs, m0, M, K, (kt + 1) * BK, tid);
      sw.load(wc, ws, n0, N, K, (kt + 1) * BK, tid);
    }
    const uint8_t* lx = lds[kt & 1];
    const uint8_t* lw = lds[kt & 1] + BM * 64;
    const uint32_t* sxl = lsc[kt & 1];
    const uint32_t* swl = lsc[kt & 1] + BM;
#pragma unroll
    for (int ks = 0; ks < BK / 64; ++ks) {
      const int c = 2 * ks + (lane >> 5);  // 32-element block of this lane's fragment
      v8i xf[WM], wf[WN];
      int xe[WM], we[WN];
#pragma unroll
      for (int i = 0; i < WM; ++i) {
        const int r = wm * WM * 32 + i * 32 + (lane & 31);
        const v4i v = *reinterpret_cast<const v4i*>(lx + lds_off64(r, c));
        xf[i] = v8i{v[0], v[1], v[2], v[3], 0, 0, 0, 0};
        xe[i] = (int)((sxl[r] >> (8 * c)) & 0xffu);
      }
#pragma unroll
      for (int j = 0; j < WN; ++j) {
        const int r = wn * WN * 32 + j * 32 + (lane & 31);
        const v4i v = *reinterpret_cast<const v4i*>(lw + lds_off64(r, c));
        wf[j] = v8i{v[0], v[1], v[2], v[3], 0, 0, 0, 0};
        we[j] = (int)((swl[r] >> (8 * c)) & 0xffu);
      }
#pragma unroll
      for (int j = 0; j < WN; ++j)
#pragma unroll
        for (int i = 0; i < WM; ++i)
          acc[j][i] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(wf[j], xf[i], acc[j][i], 4, 4,
                                                                        0, we[j], 0, xe[i]);
    }
    if (kt + 1 < nk) {
      sx.store(lds[(kt + 1) & 1], lsc[(kt + 1) & 1], tid);
      sw.store(lds[(kt + 1) & 1] + BM * 64, lsc[(kt + 1) & 1] + BM, tid);
    }
    __syncthreads();
  }

  const float scale = (*xts) * (*wts);
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

// The gated kernel around the pipelined body (gemm_fp4_pipe.h); P2: the
// two-pass form for a power-of-two scale per 16-block.
template <int OUT, bool P2>
__global__ __launch_bounds__(512) void k_gemm_fp4mx_pipe(
    const uint8_t* __restrict__ xc, const uint8_t* __restrict__ xsc, const float* __restrict__ xts,
    const uint8_t* __restrict__ wc, const uint8_t* __restrict__ wsc, const float* __restrict__ wts,
    void* __restrict__ Y, int M, int N, int K, const int32_t* __restrict__ decision, int32_t want) {
  if (decision != nullptr && *decision != want) return;
  gemm_fp4mx_pipe_body<OUT, P2>(xc, xsc, xts, wc, wsc, wts, Y, M, N, K);
}

template <int OUT, bool P2>
static hipError_t launch_fp4_pipe(const uint8_t* xc, const uint8_t* xs, const float* xts,
                                  const uint8_t* wc, const uint8_t* ws, const float* wts, void* y,
                                  int64_t M, int64_t N, int64_t K, const int32_t* decision,
                                  int32_t want, hipStream_t s) {
  constexpr size_t lds = (size_t)fp4_pipe_lds<P2>();
  auto kern = k_gemm_fp4mx_pipe<OUT, P2>;
  hipError_t e = set_dynamic_lds_once<k_gemm_fp4mx_pipe<OUT, P2>>(lds);
  if (e != hipSuccess) return e;
  const int64_t tiles = ((M + 255) / 256) * ((N + 255) / 256);
  hipLaunchKernelGGL(kern, dim3((unsigned)persistent_grid(tiles)), dim3(512), lds, s, xc, xs, xts, wc, ws,
                     wts, y, (int)M, (int)N, (int)K, decision, want);
  return hipGetLastError();
}

// The pipelined body with DeltaQuant's broadcast core term in its epilogue.
template <int OUT, bool P2>
__global__ __launch_bounds__(512) void k_gemm_fp4_core_add(
    const uint8_t* __restrict__ xc, const uint8_t* __restrict__ xsc, const float* __restrict__ xts,
    const uint8_t* __restrict__ wc, const uint8_t* __restrict__ wsc, const float* __restrict__ wts,
    void* __restrict__ Y, int M, int N, int K, const CoreAdd add) {
  gemm_fp4mx_pipe_body<OUT, P2, true>(xc, xsc, xts, wc, wsc, wts, Y, M, N, K, 0, &add);
}

template <int OUT, bool P2>
static hipError_t launch_core_add_t(const uint8_t* xc, const uint8_t* xs, const float* xts, const uint8_t* wc,
                                    const uint8_t* ws, const float* wts, const CoreAdd& add, void* y, int64_t M,
                                    int64_t N, int64_t K, hipStream_t s) {
  constexpr size_t lds = (size_t)fp4_pipe_lds<P2>();
  auto kern = k_gemm_fp4_core_add<OUT, P2>;
  hipError_t e = set_dynamic_lds_once<k_gemm_fp4_core_add<OUT, P2>>(lds);
  if (e != hipSuccess) return e;
  const int64_t tiles = ((M + 255) / 256) * ((N + 255) / 256);
  hipLaunchKernelGGL(kern, dim3((unsigned)persistent_grid(tiles)), dim3(512), lds, s, xc, xs, xts, wc, ws, wts, y,
                     (int)M, (int)N, (int)K, add);
  return hipGetLastError();
}

hipError_t launch_gemm_fp4_core_add(const uint8_t* xc, const uint8_t* xs, const float* xts, const uint8_t* wc,
                                    const uint8_t* ws, const float* wts, int fmt, const CoreAdd& add, void* y,
                                    int out_dtype, int64_t M, int64_t N, int64_t K, hipStream_t s) {
  if (!fp4_core_add_applies(fmt, M, N, K)) return hipErrorNotSupported;
  if (fmt == kNvfp4Mx)
    return out_dtype == kOutF32 ? launch_core_add_t<kOutF32, false>(xc, xs, xts, wc, ws, wts, add, y, M, N, K, s)
                                : launch_core_add_t<kOutBf16, false>(xc, xs, xts, wc, ws, wts, add, y, M, N, K, s);
  if (fmt == kNvfp4P2)
    return out_dtype == kOutF32 ? launch_core_add_t<kOutF32, true>(xc, xs, xts, wc, ws, wts, add, y, M, N, K, s)
                                : launch_core_add_t<kOutBf16, true>(xc, xs, xts, wc, ws, wts, add, y, M, N, K, s);
  return hipErrorNotSupported;
}

hipError_t launch_gemm_nvfp4_mx(const uint8_t* xc, const uint8_t* xs, const float* xts,
                                const uint8_t* wc, const uint8_t* ws, const float* wts,
                                void* y, int out_dtype, int64_t M, int64_t N, int64_t K,
                                const int32_t* decision, int32_t want, hipStream_t s) {
  // The pipelined kernel needs K % 256 == 0 and 32-bit buffer offsets.
  if (K % 256 == 0 && M * K / 2 < (1ll << 31) && N * K / 2 < (1ll << 31)) {
    if (out_dtype == kOutF32)
      return launch_fp4_pipe<kOutF32, false>(xc, xs, xts, wc, ws, wts, y, M, N, K, decision, want, s);
    return launch_fp4_pipe<kOutBf16, false>(xc, xs, xts, wc, ws, wts, y, M, N, K, decision, want, s);
  }
  constexpr int WM = 4, WN = 2;
  constexpr int BM = 64 * WM, BN = 64 * WN;
  const int64_t tiles = ((M + BM - 1) / BM) * ((N + BN - 1) / BN);
  hipLaunchKernelGGL((k_gemm_fp4mx<WM, WN>), dim3((unsigned)tiles), dim3(256), 0, s, xc, xs, xts, wc,
                     ws, wts, y, out_dtype, (int)M, (int)N, (int)K, decision, want);
  return hipGetLastError();
}

// NVFP4 with a power-of-two scale per 16-block: the two-pass pipelined FP4
// kernel, or (shapes it does not take) the exact bf16-MFMA kernel, which
// takes any NVFP4 bytes.
hipError_t launch_gemm_nvfp4_p2(const uint8_t* xc, const uint8_t* xs, const float* xts,
                                const uint8_t* wc, const uint8_t* ws, const float* wts,
                                void* y, int out_dtype, int64_t M, int64_t N, int64_t K,
                                const int32_t* decision, int32_t want, hipStream_t s) {
  if (K % 256 == 0 && M * K / 2 < (1ll << 31) && N * K / 2 < (1ll << 31)) {
    if (out_dtype == kOutF32)
      return launch_fp4_pipe<kOutF32, true>(xc, xs, xts, wc, ws, wts, y, M, N, K, decision, want, s);
    return launch_fp4_pipe<kOutBf16, true>(xc, xs, xts, wc, ws, wts, y, M, N, K, decision, want, s);
  }
  return launch_gemm_nvfp4_bf16(xc, xs, xts, wc, ws, wts, y, out_dtype, M, N, K, decision, want, s);
}

}  // namespace hdq
