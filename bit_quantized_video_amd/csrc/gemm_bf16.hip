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
#include "hdq_device.h"
#include "hdq_internal.h"

namespace hdq {

enum Src : int { kSrcBf16 = 0, kSrcNvfp4 = 1 };

// 16 NVFP4 elements (8 code bytes) with scale byte e -> 16 bf16, exact.
// Byte B of `word` (two E2M1 codes) -> bf16 pair of e2m1 * s.
template <int B>
__device__ __forceinline__ uint32_t decode_fp4x2(uint32_t word, float s) {
  const auto f = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(word, 1.0f, B);
  return pack_bf16x2(f[0] * s, f[1] * s);
}

__device__ __forceinline__ void decode_nvfp4x16(const uint2 codes, uint32_t e, uint4& lo, uint4& hi) {
  const float s = e4m3_decode(e);
  lo = make_uint4(decode_fp4x2<0>(codes.x, s), decode_fp4x2<1>(codes.x, s),
                  decode_fp4x2<2>(codes.x, s), decode_fp4x2<3>(codes.x, s));
  hi = make_uint4(decode_fp4x2<0>(codes.y, s), decode_fp4x2<1>(codes.y, s),
                  decode_fp4x2<2>(codes.y, s), decode_fp4x2<3>(codes.y, s));
}

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

  const float scale = (SRC == kSrcNvfp4) ? (*xts) * (*wts) : 1.0f;
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

// ---------------------------------------------------------------------------
// Pipelined kernel for K % 64 == 0: 256 x 256 tile, 8 waves as 2 (tokens) x
// 4 (features), each 128 x 64 (4 x 2 subtiles of 32 x 32), 64 K per stage,
// two register sets prefetching the next two stages through buffer loads
// (rows past M or N read as zero), double-buffered LDS, LDS-only barriers,
// a persistent tile loop and bf16 output tiles staged in LDS -- the
// structure of the INT8 kernel.  LDS holds bf16: 128-byte rows per
// stage (swz128), substep s (16 K) giving lane half h the 16-byte chunk
// 2s + h.  NVFP4 operands are decoded to exact bf16 when their registers are
// written to LDS, once per workgroup rather than once per wave.
// LDS: two 64 KB stages, or one staged 256 x 256 bf16 output tile with a
// padded row pitch, whichever is larger.
constexpr int kBf16OutPitch = 256 * 2 + 16;
constexpr size_t kBf16PipeLds =
    (2 * 2 * 256 * 64 * 2 > 256 * kBf16OutPitch) ? 2 * 2 * 256 * 64 * 2 : 256 * kBf16OutPitch;

template <int SRC>
struct Bf16Stage;
template <>
struct Bf16Stage<kSrcBf16> {
  uint4 x[4], w[4];  // 4 x 16-byte chunks per operand per thread
};
template <>
struct Bf16Stage<kSrcNvfp4> {
  uint4 x, w;         // 32 codes per operand per thread
  uint32_t xs, ws;    // their two E4M3 block scales
};

template <int SRC, int OUT>
__global__ __launch_bounds__(512) void k_gemm_bf16_pipe(
    const void* __restrict__ X, const uint8_t* __restrict__ xsc, const float* __restrict__ xts,
    const void* __restrict__ W, const uint8_t* __restrict__ wsc, const float* __restrict__ wts,
    void* __restrict__ Y, int M, int N, int K, const int32_t* __restrict__ decision, int32_t want) {
  if (decision != nullptr && *decision != want) return;
  constexpr int BM = 256, BN = 256, BK = 64, WM_T = 4, WN_T = 2;
  constexpr int XB = BM * BK * 2, SB = XB + BN * BK * 2;  // LDS bytes per stage
  constexpr int kOutPitch = kBf16OutPitch;                // bf16 output row staged in LDS
  using Stage = Bf16Stage<SRC>;
  extern __shared__ __attribute__((aligned(1024))) uint8_t smem[];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave % 2, wn = wave / 2;
  const int tiles_m = (M + BM - 1) / BM, tiles_n = (N + BN - 1) / BN;
  const TileSeq seq = tile_seq(tiles_m * tiles_n);
  const int nk = K / BK;

  // Buffer resources over the current tile's rows; per-thread offsets.
  __amdgpu_buffer_rsrc_t xres, wres, xsres, wsres;
  uint32_t xvoff, wvoff, svoff = 0;
  int dst;  // LDS byte offset of this thread's first chunk (same for X and W)
  if constexpr (SRC == kSrcBf16) {
    const int r = tid >> 3, c = tid & 7;  // 8 threads per 128-byte row, 64 rows per round
    xvoff = wvoff = (uint32_t)(r * 2 * K + 16 * c);
    dst = r * 128 + 16 * (c ^ swz128(r));
  } else {
    const int r = tid >> 1, c = tid & 1;  // 2 threads per row: 32 elements each
    xvoff = wvoff = (uint32_t)(r * (K / 2) + 16 * c);
    svoff = (uint32_t)(r * (K / 16) + 2 * c);
    dst = r * 128 + 64 * c;  // chunks 4c .. 4c + 3 of the row (swizzled at store)
  }
  auto open_tile = [&](int m0, int n0) {
    if constexpr (SRC == kSrcBf16) {
      const int64_t ld = 2 * (int64_t)K;
      xres = make_rsrc(reinterpret_cast<const uint8_t*>(X) + m0 * ld, (uint32_t)((M - m0) * ld));
      wres = make_rsrc(reinterpret_cast<const uint8_t*>(W) + n0 * ld, (uint32_t)((N - n0) * ld));
    } else {
      const int64_t ld = K / 2, lds_ = K / 16;
      xres = make_rsrc(reinterpret_cast<const uint8_t*>(X) + m0 * ld, (uint32_t)((M - m0) * ld));
      wres = make_rsrc(reinterpret_cast<const uint8_t*>(W) + n0 * ld, (uint32_t)((N - n0) * ld));
      xsres = make_rsrc(xsc + m0 * lds_, (uint32_t)((M - m0) * lds_));
      wsres = make_rsrc(wsc + n0 * lds_, (uint32_t)((N - n0) * lds_));
    }
  };
  auto load = [&](Stage& st, int kt) {
    if constexpr (SRC == kSrcBf16) {
#pragma unroll
      for (int p = 0; p < 4; ++p) {
        st.x[p] = buf_load16(xres, xvoff, kt * 128 + p * 64 * 2 * K);
        st.w[p] = buf_load16(wres, wvoff, kt * 128 + p * 64 * 2 * K);
      }
    } else {
      st.x = buf_load16(xres, xvoff, kt * 32);
      st.w = buf_load16(wres, wvoff, kt * 32);
      st.xs = __builtin_amdgcn_raw_buffer_load_b16(xsres, (int)svoff, kt * 4, 0);
      st.ws = __builtin_amdgcn_raw_buffer_load_b16(wsres, (int)svoff, kt * 4, 0);
    }
  };
  auto store = [&](const Stage& st, int buf) {
    uint8_t* lx = smem + buf * SB;
    uint8_t* lw = lx + XB;
    if constexpr (SRC == kSrcBf16) {
#pragma unroll
      for (int p = 0; p < 4; ++p) {
        *reinterpret_cast<uint4*>(lx + dst + p * 64 * 128) = st.x[p];
        *reinterpret_cast<uint4*>(lw + dst + p * 64 * 128) = st.w[p];
      }
    } else {
      const int r = tid >> 1, c = tid & 1;
      uint4 d[4];
      decode_nvfp4x16(make_uint2(st.x.x, st.x.y), st.xs & 0xffu, d[0], d[1]);
      decode_nvfp4x16(make_uint2(st.x.z, st.x.w), st.xs >> 8, d[2], d[3]);
#pragma unroll
      for (int q = 0; q < 4; ++q)
        *reinterpret_cast<uint4*>(lx + r * 128 + 16 * ((4 * c + q) ^ swz128(r))) = d[q];
      decode_nvfp4x16(make_uint2(st.w.x, st.w.y), st.ws & 0xffu, d[0], d[1]);
      decode_nvfp4x16(make_uint2(st.w.z, st.w.w), st.ws >> 8, d[2], d[3]);
#pragma unroll
      for (int q = 0; q < 4; ++q)
        *reinterpret_cast<uint4*>(lw + r * 128 + 16 * ((4 * c + q) ^ swz128(r))) = d[q];
    }
  };

  v16f acc[WN_T][WM_T];
  auto zero_acc = [&]() {
#pragma unroll
    for (int j = 0; j < WN_T; ++j)
#pragma unroll
      for (int i = 0; i < WM_T; ++i)
#pragma unroll
        for (int e = 0; e < 16; ++e) acc[j][i][e] = 0.0f;
  };
  zero_acc();

  const int h = lane >> 5, r32 = lane & 31;
  auto compute = [&](int buf) {
    const uint8_t* lx = smem + buf * SB;
    const uint8_t* lw = lx + XB;
#pragma unroll
    for (int ks = 0; ks < BK / 16; ++ks) {
      v8bf xf[WM_T], wf[WN_T];
#pragma unroll
      for (int i = 0; i < WM_T; ++i) {
        const int r = wm * WM_T * 32 + i * 32 + r32;
        xf[i] = *reinterpret_cast<const v8bf*>(lx + r * 128 + 16 * ((2 * ks + h) ^ swz128(r)));
      }
#pragma unroll
      for (int j = 0; j < WN_T; ++j) {
        const int r = wn * WN_T * 32 + j * 32 + r32;
        wf[j] = *reinterpret_cast<const v8bf*>(lw + r * 128 + 16 * ((2 * ks + h) ^ swz128(r)));
      }
#pragma unroll
      for (int j = 0; j < WN_T; ++j)
#pragma unroll
        for (int i = 0; i < WM_T; ++i)
          acc[j][i] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(wf[j], xf[i], acc[j][i], 0, 0, 0);
    }
  };

  const float scale = (SRC == kSrcNvfp4) ? (*xts) * (*wts) : 1.0f;
  auto epilogue = [&](int m0, int n0) {
    if constexpr (OUT == kOutBf16) {
      // Stage the bf16 tile in LDS (both pipeline buffers are free once every
      // wave is past the last stage), then write whole 512-byte rows with
      // 16-byte stores.
      lds_barrier();
      uint8_t* const lrow = smem + (wm * WM_T * 32 + r32) * kOutPitch + 2 * (wn * WN_T * 32 + 4 * h);
#pragma unroll
      for (int i = 0; i < WM_T; ++i)
#pragma unroll
        for (int j = 0; j < WN_T; ++j)
#pragma unroll
          for (int g = 0; g < 4; ++g) {
            const v16f& a = acc[j][i];
            *reinterpret_cast<uint2*>(lrow + i * 32 * kOutPitch + 2 * (j * 32 + 8 * g)) =
                make_uint2(pack_bf16x2(a[4 * g] * scale, a[4 * g + 1] * scale),
                           pack_bf16x2(a[4 * g + 2] * scale, a[4 * g + 3] * scale));
          }
      lds_barrier();
      uint16_t* y16 = reinterpret_cast<uint16_t*>(Y);
      const int n = n0 + 8 * (tid & 31);
      const bool vec = n + 8 <= N && (N & 7) == 0;
#pragma unroll 4
      for (int r = tid >> 5; r < BM; r += 16) {
        const uint8_t* src = smem + r * kOutPitch + 16 * (tid & 31);
        if (m0 + r < M) {
          uint16_t* dst16 = y16 + (int64_t)(m0 + r) * N + n;
          if (vec) {
            *reinterpret_cast<uint4*>(dst16) = *reinterpret_cast<const uint4*>(src);
          } else {
            for (int e = 0; e < 8 && n + e < N; ++e) dst16[e] = reinterpret_cast<const uint16_t*>(src)[e];
          }
        }
      }
      lds_barrier();  // the next tile's first stage may overwrite the staged tile
    } else {
      const bool full_n = n0 + BN <= N && (N & 3) == 0;
#pragma unroll
      for (int i = 0; i < WM_T; ++i) {
        const int m = m0 + wm * WM_T * 32 + i * 32 + r32;
        if (m >= M) continue;
#pragma unroll
        for (int j = 0; j < WN_T; ++j) {
#pragma unroll
          for (int g = 0; g < 4; ++g) {
            const int n = n0 + wn * WN_T * 32 + j * 32 + 8 * g + 4 * h;
            const int64_t off = (int64_t)m * N + n;
            float y[4];
#pragma unroll
            for (int r = 0; r < 4; ++r) y[r] = acc[j][i][4 * g + r] * scale;
            if (full_n) {
              *reinterpret_cast<float4*>(reinterpret_cast<float*>(Y) + off) = make_float4(y[0], y[1], y[2], y[3]);
            } else {
              for (int r = 0; r < 4 && n + r < N; ++r) reinterpret_cast<float*>(Y)[off + r] = y[r];
            }
          }
        }
      }
    }
  };

  // Persistent loop over this workgroup's tiles; per tile, the K-stages run
  // through the two-stage register prefetch and the double-buffered LDS.
  for (int t = 0; t < seq.count; ++t) {
    int tm, tn;
    grouped_tile(seq.first + t * seq.stride, tiles_m, tiles_n, tm, tn);
    const int m0 = tm * BM, n0 = tn * BN;
    open_tile(m0, n0);
    Stage ra, rb;
    load(ra, 0);
    if (nk > 1) load(rb, 1);
    store(ra, 0);
    lds_barrier();
    int kt = 0;
    for (; kt + 1 < nk; kt += 2) {
      if (kt + 2 < nk) load(ra, kt + 2);
      compute(0);
      store(rb, 1);
      lds_barrier();
      if (kt + 3 < nk) load(rb, kt + 3);
      compute(1);
      if (kt + 2 < nk) store(ra, 0);
      lds_barrier();
    }
    if (kt < nk) compute(0);
    epilogue(m0, n0);
    zero_acc();
  }
}

template <int SRC, int OUT>
static hipError_t launch_bf16_pipe(const void* x, const uint8_t* xs, const float* xts, const void* w,
                                   const uint8_t* ws, const float* wts, void* y, int64_t M, int64_t N,
                                   int64_t K, const int32_t* decision, int32_t want, hipStream_t s) {
  constexpr size_t lds = kBf16PipeLds;
  auto kern = k_gemm_bf16_pipe<SRC, OUT>;
  hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(kern),
                                     hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
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

hipError_t launch_gemm_bf16(const uint16_t* x, const uint16_t* w, void* y, int out_dtype,
                            int64_t M, int64_t N, int64_t K, const int32_t* decision,
                            int32_t want, hipStream_t s) {
  return launch_bf16mfma<kSrcBf16>(x, nullptr, nullptr, w, nullptr, nullptr, y, out_dtype, M, N, K,
                                   decision, want, s);
}

}  // namespace hdq
