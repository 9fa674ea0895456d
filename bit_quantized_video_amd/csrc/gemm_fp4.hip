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

// ---- DeltaQuant's core GEMM on the FP8 x FP4 scaled MFMA ------------------
// DeltaQuant (paper-radar CVPR 2026 listing, abstract) keeps each cube's core
// token in FP8 and multiplies it by the layer's 4-bit weights:
//   yc[c, n] = sum_k e4m3(core[c, k]) * e2m1(w[n, k]) * 2^e(n, k)
// with e the weights' power-of-two block scale (one per 32 k for the MX
// format; one per 16 k for the per-16 format, which runs every MFMA twice
// with the core operand's other 16-block zeroed).  The core codes are the
// instruction's FP8 E4M3 operand as stored (unit scale), the weight codes its
// FP4 operand with their E8M0 scales; every product is exact and only the
// float32 accumulation rounds.  Operand layout of this mixed form (measured
// on gfx950): per 64-K step an FP4 lane of half h holds k [32 h, 32 h + 32)
// and takes one scale for them; an FP8 lane of half h holds k [16 h, 16 h + 16)
// and [32 + 16 h, 48 + 16 h), and the scales follow the 32-k blocks.  The per-cube and tensor scales are applied
// where yc is used (the difference GEMM's epilogue).
//  * 256 x 256 tiles, 8 waves as 2 (cubes) x 4 (features) of 128 x 64, a
//    persistent tile loop; K advances 128 per stage, register-staged into
//    two LDS buffers (core rows 128 bytes, weight rows 64 bytes, both
//    XOR-swizzled 16-byte chunks; per weight row the stage's E8M0 bytes as
//    words that lane half h reads once per stage, byte ks selected per
//    64-K substep ks); fp32 output stored from registers.
template <bool P2>
__global__ __launch_bounds__(512) void k_gemm_dq_core(const uint8_t* __restrict__ core, const uint8_t* __restrict__ wc,
                                                     const uint8_t* __restrict__ wsc, float* __restrict__ Y, int C,
                                                     int N, int K) {
  constexpr int BM = 256, BN = 256, BK = 128, WM_T = 4, WN_T = 2;
  constexpr int AB = BM * BK, WB = BN * BK / 2;  // core and weight code bytes per stage
  constexpr int SCB = P2 ? 16 : 8;               // E8M0 bytes per weight row and stage
  constexpr int SB = AB + WB + BN * SCB;
  extern __shared__ __attribute__((aligned(1024))) uint8_t smem[];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave % 2, wn = wave / 2;
  const int tiles_m = (C + BM - 1) / BM, tiles_n = (N + BN - 1) / BN;
  const TileSeq seq = tile_seq(tiles_m * tiles_n);
  const int nk = K / BK;
  const int G = seq.count * nk;
  if (G == 0) return;
  const int ldw = K / 2, lds_ = K / 16;
  // core rows: 8 threads x 16 bytes, 64 rows per round; weight rows: 4
  // threads x 16 bytes, 128 rows per round; weight scales: one row per
  // thread of the first 256 (its 8 E4M3 bytes of the stage)
  const int ar = tid >> 3, ac = tid & 7, wr = tid >> 2, wcc = tid & 3;
  const uint32_t avoff = (uint32_t)(ar * K + 16 * ac), wvoff = (uint32_t)(wr * ldw + 16 * wcc);
  const int adst = ar * 128 + 16 * (ac ^ swz128(ar)), wdst = wr * 64 + 16 * (wcc ^ swz64(wr));
  const bool srow_t = tid < 256;
  const uint32_t svoff = (uint32_t)((tid & 255) * lds_);

  int l_logical = seq.first, l_kt = 0;
  __amdgpu_buffer_rsrc_t ares, wres, sres;
  auto open_tile = [&]() {
    int tm, tn;
    grouped_tile(l_logical, tiles_m, tiles_n, tm, tn);
    const int m0 = tm * BM, n0 = tn * BN;
    ares = make_rsrc(core + (int64_t)m0 * K, (uint32_t)((int64_t)(C - m0) * K));
    wres = make_rsrc(wc + (int64_t)n0 * ldw, (uint32_t)((int64_t)(N - n0) * ldw));
    sres = make_rsrc(wsc + (int64_t)n0 * lds_, (uint32_t)((int64_t)(N - n0) * lds_));
  };
  open_tile();
  struct Stage {
    uint4 a[4], w[2];
    uint2 sc;
  };
  auto load = [&](Stage& st) {
#pragma unroll
    for (int p = 0; p < 4; ++p) st.a[p] = buf_load16(ares, avoff, l_kt * BK + p * 64 * K);
#pragma unroll
    for (int p = 0; p < 2; ++p) st.w[p] = buf_load16(wres, wvoff, l_kt * (BK / 2) + p * 128 * ldw);
    st.sc = srow_t ? __builtin_bit_cast(uint2, __builtin_amdgcn_raw_buffer_load_b64(sres, (int)svoff, l_kt * (BK / 16), 0))
                   : make_uint2(0u, 0u);
    if (++l_kt == nk) {
      l_kt = 0;
      l_logical += seq.stride;
      if (l_logical < tiles_m * tiles_n) open_tile();
    }
  };
  auto store = [&](const Stage& st, int buf) {
    uint8_t* base = smem + buf * SB;
#pragma unroll
    for (int p = 0; p < 4; ++p) *reinterpret_cast<uint4*>(base + adst + p * 64 * 128) = st.a[p];
#pragma unroll
    for (int p = 0; p < 2; ++p) *reinterpret_cast<uint4*>(base + AB + wdst + p * 128 * 64) = st.w[p];
    if (srow_t) {
      // E4M3 byte b of the stage scales k [16 b, 16 b + 16); group q (32 k)
      // is bytes 2q, 2q + 1.  Word h holds groups h and h + 2 (MX: their
      // first byte); P2 adds words 2 + h with their second bytes.
      const uint32_t e[8] = {e4m3_pow2_to_e8m0(st.sc.x & 0xffu), e4m3_pow2_to_e8m0((st.sc.x >> 8) & 0xffu),
                             e4m3_pow2_to_e8m0((st.sc.x >> 16) & 0xffu), e4m3_pow2_to_e8m0(st.sc.x >> 24),
                             e4m3_pow2_to_e8m0(st.sc.y & 0xffu), e4m3_pow2_to_e8m0((st.sc.y >> 8) & 0xffu),
                             e4m3_pow2_to_e8m0((st.sc.y >> 16) & 0xffu), e4m3_pow2_to_e8m0(st.sc.y >> 24)};
      uint8_t* sp = base + AB + WB + (tid & 255) * SCB;
      const uint32_t w0 = e[0] | (e[4] << 8), w1 = e[2] | (e[6] << 8);
      if constexpr (P2)
        *reinterpret_cast<uint4*>(sp) = make_uint4(w0, w1, e[1] | (e[5] << 8), e[3] | (e[7] << 8));
      else
        *reinterpret_cast<uint2*>(sp) = make_uint2(w0, w1);
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
  constexpr int kUnitScale = 0x7f7f7f7f;  // E8M0 2^0 in every byte
  auto compute = [&](int buf) {
    const uint8_t* la = smem + buf * SB;
    const uint8_t* lw = la + AB;
    const uint8_t* ls = lw + WB;
    int we[WN_T], wo[WN_T];
#pragma unroll
    for (int j = 0; j < WN_T; ++j) {
      const uint8_t* p = ls + (wn * WN_T * 32 + j * 32 + r32) * SCB + 4 * h;
      we[j] = *reinterpret_cast<const int*>(p);
      if constexpr (P2) wo[j] = *reinterpret_cast<const int*>(p + 8);
    }
    auto substep = [&](auto ksc) {
      constexpr int ks = decltype(ksc)::value;
      v8i wf[WN_T];
#pragma unroll
      for (int j = 0; j < WN_T; ++j) {
        const int r = wn * WN_T * 32 + j * 32 + r32;
        const v4i v = *reinterpret_cast<const v4i*>(lw + r * 64 + 16 * ((2 * ks + h) ^ swz64(r)));
        wf[j] = v8i{v[0], v[1], v[2], v[3], 0, 0, 0, 0};
      }
#pragma unroll
      for (int i = 0; i < WM_T; ++i) {
        // the FP8 operand's 32 bytes per lane: k 64 ks + 16 h + [0, 16), then
        // k 64 ks + 32 + 16 h + [0, 16)
        const int r = wm * WM_T * 32 + i * 32 + r32;
        const v4i lo = *reinterpret_cast<const v4i*>(la + r * 128 + 16 * ((4 * ks + h) ^ swz128(r)));
        const v4i hi = *reinterpret_cast<const v4i*>(la + r * 128 + 16 * ((4 * ks + 2 + h) ^ swz128(r)));
        const v8i af = v8i{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
        if constexpr (P2) {
          // lane half 0 holds the first 16-blocks of both 32-groups, half 1
          // the second ones: pass 1 keeps half 0, pass 2 half 1
          const int keep = h == 0 ? -1 : 0;
          const v8i a0 = af & keep, a1 = af & ~keep;
#pragma unroll
          for (int j = 0; j < WN_T; ++j) {
            acc[j][i] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(wf[j], a0, acc[j][i], 4, 0, ks, we[j], 0,
                                                                         kUnitScale);
            acc[j][i] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(wf[j], a1, acc[j][i], 4, 0, ks, wo[j], 0,
                                                                         kUnitScale);
          }
        } else {
#pragma unroll
          for (int j = 0; j < WN_T; ++j)
            acc[j][i] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(wf[j], af, acc[j][i], 4, 0, ks, we[j], 0,
                                                                         kUnitScale);
        }
      }
    };
    substep(std::integral_constant<int, 0>{});
    substep(std::integral_constant<int, 1>{});
  };
  // lane: core row wm * 128 + 32 i + r32 of the tile, features
  // wn * 64 + 32 j + 8 g + 4 h + 0..3
  auto epilogue = [&](int logical) {
    int tm, tn;
    grouped_tile(logical, tiles_m, tiles_n, tm, tn);
    const int m0 = tm * BM, n0 = tn * BN;
    const bool full_n = n0 + BN <= N && (N & 3) == 0;
#pragma unroll
    for (int i = 0; i < WM_T; ++i) {
      const int m = m0 + wm * WM_T * 32 + i * 32 + r32;
      if (m >= C) continue;
#pragma unroll
      for (int j = 0; j < WN_T; ++j)
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          const int n = n0 + wn * WN_T * 32 + j * 32 + 8 * g + 4 * h;
          float* dst = Y + (int64_t)m * N + n;
          const v16f& a = acc[j][i];
          if (full_n) {
            *reinterpret_cast<float4*>(dst) = make_float4(a[4 * g], a[4 * g + 1], a[4 * g + 2], a[4 * g + 3]);
          } else {
            for (int r = 0; r < 4 && n + r < N; ++r) dst[r] = a[4 * g + r];
          }
        }
    }
  };
  int ckt = 0, clogical = seq.first;
  auto finish_stage = [&]() {
    if (++ckt == nk) {
      epilogue(clogical);
      zero_acc();
      ckt = 0;
      clogical += seq.stride;
    }
  };
  Stage ra;
  load(ra);
  store(ra, 0);
  lds_barrier();
  int g = 0;
  for (; g + 1 < G; g += 2) {
    load(ra);
    compute(0);
    finish_stage();
    store(ra, 1);
    lds_barrier();
    if (g + 2 < G) load(ra);
    compute(1);
    finish_stage();
    if (g + 2 < G) store(ra, 0);
    lds_barrier();
  }
  if (g < G) {
    compute(0);
    finish_stage();
  }
}

template <bool P2>
static hipError_t launch_dq_core_t(const uint8_t* core, const uint8_t* wc, const uint8_t* ws, float* yc, int64_t C,
                                   int64_t N, int64_t K, hipStream_t s) {
  constexpr size_t lds = 2 * (size_t)(256 * 128 + 256 * 64 + 256 * (P2 ? 16 : 8));
  hipError_t e = set_dynamic_lds_once<k_gemm_dq_core<P2>>(lds);
  if (e != hipSuccess) return e;
  const int64_t tiles = ((C + 255) / 256) * ((N + 255) / 256);
  hipLaunchKernelGGL(k_gemm_dq_core<P2>, dim3((unsigned)persistent_grid(tiles)), dim3(512), lds, s, core, wc, ws, yc,
                     (int)C, (int)N, (int)K);
  return hipGetLastError();
}

hipError_t launch_gemm_dq_core(const uint8_t* core, const uint8_t* wc, const uint8_t* ws, int fmt, float* yc,
                               int64_t C, int64_t N, int64_t K, hipStream_t s) {
  if (!dq_core_fp8_applies(fmt, C, N, K)) return hipErrorNotSupported;
  return fmt == kNvfp4P2 ? launch_dq_core_t<true>(core, wc, ws, yc, C, N, K, s)
                         : launch_dq_core_t<false>(core, wc, ws, yc, C, N, K, s);
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
