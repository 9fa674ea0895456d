// gemm_bf16_pipe.h -- the pipelined bf16-MFMA GEMM body (gfx950) for exact
// NVFP4 (decoded to bf16 while staged) and the bf16 fallback, shared by the
// gated kernel and the precision dispatch kernel.  See gemm_bf16.hip.
#ifndef HDQ_GEMM_BF16_PIPE_H
#define HDQ_GEMM_BF16_PIPE_H

#include "hdq_device.h"
#include "hdq_internal.h"

namespace hdq {

// kSrcNvfp4X: X as the exact bf16 values of its NVFP4 codes (decoded
// beforehand), W as NVFP4 codes decoded here.
enum Src : int { kSrcBf16 = 0, kSrcNvfp4 = 1, kSrcNvfp4X = 2 };

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

// ---------------------------------------------------------------------------
// Pipelined kernel for K % 64 == 0: 256 x 256 tile, 8 waves as 2 (tokens) x
// 4 (features), each 128 x 64 (4 x 2 subtiles of 32 x 32), 64 K per stage,
// double-buffered LDS, a persistent tile loop and bf16 output tiles staged
// in LDS -- the structure of the INT8 kernel.  bf16 operands go into LDS by
// LDS-DMA one stage ahead; NVFP4 operands come through two register sets
// prefetching the next two stages (buffer loads: rows past M or N read as
// zero, LDS-only barriers) and are decoded to exact bf16 when the registers
// are written to LDS, once per workgroup rather than once per wave.  LDS
// holds bf16: 128-byte rows per stage (swz128), substep s (16 K) giving lane
// half h the 16-byte chunk 2s + h.
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
template <>
struct Bf16Stage<kSrcNvfp4X> {
  uint4 w;            // 32 W codes per thread
  uint32_t ws;        // their two E4M3 block scales
};

template <int SRC, int OUT>
__device__ __forceinline__ void gemm_bf16_pipe_body(
    const void* __restrict__ X, const uint8_t* __restrict__ xsc, const float* __restrict__ xts,
    const void* __restrict__ W, const uint8_t* __restrict__ wsc, const float* __restrict__ wts,
    void* __restrict__ Y, int M, int N, int K, int nwg = 0) {
  constexpr int BM = 256, BN = 256, BK = 64, WM_T = 4, WN_T = 2;
  constexpr int XB = BM * BK * 2, SB = XB + BN * BK * 2;  // LDS bytes per stage
  constexpr int kOutPitch = kBf16OutPitch;                // bf16 output row staged in LDS
  using Stage = Bf16Stage<SRC>;
  extern __shared__ __attribute__((aligned(1024))) uint8_t smem[];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave % 2, wn = wave / 2;
  const int tiles_m = (M + BM - 1) / BM, tiles_n = (N + BN - 1) / BN;
  const TileSeq seq = tile_seq(tiles_m * tiles_n, nwg);
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
    } else if constexpr (SRC == kSrcNvfp4X) {
      const int64_t ldx = 2 * (int64_t)K, ld = K / 2, lds_ = K / 16;
      xres = make_rsrc(reinterpret_cast<const uint8_t*>(X) + m0 * ldx, (uint32_t)((M - m0) * ldx));
      wres = make_rsrc(reinterpret_cast<const uint8_t*>(W) + n0 * ld, (uint32_t)((N - n0) * ld));
      wsres = make_rsrc(wsc + n0 * lds_, (uint32_t)((N - n0) * lds_));
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
    } else if constexpr (SRC == kSrcNvfp4X) {
      st.w = buf_load16(wres, wvoff, kt * 32);
      st.ws = __builtin_amdgcn_raw_buffer_load_b16(wsres, (int)svoff, kt * 4, 0);
    } else {
      st.x = buf_load16(xres, xvoff, kt * 32);
      st.w = buf_load16(wres, wvoff, kt * 32);
      st.xs = __builtin_amdgcn_raw_buffer_load_b16(xsres, (int)svoff, kt * 4, 0);
      st.ws = __builtin_amdgcn_raw_buffer_load_b16(wsres, (int)svoff, kt * 4, 0);
    }
  };
  // LDS-DMA of stage kt (bf16 operands) into buffer buf: instruction p of
  // wave w fills LDS rows 64 p + 8 w + (lane >> 3), slot lane & 7, with the
  // row's 16-byte chunk (lane & 7) ^ swz128(row), the layout the fragment
  // reads expect; the swizzle depends on the lane and the wave only.
  const int drow = 8 * wave + (lane >> 3);
  const uint32_t dvoff = (uint32_t)(drow * 2 * K + 16 * ((lane & 7) ^ swz128(drow)));
  // The scheduling barrier keeps the loads where they are issued, ahead of
  // the stage's compute: left to itself the compiler sinks some of them
  // (their LDS destination provably differs from what the compute reads)
  // to just before the stage barrier, which then waits out their latency.
  auto issue_dma = [&](int kt, int buf) {
    uint8_t* base = smem + buf * SB + 1024 * wave;
#pragma unroll
    for (int p = 0; p < 4; ++p) lds_dma16(xres, base + 8192 * p, dvoff, kt * 128 + p * 64 * 2 * K);
    if constexpr (SRC == kSrcBf16) {
#pragma unroll
      for (int p = 0; p < 4; ++p) lds_dma16(wres, base + XB + 8192 * p, dvoff, kt * 128 + p * 64 * 2 * K);
    }
    __builtin_amdgcn_sched_barrier(0);
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
    } else if constexpr (SRC == kSrcNvfp4X) {
      const int r = tid >> 1, c = tid & 1;
      uint4 d[4];
      decode_nvfp4x16(make_uint2(st.w.x, st.w.y), st.ws & 0xffu, d[0], d[1]);
      decode_nvfp4x16(make_uint2(st.w.z, st.w.w), st.ws >> 8, d[2], d[3]);
#pragma unroll
      for (int q = 0; q < 4; ++q)
        *reinterpret_cast<uint4*>(lw + r * 128 + 16 * ((4 * c + q) ^ swz128(r))) = d[q];
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

  // NVFP4 (decoded here or beforehand): the two tensor scales; bf16: none.
  const float scale = (SRC != kSrcBf16 || xts != nullptr) ? (*xts) * (*wts) : 1.0f;
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
            store16_nt(dst16, src);
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
      // Every wave is past the last stage (in buffer 0 when nk is odd) before
      // the next tile's first stage is stored there.
      lds_barrier();
    }
  };

  // Persistent loop over this workgroup's tiles; per tile, the K-stages run
  // through the two-stage register prefetch and the double-buffered LDS.
  for (int t = 0; t < seq.count; ++t) {
    int tm, tn;
    grouped_tile(seq.first + t * seq.stride, tiles_m, tiles_n, tm, tn);
    const int m0 = tm * BM, n0 = tn * BN;
    open_tile(m0, n0);
    if constexpr (SRC == kSrcBf16) {
      // bf16 operands need no decoding: stage kt + 1 goes straight into LDS
      // by LDS-DMA while stage kt is computed, and the stage barrier waits
      // for this wave's DMA loads (vmcnt) and LDS reads.
      int kt = 0;
      issue_dma(0, 0);
      stage_barrier();
      for (; kt + 1 < nk; kt += 2) {
        issue_dma(kt + 1, 1);
        compute(0);
        stage_barrier();
        if (kt + 2 < nk) issue_dma(kt + 2, 0);
        compute(1);
        stage_barrier();
      }
      if (kt < nk) compute(0);
      epilogue(m0, n0);
      zero_acc();
      continue;
    }
    if constexpr (SRC == kSrcNvfp4X) {
      // X (decoded bf16) by LDS-DMA and W's codes through one register set,
      // both one stage ahead: stage kt + 1's DMA and W loads are issued
      // before stage kt is computed, W is decoded into the other buffer
      // after it, and the stage barrier waits for all of them.
      Stage ra;
      int kt = 0;
      issue_dma(0, 0);
      load(ra, 0);
      store(ra, 0);
      stage_barrier();
      for (; kt + 1 < nk; kt += 2) {
        issue_dma(kt + 1, 1);
        load(ra, kt + 1);
        compute(0);
        store(ra, 1);
        stage_barrier();
        if (kt + 2 < nk) {
          issue_dma(kt + 2, 0);
          load(ra, kt + 2);
        }
        compute(1);
        if (kt + 2 < nk) store(ra, 0);
        stage_barrier();
      }
      if (kt < nk) compute(0);
      epilogue(m0, n0);
      zero_acc();
      continue;
    }
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

}  // namespace hdq

#endif  // HDQ_GEMM_BF16_PIPE_H
