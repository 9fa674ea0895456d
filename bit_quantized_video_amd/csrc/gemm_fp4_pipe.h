// gemm_fp4_pipe.h -- the pipelined MX-compatible NVFP4 GEMM body on the block-scaled FP4 MFMA
// (gfx950), shared by the gated kernel and the precision dispatch kernel.
// See gemm_fp4.hip for the design.
#ifndef HDQ_GEMM_FP4_PIPE_H
#define HDQ_GEMM_FP4_PIPE_H

#include "hdq_device.h"
#include "hdq_internal.h"

#include <type_traits>

namespace hdq {

// Power-of-two E4M3 byte (0x01, 0x02, 0x04 subnormal; 8..0x7e normal) -> E8M0.
__device__ __forceinline__ uint32_t e4m3_pow2_to_e8m0(uint32_t b) {
  return b >= 8u ? (b >> 3) + 120u : 118u + (31u - (uint32_t)__builtin_clz(b | 1u));
}

// ---------------------------------------------------------------------------
// Pipelined kernel for K % 256 == 0: the INT8 kernel's structure (256 x 256
// tiles, 8 waves as 2 x 4 of 128 x 64, a persistent tile loop, prefetch
// across tile boundaries, double-buffered LDS) with 256 K per stage: stage
// g + 1 is loaded while stage g is computed, its code bytes by LDS-DMA into
// the other buffer and its scale bytes through a register (they are
// converted to E8M0 on the way into LDS).  Per stage:
// 128-byte code rows (swz128; substep s of 64 K gives lane half h chunk
// 2s + h) and, per row, the stage's eight E8M0 bytes (one per 32 K, from the
// even E4M3 byte of each MX pair) stored as two words, [g0 g2 g4 g6] and
// [g1 g3 g5 g7]: lane half h reads word h once per stage and substep s takes
// its byte through the instruction's scale byte select.
//
// P2 (NVFP4 with a power-of-two scale per 16-block): each 32-group's two
// 16-blocks have their own scales, so every MFMA runs twice, once with the
// X fragment's second half zeroed and the first block's scales, once with
// its first half zeroed and the second block's: exact, at twice the MFMA
// work.  Per row and stage the 16 E8M0 bytes are stored as four words:
// first blocks of lane half 0's and 1's groups, then their second blocks.

template <int KS>
__device__ __forceinline__ v16f mfma_fp4(const v8i& a, const v8i& b, const v16f& c, int sa, int sb) {
  return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, 4, 4, KS, sa, KS, sb);
}

// LDS bytes of the pipelined FP4 body: two stages of codes and E8M0 words.
template <bool P2>
constexpr int fp4_pipe_lds() {
  return 2 * (256 * 128 * 2 + 512 * (P2 ? 16 : 8));
}

// ADD: the output also gets the broadcast core term of `add` (N % 4 == 0).
template <int OUT, bool P2 = false, bool ADD = false>
__device__ __forceinline__ void gemm_fp4mx_pipe_body(
    const uint8_t* __restrict__ xc, const uint8_t* __restrict__ xsc, const float* __restrict__ xts,
    const uint8_t* __restrict__ wc, const uint8_t* __restrict__ wsc, const float* __restrict__ wts,
    void* __restrict__ Y, int M, int N, int K, int nwg = 0, const CoreAdd* add = nullptr) {
  constexpr int BM = 256, BN = 256, BK = 256, WM_T = 4, WN_T = 2;
  constexpr int XB = BM * BK / 2, WB = BN * BK / 2;  // code bytes per stage
  constexpr int SCB = P2 ? 16 : 8;                    // E8M0 bytes per row and stage
  constexpr int SB = XB + WB + (BM + BN) * SCB;       // + E8M0 bytes
  static_assert(2 * SB == fp4_pipe_lds<P2>(), "LDS size");
  constexpr int kOutPitch = BN * 2 + 16;              // bf16 output row staged in LDS
  static_assert(BM / 2 * kOutPitch <= SB, "half an output tile must fit one pipeline buffer");
  extern __shared__ __attribute__((aligned(1024))) uint8_t smem[];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave % 2, wn = wave / 2;
  const int tiles_m = (M + BM - 1) / BM, tiles_n = (N + BN - 1) / BN;
  const TileSeq seq = tile_seq(tiles_m * tiles_n, nwg);
  const int nk = K / BK;
  const int G = seq.count * nk;
  if (G == 0) return;
  const int ld = K / 2, lds_ = K / 16;

  // Code bytes go straight to LDS by LDS-DMA: instruction p of wave w fills
  // LDS rows 64 p + 8 w + (lane >> 3), slot lane & 7, with the row's 16-byte
  // chunk (lane & 7) ^ swz128(row), the swizzled layout the fragment reads
  // expect.  The swizzle depends on the lane and the wave only, so the four
  // instructions per operand differ by scalar offsets.
  const int drow = 8 * wave + (lane >> 3);
  const uint32_t dvoff = (uint32_t)(drow * ld + 16 * ((lane & 7) ^ swz128(drow)));
  // scales: waves 0-3 take the 256 X rows, waves 4-7 the 256 W rows
  const int sw_ = __builtin_amdgcn_readfirstlane(tid >> 8), srow = tid & 255;
  const uint32_t svoff = (uint32_t)(srow * lds_);
  const int sdst = XB + WB + sw_ * BM * SCB + srow * SCB;

  int l_logical = seq.first, l_kt = 0;
  __amdgpu_buffer_rsrc_t xres, wres, sres;
  auto open_tile = [&]() {
    int tm, tn;
    grouped_tile(l_logical, tiles_m, tiles_n, tm, tn);
    const int m0 = tm * BM, n0 = tn * BN;
    xres = make_rsrc(xc + (int64_t)m0 * ld, (uint32_t)((int64_t)(M - m0) * ld));
    wres = make_rsrc(wc + (int64_t)n0 * ld, (uint32_t)((int64_t)(N - n0) * ld));
    sres = sw_ ? make_rsrc(wsc + (int64_t)n0 * lds_, (uint32_t)((int64_t)(N - n0) * lds_))
               : make_rsrc(xsc + (int64_t)m0 * lds_, (uint32_t)((int64_t)(M - m0) * lds_));
  };
  open_tile();
  // Issues the next stage's loads: 8 LDS-DMA instructions per wave into
  // buffer buf, then this thread's 16 scale bytes into a register (sc), the
  // last of the wave's 9 vector memory operations.
  uint4 sc;
  int l_rev = 0;  // this tile's K stages in descending order (every other tile)
  auto issue = [&](int buf) {
    uint8_t* base = smem + buf * SB + 1024 * wave;
    const int kt = l_rev ? nk - 1 - l_kt : l_kt;
#pragma unroll
    for (int p = 0; p < 4; ++p) lds_dma16(xres, base + 8192 * p, dvoff, kt * (BK / 2) + p * 64 * ld);
#pragma unroll
    for (int p = 0; p < 4; ++p) lds_dma16(wres, base + XB + 8192 * p, dvoff, kt * (BK / 2) + p * 64 * ld);
    sc = buf_load16(sres, svoff, kt * (BK / 16));
    if (++l_kt == nk) {
      l_kt = 0;
      l_rev ^= 1;
      l_logical += seq.stride;
      if (l_logical < tiles_m * tiles_n) open_tile();
    }
  };
  // Writes the staged scale bytes to buffer buf as E8M0 words.
  auto store_sc = [&](int buf) {
    uint8_t* base = smem + buf * SB;
    // E8M0 of group g comes from E4M3 byte 2g (P2: and 2g + 1); word h holds
    // g = h, h+2, h+4, h+6
    const uint32_t d[4] = {sc.x, sc.y, sc.z, sc.w};
    uint32_t w0 = 0u, w1 = 0u, w2 = 0u, w3 = 0u;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      w0 |= e4m3_pow2_to_e8m0(d[q] & 0xffu) << (8 * q);
      w1 |= e4m3_pow2_to_e8m0((d[q] >> 16) & 0xffu) << (8 * q);
      if constexpr (P2) {
        w2 |= e4m3_pow2_to_e8m0((d[q] >> 8) & 0xffu) << (8 * q);
        w3 |= e4m3_pow2_to_e8m0(d[q] >> 24) << (8 * q);
      }
    }
    if constexpr (P2)
      *reinterpret_cast<uint4*>(base + sdst) = make_uint4(w0, w1, w2, w3);
    else
      *reinterpret_cast<uint2*>(base + sdst) = make_uint2(w0, w1);
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
    const uint8_t* lxs = lx + XB + WB;
    const uint8_t* lws = lxs + BM * SCB;
    int xe[WM_T], we[WN_T], xo[WM_T], wo[WN_T];  // xo, wo: the second blocks' (P2)
#pragma unroll
    for (int i = 0; i < WM_T; ++i) {
      const uint8_t* p = lxs + (wm * WM_T * 32 + i * 32 + r32) * SCB + 4 * h;
      xe[i] = *reinterpret_cast<const int*>(p);
      if constexpr (P2) xo[i] = *reinterpret_cast<const int*>(p + 8);
    }
#pragma unroll
    for (int j = 0; j < WN_T; ++j) {
      const uint8_t* p = lws + (wn * WN_T * 32 + j * 32 + r32) * SCB + 4 * h;
      we[j] = *reinterpret_cast<const int*>(p);
      if constexpr (P2) wo[j] = *reinterpret_cast<const int*>(p + 8);
    }
    auto substep = [&](auto ksc) {
      constexpr int ks = decltype(ksc)::value;
      const int g = 2 * ks + h;  // this lane's 32-K group within the stage
      auto load_w = [&](v8i (&wf)[WN_T]) {
#pragma unroll
        for (int j = 0; j < WN_T; ++j) {
          const int r = wn * WN_T * 32 + j * 32 + r32;
          const v4i v = *reinterpret_cast<const v4i*>(lw + r * 128 + 16 * (g ^ swz128(r)));
          wf[j] = v8i{v[0], v[1], v[2], v[3], 0, 0, 0, 0};
        }
      };
      v8i wf[WN_T];
      if constexpr (P2) {
        // one X fragment at a time: its two halves are two operands
        load_w(wf);
#pragma unroll
        for (int i = 0; i < WM_T; ++i) {
          const int r = wm * WM_T * 32 + i * 32 + r32;
          const v4i v = *reinterpret_cast<const v4i*>(lx + r * 128 + 16 * (g ^ swz128(r)));
          const v8i xf = v8i{v[0], v[1], 0, 0, 0, 0, 0, 0};
          const v8i xg = v8i{0, 0, v[2], v[3], 0, 0, 0, 0};
#pragma unroll
          for (int j = 0; j < WN_T; ++j) {
            acc[j][i] = mfma_fp4<ks>(wf[j], xf, acc[j][i], we[j], xe[i]);
            acc[j][i] = mfma_fp4<ks>(wf[j], xg, acc[j][i], wo[j], xo[i]);
          }
        }
      } else {
        v8i xf[WM_T];
#pragma unroll
        for (int i = 0; i < WM_T; ++i) {
          const int r = wm * WM_T * 32 + i * 32 + r32;
          const v4i v = *reinterpret_cast<const v4i*>(lx + r * 128 + 16 * (g ^ swz128(r)));
          xf[i] = v8i{v[0], v[1], v[2], v[3], 0, 0, 0, 0};
        }
        load_w(wf);
#pragma unroll
        for (int j = 0; j < WN_T; ++j)
#pragma unroll
          for (int i = 0; i < WM_T; ++i) acc[j][i] = mfma_fp4<ks>(wf[j], xf[i], acc[j][i], we[j], xe[i]);
      }
    };
    substep(std::integral_constant<int, 0>{});
    substep(std::integral_constant<int, 1>{});
    substep(std::integral_constant<int, 2>{});
    substep(std::integral_constant<int, 3>{});
  };

  const float scale = (*xts) * (*wts);
  // fragment (i, j, g) of this lane: row wm * WM_T * 32 + 32 i + r32 of the
  // tile, columns wn * WN_T * 32 + 32 j + 8 g + 4 h + 0..3.  The core rows and
  // scales of the lane's WM_T rows are looked up once per tile.
  const float* crow[WM_T];
  float ccs[WM_T];
  auto core_rows = [&](int m0) {
    if constexpr (ADD) {
#pragma unroll
      for (int i = 0; i < WM_T; ++i) {
        const int m = m0 + wm * WM_T * 32 + i * 32 + r32;
        crow[i] = nullptr;
        ccs[i] = 0.0f;
        if (m < M) {
          const int cb = dq_cube(m, add->g);
          crow[i] = add->yc + (int64_t)cb * N;
          ccs[i] = add->cs[cb];
        }
      }
    }
  };
  // The core terms of row i's 4 * WN_T column groups, loaded together before
  // they are used (one wait per row instead of one per group).
  auto core_load = [&](int n0, int i, float4 (&cv)[WN_T][4]) {
#pragma unroll
    for (int j = 0; j < WN_T; ++j)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int n = n0 + wn * WN_T * 32 + j * 32 + 8 * g + 4 * h;
        cv[j][g] = crow[i] != nullptr && n < N ? *reinterpret_cast<const float4*>(crow[i] + n)
                                               : make_float4(0.0f, 0.0f, 0.0f, 0.0f);
      }
  };
  auto core_add = [&](const float4& c, int i, float (&y)[4]) {
    const float cs = ccs[i], stw = *add->wts;
    y[0] = y[0] + (c.x * cs) * stw;
    y[1] = y[1] + (c.y * cs) * stw;
    y[2] = y[2] + (c.z * cs) * stw;
    y[3] = y[3] + (c.w * cs) * stw;
  };
  auto epilogue = [&](int logical, int buf) {
    int tm, tn;
    grouped_tile(logical, tiles_m, tiles_n, tm, tn);
    const int m0 = tm * BM, n0 = tn * BN;
    if constexpr (ADD) core_rows(m0);
    if constexpr (OUT == kOutBf16) {
      // Stage the bf16 tile in LDS buffer buf, which this stage's compute has
      // finished with (the other buffer is receiving the next stage), half a
      // tile at a time: half hh holds fragment rows i = 2 hh, 2 hh + 1 of every
      // wave, tile rows hh * 64 + 0..63 and 128 + hh * 64 + 0..63, as local rows
      // 0..127.  Then whole 512-byte rows are written with 16-byte stores.
      // The barriers wait for LDS accesses only: the next stage's DMA loads
      // stay in flight.
      uint8_t* const stage = smem + buf * SB;
      uint16_t* y16 = reinterpret_cast<uint16_t*>(Y);
      const int n = n0 + 8 * (tid & 31);
      const bool vec = n + 8 <= N && (N & 7) == 0;
#pragma unroll
      for (int hh = 0; hh < 2; ++hh) {
        lds_only_barrier();
        uint8_t* const lrow = stage + (wm * 64 + r32) * kOutPitch + 2 * (wn * WN_T * 32 + 4 * h);
#pragma unroll
        for (int ii = 0; ii < 2; ++ii) {
          const int i = 2 * hh + ii;
          float4 cv[ADD ? WN_T : 1][4];
          if constexpr (ADD) core_load(n0, i, cv);
#pragma unroll
          for (int j = 0; j < WN_T; ++j)
#pragma unroll
            for (int g = 0; g < 4; ++g) {
              const v16f& a = acc[j][i];
              if constexpr (ADD) {
                float y[4] = {a[4 * g] * scale, a[4 * g + 1] * scale, a[4 * g + 2] * scale, a[4 * g + 3] * scale};
                core_add(cv[j][g], i, y);
                *reinterpret_cast<uint2*>(lrow + ii * 32 * kOutPitch + 2 * (j * 32 + 8 * g)) =
                    make_uint2(pack_bf16x2(y[0], y[1]), pack_bf16x2(y[2], y[3]));
              } else {
                *reinterpret_cast<uint2*>(lrow + ii * 32 * kOutPitch + 2 * (j * 32 + 8 * g)) =
                    make_uint2(pack_bf16x2(a[4 * g] * scale, a[4 * g + 1] * scale),
                               pack_bf16x2(a[4 * g + 2] * scale, a[4 * g + 3] * scale));
              }
            }
        }
        lds_only_barrier();
#pragma unroll 4
        for (int r = tid >> 5; r < BM / 2; r += 16) {
          const uint8_t* src = stage + r * kOutPitch + 16 * (tid & 31);
          const int tr = (r >> 6) * 128 + hh * 64 + (r & 63);
          if (m0 + tr < M) {
            uint16_t* dst = y16 + (int64_t)(m0 + tr) * N + n;
            if (vec) {
              store16_nt(dst, src);
            } else {
              for (int e = 0; e < 8 && n + e < N; ++e) dst[e] = reinterpret_cast<const uint16_t*>(src)[e];
            }
          }
        }
      }
      // The caller's stage barrier orders these LDS reads before the buffer
      // is refilled.
    } else {
      const bool full_n = n0 + BN <= N && (N & 3) == 0;
#pragma unroll
      for (int i = 0; i < WM_T; ++i) {
        const int m = m0 + wm * WM_T * 32 + i * 32 + r32;
        if (m >= M) continue;
        float4 cv[ADD ? WN_T : 1][4];
        if constexpr (ADD) core_load(n0, i, cv);
#pragma unroll
        for (int j = 0; j < WN_T; ++j) {
#pragma unroll
          for (int g = 0; g < 4; ++g) {
            const int n = n0 + wn * WN_T * 32 + j * 32 + 8 * g + 4 * h;
            const int64_t off = (int64_t)m * N + n;
            float y[4];
#pragma unroll
            for (int r = 0; r < 4; ++r) y[r] = acc[j][i][4 * g + r] * scale;
            if constexpr (ADD) core_add(cv[j][g], i, y);
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

  int ckt = 0, clogical = seq.first;
  auto finish_stage = [&](int buf) {
    if (++ckt == nk) {
      epilogue(clogical, buf);
      zero_acc();
      ckt = 0;
      clogical += seq.stride;
    }
  };

  // Stage g lives in LDS buffer g % 2.  Stage g + 1 is issued at the start
  // of stage g's compute, into the buffer every wave finished reading before
  // the last stage barrier; the stage barrier after the compute waits for this
  // wave's DMA loads and LDS writes (vmcnt and lgkmcnt zero), so after it the
  // whole stage is in LDS.
  issue(0);
  store_sc(0);
  stage_barrier();
  int g = 0;
  for (; g + 1 < G; g += 2) {
    issue(1);
    compute(0);
    finish_stage(0);
    store_sc(1);
    stage_barrier();
    if (g + 2 < G) issue(0);
    compute(1);
    finish_stage(1);
    if (g + 2 < G) store_sc(0);
    stage_barrier();
  }
  if (g < G) {
    compute(0);
    finish_stage(0);
  }
}

}  // namespace hdq

#endif  // HDQ_GEMM_FP4_PIPE_H
