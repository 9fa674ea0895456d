// gemm_i8_pipe.h -- the pipelined INT8 x INT4 GEMM body (gfx950), shared by
// the gated INT8 kernel and the single-launch precision dispatch kernel.
// See gemm_i8.hip for the design.
#ifndef HDQ_GEMM_I8_PIPE_H
#define HDQ_GEMM_I8_PIPE_H

#include "hdq_device.h"
#include "hdq_internal.h"

#include <type_traits>

namespace hdq {

// 32 packed INT4 (uint4) -> 32 int8 holding 16 * q, in k order.
__device__ __forceinline__ void unpack_int4x32(const uint4 p, uint4& lo, uint4& hi) {
  const uint32_t d[4] = {p.x, p.y, p.z, p.w};
  uint32_t o[8];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const uint32_t even = (d[i] << 4) & 0xf0f0f0f0u;  // k = 8i, 8i+2, 8i+4, 8i+6
    const uint32_t odd = d[i] & 0xf0f0f0f0u;          // k = 8i+1, ...
    o[2 * i] = __builtin_amdgcn_perm(odd, even, 0x05010400u);
    o[2 * i + 1] = __builtin_amdgcn_perm(odd, even, 0x07030602u);
  }
  lo = make_uint4(o[0], o[1], o[2], o[3]);
  hi = make_uint4(o[4], o[5], o[6], o[7]);
}

// ---------------------------------------------------------------------------
// Pipelined kernel for K % 128 == 0 (every CogVideoX shape).
//  * Workgroup tile BM tokens x BN features; WAVES_M x WAVES_N waves, each
//    wave WM_T x WN_T subtiles of 32 x 32.  With 8 waves (two per SIMD) one
//    wave's LDS / global / barrier waits overlap the other wave's MFMAs.
//  * K advances 128 per stage.  Operands go from global memory straight to
//    LDS with LDS-DMA buffer loads (no register staging, no LDS writes by
//    the waves), into three LDS stage buffers: stage kt + 2 is issued at the
//    start of stage kt, into the buffer of stage kt - 1, so two stages of
//    compute cover its latency.
//  * Ping-pong phases: a stage is two pairs of 64 K, and each pair is a
//    memory phase (this wave's fragment reads and W unpack; for the first
//    pair also the DMA issue) followed by a compute phase (its 16 MFMAs),
//    with a workgroup barrier after every phase.  Waves 0-3 and 4-7 (one of
//    each per SIMD, as waves are dealt to SIMDs round-robin) run one phase
//    apart: group 1 passes one extra barrier at the start of a tile and
//    group 0 one at the end.  So while one wave of a SIMD reads LDS and
//    unpacks, the other issues MFMAs, and the matrix core always has work.
//    (With both waves in the same phase, both waited for their LDS reads
//    after every barrier.)
//  * Rows past M or N read as zero (buffer range); their outputs are not
//    stored.  X rows are 128 bytes in LDS (swz128), packed INT4 W rows 64
//    bytes (swz64).  Within a stage, k-substep pair p
//    (64 K) gives lane half h the K range [64p + 32h, +32): for W one
//    16-byte read of packed nibbles unpacked to the two substeps' fragments,
//    for X two 16-byte reads.  (Any assignment of K to lanes works as long as
//    both operands use the same one.)

template <int WAVES_M, int WAVES_N, int WM_T, int WN_T>
struct I8Cfg {
  static constexpr int THREADS = 64 * WAVES_M * WAVES_N;
  static constexpr int BM = WAVES_M * WM_T * 32, BN = WAVES_N * WN_T * 32, BK = 128;
  static constexpr int XB = BM * BK, SB = XB + BN * BK / 2;  // LDS bytes per stage
  static constexpr int OUT_PITCH = BN * 2 + 16;              // bf16 output row in LDS, padded
  static constexpr int NS = 3;                                // LDS stage buffers
  static constexpr int LDS = (NS * SB > BM * OUT_PITCH) ? NS * SB : BM * OUT_PITCH;
  // LDS-DMA instructions (1 KB each) per wave and stage: X, then W
  static constexpr int XI = XB / 1024 / (THREADS / 64), WI = BN * BK / 2 / 1024 / (THREADS / 64);
  static_assert(THREADS == 512 && BM == 256 && BN == 256, "the DMA row mapping assumes 8 waves, 256 x 256");
};

template <int WAVES_M, int WAVES_N, int WM_T, int WN_T, int OUT>
__device__ __forceinline__ void gemm_i8i4_pipe_body(
    const int8_t* __restrict__ X, const float* __restrict__ sx, const uint8_t* __restrict__ W4,
    const float* __restrict__ sw, void* __restrict__ Y, int M, int N, int K, int nwg = 0) {
  using C = I8Cfg<WAVES_M, WAVES_N, WM_T, WN_T>;
  constexpr int BM = C::BM, BN = C::BN, BK = C::BK, XB = C::XB, SB = C::SB;
  constexpr int kOutPitch = C::OUT_PITCH;
  extern __shared__ __attribute__((aligned(1024))) uint8_t smem[];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave % WAVES_M, wn = wave / WAVES_M;
  const int tiles_m = (M + BM - 1) / BM, tiles_n = (N + BN - 1) / BN;
  const TileSeq seq = tile_seq(tiles_m * tiles_n, nwg);
  const int nk = K / BK;
  const int ldw = K >> 1;

  // LDS-DMA staging: one wave instruction writes 1 KB of LDS, lane i's 16
  // bytes at byte 16 i.  X instruction p of wave w fills LDS rows
  // 64p + 8w + (i >> 3), slot i & 7, with logical chunk (i & 7) ^ swz128(row):
  // the swizzled layout the fragment reads expect.  W instruction p fills
  // rows 128p + 16w + (i >> 2), slot i & 3, with chunk (i & 3) ^ swz64(row).
  // Both swizzles depend on the lane only, so the instructions of a stage
  // differ by scalar offsets.
  const int xrow = 8 * wave + (lane >> 3), wrow = 16 * wave + (lane >> 2);
  const uint32_t xvoff = (uint32_t)(xrow * K + 16 * ((lane & 7) ^ swz128(xrow)));
  const uint32_t wvoff = (uint32_t)(wrow * ldw + 16 * ((lane & 3) ^ swz64(wrow)));
  __amdgpu_buffer_rsrc_t xres, wres;  // over the current tile's rows
  // Every other tile of a workgroup runs its K stages in descending order,
  // so it starts on the K slices the tiles before it loaded last, which are
  // still in this XCD's L2 (int32 sums do not depend on the order).
  int krev = 0;
  auto issue = [&](int kt0, int buf) {
    const int kt = krev ? nk - 1 - kt0 : kt0;
    uint8_t* base = smem + buf * SB + 1024 * wave;
#pragma unroll
    for (int p = 0; p < C::XI; ++p) lds_dma16(xres, base + 8192 * p, xvoff, kt * BK + p * 64 * K);
#pragma unroll
    for (int p = 0; p < C::WI; ++p) lds_dma16(wres, base + XB + 8192 * p, wvoff, kt * (BK / 2) + p * 128 * ldw);
  };

  v16i acc[WN_T][WM_T];
  auto zero_acc = [&]() {
#pragma unroll
    for (int j = 0; j < WN_T; ++j)
#pragma unroll
      for (int i = 0; i < WM_T; ++i)
#pragma unroll
        for (int e = 0; e < 16; ++e) acc[j][i][e] = 0;
  };
  zero_acc();

  const int h = lane >> 5, r32 = lane & 31;
  // Memory phase of k-substep pair p of the stage in LDS buffer buf: the X
  // fragments and the unpacked W fragments into registers.  The reads have
  // completed when it returns, so the buffer may be refilled after the next
  // barrier.
  v4i xf[WM_T][2], wf[WN_T][2];
  auto load_frags = [&](int buf, int p) {
    const uint8_t* lx = smem + buf * SB;
    const uint8_t* lw = lx + XB;
#pragma unroll
    for (int i = 0; i < WM_T; ++i) {
      const int r = wm * WM_T * 32 + i * 32 + r32;
#pragma unroll
      for (int s = 0; s < 2; ++s)
        xf[i][s] = *reinterpret_cast<const v4i*>(lx + r * 128 + 16 * ((4 * p + 2 * h + s) ^ swz128(r)));
    }
#pragma unroll
    for (int j = 0; j < WN_T; ++j) {
      const int r = wn * WN_T * 32 + j * 32 + r32;
      const uint4 packed = *reinterpret_cast<const uint4*>(lw + r * 64 + 16 * ((2 * p + h) ^ swz64(r)));
      uint4 lo, hi;
      unpack_int4x32(packed, lo, hi);
      wf[j][0] = v4i{(int)lo.x, (int)lo.y, (int)lo.z, (int)lo.w};
      wf[j][1] = v4i{(int)hi.x, (int)hi.y, (int)hi.z, (int)hi.w};
    }
    wait_lds();
  };
  // Compute phase: the pair's 16 MFMAs.
  auto mfmas = [&]() {
#pragma unroll
    for (int j = 0; j < WN_T; ++j) {
#pragma unroll
      for (int i = 0; i < WM_T; ++i)
        acc[j][i] = __builtin_amdgcn_mfma_i32_32x32x32_i8(wf[j][0], xf[i][0], acc[j][i], 0, 0, 0);
#pragma unroll
      for (int i = 0; i < WM_T; ++i)
        acc[j][i] = __builtin_amdgcn_mfma_i32_32x32x32_i8(wf[j][1], xf[i][1], acc[j][i], 0, 0, 0);
    }
  };
  const int grp = __builtin_amdgcn_readfirstlane(wave >> 2);

  // Epilogue of one tile: lane holds token m = ... + (lane & 31) and, for
  // g = 0..3, features n = 8g + 4h + 0..3 of each 32 x 32 subtile.
  auto epilogue = [&](int logical) {
    int tm, tn;
    grouped_tile(logical, tiles_m, tiles_n, tm, tn);
    const int m0 = tm * BM, n0 = tn * BN;
    if constexpr (OUT == kOutBf16) {
      // Stage the bf16 tile in LDS (the stage buffers are free at a tile
      // boundary once every wave is past the last stage), then write whole
      // rows: 32 lanes x 16 bytes per 512-byte row.
      lds_barrier();
      // Scales through buffer loads: rows past M and columns past N read 0.
      const __amdgpu_buffer_rsrc_t sxres = make_rsrc(sx, (uint32_t)M * 4u);
      const __amdgpu_buffer_rsrc_t swres = make_rsrc(sw, (uint32_t)N * 4u);
      const int rl0 = wm * WM_T * 32 + r32, nl0 = wn * WN_T * 32 + 4 * h;
      uint8_t* const lrow = smem + rl0 * kOutPitch + 2 * nl0;
#pragma unroll
      for (int i = 0; i < WM_T; ++i) {
        // acc = 16 * (the exact integer sum) and float(acc) is 16 times its
        // float, so float(acc) * (s_x / 16) is the same real product as
        // float(acc >> 4) * s_x: the same float, without the shifts (s_x / 16
        // is exact: s_x is 0 or at least 2^-107)
        const float sxm = 0.0625f * __builtin_bit_cast(
            float, __builtin_amdgcn_raw_buffer_load_b32(sxres, 4 * (rl0 + i * 32), 4 * m0, 0));
#pragma unroll
        for (int j = 0; j < WN_T; ++j) {
#pragma unroll
          for (int g = 0; g < 4; ++g) {
            const float4 swn = __builtin_bit_cast(
                float4, __builtin_amdgcn_raw_buffer_load_b128(swres, 4 * (nl0 + j * 32 + 8 * g), 4 * n0, 0));
            const float y0 = ((float)acc[j][i][4 * g + 0] * sxm) * swn.x;
            const float y1 = ((float)acc[j][i][4 * g + 1] * sxm) * swn.y;
            const float y2 = ((float)acc[j][i][4 * g + 2] * sxm) * swn.z;
            const float y3 = ((float)acc[j][i][4 * g + 3] * sxm) * swn.w;
            *reinterpret_cast<uint2*>(lrow + i * 32 * kOutPitch + 2 * (j * 32 + 8 * g)) =
                make_uint2(pack_bf16x2(y0, y1), pack_bf16x2(y2, y3));
          }
        }
      }
      lds_barrier();
      uint16_t* y16 = reinterpret_cast<uint16_t*>(Y);
      const int n = n0 + 8 * (tid & 31);
      const bool vec = n + 8 <= N && (N & 7) == 0;
#pragma unroll 4
      for (int r = tid >> 5; r < BM; r += C::THREADS / 32) {
        const uint8_t* src = smem + r * kOutPitch + 16 * (tid & 31);
        if (m0 + r < M) {
          uint16_t* dst = y16 + (int64_t)(m0 + r) * N + n;
          if (vec) {
            store16_nt(dst, src);
          } else {
            for (int e = 0; e < 8 && n + e < N; ++e) dst[e] = reinterpret_cast<const uint16_t*>(src)[e];
          }
        }
      }
      lds_barrier();  // the next stage may overwrite the staged tile
      return;
    }
    const bool full_n = n0 + BN <= N && (N & 3) == 0;
#pragma unroll
    for (int i = 0; i < WM_T; ++i) {
      const int m = m0 + wm * WM_T * 32 + i * 32 + r32;
      if (m >= M) continue;
      const float sxm = sx[m];
#pragma unroll
      for (int j = 0; j < WN_T; ++j) {
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          const int n = n0 + wn * WN_T * 32 + j * 32 + 8 * g + 4 * h;
          const int64_t off = (int64_t)m * N + n;
          int32_t a[4];
#pragma unroll
          for (int r = 0; r < 4; ++r) a[r] = acc[j][i][4 * g + r] >> 4;
          if (full_n) {
            if constexpr (OUT == kOutI32) {
              *reinterpret_cast<int4*>(reinterpret_cast<int32_t*>(Y) + off) = make_int4(a[0], a[1], a[2], a[3]);
            } else {
              const float4 swn = *reinterpret_cast<const float4*>(sw + n);
              const float y0 = ((float)a[0] * sxm) * swn.x, y1 = ((float)a[1] * sxm) * swn.y;
              const float y2 = ((float)a[2] * sxm) * swn.z, y3 = ((float)a[3] * sxm) * swn.w;
              if constexpr (OUT == kOutF32)
                *reinterpret_cast<float4*>(reinterpret_cast<float*>(Y) + off) = make_float4(y0, y1, y2, y3);
              else
                *reinterpret_cast<uint2*>(reinterpret_cast<uint16_t*>(Y) + off) =
                    make_uint2(pack_bf16x2(y0, y1), pack_bf16x2(y2, y3));
            }
          } else {
            for (int r = 0; r < 4; ++r) {
              if (n + r >= N) break;
              if constexpr (OUT == kOutI32) {
                reinterpret_cast<int32_t*>(Y)[off + r] = a[r];
              } else {
                const float y = ((float)a[r] * sxm) * sw[n + r];
                if constexpr (OUT == kOutF32)
                  reinterpret_cast<float*>(Y)[off + r] = y;
                else
                  reinterpret_cast<uint16_t*>(Y)[off + r] = __builtin_bit_cast(uint16_t, (__bf16)y);
              }
            }
          }
        }
      }
    }
    // Every wave is past the last stage before the next tile's first stages
    // are issued into the stage buffers (one of which the last stage used
    // unless nk is a multiple of three).
    lds_barrier();
  };

  // Persistent loop over this workgroup's tiles.  Per tile, stages 0 and 1
  // are issued and stage 0 waited for (stage 1's loads, C::XI + C::WI per
  // wave, may stay in flight).  Stage kt: memory phase of pair 0 with the
  // issue of stage kt + 2 into the buffer of kt - 1, compute, memory phase of
  // pair 1, compute, a barrier after each phase.  Stage kt + 1 is waited for
  // before the barrier after which group 0 reads it: group 0 waits after its
  // last compute phase of stage kt, group 1 after its last memory phase.
  // The buffer of kt - 1 is last read by group 1's second memory phase of
  // kt - 1, which ends before the barrier that opens group 0's first phase
  // of kt.  Unrolled by three, so each buffer index is a constant.
  //
  // Barriers per tile: 1 + 4 nk + 1 for every wave (the extra one at the
  // start for group 1, at the end for group 0).
  for (int t = 0; t < seq.count; ++t) {
    const int logical = seq.first + t * seq.stride;
    krev = t & 1;
    {
      int tm, tn;
      grouped_tile(logical, tiles_m, tiles_n, tm, tn);
      const int m0 = tm * BM, n0 = tn * BN;
      xres = make_rsrc(X + (int64_t)m0 * K, (uint32_t)((int64_t)(M - m0) * K));
      wres = make_rsrc(W4 + (int64_t)n0 * ldw, (uint32_t)((int64_t)(N - n0) * ldw));
    }
    issue(0, 0);
    if (nk > 1) {
      issue(1, 1);
      dma_barrier<C::XI + C::WI>();
    } else {
      dma_barrier<0>();
    }
    if (grp == 1) phase_barrier();
    auto wait_next = [&](int kt) {
      if (kt + 2 < nk)
        wait_vmem<C::XI + C::WI>();
      else if (kt + 1 < nk)
        wait_vmem<0>();
    };
    auto step = [&](int kt, auto bufc) {
      constexpr int b = decltype(bufc)::value;
      load_frags(b, 0);
      if (kt + 2 < nk) issue(kt + 2, (b + 2) % 3);
      phase_barrier();
      mfmas();
      phase_barrier();
      load_frags(b, 1);
      if (grp == 1) wait_next(kt);
      phase_barrier();
      mfmas();
      if (grp == 0) wait_next(kt);
      phase_barrier();
    };
    for (int kt = 0; kt < nk; kt += 3) {
      step(kt, std::integral_constant<int, 0>{});
      if (kt + 1 < nk) step(kt + 1, std::integral_constant<int, 1>{});
      if (kt + 2 < nk) step(kt + 2, std::integral_constant<int, 2>{});
    }
    if (grp == 0) phase_barrier();
    epilogue(logical);
    zero_acc();
  }
}

}  // namespace hdq

#endif  // HDQ_GEMM_I8_PIPE_H
