// gemm_i8.hip -- INT8 activations x INT4 weights on gfx950 int8 MFMA.
//
// The INT8 path of 6Bit-Diffusion's mixed-precision linear layers (summary
// on vetunion.cn, section one: INT8 activations for unstable steps; section
// four: 4-bit weights, "W4A6").  Both operands are block-Hadamard rotated, so
// Y = X W^T is computed directly on the codes:
//   acc[m][n] = sum_k qx[m][k] * qw[n][k]   (exact, int32)
//   y[m][n]   = fl32(fl32(float(acc) * sx[m]) * sw[n]).
//
// Design (CDNA4):
//  * v_mfma_i32_32x32x32_i8: 32x32 output, 16 int8 of K per lane per operand.
//    The instruction's A operand is a 32-row slice of W and its B operand a
//    32-row slice of X, so each output lane holds one token row m and four
//    consecutive output features n (8- or 16-byte stores).
//  * INT4 weights stay packed in LDS and are unpacked to int8 after the
//    fragment read: nibble q is placed in the high half of its byte (value
//    16 q), the interleaved low/high nibbles are put back in k order with two
//    v_perm_b32, and the epilogue divides the exact int32 sum by 16
//    (|16 acc| < 2^31 for K < 150000).
//  * Two kernels.  The pipelined one (K % 128 == 0, every CogVideoX shape):
//    256 x 256 tiles, 8 waves (two per SIMD), LDS-DMA buffer loads two stages
//    ahead into three LDS stages with XOR-swizzled rows, and the two waves of
//    each SIMD alternating between LDS-read and MFMA phases (ping-pong); see
//    gemm_i8_pipe.h.  The fallback (any K % 32 == 0):
//    4 waves as 2 x 2, 64-byte LDS rows with 16-byte chunk c of row r at
//    chunk c ^ ((r >> 1) & 3), K advancing 64 bytes per double-buffered
//    stage.
//  * Tile order (xcd_tile): workgroup i runs on XCD i % 8, each XCD takes a
//    contiguous range of a grouped order (4 tile rows walked column by
//    column), so the ~32 tiles an XCD runs at once share 4 X panels and 8 W
//    panels in its L2.
#include "gemm_i8_pipe.h"
#include "hdq_device.h"
#include "hdq_internal.h"

#include <atomic>

namespace hdq {

// Persistent GEMMs leave two CUs per XCD free: their workgroups each fill a
// CU's register file, so without free CUs no kernel on another stream (such as the
// previous-step difference pass) could run beside them.  On MI355X the
// GEMMs are power-bound, and 240 workgroups run them as fast as 256.
int64_t persistent_grid(int64_t tiles) {
  static std::atomic<int> cus[64];  // per device; 0 = not read yet
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) dev = 0;
  int n = cus[dev].load(std::memory_order_relaxed);
  if (n == 0) {
    int cu = 0;
    if (hipDeviceGetAttribute(&cu, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cu < 8)
      cu = 256;
    const int free_cus = cu >= 128 ? 16 : 0;
    n = (cu & ~7) - free_cus;
    if (n < 8) n = cu & ~7;
    cus[dev].store(n, std::memory_order_relaxed);
  }
  return tiles <= n ? tiles : n;
}

template <int WM, int WN>
__global__ __launch_bounds__(256) void k_gemm_i8i4(
    const int8_t* __restrict__ X, const float* __restrict__ sx, const uint8_t* __restrict__ W4,
    const float* __restrict__ sw, void* __restrict__ Y, int out_dtype, int M, int N, int K,
    const int32_t* __restrict__ decision, int32_t want) {
  if (decision != nullptr && *decision != want) return;
  constexpr int BM = 64 * WM, BN = 64 * WN, BK = 64;
  constexpr int XCH = BM * (BK / 16) / 256;  // X 16-byte chunks per thread per stage
  constexpr int WCH = BN * (BK / 32) / 256;  // packed W 16-byte chunks per thread per stage
  static_assert(XCH >= 1 && WCH >= 1, "tile too small for 256 threads");
  __shared__ __attribute__((aligned(16))) int8_t lds[2][(BM + BN) * BK];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave & 1, wn = wave >> 1;
  const int tiles_m = (M + BM - 1) / BM, tiles_n = (N + BN - 1) / BN;
  int tm, tn;
  xcd_tile(tiles_m, tiles_n, tm, tn);
  const int m0 = tm * BM, n0 = tn * BN;
  const int64_t ldw = K >> 1;

  uint4 xr[XCH], wr[WCH];
  auto load_stage = [&](int k0) {
#pragma unroll
    for (int p = 0; p < XCH; ++p) {
      const int q = tid + 256 * p, r = q >> 2, c = q & 3;
      const int m = m0 + r, k = k0 + 16 * c;
      xr[p] = (m < M && k < K) ? *reinterpret_cast<const uint4*>(X + (int64_t)m * K + k)
                               : make_uint4(0u, 0u, 0u, 0u);
    }
#pragma unroll
    for (int p = 0; p < WCH; ++p) {
      const int q = tid + 256 * p, r = q >> 1, c = q & 1;
      const int n = n0 + r, k = k0 + 32 * c;
      wr[p] = (n < N && k < K)
                  ? *reinterpret_cast<const uint4*>(W4 + (int64_t)n * ldw + (k >> 1))
                  : make_uint4(0u, 0u, 0u, 0u);
    }
  };
  auto store_stage = [&](int buf) {
    int8_t* lx = lds[buf];
    int8_t* lw = lds[buf] + BM * BK;
#pragma unroll
    for (int p = 0; p < XCH; ++p) {
      const int q = tid + 256 * p, r = q >> 2, c = q & 3;
      *reinterpret_cast<uint4*>(lx + lds_off64(r, c)) = xr[p];
    }
#pragma unroll
    for (int p = 0; p < WCH; ++p) {
      const int q = tid + 256 * p, r = q >> 1, c = q & 1;
      uint4 lo, hi;
      unpack_int4x32(wr[p], lo, hi);
      *reinterpret_cast<uint4*>(lw + lds_off64(r, 2 * c)) = lo;
      *reinterpret_cast<uint4*>(lw + lds_off64(r, 2 * c + 1)) = hi;
    }
  };

  v16i acc[WN][WM];
#pragma unroll
  for (int j = 0; j < WN; ++j)
#pragma unroll
    for (int i = 0; i < WM; ++i)
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[j][i][e] = 0;

  const int nk = (K + BK - 1) / BK;
  load_stage(0);
  store_stage(0);
  __syncthreads();
  for (int kt = 0; kt < nk; ++kt) {
    if (kt + 1 < nk) load_stage((kt + 1) * BK);
    const int8_t* lx = lds[kt & 1];
    const int8_t* lw = lds[kt & 1] + BM * BK;
#pragma unroll
    for (int ks = 0; ks < BK / 32; ++ks) {
      const int c = 2 * ks + (lane >> 5);
      v4i xf[WM], wf[WN];
#pragma unroll
      for (int i = 0; i < WM; ++i)
        xf[i] = *reinterpret_cast<const v4i*>(lx + lds_off64(wm * WM * 32 + i * 32 + (lane & 31), c));
#pragma unroll
      for (int j = 0; j < WN; ++j)
        wf[j] = *reinterpret_cast<const v4i*>(lw + lds_off64(wn * WN * 32 + j * 32 + (lane & 31), c));
#pragma unroll
      for (int j = 0; j < WN; ++j)
#pragma unroll
        for (int i = 0; i < WM; ++i)
          acc[j][i] = __builtin_amdgcn_mfma_i32_32x32x32_i8(wf[j], xf[i], acc[j][i], 0, 0, 0);
    }
    if (kt + 1 < nk) store_stage((kt + 1) & 1);
    __syncthreads();
  }

  // Epilogue: lane holds token m = ... + (lane & 31) and, for g = 0..3,
  // features n = 8g + 4 (lane >> 5) + 0..3 of its 32 x 32 subtile.
  const bool vec = (N & 3) == 0;
#pragma unroll
  for (int i = 0; i < WM; ++i) {
    const int m = m0 + wm * WM * 32 + i * 32 + (lane & 31);
    if (m >= M) continue;
    const float sxm = sx[m];
#pragma unroll
    for (int j = 0; j < WN; ++j) {
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int n = n0 + wn * WN * 32 + j * 32 + 8 * g + 4 * (lane >> 5);
        if (n >= N) continue;
        int32_t a[4];
#pragma unroll
        for (int r = 0; r < 4; ++r) a[r] = acc[j][i][4 * g + r] >> 4;
        const int64_t off = (int64_t)m * N + n;
        if (out_dtype == kOutI32) {
          int32_t* yp = reinterpret_cast<int32_t*>(Y) + off;
          if (vec && n + 3 < N) {
            *reinterpret_cast<int4*>(yp) = make_int4(a[0], a[1], a[2], a[3]);
          } else {
            for (int r = 0; r < 4 && n + r < N; ++r) yp[r] = a[r];
          }
          continue;
        }
        float y[4];
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const float t = (float)a[r] * sxm;
          y[r] = (n + r < N) ? t * sw[n + r] : 0.0f;
        }
        if (out_dtype == kOutF32) {
          float* yp = reinterpret_cast<float*>(Y) + off;
          if (vec && n + 3 < N) {
            *reinterpret_cast<float4*>(yp) = make_float4(y[0], y[1], y[2], y[3]);
          } else {
            for (int r = 0; r < 4 && n + r < N; ++r) yp[r] = y[r];
          }
        } else {
          uint16_t* yp = reinterpret_cast<uint16_t*>(Y) + off;
          if (vec && n + 3 < N) {
            *reinterpret_cast<uint2*>(yp) = make_uint2(pack_bf16x2(y[0], y[1]), pack_bf16x2(y[2], y[3]));
          } else {
            for (int r = 0; r < 4 && n + r < N; ++r)
              yp[r] = __builtin_bit_cast(uint16_t, (__bf16)y[r]);
          }
        }
      }
    }
  }
}

// The gated kernel around the pipelined body (gemm_i8_pipe.h).
template <int WAVES_M, int WAVES_N, int WM_T, int WN_T, int OUT>
__global__ __launch_bounds__(64 * WAVES_M * WAVES_N) void k_gemm_i8i4_pipe(
    const int8_t* __restrict__ X, const float* __restrict__ sx, const uint8_t* __restrict__ W4,
    const float* __restrict__ sw, void* __restrict__ Y, int M, int N, int K,
    const int32_t* __restrict__ decision, int32_t want) {
  if (decision != nullptr && *decision != want) return;
  gemm_i8i4_pipe_body<WAVES_M, WAVES_N, WM_T, WN_T, OUT>(X, sx, W4, sw, Y, M, N, K);
}

template <int WAVES_M, int WAVES_N, int WM_T, int WN_T, int OUT>
static hipError_t launch_pipe(const int8_t* x, const float* sx, const uint8_t* w4, const float* sw,
                              void* y, int64_t M, int64_t N, int64_t K, const int32_t* decision,
                              int32_t want, hipStream_t s) {
  using C = I8Cfg<WAVES_M, WAVES_N, WM_T, WN_T>;
  constexpr size_t lds = (size_t)C::LDS;
  auto kern = k_gemm_i8i4_pipe<WAVES_M, WAVES_N, WM_T, WN_T, OUT>;
  hipError_t e = set_dynamic_lds_once<k_gemm_i8i4_pipe<WAVES_M, WAVES_N, WM_T, WN_T, OUT>>(lds);
  if (e != hipSuccess) return e;
  const int64_t tiles = ((M + C::BM - 1) / C::BM) * ((N + C::BN - 1) / C::BN);
  const int64_t grid = persistent_grid(tiles);
  hipLaunchKernelGGL(kern, dim3((unsigned)grid), dim3(C::THREADS), lds, s, x, sx, w4, sw, y, (int)M,
                     (int)N, (int)K, decision, want);
  return hipGetLastError();
}

// 8 waves as 2 (tokens) x 4 (features), each 128 x 64: two waves per SIMD,
// the fastest of the layouts measured on the CogVideoX shapes.

static hipError_t launch_pipe_out(const int8_t* x, const float* sx, const uint8_t* w4, const float* sw,
                                  void* y, int out_dtype, int64_t M, int64_t N, int64_t K,
                                  const int32_t* decision, int32_t want, hipStream_t s) {
  if (out_dtype == kOutF32) return launch_pipe<2, 4, 4, 2, kOutF32>(x, sx, w4, sw, y, M, N, K, decision, want, s);
  if (out_dtype == kOutBf16) return launch_pipe<2, 4, 4, 2, kOutBf16>(x, sx, w4, sw, y, M, N, K, decision, want, s);
  return launch_pipe<2, 4, 4, 2, kOutI32>(x, sx, w4, sw, y, M, N, K, decision, want, s);
}

hipError_t launch_gemm_i8i4(const int8_t* x, const float* sx, const uint8_t* w4, const float* sw,
                            void* y, int out_dtype, int64_t M, int64_t N, int64_t K,
                            const int32_t* decision, int32_t want, hipStream_t s) {
  // The pipelined kernel addresses each operand with 32-bit buffer offsets.
  if (K % 128 == 0 && M * K < (1ll << 31) && N * K / 2 < (1ll << 31))
    return launch_pipe_out(x, sx, w4, sw, y, out_dtype, M, N, K, decision, want, s);
  constexpr int WM = 4, WN = 2;
  constexpr int BM = 64 * WM, BN = 64 * WN;
  const int64_t tiles = ((M + BM - 1) / BM) * ((N + BN - 1) / BN);
  hipLaunchKernelGGL((k_gemm_i8i4<WM, WN>), dim3((unsigned)tiles), dim3(256), 0, s, x, sx, w4, sw, y,
                     out_dtype, (int)M, (int)N, (int)K, decision, want);
  return hipGetLastError();
}

}  // namespace hdq
