// quant.hip -- block-Hadamard rotation fused with quantization (gfx950).
//
// The summary of 6Bit-Diffusion (vetunion.cn, section one) rotates each
// linear layer's activations with a block Hadamard transform to spread
// outliers before quantizing them to INT8 or NVFP4, and (section four) fuses
// the transform with the quantizer in one kernel.  Here the rotation never
// touches memory: a row streams HBM -> registers, is rotated with the
// in-register / cross-lane butterfly of hdq_device.h, scaled, quantized and
// written as codes.  Both kernels are HBM-bound (2 B read, 1 or 0.5625 B
// written per element).
//
//  * k_quant_int_rows: INT8 per token (or INT4 per output channel for
//    weights).  The per-row absmax needs the whole rotated row before the
//    first code, so one workgroup owns one row and keeps it in registers
//    (CPT 8-element chunks per thread).
//  * k_quant_nvfp4: NVFP4 needs only the tensor amax (given) and a 16- or
//    32-element block max (E4M3 scale per 16, or a power of two per 16 or
//    per 32), so it is a flat grid-stride kernel with no
//    workgroup synchronisation; each wave owns 128 consecutive chunks per
//    iteration (two per lane, loads issued first).
#include "hdq_device.h"
#include "hdq_internal.h"

#include <math.h>

namespace hdq {

float hadamard_scale(int hb) { return (float)(1.0 / sqrt((double)hb)); }

// ---------------------------------------------------------------- INT8/INT4

// Packs the low byte of four floats' bit patterns.
__device__ __forceinline__ uint32_t low_bytes4(uint32_t a, uint32_t b, uint32_t c, uint32_t d) {
  const uint32_t ab = __builtin_amdgcn_perm(b, a, 0x0c0c0400u);
  const uint32_t cd = __builtin_amdgcn_perm(d, c, 0x04000c0cu);
  return ab | cd;
}

// STATS (INT8 only): also the selection statistics of the current input,
// one partial per row, struct-of-arrays (psum[row] = sum |x|, pbits[row] =
// max bf16 magnitude bits, ptmax[row] = the row's max |rotated x|, which is
// the row absmax the quantizer needs anyway), so selection and quantization
// read x once.  HB > 0: the Hadamard block is HB (the argument is ignored),
// so the rotation's block-size branches fold away at compile time.
template <int BLOCK, int CPT, bool INT4, bool STATS = false, int HB = 0>
__global__ __launch_bounds__(BLOCK) void k_quant_int_rows(
    const uint16_t* __restrict__ x, int64_t cols, int hb_arg, float c_b, void* __restrict__ codes,
    float* __restrict__ row_scale, const int32_t* __restrict__ decision, int32_t want,
    double* __restrict__ psum = nullptr, uint32_t* __restrict__ pbits = nullptr,
    float* __restrict__ ptmax = nullptr) {
  if (decision != nullptr && *decision != want) return;
  const int hb = HB > 0 ? HB : hb_arg;
  const int64_t row = blockIdx.x;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int64_t nch = cols >> 3;
  const uint4* xr = reinterpret_cast<const uint4*>(x + row * cols);

  // Lane tid holds chunk fwht_src(c * BLOCK + tid) of the row: whole
  // Hadamard blocks sit in aligned lane groups (BLOCK is a multiple of 16
  // lanes), and a block past the row end is entirely zero-filled.
  float v[CPT][8];
  float maxabs = 0.0f;
  double sumabs = 0.0;
#pragma unroll
  for (int c = 0; c < CPT; ++c) {
    const int64_t idx = fwht_src((int64_t)c * BLOCK + tid, lane, hb);
    uint4 w = make_uint4(0u, 0u, 0u, 0u);
    if (idx < nch) w = xr[idx];
    bf16x8_to_f32(w, v[c]);
  }
  if constexpr (STATS) {
    // max |x| with IEEE-2019 maximum, which propagates NaN (v_maximum3_f32
    // takes two elements per instruction)
#pragma unroll
    for (int c = 0; c < CPT; ++c) {
      float s8 = 0.0f;
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        maxabs = __builtin_elementwise_maximum(maxabs, fabsf(v[c][i]));
        s8 += fabsf(v[c][i]);
      }
      sumabs += s8;
    }
  }
  float amax = 0.0f;
#pragma unroll
  for (int c = 0; c < CPT; ++c) {
    const float sc = fwht8(v[c], lane, hb) * c_b;  // sign * c_b: exact
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      v[c][i] = v[c][i] * sc;
      amax = fmaxf(amax, fabsf(v[c][i]));
    }
  }
  amax = wave_max(amax);
  if constexpr (BLOCK > 64) {
    __shared__ float red[BLOCK / 64];
    if (lane == 0) red[tid >> 6] = amax;
    __syncthreads();
    amax = red[0];
#pragma unroll
    for (int w = 1; w < BLOCK / 64; ++w) amax = fmaxf(amax, red[w]);
  }
  if constexpr (STATS) {
    // bf16 widens to float exactly: |x|'s top 16 bits are its bf16 pattern
    // (a NaN's are above every number's)
    uint32_t maxbits = __float_as_uint(maxabs) >> 16;
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) {
      sumabs += __shfl_xor(sumabs, o);
      maxbits = max(maxbits, (uint32_t)__shfl_xor((int)maxbits, o));
    }
    __shared__ double rs[BLOCK / 64];
    __shared__ uint32_t rb[BLOCK / 64];
    if (lane == 0) {
      rs[tid >> 6] = sumabs;
      rb[tid >> 6] = maxbits;
    }
    __syncthreads();
    if (tid == 0) {
      double sa = rs[0];
      uint32_t mb = rb[0];
      for (int w = 1; w < BLOCK / 64; ++w) {
        sa += rs[w];
        mb = max(mb, rb[w]);
      }
      psum[row] = sa;
      pbits[row] = mb;
      ptmax[row] = amax;
    }
  }
  constexpr float QMAX = INT4 ? 7.0f : 127.0f;
  float inv = 0.0f, s = 0.0f;
  if (amax >= kTiny) {
    s = amax / QMAX;
    inv = QMAX / amax;
  }
  if (tid == 0) row_scale[row] = s;

  // q = round_half_even(y * inv): adding 1.5 * 2^23 rounds to an integer
  // (the add rounds to nearest even) and leaves it, two's complement, in the
  // low mantissa bits.  |y * inv| <= 127.00001 (7.000001), so no clamp can
  // trigger.
  const float kMagic = 12582912.0f;
#pragma unroll
  for (int c = 0; c < CPT; ++c) {
    const int64_t idx = fwht_src((int64_t)c * BLOCK + tid, lane, hb);
    if (idx < nch) {
      uint32_t b[8];
#pragma unroll
      for (int i = 0; i < 8; ++i) b[i] = __float_as_uint(v[c][i] * inv + kMagic);
      if constexpr (INT4) {
        uint32_t p = 0;
#pragma unroll
        for (int i = 0; i < 8; ++i) p |= (b[i] & 0xfu) << (4 * i);
        reinterpret_cast<uint32_t*>(codes)[row * (cols >> 3) + idx] = p;
      } else {
        uint2 p;
        p.x = low_bytes4(b[0], b[1], b[2], b[3]);
        p.y = low_bytes4(b[4], b[5], b[6], b[7]);
        reinterpret_cast<uint2*>(codes)[row * (cols >> 3) + idx] = p;
      }
    }
  }
}

template <int BLOCK, int CPT>
static hipError_t launch_int_rows_t(const uint16_t* x, int64_t rows, int64_t cols, int hb,
                                    bool int4, void* codes, float* sc, const int32_t* dec,
                                    int32_t want, hipStream_t s) {
  const float c_b = hadamard_scale(hb);
  if (int4)
    hipLaunchKernelGGL((k_quant_int_rows<BLOCK, CPT, true>), dim3((unsigned)rows), dim3(BLOCK), 0,
                       s, x, cols, hb, c_b, codes, sc, dec, want);
  else if (hb == 128)
    hipLaunchKernelGGL((k_quant_int_rows<BLOCK, CPT, false, false, 128>), dim3((unsigned)rows), dim3(BLOCK), 0,
                       s, x, cols, hb, c_b, codes, sc, dec, want);
  else
    hipLaunchKernelGGL((k_quant_int_rows<BLOCK, CPT, false>), dim3((unsigned)rows), dim3(BLOCK), 0,
                       s, x, cols, hb, c_b, codes, sc, dec, want);
  return hipGetLastError();
}

template <int BLOCK, int CPT>
static hipError_t launch_select_q8_t(const uint16_t* x, int64_t rows, int64_t cols, int hb,
                                     void* codes, float* sc, double* psum, uint32_t* pbits,
                                     float* ptmax, hipStream_t s) {
  if (hb == 128)
    hipLaunchKernelGGL((k_quant_int_rows<BLOCK, CPT, false, true, 128>), dim3((unsigned)rows), dim3(BLOCK), 0,
                       s, x, cols, hb, hadamard_scale(hb), codes, sc, nullptr, 0, psum, pbits, ptmax);
  else
    hipLaunchKernelGGL((k_quant_int_rows<BLOCK, CPT, false, true>), dim3((unsigned)rows), dim3(BLOCK), 0,
                       s, x, cols, hb, hadamard_scale(hb), codes, sc, nullptr, 0, psum, pbits, ptmax);
  return hipGetLastError();
}

// Threads per row for CPT chunks each: the smallest instantiated multiple
// of 64 that covers the row.
template <int CPT>
static hipError_t launch_select_q8_cpt(const uint16_t* x, int64_t rows, int64_t cols, int hb,
                                       void* codes, float* sc, double* psum, uint32_t* pbits,
                                       float* ptmax, hipStream_t s) {
  const int64_t nch = cols >> 3;
#define HDQ_SQ8_CASE(B) \
  if (nch <= (B) * CPT) return launch_select_q8_t<B, CPT>(x, rows, cols, hb, codes, sc, psum, pbits, ptmax, s);
  HDQ_SQ8_CASE(64)
  HDQ_SQ8_CASE(128)
  HDQ_SQ8_CASE(192)
  HDQ_SQ8_CASE(256)
  HDQ_SQ8_CASE(384)
  HDQ_SQ8_CASE(512)
  HDQ_SQ8_CASE(768)
  HDQ_SQ8_CASE(1024)
#undef HDQ_SQ8_CASE
  return hipErrorInvalidValue;
}

hipError_t launch_quant_int8_stats(const uint16_t* x, int64_t rows, int64_t cols, int hb, void* codes,
                                   float* row_scale, double* psum, uint32_t* pbits, float* ptmax,
                                   hipStream_t s) {
  // The rows kept in registers, up to 16384 columns (beyond, callers take
  // the two-pass route), two chunks per thread: the statistics need
  // registers of their own, and more chunks per thread measured slower.
  if ((cols >> 3) > 2048) return hipErrorInvalidValue;
  return launch_select_q8_cpt<2>(x, rows, cols, hb, codes, row_scale, psum, pbits, ptmax, s);
}

// Two-pass variant for rows too long to keep in registers: pass one finds
// the rotated absmax, pass two re-reads the row (from L2) and quantizes.
template <bool INT4>
__global__ __launch_bounds__(256) void k_quant_int_rows_long(
    const uint16_t* __restrict__ x, int64_t cols, int hb, float c_b, void* __restrict__ codes,
    float* __restrict__ row_scale, const int32_t* __restrict__ decision, int32_t want) {
  if (decision != nullptr && *decision != want) return;
  const int64_t row = blockIdx.x;
  const int tid = threadIdx.x, lane = tid & 63;
  const int64_t nch = cols >> 3;
  const uint4* xr = reinterpret_cast<const uint4*>(x + row * cols);
  float amax = 0.0f;
  for (int64_t base = 0; base < nch; base += 256) {
    const int64_t idx = fwht_src(base + tid, lane, hb);
    float v[8];
    uint4 w = make_uint4(0u, 0u, 0u, 0u);
    if (idx < nch) w = xr[idx];
    bf16x8_to_f32(w, v);
    const float sc = fwht8(v, lane, hb) * c_b;
#pragma unroll
    for (int i = 0; i < 8; ++i) amax = fmaxf(amax, fabsf(v[i] * sc));
  }
  amax = wave_max(amax);
  __shared__ float red[4];
  if (lane == 0) red[tid >> 6] = amax;
  __syncthreads();
  amax = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
  constexpr float QMAX = INT4 ? 7.0f : 127.0f;
  float inv = 0.0f, s = 0.0f;
  if (amax >= kTiny) {
    s = amax / QMAX;
    inv = QMAX / amax;
  }
  if (tid == 0) row_scale[row] = s;
  const float kMagic = 12582912.0f;
  for (int64_t base = 0; base < nch; base += 256) {
    const int64_t idx = fwht_src(base + tid, lane, hb);
    float v[8];
    uint4 w = make_uint4(0u, 0u, 0u, 0u);
    if (idx < nch) w = xr[idx];
    bf16x8_to_f32(w, v);
    const float sc = fwht8(v, lane, hb) * c_b;
    if (idx < nch) {
      uint32_t b[8];
#pragma unroll
      for (int i = 0; i < 8; ++i) b[i] = __float_as_uint((v[i] * sc) * inv + kMagic);
      if constexpr (INT4) {
        uint32_t p = 0;
#pragma unroll
        for (int i = 0; i < 8; ++i) p |= (b[i] & 0xfu) << (4 * i);
        reinterpret_cast<uint32_t*>(codes)[row * nch + idx] = p;
      } else {
        uint2 p;
        p.x = low_bytes4(b[0], b[1], b[2], b[3]);
        p.y = low_bytes4(b[4], b[5], b[6], b[7]);
        reinterpret_cast<uint2*>(codes)[row * nch + idx] = p;
      }
    }
  }
}

hipError_t launch_quant_int_rows(const uint16_t* x, int64_t rows, int64_t cols, int hb, int fmt,
                                 void* codes, float* row_scale, const int32_t* decision,
                                 int32_t want, hipStream_t s) {
  const bool int4 = (fmt == kInt4Row);
  const int64_t nch = cols >> 3;
  // Workgroup = 64 threads for short rows, 256 otherwise; each thread keeps
  // CPT chunks of 8 elements of its row in registers.
  if (nch <= 64) return launch_int_rows_t<64, 1>(x, rows, cols, hb, int4, codes, row_scale, decision, want, s);
  if (nch <= 128) return launch_int_rows_t<64, 2>(x, rows, cols, hb, int4, codes, row_scale, decision, want, s);
  if (nch <= 256) return launch_int_rows_t<64, 4>(x, rows, cols, hb, int4, codes, row_scale, decision, want, s);
  if (nch <= 384) return launch_int_rows_t<128, 3>(x, rows, cols, hb, int4, codes, row_scale, decision, want, s);
  if (nch <= 512) return launch_int_rows_t<256, 2>(x, rows, cols, hb, int4, codes, row_scale, decision, want, s);
  if (nch <= 768) return launch_int_rows_t<256, 3>(x, rows, cols, hb, int4, codes, row_scale, decision, want, s);
  if (nch <= 1024) return launch_int_rows_t<256, 4>(x, rows, cols, hb, int4, codes, row_scale, decision, want, s);
  if (nch <= 1536) return launch_int_rows_t<256, 6>(x, rows, cols, hb, int4, codes, row_scale, decision, want, s);
  if (nch <= 2048) return launch_int_rows_t<256, 8>(x, rows, cols, hb, int4, codes, row_scale, decision, want, s);
  const float c_b = hadamard_scale(hb);
  if (int4)
    hipLaunchKernelGGL(k_quant_int_rows_long<true>, dim3((unsigned)rows), dim3(256), 0, s, x, cols,
                       hb, c_b, codes, row_scale, decision, want);
  else
    hipLaunchKernelGGL(k_quant_int_rows_long<false>, dim3((unsigned)rows), dim3(256), 0, s, x,
                       cols, hb, c_b, codes, row_scale, decision, want);
  return hipGetLastError();
}

// ---------------------------------------------------------------- NVFP4

// Quantizes one 8-element chunk held by this lane (already rotated and
// scaled); returns its 4 code bytes and sets *e to its 16-block's scale byte.
// FMT: kNvfp4 (E4M3 scale per 16), kNvfp4Mx (a power of two per aligned
// pair of 16-blocks), kNvfp4P2 (a power of two per 16-block).
template <int FMT>
__device__ __forceinline__ uint32_t nvfp4_chunk(float (&v)[8], float s_t, float six_st, uint32_t* e_out) {
  float a = 0.0f;
#pragma unroll
  for (int i = 0; i < 8; ++i) a = fmaxf(a, fabsf(v[i]));
  // the two chunks of a 16-element block sit on lanes l and l ^ 1, the four
  // of a 32-element group on l ^ {0, 1, 2, 3} (fwht_chunk keeps chunk bits
  // 0 and 1 on lane bits 0 and 1)
  a = fmaxf(a, xor_lane<1>(a));
  if constexpr (FMT == kNvfp4Mx) a = fmaxf(a, xor_lane<2>(a));
  uint32_t e = 0u;
  float d = 0.0f;
  if (s_t > 0.0f) {
    const float t = a / six_st;
    e = FMT == kNvfp4 ? e4m3_encode(t) : e4m3_encode(pow2_ceil_clamped(t));
    d = e4m3_decode(e) * s_t;
  }
  *e_out = e;
  if (d == 0.0f) return 0u;
  const float inv = 1.0f / d;
  return e2m1x2_encode(v[0] * inv, v[1] * inv) | (e2m1x2_encode(v[2] * inv, v[3] * inv) << 8) |
         (e2m1x2_encode(v[4] * inv, v[5] * inv) << 16) | (e2m1x2_encode(v[6] * inv, v[7] * inv) << 24);
}

// UNROLL 8-element chunks per lane per iteration, loads issued first; a wave
// covers UNROLL x 64 consecutive chunks, so every Hadamard block (<= 128)
// and every 16- or 32-element scale block lies inside aligned lane groups of
// one wave.  HB > 0: the Hadamard block is HB (the argument is ignored).
template <int FMT, int HB = 0>
__global__ __launch_bounds__(256) void k_quant_nvfp4(
    const uint16_t* __restrict__ x, int64_t nch, int hb_arg, float c_b,
    const float* __restrict__ amax_ptr, uint8_t* __restrict__ codes,
    uint8_t* __restrict__ blk_scale, float* __restrict__ tensor_scale,
    const int32_t* __restrict__ decision, int32_t want) {
  if (decision != nullptr && *decision != want) return;
  const int hb = HB > 0 ? HB : hb_arg;
  constexpr int UNROLL = 2;
  const int lane = threadIdx.x & 63;
  const float A = *amax_ptr;
  // s_t = amax / (6 * 448) for NVFP4 (the largest block maps to E4M3's top
  // value), amax / (6 * 256) with power-of-two block scales (the largest is
  // 2^8).
  const float s_t = (A >= kTiny) ? A / (FMT == kNvfp4 ? 2688.0f : 1536.0f) : 0.0f;
  if (blockIdx.x == 0 && threadIdx.x == 0) *tensor_scale = s_t;
  const float six_st = 6.0f * s_t;
  const int64_t wave = ((int64_t)blockIdx.x * blockDim.x + threadIdx.x) >> 6;
  const int64_t nwaves = ((int64_t)gridDim.x * blockDim.x) >> 6;
  const uint4* xv = reinterpret_cast<const uint4*>(x);
  uint32_t* cv = reinterpret_cast<uint32_t*>(codes);

  for (int64_t base = wave * 64 * UNROLL; base < nch; base += nwaves * 64 * UNROLL) {
    uint4 w[UNROLL];
#pragma unroll
    for (int u = 0; u < UNROLL; ++u) {
      const int64_t idx = fwht_src(base + 64 * u + lane, lane, hb);
      w[u] = (idx < nch) ? xv[idx] : make_uint4(0u, 0u, 0u, 0u);
    }
#pragma unroll
    for (int u = 0; u < UNROLL; ++u) {
      const int64_t idx = fwht_src(base + 64 * u + lane, lane, hb);
      float v[8];
      bf16x8_to_f32(w[u], v);
      const float sc = fwht8(v, lane, hb) * c_b;
#pragma unroll
      for (int i = 0; i < 8; ++i) v[i] = v[i] * sc;
      uint32_t e;
      const uint32_t packed = nvfp4_chunk<FMT>(v, s_t, six_st, &e);
      if (idx < nch) {
        cv[idx] = packed;
        // the lane with the even chunk of the 16-element block writes its scale
        if ((idx & 1) == 0) blk_scale[idx >> 1] = (uint8_t)e;
      }
    }
  }
}

hipError_t launch_quant_nvfp4(const uint16_t* x, int64_t rows, int64_t cols, int hb, int fmt,
                              const float* amax, uint8_t* codes, uint8_t* blk_scale,
                              float* tensor_scale, const int32_t* decision, int32_t want,
                              hipStream_t s) {
  const int64_t nch = rows * cols / 8;
  const int64_t waves_needed = (nch + 127) / 128;
  // 8 waves per CU x 256 CUs of 4-wave workgroups keeps enough loads in
  // flight; a grid-stride loop covers the rest.
  int64_t blocks = (waves_needed + 3) / 4;
  if (blocks > 2048) blocks = 2048;
  if (blocks < 1) blocks = 1;
  const float c_b = hadamard_scale(hb);
  auto kern = hb == 128 ? (fmt == kNvfp4Mx   ? k_quant_nvfp4<kNvfp4Mx, 128>
                           : fmt == kNvfp4P2 ? k_quant_nvfp4<kNvfp4P2, 128>
                                             : k_quant_nvfp4<kNvfp4, 128>)
                        : (fmt == kNvfp4Mx   ? k_quant_nvfp4<kNvfp4Mx>
                           : fmt == kNvfp4P2 ? k_quant_nvfp4<kNvfp4P2>
                                             : k_quant_nvfp4<kNvfp4>);
  hipLaunchKernelGGL(kern, dim3((unsigned)blocks), dim3(256), 0, s, x, nch, hb, c_b, amax, codes,
                     blk_scale, tensor_scale, decision, want);
  return hipGetLastError();
}

// ------------------------------------------------------------- DeltaQuant
// Cube-delta quantization (DeltaQuant abstract, paper-radar CVPR 2026
// listing): video tokens of an F x H x W grid (frame outermost) in cubes of
// cf x ch x cw (ragged at the far edges); a cube's mean token (the core) is
// kept in FP8 E4M3 with one fp32 scale, every token's difference from the
// stored core in NVFP4 without rotation.  The core is the float32 sum of the
// cube's tokens in token order divided by their count; its scale is
// max|core| / 448 (0 below kTiny); a code is the nearest E4M3 of |c| / s with
// the sign in bit 7 (a zero magnitude stored as +0).

// The rows of a cube's tokens in token order (at most kDqMaxCube tokens).
__device__ __forceinline__ int dq_rows(const DqGrid& g, int cube, int* rows) {
  const int a = cube / (g.nH * g.nW), b = (cube / g.nW) % g.nH, c = cube % g.nW;
  const int f0 = a * g.cf, h0 = b * g.ch, w0 = c * g.cw;
  const int nf = min(g.F, f0 + g.cf) - f0, nh = min(g.H, h0 + g.ch) - h0, nw = min(g.W, w0 + g.cw) - w0;
  const int nt = nf * nh * nw, t = threadIdx.x;
  if (t < nt) {
    const int f = t / (nh * nw), r = t - f * nh * nw, h = r / nw, w = r - h * nw;
    rows[t] = ((f0 + f) * g.H + h0 + h) * g.W + w0 + w;
  }
  __syncthreads();
  return nt;
}

// One workgroup per cube: the mean in LDS (eight tokens' loads in flight,
// added in token order), its scale and codes, the decoded code values as bf16
// (exact: E4M3 has 4 significant bits) for the core GEMM, and the largest
// |difference| of the cube's tokens into the running maximum (float bits of a
// non-negative value order as unsigned integers).
__global__ __launch_bounds__(256) void k_dq_core(const uint16_t* __restrict__ x, int K, const DqGrid g,
                                                 uint8_t* __restrict__ codes, float* __restrict__ scale,
                                                 uint16_t* __restrict__ core_bf16,
                                                 uint32_t* __restrict__ damax_bits) {
  extern __shared__ float lcore[];  // K floats: the mean, then the stored core
  __shared__ float red[4];
  __shared__ int rows[kDqMaxCube];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int cube = blockIdx.x, nt = dq_rows(g, cube, rows);
  const float n = (float)nt;
  const int kq = K >> 3;
  const uint4* xv = reinterpret_cast<const uint4*>(x);
  float amax = 0.0f;
  for (int q = tid; q < kq; q += 256) {
    float sum[8] = {0.0f, 0.0f, 0.0f, 0.0f, 0.0f, 0.0f, 0.0f, 0.0f};
    for (int t0 = 0; t0 < nt; t0 += 8) {
      uint4 w[8];
#pragma unroll
      for (int u = 0; u < 8; ++u)
        w[u] = t0 + u < nt ? xv[(int64_t)rows[t0 + u] * kq + q] : make_uint4(0u, 0u, 0u, 0u);
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        if (t0 + u < nt) {
          float v[8];
          bf16x8_to_f32(w[u], v);
#pragma unroll
          for (int i = 0; i < 8; ++i) sum[i] = sum[i] + v[i];
        }
      }
    }
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const float m = sum[i] / n;
      lcore[8 * q + i] = m;
      amax = fmaxf(amax, fabsf(m));
    }
  }
  amax = wave_max(amax);
  if (lane == 0) red[wave] = amax;
  __syncthreads();
  amax = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
  const float sc = amax >= kTiny ? amax / 448.0f : 0.0f;
  if (tid == 0) scale[cube] = sc;
  for (int q = tid; q < kq; q += 256) {
    uint32_t cw2[2] = {0u, 0u}, bw[4];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const float m = lcore[8 * q + i];
      const uint32_t mag = sc == 0.0f ? 0u : e4m3_encode(fabsf(m) / sc);
      const bool neg = mag != 0u && m < 0.0f;
      const float e = neg ? -e4m3_decode(mag) : e4m3_decode(mag);
      lcore[8 * q + i] = e * sc;
      cw2[i >> 2] |= (mag | (neg ? 0x80u : 0u)) << (8 * (i & 3));
      const uint32_t eb = __float_as_uint(e) >> 16;  // exact: 4 significant bits
      if (i & 1) bw[i >> 1] |= eb << 16; else bw[i >> 1] = eb;
    }
    reinterpret_cast<uint2*>(codes)[(int64_t)cube * kq + q] = make_uint2(cw2[0], cw2[1]);
    if (core_bf16 != nullptr)
      reinterpret_cast<uint4*>(core_bf16)[(int64_t)cube * kq + q] = make_uint4(bw[0], bw[1], bw[2], bw[3]);
  }
  __syncthreads();
  float dmax = 0.0f;
  for (int q = tid; q < kq; q += 256) {
    for (int t0 = 0; t0 < nt; t0 += 8) {
      uint4 w[8];
#pragma unroll
      for (int u = 0; u < 8; ++u)
        w[u] = t0 + u < nt ? xv[(int64_t)rows[t0 + u] * kq + q] : make_uint4(0u, 0u, 0u, 0u);
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        if (t0 + u < nt) {
          float v[8];
          bf16x8_to_f32(w[u], v);
#pragma unroll
          for (int i = 0; i < 8; ++i) dmax = fmaxf(dmax, fabsf(v[i] - lcore[8 * q + i]));
        }
      }
    }
  }
  dmax = wave_max(dmax);
  __syncthreads();
  if (lane == 0) red[wave] = dmax;
  __syncthreads();
  if (tid == 0) atomicMax(damax_bits, __float_as_uint(fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]))));
}

__global__ void k_dq_zero(uint32_t* p) { *p = 0u; }

// One workgroup per cube: each token's difference from the stored core,
// quantized to NVFP4 with the tensor scale of the largest |difference|.  A
// wave covers 64 consecutive chunks of one token row, so a 16-element block
// sits on lanes l, l ^ 1 and a 32-element group on l ^ {0..3}; every lane
// runs the block code (zeros past the row), only the stores are predicated.
template <int FMT>
__global__ __launch_bounds__(256) void k_dq_delta(const uint16_t* __restrict__ x, int K, const DqGrid g,
                                                  const uint8_t* __restrict__ ccodes,
                                                  const float* __restrict__ cscale,
                                                  const uint32_t* __restrict__ damax_bits,
                                                  uint8_t* __restrict__ codes, uint8_t* __restrict__ blk_scale,
                                                  float* __restrict__ tensor_scale) {
  extern __shared__ float lcore[];  // the stored core, K floats
  __shared__ int rows[kDqMaxCube];
  const int tid = threadIdx.x, kq = K >> 3, cube = blockIdx.x;
  const float A = __uint_as_float(*damax_bits);
  const float s_t = (A >= kTiny) ? A / (FMT == kNvfp4 ? 2688.0f : 1536.0f) : 0.0f;
  if (cube == 0 && tid == 0) *tensor_scale = s_t;
  const float six_st = 6.0f * s_t, sc = cscale[cube];
  for (int k = tid; k < K; k += 256) {
    const uint32_t b = ccodes[(int64_t)cube * K + k];
    const float e = e4m3_decode(b & 0x7fu);
    lcore[k] = ((b & 0x80u) ? -e : e) * sc;
  }
  const int nt = dq_rows(g, cube, rows);  // its barrier also publishes lcore
  const uint4* xv = reinterpret_cast<const uint4*>(x);
  uint32_t* cv = reinterpret_cast<uint32_t*>(codes);
  for (int q0 = 0; q0 < kq; q0 += 256) {
    const int q = q0 + tid;
    const bool ok = q < kq;
    for (int t0 = 0; t0 < nt; t0 += 4) {
      uint4 w[4];
#pragma unroll
      for (int u = 0; u < 4; ++u)
        w[u] = ok && t0 + u < nt ? xv[(int64_t)rows[t0 + u] * kq + q] : make_uint4(0u, 0u, 0u, 0u);
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        if (t0 + u >= nt) break;  // uniform
        float v[8];
        bf16x8_to_f32(w[u], v);
        if (ok) {
#pragma unroll
          for (int i = 0; i < 8; ++i) v[i] = v[i] - lcore[8 * q + i];
        }
        uint32_t e;
        const uint32_t packed = nvfp4_chunk<FMT>(v, s_t, six_st, &e);
        if (ok) {
          const int64_t idx = (int64_t)rows[t0 + u] * kq + q;
          cv[idx] = packed;
          if ((q & 1) == 0) blk_scale[idx >> 1] = (uint8_t)e;
        }
      }
    }
  }
}

hipError_t launch_dq_quantize(const uint16_t* x, int64_t K, const DqGrid& g, int fmt, uint8_t* ccodes,
                              float* cscale, uint16_t* core_bf16, uint32_t* damax_bits, uint8_t* codes,
                              uint8_t* blk_scale, float* tensor_scale, hipStream_t s) {
  const int64_t ncubes = (int64_t)g.nF * g.nH * g.nW;
  const size_t lds = (size_t)K * sizeof(float);
  auto kdelta = fmt == kNvfp4Mx ? k_dq_delta<kNvfp4Mx> : fmt == kNvfp4P2 ? k_dq_delta<kNvfp4P2> : k_dq_delta<kNvfp4>;
  for (const void* k : {reinterpret_cast<const void*>(k_dq_core), reinterpret_cast<const void*>(kdelta)}) {
    hipError_t e = hipFuncSetAttribute(k, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    if (e != hipSuccess) return e;
  }
  hipLaunchKernelGGL(k_dq_zero, dim3(1), dim3(1), 0, s, damax_bits);
  hipLaunchKernelGGL(k_dq_core, dim3((unsigned)ncubes), dim3(256), lds, s, x, (int)K, g, ccodes, cscale,
                     core_bf16, damax_bits);
  hipLaunchKernelGGL(kdelta, dim3((unsigned)ncubes), dim3(256), lds, s, x, (int)K, g, ccodes, cscale, damax_bits,
                     codes, blk_scale, tensor_scale);
  return hipGetLastError();
}

// NVFP4 weights to bf16 values of E2M1 x block scale (exact: at most six
// significant bits), the tensor scale left out: the core GEMM's operand.
__global__ __launch_bounds__(256) void k_dq_decode_w(const uint8_t* __restrict__ codes,
                                                     const uint8_t* __restrict__ blk, int64_t nch,
                                                     uint16_t* __restrict__ out) {
  const uint32_t* cv = reinterpret_cast<const uint32_t*>(codes);
  uint4* ov = reinterpret_cast<uint4*>(out);
  for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < nch; i += (int64_t)gridDim.x * 256) {
    const uint32_t p = cv[i];
    const float e = e4m3_decode(blk[i >> 1]);
    uint32_t o[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const uint32_t lo = (p >> (8 * j)) & 15u, hi = (p >> (8 * j + 4)) & 15u;
      o[j] = (__float_as_uint(e2m1_value(lo) * e) >> 16) | ((__float_as_uint(e2m1_value(hi) * e) >> 16) << 16);
    }
    ov[i] = make_uint4(o[0], o[1], o[2], o[3]);
  }
}

hipError_t launch_dq_decode_w(const uint8_t* codes, const uint8_t* blk, int64_t N, int64_t K, uint16_t* out,
                              hipStream_t s) {
  const int64_t nch = N * K / 8;
  int64_t blocks = (nch + 255) / 256;
  if (blocks > 4096) blocks = 4096;
  if (blocks < 1) blocks = 1;
  hipLaunchKernelGGL(k_dq_decode_w, dim3((unsigned)blocks), dim3(256), 0, s, codes, blk, nch, out);
  return hipGetLastError();
}

// y[m, n] = yd[m, n] + fl32(fl32(yc[cube(m), n] * s_c) * s_tw): the
// differences' GEMM plus the core GEMM of the token's cube, 4 columns a thread.
template <int OUT>
__global__ __launch_bounds__(256) void k_dq_combine(const float* __restrict__ yd, const float* __restrict__ yc,
                                                    const float* __restrict__ cscale,
                                                    const float* __restrict__ wts, const DqGrid g, int M,
                                                    int N, void* __restrict__ y) {
  const int nq = N >> 2;
  const float stw = *wts;
  const int64_t total = (int64_t)M * nq;
  for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < total; i += (int64_t)gridDim.x * 256) {
    const int m = (int)(i / nq), q = (int)(i - (int64_t)m * nq), cb = dq_cube(m, g);
    const float4 d = reinterpret_cast<const float4*>(yd)[i];
    const float4 c = reinterpret_cast<const float4*>(yc)[(int64_t)cb * nq + q];
    const float s = cscale[cb];
    const float r0 = d.x + (c.x * s) * stw, r1 = d.y + (c.y * s) * stw;
    const float r2 = d.z + (c.z * s) * stw, r3 = d.w + (c.w * s) * stw;
    if constexpr (OUT == kOutF32)
      reinterpret_cast<float4*>(y)[i] = make_float4(r0, r1, r2, r3);
    else
      reinterpret_cast<uint2*>(y)[i] = make_uint2(pack_bf16x2(r0, r1), pack_bf16x2(r2, r3));
  }
}

hipError_t launch_dq_combine(const float* yd, const float* yc, const float* cscale, const float* wts,
                             const DqGrid& g, int64_t N, void* y, int out_dtype, hipStream_t s) {
  const int64_t M = (int64_t)g.F * g.H * g.W, total = M * (N / 4);
  int64_t blocks = (total + 255) / 256;
  if (blocks > 8192) blocks = 8192;
  if (blocks < 1) blocks = 1;
  if (out_dtype == kOutF32)
    hipLaunchKernelGGL(k_dq_combine<kOutF32>, dim3((unsigned)blocks), dim3(256), 0, s, yd, yc, cscale, wts, g,
                       (int)M, (int)N, y);
  else
    hipLaunchKernelGGL(k_dq_combine<kOutBf16>, dim3((unsigned)blocks), dim3(256), 0, s, yd, yc, cscale, wts, g,
                       (int)M, (int)N, y);
  return hipGetLastError();
}

}  // namespace hdq
