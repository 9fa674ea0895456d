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
//  * k_quant_nvfp4_w32 / k_quant_nvfp4: NVFP4 needs only the tensor amax
//    (given) and a 16- or 32-element block max (E4M3 scale per 16, or a power
//    of two per 16 or per 32), so they are flat grid-stride kernels with no
//    workgroup synchronisation.  At Hadamard block 128 a lane holds 32
//    consecutive elements (a whole 32-element group, so its maximum and scale
//    stay in the lane); other blocks, and the plain recipe's decoded output,
//    take 8-element chunks, two per lane (each wave owns 128 consecutive
//    chunks per iteration, loads issued first).
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
// so the rotation's block-size branches fold away at compile time.  FULL:
// the row is exactly BLOCK x CPT chunks, so no chunk needs a bounds check.
template <int BLOCK, int CPT, bool INT4, bool STATS = false, int HB = 0, bool FULL = false>
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
    if (FULL || idx < nch) w = xr[idx];
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
    if (FULL || idx < nch) {
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
  else if (hb == 128 && (cols >> 3) == (int64_t)BLOCK * CPT)
    hipLaunchKernelGGL((k_quant_int_rows<BLOCK, CPT, false, false, 128, true>), dim3((unsigned)rows), dim3(BLOCK),
                       0, s, x, cols, hb, c_b, codes, sc, dec, want);
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
  if (hb == 128 && (cols >> 3) == (int64_t)BLOCK * CPT)
    hipLaunchKernelGGL((k_quant_int_rows<BLOCK, CPT, false, true, 128, true>), dim3((unsigned)rows), dim3(BLOCK),
                       0, s, x, cols, hb, hadamard_scale(hb), codes, sc, nullptr, 0, psum, pbits, ptmax);
  else if (hb == 128)
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
  // the two-pass route), six chunks per thread: fewer waves per row share
  // its reductions, divisions and partial writes (a third of the VALU work
  // at two chunks).  Measured against 2, 3, 4, 8 and 12 chunks at K 3072 and
  // 12288: 6 is fastest (2 was 6% and 19% slower).
  if ((cols >> 3) > 2048) return hipErrorInvalidValue;
  return launch_select_q8_cpt<6>(x, rows, cols, hb, codes, row_scale, psum, pbits, ptmax, s);
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
// A block's scale byte (*e_out) and fl32(1 / d), d = the block scale's value
// times s_t, from the block's max |y| (0 when s_t or d is 0).
template <int FMT>
__device__ __forceinline__ float nvfp4_block_inv(float a, float s_t, float six_st, float inv_st,
                                                 uint32_t* e_out) {
  uint32_t e = 0u;
  float inv = 0.0f;
  if (s_t > 0.0f) {
    const float t = a / six_st;
    if constexpr (FMT == kNvfp4) {
      e = e4m3_encode(t);
      const float d = e4m3_decode(e) * s_t;
      if (d != 0.0f) inv = 1.0f / d;
    } else {
      // d = 2^k s_t for the block's power of two 2^k, so fl32(1 / d) =
      // 2^-k fl32(1 / s_t) exactly (every value stays normal: s_t >= 2^-110
      // and k in [-9, 8]); 2^-k is 2^k's exponent field mirrored
      const float p2 = pow2_ceil_clamped(t);
      e = e4m3_encode(p2);
      inv = inv_st * __uint_as_float(0x7f000000u - __float_as_uint(p2));
    }
  }
  *e_out = e;
  return inv;
}

template <int FMT>
__device__ __forceinline__ uint32_t nvfp4_chunk(float (&v)[8], float s_t, float six_st, float inv_st,
                                                uint32_t* e_out) {
  float a = 0.0f;
#pragma unroll
  for (int i = 0; i < 8; ++i) a = fmaxf(a, fabsf(v[i]));
  // the two chunks of a 16-element block sit on lanes l and l ^ 1, the four
  // of a 32-element group on l ^ {0, 1, 2, 3} (fwht_chunk keeps chunk bits
  // 0 and 1 on lane bits 0 and 1)
  a = fmaxf(a, xor_lane<1>(a));
  if constexpr (FMT == kNvfp4Mx) a = fmaxf(a, xor_lane<2>(a));
  const float inv = nvfp4_block_inv<FMT>(a, s_t, six_st, inv_st, e_out);
  if (inv == 0.0f) return 0u;
  return e2m1x2_encode(v[0] * inv, v[1] * inv) | (e2m1x2_encode(v[2] * inv, v[3] * inv) << 8) |
         (e2m1x2_encode(v[4] * inv, v[5] * inv) << 16) | (e2m1x2_encode(v[6] * inv, v[7] * inv) << 24);
}

// Exact bf16 values of one chunk's 8 codes with block-scale byte e: E2M1
// value (the hardware conversion at scale 1, exact) x E4M3 value, exact in
// float32 and in bf16 (at most 6 significant bits), so the bf16 rounding
// returns it unchanged.
template <int B>
__device__ __forceinline__ uint32_t nvfp4_decode_pair(uint32_t p, float s) {
  const auto f = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(p, 1.0f, B);
  return pack_bf16x2(f[0] * s, f[1] * s);
}
__device__ __forceinline__ uint4 nvfp4_decode_chunk(uint32_t p, uint32_t e) {
  const float s = e4m3_decode(e);
  return make_uint4(nvfp4_decode_pair<0>(p, s), nvfp4_decode_pair<1>(p, s), nvfp4_decode_pair<2>(p, s),
                    nvfp4_decode_pair<3>(p, s));
}

// UNROLL 8-element chunks per lane per iteration, loads issued first; a wave
// covers UNROLL x 64 consecutive chunks, so every Hadamard block (<= 128)
// and every 16- or 32-element scale block lies inside aligned lane groups of
// one wave.  HB > 0: the Hadamard block is HB (the argument is ignored).
// DEC: also the codes' exact bf16 values, 16 bytes per chunk, into dec.
template <int FMT, int HB = 0, bool DEC = false>
__global__ __launch_bounds__(256) void k_quant_nvfp4(
    const uint16_t* __restrict__ x, int64_t nch, int hb_arg, float c_b,
    const float* __restrict__ amax_ptr, uint8_t* __restrict__ codes,
    uint8_t* __restrict__ blk_scale, float* __restrict__ tensor_scale,
    const int32_t* __restrict__ decision, int32_t want, uint16_t* __restrict__ dec) {
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
  const float six_st = 6.0f * s_t, inv_st = s_t > 0.0f ? 1.0f / s_t : 0.0f;
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
      const uint32_t packed = nvfp4_chunk<FMT>(v, s_t, six_st, inv_st, &e);
      if (idx < nch) {
        cv[idx] = packed;
        // the lane with the even chunk of the 16-element block writes its scale
        if ((idx & 1) == 0) blk_scale[idx >> 1] = (uint8_t)e;
        if constexpr (DEC) reinterpret_cast<uint4*>(dec)[idx] = nvfp4_decode_chunk(packed, e);
      }
    }
  }
}

// Eight E2M1 codes of y[0..7] * inv in k order, two per byte (the
// conversion writes the byte its last operand selects).
__device__ __forceinline__ uint32_t e2m1x8_encode(const float* y, float inv) {
  uint32_t w = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(0u, y[0] * inv, y[1] * inv, 1.0f, 0);
  w = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w, y[2] * inv, y[3] * inv, 1.0f, 1);
  w = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w, y[4] * inv, y[5] * inv, 1.0f, 2);
  w = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w, y[6] * inv, y[7] * inv, 1.0f, 3);
  return w;
}

// Hadamard block 128: one lane per 32 consecutive elements (fwht128_w32), so
// a 32-element group's maximum and scale stay inside the lane (one division
// per 16-element block -- per 32 with the MX recipe -- where the 8-element
// layout repeats it for each chunk, and no cross-lane maximum), and a lane
// writes its 16 code bytes and 2 scale bytes with one store each.  The same
// arithmetic as k_quant_nvfp4, value for value.
template <int FMT>
__global__ __launch_bounds__(256) void k_quant_nvfp4_w32(
    const uint16_t* __restrict__ x, int64_t ngrp, float c_b, const float* __restrict__ amax_ptr,
    uint8_t* __restrict__ codes, uint8_t* __restrict__ blk_scale, float* __restrict__ tensor_scale,
    const int32_t* __restrict__ decision, int32_t want) {
  if (decision != nullptr && *decision != want) return;
  const int lane = threadIdx.x & 63;
  const float A = *amax_ptr;
  const float s_t = (A >= kTiny) ? A / (FMT == kNvfp4 ? 2688.0f : 1536.0f) : 0.0f;
  if (blockIdx.x == 0 && threadIdx.x == 0) *tensor_scale = s_t;
  const float six_st = 6.0f * s_t, inv_st = s_t > 0.0f ? 1.0f / s_t : 0.0f;
  const uint4* xv = reinterpret_cast<const uint4*>(x);
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  // ngrp is a multiple of 4 and the lanes of a wave take consecutive
  // groups, so the four lanes of a Hadamard block stay active together
  for (int64_t g = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; g < ngrp; g += stride) {
    uint4 w[4];
#pragma unroll
    for (int c = 0; c < 4; ++c) w[c] = xv[4 * g + c];
    float v[32];
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      v[8 * c + 0] = bf16_lo(w[c].x);
      v[8 * c + 1] = bf16_hi(w[c].x);
      v[8 * c + 2] = bf16_lo(w[c].y);
      v[8 * c + 3] = bf16_hi(w[c].y);
      v[8 * c + 4] = bf16_lo(w[c].z);
      v[8 * c + 5] = bf16_hi(w[c].z);
      v[8 * c + 6] = bf16_lo(w[c].w);
      v[8 * c + 7] = bf16_hi(w[c].w);
    }
    const float sc = fwht128_w32(v, lane) * c_b;
#pragma unroll
    for (int i = 0; i < 32; ++i) v[i] = v[i] * sc;
    float a0 = 0.0f, a1 = 0.0f;
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      a0 = fmaxf(a0, fabsf(v[i]));
      a1 = fmaxf(a1, fabsf(v[16 + i]));
    }
    uint32_t e0, e1;
    float inv0, inv1;
    if constexpr (FMT == kNvfp4Mx) {
      inv0 = inv1 = nvfp4_block_inv<FMT>(fmaxf(a0, a1), s_t, six_st, inv_st, &e0);
      e1 = e0;
    } else {
      inv0 = nvfp4_block_inv<FMT>(a0, s_t, six_st, inv_st, &e0);
      inv1 = nvfp4_block_inv<FMT>(a1, s_t, six_st, inv_st, &e1);
    }
    // encoded unconditionally, then selected (no branch per block): a block
    // without a scale (inv 0) stores zero codes
    uint32_t p[4];
    p[0] = e2m1x8_encode(v + 0, inv0);
    p[1] = e2m1x8_encode(v + 8, inv0);
    p[2] = e2m1x8_encode(v + 16, inv1);
    p[3] = e2m1x8_encode(v + 24, inv1);
    if (inv0 == 0.0f) p[0] = p[1] = 0u;
    if (inv1 == 0.0f) p[2] = p[3] = 0u;
    reinterpret_cast<uint4*>(codes)[g] = make_uint4(p[0], p[1], p[2], p[3]);
    reinterpret_cast<uint16_t*>(blk_scale)[g] = (uint16_t)(e0 | (e1 << 8));
  }
}

template <bool DEC>
static hipError_t launch_quant_nvfp4_t(const uint16_t* x, int64_t rows, int64_t cols, int hb, int fmt,
                                       const float* amax, uint8_t* codes, uint8_t* blk_scale,
                                       float* tensor_scale, const int32_t* decision, int32_t want,
                                       uint16_t* dec, hipStream_t s) {
  const int64_t nch = rows * cols / 8;
  const int64_t waves_needed = (nch + 127) / 128;
  // 16 waves per CU x 256 CUs of 4-wave workgroups keeps enough loads in
  // flight (4096 workgroups measured 3-4% faster than 2048, 1024 8%
  // slower); a grid-stride loop covers the rest.
  int64_t blocks = (waves_needed + 3) / 4;
  if (blocks > 4096) blocks = 4096;
  if (blocks < 1) blocks = 1;
  const float c_b = hadamard_scale(hb);
  if (hb == 128 && !DEC) {
    // cols is a multiple of 128, so the 32-element groups come in fours.
    // (With the decoded values, 64 bytes per lane in four 16-byte stores at
    // a 64-byte lane stride, this layout measured slower at K = 12288 than
    // the 8-element chunks below, whose stores are contiguous across lanes.)
    const int64_t ngrp = rows * cols / 32;
    int64_t wgs = (ngrp + 255) / 256;
    if (wgs > 4096) wgs = 4096;
    if (wgs < 1) wgs = 1;
    auto k32 = fmt == kNvfp4Mx ? k_quant_nvfp4_w32<kNvfp4Mx>
                               : fmt == kNvfp4P2 ? k_quant_nvfp4_w32<kNvfp4P2> : k_quant_nvfp4_w32<kNvfp4>;
    hipLaunchKernelGGL(k32, dim3((unsigned)wgs), dim3(256), 0, s, x, ngrp, c_b, amax, codes, blk_scale,
                       tensor_scale, decision, want);
    return hipGetLastError();
  }
  auto kern = hb == 128 ? (fmt == kNvfp4Mx   ? k_quant_nvfp4<kNvfp4Mx, 128, DEC>
                           : fmt == kNvfp4P2 ? k_quant_nvfp4<kNvfp4P2, 128, DEC>
                                             : k_quant_nvfp4<kNvfp4, 128, DEC>)
                        : (fmt == kNvfp4Mx   ? k_quant_nvfp4<kNvfp4Mx, 0, DEC>
                           : fmt == kNvfp4P2 ? k_quant_nvfp4<kNvfp4P2, 0, DEC>
                                             : k_quant_nvfp4<kNvfp4, 0, DEC>);
  hipLaunchKernelGGL(kern, dim3((unsigned)blocks), dim3(256), 0, s, x, nch, hb, c_b, amax, codes,
                     blk_scale, tensor_scale, decision, want, dec);
  return hipGetLastError();
}

hipError_t launch_quant_nvfp4(const uint16_t* x, int64_t rows, int64_t cols, int hb, int fmt,
                              const float* amax, uint8_t* codes, uint8_t* blk_scale,
                              float* tensor_scale, const int32_t* decision, int32_t want,
                              hipStream_t s, uint16_t* dec) {
  return dec != nullptr
             ? launch_quant_nvfp4_t<true>(x, rows, cols, hb, fmt, amax, codes, blk_scale, tensor_scale, decision,
                                          want, dec, s)
             : launch_quant_nvfp4_t<false>(x, rows, cols, hb, fmt, amax, codes, blk_scale, tensor_scale, decision,
                                           want, nullptr, s);
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

// A core mean or a difference that is not finite (a NaN or infinite token
// element, or a sum that overflows) sets the running maximum to a NaN, whose
// bits exceed those of every other value, and the difference pass turns that
// into a NaN tensor scale: the caller's flag that the codes are meaningless.
constexpr uint32_t kDqNonFinite = 0x7fc00000u;
__device__ __forceinline__ bool dq_finite(float v) { return fabsf(v) <= 3.40282347e38f; }

// The rows of cube `cube`'s first 8 tokens in token order (thread t < 8
// computes row t; nt is the cube's token count).
__device__ __forceinline__ int dq_rows8(const DqGrid& g, int cube, int t, int* nt_out) {
  const int a = cube / (g.nH * g.nW), b = (cube / g.nW) % g.nH, c = cube % g.nW;
  const int f0 = a * g.cf, h0 = b * g.ch, w0 = c * g.cw;
  const int nf = min(g.F, f0 + g.cf) - f0, nh = min(g.H, h0 + g.ch) - h0, nw = min(g.W, w0 + g.cw) - w0;
  *nt_out = nf * nh * nw;
  const int f = t / (nh * nw), r = t - f * nh * nw, h = r / nw, w = r - h * nw;
  return ((f0 + f) * g.H + h0 + h) * g.W + w0 + w;
}

// One workgroup per cube of at most 8 tokens, blockDim.x (a multiple of 64,
// at most MAXT) times ITER chunk columns covering K / 8: every thread keeps
// its columns of all the cube's tokens in registers (eight 16-byte loads per
// column in flight), so the mean (added in token order), the codes and
// scale, the bf16 code values for the bf16 core GEMM and the largest
// |difference| from the stored core all come from one read of the tokens.
// PIPE (ITER 1): persistent over cubes blockIdx.x, + gridDim.x, ..., the
// next cube's tokens loaded into a second register set as soon as its rows
// are known (after the current cube's first barrier), so the loads overlap
// the current cube's arithmetic and reductions.
template <int ITER, int MAXT, bool PIPE>
__global__ __launch_bounds__(MAXT) void k_dq_core_reg(const uint16_t* __restrict__ x, int K, const DqGrid g,
                                                     int ncubes, uint8_t* __restrict__ codes,
                                                     float* __restrict__ scale, uint16_t* __restrict__ core_bf16,
                                                     uint32_t* __restrict__ damax_bits) {
  static_assert(!PIPE || ITER == 1, "the pipelined form holds one column per thread");
  // rows, nts and red are double-buffered by cube parity, so one barrier per
  // cube orders every write after the last read of the same buffer (two
  // cubes earlier); the largest |difference| and the non-finite flag are
  // kept per thread over all of the workgroup's cubes and merged once
  __shared__ float red[2][16];
  __shared__ float redd[16];
  __shared__ int rows[2][8];
  __shared__ int nts[2];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, nwaves = blockDim.x >> 6;
  const int kq = K >> 3;
  const uint4* xv = reinterpret_cast<const uint4*>(x);
  const int step = PIPE ? (int)gridDim.x : ncubes;
  // a cube's rows into rows[] and its token count into nts
  auto cube_rows = [&](int cb, int buf) {
    if (tid < 8 && cb < ncubes) {
      int ntc;
      const int r = dq_rows8(g, cb, tid, &ntc);
      if (tid < ntc) rows[buf][tid] = r;
      if (tid == 0) nts[buf] = ntc;
    }
  };
  uint4 wn[ITER][8];
  int ntn = 0;  // the token count of the cube in wn (read with its rows)
  auto load = [&](int buf) {
    const int ntc = nts[buf];
    ntn = ntc;
#pragma unroll
    for (int it = 0; it < ITER; ++it) {
      const int q = tid + it * (int)blockDim.x;
#pragma unroll
      for (int u = 0; u < 8; ++u)
        wn[it][u] = q < kq && u < ntc ? xv[(int64_t)rows[buf][u] * kq + q] : make_uint4(0u, 0u, 0u, 0u);
    }
  };
  int cube = blockIdx.x, par = 0;
  cube_rows(cube, 0);
  __syncthreads();
  load(0);
  float dmax = 0.0f;
  bool bad = false;
  do {
    const int nt = ntn;
    uint4 w[ITER][8];
#pragma unroll
    for (int it = 0; it < ITER; ++it)
#pragma unroll
      for (int u = 0; u < 8; ++u) w[it][u] = wn[it][u];
    // the next cube's rows into the other buffer (last read by the loads of
    // the cube before this one, which every wave finished before the
    // previous cube's barrier); its loads follow the barrier below
    if (PIPE) cube_rows(cube + step, par ^ 1);
    const float n = (float)nt;
    float c[ITER][8];  // the mean, then the stored core
    float amax = 0.0f;
#pragma unroll
    for (int it = 0; it < ITER; ++it) {
      float sum[8] = {0.0f, 0.0f, 0.0f, 0.0f, 0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        if (u < nt) {
          float v[8];
          bf16x8_to_f32(w[it][u], v);
#pragma unroll
          for (int i = 0; i < 8; ++i) sum[i] = sum[i] + v[i];
        }
      }
      // sum / n: a product with the exact reciprocal when n is a power of
      // two (the same correctly rounded quotient), else the division
      if ((nt & (nt - 1)) == 0) {
        const float rn = 1.0f / n;
#pragma unroll
        for (int i = 0; i < 8; ++i) c[it][i] = sum[i] * rn;
      } else {
#pragma unroll
        for (int i = 0; i < 8; ++i) c[it][i] = sum[i] / n;
      }
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        amax = fmaxf(amax, fabsf(c[it][i]));
        bad |= !dq_finite(c[it][i]);
      }
    }
    // the tokens stay packed until the difference step converts them again
    // (otherwise the compiler keeps all their float values live)
#pragma unroll
    for (int it = 0; it < ITER; ++it)
#pragma unroll
      for (int u = 0; u < 8; ++u)
        asm volatile("" : "+v"(w[it][u].x), "+v"(w[it][u].y), "+v"(w[it][u].z), "+v"(w[it][u].w));
    amax = wave_max(amax);
    if (lane == 0) red[par][wave] = amax;
    __syncthreads();  // also publishes the next cube's rows
    if (PIPE && cube + step < ncubes) load(par ^ 1);
    amax = 0.0f;
    for (int i = 0; i < nwaves; ++i) amax = fmaxf(amax, red[par][i]);
    const float sc = amax >= kTiny ? amax / 448.0f : 0.0f;
    if (tid == 0) scale[cube] = sc;
#pragma unroll
    for (int it = 0; it < ITER; ++it) {
      const int q = tid + it * (int)blockDim.x;
      uint32_t cw2[2] = {0u, 0u}, bw[4];
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const float m = c[it][i];
        const uint32_t mag = sc == 0.0f ? 0u : e4m3_encode(fabsf(m) / sc);
        const bool neg = mag != 0u && m < 0.0f;
        cw2[i >> 2] |= (mag | (neg ? 0x80u : 0u)) << (8 * (i & 3));
      }
      // the signed code values (the hardware conversion, exact), the stored
      // core and the values' bf16 bits (exact: 4 significant bits)
      float e[8];
      e4m3x4_to_f32(cw2[0], &e[0]);
      e4m3x4_to_f32(cw2[1], &e[4]);
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        c[it][i] = e[i] * sc;
        const uint32_t eb = __float_as_uint(e[i]) >> 16;
        if (i & 1) bw[i >> 1] |= eb << 16; else bw[i >> 1] = eb;
      }
      if (q < kq) {
        reinterpret_cast<uint2*>(codes)[(int64_t)cube * kq + q] = make_uint2(cw2[0], cw2[1]);
        if (core_bf16 != nullptr)
          reinterpret_cast<uint4*>(core_bf16)[(int64_t)cube * kq + q] = make_uint4(bw[0], bw[1], bw[2], bw[3]);
#pragma unroll
        for (int u = 0; u < 8; ++u) {
          if (u < nt) {
            float v[8];
            bf16x8_to_f32(w[it][u], v);
#pragma unroll
            for (int i = 0; i < 8; ++i) dmax = fmaxf(dmax, fabsf(v[i] - c[it][i]));
          }
        }
      }
    }
    cube += step;
    par ^= 1;
  } while (PIPE && cube < ncubes);
  // a NaN difference needs a non-finite token element or stored core, and
  // so a non-finite mean (flagged above); an overflowing one is infinite and
  // reaches the maximum
  bad |= !dq_finite(dmax);
  dmax = wave_max(dmax);
  if (lane == 0) redd[wave] = dmax;
  bad = __syncthreads_or(bad);
  if (tid == 0) {
    float m = 0.0f;
    for (int i = 0; i < nwaves; ++i) m = fmaxf(m, redd[i]);
    atomicMax(damax_bits, bad ? kDqNonFinite : __float_as_uint(m));
  }
}

// The same for any cube (up to kDqMaxCube tokens) and K: the mean in LDS
// (eight tokens' loads in flight, added in token order), then a second read
// of the tokens for the largest |difference|.
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
  bool bad = false;
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
      bad |= !dq_finite(m);
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
          for (int i = 0; i < 8; ++i) {
            const float d = fabsf(v[i] - lcore[8 * q + i]);
            dmax = fmaxf(dmax, d);
            bad |= !dq_finite(d);
          }
        }
      }
    }
  }
  dmax = wave_max(dmax);
  bad = __syncthreads_or(bad);
  if (lane == 0) red[wave] = dmax;
  __syncthreads();
  if (tid == 0)
    atomicMax(damax_bits, bad ? kDqNonFinite : __float_as_uint(fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]))));
}

__global__ void k_dq_zero(uint32_t* p) { *p = 0u; }

// Each token's difference from the stored core (signed E4M3 code value x the
// cube's scale), quantized to NVFP4 with the tensor scale of the largest
// |difference| (a NaN when that is not finite).  A streaming pass with one
// lane per 32 consecutive elements of a token row (K % 32 == 0), NVFP4 as in
// k_quant_nvfp4_w32: a 32-element group's maximum and scale stay in the lane,
// and its 16 code bytes and 2 scale bytes are stored at once.  The groups of
// all rows are dealt to the grid's threads in order (M * K / 32 < 2^29).
template <int FMT>
__global__ __launch_bounds__(256) void k_dq_delta_w32(const uint16_t* __restrict__ x, int K, const DqGrid g,
                                                      int ngrp, const uint8_t* __restrict__ ccodes,
                                                      const float* __restrict__ cscale,
                                                      const uint32_t* __restrict__ damax_bits,
                                                      uint8_t* __restrict__ codes, uint8_t* __restrict__ blk_scale,
                                                      float* __restrict__ tensor_scale) {
  const float A = __uint_as_float(*damax_bits);
  const float s_t = (A >= kTiny) ? A / (FMT == kNvfp4 ? 2688.0f : 1536.0f) : (A == A ? 0.0f : A);
  if (blockIdx.x == 0 && threadIdx.x == 0) *tensor_scale = s_t;
  const float six_st = 6.0f * s_t, inv_st = s_t > 0.0f ? 1.0f / s_t : 0.0f;
  const uint32_t gpr = (uint32_t)K >> 5;  // groups per row
  const uint4* xv = reinterpret_cast<const uint4*>(x);
  const uint4* cv = reinterpret_cast<const uint4*>(ccodes);
  const int stride = (int)gridDim.x * (int)blockDim.x;
  for (int gi = (int)blockIdx.x * (int)blockDim.x + (int)threadIdx.x; gi < ngrp; gi += stride) {
    const uint32_t row = (uint32_t)gi / gpr, col = (uint32_t)gi - row * gpr;
    const int cube = dq_cube((int)row, g);
    uint4 w[4], e16[2];
#pragma unroll
    for (int c = 0; c < 4; ++c) w[c] = xv[4 * (int64_t)gi + c];
    const int64_t cb = ((int64_t)cube * gpr + col) * 2;
    e16[0] = cv[cb];
    e16[1] = cv[cb + 1];
    const float sc = cscale[cube];
    float v[32], e[32];
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      v[8 * c + 0] = bf16_lo(w[c].x);
      v[8 * c + 1] = bf16_hi(w[c].x);
      v[8 * c + 2] = bf16_lo(w[c].y);
      v[8 * c + 3] = bf16_hi(w[c].y);
      v[8 * c + 4] = bf16_lo(w[c].z);
      v[8 * c + 5] = bf16_hi(w[c].z);
      v[8 * c + 6] = bf16_lo(w[c].w);
      v[8 * c + 7] = bf16_hi(w[c].w);
    }
    // the stored core: signed E4M3 value (the hardware conversion, exact)
    // times the cube's scale
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      e4m3x4_to_f32(e16[h].x, &e[16 * h + 0]);
      e4m3x4_to_f32(e16[h].y, &e[16 * h + 4]);
      e4m3x4_to_f32(e16[h].z, &e[16 * h + 8]);
      e4m3x4_to_f32(e16[h].w, &e[16 * h + 12]);
    }
#pragma unroll
    for (int i = 0; i < 32; ++i) v[i] = v[i] - e[i] * sc;
    float a0 = 0.0f, a1 = 0.0f;
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      a0 = fmaxf(a0, fabsf(v[i]));
      a1 = fmaxf(a1, fabsf(v[16 + i]));
    }
    uint32_t e0, e1;
    float inv0, inv1;
    if constexpr (FMT == kNvfp4Mx) {
      inv0 = inv1 = nvfp4_block_inv<FMT>(fmaxf(a0, a1), s_t, six_st, inv_st, &e0);
      e1 = e0;
    } else {
      inv0 = nvfp4_block_inv<FMT>(a0, s_t, six_st, inv_st, &e0);
      inv1 = nvfp4_block_inv<FMT>(a1, s_t, six_st, inv_st, &e1);
    }
    // encoded unconditionally, then selected (no branch per block): a block
    // without a scale (inv 0) stores zero codes
    uint32_t p[4];
    p[0] = e2m1x8_encode(v + 0, inv0);
    p[1] = e2m1x8_encode(v + 8, inv0);
    p[2] = e2m1x8_encode(v + 16, inv1);
    p[3] = e2m1x8_encode(v + 24, inv1);
    if (inv0 == 0.0f) p[0] = p[1] = 0u;
    if (inv1 == 0.0f) p[2] = p[3] = 0u;
    reinterpret_cast<uint4*>(codes)[gi] = make_uint4(p[0], p[1], p[2], p[3]);
    reinterpret_cast<uint16_t*>(blk_scale)[gi] = (uint16_t)(e0 | (e1 << 8));
  }
}

// Workgroups of `kern` (threads each, lds dynamic bytes) resident per CU
// times the CUs: the grid of a persistent pass (at least 1).
template <auto KERNEL>
static int64_t resident_grid(int threads, size_t lds) {
  int dev = 0, cus = 0, per = 0;
  if (hipGetDevice(&dev) != hipSuccess ||
      hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus < 1)
    cus = 256;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per, KERNEL, threads, lds) != hipSuccess || per < 1) per = 1;
  return (int64_t)cus * per;
}

hipError_t launch_dq_quantize(const uint16_t* x, int64_t K, const DqGrid& g, int fmt, uint8_t* ccodes,
                              float* cscale, uint16_t* core_bf16, uint32_t* damax_bits, uint8_t* codes,
                              uint8_t* blk_scale, float* tensor_scale, hipStream_t s) {
  const int64_t ncubes = (int64_t)g.nF * g.nH * g.nW, M = (int64_t)g.F * g.H * g.W;
  const size_t lds = (size_t)K * sizeof(float);
  const int kq = (int)(K >> 3);
  // cubes of at most 8 tokens and K <= 16384: the register-resident core pass
  // (one column per thread, pipelined over cubes, up to K 8192; else one cube
  // per workgroup with four columns per thread)
  const bool reg = g.cf * g.ch * g.cw <= 8 && kq <= 2048;
  const int iter = kq <= 1024 ? 1 : 4;
  const int threads = (((kq + iter - 1) / iter) + 63) / 64 * 64;
  if (!reg) {
    const hipError_t e = set_dynamic_lds_once<k_dq_core>(lds);
    if (e != hipSuccess) return e;
  }
  hipLaunchKernelGGL(k_dq_zero, dim3(1), dim3(1), 0, s, damax_bits);
  if (reg && iter == 1) {
    const int64_t slots = resident_grid<k_dq_core_reg<1, 1024, true>>(threads, 0);
    auto kern = k_dq_core_reg<1, 1024, true>;
    hipLaunchKernelGGL(kern, dim3((unsigned)(ncubes < slots ? ncubes : slots)), dim3((unsigned)threads), 0, s, x,
                       (int)K, g, (int)ncubes, ccodes, cscale, core_bf16, damax_bits);
  } else if (reg) {
    auto kern = k_dq_core_reg<4, 512, false>;
    hipLaunchKernelGGL(kern, dim3((unsigned)ncubes), dim3((unsigned)threads), 0, s, x, (int)K, g, (int)ncubes,
                       ccodes, cscale, core_bf16, damax_bits);
  } else {
    hipLaunchKernelGGL(k_dq_core, dim3((unsigned)ncubes), dim3(256), lds, s, x, (int)K, g, ccodes, cscale,
                       core_bf16, damax_bits);
  }
  const int ngrp = (int)(M * (K >> 5));
  int64_t dblocks = (ngrp + 255) / 256;
  if (dblocks > 4096) dblocks = 4096;
  auto kdelta = fmt == kNvfp4Mx   ? k_dq_delta_w32<kNvfp4Mx>
                : fmt == kNvfp4P2 ? k_dq_delta_w32<kNvfp4P2>
                                  : k_dq_delta_w32<kNvfp4>;
  hipLaunchKernelGGL(kdelta, dim3((unsigned)dblocks), dim3(256), 0, s, x, (int)K, g, ngrp, ccodes, cscale,
                     damax_bits, codes, blk_scale, tensor_scale);
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
    ov[i] = nvfp4_decode_chunk(cv[i], blk[i >> 1]);
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
