// hdq_device.h -- device helpers shared by the gfx950 kernels of libhdq.
//
// Rotation, codecs and reductions used by the quantize, statistics and GEMM
// kernels.  Written for CDNA4 wave64; every helper that talks across lanes
// assumes all 64 lanes of the wave execute it.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace hdq {

typedef int v4i __attribute__((ext_vector_type(4)));
typedef int v8i __attribute__((ext_vector_type(8)));
typedef int v16i __attribute__((ext_vector_type(16)));
typedef float v4f __attribute__((ext_vector_type(4)));
typedef float v16f __attribute__((ext_vector_type(16)));
typedef __bf16 v8bf __attribute__((ext_vector_type(8)));
typedef short v8s __attribute__((ext_vector_type(8)));

// Rows whose max |rotated value| is below this quantize to zero codes with a
// zero scale (below it the reciprocal scales overflow float32).
constexpr float kTiny = 0x1p-100f;

__device__ __forceinline__ int lane_id() { return __lane_id(); }

// ---- bf16 <-> f32 -------------------------------------------------------
__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

// Eight consecutive bf16 (one 16-byte load) to float.
__device__ __forceinline__ void bf16x8_to_f32(const uint4 w, float (&x)[8]) {
  x[0] = bf16_lo(w.x); x[1] = bf16_hi(w.x);
  x[2] = bf16_lo(w.y); x[3] = bf16_hi(w.y);
  x[4] = bf16_lo(w.z); x[5] = bf16_hi(w.z);
  x[6] = bf16_lo(w.w); x[7] = bf16_hi(w.w);
}

// float -> bf16, round to nearest even (v_cvt_pk_bf16_f32 on gfx950).
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  uint16_t a = __builtin_bit_cast(uint16_t, (__bf16)lo);
  uint16_t b = __builtin_bit_cast(uint16_t, (__bf16)hi);
  return (uint32_t)a | ((uint32_t)b << 16);
}

// ---- cross-lane ---------------------------------------------------------
// Value held by lane (lane ^ G), G < 32: ds_swizzle in bit-mask mode.
template <int G>
__device__ __forceinline__ float xor_lane(float v) {
  static_assert(G > 0 && G < 32, "swizzle xor mask is 5 bits");
  return __int_as_float(__builtin_amdgcn_ds_swizzle(__float_as_int(v), 0x1F | (G << 10)));
}

__device__ __forceinline__ float wave_max(float v) {
  v = fmaxf(v, xor_lane<1>(v));
  v = fmaxf(v, xor_lane<2>(v));
  v = fmaxf(v, xor_lane<4>(v));
  v = fmaxf(v, xor_lane<8>(v));
  v = fmaxf(v, xor_lane<16>(v));
  v = fmaxf(v, __shfl_xor(v, 32));
  return v;
}

// ---- block Hadamard rotation --------------------------------------------
// Fast Walsh-Hadamard butterfly on blocks of hb (2..128) consecutive
// elements, strides h = 1, 2, 4, ... ascending: the pair (i, i + h),
// i & h == 0, becomes (u + v, u - v), evaluated in float32 exactly as that
// sequence (every rotated value is bit-identical to it).
//
// Each lane holds one 8-element chunk of a block; strides 1..4 run inside
// the lane.  For hb >= 16 the hb/8 lanes of a block exchange values, and
// lane l of the group does not hold chunk l but chunk fwht_chunk(l): lanes
// are numbered so that chunk bit k is lane mask m_k = 1, 2, 7, 15 (a linear
// relabelling over GF(2)), because lane ^ m_k is exactly what DPP reaches in
// one instruction (quad_perm [1,0,3,2], quad_perm [2,3,0,1], row_half_mirror,
// row_mirror).  Stride 8 * 2^k is then one v_fmac_f32_dpp per element:
//   x <- partner * S + x,  S = +1 on the lane whose chunk has bit k clear
// (u + v) and -1 on the other, which computes -(u - v): each lane carries a
// sign it knows (its lane partner always carries the same one), multiplying
// by +-1 is exact, and the one rounding is that of u + v or u - v.  The
// returned sign (+-1, the parity of the lane's chunk bits) restores the
// values; callers fold it into the 1/sqrt(hb) multiply.
__device__ __forceinline__ int fwht_lanes(int hb) { return hb >= 16 ? hb >> 3 : 1; }

// The chunk of its block that lane l holds (0 for hb <= 8).
__device__ __forceinline__ int fwht_chunk(int lane, int hb) {
  const int nl = fwht_lanes(hb);
  int L = lane & (nl - 1), c = 0;
  if (nl >= 16 && (L & 8)) { c |= 8; L ^= 15; }
  if (nl >= 8 && (L & 4)) { c |= 4; L ^= 7; }
  return c | L;
}

// Index of the chunk lane `lane` loads, given the natural index `idx` of
// chunk lane-slot `lane` (blocks of fwht_lanes(hb) slots are aligned).
__device__ __forceinline__ int64_t fwht_src(int64_t idx, int lane, int hb) {
  const int nl = fwht_lanes(hb);
  return (idx & ~(int64_t)(nl - 1)) + fwht_chunk(lane, hb);
}

template <int H>
__device__ __forceinline__ void fwht_stage_in(float (&x)[8]) {
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    if ((i & H) == 0) {
      const float u = x[i], v = x[i + H];
      x[i] = u + v;
      x[i + H] = u - v;
    }
  }
}

// x <- dpp(x) * s + x for the 8 values.  The leading s_nop gives the two
// wait states a DPP read needs after a VALU write of the same register;
// inside and between these blocks every register is written >= 7
// instructions before it is read again.
#define HDQ_FMAC_DPP8(CTRL, NOP)                                                             \
  asm(NOP                                                                                    \
      "v_fmac_f32_dpp %0, %0, %8 " CTRL " row_mask:0xf bank_mask:0xf bound_ctrl:1\n\t"       \
      "v_fmac_f32_dpp %1, %1, %8 " CTRL " row_mask:0xf bank_mask:0xf bound_ctrl:1\n\t"       \
      "v_fmac_f32_dpp %2, %2, %8 " CTRL " row_mask:0xf bank_mask:0xf bound_ctrl:1\n\t"       \
      "v_fmac_f32_dpp %3, %3, %8 " CTRL " row_mask:0xf bank_mask:0xf bound_ctrl:1\n\t"       \
      "v_fmac_f32_dpp %4, %4, %8 " CTRL " row_mask:0xf bank_mask:0xf bound_ctrl:1\n\t"       \
      "v_fmac_f32_dpp %5, %5, %8 " CTRL " row_mask:0xf bank_mask:0xf bound_ctrl:1\n\t"       \
      "v_fmac_f32_dpp %6, %6, %8 " CTRL " row_mask:0xf bank_mask:0xf bound_ctrl:1\n\t"       \
      "v_fmac_f32_dpp %7, %7, %8 " CTRL " row_mask:0xf bank_mask:0xf bound_ctrl:1"           \
      : "+v"(x[0]), "+v"(x[1]), "+v"(x[2]), "+v"(x[3]), "+v"(x[4]), "+v"(x[5]), "+v"(x[6]),  \
        "+v"(x[7])                                                                           \
      : "v"(s))

// Rotates the chunk held by this lane (see above); returns its sign.
__device__ __forceinline__ float fwht8(float (&x)[8], int lane, int hb) {
  if (hb >= 2) fwht_stage_in<1>(x);
  if (hb >= 4) fwht_stage_in<2>(x);
  if (hb >= 8) fwht_stage_in<4>(x);
  if (hb < 16) return 1.0f;
  const int c = fwht_chunk(lane, hb);
  {
    const float s = (c & 1) ? -1.0f : 1.0f;
    HDQ_FMAC_DPP8("quad_perm:[1,0,3,2]", "s_nop 1\n\t");
  }
  if (hb >= 32) {
    const float s = (c & 2) ? -1.0f : 1.0f;
    HDQ_FMAC_DPP8("quad_perm:[2,3,0,1]", "");
  }
  if (hb >= 64) {
    const float s = (c & 4) ? -1.0f : 1.0f;
    HDQ_FMAC_DPP8("row_half_mirror", "");
  }
  if (hb >= 128) {
    const float s = (c & 8) ? -1.0f : 1.0f;
    HDQ_FMAC_DPP8("row_mirror", "");
  }
  return (__builtin_popcount(c) & 1) ? -1.0f : 1.0f;
}

// Hadamard blocks of 128 with 32 consecutive elements per lane: block q
// spans lanes 4q .. 4q + 3 in natural order (lane bit 0 = element bit 5,
// lane bit 1 = element bit 6).  Strides 1..16 run inside the lane, strides
// 32 and 64 are one v_fmac_f32_dpp per element over quad_perm [1,0,3,2] and
// [2,3,0,1], with the sign bookkeeping described above: the returned sign is
// the parity of lane bits 0 and 1.
#define HDQ_FMAC_DPP8_AT(CTRL, NOP, O)                                                       \
  asm(NOP                                                                                    \
      "v_fmac_f32_dpp %0, %0, %8 " CTRL " row_mask:0xf bank_mask:0xf bound_ctrl:1\n\t"       \
      "v_fmac_f32_dpp %1, %1, %8 " CTRL " row_mask:0xf bank_mask:0xf bound_ctrl:1\n\t"       \
      "v_fmac_f32_dpp %2, %2, %8 " CTRL " row_mask:0xf bank_mask:0xf bound_ctrl:1\n\t"       \
      "v_fmac_f32_dpp %3, %3, %8 " CTRL " row_mask:0xf bank_mask:0xf bound_ctrl:1\n\t"       \
      "v_fmac_f32_dpp %4, %4, %8 " CTRL " row_mask:0xf bank_mask:0xf bound_ctrl:1\n\t"       \
      "v_fmac_f32_dpp %5, %5, %8 " CTRL " row_mask:0xf bank_mask:0xf bound_ctrl:1\n\t"       \
      "v_fmac_f32_dpp %6, %6, %8 " CTRL " row_mask:0xf bank_mask:0xf bound_ctrl:1\n\t"       \
      "v_fmac_f32_dpp %7, %7, %8 " CTRL " row_mask:0xf bank_mask:0xf bound_ctrl:1"           \
      : "+v"(x[O + 0]), "+v"(x[O + 1]), "+v"(x[O + 2]), "+v"(x[O + 3]), "+v"(x[O + 4]),       \
        "+v"(x[O + 5]), "+v"(x[O + 6]), "+v"(x[O + 7])                                        \
      : "v"(s))

__device__ __forceinline__ float fwht128_w32(float (&x)[32], int lane) {
#pragma unroll
  for (int h = 1; h < 32; h <<= 1) {
#pragma unroll
    for (int i = 0; i < 32; ++i) {
      if ((i & h) == 0) {
        const float u = x[i], v = x[i + h];
        x[i] = u + v;
        x[i + h] = u - v;
      }
    }
  }
  // Every block of the first cross-lane stage starts with the two wait
  // states a DPP read needs after a VALU write (the compiler may place the
  // last in-lane writes of any register right before it); the second
  // stage's sources were last written by the first stage's blocks, at
  // least 24 instructions earlier.
  {
    const float s = (lane & 1) ? -1.0f : 1.0f;
    HDQ_FMAC_DPP8_AT("quad_perm:[1,0,3,2]", "s_nop 1\n\t", 0);
    HDQ_FMAC_DPP8_AT("quad_perm:[1,0,3,2]", "s_nop 1\n\t", 8);
    HDQ_FMAC_DPP8_AT("quad_perm:[1,0,3,2]", "s_nop 1\n\t", 16);
    HDQ_FMAC_DPP8_AT("quad_perm:[1,0,3,2]", "s_nop 1\n\t", 24);
  }
  {
    const float s = (lane & 2) ? -1.0f : 1.0f;
    HDQ_FMAC_DPP8_AT("quad_perm:[2,3,0,1]", "s_nop 1\n\t", 0);
    HDQ_FMAC_DPP8_AT("quad_perm:[2,3,0,1]", "", 8);
    HDQ_FMAC_DPP8_AT("quad_perm:[2,3,0,1]", "", 16);
    HDQ_FMAC_DPP8_AT("quad_perm:[2,3,0,1]", "", 24);
  }
  return (((lane ^ (lane >> 1)) & 1) != 0) ? -1.0f : 1.0f;
}
#undef HDQ_FMAC_DPP8_AT
#undef HDQ_FMAC_DPP8

// ---- FP8 E4M3 block scales (unsigned) -------------------------------------
// Nearest E4M3 value of t >= 0, ties to even, saturating at 448 (0x7e).
// v_cvt_pk_fp8_f32 rounds to nearest even for t <= 448 but turns values
// above 464 into the NaN code, hence the clamp.
__device__ __forceinline__ uint32_t e4m3_encode(float t) {
  const float c = fminf(t, 448.0f);
  return (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(c, c, 0, false) & 0xffu;
}

// Value of an unsigned E4M3 byte (0x00..0x7e).
__device__ __forceinline__ float e4m3_decode(uint32_t c) {
  const uint32_t e = c >> 3, m = c & 7u;
  return e ? __uint_as_float(((e + 120u) << 23) | (m << 20)) : (float)m * 0x1p-9f;
}

// Four signed E4M3 bytes of w (byte i -> out[i]) as float32: the hardware
// conversion (OCP E4M3 on gfx950), exact.
__device__ __forceinline__ void e4m3x4_to_f32(uint32_t w, float* out) {
  const float2 lo = __builtin_bit_cast(float2, __builtin_amdgcn_cvt_pk_f32_fp8((int)w, false));
  const float2 hi = __builtin_bit_cast(float2, __builtin_amdgcn_cvt_pk_f32_fp8((int)w, true));
  out[0] = lo.x;
  out[1] = lo.y;
  out[2] = hi.x;
  out[3] = hi.y;
}

// Smallest power of two >= t, clamped to [2^-9, 2^8] (t >= 0).
__device__ __forceinline__ float pow2_ceil_clamped(float t) {
  if (!(t > 0x1p-9f)) return 0x1p-9f;
  if (t >= 256.0f) return 256.0f;
  const uint32_t u = __float_as_uint(t);
  if ((u & 0x007fffffu) == 0u) return t;
  return __uint_as_float((u & 0x7f800000u) + 0x00800000u);
}

// ---- FP4 E2M1 elements -----------------------------------------------------
// Two E2M1 codes (nearest, ties to even, saturating at 6, sign bit = sign of
// the input) in the low byte: a in bits 3:0, b in bits 7:4.
__device__ __forceinline__ uint32_t e2m1x2_encode(float a, float b) {
  return __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(0u, a, b, 1.0f, 0) & 0xffu;
}

// ---- GEMM tiling ------------------------------------------------------------
// 64-byte LDS rows: 16-byte chunk c of row r lives at chunk c ^ ((r >> 1) & 3),
// so a 16-byte fragment read of 8 consecutive rows touches distinct banks.
__device__ __forceinline__ int lds_off64(int r, int c) { return r * 64 + 16 * (c ^ ((r >> 1) & 3)); }

// Tile order.  Workgroups go round-robin to the 8 XCDs (blockIdx % 8), each
// with its own L2, so every XCD takes a contiguous range of the logical
// order.  The logical order walks groups of kGroupM tile rows column by
// column: the ~32 tiles an XCD runs at once then span kGroupM rows x
// 32/kGroupM columns and share their A and B strips in that XCD's L2,
// instead of one A strip and 32 B strips.
constexpr int kGroupM = 4;

// Logical tile index -> (tile row, tile column) in the grouped order.
__device__ __forceinline__ void grouped_tile(int logical, int tiles_m, int tiles_n, int& tm, int& tn) {
  const int per_group = kGroupM * tiles_n;
  const int g = logical / per_group, in_g = logical - g * per_group;
  const int rows = min(kGroupM, tiles_m - g * kGroupM);
  tn = in_g / rows;
  tm = g * kGroupM + (in_g - tn * rows);
}

// XCD x's contiguous range [lo, hi) of the logical order.
__device__ __forceinline__ void xcd_range(int total, int xcd, int& lo, int& hi) {
  const int q = total >> 3, r = total & 7;
  lo = xcd * q + (xcd < r ? xcd : r);
  hi = lo + q + (xcd < r ? 1 : 0);
}

// Logical tile of a workgroup in a grid of one workgroup per tile.
__device__ __forceinline__ void xcd_tile(int tiles_m, int tiles_n, int& tm, int& tn) {
  int lo, hi;
  xcd_range(tiles_m * tiles_n, blockIdx.x & 7, lo, hi);
  grouped_tile(lo + (blockIdx.x >> 3), tiles_m, tiles_n, tm, tn);
}

// Tiles of a persistent workgroup: logical tiles first, first + stride, ...
// below end.  With one workgroup per tile (nwg == total) that is the
// xcd_tile tile alone; otherwise nwg is a multiple of 8 and the nwg / 8
// workgroups of an XCD deal its range round-robin, so the ones running at
// the same time hold consecutive logical tiles.
struct TileSeq {
  int first, stride, count;
};
// nwg: the workgroups that share the tiles (0: the whole grid), a multiple of
// 8 when smaller than total; workgroups beyond them do other work.
__device__ __forceinline__ TileSeq tile_seq(int total, int nwg = 0) {
  if (nwg <= 0) nwg = (int)gridDim.x;
  int lo, hi;
  xcd_range(total, blockIdx.x & 7, lo, hi);
  const int local = blockIdx.x >> 3;
  if (nwg >= total) return TileSeq{lo + local, 1, 1};
  const int per = nwg >> 3;
  const int n = hi - lo - local;
  return TileSeq{lo + local, per, n > 0 ? (n + per - 1) / per : 0};
}

// ---- multi-stage LDS pipelines ------------------------------------------------
// Conflict-free 16-byte-chunk swizzles for fragment reads in which lane l
// reads row l % 32 (consecutive lanes, consecutive rows), both under a 32-bank
// (8 lanes per LDS cycle) and a 64-bank (16 lanes per cycle) model.
// 64-byte rows (4 chunks) and 128-byte rows (8 chunks):
__device__ __forceinline__ int swz64(int r) { return ((r >> 2) & 3) ^ (r & 2); }
__device__ __forceinline__ int swz128(int r) { return (r & 7) ^ ((r >> 3) & 1); }

// Workgroup barrier that orders LDS only: waits for this wave's LDS accesses
// (lgkmcnt) but not for its outstanding global loads, so prefetches for later
// pipeline stages stay in flight across the barrier.  (__syncthreads()'s
// fence would also wait for every global load.)
__device__ __forceinline__ void lds_barrier() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

// Barrier for LDS filled by LDS-DMA loads (lds_dma16): wait until at most
// PENDING of this wave's vector memory operations are outstanding (they
// complete in order, so the older ones have landed in LDS), then s_barrier.
// No fence: a workgroup LDS fence would wait for every DMA load in flight.
// The empty asm statements keep the compiler from moving LDS accesses
// across the barrier.
template <int PENDING>
__device__ __forceinline__ void dma_barrier() {
  static_assert(PENDING >= 0 && PENDING < 64, "vmcnt has six bits");
  // s_waitcnt: vmcnt bits [3:0] and [15:14], expcnt and lgkmcnt left at max.
  __builtin_amdgcn_s_waitcnt(0x0F70 | (PENDING & 15) | ((PENDING >> 4) << 14));
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

// Wait until at most PENDING of this wave's vector memory operations are
// outstanding (LDS-DMA loads complete in order).
template <int PENDING>
__device__ __forceinline__ void wait_vmem() {
  static_assert(PENDING >= 0 && PENDING < 64, "vmcnt has six bits");
  __builtin_amdgcn_s_waitcnt(0x0F70 | (PENDING & 15) | ((PENDING >> 4) << 14));
}

// Wait for all of this wave's LDS reads (lgkmcnt(0), the other counters at
// their maximum).
__device__ __forceinline__ void wait_lds() { __builtin_amdgcn_s_waitcnt(0xC07F); }

// Workgroup barrier after this wave's LDS accesses only (lgkmcnt(0)), for
// LDS that is not being filled by LDS-DMA: unlike lds_barrier's fence it does
// not wait for DMA loads in flight to other LDS.  The empty asm statements
// keep the compiler from moving memory accesses across it.
__device__ __forceinline__ void lds_only_barrier() {
  wait_lds();
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

// Workgroup barrier after all of this wave's vector memory operations
// (LDS-DMA loads included) and LDS accesses have completed.
__device__ __forceinline__ void stage_barrier() {
  __builtin_amdgcn_s_waitcnt(0x0070);  // vmcnt(0) lgkmcnt(0), expcnt at its maximum
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

// Bare workgroup barrier for a phase-scheduled loop: the compiler may move
// no instruction across it (sched_barrier) and no memory access (empty asm
// with a memory clobber); no fence and no wait.
__device__ __forceinline__ void phase_barrier() {
  __builtin_amdgcn_sched_barrier(0);
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
  __builtin_amdgcn_sched_barrier(0);
}

// A staged 16-byte piece of a GEMM output row, stored non-temporally: the
// output is written once and read by a later kernel, so it should not evict
// the operand panels the other tiles of this launch still reuse from L2
// (measured 1-3% faster GEMMs).
__device__ __forceinline__ void store16_nt(void* dst, const void* src) {
  __builtin_nontemporal_store(*reinterpret_cast<const v4i*>(src), reinterpret_cast<v4i*>(dst));
}

// ---- buffer loads ----------------------------------------------------------------
// Raw buffer resource over [base, base + bytes): loads at offsets >= bytes
// return zeros, so tile rows past the end of a tensor read as zero.  The
// scalar offset argument keeps per-stage / per-row-block offsets in SGPRs.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes, 0x00020000);
}
__device__ __forceinline__ uint4 buf_load16(__amdgpu_buffer_rsrc_t r, uint32_t voff, uint32_t soff) {
  return __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(r, (int)voff, (int)soff, 0));
}
// LDS-DMA buffer load: the wave's 64 lanes each read 16 bytes (at voff + soff
// of the resource; past its end they read zero) and write them to LDS at
// lds + 16 * lane.  lds must be the same for the whole wave.
__device__ __forceinline__ void lds_dma16(__amdgpu_buffer_rsrc_t r, void* lds, uint32_t voff, uint32_t soff) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (__attribute__((address_space(3))) void*)lds, 16, (int)voff,
                                           (int)soff, 0, 0);
}

}  // namespace hdq
