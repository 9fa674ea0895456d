// stats.hip -- selection statistics and the precision decision (gfx950).
//
// The summary of 6Bit-Diffusion (vetunion.cn) picks each module's precision
// per step from the difference between its input and output at the previous
// step (section one: large -> INT8, small -> NVFP4), falls back to full
// precision when the input's outlier ratio max/mean is too large (section
// three, purified delta refresh), and uses INT8 when no previous-step
// difference exists (section three, last paragraph).  The explainer on
// gist.science restates both rules (sections 2 and 4).
//
// One streaming pass reads prev_in, prev_out and cur (6 bytes per element,
// HBM-bound) and writes per-workgroup partials; a one-workgroup finalize
// reduces them in a fixed order in double, so the statistics and the
// decision are deterministic.  The same pass yields the rotated amax that
// NVFP4's tensor scale needs, so the quantizer never reads its input twice.
#include "hdq_device.h"
#include "hdq_internal.h"

#include <math.h>

namespace hdq {

// Partial slots per workgroup.
enum { P_DIFF = 0, P_BASE = 1, P_SUMABS = 2, P_MAXBITS = 3, P_ROTMAX = 4, P_COUNT = 6 };

__device__ __forceinline__ double wave_sum_d(double v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v += __shfl_xor(v, o);
  return v;
}
__device__ __forceinline__ uint32_t wave_max_u(uint32_t v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v = max(v, (uint32_t)__shfl_xor((int)v, o));
  return v;
}

// Sums of the pairs {p[2i], p[2i + 1]}, i < n, in a fixed order: thread t
// adds i = t, t + T, ... in turn, then a fixed tree over the threads (red:
// 2T doubles of LDS).  Every thread calls it; thread 0 gets the sums.  One
// pair (n = 1) comes out exactly as stored.
template <int T>
__device__ __forceinline__ void pair_sums(const double* __restrict__ p, int64_t n, double* red, double& d,
                                          double& b) {
  const int tid = threadIdx.x;
  double x = 0.0, y = 0.0;
  for (int64_t i = tid; i < n; i += T) {
    x += p[2 * i];
    y += p[2 * i + 1];
  }
  red[2 * tid] = x;
  red[2 * tid + 1] = y;
  __syncthreads();
  for (int h = T / 2; h >= 1; h >>= 1) {
    if (tid < h) {
      red[2 * tid] += red[2 * (tid + h)];
      red[2 * tid + 1] += red[2 * (tid + h) + 1];
    }
    __syncthreads();
  }
  d = red[0];
  b = red[1];
}

// MODE: 0 both passes (prev_in may be null), 1 the difference pass alone,
// 2 the current-input pass alone.  The modes share the loops, so a split
// pair of launches gives the partials of one combined launch bit for bit.
enum { kPassBoth = 0, kPassDelta = 1, kPassCur = 2 };

template <int MODE>
__global__ __launch_bounds__(256) void k_stats_partial(
    const uint16_t* __restrict__ prev_in, const uint16_t* __restrict__ prev_out, int64_t n_prev,
    const uint16_t* __restrict__ cur, int64_t n_cur, int hb, double* __restrict__ part,
    const int32_t* __restrict__ gate, int32_t want) {
  if (gate != nullptr && *gate != want) return;
  const int tid = threadIdx.x, lane = tid & 63;
  const int64_t gtid = (int64_t)blockIdx.x * 256 + tid;
  const int64_t gthreads = (int64_t)gridDim.x * 256;

  // --- relative L1 difference of the previous step's input and output.
  // float32 sums over each 8-element chunk, double across chunks.
  double diff = 0.0, base = 0.0;
  if (MODE != kPassCur && prev_in != nullptr) {
    const int64_t nch = n_prev >> 3;
    const uint4* a4 = reinterpret_cast<const uint4*>(prev_in);
    const uint4* o4 = reinterpret_cast<const uint4*>(prev_out);
    // two chunks per thread per iteration: four loads in flight
    for (int64_t j = gtid; j < nch; j += 2 * gthreads) {
      const int64_t j2 = j + gthreads;
      const uint4 ra = a4[j], ro = o4[j];
      const uint4 ra2 = j2 < nch ? a4[j2] : make_uint4(0u, 0u, 0u, 0u);
      const uint4 ro2 = j2 < nch ? o4[j2] : make_uint4(0u, 0u, 0u, 0u);
      float a[8], o[8];
      bf16x8_to_f32(ra, a);
      bf16x8_to_f32(ro, o);
      float d8 = 0.0f, b8 = 0.0f;
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        d8 += fabsf(o[i] - a[i]);
        b8 += fabsf(a[i]);
      }
      diff += d8;
      base += b8;
      bf16x8_to_f32(ra2, a);
      bf16x8_to_f32(ro2, o);
      d8 = 0.0f;
      b8 = 0.0f;
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        d8 += fabsf(o[i] - a[i]);
        b8 += fabsf(a[i]);
      }
      diff += d8;
      base += b8;
    }
    const int64_t tail = n_prev - (nch << 3);
    if (gtid < tail) {
      const float a = bf16_lo(prev_in[(nch << 3) + gtid]);
      const float o = bf16_lo(prev_out[(nch << 3) + gtid]);
      diff += fabsf(o - a);
      base += fabsf(a);
    }
  }

  // --- current input: max |x| (on the bf16 bit patterns: for finite values
  // the order of |x| is the order of (bits & 0x7fff), and a pattern >= 0x7f80
  // flags an infinity or NaN), sum |x|, and max |rotated x| (unnormalised).
  uint32_t maxbits = 0u;
  double sumabs = 0.0;
  float rotmax = 0.0f;
  if (MODE != kPassDelta) {
    const int64_t nch = n_cur >> 3;
    const uint4* c4 = reinterpret_cast<const uint4*>(cur);
    const int64_t wave = gtid >> 6, nwaves = gthreads >> 6;
    // two chunks per lane per iteration (loads first); a wave covers 128
    // consecutive chunks, keeping Hadamard blocks inside aligned lane groups
    for (int64_t b0 = wave * 128; b0 < nch; b0 += nwaves * 128) {
      uint4 w2[2];
#pragma unroll
      for (int u = 0; u < 2; ++u) {
        const int64_t j = hb > 0 ? fwht_src(b0 + 64 * u + lane, lane, hb) : b0 + 64 * u + lane;
        w2[u] = (j < nch) ? c4[j] : make_uint4(0u, 0u, 0u, 0u);
      }
#pragma unroll
      for (int u = 0; u < 2; ++u) {
        const uint32_t wd[4] = {w2[u].x, w2[u].y, w2[u].z, w2[u].w};
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          maxbits = max(maxbits, wd[q] & 0x7fffu);
          maxbits = max(maxbits, (wd[q] >> 16) & 0x7fffu);
        }
        float v[8];
        bf16x8_to_f32(w2[u], v);
        float s8 = 0.0f;
#pragma unroll
        for (int i = 0; i < 8; ++i) s8 += fabsf(v[i]);
        sumabs += s8;
        if (hb > 0) {
          fwht8(v, lane, hb);
#pragma unroll
          for (int i = 0; i < 8; ++i) rotmax = fmaxf(rotmax, fabsf(v[i]));
        }
      }
    }
    const int64_t tail = n_cur - (nch << 3);
    if (gtid < tail) {  // only reachable without rotation (cols % 8 != 0)
      const uint32_t bits = cur[(nch << 3) + gtid];
      maxbits = max(maxbits, bits & 0x7fffu);
      sumabs += fabsf(bf16_lo(bits));
    }
  }

  // --- fixed-order workgroup reduction.
  __shared__ double red[4][5];
  diff = wave_sum_d(diff);
  base = wave_sum_d(base);
  sumabs = wave_sum_d(sumabs);
  maxbits = wave_max_u(maxbits);
  const float rm = wave_max(rotmax);
  if (lane == 0) {
    red[tid >> 6][0] = diff;
    red[tid >> 6][1] = base;
    red[tid >> 6][2] = sumabs;
    red[tid >> 6][3] = (double)maxbits;
    red[tid >> 6][4] = (double)rm;
  }
  __syncthreads();
  if (tid < 5) {
    double r = red[0][tid];
    for (int w = 1; w < 4; ++w) r = (tid == 3 || tid == 4) ? fmax(r, red[w][tid]) : r + red[w][tid];
    part[(int64_t)blockIdx.x * P_COUNT + tid] = r;
  }
}

// The statistics and the decision from the reduced sums (one thread).
__device__ void finish_stats(double diff, double base, double sumabs, uint32_t maxbits, float tmax,
                             int64_t n_cur, int has_history, float c_b, float delta_thresh,
                             float ratio_thresh, int32_t* decision, float* stats, float* amax_out) {
  const bool nonfinite = maxbits >= 0x7f80u;
  const double maxabs = (double)bf16_lo(maxbits);
  double delta;
  if (!has_history)
    delta = __builtin_nan("");
  else if (base == 0.0)
    delta = (diff == 0.0) ? 0.0 : __builtin_inf();
  else
    delta = diff / base;
  const double mean = sumabs / (double)n_cur;
  double ratio;
  if (nonfinite)
    ratio = __builtin_nan("");
  else
    ratio = (sumabs == 0.0) ? 0.0 : maxabs / mean;
  // max over fl32(|t| * c_b) equals fl32(max |t| * c_b): rounding is monotone.
  const float rot_amax = nonfinite ? 0.0f : tmax * c_b;
  if (stats != nullptr) {
    stats[0] = (float)delta;
    stats[1] = (float)ratio;
    stats[2] = (float)maxabs;
    stats[3] = (float)mean;
    stats[4] = rot_amax;
  }
  if (amax_out != nullptr) *amax_out = rot_amax;
  if (decision != nullptr) {
    int32_t d;
    if (!(ratio <= (double)ratio_thresh))
      d = kPrecBf16;  // purified delta refresh: outliers -> full precision
    else if (!has_history)
      d = kPrecInt8;  // no previous-step difference -> INT8
    else if (!(delta < (double)delta_thresh))
      d = kPrecInt8;  // large previous-step difference -> INT8
    else
      d = kPrecNvfp4;
    *decision = d;
  }
}

// Finalize.  With sums_out, only the two difference sums are written
// (sums_out[0] = sum|prev_out - prev_in|, sums_out[1] = sum|prev_in|).  With
// sums_in, those two sums come from an earlier difference-only pass instead
// of this pass's partials (which then hold the current input alone).  The
// reduction order is the same in every mode, so the split passes give the
// same bits as one pass over all three tensors on the same grid.
__global__ __launch_bounds__(256) void k_stats_final(
    const double* __restrict__ part, int nparts, int64_t n_cur, int has_history, float c_b,
    float delta_thresh, float ratio_thresh, int32_t* __restrict__ decision,
    float* __restrict__ stats, float* __restrict__ amax_out, const int32_t* __restrict__ gate,
    int32_t want, const double* __restrict__ sums_in, double* __restrict__ sums_out, int64_t sums_parts) {
  if (gate != nullptr && *gate != want) return;
  const int tid = threadIdx.x;
  __shared__ double pr[2 * 256];
  double din = 0.0, bin = 0.0;
  if (sums_in != nullptr) pair_sums<256>(sums_in, sums_parts, pr, din, bin);
  double acc[5] = {0.0, 0.0, 0.0, 0.0, 0.0};
  for (int p = tid; p < nparts; p += 256) {
    acc[0] += part[p * P_COUNT + 0];
    acc[1] += part[p * P_COUNT + 1];
    acc[2] += part[p * P_COUNT + 2];
    acc[3] = fmax(acc[3], part[p * P_COUNT + 3]);
    acc[4] = fmax(acc[4], part[p * P_COUNT + 4]);
  }
  __shared__ double red[256][5];
#pragma unroll
  for (int q = 0; q < 5; ++q) red[tid][q] = acc[q];
  __syncthreads();
  for (int s = 128; s >= 1; s >>= 1) {
    if (tid < s) {
      red[tid][0] += red[tid + s][0];
      red[tid][1] += red[tid + s][1];
      red[tid][2] += red[tid + s][2];
      red[tid][3] = fmax(red[tid][3], red[tid + s][3]);
      red[tid][4] = fmax(red[tid][4], red[tid + s][4]);
    }
    __syncthreads();
  }
  if (tid != 0) return;
  if (sums_out != nullptr) {
    sums_out[0] = red[0][0];
    sums_out[1] = red[0][1];
    return;
  }
  const double diff = sums_in != nullptr ? din : red[0][0];
  const double base = sums_in != nullptr ? bin : red[0][1];
  finish_stats(diff, base, red[0][2], (uint32_t)red[0][3], (float)red[0][4], n_cur, has_history, c_b,
               delta_thresh, ratio_thresh, decision, stats, amax_out);
}

// Finalize over one partial per row, struct-of-arrays (sum |x| doubles, max
// bf16 magnitude bits, max |rotated x| times c_b -- c_b is then 1), as the
// selection fused with INT8 quantization writes them: 1024 threads,
// coalesced, fixed order.
__global__ __launch_bounds__(1024) void k_stats_final_rows(
    const double* __restrict__ psum, const uint32_t* __restrict__ pbits,
    const float* __restrict__ ptmax, int nrows, int64_t n_cur, float c_b, float delta_thresh,
    float ratio_thresh, int32_t* __restrict__ decision, float* __restrict__ stats,
    const double* __restrict__ sums_in, int64_t sums_parts) {
  const int tid = threadIdx.x, lane = tid & 63;
  __shared__ double pr[2 * 1024];
  double din = 0.0, bin = 0.0;
  if (sums_in != nullptr) pair_sums<1024>(sums_in, sums_parts, pr, din, bin);
  // four independent accumulators (fixed order) keep several loads in flight
  double s4[4] = {0.0, 0.0, 0.0, 0.0};
  uint32_t mb = 0u;
  float tm = 0.0f;
  int r = tid;
  for (; r + 3 * 1024 < nrows; r += 4 * 1024) {
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      s4[u] += psum[r + u * 1024];
      mb = max(mb, pbits[r + u * 1024]);
      tm = fmaxf(tm, ptmax[r + u * 1024]);
    }
  }
  for (int u = 0; r < nrows; r += 1024, ++u) {
    s4[u] += psum[r];
    mb = max(mb, pbits[r]);
    tm = fmaxf(tm, ptmax[r]);
  }
  double sa = (s4[0] + s4[1]) + (s4[2] + s4[3]);
  sa = wave_sum_d(sa);
  mb = wave_max_u(mb);
  tm = wave_max(tm);
  __shared__ double rs[16];
  __shared__ uint32_t rb[16];
  __shared__ float rt[16];
  if (lane == 0) {
    rs[tid >> 6] = sa;
    rb[tid >> 6] = mb;
    rt[tid >> 6] = tm;
  }
  __syncthreads();
  if (tid != 0) return;
  for (int w = 1; w < 16; ++w) {
    rs[0] += rs[w];
    rb[0] = max(rb[0], rb[w]);
    rt[0] = fmaxf(rt[0], rt[w]);
  }
  const bool hist = sums_in != nullptr;
  finish_stats(din, bin, rs[0], rb[0], rt[0], n_cur,
               hist ? 1 : 0, c_b, delta_thresh, ratio_thresh, decision, stats, nullptr);
}

hipError_t launch_stats(const uint16_t* prev_in, const uint16_t* prev_out, int64_t prev_numel,
                        const uint16_t* cur, int64_t cur_numel, int hb, float delta_thresh,
                        float ratio_thresh, int32_t* decision, float* stats, float* amax_out,
                        double* partials, const int32_t* gate, int32_t want, hipStream_t s,
                        const double* delta_sums_in, double* delta_sums_out, int64_t delta_parts) {
  const int64_t work = (prev_numel > cur_numel ? prev_numel : cur_numel) / 8;
  int64_t blocks = (work + 255) / 256;
  if (blocks > kStatsMaxBlocks) blocks = kStatsMaxBlocks;
  if (blocks < 1) blocks = 1;
  const bool hist = prev_in != nullptr && prev_out != nullptr;
  auto kern = !hist ? k_stats_partial<kPassCur>
                    : (cur == nullptr ? k_stats_partial<kPassDelta> : k_stats_partial<kPassBoth>);
  hipLaunchKernelGGL(kern, dim3((unsigned)blocks), dim3(256), 0, s, hist ? prev_in : nullptr,
                     hist ? prev_out : nullptr, hist ? prev_numel : 0, cur, cur_numel, hb, partials,
                     gate, want);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const float c_b = hb > 0 ? hadamard_scale(hb) : 0.0f;
  hipLaunchKernelGGL(k_stats_final, dim3(1), dim3(256), 0, s, partials, (int)blocks, cur_numel,
                     (hist || delta_sums_in != nullptr) ? 1 : 0, c_b, delta_thresh, ratio_thresh,
                     decision, stats, amax_out, gate, want, delta_sums_in, delta_sums_out, delta_parts);
  return hipGetLastError();
}

hipError_t launch_stats_finalize_rows(const double* psum, const uint32_t* pbits, const float* ptmax,
                                      int64_t rows, int64_t cur_numel, int hb, float delta_thresh,
                                      float ratio_thresh, int32_t* decision, float* stats,
                                      const double* delta_sums_in, int64_t delta_parts, hipStream_t s) {
  // ptmax holds rows' max |rotated x| already scaled by fl32(1/sqrt(hb)):
  // fl32(max |t| * c_b) = max fl32(|t| * c_b), so the finalize scales by 1
  (void)hb;
  hipLaunchKernelGGL(k_stats_final_rows, dim3(1), dim3(1024), 0, s, psum, pbits, ptmax, (int)rows,
                     cur_numel, 1.0f, delta_thresh, ratio_thresh, decision, stats, delta_sums_in, delta_parts);
  return hipGetLastError();
}

// ---------------------------------------------------- temporal delta cache

// The temporal delta cache's skip rule (summary on vetunion.cn, section
// two; gist.science explainer, section three), one thread per module: a
// module computed at this step (state 1: no earlier output; 2: with one,
// sums = {sum|new - earlier|, sum|earlier|}) resets its accumulator and
// takes a new relative change c; every module then reuses its cache at the
// next step when c < tau_skip and fl32(acc + c) <= tau_acc, adding c to acc.
// The rule for module i from its state, change sums and accumulator.
__device__ __forceinline__ void tdc_rule(int i, int st, double diff, double base, float* __restrict__ c,
                                         float* __restrict__ acc, int32_t* __restrict__ skip,
                                         float tau_skip, float tau_acc) {
  float ci = c[i], ai = acc[i];
  if (st != 0) {
    ai = 0.0f;
    if (st == 1) {
      ci = __builtin_nanf("");
    } else {
      ci = (float)(base == 0.0 ? (diff == 0.0 ? 0.0 : __builtin_inf()) : diff / base);
    }
  }
  const float next = ai + ci;
  const bool sk = ci < tau_skip && next <= tau_acc;
  c[i] = ci;
  acc[i] = sk ? next : ai;
  skip[i] = sk ? 1 : 0;
}

__global__ __launch_bounds__(256) void k_tdc_decide(const double* __restrict__ sums,
                                                    const int32_t* __restrict__ state,
                                                    float* __restrict__ c, float* __restrict__ acc,
                                                    int32_t* __restrict__ skip, int n, float tau_skip,
                                                    float tau_acc) {
  for (int i = blockIdx.x * 256 + threadIdx.x; i < n; i += gridDim.x * 256) {
    const int st = state[i];
    tdc_rule(i, st, st == 2 ? sums[2 * i] : 0.0, st == 2 ? sums[2 * i + 1] : 0.0, c, acc, skip, tau_skip,
             tau_acc);
  }
}

// Change sums given as pairs: module i's are pairs [off[i], off[i + 1]),
// summed in a fixed order by the module's workgroup.
__global__ __launch_bounds__(256) void k_tdc_decide_parts(const double* __restrict__ parts,
                                                          const int64_t* __restrict__ off,
                                                          const int32_t* __restrict__ state,
                                                          float* __restrict__ c, float* __restrict__ acc,
                                                          int32_t* __restrict__ skip, float tau_skip,
                                                          float tau_acc) {
  __shared__ double red[2 * 256];
  const int i = blockIdx.x;
  const int st = state[i];
  double d = 0.0, b = 0.0;
  if (st == 2) pair_sums<256>(parts + 2 * off[i], off[i + 1] - off[i], red, d, b);
  if (threadIdx.x == 0) tdc_rule(i, st, d, b, c, acc, skip, tau_skip, tau_acc);
}

hipError_t launch_tdc_decide(const double* sums, const int64_t* parts_off, const int32_t* state, float* c,
                             float* acc, int32_t* skip, int64_t n, float tau_skip, float tau_acc,
                             hipStream_t s) {
  if (parts_off != nullptr) {
    hipLaunchKernelGGL(k_tdc_decide_parts, dim3((unsigned)n), dim3(256), 0, s, sums, parts_off, state, c,
                       acc, skip, tau_skip, tau_acc);
    return hipGetLastError();
  }
  int64_t blocks = (n + 255) / 256;
  if (blocks > 1024) blocks = 1024;
  hipLaunchKernelGGL(k_tdc_decide, dim3((unsigned)blocks), dim3(256), 0, s, sums, state, c, acc, skip,
                     (int)n, tau_skip, tau_acc);
  return hipGetLastError();
}

}  // namespace hdq
