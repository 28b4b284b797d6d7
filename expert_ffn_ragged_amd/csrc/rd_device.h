// Device-side building blocks shared by the grouped-GEMM kernels:
// vector types, bf16 conversions, block scans and the device-resident group
// schedule (boundaries of the local groups computed from group_sizes without
// any host involvement).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "rd.h"

namespace rd {

constexpr int kThreads = 256;  // default workgroup: 4 wave64s (the wide GEMM tiles run 8)
constexpr int kXcds = 8;       // MI355X: workgroups are dealt round-robin over 8 XCDs

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef short s16x4_t __attribute__((ext_vector_type(4)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));

__device__ __forceinline__ float bf16_to_f32(uint32_t bits16) { return __uint_as_float(bits16 << 16); }

// float32 -> bf16 bits, round to nearest even (gfx950 converts in hardware; NaN stays NaN).
__device__ __forceinline__ uint32_t f32_to_bf16(float f) {
  return static_cast<uint32_t>(__builtin_bit_cast(uint16_t, static_cast<__bf16>(f)));
}

__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  return f32_to_bf16(lo) | (f32_to_bf16(hi) << 16);
}

// Inclusive scan of one int64 per lane across a wave64.
__device__ __forceinline__ long long wave_incl_scan(long long x) {
  const int lane = threadIdx.x & 63;
#pragma unroll
  for (int d = 1; d < 64; d <<= 1) {
    long long y = __shfl_up(x, d, 64);
    if (lane >= d) x += y;
  }
  return x;
}

// Exclusive scan of one int64 per thread across the NT-thread block.
// s_wave: NT / 64 int64 of LDS.  Contains two barriers; call from uniform control flow.
template <int NT = kThreads>
__device__ __forceinline__ long long block_excl_scan(long long tot, long long* s_wave) {
  const long long inc = wave_incl_scan(tot);
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  if (lane == 63) s_wave[w] = inc;
  __syncthreads();
  long long base = 0;
  for (int i = 0; i < w; ++i) base += s_wave[i];
  __syncthreads();
  return base + inc - tot;
}

struct Window {
  int lo, hi, L;
};

// Local group boundaries, computed by every workgroup from device memory.
//
// c[i] = sum_{t<i} max(gs[t], 0) (exclusive prefix, int64), b[i] = min(c[i], L),
// s_lb[j] = b[off + j] for j in [0, gl].  A window that does not fit
// (off < 0 or off + gl > G) gives s_lb = 0 everywhere (no rows).
// L = clamp(*limit, 0, m), or m without a limit.
// Requires G, gl <= 4 * NT (NT threads in the block).  Ends with a barrier.
template <int NT = kThreads>
__device__ __forceinline__ Window build_local_bounds(const int32_t* __restrict__ gs, int G,
                                                     const int32_t* __restrict__ offp, int gl,
                                                     const int32_t* __restrict__ limp, int m, int* s_lb,
                                                     long long* s_wave) {
  int L = m;
  if (limp != nullptr) {
    const int v = *limp;
    L = v < 0 ? 0 : (v > m ? m : v);
  }
  const int off = offp != nullptr ? *offp : 0;
  const bool ok = off >= 0 && off <= G - gl;
  const int t = threadIdx.x;
  long long v[4];
  long long tot = 0;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int idx = 4 * t + i;
    const int s = idx < G ? gs[idx] : 0;
    v[i] = s > 0 ? s : 0;
    tot += v[i];
  }
  long long run = block_excl_scan<NT>(tot, s_wave);
  if (ok) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int pos = 4 * t + i - off;
      if (pos >= 0 && pos <= gl) s_lb[pos] = static_cast<int>(run < L ? run : L);
      run += v[i];
    }
    if (t == NT - 1) {  // boundary G when G == 4 * NT
      const int pos = 4 * NT - off;
      if (pos >= 0 && pos <= gl) s_lb[pos] = static_cast<int>(run < L ? run : L);
    }
  } else {
    for (int j = t; j <= gl; j += NT) s_lb[j] = 0;
  }
  __syncthreads();
  return Window{s_lb[0], s_lb[gl], L};
}

// s_out[j] = sum_{i<j} cnt(i) for j in [0, n], cnt(i) = ceil((s_lb[i+1]-s_lb[i]) / tile).
// Returns the total.  Requires n <= 4 * NT.  Ends with a barrier.
template <int NT = kThreads>
__device__ __forceinline__ int tile_prefix(const int* s_lb, int n, int tile, int* s_out, long long* s_wave) {
  const int t = threadIdx.x;
  int c[4];
  long long tot = 0;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int j = 4 * t + i;
    c[i] = j < n ? (s_lb[j + 1] - s_lb[j] + tile - 1) / tile : 0;
    tot += c[i];
  }
  long long run = block_excl_scan<NT>(tot, s_wave);
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int j = 4 * t + i;
    if (j <= n) s_out[j] = static_cast<int>(run);
    run += c[i];
  }
  if (t == NT - 1 && n == 4 * NT) s_out[n] = static_cast<int>(run);
  __syncthreads();
  return s_out[n];
}

// Largest j in [0, n-1] with s_pre[j] <= x (s_pre non-decreasing, s_pre[0] <= x < s_pre[n]).
__device__ __forceinline__ int upper_index(const int* s_pre, int n, int x) {
  int lo = 0, hi = n - 1;
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (s_pre[mid] <= x)
      lo = mid;
    else
      hi = mid - 1;
  }
  return lo;
}

// Persistent-grid tile order that keeps consecutive logical tiles on one XCD.
// Slot s (= blockIdx + iteration * gridDim) runs on XCD s % kXcds when gridDim is a
// multiple of kXcds; logical tiles [x*C, (x+1)*C) go to XCD x, in order.
__device__ __forceinline__ long long xcd_logical(long long slot, long long per_xcd) {
  return (slot % kXcds) * per_xcd + slot / kXcds;
}

}  // namespace rd
