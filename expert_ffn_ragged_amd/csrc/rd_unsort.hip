// Limit-aware weighted unsort backward for gfx950.
//
// MaxText PR #5760 ("397B v7x trainer: MoE wo FSDP sharding and
// valid-rows-only MoE kernels"), commit on valid rows, unsort_bwd_rows: for
// the rows [0, limit) of the packed expert buffer, the gradient of the
// expert outputs is bf16(f32(g) * w[row]) (one float32 multiply, rounded once
// to bf16) and the gradient of the routing weights is the float32 row dot
// sum_c f32(g[row, c]) * f32(y[row, c]); only the dot's summation order is
// free.  Rows at or past the limit are neither read nor written.
//
// One wave64 owns a row: lane l handles the 16-byte chunks l, l + 64, ... of
// it (128-bit non-temporal loads of g and y and stores of the gradient, eight
// chunks in flight per lane), keeps its part of the dot in float64, and the
// wave adds the 64 parts in a fixed butterfly order before one rounding to
// float32.  Each product of two bf16 values is exact in float32, and a
// float64 sum of a few thousand of them is within about 1e-12 relative of the
// exact dot, so the float32 result is the exact dot rounded once (within half
// a float32 ulp), whatever the order.  A row's dot is produced by exactly one
// wave: no partial sums cross workgroups, no atomics, and the result is the
// same on every run.  A persistent grid of waves (32
// workgroups per CU) strides over the valid rows.  HBM-bound: 3 * 2 * hidden + 8 bytes per row.
#include "rd_device.h"
#include "rd_launch.h"

namespace rd {
namespace {

constexpr int kUnroll = 8;  // 16-byte chunks per lane in flight (all of a 4096-wide row: 558 -> 545 us)

typedef unsigned int nt_u32x4 __attribute__((ext_vector_type(4)));

// 128-bit loads and stores marked non-temporal (every byte is touched once).
__device__ __forceinline__ uint4 nt_load(const uint4* p) {
  const nt_u32x4 v = __builtin_nontemporal_load(reinterpret_cast<const nt_u32x4*>(p));
  return make_uint4(v.x, v.y, v.z, v.w);
}
__device__ __forceinline__ void nt_store(uint4* p, uint4 v) {
  const nt_u32x4 x = {v.x, v.y, v.z, v.w};
  __builtin_nontemporal_store(x, reinterpret_cast<nt_u32x4*>(p));
}

__device__ __forceinline__ float bf_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf_hi(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }

// Gradient word (two bf16) and the dot contribution of one 32-bit word pair.
__device__ __forceinline__ uint32_t grad_word(uint32_t gw, float w) {
  const float a = bf_lo(gw) * w;  // a single float32 multiply: rounded once, then once more to bf16
  const float b = bf_hi(gw) * w;
  return pack_bf16x2(a, b);
}

// Exact float32 products (8-bit significands), accumulated in float64.
__device__ __forceinline__ double dot_word(uint32_t gw, uint32_t yw, double acc) {
  acc += static_cast<double>(bf_lo(gw) * bf_lo(yw));
  acc += static_cast<double>(bf_hi(gw) * bf_hi(yw));
  return acc;
}

__global__ __launch_bounds__(kThreads) void unsort_bwd_rows_kernel(const uint16_t* __restrict__ g,
                                                                   const uint16_t* __restrict__ y,
                                                                   const float* __restrict__ w,
                                                                   const int32_t* __restrict__ limp,
                                                                   uint16_t* __restrict__ grad,
                                                                   float* __restrict__ dot, int rows, int hidden) {
  int L = rows;
  if (limp != nullptr) {
    const int v = *limp;
    L = v < 0 ? 0 : (v > rows ? rows : v);
  }
  const int lane = threadIdx.x & 63;
  const int waves = gridDim.x * (kThreads / 64);
  const int chunks = hidden >> 3;  // 16-byte chunks per row
  for (int r = blockIdx.x * (kThreads / 64) + (threadIdx.x >> 6); r < L; r += waves) {
    const float wr = w[r];
    const uint4* gr = reinterpret_cast<const uint4*>(g + static_cast<long long>(r) * hidden);
    const uint4* yr = reinterpret_cast<const uint4*>(y + static_cast<long long>(r) * hidden);
    uint4* dr = reinterpret_cast<uint4*>(grad + static_cast<long long>(r) * hidden);
    double acc = 0.0;
    int c = lane;
    for (; c + 64 * (kUnroll - 1) < chunks; c += 64 * kUnroll) {
      uint4 gv[kUnroll], yv[kUnroll];
#pragma unroll
      for (int u = 0; u < kUnroll; ++u) {
        gv[u] = nt_load(gr + c + 64 * u);
        yv[u] = nt_load(yr + c + 64 * u);
      }
#pragma unroll
      for (int u = 0; u < kUnroll; ++u) {
        nt_store(dr + c + 64 * u, make_uint4(grad_word(gv[u].x, wr), grad_word(gv[u].y, wr),
                                             grad_word(gv[u].z, wr), grad_word(gv[u].w, wr)));
        acc = dot_word(gv[u].x, yv[u].x, acc);
        acc = dot_word(gv[u].y, yv[u].y, acc);
        acc = dot_word(gv[u].z, yv[u].z, acc);
        acc = dot_word(gv[u].w, yv[u].w, acc);
      }
    }
    for (; c < chunks; c += 64) {
      const uint4 gv = nt_load(gr + c), yv = nt_load(yr + c);
      nt_store(dr + c,
               make_uint4(grad_word(gv.x, wr), grad_word(gv.y, wr), grad_word(gv.z, wr), grad_word(gv.w, wr)));
      acc = dot_word(gv.x, yv.x, acc);
      acc = dot_word(gv.y, yv.y, acc);
      acc = dot_word(gv.z, yv.z, acc);
      acc = dot_word(gv.w, yv.w, acc);
    }
#pragma unroll
    for (int d = 32; d >= 1; d >>= 1) acc += __shfl_xor(acc, d, 64);
    if (lane == 0) dot[r] = static_cast<float>(acc);
  }
}

}  // namespace

int launch_unsort_bwd_rows(const void* g, const void* y, const float* w, const int32_t* limit, void* grad,
                           float* dot, int rows, int hidden, hipStream_t stream) {
  const long long waves_needed = rows;
  long long blocks = (waves_needed + (kThreads / 64) - 1) / (kThreads / 64);
  const long long cap = static_cast<long long>(device_cu_count()) * 32;
  if (blocks > cap) blocks = cap;
  if (blocks < 1) blocks = 1;
  unsort_bwd_rows_kernel<<<static_cast<int>(blocks), kThreads, 0, stream>>>(
      static_cast<const uint16_t*>(g), static_cast<const uint16_t*>(y), w, limit, static_cast<uint16_t*>(grad), dot,
      rows, hidden);
  return hipGetLastError() == hipSuccess ? RD_OK : RD_EHIP;
}

}  // namespace rd
