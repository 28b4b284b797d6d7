// Limit-aware silu(gate) * up GLU, forward and backward, for gfx950.
//
// MaxText PR #5760 ("397B v7x trainer: MoE wo FSDP sharding and
// valid-rows-only MoE kernels"), commit on valid rows: only rows [0, limit)
// of the packed expert buffer are read or written; gate and up are read in
// place from the fused [gate | up] buffer; the forward evaluates negate, exp,
// + 1, divide, multiply in float32 and rounds only the output; the backward
// writes [d_gate | d_up] in one pass and maps -0 to +0.
//
// This translation unit is compiled with -ffp-contract=off (no FMA
// contraction) and without fast-math: '/' is IEEE correctly rounded, expf is
// the device library's accurate exp, and float32 denormals are preserved.
//
// Both kernels are HBM-bound streams: a persistent grid walks 16-byte chunks
// (8 bf16) of the valid rows with 128-bit loads and stores, two chunks per
// thread per iteration to keep more bytes in flight.
#include "rd_device.h"
#include "rd_launch.h"

#pragma clang fp contract(off)

namespace rd {
namespace {

__device__ __forceinline__ int clamp_limit(const int32_t* limp, int rows) {
  if (limp == nullptr) return rows;
  const int v = *limp;
  return v < 0 ? 0 : (v > rows ? rows : v);
}

__device__ __forceinline__ float lo16(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float hi16(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }

// silu(g) * u in the page's op order: negate, exp, + 1, divide, multiply.
__device__ __forceinline__ float glu_f32(float g, float u) {
  const float e = expf(-g);
  const float den = e + 1.0f;
  const float s = g / den;
  return s * u;
}

__device__ __forceinline__ uint32_t glu_word(uint32_t gw, uint32_t uw) {
  return pack_bf16x2(glu_f32(lo16(gw), lo16(uw)), glu_f32(hi16(gw), hi16(uw)));
}

__device__ __forceinline__ uint4 glu_chunk(uint4 g, uint4 u) {
  return make_uint4(glu_word(g.x, u.x), glu_word(g.y, u.y), glu_word(g.z, u.z), glu_word(g.w, u.w));
}

// -0 (0x8000) becomes +0 in each bf16 half of a word.
__device__ __forceinline__ uint32_t no_negzero(uint32_t w) {
  const uint32_t lo = (w & 0xFFFFu) == 0x8000u ? 0u : (w & 0xFFFFu);
  const uint32_t hi = (w >> 16) == 0x8000u ? 0u : (w & 0xFFFF0000u);
  return lo | hi;
}

// Backward of one element: d_gate and d_up as float32, in a fixed op order.
__device__ __forceinline__ void glu_grad_f32(float g, float u, float d, float& d_gate, float& d_up) {
  const float e = expf(-g);
  const float den = e + 1.0f;
  const float sig = 1.0f / den;
  const float silu = g / den;
  d_up = d * silu;
  d_gate = ((d * u) * sig) * (1.0f + g * (1.0f - sig));
}

__device__ __forceinline__ void glu_grad_word(uint32_t gw, uint32_t uw, uint32_t dw, uint32_t& ogw, uint32_t& ouw) {
  float g0, u0, g1, u1;
  glu_grad_f32(lo16(gw), lo16(uw), lo16(dw), g0, u0);
  glu_grad_f32(hi16(gw), hi16(uw), hi16(dw), g1, u1);
  ogw = no_negzero(pack_bf16x2(g0, g1));
  ouw = no_negzero(pack_bf16x2(u0, u1));
}

__global__ __launch_bounds__(kThreads) void glu_fwd_kernel(const uint16_t* __restrict__ fused,
                                                           const int32_t* __restrict__ limp,
                                                           uint16_t* __restrict__ out, int rows, int h) {
  const int L = clamp_limit(limp, rows);
  const int hc = h >> 3;  // 16-byte chunks per output row
  const long long total = static_cast<long long>(L) * hc;
  const long long stride = static_cast<long long>(gridDim.x) * kThreads;
  long long q = static_cast<long long>(blockIdx.x) * kThreads + threadIdx.x;
  for (; q + stride < total; q += 2 * stride) {
    const long long q1 = q + stride;
    const int r0 = static_cast<int>(q / hc), c0 = static_cast<int>(q - static_cast<long long>(r0) * hc);
    const int r1 = static_cast<int>(q1 / hc), c1 = static_cast<int>(q1 - static_cast<long long>(r1) * hc);
    const uint16_t* f0 = fused + static_cast<long long>(r0) * 2 * h + c0 * 8;
    const uint16_t* f1 = fused + static_cast<long long>(r1) * 2 * h + c1 * 8;
    const uint4 g0 = *reinterpret_cast<const uint4*>(f0);
    const uint4 u0 = *reinterpret_cast<const uint4*>(f0 + h);
    const uint4 g1 = *reinterpret_cast<const uint4*>(f1);
    const uint4 u1 = *reinterpret_cast<const uint4*>(f1 + h);
    *reinterpret_cast<uint4*>(out + static_cast<long long>(r0) * h + c0 * 8) = glu_chunk(g0, u0);
    *reinterpret_cast<uint4*>(out + static_cast<long long>(r1) * h + c1 * 8) = glu_chunk(g1, u1);
  }
  if (q < total) {
    const int r0 = static_cast<int>(q / hc), c0 = static_cast<int>(q - static_cast<long long>(r0) * hc);
    const uint16_t* f0 = fused + static_cast<long long>(r0) * 2 * h + c0 * 8;
    const uint4 g0 = *reinterpret_cast<const uint4*>(f0);
    const uint4 u0 = *reinterpret_cast<const uint4*>(f0 + h);
    *reinterpret_cast<uint4*>(out + static_cast<long long>(r0) * h + c0 * 8) = glu_chunk(g0, u0);
  }
}

__device__ __forceinline__ void glu_bwd_one(const uint16_t* __restrict__ fused, const uint16_t* __restrict__ d_out,
                                            uint16_t* __restrict__ d_fused, long long q, int hc, int h) {
  const int r = static_cast<int>(q / hc), c = static_cast<int>(q - static_cast<long long>(r) * hc);
  const long long frow = static_cast<long long>(r) * 2 * h + c * 8;
  const uint4 g = *reinterpret_cast<const uint4*>(fused + frow);
  const uint4 u = *reinterpret_cast<const uint4*>(fused + frow + h);
  const uint4 d = *reinterpret_cast<const uint4*>(d_out + static_cast<long long>(r) * h + c * 8);
  uint4 og, ou;
  glu_grad_word(g.x, u.x, d.x, og.x, ou.x);
  glu_grad_word(g.y, u.y, d.y, og.y, ou.y);
  glu_grad_word(g.z, u.z, d.z, og.z, ou.z);
  glu_grad_word(g.w, u.w, d.w, og.w, ou.w);
  *reinterpret_cast<uint4*>(d_fused + frow) = og;
  *reinterpret_cast<uint4*>(d_fused + frow + h) = ou;
}

__global__ __launch_bounds__(kThreads) void glu_bwd_kernel(const uint16_t* __restrict__ fused,
                                                           const uint16_t* __restrict__ d_out,
                                                           const int32_t* __restrict__ limp,
                                                           uint16_t* __restrict__ d_fused, int rows, int h) {
  const int L = clamp_limit(limp, rows);
  const int hc = h >> 3;
  const long long total = static_cast<long long>(L) * hc;
  const long long stride = static_cast<long long>(gridDim.x) * kThreads;
  for (long long q = static_cast<long long>(blockIdx.x) * kThreads + threadIdx.x; q < total; q += stride)
    glu_bwd_one(fused, d_out, d_fused, q, hc, h);
}

int elementwise_grid(int rows, int h) {
  const long long chunks = static_cast<long long>(rows) * (h / 8);
  const long long blocks = (chunks + kThreads - 1) / kThreads;
  const long long cap = static_cast<long long>(device_cu_count()) * 8;
  const long long g = blocks < cap ? blocks : cap;
  return static_cast<int>(g < 1 ? 1 : g);
}

}  // namespace

int launch_glu_fwd(const void* fused, const int32_t* limit, void* out, int rows, int h, hipStream_t stream) {
  glu_fwd_kernel<<<elementwise_grid(rows, h), kThreads, 0, stream>>>(static_cast<const uint16_t*>(fused), limit,
                                                                       static_cast<uint16_t*>(out), rows, h);
  return hipGetLastError() == hipSuccess ? RD_OK : RD_EHIP;
}

int launch_glu_bwd(const void* fused, const void* d_out, const int32_t* limit, void* d_fused, int rows, int h,
                   hipStream_t stream) {
  glu_bwd_kernel<<<elementwise_grid(rows, h), kThreads, 0, stream>>>(
      static_cast<const uint16_t*>(fused), static_cast<const uint16_t*>(d_out), limit,
      static_cast<uint16_t*>(d_fused), rows, h);
  return hipGetLastError() == hipSuccess ? RD_OK : RD_EHIP;
}

}  // namespace rd
