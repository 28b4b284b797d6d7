// Limit-aware silu(gate) * up GLU, forward and backward, for gfx950.
//
// MaxText PR #5760 ("397B v7x trainer: MoE wo FSDP sharding and
// valid-rows-only MoE kernels"), commit on valid rows: only rows [0, limit)
// of the packed expert buffer are read or written; gate and up are read in
// place from the fused [gate | up] buffer; the forward evaluates negate, exp,
// + 1, divide, multiply in float32 and rounds only the output; the backward
// writes [d_gate | d_up] in one pass and maps -0 to +0.
//
// Arithmetic: float32, in the page's op order, compiled with
// -ffp-contract=off (no FMA contraction) and without fast-math, denormals
// kept.  exp(-g) is the hardware base-2 exponential of -g * log2(e), and a
// divide by den = 1 + exp(-g) is a multiply by the hardware reciprocal; when
// den > 2^64 the reciprocal is taken of den * 2^-64 and the product scaled
// back by 2^-64, so the reciprocal stays in the normal range where the
// hardware keeps its accuracy (den reaches 2^128 or inf) and a denormal
// result is rounded once, by the final scaling.  The error is within about
// 2^-16 relative of the exact value (the rounding of -g * log2(e) dominates,
// |g| <= 89), far inside the 2^-9 of a bf16 half-ulp, so every output is
// within one bf16 ulp of the correctly rounded float32 evaluation.  Special values follow the op
// sequence: g = -inf gives NaN, exp overflow gives -0, g = +inf gives inf.
//
// Both kernels are HBM-bound streams: a persistent grid of waves walks the
// valid rows, one wave per row, with 128-bit non-temporal loads and stores of
// 16-byte chunks (8 bf16; the data is touched once).
#include "rd_device.h"
#include "rd_glu_math.h"
#include "rd_launch.h"

#pragma clang fp contract(off)

namespace rd {
namespace {

__device__ __forceinline__ int clamp_limit(const int32_t* limp, int rows) {
  if (limp == nullptr) return rows;
  const int v = *limp;
  return v < 0 ? 0 : (v > rows ? rows : v);
}

typedef unsigned int nt_u32x4 __attribute__((ext_vector_type(4)));

// 128-bit loads and stores marked non-temporal (streamed once, not kept in cache).
__device__ __forceinline__ uint4 nt_load(const uint16_t* p) {
  const nt_u32x4 v = __builtin_nontemporal_load(reinterpret_cast<const nt_u32x4*>(p));
  return make_uint4(v.x, v.y, v.z, v.w);
}
__device__ __forceinline__ void nt_store(uint16_t* p, uint4 v) {
  const nt_u32x4 x = {v.x, v.y, v.z, v.w};
  __builtin_nontemporal_store(x, reinterpret_cast<nt_u32x4*>(p));
}

__device__ __forceinline__ float lo16(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float hi16(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }

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
  const ScaledRcp q = rcp_den(g);
  const float sig = div_den(1.0f, q);
  const float silu = div_den(g, q);
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

// One wave per row: lane l takes the row's 16-byte chunks l, l + 64, ...
// (two per iteration); rows are strided over all waves of the grid.  No
// division per chunk.
__global__ __launch_bounds__(kThreads) void glu_fwd_kernel(const uint16_t* __restrict__ fused,
                                                           const int32_t* __restrict__ limp,
                                                           uint16_t* __restrict__ out, int rows, int h) {
  const int L = clamp_limit(limp, rows);
  const int hc = h >> 3;  // 16-byte chunks per output row
  const int lane = threadIdx.x & 63;
  const int waves = gridDim.x * (kThreads / 64);
  for (int r = blockIdx.x * (kThreads / 64) + (threadIdx.x >> 6); r < L; r += waves) {
    const uint16_t* f = fused + static_cast<long long>(r) * 2 * h;
    uint16_t* o = out + static_cast<long long>(r) * h;
    int c = lane;
    for (; c + 64 < hc; c += 128) {
      const uint4 g0 = nt_load(f + c * 8);
      const uint4 u0 = nt_load(f + h + c * 8);
      const uint4 g1 = nt_load(f + (c + 64) * 8);
      const uint4 u1 = nt_load(f + h + (c + 64) * 8);
      nt_store(o + c * 8, glu_chunk(g0, u0));
      nt_store(o + (c + 64) * 8, glu_chunk(g1, u1));
    }
    if (c < hc) nt_store(o + c * 8, glu_chunk(nt_load(f + c * 8), nt_load(f + h + c * 8)));
  }
}

__device__ __forceinline__ void glu_bwd_chunk(const uint16_t* __restrict__ f, const uint16_t* __restrict__ d,
                                              uint16_t* __restrict__ df, int c, int h) {
  const uint4 g = nt_load(f + c * 8);
  const uint4 u = nt_load(f + h + c * 8);
  const uint4 dv = nt_load(d + c * 8);
  uint4 og, ou;
  glu_grad_word(g.x, u.x, dv.x, og.x, ou.x);
  glu_grad_word(g.y, u.y, dv.y, og.y, ou.y);
  glu_grad_word(g.z, u.z, dv.z, og.z, ou.z);
  glu_grad_word(g.w, u.w, dv.w, og.w, ou.w);
  nt_store(df + c * 8, og);
  nt_store(df + h + c * 8, ou);
}

__global__ __launch_bounds__(kThreads) void glu_bwd_kernel(const uint16_t* __restrict__ fused,
                                                           const uint16_t* __restrict__ d_out,
                                                           const int32_t* __restrict__ limp,
                                                           uint16_t* __restrict__ d_fused, int rows, int h) {
  const int L = clamp_limit(limp, rows);
  const int hc = h >> 3;
  const int lane = threadIdx.x & 63;
  const int waves = gridDim.x * (kThreads / 64);
  for (int r = blockIdx.x * (kThreads / 64) + (threadIdx.x >> 6); r < L; r += waves) {
    const long long fo = static_cast<long long>(r) * 2 * h;
    const uint16_t* d = d_out + static_cast<long long>(r) * h;
    for (int c = lane; c < hc; c += 64) glu_bwd_chunk(fused + fo, d, d_fused + fo, c, h);
  }
}

// A wave per row, at most per_cu workgroups per CU.
int elementwise_grid(int rows, int h, int per_cu) {
  (void)h;
  const long long blocks = (static_cast<long long>(rows) + kThreads / 64 - 1) / (kThreads / 64);
  const long long cap = static_cast<long long>(device_cu_count()) * per_cu;
  const long long g = blocks < cap ? blocks : cap;
  return static_cast<int>(g < 1 ? 1 : g);
}

}  // namespace

int launch_glu_fwd(const void* fused, const int32_t* limit, void* out, int rows, int h, hipStream_t stream) {
  glu_fwd_kernel<<<elementwise_grid(rows, h, 32), kThreads, 0, stream>>>(static_cast<const uint16_t*>(fused), limit,
                                                                       static_cast<uint16_t*>(out), rows, h);
  return hipGetLastError() == hipSuccess ? RD_OK : RD_EHIP;
}

int launch_glu_bwd(const void* fused, const void* d_out, const int32_t* limit, void* d_fused, int rows, int h,
                   hipStream_t stream) {
  glu_bwd_kernel<<<elementwise_grid(rows, h, 32), kThreads, 0, stream>>>(
      static_cast<const uint16_t*>(fused), static_cast<const uint16_t*>(d_out), limit,
      static_cast<uint16_t*>(d_fused), rows, h);
  return hipGetLastError() == hipSuccess ? RD_OK : RD_EHIP;
}

}  // namespace rd
