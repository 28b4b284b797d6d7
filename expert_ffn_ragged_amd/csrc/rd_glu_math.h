// silu(gate) * up in float32, shared by the standalone GLU kernels and the
// GLU epilogue of the fused up-projection GEMM, so both give the same bits.
//
// MaxText PR #5760 ("397B v7x trainer: MoE wo FSDP sharding and
// valid-rows-only MoE kernels"), commit on valid rows: the forward evaluates
// negate, exp, + 1, divide, multiply in float32 and rounds only the output.
// exp(-g) is the hardware base-2 exponential of -g * log2(e), and a divide by
// den = 1 + exp(-g) is a multiply by the hardware reciprocal; when den > 2^64
// the reciprocal is taken of den * 2^-64 and the product scaled back by
// 2^-64, so the reciprocal stays in the normal range where the hardware keeps
// its accuracy and a denormal result is rounded once, by the final scaling.
// Within about 2^-16 relative of the exact value (far inside a bf16 half-ulp).
// No operation here may be fused into an FMA: every function body turns
// contraction off.
#pragma once

#include <hip/hip_runtime.h>

namespace rd {

constexpr float kLog2e = 1.44269504088896341f;
constexpr float kTwoM64 = 5.42101086242752217e-20f;  // 2^-64
constexpr float kTwo64 = 1.8446744073709551616e19f;  // 2^64

// den = 1 + exp(-g); x / den as (x * rcp(den * sc)) * sc with sc = 2^-64
// when den > 2^64 (then g < -44, so x * rcp stays finite) and sc = 1 otherwise.
struct ScaledRcp {
  float r, sc;
};
__device__ __forceinline__ ScaledRcp rcp_den(float g) {
#pragma clang fp contract(off)
  const float den = __builtin_amdgcn_exp2f(-g * kLog2e) + 1.0f;
  const float sc = den > kTwo64 ? kTwoM64 : 1.0f;
  return ScaledRcp{__builtin_amdgcn_rcpf(den * sc), sc};
}
__device__ __forceinline__ float div_den(float x, const ScaledRcp& q) {
#pragma clang fp contract(off)
  return (x * q.r) * q.sc;
}

// silu(g) * u in the page's op order: negate, exp, + 1, divide, multiply.
__device__ __forceinline__ float glu_f32(float g, float u) {
#pragma clang fp contract(off)
  const float s = div_den(g, rcp_den(g));
  return s * u;
}

}  // namespace rd
