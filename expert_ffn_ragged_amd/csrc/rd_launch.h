// Internal launch interface between the C-ABI layer (rd_api.cpp) and the
// kernel translation units.  Not part of the public ABI.
#pragma once

#include <hip/hip_runtime_api.h>
#include <stdint.h>

namespace rd {

// One grouped-GEMM call as the host sees it.  Device-resident values
// (group sizes, offset, limit) stay behind their pointers.
struct GemmProblem {
  const void* a;             // forward: x [m,k]; trans: x [m,k]
  const void* b;             // forward: w [gl,k,n] or [gl,n,k]; trans: dy [m,n]
  const int32_t* group_sizes;
  int32_t num_groups;
  const int32_t* group_offset;  // may be null
  int32_t num_local;
  const int32_t* limit;          // may be null
  void* out;                 // forward: [m,n]; trans: [gl,k,n]; fused GLU: silu(gate) * up [m,n]
  bool out_f32;
  int m, k, n;                // fused GLU: n = h, the weight is [gl,k,2h]
  void* out2 = nullptr;       // fused GLU only: the [gate | up] buffer [m,2h], or null
};

// Workspace plan of the split-contraction decode path (use == false: the
// forward needs no workspace).
struct DecodePlan {
  bool use;
  int nb, grid, seg_max;
  size_t ws_bytes;
};
DecodePlan plan_decode(const GemmProblem& p, bool trans_rhs);

// workspace may be null; the decode path runs only with ws_bytes of it.
int launch_forward(const GemmProblem& p, bool trans_rhs, void* workspace, size_t workspace_bytes,
                   hipStream_t stream);
// trans_ragged_dot; with a workspace, groups long enough to hold up the grid
// are split over rows (fp32 partials, then a fixed-order reduction kernel).
int launch_trans(const GemmProblem& p, void* workspace, size_t workspace_bytes, hipStream_t stream);
// Workspace bytes that let launch_trans split every group that qualifies (0: it never splits).
size_t trans_workspace_size(const GemmProblem& p);
// launch_forward (plain form) with the decode path's partial sums in the library's static device
// scratch (RD_NOALLOC_SCRATCH_BYTES); RD_ESCRATCH when the sizes need more.
int launch_forward_noalloc(const GemmProblem& p, hipStream_t stream);
// fp8 (OCP E4M3) x [m, k] and w [g, n, k] (trans_rhs) or [g, k, n]; requires k % 128 == 0,
// n % 16 == 0 and k * max(m, n) < 2^32.
int launch_forward_fp8(const GemmProblem& p, bool trans_rhs, hipStream_t stream);
// fp8 x [m, k] and dy [m, n]; requires k % 16 == 0, n % 16 == 0, m * max(k, n) < 2^32.
int launch_trans_fp8(const GemmProblem& p, void* workspace, size_t workspace_bytes, hipStream_t stream);
// ragged_dot(x, w) with the GLU as its epilogue; requires k % 64 == 0, n (= h) % 128 == 0 and
// operands under 4 GiB (fused_glu_supported).
bool fused_glu_supported(const GemmProblem& p);
int launch_forward_glu(const GemmProblem& p, hipStream_t stream);
int launch_glu_fwd(const void* fused, const int32_t* limit, void* out, int rows, int h, hipStream_t stream);
int launch_glu_bwd(const void* fused, const void* d_out, const int32_t* limit, void* d_fused, int rows, int h,
                   hipStream_t stream);

int launch_unsort_bwd_rows(const void* g, const void* y, const float* w, const int32_t* limit, void* grad,
                           float* dot, int rows, int hidden, hipStream_t stream);

// Rows [clamp(*limit, 0, rows), rows) of a [rows, row_bytes] buffer set to zero (row_bytes % 16 == 0).
int launch_zero_rows(void* buf, const int32_t* limit, long long rows, long long row_bytes, hipStream_t stream);

// Number of compute units of the current device (cached per device, thread-safe).
int device_cu_count();

// Tuning overrides (rd_tune_set) and the number of grouped-GEMM tile shapes.
int tune_set(int which, int value);
int tile_count();

}  // namespace rd
