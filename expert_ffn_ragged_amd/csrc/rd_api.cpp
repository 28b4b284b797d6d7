// C ABI of librd.so (declared in include/rd.h): host-side validation and
// dispatch.  Everything that depends on device-resident values (group sizes,
// offset, limit) is decided inside the kernels; this file only checks what
// the host can see and sizes the persistent grids.
#include "rd.h"

#include <hip/hip_runtime_api.h>

#include "rd_launch.h"

namespace {

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

int check_groups(int32_t num_groups, const int32_t* group_offset, int32_t num_local) {
  if (num_groups < 1 || num_local < 1) return RD_EINVAL;
  if (num_groups > RD_MAX_GROUPS || num_local > RD_MAX_GROUPS) return RD_EUNSUPPORTED;
  if (num_local > num_groups) return RD_EINVAL;
  if (group_offset == nullptr && num_local != num_groups) return RD_EINVAL;
  if (group_offset != nullptr && (reinterpret_cast<uintptr_t>(group_offset) & 3u)) return RD_EINVAL;
  return RD_OK;
}

int check_dims(int64_t m, int64_t k, int64_t n) {
  if (m < 0 || k <= 0 || n <= 0) return RD_EINVAL;
  if (m >= (int64_t(1) << 31) || k >= (int64_t(1) << 31) || n >= (int64_t(1) << 31)) return RD_EUNSUPPORTED;
  if ((k % 8) != 0 || (n % 8) != 0) return RD_EUNSUPPORTED;
  return RD_OK;
}

int forward_common(const void* x, const void* w, const int32_t* group_sizes, int32_t num_groups,
                   const int32_t* group_offset, int32_t num_local, const int32_t* limit, void* out,
                   int32_t out_dtype, int64_t m, int64_t k, int64_t n, void* workspace, size_t workspace_bytes,
                   void* stream, bool trans_rhs, bool noalloc = false) {
  int st = check_dims(m, k, n);
  if (st != RD_OK) return st;
  st = check_groups(num_groups, group_offset, num_local);
  if (st != RD_OK) return st;
  if (out_dtype != RD_BF16 && out_dtype != RD_F32) return RD_EINVAL;
  if (!w || !group_sizes) return RD_EINVAL;
  if (m == 0) return RD_OK;  // no rows: x and out may be empty (null)
  if (!x || !out) return RD_EINVAL;
  if (!aligned16(x) || !aligned16(w) || !aligned16(out) || !aligned16(workspace)) return RD_EINVAL;
  if ((reinterpret_cast<uintptr_t>(group_sizes) & 3u) || (reinterpret_cast<uintptr_t>(limit) & 3u))
    return RD_EINVAL;
  rd::GemmProblem p{};
  p.a = x;
  p.b = w;
  p.group_sizes = group_sizes;
  p.num_groups = num_groups;
  p.group_offset = group_offset;
  p.num_local = num_local;
  p.limit = limit;
  p.out = out;
  p.out_f32 = out_dtype == RD_F32;
  p.m = static_cast<int>(m);
  p.k = static_cast<int>(k);
  p.n = static_cast<int>(n);
  if (noalloc) return rd::launch_forward_noalloc(p, static_cast<hipStream_t>(stream));
  return rd::launch_forward(p, trans_rhs, workspace, workspace_bytes, static_cast<hipStream_t>(stream));
}

// The GemmProblem of a forward call of these sizes (pointers unset).
rd::GemmProblem shape_only(int64_t m, int64_t k, int64_t n, int32_t num_local) {
  rd::GemmProblem p{};
  p.num_groups = num_local;
  p.num_local = num_local;
  p.m = static_cast<int>(m);
  p.k = static_cast<int>(k);
  p.n = static_cast<int>(n);
  return p;
}

}  // namespace

extern "C" {

int rd_abi_version(void) { return RD_ABI_VERSION; }

const char* rd_status_string(int status) {
  switch (status) {
    case RD_OK: return "ok";
    case RD_EINVAL: return "invalid argument (null or misaligned pointer, bad size or dtype)";
    case RD_EUNSUPPORTED: return "unsupported size (k, n, h, hidden must be multiples of 8; dims < 2^31; groups <= RD_MAX_GROUPS)";
    case RD_EHIP: return "HIP runtime error while launching";
    case RD_ESCRATCH: return "the call needs more device scratch than rd_forward_noalloc holds (RD_NOALLOC_SCRATCH_BYTES)";
    default: return "unknown status";
  }
}

size_t rd_forward_workspace_size(int64_t m, int64_t k, int64_t n, int32_t num_local, int32_t trans_rhs) {
  if (check_dims(m, k, n) != RD_OK || num_local < 1 || num_local > RD_MAX_GROUPS) return 0;
  const rd::DecodePlan d = rd::plan_decode(shape_only(m, k, n, num_local), trans_rhs != 0);
  return d.use ? d.ws_bytes : 0;
}

int rd_forward(const void* x, const void* w, const int32_t* group_sizes, int32_t num_groups,
               const int32_t* group_offset, int32_t num_local, const int32_t* limit, void* out,
               int32_t out_dtype, int64_t m, int64_t k, int64_t n, void* workspace, size_t workspace_bytes,
               void* stream) {
  return forward_common(x, w, group_sizes, num_groups, group_offset, num_local, limit, out, out_dtype, m,
                        k, n, workspace, workspace_bytes, stream, false);
}

int rd_forward_noalloc(const void* x, const void* w, const int32_t* group_sizes, int32_t num_groups,
                       const int32_t* group_offset, int32_t num_local, const int32_t* limit, void* out,
                       int32_t out_dtype, int64_t m, int64_t k, int64_t n, void* stream) {
  return forward_common(x, w, group_sizes, num_groups, group_offset, num_local, limit, out, out_dtype, m, k, n,
                        nullptr, 0, stream, false, true);
}

int rd_forward_trans_rhs(const void* x, const void* w, const int32_t* group_sizes,
                         int32_t num_groups, const int32_t* group_offset, int32_t num_local,
                         const int32_t* limit, void* out, int32_t out_dtype, int64_t m, int64_t k,
                         int64_t n, void* workspace, size_t workspace_bytes, void* stream) {
  return forward_common(x, w, group_sizes, num_groups, group_offset, num_local, limit, out, out_dtype, m,
                        k, n, workspace, workspace_bytes, stream, true);
}

int rd_forward_glu(const void* x, const void* wi, const int32_t* group_sizes, int32_t num_groups,
                   const int32_t* group_offset, int32_t num_local, const int32_t* limit, void* act,
                   void* fused, int64_t m, int64_t k, int64_t h, void* stream) {
  if (h <= 0) return RD_EINVAL;
  if (h >= (int64_t(1) << 30)) return RD_EUNSUPPORTED;  // the weight's width 2h stays below 2^31
  int st = check_dims(m, k, 2 * h);
  if (st != RD_OK) return st;
  st = check_groups(num_groups, group_offset, num_local);
  if (st != RD_OK) return st;
  if (!wi || !group_sizes) return RD_EINVAL;
  if (m == 0) return RD_OK;  // no rows: x, act and fused may be empty (null)
  if (!x || !act) return RD_EINVAL;
  if (!aligned16(x) || !aligned16(wi) || !aligned16(act) || (fused && !aligned16(fused))) return RD_EINVAL;
  if ((reinterpret_cast<uintptr_t>(group_sizes) & 3u) || (reinterpret_cast<uintptr_t>(limit) & 3u) ||
      (reinterpret_cast<uintptr_t>(group_offset) & 3u))
    return RD_EINVAL;
  rd::GemmProblem p{};
  p.a = x;
  p.b = wi;
  p.group_sizes = group_sizes;
  p.num_groups = num_groups;
  p.group_offset = group_offset;
  p.num_local = num_local;
  p.limit = limit;
  p.out = act;
  p.out2 = fused;
  p.out_f32 = false;
  p.m = static_cast<int>(m);
  p.k = static_cast<int>(k);
  p.n = static_cast<int>(h);
  if (!rd::fused_glu_supported(p)) return RD_EUNSUPPORTED;
  return rd::launch_forward_glu(p, static_cast<hipStream_t>(stream));
}

namespace {
int forward_fp8(const void* x, const void* w, const int32_t* group_sizes, int32_t num_groups,
                const int32_t* group_offset, int32_t num_local, const int32_t* limit, void* out, int32_t out_dtype,
                int64_t m, int64_t k, int64_t n, void* stream, bool trans_rhs) {
  int st = check_dims(m, k, n);
  if (st != RD_OK) return st;
  if ((k % 128) != 0 || (!trans_rhs && (n % 16) != 0)) return RD_EUNSUPPORTED;
  if (k * (m > n ? m : n) >= (int64_t(1) << 32)) return RD_EUNSUPPORTED;
  st = check_groups(num_groups, group_offset, num_local);
  if (st != RD_OK) return st;
  if (out_dtype != RD_BF16 && out_dtype != RD_F32) return RD_EINVAL;
  if (!w || !group_sizes) return RD_EINVAL;
  if (m == 0) return RD_OK;  // no rows: x and out may be empty (null)
  if (!x || !out) return RD_EINVAL;
  if (!aligned16(x) || !aligned16(w) || !aligned16(out)) return RD_EINVAL;
  if ((reinterpret_cast<uintptr_t>(group_sizes) & 3u) || (reinterpret_cast<uintptr_t>(limit) & 3u) ||
      (reinterpret_cast<uintptr_t>(group_offset) & 3u))
    return RD_EINVAL;
  rd::GemmProblem p{};
  p.a = x;
  p.b = w;
  p.group_sizes = group_sizes;
  p.num_groups = num_groups;
  p.group_offset = group_offset;
  p.num_local = num_local;
  p.limit = limit;
  p.out = out;
  p.out_f32 = out_dtype == RD_F32;
  p.m = static_cast<int>(m);
  p.k = static_cast<int>(k);
  p.n = static_cast<int>(n);
  return rd::launch_forward_fp8(p, trans_rhs, static_cast<hipStream_t>(stream));
}
}  // namespace

int rd_forward_fp8(const void* x, const void* w, const int32_t* group_sizes, int32_t num_groups,
                   const int32_t* group_offset, int32_t num_local, const int32_t* limit, void* out,
                   int32_t out_dtype, int64_t m, int64_t k, int64_t n, void* stream) {
  return forward_fp8(x, w, group_sizes, num_groups, group_offset, num_local, limit, out, out_dtype, m, k, n, stream,
                     false);
}

int rd_forward_trans_rhs_fp8(const void* x, const void* w, const int32_t* group_sizes, int32_t num_groups,
                             const int32_t* group_offset, int32_t num_local, const int32_t* limit, void* out,
                             int32_t out_dtype, int64_t m, int64_t k, int64_t n, void* stream) {
  return forward_fp8(x, w, group_sizes, num_groups, group_offset, num_local, limit, out, out_dtype, m, k, n, stream,
                     true);
}

size_t rd_trans_workspace_size(int64_t m, int64_t k, int64_t n, int32_t num_local) {
  if (check_dims(m, k, n) != RD_OK || num_local <= 0 || num_local > RD_MAX_GROUPS || m == 0) return 0;
  rd::GemmProblem p{};
  p.num_local = num_local;
  p.m = static_cast<int>(m);
  p.k = static_cast<int>(k);
  p.n = static_cast<int>(n);
  return rd::trans_workspace_size(p);
}

int rd_trans_fp8(const void* x, const void* dy, const int32_t* group_sizes, int32_t num_groups,
                 const int32_t* group_offset, int32_t num_local, const int32_t* limit, void* dw,
                 int32_t dw_dtype, int64_t m, int64_t k, int64_t n, void* workspace, size_t workspace_bytes,
                 void* stream) {
  int st = check_dims(m, k, n);
  if (st != RD_OK) return st;
  if ((k % 16) != 0 || (n % 16) != 0) return RD_EUNSUPPORTED;
  if (m * (k > n ? k : n) >= (int64_t(1) << 32)) return RD_EUNSUPPORTED;
  st = check_groups(num_groups, group_offset, num_local);
  if (st != RD_OK) return st;
  if (dw_dtype != RD_BF16 && dw_dtype != RD_F32) return RD_EINVAL;
  if (!group_sizes || !dw) return RD_EINVAL;
  if (m > 0 && (!x || !dy)) return RD_EINVAL;  // no rows: x and dy may be empty (null)
  if ((m > 0 && (!aligned16(x) || !aligned16(dy))) || !aligned16(dw)) return RD_EINVAL;
  if ((reinterpret_cast<uintptr_t>(group_sizes) & 3u) || (reinterpret_cast<uintptr_t>(limit) & 3u) ||
      (reinterpret_cast<uintptr_t>(group_offset) & 3u))
    return RD_EINVAL;
  if (workspace_bytes > 0 && (workspace == nullptr || !aligned16(workspace))) return RD_EINVAL;
  rd::GemmProblem p{};
  p.a = x;
  p.b = dy;
  p.group_sizes = group_sizes;
  p.num_groups = num_groups;
  p.group_offset = group_offset;
  p.num_local = num_local;
  p.limit = limit;
  p.out = dw;
  p.out_f32 = dw_dtype == RD_F32;
  p.m = static_cast<int>(m);
  p.k = static_cast<int>(k);
  p.n = static_cast<int>(n);
  return rd::launch_trans_fp8(p, workspace_bytes > 0 ? workspace : nullptr, workspace_bytes,
                              static_cast<hipStream_t>(stream));
}

int rd_trans(const void* x, const void* dy, const int32_t* group_sizes, int32_t num_groups,
             const int32_t* group_offset, int32_t num_local, const int32_t* limit, void* dw,
             int32_t dw_dtype, int64_t m, int64_t k, int64_t n, void* workspace,
             size_t workspace_bytes, void* stream) {
  int st = check_dims(m, k, n);
  if (st != RD_OK) return st;
  st = check_groups(num_groups, group_offset, num_local);
  if (st != RD_OK) return st;
  if (dw_dtype != RD_BF16 && dw_dtype != RD_F32) return RD_EINVAL;
  if (!group_sizes || !dw) return RD_EINVAL;
  if (m > 0 && (!x || !dy)) return RD_EINVAL;  // no rows: x and dy may be empty (null)
  if ((m > 0 && (!aligned16(x) || !aligned16(dy))) || !aligned16(dw)) return RD_EINVAL;
  if ((reinterpret_cast<uintptr_t>(group_sizes) & 3u) || (reinterpret_cast<uintptr_t>(limit) & 3u))
    return RD_EINVAL;
  if (workspace_bytes > 0 && (workspace == nullptr || !aligned16(workspace))) return RD_EINVAL;
  rd::GemmProblem p{};
  p.a = x;
  p.b = dy;
  p.group_sizes = group_sizes;
  p.num_groups = num_groups;
  p.group_offset = group_offset;
  p.num_local = num_local;
  p.limit = limit;
  p.out = dw;
  p.out_f32 = dw_dtype == RD_F32;
  p.m = static_cast<int>(m);
  p.k = static_cast<int>(k);
  p.n = static_cast<int>(n);
  return rd::launch_trans(p, workspace_bytes > 0 ? workspace : nullptr, workspace_bytes,
                          static_cast<hipStream_t>(stream));
}

int rd_glu_fwd(const void* fused, const int32_t* limit, void* out, int64_t rows, int64_t h,
               void* stream) {
  if (rows < 0 || h <= 0) return RD_EINVAL;
  if ((h % 8) != 0) return RD_EUNSUPPORTED;
  if (rows >= (int64_t(1) << 31) || h >= (int64_t(1) << 30)) return RD_EUNSUPPORTED;
  if (rows == 0) return RD_OK;  // no rows: the buffers may be empty (null)
  if (!fused || !out) return RD_EINVAL;
  if (!aligned16(fused) || !aligned16(out) || (reinterpret_cast<uintptr_t>(limit) & 3u)) return RD_EINVAL;
  return rd::launch_glu_fwd(fused, limit, out, static_cast<int>(rows), static_cast<int>(h),
                            static_cast<hipStream_t>(stream));
}

int rd_glu_bwd(const void* fused, const void* d_out, const int32_t* limit, void* d_fused,
               int64_t rows, int64_t h, void* stream) {
  if (rows < 0 || h <= 0) return RD_EINVAL;
  if ((h % 8) != 0) return RD_EUNSUPPORTED;
  if (rows >= (int64_t(1) << 31) || h >= (int64_t(1) << 30)) return RD_EUNSUPPORTED;
  if (rows == 0) return RD_OK;  // no rows: the buffers may be empty (null)
  if (!fused || !d_out || !d_fused) return RD_EINVAL;
  if (!aligned16(fused) || !aligned16(d_out) || !aligned16(d_fused) ||
      (reinterpret_cast<uintptr_t>(limit) & 3u))
    return RD_EINVAL;
  return rd::launch_glu_bwd(fused, d_out, limit, d_fused, static_cast<int>(rows), static_cast<int>(h),
                            static_cast<hipStream_t>(stream));
}

int rd_unsort_bwd_rows(const void* g, const void* y, const float* w, const int32_t* limit, void* grad, float* dot,
                       int64_t rows, int64_t hidden, void* stream) {
  if (rows < 0 || hidden <= 0) return RD_EINVAL;
  if ((hidden % 8) != 0) return RD_EUNSUPPORTED;
  if (rows >= (int64_t(1) << 31) || hidden >= (int64_t(1) << 30)) return RD_EUNSUPPORTED;
  if (rows == 0) return RD_OK;  // no rows: the buffers may be empty (null)
  if (!g || !y || !w || !grad || !dot) return RD_EINVAL;
  if (!aligned16(g) || !aligned16(y) || !aligned16(grad) || (reinterpret_cast<uintptr_t>(w) & 3u) ||
      (reinterpret_cast<uintptr_t>(dot) & 3u) || (reinterpret_cast<uintptr_t>(limit) & 3u))
    return RD_EINVAL;
  return rd::launch_unsort_bwd_rows(g, y, w, limit, grad, dot, static_cast<int>(rows), static_cast<int>(hidden),
                                    static_cast<hipStream_t>(stream));
}

int rd_zero_rows_from_limit(void* buf, const int32_t* limit, int64_t rows, int64_t row_bytes, void* stream) {
  if (rows < 0 || row_bytes <= 0) return RD_EINVAL;
  if ((row_bytes % 16) != 0) return RD_EUNSUPPORTED;
  if (rows > 0 && row_bytes > (int64_t(1) << 62) / rows) return RD_EUNSUPPORTED;
  if (rows == 0 || limit == nullptr) return RD_OK;  // no rows past the limit: nothing to write
  if (!buf) return RD_EINVAL;
  if (!aligned16(buf) || (reinterpret_cast<uintptr_t>(limit) & 3u)) return RD_EINVAL;
  return rd::launch_zero_rows(buf, limit, rows, row_bytes, static_cast<hipStream_t>(stream));
}

int rd_tune_set(int32_t which, int32_t value) { return rd::tune_set(which, value); }

int rd_tune_tile_count(void) { return rd::tile_count(); }

}  // extern "C"
