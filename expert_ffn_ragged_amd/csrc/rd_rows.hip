// Row utility of the packed expert buffer, for gfx950: rows at or past the
// valid-row limit written as +0.
//
// MaxText PR #5760 ("397B v7x trainer: MoE wo FSDP sharding and
// valid-rows-only MoE kernels"), commit on valid rows: the kernels of the
// packed buffer touch only rows [0, limit), the limit being a device scalar.
// Rows past it take no part in the computation, so the gradient of an input
// of that buffer is exactly zero there; the autograd layer writes those zeros
// with this kernel, which reads the limit on the device (no host copy, so a
// captured graph stays valid when the limit changes).
#include "rd_device.h"
#include "rd_launch.h"

namespace rd {
namespace {

__global__ __launch_bounds__(kThreads) void zero_rows_kernel(uint4* __restrict__ buf, const int32_t* __restrict__ limp,
                                                             long long rows, long long chunks_per_row) {
  long long L = rows;
  if (limp != nullptr) {
    const long long v = *limp;
    L = v < 0 ? 0 : (v > rows ? rows : v);
  }
  const long long first = L * chunks_per_row, last = rows * chunks_per_row;
  for (long long i = first + static_cast<long long>(blockIdx.x) * kThreads + threadIdx.x; i < last;
       i += static_cast<long long>(gridDim.x) * kThreads)
    buf[i] = make_uint4(0, 0, 0, 0);
}

}  // namespace

int launch_zero_rows(void* buf, const int32_t* limit, long long rows, long long row_bytes, hipStream_t stream) {
  const long long chunks = rows * (row_bytes / 16);
  const long long blocks = (chunks + kThreads - 1) / kThreads;
  const long long cap = static_cast<long long>(device_cu_count()) * 8;
  const int grid = static_cast<int>(blocks < cap ? (blocks < 1 ? 1 : blocks) : cap);
  zero_rows_kernel<<<grid, kThreads, 0, stream>>>(static_cast<uint4*>(buf), limit, rows, row_bytes / 16);
  return hipGetLastError() == hipSuccess ? RD_OK : RD_EHIP;
}

}  // namespace rd
