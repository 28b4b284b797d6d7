// Grouped GEMM kernels for gfx950: ragged_dot (w[g,k,n]), ragged_dot with
// trans_rhs (w[g,n,k]) and trans_ragged_dot (dW[g,k,n] = x_g^T dy_g).
//
// Operations follow SkyRL-tx PR #867 ("Integrate ragged_dot pallas kernel with
// group_offset support": ragged_dot, trans_rhs, trans_ragged_dot and the
// group_offset window of fast_ragged_dot) and MaxText PR #5760 (valid-rows
// commit: the packed-buffer limit, and the transposed grouped matmul removing
// out-of-group rows by selection).  The schedule is computed on the device
// from group_sizes (TransformerEngine PR #2213, Description: a host copy of
// group_sizes stalls the GPU and breaks graph capture).
//
// Design (MI355X):
//  * one persistent grid of 256-thread workgroups (4 wave64s in a 2x2 layout);
//    every workgroup scans group_sizes into LDS and walks the tile list;
//  * bf16 MFMA 32x32x16 with fp32 accumulation; A/B tiles are staged through
//    a double-buffered LDS with one barrier per 64-wide K step;
//  * operands whose contraction dimension is contiguous in memory are stored
//    row-per-MN-index and read with 128-bit LDS loads; operands whose MN
//    dimension is contiguous (the weight of ragged_dot, both operands of
//    trans_ragged_dot) are stored as they sit in memory and fed to the MFMA
//    through the gfx950 LDS transpose read (ds_read_b64_tr_b16), so no
//    operand is ever transposed in registers;
//  * LDS tiles are XOR-swizzled at 16-byte granularity instead of padded;
//  * tiles are ordered so that consecutive logical tiles land on one XCD,
//    which keeps a group's weight slab and rows in that XCD's L2.
#include "rd_device.h"
#include "rd_launch.h"

namespace rd {
namespace {

enum Mode { kFwdNN = 0, kFwdNT = 1, kTransTN = 2 };

constexpr int BK = 64;  // contraction elements per pipeline stage
constexpr int kZeroRows = 16;

struct KArgs {
  const uint16_t* a;
  const uint16_t* b;
  const int32_t* gs;
  const int32_t* offp;
  const int32_t* limp;
  void* out;
  int G, gl, out_f32;
  int m, k, n;
};

#define RD_LDS(T, p) ((__attribute__((address_space(3))) T*)(p))

// ---------------------------------------------------------------- LDS layouts

// K-contiguous operand tile: ROWS rows (one per M or N index) of BK elements.
// 16-byte chunk c of row r sits at chunk slot c ^ (r & 7): the 16 rows read by
// one 128-bit LDS access phase hit distinct banks.
struct KLayout {
  __device__ __forceinline__ static int offset(int r, int c) { return r * BK + ((c ^ (r & 7)) << 3); }
};

// MN-contiguous operand tile: BK rows (one per contraction index) of COLS
// elements.  Chunk c of row r sits at slot c ^ swz(r), so the four rows one
// transposed read touches fall on disjoint banks.
template <int COLS>
struct MNLayout {
  static constexpr int kChunks = COLS / 8;
  __device__ __forceinline__ static int swz(int r) { return kChunks >= 16 ? ((r & 3) << 2) : ((r & 1) << 2); }
  __device__ __forceinline__ static int offset(int r, int c) { return r * COLS + ((c ^ swz(r)) << 3); }
};

// ---------------------------------------------------------------- operands

// Operand whose contraction index is contiguous: rows [row0, row_end) of a
// row-major [*, ld] matrix, contraction columns [k0, k0 + BK) below kdim.
// Rows or columns outside the bounds load as zeros (selection, NaN-safe).
template <int ROWS>
struct KOperand {
  static constexpr int kPer = ROWS * BK / 8 / kThreads;
  static_assert(kPer >= 1, "tile too small for one 16-byte chunk per thread");
  const uint16_t* base;
  long long ld;
  int row0, row_end, kdim;
  uint4 v[kPer];

  __device__ __forceinline__ void load(int kt) {
    const int k0 = kt * BK;
#pragma unroll
    for (int i = 0; i < kPer; ++i) {
      const int ch = threadIdx.x + i * kThreads;
      const int r = ch >> 3, c = ch & 7;
      const int row = row0 + r, col = k0 + c * 8;
      if (row < row_end && col < kdim)
        v[i] = *reinterpret_cast<const uint4*>(base + row * ld + col);
      else
        v[i] = make_uint4(0, 0, 0, 0);
    }
  }
  __device__ __forceinline__ void store(uint16_t* tile) const {
#pragma unroll
    for (int i = 0; i < kPer; ++i) {
      const int ch = threadIdx.x + i * kThreads;
      *reinterpret_cast<uint4*>(tile + KLayout::offset(ch >> 3, ch & 7)) = v[i];
    }
  }
  // MFMA fragment: lane l gets tile row (r_base + l % 32), contraction
  // elements ks*16 + 8*(l/32) .. +7.
  __device__ __forceinline__ static bf16x8_t frag(const uint16_t* tile, int r_base, int ks) {
    const int l = threadIdx.x & 63;
    const int r = r_base + (l & 31);
    return *reinterpret_cast<const bf16x8_t*>(tile + KLayout::offset(r, 2 * ks + (l >> 5)));
  }
};

// Operand whose MN index is contiguous: contraction rows [krow0 + kt*BK, +BK)
// below krow_end of a row-major [*, ld] matrix, MN columns [mn0, mn0 + COLS)
// below mndim.  Out-of-bounds elements load as zeros.
template <int COLS>
struct MNOperand {
  static constexpr int kCpr = COLS / 8;  // 16-byte chunks per row
  static constexpr int kPer = BK * COLS / 8 / kThreads;
  static_assert(kPer >= 1, "tile too small for one 16-byte chunk per thread");
  const uint16_t* base;
  long long ld;
  int krow0, krow_end, mn0, mndim;
  uint4 v[kPer];

  __device__ __forceinline__ void load(int kt) {
#pragma unroll
    for (int i = 0; i < kPer; ++i) {
      const int ch = threadIdx.x + i * kThreads;
      const int r = ch / kCpr, c = ch % kCpr;
      const int row = krow0 + kt * BK + r, col = mn0 + c * 8;
      if (row < krow_end && col < mndim)
        v[i] = *reinterpret_cast<const uint4*>(base + row * ld + col);
      else
        v[i] = make_uint4(0, 0, 0, 0);
    }
  }
  __device__ __forceinline__ void store(uint16_t* tile) const {
#pragma unroll
    for (int i = 0; i < kPer; ++i) {
      const int ch = threadIdx.x + i * kThreads;
      *reinterpret_cast<uint4*>(tile + MNLayout<COLS>::offset(ch / kCpr, ch % kCpr)) = v[i];
    }
  }
  // MFMA fragment through the LDS transpose unit.  Within each 16-lane group,
  // lanes 4e..4e+3 name row e of a 4 x 16 block and lane i receives element i
  // of each of the 4 rows.  Lane l thus gets T[ks*16 + 8*(l/32) + e][c_base +
  // l % 32] for e = 0..7 (two reads: rows +0..3 and +4..7), matching the
  // contraction slots of KOperand::frag.
  __device__ __forceinline__ static bf16x8_t frag(const uint16_t* tile, int c_base, int ks) {
    const int l = threadIdx.x & 63;
    const int q = l & 15;
    const int krow = ks * 16 + 8 * (l >> 5) + (q >> 2);
    const int col = c_base + 16 * ((l >> 4) & 1) + 4 * (q & 3);
    const uint16_t* p0 = tile + MNLayout<COLS>::offset(krow, col >> 3) + (col & 7);
    const uint16_t* p1 = tile + MNLayout<COLS>::offset(krow + 4, col >> 3) + (col & 7);
    const s16x4_t lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(RD_LDS(s16x4_t, p0));
    const s16x4_t hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(RD_LDS(s16x4_t, p1));
    typedef short s16x8_t __attribute__((ext_vector_type(8)));
    const s16x8_t both = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
    return __builtin_bit_cast(bf16x8_t, both);
  }
};

// ---------------------------------------------------------------- tile main loop

// acc[MI][NI] += A_tile(BM x K) * B_tile(K x BN) over nk steps of BK.
// Register prefetch of step kt+1 overlaps the MFMAs of step kt; LDS is double
// buffered, one barrier per step.  Starts and ends with every wave past a
// barrier, so LDS may be rewritten by the next tile right away.
template <class OpA, class OpB, int MI, int NI, int A_EL, int B_EL>
__device__ __forceinline__ void k_loop(OpA& A, OpB& B, int nk, uint16_t* s_tiles, f32x16_t (&acc)[MI][NI],
                                       int wm_off, int wn_off) {
  if (nk <= 0) return;
  uint16_t* sa[2] = {s_tiles, s_tiles + A_EL};
  uint16_t* sb[2] = {s_tiles + 2 * A_EL, s_tiles + 2 * A_EL + B_EL};
  A.load(0);
  B.load(0);
  A.store(sa[0]);
  B.store(sb[0]);
  __syncthreads();
  for (int kt = 0; kt < nk; ++kt) {
    const int cur = kt & 1;
    const bool more = kt + 1 < nk;
    if (more) {
      A.load(kt + 1);
      B.load(kt + 1);
    }
#pragma unroll
    for (int ks = 0; ks < BK / 16; ++ks) {
      bf16x8_t af[MI], bfr[NI];
#pragma unroll
      for (int mi = 0; mi < MI; ++mi) af[mi] = OpA::frag(sa[cur], wm_off + mi * 32, ks);
#pragma unroll
      for (int ni = 0; ni < NI; ++ni) bfr[ni] = OpB::frag(sb[cur], wn_off + ni * 32, ks);
#pragma unroll
      for (int mi = 0; mi < MI; ++mi)
#pragma unroll
        for (int ni = 0; ni < NI; ++ni)
          acc[mi][ni] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[mi], bfr[ni], acc[mi][ni], 0, 0, 0);
    }
    if (more) {
      A.store(sa[cur ^ 1]);
      B.store(sb[cur ^ 1]);
    }
    __syncthreads();
  }
}

// Store one 32x32 accumulator block.  MFMA 32x32 result layout: lane l, value v
// holds row 8*(v/4) + 4*(l/32) + v%4, column l%32 of the block.
__device__ __forceinline__ void store_block(const f32x16_t& acc, void* out, bool f32, long long ld, int r0, int rlim,
                                            int c0, int clim) {
  const int l = threadIdx.x & 63;
  const int c = c0 + (l & 31);
  if (c >= clim) return;
#pragma unroll
  for (int v = 0; v < 16; ++v) {
    const int r = r0 + 8 * (v >> 2) + 4 * (l >> 5) + (v & 3);
    if (r < rlim) {
      if (f32)
        static_cast<float*>(out)[r * ld + c] = acc[v];
      else
        static_cast<uint16_t*>(out)[r * ld + c] = static_cast<uint16_t>(f32_to_bf16(acc[v]));
    }
  }
}

// ---------------------------------------------------------------- kernels

template <int MODE, int BM, int BN>
__global__ __launch_bounds__(kThreads, 2) void grouped_gemm_kernel(KArgs p) {
  constexpr int WM = BM / 2, WN = BN / 2;
  constexpr int MI = WM / 32, NI = WN / 32;
  constexpr int A_EL = BM * BK, B_EL = BN * BK;
  __shared__ __attribute__((aligned(16))) uint16_t s_tiles[2 * (A_EL + B_EL)];
  __shared__ int s_lb[RD_MAX_GROUPS + 1];
  __shared__ int s_aux[RD_MAX_GROUPS + 1];
  __shared__ long long s_wave[kThreads / 64];

  const int wave = threadIdx.x >> 6;
  const int wm_off = (wave >> 1) * WM, wn_off = (wave & 1) * WN;
  const Window win = build_local_bounds(p.gs, p.G, p.offp, p.gl, p.limp, p.m, s_lb, s_wave);
  const int lane = threadIdx.x & 63;
  (void)lane;

  if constexpr (MODE == kFwdNN || MODE == kFwdNT) {
    // Tiles: local group j owns ceil(rows_j / BM) m-tiles, each with n_tiles
    // n-tiles; logical order (group, n-tile, m-tile).
    const int total_m = tile_prefix(s_lb, p.gl, BM, s_aux, s_wave);
    const int n_tiles = (p.n + BN - 1) / BN;
    const long long T = static_cast<long long>(total_m) * n_tiles;
    const long long per_xcd = (T + kXcds - 1) / kXcds;
    for (long long s = blockIdx.x; s < per_xcd * kXcds; s += gridDim.x) {
      const long long lt = xcd_logical(s, per_xcd);
      if (lt >= T) continue;
      const int j = upper_index(s_aux, p.gl, static_cast<int>(lt / n_tiles));
      const int mj = s_aux[j + 1] - s_aux[j];
      const int within = static_cast<int>(lt - static_cast<long long>(s_aux[j]) * n_tiles);
      const int nt = within / mj, mt = within - nt * mj;
      const int row0 = s_lb[j] + mt * BM, row_end = s_lb[j + 1];
      const int n0 = nt * BN;
      const uint16_t* wj = p.b + static_cast<long long>(j) * p.k * p.n;
      f32x16_t acc[MI][NI];
#pragma unroll
      for (int mi = 0; mi < MI; ++mi)
#pragma unroll
        for (int ni = 0; ni < NI; ++ni) acc[mi][ni] = f32x16_t{};
      KOperand<BM> A{p.a, p.k, row0, row_end, p.k};
      const int nk = (p.k + BK - 1) / BK;
      if constexpr (MODE == kFwdNN) {
        MNOperand<BN> B{wj, p.n, 0, p.k, n0, p.n};
        k_loop<KOperand<BM>, MNOperand<BN>, MI, NI, A_EL, B_EL>(A, B, nk, s_tiles, acc, wm_off, wn_off);
      } else {
        KOperand<BN> B{wj, p.k, n0, p.n, p.k};
        k_loop<KOperand<BM>, KOperand<BN>, MI, NI, A_EL, B_EL>(A, B, nk, s_tiles, acc, wm_off, wn_off);
      }
#pragma unroll
      for (int mi = 0; mi < MI; ++mi)
#pragma unroll
        for (int ni = 0; ni < NI; ++ni)
          store_block(acc[mi][ni], p.out, p.out_f32, p.n, row0 + wm_off + mi * 32, row_end, n0 + wn_off + ni * 32,
                      p.n);
    }
    // Rows below L outside the window are written as +0; rows >= L are untouched.
    const int z1 = (win.lo + kZeroRows - 1) / kZeroRows;
    const int z2 = (win.L - win.hi + kZeroRows - 1) / kZeroRows;
    const int esz = p.out_f32 ? 4 : 2;
    const int cpr = p.n * esz / 16;
    for (int z = blockIdx.x; z < z1 + z2; z += gridDim.x) {
      int r0, r1;
      if (z < z1) {
        r0 = z * kZeroRows;
        r1 = min(r0 + kZeroRows, win.lo);
      } else {
        r0 = win.hi + (z - z1) * kZeroRows;
        r1 = min(r0 + kZeroRows, win.L);
      }
      uint4* dst = reinterpret_cast<uint4*>(static_cast<char*>(p.out) + static_cast<long long>(r0) * p.n * esz);
      const int nch = (r1 - r0) * cpr;
      for (int q = threadIdx.x; q < nch; q += kThreads) dst[q] = make_uint4(0, 0, 0, 0);
    }
  } else {
    // trans_ragged_dot: every local group owns ka x nc output tiles of dW[j];
    // the contraction runs over the group's rows.  Groups are visited largest
    // first; each XCD owns a contiguous slice of the n-tiles, so it streams
    // only its slice of dy while every XCD reads the (narrower) x rows.
    const int gl = p.gl;
    if (gl <= kThreads) {
      const int t = threadIdx.x;
      if (t < gl) {
        const int sz = s_lb[t + 1] - s_lb[t];
        int rank = 0;
        for (int i = 0; i < gl; ++i) {
          const int si = s_lb[i + 1] - s_lb[i];
          rank += (si > sz) || (si == sz && i < t);
        }
        s_aux[rank] = t;
      }
    } else {
      for (int t = threadIdx.x; t < gl; t += kThreads) s_aux[t] = t;
    }
    __syncthreads();
    const int ka = (p.k + BM - 1) / BM;
    const int nc = (p.n + BN - 1) / BN;
    const bool split = nc >= kXcds;
    const int ncx = split ? (nc + kXcds - 1) / kXcds : nc;
    const long long per_x = static_cast<long long>(gl) * ka * ncx;  // tiles per XCD slice
    const long long slots = split ? per_x * kXcds : per_x;
    for (long long s = blockIdx.x; s < slots; s += gridDim.x) {
      int x = 0;
      long long i = s;
      if (split) {
        x = static_cast<int>(s % kXcds);
        i = s / kXcds;
      }
      const int q = static_cast<int>(i / (static_cast<long long>(ka) * ncx));
      const int rem = static_cast<int>(i - static_cast<long long>(q) * ka * ncx);
      const int at = rem / ncx;
      const int ct = x * ncx + (rem - at * ncx);
      if (ct >= nc) continue;
      const int j = s_aux[q];
      const int r_begin = s_lb[j], r_end = s_lb[j + 1];
      const int a0 = at * BM, c0 = ct * BN;
      f32x16_t acc[MI][NI];
#pragma unroll
      for (int mi = 0; mi < MI; ++mi)
#pragma unroll
        for (int ni = 0; ni < NI; ++ni) acc[mi][ni] = f32x16_t{};
      MNOperand<BM> A{p.a, p.k, r_begin, r_end, a0, p.k};
      MNOperand<BN> B{p.b, p.n, r_begin, r_end, c0, p.n};
      const int nk = (r_end - r_begin + BK - 1) / BK;
      k_loop<MNOperand<BM>, MNOperand<BN>, MI, NI, A_EL, B_EL>(A, B, nk, s_tiles, acc, wm_off, wn_off);
      char* dwj = static_cast<char*>(p.out) + static_cast<long long>(j) * p.k * p.n * (p.out_f32 ? 4 : 2);
#pragma unroll
      for (int mi = 0; mi < MI; ++mi)
#pragma unroll
        for (int ni = 0; ni < NI; ++ni)
          store_block(acc[mi][ni], dwj, p.out_f32, p.n, a0 + wm_off + mi * 32, p.k, c0 + wn_off + ni * 32, p.n);
    }
  }
}

KArgs make_args(const GemmProblem& p) {
  KArgs a{};
  a.a = static_cast<const uint16_t*>(p.a);
  a.b = static_cast<const uint16_t*>(p.b);
  a.gs = p.group_sizes;
  a.offp = p.group_offset;
  a.limp = p.limit;
  a.out = p.out;
  a.G = p.num_groups;
  a.gl = p.num_local;
  a.out_f32 = p.out_f32 ? 1 : 0;
  a.m = p.m;
  a.k = p.k;
  a.n = p.n;
  return a;
}

int grid_size(long long work_items, int per_cu) {
  long long cap = static_cast<long long>(device_cu_count()) * per_cu;
  long long g = work_items < cap ? work_items : cap;
  if (g >= kXcds) g -= g % kXcds;
  return static_cast<int>(g < 1 ? 1 : g);
}

}  // namespace

int launch_forward(const GemmProblem& p, bool trans_rhs, hipStream_t stream) {
  constexpr int BM = 128, BN = 128;
  const KArgs a = make_args(p);
  const long long m_tiles = (p.m + BM - 1) / BM + p.num_local;
  const long long n_tiles = (p.n + BN - 1) / BN;
  const long long work = m_tiles * n_tiles + (p.m + kZeroRows - 1) / kZeroRows + 2;
  const int grid = grid_size(work, 2);
  if (trans_rhs)
    grouped_gemm_kernel<kFwdNT, BM, BN><<<grid, kThreads, 0, stream>>>(a);
  else
    grouped_gemm_kernel<kFwdNN, BM, BN><<<grid, kThreads, 0, stream>>>(a);
  return hipGetLastError() == hipSuccess ? RD_OK : RD_EHIP;
}

int launch_trans(const GemmProblem& p, hipStream_t stream) {
  constexpr int BM = 128, BN = 128;
  const KArgs a = make_args(p);
  const long long tiles =
      static_cast<long long>(p.num_local) * ((p.k + BM - 1) / BM) * ((p.n + BN - 1) / BN);
  const int grid = grid_size(tiles, 2);
  grouped_gemm_kernel<kTransTN, BM, BN><<<grid, kThreads, 0, stream>>>(a);
  return hipGetLastError() == hipSuccess ? RD_OK : RD_EHIP;
}

int device_cu_count() {
  static int cache[64] = {0};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) dev = 0;
  if (cache[dev] == 0) {
    int v = 0;
    if (hipDeviceGetAttribute(&v, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || v <= 0) v = 256;
    cache[dev] = v;
  }
  return cache[dev];
}

}  // namespace rd
