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
//  * bf16 MFMA 32x32x16 with fp32 accumulation over 64-wide K steps;
//  * main pipeline: A/B tiles go straight from HBM into a 4-stage LDS ring
//    with 16-byte buffer-to-LDS loads (no VGPR staging), three stages in
//    flight behind the one being multiplied; per-tile buffer descriptors
//    bound every operand to its valid rows, and the hardware returns zeros
//    past that bound, so group edges and the packed-buffer limit cost no
//    instructions and rows >= limit are never fetched;
//  * fallback pipeline (contraction length not a multiple of 64, or operands
//    past 4 GiB): register-staged double-buffered LDS with explicit zeroing;
//  * operands whose contraction dimension is contiguous in memory are stored
//    row-per-MN-index and read with 128-bit LDS loads; operands whose MN
//    dimension is contiguous (the weight of ragged_dot, both operands of
//    trans_ragged_dot) are stored as they sit in memory and fed to the MFMA
//    through the gfx950 LDS transpose read (ds_read_b64_tr_b16), so no
//    operand is ever transposed in registers;
//  * LDS tiles are XOR-swizzled at 16-byte granularity instead of padded;
//  * tiles are ordered so that consecutive logical tiles land on one XCD,
//    which keeps a group's weight slab and rows in that XCD's L2.
#include <cstdlib>

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

// K-contiguous operand tile: ROWS rows (one per M or N index) of BK elements
// (128 bytes, half of the 64 four-byte banks).  A 128-bit LDS read serves 16
// lanes per phase, here 16 consecutive rows at one logical chunk; chunk c of
// row r sits at slot c ^ ((r >> 1) & 7), so rows of equal parity (same bank
// half) get 8 distinct slots and the 16 rows hit 16 distinct bank groups.
struct KLayout {
  __device__ __forceinline__ static int slot(int r, int c) { return c ^ ((r >> 1) & 7); }
  __device__ __forceinline__ static int offset(int r, int c) { return r * BK + (slot(r, c) << 3); }
};

// MN-contiguous operand tile: BK rows (one per contraction index) of COLS
// elements.  Chunk c of row r sits at slot c ^ swz(r), so the four rows one
// transposed read touches fall on disjoint banks.
template <int COLS>
struct MNLayout {
  static constexpr int kChunks = COLS / 8;
  __device__ __forceinline__ static int swz(int r) {
    if constexpr (kChunks >= 16) return (r & 3) << 2;       // rows span all banks: shift 4 rows apart
    else if constexpr (kChunks == 8) return ((r >> 1) & 1) << 2;  // two rows per bank line
    else return 0;
  }
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


// ---------------------------------------------------------------- buffer-to-LDS operands

// s_waitcnt immediate for gfx9-family "vmcnt(n)" leaving expcnt/lgkmcnt unconstrained.
constexpr int vmcnt_imm(int n) { return (n & 0xF) | ((n >> 4) << 14) | (0x7 << 4) | (0xF << 8); }

constexpr uint32_t kBufFlags = 0x00020000;  // raw buffer, 32-bit data format: out-of-range reads return 0

typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));

// Buffer resource (V#) over [base, base + bytes), bytes clamped to 4 GiB - 1, stride 0.
__device__ __forceinline__ u32x4_t make_rsrc(const void* base, unsigned long long bytes) {
  const unsigned long long a = reinterpret_cast<unsigned long long>(base);
  const uint32_t nrec = bytes < 0xFFFFFFFFull ? static_cast<uint32_t>(bytes) : 0xFFFFFFFFu;
  return u32x4_t{static_cast<uint32_t>(a), static_cast<uint32_t>(a >> 32) & 0xFFFFu, nrec, kBufFlags};
}

// One 16-byte buffer-to-LDS load per lane: lane i lands at lds + 16 * i
// (lds must be wave-uniform).  Issued as inline assembly so that the
// compiler does not drain the queue before every later LDS read; the
// pipeline below waits for these loads explicitly with s_waitcnt vmcnt.
// M0 holds the LDS base and needs one wait state before the load uses it.
// M0 is a reserved register (never allocated; the compiler sets it right
// before each instruction that reads it), so it is not listed as clobbered.
__device__ __forceinline__ void dma16(u32x4_t r, uint16_t* lds, uint32_t voff, uint32_t soff) {
  const uint32_t a = static_cast<uint32_t>(reinterpret_cast<uintptr_t>(RD_LDS(void, lds)));
  asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tbuffer_load_dwordx4 %1, %2, %3 offen lds"
               :
               : "s"(a), "v"(voff), "s"(r), "s"(soff)
               : "memory");
}

// K-contiguous operand fed by DMA.  The buffer starts at the tile's first row
// and covers only its valid rows; tile row r is buffer row r, contraction
// step kt covers columns [kt*BK, kt*BK + BK).  Each wave fills 1 KB slices
// (8 rows) of the KLayout tile: lane i writes slot i % 8 of row i / 8, so it
// fetches the logical chunk stored there, (i % 8) ^ ((row >> 1) & 7).
template <int ROWS>
struct KDma {
  static constexpr int kInstr = ROWS / 32;  // 1 KB slices per wave per stage
  static_assert(kInstr >= 1, "tile too small");
  u32x4_t rsrc;
  uint32_t voff[kInstr];

  __device__ __forceinline__ void init(const uint16_t* base, long long rows_valid, int ld, int wave) {
    rsrc = make_rsrc(base, static_cast<unsigned long long>(rows_valid) * ld * 2);
    const int lane = threadIdx.x & 63;
#pragma unroll
    for (int q = 0; q < kInstr; ++q) {
      const int row = 8 * (wave * kInstr + q) + (lane >> 3);
      const int c = KLayout::slot(row, lane & 7);  // the slot map is an involution
      voff[q] = static_cast<uint32_t>(row) * ld * 2 + c * 16;
    }
  }
  __device__ __forceinline__ void issue(uint16_t* tile, int kt, int wave) const {
#pragma unroll
    for (int q = 0; q < kInstr; ++q) dma16(rsrc, tile + (wave * kInstr + q) * 512, voff[q], kt * BK * 2);
  }
  __device__ __forceinline__ static bf16x8_t frag(const uint16_t* tile, int r_base, int ks) {
    return KOperand<ROWS>::frag(tile, r_base, ks);
  }
};

// MN-contiguous operand fed by DMA.  The buffer starts at the first
// contraction row and covers only valid rows; step kt covers rows
// [kt*BK, kt*BK + BK), tile columns are [mn0, mn0 + COLS).  A 1 KB slice is
// 512 / COLS rows of the MNLayout tile; lane i writes slot i % (COLS/8) of its
// row and fetches logical chunk slot ^ swz(row).
template <int COLS>
struct MNDma {
  static constexpr int kCpr = COLS / 8;
  static constexpr int kRowsPerSlice = 512 / COLS;
  static constexpr int kInstr = COLS / 32;
  static_assert(kInstr >= 1, "tile too small");
  u32x4_t rsrc;
  uint32_t voff[kInstr];
  uint32_t step_bytes;

  __device__ __forceinline__ void init(const uint16_t* base, long long rows_valid, int ld, int mn0, int wave) {
    rsrc = make_rsrc(base, static_cast<unsigned long long>(rows_valid) * ld * 2);
    step_bytes = static_cast<uint32_t>(BK) * ld * 2;
    const int lane = threadIdx.x & 63;
#pragma unroll
    for (int q = 0; q < kInstr; ++q) {
      const int row = (wave * kInstr + q) * kRowsPerSlice + lane / kCpr;
      const int c = (lane % kCpr) ^ MNLayout<COLS>::swz(row);
      voff[q] = static_cast<uint32_t>(row) * ld * 2 + (mn0 + c * 8) * 2;
    }
  }
  __device__ __forceinline__ void issue(uint16_t* tile, int kt, int wave) const {
#pragma unroll
    for (int q = 0; q < kInstr; ++q) dma16(rsrc, tile + (wave * kInstr + q) * 512, voff[q], kt * step_bytes);
  }
  __device__ __forceinline__ static bf16x8_t frag(const uint16_t* tile, int c_base, int ks) {
    return MNOperand<COLS>::frag(tile, c_base, ks);
  }
};

// MFMAs of one BK stage.  Fragments are double-buffered across the four
// 16-deep slices: slice ks+1 is read from LDS while slice ks multiplies, and a
// scheduling fence per slice keeps at most two fragment sets live (with 256
// accumulators per lane a deeper hoist would spill).
template <class OpA, class OpB, int MI, int NI>
__device__ __forceinline__ void mma_stage(const uint16_t* ta, const uint16_t* tb, f32x16_t (&acc)[MI][NI],
                                          int wm_off, int wn_off) {
  bf16x8_t af[2][MI], bfr[2][NI];
#pragma unroll
  for (int mi = 0; mi < MI; ++mi) af[0][mi] = OpA::frag(ta, wm_off + mi * 32, 0);
#pragma unroll
  for (int ni = 0; ni < NI; ++ni) bfr[0][ni] = OpB::frag(tb, wn_off + ni * 32, 0);
#pragma unroll
  for (int ks = 0; ks < BK / 16; ++ks) {
    const int cur = ks & 1;
    if (ks + 1 < BK / 16) {
#pragma unroll
      for (int mi = 0; mi < MI; ++mi) af[cur ^ 1][mi] = OpA::frag(ta, wm_off + mi * 32, ks + 1);
#pragma unroll
      for (int ni = 0; ni < NI; ++ni) bfr[cur ^ 1][ni] = OpB::frag(tb, wn_off + ni * 32, ks + 1);
    }
#pragma unroll
    for (int mi = 0; mi < MI; ++mi)
#pragma unroll
      for (int ni = 0; ni < NI; ++ni)
        acc[mi][ni] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[cur][mi], bfr[cur][ni], acc[mi][ni], 0, 0, 0);
    __builtin_amdgcn_sched_barrier(0);
  }
}

template <int N>
__device__ __forceinline__ void wait_vm() {
  __builtin_amdgcn_s_waitcnt(vmcnt_imm(N));
}

// Wait until at most `after` stages of this wave's loads remain in flight
// (after in [0, S-2], uniform).  vmcnt needs an immediate, hence the ladder.
template <int L, int S>
__device__ __forceinline__ void wait_stages(int after) {
  static_assert(S >= 2 && S <= 6 && (S - 2) * L <= 63, "pipeline depth");
  if constexpr (S >= 6) {
    if (after >= 4) { wait_vm<4 * L>(); return; }
  }
  if constexpr (S >= 5) {
    if (after >= 3) { wait_vm<3 * L>(); return; }
  }
  if constexpr (S >= 4) {
    if (after >= 2) { wait_vm<2 * L>(); return; }
  }
  if constexpr (S >= 3) {
    if (after >= 1) { wait_vm<L>(); return; }
  }
  wait_vm<0>();
}

// acc += A_tile * B_tile over nk steps through an S-stage LDS ring fed by
// buffer-to-LDS loads.  Step kt: wait for this wave's loads of stage kt,
// barrier (every wave's loads of stage kt have landed and every wave is done
// with step kt-1), refill the stage step kt-1 used with step kt+S-1, then
// multiply stage kt.  The raw s_barrier keeps later stages in flight across
// it (a __syncthreads fence would drain them).  Ends with a barrier so the
// next tile may refill any stage.
template <class OpA, class OpB, int MI, int NI, int S, int A_EL, int B_EL>
__device__ __forceinline__ void k_loop_dma(const OpA& A, const OpB& B, int nk, uint16_t* s_tiles,
                                           f32x16_t (&acc)[MI][NI], int wm_off, int wn_off, int wave) {
  if (nk <= 0) return;
  constexpr int L = OpA::kInstr + OpB::kInstr;  // loads per wave per stage
  constexpr int ST = A_EL + B_EL;
#pragma unroll
  for (int s = 0; s < S - 1; ++s) {
    if (s < nk) {
      A.issue(s_tiles + s * ST, s, wave);
      B.issue(s_tiles + s * ST + A_EL, s, wave);
    }
  }
  for (int kt = 0; kt < nk; ++kt) {
    const int after = min(nk - 1 - kt, S - 2);
    __builtin_amdgcn_sched_barrier(0);
    wait_stages<L, S>(after);
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_sched_barrier(0);
    const int nxt = kt + S - 1;
    if (nxt < nk) {
      const int s = nxt % S;
      A.issue(s_tiles + s * ST, nxt, wave);
      B.issue(s_tiles + s * ST + A_EL, nxt, wave);
    }
    const int cur = kt % S;
    mma_stage<OpA, OpB, MI, NI>(s_tiles + cur * ST, s_tiles + cur * ST + A_EL, acc, wm_off, wn_off);
  }
  __builtin_amdgcn_sched_barrier(0);
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_sched_barrier(0);
}

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

// Store one 32x32 accumulator block directly.  MFMA 32x32 result layout: lane
// l, value v holds row 8*(v/4) + 4*(l/32) + v%4, column l%32 of the block.
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

// Store a wave's (MI*32) x (NI*32) accumulator block at out[r0.., c0..].
// float32 goes out directly (32 lanes cover 128 contiguous bytes of a row).
// bf16 is rounded and staged through this wave's private LDS area as the
// transposed block T[col][row] (4 consecutive rows per 8-byte write); the LDS
// transpose read then hands each lane 4 + 4 consecutive columns of one row,
// so the block leaves in 16-byte stores.  Only this wave touches `stage`.
template <int MI, int NI>
__device__ __forceinline__ void store_wave_tile(const f32x16_t (&acc)[MI][NI], void* out, bool f32, long long ld,
                                                int r0, int rlim, int c0, int clim, uint16_t* stage) {
  constexpr int WM = MI * 32, WN = NI * 32;
  // Fences per 32-row block keep at most NI accumulator blocks in VGPRs at a time.
  if (f32) {
#pragma unroll
    for (int mi = 0; mi < MI; ++mi) {
#pragma unroll
      for (int ni = 0; ni < NI; ++ni) store_block(acc[mi][ni], out, true, ld, r0 + mi * 32, rlim, c0 + ni * 32, clim);
      __builtin_amdgcn_sched_barrier(0);
    }
    return;
  }
  using T = MNLayout<WM>;
  const int l = threadIdx.x & 63;
#pragma unroll
  for (int mi = 0; mi < MI; ++mi) {
#pragma unroll
    for (int ni = 0; ni < NI; ++ni)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int col = ni * 32 + (l & 31);
        const int row = mi * 32 + 8 * i + 4 * (l >> 5);
        const uint2 v = make_uint2(pack_bf16x2(acc[mi][ni][4 * i], acc[mi][ni][4 * i + 1]),
                                   pack_bf16x2(acc[mi][ni][4 * i + 2], acc[mi][ni][4 * i + 3]));
        *reinterpret_cast<uint2*>(stage + T::offset(col, row >> 3) + (row & 7)) = v;
      }
    __builtin_amdgcn_sched_barrier(0);
  }
  const int g = l >> 4, q = l & 15;
  uint16_t* o = static_cast<uint16_t*>(out);
#pragma unroll
  for (int rb = 0; rb < WM / 16; ++rb)
#pragma unroll
    for (int cb = 0; cb < WN / 32; ++cb) {
      const int rl = rb * 16, cl = cb * 32 + 8 * g;
      const int tcol = rl + 4 * (q & 3);
      const uint16_t* p0 = stage + T::offset(cl + (q >> 2), tcol >> 3) + (tcol & 7);
      const uint16_t* p1 = stage + T::offset(cl + 4 + (q >> 2), tcol >> 3) + (tcol & 7);
      const s16x4_t lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(RD_LDS(s16x4_t, p0));
      const s16x4_t hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(RD_LDS(s16x4_t, p1));
      const int grow = r0 + rl + q, gcol = c0 + cl;
      if (grow < rlim && gcol < clim) {
        typedef short s16x8_t __attribute__((ext_vector_type(8)));
        const s16x8_t both = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
        *reinterpret_cast<s16x8_t*>(o + grow * ld + gcol) = both;
      }
    }
}

// ---------------------------------------------------------------- kernels

// STAGES > 0: buffer-to-LDS pipeline with that many LDS stages (one workgroup
// per CU); STAGES == 0: register-staged fallback (two workgroups per CU).
// Occupancy: the register-staged and the 2-stage 128x128 variants run two
// workgroups per CU (their LDS fits twice), every other shape one.
template <int MODE, int BM, int BN, int STAGES>
__global__ __launch_bounds__(kThreads, (STAGES == 0 || (STAGES == 2 && BM * BN <= 128 * 128)) ? 2 : 1)
void grouped_gemm_kernel(KArgs p) {
  constexpr int WM = BM / 2, WN = BN / 2;
  constexpr int MI = WM / 32, NI = WN / 32;
  constexpr int A_EL = BM * BK, B_EL = BN * BK;
  constexpr int NBUF = STAGES > 0 ? STAGES : 2;
  __shared__ __attribute__((aligned(1024))) uint16_t s_tiles[NBUF * (A_EL + B_EL)];
  static_assert(4 * WM * WN <= NBUF * (A_EL + B_EL), "epilogue staging must fit in the pipeline ring");
  __shared__ int s_lb[RD_MAX_GROUPS + 1];
  __shared__ int s_aux[RD_MAX_GROUPS + 1];
  __shared__ long long s_wave[kThreads / 64];

  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int wm_off = (wave >> 1) * WM, wn_off = (wave & 1) * WN;
  const Window win = build_local_bounds(p.gs, p.G, p.offp, p.gl, p.limp, p.m, s_lb, s_wave);

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
      const int nk = (p.k + BK - 1) / BK;
      if constexpr (STAGES > 0) {
        KDma<BM> A;
        A.init(p.a + static_cast<long long>(row0) * p.k, row_end - row0, p.k, wave);
        if constexpr (MODE == kFwdNN) {
          MNDma<BN> B;
          B.init(wj, p.k, p.n, n0, wave);
          k_loop_dma<KDma<BM>, MNDma<BN>, MI, NI, STAGES, A_EL, B_EL>(A, B, nk, s_tiles, acc, wm_off, wn_off,
                                                                       wave);
        } else {
          KDma<BN> B;
          B.init(wj + static_cast<long long>(n0) * p.k, p.n - n0, p.k, wave);
          k_loop_dma<KDma<BM>, KDma<BN>, MI, NI, STAGES, A_EL, B_EL>(A, B, nk, s_tiles, acc, wm_off, wn_off,
                                                                      wave);
        }
      } else {
        KOperand<BM> A{p.a, p.k, row0, row_end, p.k};
        if constexpr (MODE == kFwdNN) {
          MNOperand<BN> B{wj, p.n, 0, p.k, n0, p.n};
          k_loop<KOperand<BM>, MNOperand<BN>, MI, NI, A_EL, B_EL>(A, B, nk, s_tiles, acc, wm_off, wn_off);
        } else {
          KOperand<BN> B{wj, p.k, n0, p.n, p.k};
          k_loop<KOperand<BM>, KOperand<BN>, MI, NI, A_EL, B_EL>(A, B, nk, s_tiles, acc, wm_off, wn_off);
        }
      }
      store_wave_tile<MI, NI>(acc, p.out, p.out_f32, p.n, row0 + wm_off, row_end, n0 + wn_off, p.n,
                              s_tiles + wave * (WM * WN));
      __syncthreads();  // staging area = pipeline ring: drain before the next tile refills it
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
      const int nk = (r_end - r_begin + BK - 1) / BK;
      if constexpr (STAGES > 0) {
        MNDma<BM> A;
        A.init(p.a + static_cast<long long>(r_begin) * p.k, r_end - r_begin, p.k, a0, wave);
        MNDma<BN> B;
        B.init(p.b + static_cast<long long>(r_begin) * p.n, r_end - r_begin, p.n, c0, wave);
        k_loop_dma<MNDma<BM>, MNDma<BN>, MI, NI, STAGES, A_EL, B_EL>(A, B, nk, s_tiles, acc, wm_off, wn_off, wave);
      } else {
        MNOperand<BM> A{p.a, p.k, r_begin, r_end, a0, p.k};
        MNOperand<BN> B{p.b, p.n, r_begin, r_end, c0, p.n};
        k_loop<MNOperand<BM>, MNOperand<BN>, MI, NI, A_EL, B_EL>(A, B, nk, s_tiles, acc, wm_off, wn_off);
      }
      char* dwj = static_cast<char*>(p.out) + static_cast<long long>(j) * p.k * p.n * (p.out_f32 ? 4 : 2);
      store_wave_tile<MI, NI>(acc, dwj, p.out_f32, p.n, a0 + wm_off, p.k, c0 + wn_off, p.n,
                              s_tiles + wave * (WM * WN));
      __syncthreads();  // staging area = pipeline ring: drain before the next tile refills it
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

// Tile shapes (BM x BN, LDS stages) of the buffer-to-LDS pipeline.  Every
// shape runs 4 waves in a 2 x 2 layout; larger wave tiles read fewer LDS bytes
// per MFMA, smaller BM wastes fewer MFMA rows on short groups.
enum Tile { kT64x128 = 0, kT128x128 = 1, kT128x256 = 2, kT256x256 = 3, kT128x128x2 = 4, kTileCount };

// RD_FWD_TILE / RD_TRANS_TILE (0..4) force a shape, for tile sweeps.
int forced_tile(const char* name) {
  const char* v = getenv(name);
  if (v == nullptr || *v == 0) return -1;
  const int t = atoi(v);
  return (t >= 0 && t < kTileCount) ? t : -1;
}

// Forward shape from what the host knows (never the device-resident group
// sizes): m / num_local bounds the mean rows per local group.  Decode-sized
// groups take the 64-row tile; otherwise a 128 x 256 tile when n allows it
// (fewer passes over each row block of x), else 128 x 128.  Chosen from a
// sweep of every shape on the up-projection, backward, window+limit and
// decode workloads.
int pick_forward_tile(const GemmProblem& p) {
  const int forced = forced_tile("RD_FWD_TILE");
  if (forced >= 0) return forced;
  const long long avg_rows = p.m / (p.num_local > 0 ? p.num_local : 1);
  if (avg_rows <= 48) return kT64x128;
  return p.n >= 256 ? kT128x256 : kT128x128;
}

// trans_ragged_dot: the contraction runs over a group's rows, often short, so
// two co-resident workgroups per CU (128 x 128, 2 stages) hide each other's
// pipeline fill and epilogue better than one deep pipeline.
int pick_trans_tile(const GemmProblem& p) {
  const int forced = forced_tile("RD_TRANS_TILE");
  if (forced >= 0) return forced;
  (void)p;
  return kT128x128x2;
}

template <int MODE, int BM, int BN, int S>
void launch_one(const KArgs& a, long long work, hipStream_t stream) {
  grouped_gemm_kernel<MODE, BM, BN, S><<<grid_size(work, (S > 0 && S != 2) || BM * BN > 128 * 128 ? 1 : 2),
                                        kThreads, 0, stream>>>(a);
}

template <int MODE>
void launch_tile(int tile, const KArgs& a, const GemmProblem& p, hipStream_t stream) {
  auto work = [&](int BM, int BN) {
    if (MODE == kTransTN)
      return static_cast<long long>(p.num_local) * ((p.k + BM - 1) / BM) * ((p.n + BN - 1) / BN);
    return (static_cast<long long>((p.m + BM - 1) / BM) + p.num_local) * ((p.n + BN - 1) / BN) +
           (p.m + kZeroRows - 1) / kZeroRows + 2;
  };
  switch (tile) {
    case kT64x128: launch_one<MODE, 64, 128, 6>(a, work(64, 128), stream); break;
    case kT128x256: launch_one<MODE, 128, 256, 3>(a, work(128, 256), stream); break;
    case kT256x256: launch_one<MODE, 256, 256, 2>(a, work(256, 256), stream); break;
    case kT128x128x2: launch_one<MODE, 128, 128, 2>(a, work(128, 128), stream); break;
    default: launch_one<MODE, 128, 128, 4>(a, work(128, 128), stream); break;
  }
}

// The buffer-to-LDS pipeline addresses every operand through 32-bit buffer
// offsets, so each operand must span less than 4 GiB.
bool fits_32bit(long long a, long long b) { return a * b * 2 < (1ll << 32); }

}  // namespace

int launch_forward(const GemmProblem& p, bool trans_rhs, hipStream_t stream) {
  const KArgs a = make_args(p);
  const bool dma = (p.k % BK) == 0 && fits_32bit(p.m, p.k) && fits_32bit(p.k, p.n);
  if (dma) {
    const int tile = pick_forward_tile(p);
    if (trans_rhs)
      launch_tile<kFwdNT>(tile, a, p, stream);
    else
      launch_tile<kFwdNN>(tile, a, p, stream);
  } else {
    const long long work = (static_cast<long long>((p.m + 127) / 128) + p.num_local) * ((p.n + 127) / 128) +
                           (p.m + kZeroRows - 1) / kZeroRows + 2;
    if (trans_rhs)
      launch_one<kFwdNT, 128, 128, 0>(a, work, stream);
    else
      launch_one<kFwdNN, 128, 128, 0>(a, work, stream);
  }
  return hipGetLastError() == hipSuccess ? RD_OK : RD_EHIP;
}

int launch_trans(const GemmProblem& p, hipStream_t stream) {
  const KArgs a = make_args(p);
  if (fits_32bit(p.m, p.k) && fits_32bit(p.m, p.n)) {
    launch_tile<kTransTN>(pick_trans_tile(p), a, p, stream);
  } else {
    const long long tiles = static_cast<long long>(p.num_local) * ((p.k + 127) / 128) * ((p.n + 127) / 128);
    launch_one<kTransTN, 128, 128, 0>(a, tiles, stream);
  }
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
