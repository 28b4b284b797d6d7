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
//  * one persistent grid of workgroups of 4 wave64s (2x2 layout; one or two
//    workgroups per CU) or 8 wave64s (2x4 or 4x2; two waves per SIMD, so a
//    wave's MFMAs issue while its SIMD partner waits on a barrier or an LDS
//    read); every workgroup scans group_sizes into LDS and walks the tile list;
//  * bf16 MFMA 32x32x16 with fp32 accumulation over 32- or 64-wide K steps;
//  * main pipeline: A/B tiles go straight from HBM into a 2- to 8-slot LDS
//    ring with 16-byte buffer-to-LDS loads (no VGPR staging), every slot but
//    one in flight behind the one being multiplied; per-tile buffer descriptors
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
#include <atomic>
#include <mutex>
#include <type_traits>

#include "rd_device.h"
#include "rd_glu_math.h"
#include "rd_launch.h"

namespace rd {
namespace {

enum Mode { kFwdNN = 0, kFwdNT = 1, kTransTN = 2, kFwdNT8 = 3, kFwdGLU = 4, kFwdNN8 = 5, kTransTN8 = 6 };
constexpr bool is_trans(int mode) { return mode == kTransTN || mode == kTransTN8; }
constexpr bool is_fp8(int mode) { return mode == kFwdNT8 || mode == kFwdNN8 || mode == kTransTN8; }

constexpr int BK = 64;  // contraction elements per pipeline stage
constexpr int kZeroRows = 16;

struct KArgs {
  const uint16_t* a;
  const uint16_t* b;
  const int32_t* gs;
  const int32_t* offp;
  const int32_t* limp;
  void* out;
  void* out2;  // kFwdGLU: the [gate | up] buffer [m, 2n] (may be null); out is silu(gate) * up [m, n]
  void* ws;    // kTransTN: row-split workspace (header, then fp32 partial tiles), or null
  long long ws_bytes;
  int per_cu;  // workgroups of this launch sharing a CU (ceil(grid / CUs))
  int G, gl, out_f32;
  int m, k, n;
};

#define RD_LDS(T, p) ((__attribute__((address_space(3))) T*)(p))

typedef int i32x4_t __attribute__((ext_vector_type(4)));
typedef int i32x8_t __attribute__((ext_vector_type(8)));

// ---------------------------------------------------------------- LDS layouts

// K-contiguous operand tile: ROWS rows (one per M or N index) of BK elements
// (128 bytes, half of the 64 four-byte banks).  A 128-bit LDS read serves 16
// lanes per phase, here 16 consecutive rows at one logical chunk; chunk c of
// row r sits at slot c ^ ((r >> 1) & 7), so rows of equal parity (same bank
// half) get 8 distinct slots and the 16 rows hit 16 distinct bank groups.
//
// With 32-element rows (64 bytes, four rows per bank line) the key is
// c ^ ((r >> 2) & 3): rows with equal r % 4 share a bank quarter and get 4
// distinct slots, so 16 consecutive rows again hit 16 distinct bank groups.
template <int KS>
struct KLayoutT {
  static constexpr int kChunks = KS / 8;
  static_assert(kChunks == 8 || kChunks == 4, "K-tile rows of 64 or 32 elements");
  __device__ __forceinline__ static int slot(int r, int c) {
    if constexpr (kChunks == 8) return c ^ ((r >> 1) & 7);
    else return c ^ ((r >> 2) & 3);
  }
  __device__ __forceinline__ static int offset(int r, int c) { return r * KS + (slot(r, c) << 3); }
  // MFMA fragment: lane l gets tile row (r_base + l % 32), contraction
  // elements ks*16 + 8*(l/32) .. +7.
  __device__ __forceinline__ static bf16x8_t frag(const uint16_t* tile, int r_base, int ks) {
    const int l = threadIdx.x & 63;
    return *reinterpret_cast<const bf16x8_t*>(tile + offset(r_base + (l & 31), 2 * ks + (l >> 5)));
  }
  // fp8 operand (two fp8 per 16-bit element): lane l gets row (r_base + l %
  // 32), fp8 contraction elements 64*kk + 32*(l/32) .. +31, i.e. 16-byte
  // chunks 4*kk + 2*(l/32) and the next one.
  __device__ __forceinline__ static i32x8_t frag8(const uint16_t* tile, int r_base, int kk) {
    const int l = threadIdx.x & 63;
    const int r = r_base + (l & 31), c = 4 * kk + 2 * (l >> 5);
    const i32x4_t lo = *reinterpret_cast<const i32x4_t*>(tile + offset(r, c));
    const i32x4_t hi = *reinterpret_cast<const i32x4_t*>(tile + offset(r, c + 1));
    return __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
  }
};
using KLayout = KLayoutT<BK>;

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
// M0 holds the LDS base and needs one wait state before the load uses it;
// it is declared clobbered, so the compiler re-establishes any M0 value of
// its own after the load.  M0 must also not change in the cycle right after
// the load: a build where the compiler wrote the next load's M0 immediately
// after it (M0 as an input operand of the statement) gave wrong
// trans_ragged_dot results from call to call, and every working build had at
// least one instruction in between.  So the statement writes M0 itself and
// ends with a wait state of its own.  (clang notes that a reserved register
// in a clobber list may not be preserved; here that is the intent, so the
// note is silenced.)
#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"
__device__ __forceinline__ void dma16(u32x4_t r, uint32_t lds_addr, uint32_t voff, uint32_t soff) {
  asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tbuffer_load_dwordx4 %1, %2, %3 offen lds\n\ts_nop 0"
               :
               : "s"(lds_addr), "v"(voff), "s"(r), "s"(soff)
               : "memory", "m0");
}

// The same load marked non-temporal, for data read exactly once (the decode
// path's weight stream): it does not displace reused lines from the caches.
__device__ __forceinline__ void dma16_nt(u32x4_t r, uint32_t lds_addr, uint32_t voff, uint32_t soff) {
  asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tbuffer_load_dwordx4 %1, %2, %3 offen nt lds\n\ts_nop 0"
               :
               : "s"(lds_addr), "v"(voff), "s"(r), "s"(soff)
               : "memory", "m0");
}
#pragma clang diagnostic pop

// Scalar operands of dma16 are wave-uniform by construction; readfirstlane
// states it, so the compiler keeps them in SGPRs as the instruction needs.
__device__ __forceinline__ uint32_t uniform(uint32_t v) {
  return static_cast<uint32_t>(__builtin_amdgcn_readfirstlane(static_cast<int>(v)));
}
__device__ __forceinline__ u32x4_t uniform(u32x4_t r) {
  return u32x4_t{uniform(r[0]), uniform(r[1]), uniform(r[2]), uniform(r[3])};
}

// 32-bit LDS address of a pointer into a __shared__ array.
__device__ __forceinline__ uint32_t lds_address(const void* p) {
  return uniform(static_cast<uint32_t>(reinterpret_cast<uintptr_t>(RD_LDS(const void, p))));
}

// K-contiguous operand fed by DMA, KS contraction elements per stage.  The
// buffer starts at the tile's first row and covers only its valid rows; tile
// row r is buffer row r, stage kt covers columns [kt*KS, kt*KS + KS).  Each
// wave fills 1 KB slices (64 / (KS/8) rows) of the KLayoutT<KS> tile: lane i
// writes slot i % (KS/8) of its row, so it fetches the logical chunk stored
// there (the slot map is an involution).
template <int ROWS, int KS, int NW = 4>
struct KDma {
  static constexpr int kFragReads = 1;  // LDS reads per MFMA fragment
  static constexpr int kCh = KS / 8;
  static constexpr int kRowsPerSlice = 64 / kCh;
  static constexpr int kInstr = ROWS / kRowsPerSlice / NW;  // 1 KB slices per wave per stage (NW waves)
  static_assert(kInstr >= 1, "tile too small");
  u32x4_t rsrc;
  uint32_t voff[kInstr];

  __device__ __forceinline__ void init(const uint16_t* base, long long rows_valid, int ld, int wave) {
    rsrc = uniform(make_rsrc(base, static_cast<unsigned long long>(rows_valid) * ld * 2));
    const int lane = threadIdx.x & 63;
#pragma unroll
    for (int q = 0; q < kInstr; ++q) {
      const int row = kRowsPerSlice * (wave * kInstr + q) + lane / kCh;
      const int c = KLayoutT<KS>::slot(row, lane % kCh);
      voff[q] = static_cast<uint32_t>(row) * ld * 2 + c * 16;
    }
  }
  // tile: LDS byte address of this operand's stage buffer.
  __device__ __forceinline__ void issue(uint32_t tile, int kt, int wave) const {
    const uint32_t soff = uniform(kt * KS * 2);
#pragma unroll
    for (int q = 0; q < kInstr; ++q) dma16(rsrc, tile + (wave * kInstr + q) * 1024, voff[q], soff);
  }
  __device__ __forceinline__ static bf16x8_t frag(const uint16_t* tile, int r_base, int ks) {
    return KLayoutT<KS>::frag(tile, r_base, ks);
  }
};

// MN-contiguous operand fed by DMA, KS contraction rows per stage.  The
// buffer starts at the first contraction row and covers only valid rows;
// stage kt covers rows [kt*KS, kt*KS + KS), tile columns are
// [mn0, mn0 + COLS).  A 1 KB slice is 512 / COLS rows of the MNLayout tile;
// lane i writes slot i % (COLS/8) of its row and fetches logical chunk
// slot ^ swz(row).
template <int COLS, int KS, int NW = 4>
struct MNDma {
  static constexpr int kFragReads = 2;  // LDS reads per MFMA fragment (two transposed 64-bit reads)
  static constexpr int kCpr = COLS / 8;
  static constexpr int kRowsPerSlice = 512 / COLS;
  static constexpr int kInstr = KS * COLS / (512 * NW);  // 1 KB slices per wave per stage (NW waves)
  static_assert(kInstr >= 1, "tile too small");
  u32x4_t rsrc;
  uint32_t voff[kInstr];
  uint32_t step_bytes;

  __device__ __forceinline__ void init(const uint16_t* base, long long rows_valid, int ld, int mn0, int wave) {
    rsrc = uniform(make_rsrc(base, static_cast<unsigned long long>(rows_valid) * ld * 2));
    step_bytes = uniform(static_cast<uint32_t>(KS) * ld * 2);
    const int lane = threadIdx.x & 63;
#pragma unroll
    for (int q = 0; q < kInstr; ++q) {
      const int row = (wave * kInstr + q) * kRowsPerSlice + lane / kCpr;
      const int c = (lane % kCpr) ^ MNLayout<COLS>::swz(row);
      voff[q] = static_cast<uint32_t>(row) * ld * 2 + (mn0 + c * 8) * 2;
    }
  }
  // tile: LDS byte address of this operand's stage buffer.
  __device__ __forceinline__ void issue(uint32_t tile, int kt, int wave) const {
    const uint32_t soff = uniform(kt * step_bytes);
#pragma unroll
    for (int q = 0; q < kInstr; ++q) dma16(rsrc, tile + (wave * kInstr + q) * 1024, voff[q], soff);
  }
  __device__ __forceinline__ static bf16x8_t frag(const uint16_t* tile, int c_base, int ks) {
    return MNOperand<COLS>::frag(tile, c_base, ks);
  }
};

// MFMAs of one KS-deep stage, in 16-deep slices with double-buffered
// fragments: stage_frags loads slice 0 (called right after the stage's
// barrier, before the next stage's loads are issued, so their issue covers the
// LDS latency); mma_stage then, for each slice, first issues the LDS reads of
// the next slice and then the slice's MFMAs (a scheduling group pins that
// order, so every read has a whole slice of MFMAs to land).  A fence per slice
// keeps at most two fragment sets live (with 256 accumulators per lane a
// deeper hoist would spill).
// Operands whose tile columns are split in two strips (the fused GLU weight).
template <class T>
struct SplitCols : std::false_type {};

// Tile column of a wave's B block ni (wn_off: the wave's column offset, NI
// blocks per wave).  Split-column operands give each wave NI/2 gate blocks and
// the NI/2 up blocks of the same columns.
template <class OpB, int NI>
__device__ __forceinline__ int b_col(int wn_off, int ni) {
  if constexpr (SplitCols<OpB>::value)
    return ni < NI / 2 ? wn_off / 2 + ni * 32 : OpB::kHalf + wn_off / 2 + (ni - NI / 2) * 32;
  else
    return wn_off + ni * 32;
}

template <class OpA, class OpB, int MI, int NI>
struct StageFrags {
  bf16x8_t a[2][MI], b[2][NI];
};

template <class OpA, class OpB, int MI, int NI>
__device__ __forceinline__ void stage_frags(const uint16_t* ta, const uint16_t* tb, StageFrags<OpA, OpB, MI, NI>& f,
                                            int wm_off, int wn_off) {
#pragma unroll
  for (int mi = 0; mi < MI; ++mi) f.a[0][mi] = OpA::frag(ta, wm_off + mi * 32, 0);
#pragma unroll
  for (int ni = 0; ni < NI; ++ni) f.b[0][ni] = OpB::frag(tb, b_col<OpB, NI>(wn_off, ni), 0);
}

template <class OpA, class OpB, int MI, int NI, int KS = BK>
__device__ __forceinline__ void mma_stage(const uint16_t* ta, const uint16_t* tb, StageFrags<OpA, OpB, MI, NI>& f,
                                          f32x16_t (&acc)[MI][NI], int wm_off, int wn_off) {
  constexpr int kReads = MI * OpA::kFragReads + NI * OpB::kFragReads;
#pragma unroll
  for (int ks = 0; ks < KS / 16; ++ks) {
    const int cur = ks & 1;
    if (ks + 1 < KS / 16) {
#pragma unroll
      for (int mi = 0; mi < MI; ++mi) f.a[cur ^ 1][mi] = OpA::frag(ta, wm_off + mi * 32, ks + 1);
#pragma unroll
      for (int ni = 0; ni < NI; ++ni) f.b[cur ^ 1][ni] = OpB::frag(tb, b_col<OpB, NI>(wn_off, ni), ks + 1);
    }
#pragma unroll
    for (int mi = 0; mi < MI; ++mi)
#pragma unroll
      for (int ni = 0; ni < NI; ++ni)
        acc[mi][ni] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(f.a[cur][mi], f.b[cur][ni], acc[mi][ni], 0, 0, 0);
    if (ks + 1 < KS / 16) __builtin_amdgcn_sched_group_barrier(0x100, kReads, 0);  // next slice's LDS reads
    __builtin_amdgcn_sched_group_barrier(0x008, MI * NI, 0);                       // then this slice's MFMAs
    __builtin_amdgcn_sched_barrier(0);
  }
}

template <int N>
__device__ __forceinline__ void wait_vm() {
  __builtin_amdgcn_s_waitcnt(vmcnt_imm(N));
}

// Wait until at most `after` stages of this wave's loads remain in flight
// (after in [0, K], uniform); vmcnt takes an immediate, hence the ladder.
template <int L, int K>
__device__ __forceinline__ void wait_ladder(int after) {
  static_assert(K * L <= 63, "vmcnt counts up to 63 operations");
  if constexpr (K > 0) {
    if (after >= K) {
      wait_vm<K * L>();
      return;
    }
    wait_ladder<L, K - 1>(after);
  } else {
    wait_vm<0>();
  }
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

// Epilogue staging: 16 rows x 32 floats per wave at a time, row-major, rows
// padded to 36 floats (144 bytes: consecutive rows start in distinct 16-byte
// bank slots).
constexpr int kStagePitch = 36;
constexpr int kStageFloats = 16 * kStagePitch;  // per wave
// bf16 staging of a block half: rows of 40 halves (80 bytes: rows r and r + 4
// of one MFMA-layout write fall 16 banks apart), blocks 1344 bytes apart (the
// two blocks of a read-back pair start 16 banks apart); fits in kStageFloats.
constexpr int kStagePitchH = 40;
constexpr int kStageHalves = 16 * kStagePitchH + 32;
static_assert(kStageHalves * 2 <= kStageFloats * 4, "bf16 staging fits in the float32 staging area");

// Store a wave's (MI*32) x (NI*32) accumulator block at out[r0.., c0..]
// (row pitch ld elements, rows < rlim, columns < clim).  Each 32 x 32 block
// goes through this wave's private LDS area in two 16-row halves: the
// accumulators are written straight from their registers (MFMA layout: lane
// l holds column l % 32 of rows 8*(v/4) + 4*(l/32) + v%4; half h takes v/4 in
// {2h, 2h+1}), so 32 lanes fill 128 contiguous bytes of a row per write;
// then every lane reads 8 consecutive floats of one row, rounds them (bf16,
// round-to-nearest-even) or keeps them (f32), and issues 16-byte stores.  The
// NI blocks of one row half are staged side by side (NI areas of
// kStageFloats) before any is read back, so the LDS write-to-read latency is
// paid once per NI blocks.  No accumulator is copied into general registers
// wholesale, which keeps 256-accumulator tiles unspilled.  LDS operations of
// one wave run in order, so the areas are reused safely.
// Largest divisor of NI whose staging areas (NW waves x NB x kStageFloats
// floats) fit in `elems` bf16 elements of LDS.
constexpr int epilogue_batch(int NI, int elems, int NW) {
  int best = 0;
  for (int nb = 1; nb <= NI; ++nb)
    if (NI % nb == 0 && NW * nb * kStageFloats * 2 <= elems) best = nb;
  return best;
}
// The same for bf16 staging (blocks of kStageHalves 16-bit elements).
constexpr int epilogue_batch16(int NI, int elems, int NW) {
  int best = 0;
  for (int nb = 1; nb <= NI; ++nb)
    if (NI % nb == 0 && NW * nb * kStageHalves <= elems) best = nb;
  return best;
}

// One 16-byte store, non-temporal (write-once data) when NT.
template <bool NT, class V>
__device__ __forceinline__ void store16(V v, void* p) {
  if constexpr (NT)
    __builtin_nontemporal_store(v, reinterpret_cast<V*>(p));
  else
    *reinterpret_cast<V*>(p) = v;
}

// Blocks [B0, B0 + NBLK) of the NI are stored, the first at column c0.
// Read-back: every store instruction writes whole 128-byte row segments, 8
// rows of them: f32 lane l takes row l / 8 of a 16-row half, floats
// 4 (l % 8) .. +3 of one block; bf16 (blocks staged in pairs) lane l takes
// row l / 8, block (l / 4) % 2 of the pair, floats 8 (l % 4) .. +7.  NT marks
// the stores non-temporal.
// S16: bf16 results are rounded before staging (the same RNE per element) and
// staged as bf16, NB16 blocks at a time: half the staging traffic and, with
// the smaller blocks, fewer LDS round trips (used by trans_ragged_dot, whose
// dW tiles dominate its time; the register-heavy fused-GLU tiles would
// spill).  float32 results, and every result without S16, are staged as
// float32, NB blocks at a time.
template <int MI, int NI, int NB = NI, int B0 = 0, int NBLK = NI, bool NT = false, bool S16 = false, int NB16 = NB>
__device__ __forceinline__ void store_wave_tile(const f32x16_t (&acc)[MI][NI], void* out, bool f32, long long ld,
                                                int r0, int rlim, int c0, int clim, float* stage) {
  static_assert(NBLK % NB == 0 && NBLK % NB16 == 0 && B0 + NBLK <= NI, "staged blocks must divide the range");
  const int l = threadIdx.x & 63;
  const int rr = l >> 3;
  // staging row of MFMA-layout value v of half h
  auto srow = [&](int v, int h) { return 8 * (v >> 2) - 16 * h + 4 * (l >> 5) + (v & 3); };
  if (S16 && !f32) {
    uint16_t* st = reinterpret_cast<uint16_t*>(stage);
    constexpr int PAIR = NB16 % 2 == 0 ? 2 : 1;
    const int cc = (l & 3) * 8;
    const int sub = PAIR == 2 ? (l >> 2) & 1 : 0;
    const int rows_per = PAIR == 2 ? 8 : 16;
    const int rw = PAIR == 2 ? rr : (l >> 2);
#pragma unroll
    for (int mi = 0; mi < MI; ++mi)
#pragma unroll
      for (int h = 0; h < 2; ++h)
#pragma unroll
        for (int n0 = 0; n0 < NBLK; n0 += NB16) {
#pragma unroll
          for (int b = 0; b < NB16; ++b)
#pragma unroll
            for (int v = 8 * h; v < 8 * h + 8; ++v)
              st[b * kStageHalves + srow(v, h) * kStagePitchH + (l & 31)] =
                  static_cast<uint16_t>(f32_to_bf16(acc[mi][B0 + n0 + b][v]));
#pragma unroll
          for (int bp = 0; bp < NB16; bp += PAIR)
#pragma unroll
            for (int q = 0; q < 16 / rows_per; ++q) {
              const int row = rows_per * q + rw, b = bp + sub;
              const int grow = r0 + mi * 32 + 16 * h + row, gcol = c0 + (n0 + b) * 32 + cc;
              const u32x4_t v = *reinterpret_cast<const u32x4_t*>(st + b * kStageHalves + row * kStagePitchH + cc);
              if (grow < rlim && gcol < clim) store16<NT>(v, static_cast<uint16_t*>(out) + grow * ld + gcol);
            }
          __builtin_amdgcn_sched_barrier(0);
        }
    return;
  }
#pragma unroll
  for (int mi = 0; mi < MI; ++mi)
#pragma unroll
    for (int h = 0; h < 2; ++h)
#pragma unroll
      for (int n0 = 0; n0 < NBLK; n0 += NB) {
#pragma unroll
        for (int b = 0; b < NB; ++b)
#pragma unroll
          for (int v = 8 * h; v < 8 * h + 8; ++v)
            stage[b * kStageFloats + srow(v, h) * kStagePitch + (l & 31)] = acc[mi][B0 + n0 + b][v];
        if (f32) {
          const int cc = (l & 7) * 4;
#pragma unroll
          for (int b = 0; b < NB; ++b)
#pragma unroll
            for (int q = 0; q < 2; ++q) {
              const int row = 8 * q + rr;
              const f32x4_t v = *reinterpret_cast<const f32x4_t*>(stage + b * kStageFloats + row * kStagePitch + cc);
              const int grow = r0 + mi * 32 + 16 * h + row, gcol = c0 + (n0 + b) * 32 + cc;
              if (grow < rlim && gcol < clim) store16<NT>(v, static_cast<float*>(out) + grow * ld + gcol);
            }
        } else {
          const int cc = (l & 3) * 8;
          constexpr int PAIR = NB % 2 == 0 ? 2 : 1;
          const int sub = PAIR == 2 ? (l >> 2) & 1 : 0;
          const int rows_per = PAIR == 2 ? 8 : 16;  // rows one instruction covers
          const int rw = PAIR == 2 ? rr : (l >> 2);
#pragma unroll
          for (int bp = 0; bp < NB; bp += PAIR)
#pragma unroll
            for (int q = 0; q < 16 / rows_per; ++q) {
              const int row = rows_per * q + rw, b = bp + sub;
              const float* src = stage + b * kStageFloats + row * kStagePitch + cc;
              const f32x4_t lo = *reinterpret_cast<const f32x4_t*>(src);
              const f32x4_t hi = *reinterpret_cast<const f32x4_t*>(src + 4);
              const int grow = r0 + mi * 32 + 16 * h + row, gcol = c0 + (n0 + b) * 32 + cc;
              if (grow < rlim && gcol < clim) {
                const u32x4_t v = {pack_bf16x2(lo[0], lo[1]), pack_bf16x2(lo[2], lo[3]), pack_bf16x2(hi[0], hi[1]),
                                   pack_bf16x2(hi[2], hi[3])};
                store16<NT>(v, static_cast<uint16_t*>(out) + grow * ld + gcol);
              }
            }
        }
        __builtin_amdgcn_sched_barrier(0);
      }
}

// Zeros for a wave's block (a local group with no rows gets an all +0 dW).
template <int MI, int NI>
__device__ __forceinline__ void store_wave_zero(void* out, bool f32, long long ld, int r0, int rlim, int c0,
                                                int clim) {
  constexpr int WM = MI * 32, WN = NI * 32;
  const int esz = f32 ? 4 : 2;
  const int cpr = WN * esz / 16;  // 16-byte chunks per row of the block
  const int l = threadIdx.x & 63;
  for (int i = l; i < WM * cpr; i += 64) {
    const int r = r0 + i / cpr, c = c0 + (i % cpr) * (16 / esz);
    if (r < rlim && c < clim)
      store16<true>(u32x4_t{0, 0, 0, 0}, static_cast<char*>(out) + (r * ld + c) * esz);
  }
}

// Epilogue of the fused up-projection: the wave's first NI/2 blocks are gate
// columns and the last NI/2 the matching up columns.  Gate and up are rounded
// to bf16 (what the [gate | up] buffer holds), the GLU takes them in float32
// and its result is rounded once: bit for bit what the separate GEMM and GLU
// kernels give.  The [gate | up] buffer itself is written when fused != null.
template <int MI, int NI, int NB, int NBH, bool NT>
__device__ __forceinline__ void store_glu_tile(const f32x16_t (&acc)[MI][NI], void* act, void* fused, int h,
                                               int r0, int rlim, int c0, float* stage) {
  constexpr int NH = NI / 2;
  if (fused != nullptr) {
    store_wave_tile<MI, NI, NB, 0, NH, NT>(acc, fused, false, 2ll * h, r0, rlim, c0, h, stage);
    store_wave_tile<MI, NI, NB, NH, NH, NT>(acc, fused, false, 2ll * h, r0, rlim, h + c0, 2 * h, stage);
  }
  f32x16_t g[MI][NH];
#pragma unroll
  for (int mi = 0; mi < MI; ++mi)
#pragma unroll
    for (int b = 0; b < NH; ++b)
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const float gate = bf16_to_f32(f32_to_bf16(acc[mi][b][v]));
        const float up = bf16_to_f32(f32_to_bf16(acc[mi][NH + b][v]));
        g[mi][b][v] = glu_f32(gate, up);
      }
  store_wave_tile<MI, NH, NBH, 0, NH, NT>(g, act, false, h, r0, rlim, c0, h, stage);
}

// ---------------------------------------------------------------- tile lists

// Forward tiles: local group j owns ceil(rows_j / BM) m-tiles, each with
// n_tiles n-tiles.  Within a group, tiles come in blocks of gm m-tiles x all
// n-tiles (m-tile fastest), gm sized so one block roughly fills the
// workgroups of one XCD: tiles running together share each row block of x
// across the n-tiles and each weight slice across gm m-tiles.  Logical tiles
// are dealt so that consecutive ones land on one XCD.
struct FwdTiles {
  long long T, per_xcd, slots;
  int n_tiles, gm;
  struct Tile {
    int j, row0, row_end, n0, nk;
  };
  __device__ __forceinline__ void init(int total_m, int n, int BN, int k) {
    n_tiles = (n + BN - 1) / BN;
    T = static_cast<long long>(total_m) * n_tiles;
    per_xcd = (T + kXcds - 1) / kXcds;
    slots = per_xcd * kXcds;
    gm = max(1, max(1, static_cast<int>(gridDim.x) / kXcds) / n_tiles);
    (void)k;
  }
  template <int BM, int BN, int KS = BK>
  __device__ __forceinline__ bool get(long long s, const int* s_lb, const int* s_aux, int gl, int k, Tile& t) const {
    const long long lt = xcd_logical(s, per_xcd);
    if (lt >= T) return false;
    const int j = upper_index(s_aux, gl, static_cast<int>(lt / n_tiles));
    const int mj = s_aux[j + 1] - s_aux[j];
    const int within = static_cast<int>(lt - static_cast<long long>(s_aux[j]) * n_tiles);
    const int mb = within / (gm * n_tiles);  // m-block of this group
    const int rem = within - mb * gm * n_tiles;
    const int bm = min(gm, mj - mb * gm);     // m-tiles in this (possibly short) block
    const int nt = rem / bm, mt = mb * gm + (rem - nt * bm);
    t.j = j;
    t.row0 = s_lb[j] + mt * BM;
    t.row_end = s_lb[j + 1];
    t.n0 = nt * BN;
    t.nk = (k + KS - 1) / KS;
    return true;
  }
};

// The slots a workgroup walks: round u takes slot origin + u * step + pos,
// pos = p, or step - 1 - p on odd rounds when snake is set (count of them).
struct SlotSeq {
  long long origin, step, count;
  long long p;
  bool snake;
  __device__ __forceinline__ long long at(long long u) const {
    return origin + u * step + ((snake && (u & 1)) ? step - 1 - p : p);
  }
};

// Every gridDim.x-th slot from blockIdx.x (the forward tiles all cost the same).
__device__ __forceinline__ SlotSeq strided_slots(long long slots) {
  const long long b = blockIdx.x, g = gridDim.x;
  return SlotSeq{0, g, b < slots ? (slots - b + g - 1) / g : 0, b, false};
}

// Position p of `step` in every round of slots [origin, end), the order
// reversed on odd rounds: the slots of a list sorted by falling cost even out
// over the positions (round-robin gives the first positions the dearest slot
// of every round).
__device__ __forceinline__ SlotSeq snake_slots(long long origin, long long end, long long step, long long p) {
  const long long n = end - origin;
  if (n <= 0 || step <= 0) return SlotSeq{origin, 1, 0, 0, false};
  const long long rounds = n / step, rem = n % step;
  const long long last = (rounds & 1) ? step - 1 - p : p;  // position taken in the partial round
  return SlotSeq{origin, step, rounds + (last < rem ? 1 : 0), p, true};
}

// trans_ragged_dot tiles: every local group owns ka x nc output tiles of
// dW[j]; the contraction runs over the group's rows.  Groups are visited
// largest first (s_order).  The eight XCDs form an xa x xc grid: XCD
// (xa_i, xc_i) owns the a-tiles of slice xa_i and the c-tiles of slice xc_i of
// every group, so each XCD does an equal share of every group and a row block
// of x (dy) is fetched by xc (xa) XCDs.  The grid shape minimises that
// re-read traffic, k * xc + n * xa.
//
// Row split (plan(), with a caller workspace): a group whose contraction
// costs at least the mean work per CU, and more than one chunk, is cut into P
// row chunks of equal step counts, so that no tile holds up the grid.
// Those groups are a prefix of the largest-first order (at most kMaxSplit of
// them).  A chunk's tile is written as an fp32 partial to the workspace; a
// second kernel (trans_split_reduce) adds a tile's P partials in chunk order,
// so the result does not depend on scheduling.  The list holds, in order,
// every chunk of the split groups (chunk-major: the tiles of one chunk share
// its rows), then every other group.  Without the split (no workspace, or
// kernels that do not call plan()) the list is as before, one unit per group.
constexpr int kMaxSplit = 16;
// workspace header: [0] ns, [1] BM, [2] BN, then (j, P, first chunk) per split group from [3]
constexpr int kSplitHeaderInts = 64;
constexpr int kSplitMinSteps = 32;  // shortest chunk, in contraction steps
static_assert(3 + 3 * kMaxSplit <= kSplitHeaderInts, "split header");

struct TransTiles {
  long long tpg, slots;  // slots per list unit (a group, or a chunk of a split group), slots
  int ka, nc, kax, ncx, xc;
  bool split;            // the XCD grid
  int ns, cs;            // split groups, chunk length bound (steps)
  struct Tile {
    int j, r_begin, r_end, a0, c0, nk;
    int part;  // partial tile index in the workspace, or -1: write dW directly
  };
  __device__ __forceinline__ void init(int gl, int k, int n, int BM, int BN) {
    ka = (k + BM - 1) / BM;
    nc = (n + BN - 1) / BN;
    int xa = 0;
    xc = 0;
    long long best = 0;
    for (int a = 1; a <= kXcds; a *= 2) {
      const int c = kXcds / a;
      if (a > ka || c > nc) continue;
      const long long cost = static_cast<long long>(k) * c + static_cast<long long>(n) * a;
      if (xa == 0 || cost < best) {
        xa = a;
        xc = c;
        best = cost;
      }
    }
    split = xa > 0;
    if (!split) xa = xc = 1;
    kax = (ka + xa - 1) / xa;
    ncx = (nc + xc - 1) / xc;
    tpg = static_cast<long long>(kax) * ncx * (split ? kXcds : 1);
    slots = static_cast<long long>(gl) * tpg;
    ns = 0;
    cs = 0;
  }

  // Contraction steps of the group at position q of s_order (at least 1: an
  // empty group's tile still costs its zero store).
  template <int KS>
  __device__ __forceinline__ static long long steps_at(const int* s_lb, const int* s_order, int q) {
    const int j = s_order[q];
    const long long st = (s_lb[j + 1] - s_lb[j] + KS - 1) / KS;
    return st < 1 ? 1ll : st;
  }

  // Sum of v over the workgroup's NT threads (uses s_wave; ends with a barrier).
  template <int NT>
  __device__ __forceinline__ static long long block_sum(long long v, long long* s_wave) {
#pragma unroll
    for (int d = 32; d >= 1; d >>= 1) v += __shfl_xor(v, d, 64);
    __syncthreads();
    if ((threadIdx.x & 63) == 0) s_wave[threadIdx.x >> 6] = v;
    __syncthreads();
    long long sum = 0;
    for (int w = 0; w < NT / 64; ++w) sum += s_wave[w];
    __syncthreads();
    return sum;
  }

  // The row split plan, the same in every workgroup (it depends on the group
  // sizes, the grid, per_cu and cap_tiles only): ns groups and s_cp[i] =
  // chunks of the first i split groups (s_cp[0..ns]).  A group is split when
  // one of its tiles costs at least the mean work per CU (per_cu workgroups
  // share a CU): below that, the CU holding it also runs lighter work of its
  // co-resident workgroups, and the partials' round trip through memory costs
  // more than the balance gains (measured on the 32768-row backward, whose
  // largest expert is 0.57 of that mean: 362 us unsplit, 386 us split).
  // F10 / 10 scales that threshold: 1 for bf16, 1.3 for fp8 operands, whose
  // tiles take half the steps for the same partial traffic (one expert
  // holding 60 % of the backward's rows, 1.13 of the mean: 212 us unsplit,
  // 231 us split; 80 %, 1.5 of it: 242 vs 232 us; 95 %: 279 vs 234 us).  At
  // most cap_tiles partial tiles (the workspace); fewer split groups when
  // they would not fit.  Workgroup 0 writes the plan to the workspace header
  // for the reduction.  NT threads; ends with a barrier.
  template <int NT, int KS, int F10 = 10>
  __device__ void plan(const int* s_lb, const int* s_order, int gl, long long* s_wave, int* s_cp, long long cap_tiles,
                       int per_cu, int* header) {
    long long mine = 0;
    for (int q = threadIdx.x; q < gl; q += NT) mine += steps_at<KS>(s_lb, s_order, q);
    const long long total = block_sum<NT>(mine, s_wave) * tpg;
    const long long G = gridDim.x;
    long long c = (total + 2 * G - 1) / (2 * G);  // half the mean work per workgroup
    if (c < kSplitMinSteps) c = kSplitMinSteps;
    cs = static_cast<int>(c);
    if (threadIdx.x == 0) {
      // the prefix of the largest-first order that is heavy and longer than a chunk
      int n = 0, cp = 0;
      s_cp[0] = 0;
      const long long tiles = static_cast<long long>(ka) * nc;
      while (n < kMaxSplit && n < gl) {
        const long long st = steps_at<KS>(s_lb, s_order, n);
        if (st * G * 10 < total * per_cu * F10 || st <= c) break;
        const int P = static_cast<int>((st + c - 1) / c);
        if ((cp + P) * tiles > cap_tiles) break;
        cp += P;
        s_cp[++n] = cp;
      }
      s_cp[kMaxSplit + 1] = n;
      if (blockIdx.x == 0 && header != nullptr) {
        header[0] = n;
        for (int i = 0; i < n; ++i) {
          header[3 + 3 * i] = s_order[i];
          header[4 + 3 * i] = s_cp[i + 1] - s_cp[i];
          header[5 + 3 * i] = s_cp[i];
        }
      }
    }
    __syncthreads();
    ns = s_cp[kMaxSplit + 1];
    slots = (static_cast<long long>(s_cp[ns]) + (gl - ns)) * tpg;
    __syncthreads();
  }

  template <int BM, int BN, int KS = BK>
  __device__ __forceinline__ bool get(long long s, const int* s_lb, const int* s_order, Tile& t,
                                      const int* s_cp = nullptr) const {
    const long long unit = s / tpg;
    const int within = static_cast<int>(s - unit * tpg);
    int x = 0, i = within;
    if (split) {
      x = within % kXcds;
      i = within / kXcds;
    }
    const int at = (x / xc) * kax + i / ncx;
    const int ct = (x % xc) * ncx + i % ncx;
    if (at >= ka || ct >= nc) return false;
    int q, chunk = 0, P = 1;
    if (ns > 0 && unit < s_cp[ns]) {
      q = 0;
      while (unit >= s_cp[q + 1]) ++q;
      chunk = static_cast<int>(unit) - s_cp[q];
      P = s_cp[q + 1] - s_cp[q];
    } else {
      q = ns + static_cast<int>(unit - (ns > 0 ? s_cp[ns] : 0));
    }
    t.j = s_order[q];
    t.r_begin = s_lb[t.j];
    t.r_end = s_lb[t.j + 1];
    t.part = -1;
    if (P > 1) {  // chunk `chunk` of P equal step ranges
      const int st = (t.r_end - t.r_begin + KS - 1) / KS;
      const int per = (st + P - 1) / P;
      const int rb = t.r_begin + chunk * per * KS;
      t.r_end = min(t.r_end, rb + per * KS);
      t.r_begin = rb;
      t.part = (s_cp[q] + chunk) * ka * nc + at * nc + ct;
    }
    t.a0 = at * BM;
    t.c0 = ct * BN;
    t.nk = (t.r_end - t.r_begin + KS - 1) / KS;
    return true;
  }

  // Which slots this workgroup takes.  A slot costs its unit's contraction
  // steps.  Without a row split, tiles costing at least the mean work per
  // workgroup (the "heavy" tiles, a prefix of the list) get a workgroup each:
  // dealt round-robin, every workgroup that takes one of the largest groups'
  // tiles would also take its full share of the later ones (with Zipf-sized
  // groups on the 32768-row backward the busiest workgroup had 450 steps
  // against 264 on average).  The other slots are dealt in snake order among
  // the remaining workgroups.  Workgroups keep walking the list together, so
  // the ones running at the same time work on neighbouring tiles that share
  // their rows in L2 (contiguous per-workgroup ranges, also tried, lose that
  // and are 30 % slower).  With a row split no unit is heavy, and every slot
  // is dealt in snake order.  NT threads; uses s_wave; ends with a barrier.
  template <int NT, int KS>
  __device__ SlotSeq dealt_slots(const int* s_lb, const int* s_order, int gl, long long* s_wave) const {
    const long long G = gridDim.x;
    const long long b = blockIdx.x;
    if (slots <= G) return strided_slots(slots);
    if (ns > 0) return snake_slots(0, slots, G, b);
    long long mine = 0;
    for (int q = threadIdx.x; q < gl; q += NT) mine += tpg * steps_at<KS>(s_lb, s_order, q);
    const long long total = block_sum<NT>(mine, s_wave);
    long long heavy = 0;
    for (int q = threadIdx.x; q < gl; q += NT) heavy += steps_at<KS>(s_lb, s_order, q) * G >= total ? 1 : 0;
    heavy = block_sum<NT>(heavy, s_wave);
    long long H = heavy * tpg;
    if (H > G - 1) H = G - 1;
    if (H <= 0) return snake_slots(0, slots, G, b);
    if (b < H) return SlotSeq{b, 1, 1, 0, false};
    return snake_slots(H, slots, G - H, b - H);
  }
};

// Groups of the window, largest first (stable), into s_order; plain order
// when there are more than NT local groups (NT threads).  Ends with a barrier.
template <int NT = kThreads>
__device__ __forceinline__ void order_groups(const int* s_lb, int gl, int* s_order) {
  if (gl <= NT) {
    const int t = threadIdx.x;
    if (t < gl) {
      const int sz = s_lb[t + 1] - s_lb[t];
      int rank = 0;
      for (int i = 0; i < gl; ++i) {
        const int si = s_lb[i + 1] - s_lb[i];
        rank += (si > sz) || (si == sz && i < t);
      }
      s_order[rank] = t;
    }
  } else {
    for (int t = threadIdx.x; t < gl; t += NT) s_order[t] = t;
  }
  __syncthreads();
}

// Rows below L outside the window are written as +0 (rows >= L untouched),
// in tasks of kZeroRows rows shared by the whole grid (NT threads per workgroup).
template <int NT = kThreads>
__device__ __forceinline__ void zero_outside_window(void* out, int n, bool f32, const Window& win) {
  const int z1 = (win.lo + kZeroRows - 1) / kZeroRows;
  const int z2 = (win.L - win.hi + kZeroRows - 1) / kZeroRows;
  const int esz = f32 ? 4 : 2;
  const int cpr = n * esz / 16;
  for (int z = blockIdx.x; z < z1 + z2; z += gridDim.x) {
    int r0, r1;
    if (z < z1) {
      r0 = z * kZeroRows;
      r1 = min(r0 + kZeroRows, win.lo);
    } else {
      r0 = win.hi + (z - z1) * kZeroRows;
      r1 = min(r0 + kZeroRows, win.L);
    }
    u32x4_t* dst = reinterpret_cast<u32x4_t*>(static_cast<char*>(out) + static_cast<long long>(r0) * n * esz);
    const int nch = (r1 - r0) * cpr;
    for (int q = threadIdx.x; q < nch; q += NT) store16<true>(u32x4_t{0, 0, 0, 0}, dst + q);
  }
}

// ---------------------------------------------------------------- register-staged kernel (fallback)

// Two workgroups per CU; the contraction length may be any multiple of 8 and
// operands may exceed 4 GiB.  Tiles run one after another, each with its own
// double-buffered pipeline.
template <int MODE, int BM, int BN>
__global__ __launch_bounds__(kThreads, 2) void grouped_gemm_regs(KArgs p) {
  constexpr int WM = BM / 2, WN = BN / 2;
  constexpr int MI = WM / 32, NI = WN / 32;
  constexpr int A_EL = BM * BK, B_EL = BN * BK;
  __shared__ __attribute__((aligned(1024))) uint16_t s_tiles[2 * (A_EL + B_EL)];
  static_assert(4 * NI * kStageFloats * 2 <= 2 * (A_EL + B_EL), "epilogue staging must fit");
  __shared__ int s_lb[RD_MAX_GROUPS + 1];
  __shared__ int s_aux[RD_MAX_GROUPS + 1];
  __shared__ long long s_wave[kThreads / 64];

  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int wm_off = (wave >> 1) * WM, wn_off = (wave & 1) * WN;
  float* stage = reinterpret_cast<float*>(s_tiles) + wave * NI * kStageFloats;
  const Window win = build_local_bounds(p.gs, p.G, p.offp, p.gl, p.limp, p.m, s_lb, s_wave);

  if constexpr (MODE == kFwdNN || MODE == kFwdNT) {
    const int total_m = tile_prefix(s_lb, p.gl, BM, s_aux, s_wave);
    FwdTiles tl;
    tl.init(total_m, p.n, BN, p.k);
    for (long long s = blockIdx.x; s < tl.slots; s += gridDim.x) {
      FwdTiles::Tile t;
      if (!tl.get<BM, BN>(s, s_lb, s_aux, p.gl, p.k, t)) continue;
      const uint16_t* wj = p.b + static_cast<long long>(t.j) * p.k * p.n;
      f32x16_t acc[MI][NI];
#pragma unroll
      for (int mi = 0; mi < MI; ++mi)
#pragma unroll
        for (int ni = 0; ni < NI; ++ni) acc[mi][ni] = f32x16_t{};
      KOperand<BM> A{p.a, p.k, t.row0, t.row_end, p.k};
      if constexpr (MODE == kFwdNN) {
        MNOperand<BN> B{wj, p.n, 0, p.k, t.n0, p.n};
        k_loop<KOperand<BM>, MNOperand<BN>, MI, NI, A_EL, B_EL>(A, B, t.nk, s_tiles, acc, wm_off, wn_off);
      } else {
        KOperand<BN> B{wj, p.k, t.n0, p.n, p.k};
        k_loop<KOperand<BM>, KOperand<BN>, MI, NI, A_EL, B_EL>(A, B, t.nk, s_tiles, acc, wm_off, wn_off);
      }
      store_wave_tile<MI, NI>(acc, p.out, p.out_f32, p.n, t.row0 + wm_off, t.row_end, t.n0 + wn_off, p.n, stage);
      __syncthreads();  // staging area = pipeline buffers: drain before the next tile refills them
    }
    zero_outside_window(p.out, p.n, p.out_f32 != 0, win);
  } else {
    order_groups(s_lb, p.gl, s_aux);
    TransTiles tl;
    tl.init(p.gl, p.k, p.n, BM, BN);
    for (long long s = blockIdx.x; s < tl.slots; s += gridDim.x) {
      TransTiles::Tile t;
      if (!tl.get<BM, BN>(s, s_lb, s_aux, t)) continue;
      f32x16_t acc[MI][NI];
#pragma unroll
      for (int mi = 0; mi < MI; ++mi)
#pragma unroll
        for (int ni = 0; ni < NI; ++ni) acc[mi][ni] = f32x16_t{};
      MNOperand<BM> A{p.a, p.k, t.r_begin, t.r_end, t.a0, p.k};
      MNOperand<BN> B{p.b, p.n, t.r_begin, t.r_end, t.c0, p.n};
      k_loop<MNOperand<BM>, MNOperand<BN>, MI, NI, A_EL, B_EL>(A, B, t.nk, s_tiles, acc, wm_off, wn_off);
      char* dwj = static_cast<char*>(p.out) + static_cast<long long>(t.j) * p.k * p.n * (p.out_f32 ? 4 : 2);
      store_wave_tile<MI, NI>(acc, dwj, p.out_f32, p.n, t.a0 + wm_off, p.k, t.c0 + wn_off, p.n, stage);
      __syncthreads();
    }
  }
}

// ---------------------------------------------------------------- streamed buffer-to-LDS kernel

// fp8 K-contiguous operand: the bf16 machinery moves it as pairs of bytes
// (KS 16-bit elements = 2 * KS fp8 per stage row), only the fragment differs.
template <int ROWS, int KS, int NW = 4>
struct K8Dma : KDma<ROWS, KS, NW> {
  static constexpr int kFrag8Reads = 2;
  __device__ __forceinline__ static i32x8_t frag8(const uint16_t* tile, int r_base, int kk) {
    return KLayoutT<KS>::frag8(tile, r_base, kk);
  }
};

// fp8 MN-contiguous operand (the weight w [k, n] of the plain form): a stage
// is 2 * KS contraction rows of COLS fp8, moved as COLS / 2 16-bit elements
// by the bf16 machinery (MNLayout<COLS / 2> rows).  The fragment comes
// through the gfx950 8-bit LDS transpose read: within each 16-lane group,
// lanes 2e and 2e+1 name row e of an 8 x 16-byte block (bytes 0..7 and 8..15)
// and lane i receives byte i of each of the 8 rows (measured on the GPU).
// Four reads give lane l the 32 contraction rows 64*kk + 32*(l/32) .. +31 of
// column c_base + l % 32, in the order KLayoutT::frag8 gives the other
// operand.
template <int COLS, int KS, int NW = 4>
struct MN8Dma : MNDma<COLS / 2, 2 * KS, NW> {
  static constexpr int kFrag8Reads = 4;
  __device__ __forceinline__ static i32x8_t frag8(const uint16_t* tile, int c_base, int kk) {
    const int l = threadIdx.x & 63;
    const int q = l & 15;
    const int col = c_base + 16 * ((l >> 4) & 1) + 8 * (q & 1);  // fp8 column of this lane's 8 bytes
    const int row0 = 64 * kk + 32 * (l >> 5) + (q >> 1);
    typedef int i32x2_t __attribute__((ext_vector_type(2)));
    i32x2_t r[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const unsigned char* p = reinterpret_cast<const unsigned char*>(
                                   tile + MNLayout<COLS / 2>::offset(row0 + 8 * j, col >> 4)) + (col & 15);
      r[j] = __builtin_amdgcn_ds_read_tr8_b64_v2i32(RD_LDS(i32x2_t, p));
    }
    return i32x8_t{r[0].x, r[0].y, r[1].x, r[1].y, r[2].x, r[2].y, r[3].x, r[3].y};
  }
};

// Weight operand of the fused up-projection: the tile's BN columns are two
// strips of w [k, 2h], gate columns [c0, c0 + BN/2) and the matching up
// columns [h + c0, h + c0 + BN/2), stored as two MN-contiguous sub-tiles.
template <int BN, int KS, int NW = 4>
struct GluDma {
  using Half = MNDma<BN / 2, KS, NW>;
  static constexpr int kHalf = BN / 2;
  static constexpr int kFragReads = Half::kFragReads;
  static constexpr int kInstr = 2 * Half::kInstr;
  Half g, u;
  __device__ __forceinline__ void init(const uint16_t* base, long long rows_valid, int ld, int c0, int h, int wave) {
    g.init(base, rows_valid, ld, c0, wave);
    u.init(base, rows_valid, ld, h + c0, wave);
  }
  __device__ __forceinline__ void issue(uint32_t tile, int kt, int wave) const {
    g.issue(tile, kt, wave);
    u.issue(tile + KS * kHalf * 2, kt, wave);
  }
  __device__ __forceinline__ static bf16x8_t frag(const uint16_t* tile, int c_base, int ks) {
    return c_base < kHalf ? MNOperand<kHalf>::frag(tile, c_base, ks)
                          : MNOperand<kHalf>::frag(tile + KS * kHalf, c_base - kHalf, ks);
  }
};
template <int BN, int KS, int NW>
struct SplitCols<GluDma<BN, KS, NW>> : std::true_type {};

// MFMAs of one stage of fp8 operands: 2 * KS fp8 contraction elements, i.e.
// KS / 32 slices of the 32x32x64 fp8 MFMA (fp32 accumulation; operand
// format fields select OCP E4M3 for both operands, no block scaling).
// Fragments are double-buffered across the slices.
template <class OpA, class OpB, int MI, int NI, int KS>
__device__ __forceinline__ void mma_stage8(const uint16_t* ta, const uint16_t* tb, f32x16_t (&acc)[MI][NI],
                                           int wm_off, int wn_off) {
  constexpr int kSlices = KS / 32;
  i32x8_t af[2][MI], bfr[2][NI];
#pragma unroll
  for (int mi = 0; mi < MI; ++mi) af[0][mi] = OpA::frag8(ta, wm_off + mi * 32, 0);
#pragma unroll
  for (int ni = 0; ni < NI; ++ni) bfr[0][ni] = OpB::frag8(tb, wn_off + ni * 32, 0);
#pragma unroll
  for (int kk = 0; kk < kSlices; ++kk) {
    const int cur = kk & 1;
    if (kk + 1 < kSlices) {
#pragma unroll
      for (int mi = 0; mi < MI; ++mi) af[cur ^ 1][mi] = OpA::frag8(ta, wm_off + mi * 32, kk + 1);
#pragma unroll
      for (int ni = 0; ni < NI; ++ni) bfr[cur ^ 1][ni] = OpB::frag8(tb, wn_off + ni * 32, kk + 1);
    }
#pragma unroll
    for (int mi = 0; mi < MI; ++mi)
#pragma unroll
      for (int ni = 0; ni < NI; ++ni)
        acc[mi][ni] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(af[cur][mi], bfr[cur][ni], acc[mi][ni], 0, 0,
                                                                      0, 0, 0, 0);
    if (kk + 1 < kSlices)
      __builtin_amdgcn_sched_group_barrier(0x100, OpA::kFrag8Reads * MI + OpB::kFrag8Reads * NI, 0);
    __builtin_amdgcn_sched_group_barrier(0x008, MI * NI, 0);
    __builtin_amdgcn_sched_barrier(0);
  }
}

// Operands of one tile, per mode, loaded by NW waves.
template <int MODE, int BM, int BN, int KS, int NW>
struct StreamOps;
template <int BM, int BN, int KS, int NW>
struct StreamOps<kFwdNN, BM, BN, KS, NW> {
  using A = KDma<BM, KS, NW>;
  using B = MNDma<BN, KS, NW>;
  __device__ __forceinline__ static void make(const KArgs& p, const FwdTiles::Tile& t, int wave, A& a, B& b) {
    a.init(p.a + static_cast<long long>(t.row0) * p.k, t.row_end - t.row0, p.k, wave);
    b.init(p.b + static_cast<long long>(t.j) * p.k * p.n, p.k, p.n, t.n0, wave);
  }
};
template <int BM, int BN, int KS, int NW>
struct StreamOps<kFwdNT, BM, BN, KS, NW> {
  using A = KDma<BM, KS, NW>;
  using B = KDma<BN, KS, NW>;
  __device__ __forceinline__ static void make(const KArgs& p, const FwdTiles::Tile& t, int wave, A& a, B& b) {
    a.init(p.a + static_cast<long long>(t.row0) * p.k, t.row_end - t.row0, p.k, wave);
    b.init(p.b + static_cast<long long>(t.j) * p.k * p.n + static_cast<long long>(t.n0) * p.k, p.n - t.n0, p.k,
           wave);
  }
};
// fp8 trans_rhs: x [m, k] and w [g, n, k] as fp8; the kernel sees k / 2
// 16-bit elements per row (KArgs::k), so the bf16 addressing applies as is.
template <int BM, int BN, int KS, int NW>
struct StreamOps<kFwdNT8, BM, BN, KS, NW> {
  using A = K8Dma<BM, KS, NW>;
  using B = K8Dma<BN, KS, NW>;
  __device__ __forceinline__ static void make(const KArgs& p, const FwdTiles::Tile& t, int wave, A& a, B& b) {
    StreamOps<kFwdNT, BM, BN, KS, NW>::make(p, t, wave, a, b);
  }
};
// fp8 plain form: x [m, k] as k / 2 16-bit elements per row (KArgs::k) and
// w [g, k, n] as 2 * KArgs::k rows of n / 2 16-bit elements.
template <int BM, int BN, int KS, int NW>
struct StreamOps<kFwdNN8, BM, BN, KS, NW> {
  using A = K8Dma<BM, KS, NW>;
  using B = MN8Dma<BN, KS, NW>;
  __device__ __forceinline__ static void make(const KArgs& p, const FwdTiles::Tile& t, int wave, A& a, B& b) {
    a.init(p.a + static_cast<long long>(t.row0) * p.k, t.row_end - t.row0, p.k, wave);
    b.init(p.b + static_cast<long long>(t.j) * p.k * p.n, 2 * p.k, p.n / 2, t.n0 / 2, wave);
  }
};
// fp8 trans_ragged_dot: x [m, k] and dy [m, n] as fp8 rows of k / 2 and
// n / 2 16-bit elements; a stage is 2 * KS rows of the group.
template <int BM, int BN, int KS, int NW>
struct StreamOps<kTransTN8, BM, BN, KS, NW> {
  using A = MN8Dma<BM, KS, NW>;
  using B = MN8Dma<BN, KS, NW>;
  __device__ __forceinline__ static void make(const KArgs& p, const TransTiles::Tile& t, int wave, A& a, B& b) {
    a.init(p.a + static_cast<long long>(t.r_begin) * (p.k / 2), t.r_end - t.r_begin, p.k / 2, t.a0 / 2, wave);
    b.init(p.b + static_cast<long long>(t.r_begin) * (p.n / 2), t.r_end - t.r_begin, p.n / 2, t.c0 / 2, wave);
  }
};
template <int BM, int BN, int KS, int NW>
struct StreamOps<kTransTN, BM, BN, KS, NW> {
  using A = MNDma<BM, KS, NW>;
  using B = MNDma<BN, KS, NW>;
  __device__ __forceinline__ static void make(const KArgs& p, const TransTiles::Tile& t, int wave, A& a, B& b) {
    a.init(p.a + static_cast<long long>(t.r_begin) * p.k, t.r_end - t.r_begin, p.k, t.a0, wave);
    b.init(p.b + static_cast<long long>(t.r_begin) * p.n, t.r_end - t.r_begin, p.n, t.c0, wave);
  }
};

// Fused up-projection: x [m, k] and w [g, k, 2h]; the tile's gate columns
// start at t.n0 (KArgs::n is h).
template <int BM, int BN, int KS, int NW>
struct StreamOps<kFwdGLU, BM, BN, KS, NW> {
  using A = KDma<BM, KS, NW>;
  using B = GluDma<BN, KS, NW>;
  __device__ __forceinline__ static void make(const KArgs& p, const FwdTiles::Tile& t, int wave, A& a, B& b) {
    a.init(p.a + static_cast<long long>(t.row0) * p.k, t.row_end - t.row0, p.k, wave);
    b.init(p.b + static_cast<long long>(t.j) * p.k * 2 * p.n, p.k, 2 * p.n, t.n0, p.n, wave);
  }
};

// One persistent stream of contraction steps across all of a workgroup's
// tiles.  A producer walks the workgroup's tile list issuing buffer-to-LDS
// loads S-1 steps ahead of the consumer, crossing tile boundaries, so the
// next tile's first stages load while the current tile multiplies and its
// epilogue stores drain.  Step g lives in ring slot g % S.  Before step g the
// wave waits until at most (younger loads) vector-memory operations are in
// flight: loads complete in issue order, so step g's loads are then done
// whatever the pending stores do.  The barrier that follows also tells every
// wave that slot (g-1) % S is free, and the producer refills it.  A tile's
// epilogue stages its bf16 results in the slot of its last step.
// WGS workgroups share a CU (1, or 2 for the small-ring variant).
// MAXL bounds num_local for the LDS schedule arrays (a smaller bound frees
// LDS for a deeper ring; the host only picks such a variant when num_local
// fits).  The workgroup is WR x WC waves (each owns a BM/WR x BN/WC block of
// the tile): 2 x 2, or 8 waves (two per SIMD, so one wave's MFMAs issue
// while the other waits on a barrier or an LDS read).
// The zero rows of a window, written by the forward tiles while they run
// (the ZIL instance of grouped_gemm_stream; see there).  One wave's share:
// 1 KB chunks (64 lanes x 16 B) of the two contiguous ranges [0, lo) and
// [hi, L), every (grid waves)-th chunk from the wave's global index.  The
// false specialisation holds nothing, so the other instances compile as if
// it were not there.
template <bool ON>
struct WindowZeros {
  __device__ WindowZeros(const KArgs&, const Window&, int, int) {}
};
template <>
struct WindowZeros<true> {
  char* out;
  long long row, v1, v, next, end, stride, hi_off;
  __device__ WindowZeros(const KArgs& p, const Window& win, int nw, int wave) {
    out = static_cast<char*>(p.out);
    row = static_cast<long long>(p.n) * (p.out_f32 ? 4 : 2);
    v1 = static_cast<long long>(win.lo) * (row / 16);
    v = v1 + static_cast<long long>(win.L - win.hi) * (row / 16);
    end = (v + 63) / 64;
    stride = static_cast<long long>(gridDim.x) * nw;
    next = static_cast<long long>(blockIdx.x) * nw + wave;
    hi_off = static_cast<long long>(win.hi) * row;
  }
  __device__ __forceinline__ void chunk() {
    const long long q = next * 64 + (threadIdx.x & 63);
    if (q < v) store16<true>(u32x4_t{0, 0, 0, 0}, out + (q < v1 ? q * 16 : hi_off + (q - v1) * 16));
    next += stride;
  }
  // one chunk per contraction step, before the step's loads
  __device__ __forceinline__ void step() {
    if (next < end) chunk();
  }
  // what is left after the wave's last tile
  __device__ __forceinline__ void drain() {
    while (next < end) chunk();
  }
};

template <int MODE, int BM, int BN, int S, int KS, int WGS, int MAXL = RD_MAX_GROUPS, int WR = 2, int WC = 2,
          bool ZIL = false>
__global__ __launch_bounds__(WR * WC * 64, WGS) void grouped_gemm_stream(KArgs p) {
  constexpr int NW = WR * WC, NT = NW * 64;
  constexpr int WM = BM / WR, WN = BN / WC;
  constexpr int MI = WM / 32, NI = WN / 32;
  static_assert(MI * 32 == WM && NI * 32 == WN, "wave blocks are whole 32 x 32 MFMA blocks");
  constexpr int A_EL = BM * KS, B_EL = BN * KS, ST = A_EL + B_EL;
  constexpr int EPI = epilogue_batch(NI, ST, NW);
  // trans_ragged_dot stages bf16 results as bf16, EPI16 blocks at a time; a
  // wave's staging area covers either layout
  constexpr int EPI16 = is_trans(MODE) ? epilogue_batch16(NI, ST, NW) : EPI;
  constexpr int STAGE_HALVES = is_trans(MODE) && EPI16 * kStageHalves > 2 * EPI * kStageFloats
                                   ? EPI16 * kStageHalves
                                   : 2 * EPI * kStageFloats;  // per wave
  static_assert(NW * STAGE_HALVES <= ST, "epilogue staging must fit in one ring slot");
  static_assert(EPI >= 1 && NW * EPI * kStageFloats * 2 <= ST, "epilogue staging must fit in one ring slot");
  // the fused GLU tile: BN weight columns are BN/2 gate + BN/2 up, giving BN/2 output columns
  constexpr int TN = MODE == kFwdGLU ? BN / 2 : BN;
  constexpr int EPI_H = MODE == kFwdGLU ? epilogue_batch(NI / 2, ST, NW) : 1;
  static_assert(MODE != kFwdGLU || (NI % 2 == 0 && EPI_H >= 1 && EPI_H <= EPI), "GLU tiles pair gate and up blocks");
  // results are written once and read by a later kernel: non-temporal stores
  // leave them out of the caches' dirty lines, so no write-back is left over
  // for the next kernel to pay for (measured: the up-projection forward takes
  // 10 % less time after a trans_ragged_dot whose dW went out this way)
  constexpr bool kNtStores = true;
  using Ops = StreamOps<MODE, BM, BN, KS, NW>;
  using OpA = typename Ops::A;
  using OpB = typename Ops::B;
  using Tiles = typename std::conditional<is_trans(MODE), TransTiles, FwdTiles>::type;
  // contraction rows per stage in the tile lists (fp8 trans: 2 * KS rows of fp8 per stage)
  constexpr int KSTEP = MODE == kTransTN8 ? 2 * KS : KS;
  constexpr int L = OpA::kInstr + OpB::kInstr;  // loads per wave per step
  __shared__ __attribute__((aligned(1024))) uint16_t s_tiles[S * ST];
  __shared__ int s_lb[MAXL + 1];
  __shared__ int s_aux[MAXL + 1];
  __shared__ int s_cp[kMaxSplit + 2];
  __shared__ long long s_wave[NW];

  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int wm_off = (wave / WC) * WM, wn_off = (wave % WC) * WN;
  const Window win = build_local_bounds<NT>(p.gs, p.G, p.offp, p.gl, p.limp, p.m, s_lb, s_wave);

  // ZIL (forward tiles of calls with a window): rows below the limit
  // outside the window are written as +0 while the tiles run.  The rows
  // [0, lo) and [hi, L) form two contiguous ranges, cut into 1 KB chunks (64
  // lanes x 16 B) dealt round-robin over every wave of the grid; each wave
  // stores one chunk per contraction step, before the step's loads, so the
  // next step's load wait also covers it (loads complete in order among
  // themselves, so the wait's count stays right), and the rest after its
  // last tile.  The stores share the vector-memory path with the loads, so
  // the overlap is partial (the window+limit forward: 236 -> 225 us).  A
  // separate instance: the chunk state costs the other forward tiles SGPR
  // spills in their loop.
  constexpr bool kZil = ZIL && (MODE == kFwdNN || MODE == kFwdNT);
  WindowZeros<kZil> zeros(p, win, NW, wave);
  Tiles tl;
  if constexpr (is_trans(MODE)) {
    order_groups<NT>(s_lb, p.gl, s_aux);
    tl.init(p.gl, p.k, p.n, BM, BN);
    if ((MODE == kTransTN || MODE == kTransTN8) && p.ws != nullptr) {
      const long long part_bytes = static_cast<long long>(BM) * BN * 4;
      const long long cap = (p.ws_bytes - kSplitHeaderInts * 4) / part_bytes;
      int* header = static_cast<int*>(p.ws);
      if (blockIdx.x == 0 && threadIdx.x == 0) {
        header[1] = BM;
        header[2] = BN;
      }
      tl.template plan<NT, KSTEP, MODE == kTransTN8 ? 13 : 10>(s_lb, s_aux, p.gl, s_wave, s_cp, cap > 0 ? cap : 0,
                                                               p.per_cu > 0 ? p.per_cu : 1, header);
    }
  } else {
    const int total_m = tile_prefix<NT>(s_lb, p.gl, BM, s_aux, s_wave);
    tl.init(total_m, p.n, TN, p.k);
  }
  auto tile_at = [&](long long s, typename Tiles::Tile& t) -> bool {
    if constexpr (is_trans(MODE))
      return tl.template get<BM, BN, KSTEP>(s, s_lb, s_aux, t, s_cp);
    else
      return tl.template get<BM, TN, KS>(s, s_lb, s_aux, p.gl, p.k, t);
  };
  const uint32_t ring = lds_address(s_tiles);
  SlotSeq seq;
  if constexpr (is_trans(MODE))
    seq = tl.template dealt_slots<NT, KSTEP>(s_lb, s_aux, p.gl, s_wave);
  else
    seq = strided_slots(tl.slots);

  // producer state: its tile (slot ps), operands, next step
  long long pu = -1;  // producer: index into seq of its current tile
  int p_kt = 0, p_nk = 0;
  bool p_done = false;
  OpA pa;
  OpB pb;
  int issued = 0;
  auto produce = [&]() {
    while (!p_done && p_kt >= p_nk) {
      if (++pu >= seq.count) {
        p_done = true;
        break;
      }
      typename Tiles::Tile t;
      if (tile_at(seq.at(pu), t) && t.nk > 0) {
        Ops::make(p, t, wave, pa, pb);
        p_kt = 0;
        p_nk = t.nk;
      }
    }
    if (p_done) return;
    const uint32_t slot = ring + 2 * (issued % S) * ST;
    pa.issue(slot, p_kt, wave);
    pb.issue(slot + 2 * A_EL, p_kt, wave);
    ++p_kt;
    ++issued;
  };

#pragma unroll
  for (int i = 0; i < S - 1; ++i) produce();

  int g = 0;  // consumer step
  for (long long u = 0; u < seq.count; ++u) {
    typename Tiles::Tile t;
    if (!tile_at(seq.at(u), t)) continue;
    char* out;
    int r0, rlim, c0, clim = p.n;
    bool of32 = p.out_f32 != 0;
    long long ld = p.n;
    if constexpr (is_trans(MODE)) {
      if (t.part >= 0) {  // a row chunk of a split group: its fp32 partial tile [BM, BN]
        out = static_cast<char*>(p.ws) + kSplitHeaderInts * 4 + static_cast<long long>(t.part) * BM * BN * 4;
        of32 = true;
        ld = BN;
        r0 = wm_off;
        rlim = min(BM, p.k - t.a0);
        c0 = wn_off;
        clim = min(BN, p.n - t.c0);
      } else {
        out = static_cast<char*>(p.out) + static_cast<long long>(t.j) * p.k * p.n * (p.out_f32 ? 4 : 2);
        r0 = t.a0 + wm_off;
        rlim = p.k;
        c0 = t.c0 + wn_off;
      }
    } else {
      out = static_cast<char*>(p.out);
      r0 = t.row0 + wm_off;
      rlim = t.row_end;
      c0 = t.n0 + (MODE == kFwdGLU ? wn_off / 2 : wn_off);
    }
    if (t.nk == 0) {  // a local group with no rows: its dW tile is +0
      store_wave_zero<MI, NI>(out, p.out_f32, p.n, r0, rlim, c0, p.n);
      continue;
    }
    f32x16_t acc[MI][NI];
#pragma unroll
    for (int mi = 0; mi < MI; ++mi)
#pragma unroll
      for (int ni = 0; ni < NI; ++ni) acc[mi][ni] = f32x16_t{};
    for (int kt = 0; kt < t.nk; ++kt) {
      __builtin_amdgcn_sched_barrier(0);
      wait_ladder<L, S - 2>(issued - 1 - g);
      __builtin_amdgcn_s_barrier();
      __builtin_amdgcn_sched_barrier(0);
      const uint16_t* slot = s_tiles + (g % S) * ST;
      if constexpr (is_fp8(MODE)) {
        produce();
        __builtin_amdgcn_sched_barrier(0);
        mma_stage8<OpA, OpB, MI, NI, KS>(slot, slot + A_EL, acc, wm_off, wn_off);
      } else {
        StageFrags<OpA, OpB, MI, NI> fr;
        stage_frags(slot, slot + A_EL, fr, wm_off, wn_off);
        __builtin_amdgcn_sched_barrier(0);
        if constexpr (kZil) {
          zeros.step();
          __builtin_amdgcn_sched_barrier(0);
        }
        produce();
        __builtin_amdgcn_sched_barrier(0);
        mma_stage<OpA, OpB, MI, NI, KS>(slot, slot + A_EL, fr, acc, wm_off, wn_off);
      }
      ++g;
    }
    __builtin_amdgcn_sched_barrier(0);
    __builtin_amdgcn_s_barrier();  // every wave is done with the last step's slot
    __builtin_amdgcn_sched_barrier(0);
    float* stage = reinterpret_cast<float*>(s_tiles + ((g + S - 1) % S) * ST + wave * STAGE_HALVES);
    if constexpr (MODE == kFwdGLU)
      store_glu_tile<MI, NI, EPI_H, EPI_H, kNtStores>(acc, p.out, p.out2, p.n, r0, rlim, c0, stage);
    else
      store_wave_tile<MI, NI, EPI, 0, NI, kNtStores, is_trans(MODE), EPI16>(acc, out, of32, ld, r0, rlim, c0, clim,
                                                                            stage);
  }
  if constexpr (kZil) {
    zeros.drain();
  } else if constexpr (!is_trans(MODE)) {
    zero_outside_window<NT>(p.out, p.n, p.out_f32 != 0, win);
  }
  if constexpr (MODE == kFwdGLU)
    if (p.out2 != nullptr) zero_outside_window<NT>(p.out2, 2 * p.n, false, win);
}

// ---------------------------------------------------------------- ping-pong 256 x 256 kernel

// s_waitcnt immediate for "lgkmcnt(0)" leaving vmcnt/expcnt unconstrained.
constexpr int kLgkm0 = 0xF | (0x3 << 14) | (0x7 << 4);

// Fragments of one phase: NSL slices of the 32x32x16 MFMA.
template <int MI, int NI, int NSL>
struct PPFrags {
  bf16x8_t a[NSL][MI], b[NSL][NI];
};

// 256 x 256 output tiles on eight waves that take turns (ping-pong).  The
// waves form two groups of four, one wave of each group per SIMD (a
// workgroup's waves w and w + 4 share a SIMD, measured).  Each KS-deep stage
// of the buffer-to-LDS ring (whole 128-byte rows of a contraction-contiguous
// operand at KS = 64) is consumed in two halves, and every half has two
// phases separated by workgroup barriers: a memory phase (the half's LDS ->
// register fragment reads) and a compute phase (its MFMAs from registers).
// Group B runs one phase behind group A, so in every phase one wave per SIMD
// issues MFMAs back to back while its SIMD partner reads LDS:
//
//   phase   0       1       2       3       4    ...
//   A      M(0a)   C(0a)   M(0b)   C(0b)   M(1a)
//   B       -      M(0a)   C(0a)   M(0b)   C(0b)
//
// Ring discipline (S slots, stage g in slot g % S): stage g's slot is read
// last in phase 4g + 3, so its refill with stage g + S starts in phase
// 4g + 4 (group A at the start of M((g+1)a), group B at the start of its
// compute phase C(gb)); group B's prologue loads one stage more than A's.
// Stage g + 1 must have landed by phase 4g + 4: each wave waits for its own
// share before the barrier that opens that phase, and finishes its LDS reads
// (lgkmcnt 0) before the barrier that closes each memory phase.  Each wave
// owns a 64 x 128 block (rows 64 (w / 2), columns 128 (w % 2)): group A holds
// the tile's first 128 rows, so a forward tile with at most 128 valid rows
// leaves group B's MFMAs and fragment reads out.  A tile's epilogue runs in
// the wave's next memory phase (staged through a private LDS area), while
// the other group multiplies.
template <int MODE, int S, int KS, int MAXL = RD_MAX_GROUPS>
__global__ __launch_bounds__(512, 1) void grouped_gemm_pp(KArgs p) {
  constexpr int BM = 256, BN = 256, NW = 8, NT = NW * 64;
  constexpr int WM = 64, WN = 128, MI = WM / 32, NI = WN / 32;
  constexpr int HALVES = 2, NSL = KS / 16 / HALVES;  // phases per stage, MFMA slices per phase
  constexpr int A_EL = BM * KS, B_EL = BN * KS, ST = A_EL + B_EL;
  constexpr int EPI16 = 2;  // bf16 results: blocks staged per LDS round trip
  constexpr int STAGE_F = (kStageHalves * EPI16 + 1) / 2 > kStageFloats ? (kStageHalves * EPI16 + 1) / 2
                                                                         : kStageFloats;  // floats per wave
  static_assert(STAGE_F % 4 == 0 && NSL >= 1, "staging areas stay 16-byte aligned");
  constexpr bool kNtStores = true;
  using Ops = StreamOps<MODE, BM, BN, KS, NW>;
  using OpA = typename Ops::A;
  using OpB = typename Ops::B;
  using Tiles = typename std::conditional<is_trans(MODE), TransTiles, FwdTiles>::type;
  constexpr int L = OpA::kInstr + OpB::kInstr;  // loads per wave per stage
  static_assert(S >= 2 && (S - 1) * L <= 63, "ring depth");
  __shared__ __attribute__((aligned(1024))) uint16_t s_tiles[S * ST];
  __shared__ __attribute__((aligned(16))) float s_stage[NW * STAGE_F];
  __shared__ int s_lb[MAXL + 1];
  __shared__ int s_aux[MAXL + 1];
  __shared__ long long s_wave[NW];

  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int grp = wave >> 2;
  const int wm_off = (wave >> 1) * WM, wn_off = (wave & 1) * WN;
  float* stage = s_stage + wave * STAGE_F;
  const Window win = build_local_bounds<NT>(p.gs, p.G, p.offp, p.gl, p.limp, p.m, s_lb, s_wave);

  Tiles tl;
  if constexpr (is_trans(MODE)) {
    order_groups<NT>(s_lb, p.gl, s_aux);
    tl.init(p.gl, p.k, p.n, BM, BN);
  } else {
    const int total_m = tile_prefix<NT>(s_lb, p.gl, BM, s_aux, s_wave);
    tl.init(total_m, p.n, BN, p.k);
  }
  auto tile_at = [&](long long s, typename Tiles::Tile& t) -> bool {
    if constexpr (is_trans(MODE))
      return tl.template get<BM, BN, KS>(s, s_lb, s_aux, t);
    else
      return tl.template get<BM, BN, KS>(s, s_lb, s_aux, p.gl, p.k, t);
  };
  const uint32_t ring = lds_address(s_tiles);
  SlotSeq seq;
  if constexpr (is_trans(MODE))
    seq = tl.template dealt_slots<NT, KS>(s_lb, s_aux, p.gl, s_wave);
  else
    seq = strided_slots(tl.slots);

  // producer: this wave's share of every stage, walking the tile list ahead of the consumer
  long long pu = -1;  // producer: index into seq of its current tile
  int p_kt = 0, p_nk = 0;
  bool p_done = false;
  OpA pa;
  OpB pb;
  int issued = 0;
  auto produce = [&]() {
    while (!p_done && p_kt >= p_nk) {
      if (++pu >= seq.count) {
        p_done = true;
        break;
      }
      typename Tiles::Tile t;
      if (tile_at(seq.at(pu), t) && t.nk > 0) {
        Ops::make(p, t, wave, pa, pb);
        p_kt = 0;
        p_nk = t.nk;
      }
    }
    if (p_done) return;
    const uint32_t slot = ring + 2 * (issued % S) * ST;
    pa.issue(slot, p_kt, wave);
    pb.issue(slot + 2 * A_EL, p_kt, wave);
    ++p_kt;
    ++issued;
  };
  auto barrier = []() {
    __builtin_amdgcn_sched_barrier(0);
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_sched_barrier(0);
  };

#pragma unroll
  for (int i = 0; i < S - 1; ++i) produce();
  if (grp == 1) produce();                              // group B issues its stage-(S-1) share up front
  if (issued > 0) wait_ladder<L, S - 1>(issued - 1);  // stage 0 of this wave landed
  barrier();
  if (grp == 1) barrier();  // group B runs one phase behind

  int g = 0;  // consumer stage
  for (long long u = 0; u < seq.count; ++u) {
    typename Tiles::Tile t;
    if (!tile_at(seq.at(u), t)) continue;
    char* out;
    int r0, rlim, c0;
    if constexpr (is_trans(MODE)) {
      out = static_cast<char*>(p.out) + static_cast<long long>(t.j) * p.k * p.n * (p.out_f32 ? 4 : 2);
      r0 = t.a0 + wm_off;
      rlim = p.k;
      c0 = t.c0 + wn_off;
    } else {
      out = static_cast<char*>(p.out);
      r0 = t.row0 + wm_off;
      rlim = t.row_end;
      c0 = t.n0 + wn_off;
    }
    if (t.nk == 0) {  // a local group with no rows: its dW tile is +0
      store_wave_zero<MI, NI>(out, p.out_f32, p.n, r0, rlim, c0, p.n);
      continue;
    }
    if (r0 >= rlim) {
      // this wave's rows lie past the tile's valid rows: only its share of the loads, the waits and
      // the barriers, so that its SIMD partner multiplies alone
      for (int kt = 0; kt < t.nk; ++kt) {
#pragma unroll
        for (int h = 0; h < HALVES; ++h) {
          __builtin_amdgcn_sched_barrier(0);
          if (grp == 0 && h == 0) produce();
          __builtin_amdgcn_sched_barrier(0);
          const bool more = issued > g + 1;
          if (grp == 1 && h == HALVES - 1 && more) wait_ladder<L, S - 1>(issued - 2 - g);
          barrier();
          if (grp == 1 && h == HALVES - 1) produce();
          __builtin_amdgcn_sched_barrier(0);
          if (grp == 0 && h == HALVES - 1 && more) wait_ladder<L, S - 1>(issued - 2 - g);
          barrier();
        }
        ++g;
      }
      continue;
    }
    f32x16_t acc[MI][NI];
#pragma unroll
    for (int mi = 0; mi < MI; ++mi)
#pragma unroll
      for (int ni = 0; ni < NI; ++ni) acc[mi][ni] = f32x16_t{};
    for (int kt = 0; kt < t.nk; ++kt) {
      const uint16_t* slot = s_tiles + (g % S) * ST;
#pragma unroll
      for (int h = 0; h < HALVES; ++h) {
        // ---- memory phase of half h of stage g
        __builtin_amdgcn_sched_barrier(0);
        if (grp == 0 && h == 0) produce();  // refill the slot stage g - 1 left
        __builtin_amdgcn_sched_barrier(0);
        PPFrags<MI, NI, NSL> fr;
#pragma unroll
        for (int q = 0; q < NSL; ++q) {
#pragma unroll
          for (int mi = 0; mi < MI; ++mi) fr.a[q][mi] = OpA::frag(slot, wm_off + mi * 32, h * NSL + q);
#pragma unroll
          for (int ni = 0; ni < NI; ++ni) fr.b[q][ni] = OpB::frag(slot + A_EL, wn_off + ni * 32, h * NSL + q);
        }
        __builtin_amdgcn_sched_barrier(0);
        __builtin_amdgcn_s_waitcnt(kLgkm0);  // fragments in registers before the slot may be refilled
        const bool more = issued > g + 1;
        if (grp == 1 && h == HALVES - 1 && more) wait_ladder<L, S - 1>(issued - 2 - g);  // stage g + 1 landed
        barrier();
        // ---- compute phase of half h of stage g
        if (grp == 1 && h == HALVES - 1) produce();  // refill the slot stage g - 1 left
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int q = 0; q < NSL; ++q)
#pragma unroll
          for (int mi = 0; mi < MI; ++mi)
#pragma unroll
            for (int ni = 0; ni < NI; ++ni)
              acc[mi][ni] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fr.a[q][mi], fr.b[q][ni], acc[mi][ni], 0, 0, 0);
        __builtin_amdgcn_sched_barrier(0);
        if (grp == 0 && h == HALVES - 1 && more) wait_ladder<L, S - 1>(issued - 2 - g);
        barrier();
      }
      ++g;
    }
    // epilogue: the start of this wave's next memory phase, while the other group multiplies
    store_wave_tile<MI, NI, 1, 0, NI, kNtStores, true, EPI16>(acc, out, p.out_f32, p.n, r0, rlim, c0, p.n, stage);
  }
  if (grp == 0) barrier();  // group A matches group B's leading barrier
  if constexpr (!is_trans(MODE)) zero_outside_window<NT>(p.out, p.n, p.out_f32 != 0, win);
}

// ---------------------------------------------------------------- decode: split contraction

// ragged_dot with a few rows per group (decode: ~5 rows per expert) is a
// stream of expert weights; its speed is set by how evenly the weight bytes
// are spread over the CUs and by how little else interrupts the stream.
// Work is counted in steps: a block is (32-row block of a group, NW columns)
// and has k / 16 steps of 16 contraction rows.  The grid splits the
// concatenated step list into equal contiguous ranges, one per workgroup
// (so every CU streams the same number of weight bytes), and a range crosses
// block boundaries wherever they fall.  A workgroup keeps the fp32 sums of
// the blocks its range touches in registers (two at a time) and writes them,
// for the block's valid rows only, when its range is done: a store in flight
// would otherwise hold the next load wait (the counter does not tell loads
// from stores).  decode_streamk_reduce adds the partial sums of each block
// in workgroup order (deterministic: a bf16 result is the RNE of the f32 one)
// and applies the window and limit rules.  Per step, wave w loads 16 x 16 B
// of the row block (lanes 0..15) and NB KB of the weight slab; the slab is
// stored as it sits in memory (MNLayout) and fed to the MFMA through the LDS
// transpose read.
constexpr int kDecKS = 16;  // contraction rows per step: one MFMA k-slice
constexpr int kDecBM = 32;  // rows per block: one MFMA row block

// The step split shared by both decode kernels.
struct StepSplit {
  int nnc, spb;   // column strips, steps per block
  long long per;  // steps per workgroup
  __device__ __forceinline__ void init(int total_m, int n, int nw, int k, int grid) {
    nnc = n / nw;
    spb = k / kDecKS;
    const long long total = static_cast<long long>(total_m) * nnc * spb;
    per = (total + grid - 1) / grid;
    if (per < 1) per = 1;
  }
};

template <int NB, int S>
__global__ __launch_bounds__(kThreads, 1) void decode_streamk_gemm(KArgs p, float* __restrict__ ws, int seg_max) {
  constexpr int NW = 128 * NB;                   // block columns: 4 waves x NB MFMA blocks of 32
  constexpr int A_BYTES = kDecBM * kDecKS * 2;   // 1 KB
  constexpr int B_BYTES = kDecKS * NW * 2;
  constexpr int ST = A_BYTES + B_BYTES;          // bytes per ring slot
  constexpr int BI = B_BYTES / 4096;             // 1 KB weight loads per wave per step (= NB)
  constexpr int L = BI + 1;                      // loads per wave per step
  static_assert(BI * 4096 == B_BYTES, "weight step must split into 1 KB slices per wave");
  __shared__ __attribute__((aligned(1024))) char s_ring[S * ST];
  __shared__ int s_lb[RD_MAX_GROUPS + 1];
  __shared__ int s_aux[RD_MAX_GROUPS + 1];
  __shared__ long long s_wave[kThreads / 64];

  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  build_local_bounds(p.gs, p.G, p.offp, p.gl, p.limp, p.m, s_lb, s_wave);
  const int total_m = tile_prefix(s_lb, p.gl, kDecBM, s_aux, s_wave);
  StepSplit sp;
  sp.init(total_m, p.n, NW, p.k, gridDim.x);
  const long long total = static_cast<long long>(total_m) * sp.nnc * sp.spb;
  const long long s_begin = static_cast<long long>(blockIdx.x) * sp.per;
  const long long s_end = min(s_begin + sp.per, total);
  if (s_begin >= s_end) return;  // uniform: this workgroup has no steps
  const long long first_blk = s_begin / sp.spb;

  struct Block {
    int j, row0, nrows, n0;
  };
  auto block_at = [&](long long i, Block& d) {
    const int mt = static_cast<int>(i / sp.nnc);
    d.n0 = static_cast<int>(i % sp.nnc) * NW;
    d.j = upper_index(s_aux, p.gl, mt);
    d.row0 = s_lb[d.j] + (mt - s_aux[d.j]) * kDecBM;
    d.nrows = min(kDecBM, s_lb[d.j + 1] - d.row0);
  };

  const uint32_t ring = lds_address(s_ring);
  const int nsteps = static_cast<int>(s_end - s_begin);
  const int kt0 = static_cast<int>(s_begin - first_blk * sp.spb);  // step of the first block to start at
  // producer: steps issued, current block and step in it, the block's buffer
  // resources and per-lane offsets (no divisions per step)
  int issued = 0, p_kt = kt0;
  long long p_blk = first_blk;
  bool p_new = true;
  u32x4_t ra, rb;
  uint32_t va = 0, vb[BI];
  auto produce = [&]() {
    if (issued >= nsteps) return;
    if (p_kt == sp.spb) {
      ++p_blk;
      p_kt = 0;
      p_new = true;
    }
    if (p_new) {
      Block d;
      block_at(p_blk, d);
      // rows past the block's valid rows read as zeros (buffer range check)
      ra = uniform(make_rsrc(p.a + static_cast<long long>(d.row0) * p.k,
                             static_cast<unsigned long long>(d.nrows) * p.k * 2));
      rb = uniform(make_rsrc(p.b + static_cast<long long>(d.j) * p.k * p.n,
                             static_cast<unsigned long long>(p.k) * p.n * 2));
      const int c = wave * 16 + (lane & 15);  // row-block chunk: row c / 2, 16-byte half c % 2
      va = static_cast<uint32_t>(c >> 1) * p.k * 2 + (c & 1) * 16;
#pragma unroll
      for (int q = 0; q < BI; ++q) {
        const int cq = (wave * BI + q) * 64 + lane;
        const int row = cq / (NW / 8), slot = cq % (NW / 8);
        vb[q] = static_cast<uint32_t>(row) * p.n * 2 + (d.n0 + ((slot ^ MNLayout<NW>::swz(row)) << 3)) * 2;
      }
      p_new = false;
    }
    const uint32_t slot = ring + (issued % S) * ST;
    const int kr = p_kt * kDecKS;
    if (lane < 16) dma16(ra, slot + wave * 256, va, uniform(static_cast<uint32_t>(kr) * 2));
    const uint32_t sb = uniform(static_cast<uint32_t>(kr) * p.n * 2);
#pragma unroll
    for (int q = 0; q < BI; ++q) dma16_nt(rb, slot + A_BYTES + (wave * BI + q) * 1024, vb[q], sb);
    ++p_kt;
    ++issued;
  };

  // Partial sums of block segment seg, valid rows only: lane l holds column
  // l % 32 of rows 8 * (v / 4) + 4 * (l / 32) + v % 4.
  auto store_partials = [&](const f32x16_t (&v)[NB], long long blk, long long seg) {
    if (seg >= seg_max) return;  // cannot happen: seg_max bounds the blocks one range touches
    Block d;
    block_at(blk, d);
    float* dst = ws + ((static_cast<long long>(blockIdx.x) * seg_max + seg) * kDecBM) * NW + wave * NB * 32 +
                 (lane & 31);
#pragma unroll
    for (int jb = 0; jb < 4; ++jb) {
      if (8 * jb >= d.nrows) break;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int r = 8 * jb + 4 * (lane >> 5) + i;
        if (r < d.nrows) {
#pragma unroll
          for (int nb = 0; nb < NB; ++nb) dst[r * NW + nb * 32] = v[nb][4 * jb + i];
        }
      }
    }
  };

#pragma unroll
  for (int i = 0; i < S - 1; ++i) produce();

  f32x16_t acc[NB], prev[NB];
#pragma unroll
  for (int nb = 0; nb < NB; ++nb) acc[nb] = f32x16_t{};
  long long prev_blk = -1, c_blk = first_blk;
  int c_kt = kt0;
  for (int g = 0; g < nsteps; ++g) {
    __builtin_amdgcn_sched_barrier(0);
    wait_ladder<L, S - 2>(issued - 1 - g);
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_sched_barrier(0);
    produce();
    const char* slot = s_ring + (g % S) * ST;
    const bf16x8_t af = *reinterpret_cast<const bf16x8_t*>(slot + (((lane & 31) << 1) + (lane >> 5)) * 16);
    const uint16_t* tb = reinterpret_cast<const uint16_t*>(slot + A_BYTES);
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) {
      const bf16x8_t bf = MNOperand<NW>::frag(tb, (wave * NB + nb) * 32, 0);
      acc[nb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af, bf, acc[nb], 0, 0, 0);
    }
    if (++c_kt == sp.spb && g + 1 < nsteps) {  // a block ends inside the range
      if (prev_blk >= 0) store_partials(prev, prev_blk, prev_blk - first_blk);  // a third block: rare
#pragma unroll
      for (int nb = 0; nb < NB; ++nb) {
        prev[nb] = acc[nb];
        acc[nb] = f32x16_t{};
      }
      prev_blk = c_blk;
      ++c_blk;
      c_kt = 0;
    }
  }
  if (prev_blk >= 0) store_partials(prev, prev_blk, prev_blk - first_blk);
  store_partials(acc, c_blk, c_blk - first_blk);
}

// out[r, :] = sum of the partial sums of r's block, in workgroup order, for
// rows of the window; +0 for the other rows below L; rows >= L untouched.
template <int NB>
__global__ __launch_bounds__(kThreads) void decode_streamk_reduce(KArgs p, const float* __restrict__ ws, int seg_max,
                                                                  int grid) {
  constexpr int NW = 128 * NB;
  __shared__ int s_lb[RD_MAX_GROUPS + 1];
  __shared__ int s_aux[RD_MAX_GROUPS + 1];
  __shared__ long long s_wave[kThreads / 64];
  const Window win = build_local_bounds(p.gs, p.G, p.offp, p.gl, p.limp, p.m, s_lb, s_wave);
  const int total_m = tile_prefix(s_lb, p.gl, kDecBM, s_aux, s_wave);
  StepSplit sp;
  sp.init(total_m, p.n, NW, p.k, grid);
  const int cpr = p.n / 8;
  const long long total = static_cast<long long>(win.L) * cpr;
  for (long long e = static_cast<long long>(blockIdx.x) * kThreads + threadIdx.x; e < total;
       e += static_cast<long long>(gridDim.x) * kThreads) {
    const int r = static_cast<int>(e / cpr);
    const int c = static_cast<int>(e - static_cast<long long>(r) * cpr) * 8;
    f32x4_t lo = f32x4_t{0.f, 0.f, 0.f, 0.f}, hi = lo;
    if (r >= win.lo && r < win.hi) {
      const int j = upper_index(s_lb, p.gl, r);
      const int mt = s_aux[j] + (r - s_lb[j]) / kDecBM, rr = (r - s_lb[j]) % kDecBM;
      const int nc = c / NW;
      const long long i = static_cast<long long>(mt) * sp.nnc + nc;
      const long long b0 = i * sp.spb / sp.per, b1 = ((i + 1) * sp.spb - 1) / sp.per;
      for (long long b = b0; b <= b1; ++b) {
        const long long seg = i - b * sp.per / sp.spb;
        if (b >= grid || seg >= seg_max) break;  // cannot happen (see decode_streamk_gemm)
        const float* src = ws + ((b * seg_max + seg) * kDecBM + rr) * NW + (c - nc * NW);
        lo += *reinterpret_cast<const f32x4_t*>(src);
        hi += *reinterpret_cast<const f32x4_t*>(src + 4);
      }
    }
    const long long o = static_cast<long long>(r) * p.n + c;
    if (p.out_f32) {
      *reinterpret_cast<f32x4_t*>(static_cast<float*>(p.out) + o) = lo;
      *reinterpret_cast<f32x4_t*>(static_cast<float*>(p.out) + o + 4) = hi;
    } else {
      *reinterpret_cast<uint4*>(static_cast<uint16_t*>(p.out) + o) =
          make_uint4(pack_bf16x2(lo[0], lo[1]), pack_bf16x2(lo[2], lo[3]), pack_bf16x2(hi[0], hi[1]),
                     pack_bf16x2(hi[2], hi[3]));
    }
  }
}

// Second pass of the trans_ragged_dot row split: every element of dW[j] of
// each split group j is the sum of its P fp32 partials, added in chunk order
// (0, 1, ..., P - 1) and rounded once.  The plan comes from the workspace
// header the GEMM's workgroup 0 wrote: ns, the tile shape, then (j, P, first
// chunk) per split group.  Eight columns per thread (n % 8 == 0).  Workgroups
// of 1024 threads, one per CU: the launch costs little when nothing was split.
constexpr int kReduceThreads = 1024;
__global__ __launch_bounds__(kReduceThreads) void trans_split_reduce(const int* header, long long ws_bytes, void* out,
                                                               int out_f32, int k, int n, int gl) {
  const int ns = header[0];
  const int BM = header[1], BN = header[2];
  // a header the GEMM did not write in full reads as no split
  if (ns <= 0 || ns > kMaxSplit || BM <= 0 || BN <= 0 || BM % 32 != 0 || BN % 32 != 0) return;
  const int ka = (k + BM - 1) / BM, nc = (n + BN - 1) / BN;
  const long long cap = (ws_bytes - kSplitHeaderInts * 4) / (static_cast<long long>(BM) * BN * 4);
  const float* parts = reinterpret_cast<const float*>(header + kSplitHeaderInts);
  const int cpr = n / 8;
  const long long per_group = static_cast<long long>(k) * cpr;
  const long long total = per_group * ns;
  for (long long e = static_cast<long long>(blockIdx.x) * kReduceThreads + threadIdx.x; e < total;
       e += static_cast<long long>(gridDim.x) * kReduceThreads) {
    const int i = static_cast<int>(e / per_group);
    const long long rem = e - i * per_group;
    const int a = static_cast<int>(rem / cpr);
    const int c = static_cast<int>(rem - static_cast<long long>(a) * cpr) * 8;
    const int j = header[3 + 3 * i], P = header[4 + 3 * i], cp = header[5 + 3 * i];
    const long long tiles = static_cast<long long>(ka) * nc;
    if (j < 0 || j >= gl || P < 1 || cp < 0 || (static_cast<long long>(cp) + P) * tiles > cap) continue;
    const long long tile = static_cast<long long>(a / BM) * nc + c / BN;
    const long long off = static_cast<long long>(a % BM) * BN + c % BN;
    const float* src = parts + (cp * tiles + tile) * BM * BN + off;
    f32x4_t lo = __builtin_nontemporal_load(reinterpret_cast<const f32x4_t*>(src));
    f32x4_t hi = __builtin_nontemporal_load(reinterpret_cast<const f32x4_t*>(src + 4));
    for (int ch = 1; ch < P; ++ch) {
      src += tiles * BM * BN;
      lo += __builtin_nontemporal_load(reinterpret_cast<const f32x4_t*>(src));
      hi += __builtin_nontemporal_load(reinterpret_cast<const f32x4_t*>(src + 4));
    }
    const long long o = (static_cast<long long>(j) * k + a) * n + c;
    if (out_f32) {
      store16<true>(lo, static_cast<float*>(out) + o);
      store16<true>(hi, static_cast<float*>(out) + o + 4);
    } else {
      store16<true>(u32x4_t{pack_bf16x2(lo[0], lo[1]), pack_bf16x2(lo[2], lo[3]), pack_bf16x2(hi[0], hi[1]),
                            pack_bf16x2(hi[2], hi[3])},
                    static_cast<uint16_t*>(out) + o);
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
  a.out2 = p.out2;
  return a;
}

int grid_size(long long work_items, int per_cu) {
  long long cap = static_cast<long long>(device_cu_count()) * per_cu;
  long long g = work_items < cap ? work_items : cap;
  if (g >= kXcds) g -= g % kXcds;
  return static_cast<int>(g < 1 ? 1 : g);
}

// Tile shapes (BM x BN, LDS stages) of the buffer-to-LDS pipeline.  kT shapes
// run 4 waves in a 2 x 2 layout (the x2 / x3 ones two or three workgroups per
// CU), kW shapes 8 waves sharing one ring, kP the ping-pong kernel; larger
// wave tiles read fewer LDS bytes per MFMA, smaller BM wastes fewer MFMA rows
// on short groups.
enum Tile { kT64x128 = 0, kT128x128 = 1, kT128x256 = 2, kT256x256 = 3, kT128x128x2 = 4, kT64x64 = 5, kT256x256k32 = 6,
            kT128x256k32 = 7, kT128x256x2 = 8, kT128x128k32x2 = 9, kT128x128x3 = 10, kT256x128x2 = 11,
            kT128x256s3x2 = 12, kW256x256 = 13, kW128x256 = 14, kW256x256k64 = 15, kW128x512 = 16, kW128x256k32 = 17, kP256x256 = 18, kTileCount };

// Output tile and workgroups per CU of each shape (as launch_tile launches them).
struct TileShape {
  int bm, bn, wgs;
};
constexpr TileShape kTileShapes[kTileCount] = {
    {64, 128, 1},  {128, 128, 1}, {128, 256, 1}, {256, 256, 1}, {128, 128, 2}, {64, 64, 1},   {256, 256, 1},
    {128, 256, 1}, {128, 256, 2}, {128, 128, 2}, {128, 128, 3}, {256, 128, 2}, {128, 256, 2}, {256, 256, 1},
    {128, 256, 1}, {256, 256, 1}, {128, 512, 1}, {128, 256, 1}, {256, 256, 1}};
TileShape tile_shape(int tile) { return kTileShapes[tile >= 0 && tile < kTileCount ? tile : kT128x128]; }

// Tuning overrides set through rd_tune_set (tile sweeps only): a forced
// forward / trans tile shape (-1: the host heuristic) and the decode path
// switch (1 on, 0 off).  Plain atomics: a call reads each once.
std::atomic<int> g_tune[3] = {{-1}, {-1}, {1}};

int forced_tile(int which) {
  const int t = g_tune[which].load(std::memory_order_relaxed);
  return (t >= 0 && t < kTileCount) ? t : -1;
}

// Forward shape from what the host knows (never the device-resident group
// sizes): m / num_local bounds the mean rows per local group.  Decode-sized
// groups take a 64-row tile (when no workspace allows the split-contraction
// path).  trans_rhs calls and long groups take 128 x 256 tiles of eight
// waves sharing a 3 x 64-deep ring (two waves per SIMD).  Groups of at most
// 256 rows (mean), where streaming the weights dominates, take 128 x 512
// tiles of eight waves when n allows (each x row block is read by half as
// many tiles, each weight row is read 1 KB at a time), else two 4-wave
// 128 x 256 workgroups per CU (one multiplies while the other drains its
// stores).  Chosen from sweeps of every shape on the up-projection,
// backward, window+limit and decode workloads.
int pick_forward_tile(const GemmProblem& p, bool trans_rhs) {
  const int forced = forced_tile(RD_TUNE_FWD_TILE);
  if (forced >= 0) return forced;
  const long long avg_rows = p.m / (p.num_local > 0 ? p.num_local : 1);
  if (avg_rows <= 48) return kT64x128;
  if (p.n < 256) return kT128x128;
  if (trans_rhs) return kW128x256;
  if (avg_rows <= 256) return p.n % 512 == 0 ? kW128x512 : kT128x256x2;
  return kW128x256;
}

// trans_ragged_dot: the contraction runs over a group's rows.  Two
// co-resident 128 x 256 workgroups per CU with 3-slot rings of 32-deep stages
// (one workgroup multiplies while the other drains its dW stores).
int pick_trans_tile(const GemmProblem& p) {
  const int forced = forced_tile(RD_TUNE_TRANS_TILE);
  if (forced >= 0) return forced;
  return p.k >= 128 && p.n >= 256 ? kT128x256s3x2 : kT128x128x2;
}

KArgs with_per_cu(KArgs a, int grid) {
  const int cus = device_cu_count();
  a.per_cu = (grid + cus - 1) / cus;
  return a;
}

template <int MODE, int BM, int BN, int S, int KS = 32, int WGS = 1, int MAXL = RD_MAX_GROUPS, int WR = 2,
          int WC = 2, bool ZIL = false>
void launch_one(const KArgs& a, long long work, hipStream_t stream) {
  if constexpr (S == 0)
    grouped_gemm_regs<MODE, BM, BN><<<grid_size(work, 2), kThreads, 0, stream>>>(a);
  else
    grouped_gemm_stream<MODE, BM, BN, S, KS, WGS, MAXL, WR, WC, ZIL>
        <<<grid_size(work, WGS), WR * WC * 64, 0, stream>>>(with_per_cu(a, grid_size(work, WGS)));
}

// launch_one for tile shape TILE, checked against kTileShapes (which sizes the trans workspace).
template <int TILE, int MODE, int BM, int BN, int S, int KS = 32, int WGS = 1, int MAXL = RD_MAX_GROUPS, int WR = 2,
          int WC = 2, bool ZIL = false>
void launch_checked(const KArgs& a, long long work, hipStream_t stream) {
  static_assert(kTileShapes[TILE].bm == BM && kTileShapes[TILE].bn == BN && kTileShapes[TILE].wgs == WGS,
                "kTileShapes must match the launched shape");
  launch_one<MODE, BM, BN, S, KS, WGS, MAXL, WR, WC, ZIL>(a, work, stream);
}

template <int MODE, int S, int KS>
void launch_pp(const KArgs& a, long long work, hipStream_t stream) {
  grouped_gemm_pp<MODE, S, KS><<<grid_size(work, 1), 512, 0, stream>>>(a);
}

// zil: the call has a window, whose zero rows the kW128x256 forward tile
// writes while its tiles run (the ZIL instance of grouped_gemm_stream).
template <int MODE>
void launch_tile(int tile, const KArgs& a, const GemmProblem& p, hipStream_t stream, bool zil = false) {
  auto work = [&](int BM, int BN) {
    if (is_trans(MODE))
      return static_cast<long long>(p.num_local) * ((p.k + BM - 1) / BM) * ((p.n + BN - 1) / BN);
    return (static_cast<long long>((p.m + BM - 1) / BM) + p.num_local) * ((p.n + BN - 1) / BN) +
           (p.m + kZeroRows - 1) / kZeroRows + 2;
  };
  switch (tile) {
    // 64-deep stages (measured faster than 32-deep ones with more stages: the
    // per-stage barrier costs more than the extra depth gains); the LDS ring
    // takes 128-144 KB, 64 KB per workgroup for the two-per-CU variant
    case kT64x128: launch_checked<kT64x128, MODE, 64, 128, 6, 64>(a, work(64, 128), stream); break;
    case kT128x256: launch_checked<kT128x256, MODE, 128, 256, 3, 64>(a, work(128, 256), stream); break;
    case kT256x256: launch_checked<kT256x256, MODE, 256, 256, 2, 64>(a, work(256, 256), stream); break;
    case kT128x128x2: launch_checked<kT128x128x2, MODE, 128, 128, 2, 64, 2>(a, work(128, 128), stream); break;
    case kT64x64: launch_checked<kT64x64, MODE, 64, 64, 8, 64>(a, work(64, 64), stream); break;
    case kT256x256k32: launch_checked<kT256x256k32, MODE, 256, 256, 4, 32>(a, work(256, 256), stream); break;
    case kT128x256k32: launch_checked<kT128x256k32, MODE, 128, 256, 6, 32>(a, work(128, 256), stream); break;
    case kT128x256x2: launch_checked<kT128x256x2, MODE, 128, 256, 2, 32, 2>(a, work(128, 256), stream); break;
    case kT128x128k32x2: launch_checked<kT128x128k32x2, MODE, 128, 128, 3, 32, 2>(a, work(128, 128), stream); break;
    case kT128x128x3: launch_checked<kT128x128x3, MODE, 128, 128, 2, 32, 3>(a, work(128, 128), stream); break;
    case kT256x128x2: launch_checked<kT256x128x2, MODE, 256, 128, 2, 32, 2>(a, work(256, 128), stream); break;
    case kT128x256s3x2:  // a 3-slot ring for two workgroups per CU fits only with num_local <= 512
      if (p.num_local <= 512)
        launch_checked<kT128x256s3x2, MODE, 128, 256, 3, 32, 2, 512>(a, work(128, 256), stream);
      else
        launch_checked<kT128x256s3x2, MODE, 128, 256, 2, 32, 2>(a, work(128, 256), stream);
      break;
    // eight waves (two per SIMD) sharing one ring: 4 x 2 waves of 64 x 128,
    // 2 x 4 waves of 64 x 64, and the 256 x 256 tile with 64-deep stages
    case kW256x256: launch_checked<kW256x256, MODE, 256, 256, 4, 32, 1, RD_MAX_GROUPS, 4, 2>(a, work(256, 256), stream); break;
    case kW128x256:
      if constexpr (MODE == kFwdNN || MODE == kFwdNT)
        if (zil) {
          launch_checked<kW128x256, MODE, 128, 256, 3, 64, 1, RD_MAX_GROUPS, 2, 4, true>(a, work(128, 256), stream);
          break;
        }
      launch_checked<kW128x256, MODE, 128, 256, 3, 64, 1, RD_MAX_GROUPS, 2, 4>(a, work(128, 256), stream);
      break;
    case kW256x256k64: launch_checked<kW256x256k64, MODE, 256, 256, 2, 64, 1, RD_MAX_GROUPS, 4, 2>(a, work(256, 256), stream); break;
    case kW128x512: launch_checked<kW128x512, MODE, 128, 512, 3, 32, 1, RD_MAX_GROUPS, 2, 4>(a, work(128, 512), stream); break;
    case kW128x256k32: launch_checked<kW128x256k32, MODE, 128, 256, 6, 32, 1, RD_MAX_GROUPS, 2, 4>(a, work(128, 256), stream); break;
    // eight waves in two ping-pong groups on 256 x 256 tiles, a 2-slot ring of 64-deep stages
    case kP256x256:
      static_assert(kTileShapes[kP256x256].bm == 256 && kTileShapes[kP256x256].bn == 256, "pp tile shape");
      launch_pp<MODE, 2, 64>(a, work(256, 256), stream);
      break;
    default: launch_checked<kT128x128, MODE, 128, 128, 4, 64>(a, work(128, 128), stream); break;
  }
}

// The buffer-to-LDS pipeline addresses every operand through 32-bit buffer
// offsets, so each operand must span less than 4 GiB.
bool fits_32bit(long long a, long long b) { return a * b * 2 < (1ll << 32); }

// Split-contraction decode path (decode_streamk_gemm): chosen from host-known
// sizes when groups average at most 24 rows, n splits into 768-, 512- or
// 256-column strips and k into 16-row steps.  One workgroup per CU; the
// workspace holds seg_max partial blocks per workgroup, seg_max bounding the
// blocks one range can touch (from at most ceil(m/32) + num_local row blocks);
// it must fit in 256 MiB.  rd_tune_set(RD_TUNE_DECODE, 0) turns the path off (for sweeps).
DecodePlan plan_decode_impl(const GemmProblem& p, bool trans_rhs) {
  DecodePlan d{};
  if (trans_rhs || g_tune[RD_TUNE_DECODE].load(std::memory_order_relaxed) == 0) return d;
  const long long avg_rows = p.m / (p.num_local > 0 ? p.num_local : 1);
  if (p.m <= 0 || avg_rows > 24 || p.k % kDecKS != 0 || !fits_32bit(p.m, p.k) || !fits_32bit(p.k, p.n)) return d;
  const int nb = p.n % 768 == 0 ? 6 : p.n % 512 == 0 ? 4 : p.n % 256 == 0 ? 2 : 0;
  if (nb == 0) return d;
  const long long grid = device_cu_count();
  const long long nnc = p.n / (128 * nb), spb = p.k / kDecKS;
  const long long blocks_max = ((p.m + kDecBM - 1) / kDecBM + p.num_local) * nnc;
  const long long per_max = (blocks_max * spb + grid - 1) / grid;
  const long long seg_max = (per_max + spb - 1) / spb + 1;
  const unsigned long long ws =
      static_cast<unsigned long long>(grid) * seg_max * kDecBM * (128ull * nb) * sizeof(float);
  if (ws > (256ull << 20)) return d;
  d.use = true;
  d.nb = nb;
  d.grid = static_cast<int>(grid);
  d.seg_max = static_cast<int>(seg_max);
  d.ws_bytes = ws;
  return d;
}

template <int NB, int S>
void launch_decode(const KArgs& a, const GemmProblem& p, const DecodePlan& d, float* ws, hipStream_t stream) {
  decode_streamk_gemm<NB, S><<<d.grid, kThreads, 0, stream>>>(a, ws, d.seg_max);
  const long long chunks = (static_cast<long long>(p.m) * (p.n / 8) + kThreads - 1) / kThreads;
  decode_streamk_reduce<NB><<<grid_size(chunks, 4), kThreads, 0, stream>>>(a, ws, d.seg_max, d.grid);
}

// ---------------------------------------------------------------- allocation-free forward

// The decode split path's partial sums for callers that cannot allocate (a
// HIP graph under capture, a serving loop that must not call hipMalloc): a
// file-scope device array, one per GPU the library runs on, held until the
// process ends.  Host code never passes the array's name to a kernel (in
// host code it is a stand-in, not a device address): each device's address
// comes from hipGetSymbolAddress, looked up once with that device current.
static __device__ __align__(256) unsigned char scratch[RD_NOALLOC_SCRATCH_BYTES];

std::mutex g_scratch_mu;
void* g_scratch_ptr[64] = {};

// This device's scratch address (looked up on the first call on the device), or null with *status set.
void* scratch_address(int* status) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) {
    *status = RD_EHIP;
    return nullptr;
  }
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (g_scratch_ptr[dev] == nullptr) {
    void* ptr = nullptr;
    if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) != hipSuccess || ptr == nullptr) {
      *status = RD_EHIP;
      return nullptr;
    }
    g_scratch_ptr[dev] = ptr;
  }
  return g_scratch_ptr[dev];
}

}  // namespace

DecodePlan plan_decode(const GemmProblem& p, bool trans_rhs) { return plan_decode_impl(p, trans_rhs); }

int launch_forward_noalloc(const GemmProblem& p, hipStream_t stream) {
  const DecodePlan d = plan_decode_impl(p, false);
  if (!d.use) return launch_forward(p, false, nullptr, 0, stream);  // the tile kernels use no scratch
  if (d.ws_bytes > RD_NOALLOC_SCRATCH_BYTES) return RD_ESCRATCH;
  int status = RD_OK;
  void* ptr = scratch_address(&status);
  if (ptr == nullptr) return status;
  return launch_forward(p, false, ptr, d.ws_bytes, stream);
}

int launch_forward(const GemmProblem& p, bool trans_rhs, void* workspace, size_t workspace_bytes,
                   hipStream_t stream) {
  const KArgs a = make_args(p);
  const DecodePlan d = plan_decode_impl(p, trans_rhs);
  if (d.use && workspace != nullptr && workspace_bytes >= d.ws_bytes) {
    float* ws = static_cast<float*>(workspace);
    switch (d.nb) {
      // ring: 6 x 25 KB, 8 x 17 KB, 8 x 9 KB
      case 6: launch_decode<6, 6>(a, p, d, ws, stream); break;
      case 4: launch_decode<4, 8>(a, p, d, ws, stream); break;
      default: launch_decode<2, 8>(a, p, d, ws, stream); break;
    }
    return hipGetLastError() == hipSuccess ? RD_OK : RD_EHIP;
  }
  const bool dma = (p.k % BK) == 0 && fits_32bit(p.m, p.k) && fits_32bit(p.k, p.n);
  if (dma) {
    const int tile = pick_forward_tile(p, trans_rhs);
    const bool zil = p.group_offset != nullptr;  // a window: rows outside it are zeroed
    if (trans_rhs)
      launch_tile<kFwdNT>(tile, a, p, stream, zil);
    else
      launch_tile<kFwdNN>(tile, a, p, stream, zil);
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

bool fused_glu_supported(const GemmProblem& p) {
  return p.k % BK == 0 && p.n % 128 == 0 && fits_32bit(p.m, p.k) && fits_32bit(p.k, 2ll * p.n);
}

// The fused up-projection takes the forward's tile shapes, each weight tile
// split into gate and up halves (a 512-wide tile gives 256 GLU columns, a
// 256-wide one 128, the short-group 128-wide one 64).
int launch_forward_glu(const GemmProblem& p, hipStream_t stream) {
  if (!fused_glu_supported(p)) return RD_EUNSUPPORTED;
  const KArgs a = make_args(p);
  auto work = [&](int BM, int TN) {
    return (static_cast<long long>((p.m + BM - 1) / BM) + p.num_local) * ((p.n + TN - 1) / TN) +
           (p.m + kZeroRows - 1) / kZeroRows + 2;
  };
  int tile = forced_tile(RD_TUNE_FWD_TILE);
  if (tile == kW128x512 && p.n % 256 != 0) tile = -1;  // the 512-column tile needs h % 256 == 0
  if (tile != kT64x128 && tile != kT128x256 && tile != kT128x256x2 && tile != kW128x256 && tile != kW128x512) {
    const long long avg_rows = p.m / (p.num_local > 0 ? p.num_local : 1);
    tile = avg_rows <= 48 ? kT64x128 : avg_rows > 256 ? kW128x256 : p.n % 256 == 0 ? kW128x512 : kT128x256x2;
  }
  switch (tile) {
    case kT64x128: launch_one<kFwdGLU, 64, 128, 6, 64>(a, work(64, 64), stream); break;
    case kT128x256: launch_one<kFwdGLU, 128, 256, 3, 64>(a, work(128, 128), stream); break;
    case kT128x256x2: launch_one<kFwdGLU, 128, 256, 2, 32, 2>(a, work(128, 128), stream); break;
    // 256 gate + 256 up columns per tile (512-byte weight rows), 2 x 4 waves of 64 x 128
    case kW128x512: launch_one<kFwdGLU, 128, 512, 3, 32, 1, RD_MAX_GROUPS, 2, 4>(a, work(128, 256), stream); break;
    default: launch_one<kFwdGLU, 128, 256, 3, 64, 1, RD_MAX_GROUPS, 2, 4>(a, work(128, 128), stream); break;
  }
  return hipGetLastError() == hipSuccess ? RD_OK : RD_EHIP;
}

int launch_forward_fp8(const GemmProblem& p, bool trans_rhs, hipStream_t stream) {
  // the kernels address fp8 rows as k / 2 16-bit elements
  GemmProblem q = p;
  q.k = p.k / 2;
  const KArgs a = make_args(q);
  const long long work = (static_cast<long long>((p.m + 127) / 128) + p.num_local) * ((p.n + 255) / 256) +
                         (p.m + kZeroRows - 1) / kZeroRows + 2;
  // the bf16 forward's shapes: 8-wave 128 x 256 tiles (64-deep bf16 = 128-deep
  // fp8 stages), and 128 x 512 tiles for the plain form's short groups (<= 256
  // rows on average); decode-sized groups keep the 4-wave 128 x 256 tile.
  // Measured: backward dx 208 -> 186 us, up-projection forward 174 -> 146 us.
  const long long avg_rows = p.m / (p.num_local > 0 ? p.num_local : 1);
  auto go = [&](auto mode) {
    constexpr int M = decltype(mode)::value;
    if (avg_rows <= 48) {
      launch_one<M, 128, 256, 3, 64>(a, work, stream);
      return;
    }
    if constexpr (M == kFwdNN8) {
      if (avg_rows <= 256 && p.n % 512 == 0) {
        launch_one<M, 128, 512, 3, 32, 1, RD_MAX_GROUPS, 2, 4>(a, work, stream);
        return;
      }
    }
    launch_one<M, 128, 256, 3, 64, 1, RD_MAX_GROUPS, 2, 4>(a, work, stream);
  };
  if (trans_rhs)
    go(std::integral_constant<int, kFwdNT8>{});
  else
    go(std::integral_constant<int, kFwdNN8>{});
  return hipGetLastError() == hipSuccess ? RD_OK : RD_EHIP;
}

int launch_trans_fp8(const GemmProblem& p, void* workspace, size_t workspace_bytes, hipStream_t stream) {
  KArgs a = make_args(p);
  const long long tiles = static_cast<long long>(p.num_local) * ((p.k + 127) / 128) * ((p.n + 255) / 256);
  // the row split of long groups as for bf16 (same 128 x 256 tiles, the
  // same workspace header and partial layout, the same reduction)
  const bool split = workspace != nullptr && workspace_bytes > kSplitHeaderInts * 4;
  if (split) {
    a.ws = workspace;
    a.ws_bytes = static_cast<long long>(workspace_bytes);
  }
  // two co-resident workgroups per CU with 3-slot rings of 64-row stages (one
  // multiplies while the other drains its dW stores), as for bf16; measured
  // 317 -> 232 us at the backward shape (m32768, k1024, n4096)
  if (p.num_local <= 512)
    launch_one<kTransTN8, 128, 256, 3, 32, 2, 512>(a, tiles, stream);
  else
    launch_one<kTransTN8, 128, 256, 3, 64>(a, tiles, stream);
  if (split)
    trans_split_reduce<<<grid_size(static_cast<long long>(p.k) * (p.n / 8) / kReduceThreads + 1, 1), kReduceThreads, 0,
                         stream>>>(static_cast<const int*>(workspace), static_cast<long long>(workspace_bytes), p.out,
                                   p.out_f32 ? 1 : 0, p.k, p.n, p.num_local);
  return hipGetLastError() == hipSuccess ? RD_OK : RD_EHIP;
}

size_t trans_workspace_size(const GemmProblem& p) {
  if (!fits_32bit(p.m, p.k) || !fits_32bit(p.m, p.n)) return 0;  // the fallback pipeline does not split
  const int tile = pick_trans_tile(p);
  if (tile == kP256x256) return 0;
  const TileShape ts = tile_shape(tile);
  const long long tiles = static_cast<long long>(p.num_local) * ((p.k + ts.bm - 1) / ts.bm) *
                          ((p.n + ts.bn - 1) / ts.bn);
  const long long G = grid_size(tiles, ts.wgs);
  // split groups carry at least the mean work per CU (no less than the mean
  // per workgroup) and chunks at least half the mean per workgroup, so the
  // partials never exceed 3 G tiles
  return kSplitHeaderInts * 4 + static_cast<size_t>(3 * G) * ts.bm * ts.bn * 4;
}

int launch_trans(const GemmProblem& p, void* workspace, size_t workspace_bytes, hipStream_t stream) {
  KArgs a = make_args(p);
  if (fits_32bit(p.m, p.k) && fits_32bit(p.m, p.n)) {
    const int tile = pick_trans_tile(p);
    const bool split = workspace != nullptr && workspace_bytes > kSplitHeaderInts * 4 && tile != kP256x256;
    if (split) {
      a.ws = workspace;
      a.ws_bytes = static_cast<long long>(workspace_bytes);
    }
    launch_tile<kTransTN>(tile, a, p, stream);
    if (split)
      trans_split_reduce<<<grid_size(static_cast<long long>(p.k) * (p.n / 8) / kReduceThreads + 1, 1),
                           kReduceThreads, 0, stream>>>(static_cast<const int*>(workspace), static_cast<long long>(workspace_bytes), p.out,
                                     p.out_f32 ? 1 : 0, p.k, p.n, p.num_local);
  } else {
    const long long tiles = static_cast<long long>(p.num_local) * ((p.k + 127) / 128) * ((p.n + 127) / 128);
    launch_one<kTransTN, 128, 128, 0>(a, tiles, stream);
  }
  return hipGetLastError() == hipSuccess ? RD_OK : RD_EHIP;
}

int device_cu_count() {
  // one entry per device, filled on first use; concurrent first calls store the same value
  static std::atomic<int> cache[64];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) dev = 0;
  int v = cache[dev].load(std::memory_order_acquire);
  if (v == 0) {
    if (hipDeviceGetAttribute(&v, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || v <= 0) v = 256;
    cache[dev].store(v, std::memory_order_release);
  }
  return v;
}

int tune_set(int which, int value) {
  if (which == RD_TUNE_FWD_TILE || which == RD_TUNE_TRANS_TILE) {
    if (value < -1 || value >= kTileCount) return RD_EINVAL;
  } else if (which == RD_TUNE_DECODE) {
    if (value != 0 && value != 1) return RD_EINVAL;
  } else {
    return RD_EINVAL;
  }
  g_tune[which].store(value, std::memory_order_relaxed);
  return RD_OK;
}

int tile_count() { return kTileCount; }

}  // namespace rd
