// gmm_big.hpp -- the large-group kernel of the gfx950 grouped matmul (bf16
// operands, no scales; an optional bias).
//
// Output tiles are 256 x 256 (group-aligned in M, as in the general kernel),
// computed by eight waves, two per SIMD, of 128 x 64 each with 32x32x16 bf16
// MFMAs.  Two waves per SIMD keep the matrix core busy while either of them
// waits on a barrier or an LDS read.  The weight fragment is the MFMA's first
// operand, so a lane holds runs of output columns of one row.  When a tile's
// valid part is at most 128 rows or 128 columns, the waves switch to 64 x 64
// each, laid out over the valid half, so such a tile costs half a tile of
// MFMA work.
//
// K is consumed 32 at a time.  A K step of both operands (32 KB) sits in one
// of four LDS stages that form a ring: while the waves multiply step s, they
// read step s+1's fragments from LDS into the registers each MFMA has just
// consumed, and steps s+2 and s+3 -- of the same output tile or, near its
// end, the first ones of the workgroup's next tile -- are in flight.  Both
// operands reach LDS by direct-to-LDS buffer loads.  The lhs and an [G,N,K]
// weight are stored K-contiguous (64-byte rows); an [G,K,N] weight keeps its
// N-contiguous layout (512-byte K rows) and its fragments are read with the
// LDS transpose read.
//
// The epilogue exchanges half-rows between the two halves of the wave
// (permlane32 swap) so each lane stores eight consecutive columns with one
// 16-byte buffer store.  Stores outside the tile's valid rows and columns
// are dropped by the buffer range check, so every wave issues the same
// number of memory instructions per tile, which the wait counts rely on.
#pragma once

#include <type_traits>

#include "gmm_device.hpp"

namespace gmmk {

// BIAS_: the problem has a bias (without one the epilogue adds nothing)
template <bool NN_, bool OUT_F32_, bool BIAS_>
struct BigCfg {
  static constexpr bool NN = NN_;
  static constexpr bool OUT_F32 = OUT_F32_;
  static constexpr bool BIAS = BIAS_;
  static constexpr int BM = 256, BN = 256;
  static constexpr int WM = 2, WN = 4, NWAVES = WM * WN, T = 64 * NWAVES;
  static constexpr int FM = 4, FN = 2;    // 32 x 32 blocks of a full-tile wave (128 x 64)
  static constexpr int BK = 32;           // K per stage (two 32x32x16 MFMA steps)
  static constexpr int ROW = BK * 2;      // bytes of a K-contiguous operand row in a stage
  static constexpr int NN_ROW = BN * 2;   // bytes of an N-contiguous weight K row
  static constexpr int A_BYTES = BM * ROW, B_BYTES = BN * BK * 2;
  static constexpr int STAGE = A_BYTES + B_BYTES;
  static constexpr int S = 4;  // stages in the ring
  static constexpr int RING = S * STAGE;
  static constexpr int BIAS_SLOT = 2048;  // a tile's bias row (<= 1 KB) and range-checked padding
  static constexpr int LDS = RING + 2 * BIAS_SLOT;  // bias slots of the current and the next tile
  // direct-to-LDS instructions (1 KB each) per wave, operand and stage
  static constexpr int DMA_A = A_BYTES / 1024 / NWAVES, DMA_B = B_BYTES / 1024 / NWAVES;
  static constexpr int DMA_STEP = DMA_A + DMA_B;
  static constexpr int es_out = OUT_F32 ? 4 : 2;
  // stores per wave and tile: 16-byte stores of 8 columns, per 32 x 32 block
  static constexpr int ST_BLOCK = OUT_F32 ? 4 : 2;
  static constexpr int E_FULL = FM * FN * ST_BLOCK, E_HALF = (FM / 2) * FN * ST_BLOCK;
  // memory operations per wave: a K step issues DMA_STEP loads (DMA_OPS for
  // a tile's first step, with its bias row); a tile's epilogue issues E
  // stores (a half tile pads with range-dropped stores)
  static constexpr int DMA_OPS = DMA_STEP + 1, E = E_FULL;
  static_assert(DMA_A == 2 && DMA_B == 2, "DMA split");
  static_assert(NN_ROW * BK == B_BYTES, "NN weight stage");
};

typedef __attribute__((address_space(3))) void* lds_ptr_t;

// 64-byte LDS rows: 16-byte chunk c of row r is stored at chunk c ^ swz64(r).
// Four rows share a 256-byte line of the 64 banks (rows r, r + 4, r + 8,
// r + 12 the same quarter of it) and two a 128-byte half: the swizzle gives
// rows 0, 4, 8, 12 and rows 0, 2, 4, 6 (and their shifts) four distinct
// chunks, so sixteen consecutive rows read at one logical chunk hit sixteen
// distinct 16-byte bank groups, and any eight consecutive ones eight.
__device__ __forceinline__ int swz64(int r) { return (((r >> 1) ^ (r >> 3)) & 1) | (r & 4) >> 1; }
// 512-byte K rows of an N-contiguous operand (the big kernel's [G,K,N]
// weight, both operands of the weight gradient): chunk c of K row k is
// stored at chunk c ^ swz_nn(k).  The 32 lanes an LDS cycle serves
// in a transpose read cover four K rows (512 bytes apart, so the same bank
// offsets) by four chunks each; the swizzle moves the four rows to the four
// quarters of the 64 banks.
__device__ __forceinline__ int swz_nn(int k) { return 4 * (k & 3); }

struct BigItem {
  int h, row0, rows, n0, ncols;
  int half;          // 1: 64 x 64 per wave (valid part <= 128 rows or columns)
  int rbase, cbase;  // this wave's first row / column in the tile
};

template <class C>
__device__ __forceinline__ BigItem decode_big(const Plan& pl, int L, int n_ntiles, int N, int w) {
  BigItem it;
  const int t = L / n_ntiles;
  const int j = L % n_ntiles;
  const int h = find_group(pl, t);
  const int row0 = pl.row_start[h] + (t - pl.tile_start[h]) * C::BM;
  const int left = pl.row_start[h + 1] - row0;
  // the values are the same in every lane: keep them in scalar registers
  it.h = __builtin_amdgcn_readfirstlane(h);
  it.row0 = __builtin_amdgcn_readfirstlane(row0);
  it.rows = __builtin_amdgcn_readfirstlane(left < C::BM ? left : C::BM);
  it.n0 = j * C::BN;
  it.ncols = N - it.n0 < C::BN ? N - it.n0 : C::BN;
  const bool half_m = it.rows <= C::BM / 2, half_n = it.ncols <= C::BN / 2;
  it.half = half_m || half_n;
  if (!it.half) {  // 2 x 4 waves of 128 x 64
    it.rbase = (w / C::WN) * 128;
    it.cbase = (w % C::WN) * 64;
  } else if (!half_n) {  // 2 x 4 waves of 64 x 64 over 128 x 256
    it.rbase = (w / 4) * 64;
    it.cbase = (w % 4) * 64;
  } else {  // 4 x 2 waves of 64 x 64 over 256 x 128
    it.rbase = (w / 2) * 64;
    it.cbase = (w % 2) * 64;
  }
  return it;
}

// Operand sources of an item as scalars (buffer resources are built at the
// point of use, so they stay in scalar registers).  Reads past a range
// return zero.
struct BigSrc {
  const char* a;     // lhs rows of the tile
  const char* b;     // NT: weight rows of the n-tile; NN: the group's weight from column n0
  const char* bias;  // the group's bias from column n0 (any address when absent)
  int a_bytes, b_bytes, bias_bytes, ncols;
};

template <class C>
__device__ __forceinline__ BigSrc big_src(const Params& p, const BigItem& it) {
  const int K = p.K, N = p.N;
  BigSrc s;
  s.a = reinterpret_cast<const char*>(p.lhs) + (long long)it.row0 * K * 2;
  s.a_bytes = it.rows * K * 2;
  const char* rhs_h = reinterpret_cast<const char*>(p.rhs) + (long long)it.h * N * K * 2;
  if constexpr (C::NN) {
    s.b = rhs_h + (long long)it.n0 * 2;
    s.b_bytes = K * N * 2 - it.n0 * 2;
  } else {
    s.b = rhs_h + (long long)it.n0 * K * 2;
    s.b_bytes = it.ncols * K * 2;
  }
  const int bes = p.bias_f32 ? 4 : 2;
  if (p.rhs_bias) {
    s.bias = reinterpret_cast<const char*>(p.rhs_bias) + ((long long)it.h * N + it.n0) * bes;
    s.bias_bytes = it.ncols * bes;
  } else {
    s.bias = reinterpret_cast<const char*>(p.lhs);
    s.bias_bytes = 0;
  }
  s.ncols = it.ncols;
  return s;
}

__device__ __forceinline__ __amdgpu_buffer_rsrc_t uniform_rsrc(const char* base, int bytes) {
  const unsigned long long u = reinterpret_cast<unsigned long long>(base);
  const unsigned lo = __builtin_amdgcn_readfirstlane((unsigned)u);
  const unsigned hi = __builtin_amdgcn_readfirstlane((unsigned)(u >> 32));
  const int n = __builtin_amdgcn_readfirstlane(bytes);
  const char* b = reinterpret_cast<const char*>(((unsigned long long)hi << 32) | lo);
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<char*>(b), (short)0, n, kBufferRsrcWord3);
}

// Per-lane byte offsets of this wave's direct-to-LDS loads (the K step adds
// a scalar offset).  K-contiguous operand: instruction i fills rows
// 32 w + 16 i + lane/4.  N-contiguous weight: instruction i fills K rows
// 4 w + 2 i + lane/32, 16-byte chunk lane%32 of each, which holds columns
// bcol[i] + [0, 8) of the tile.
struct DmaOff {
  int a[2], b[2], bcol[2];
};

template <class C>
__device__ __forceinline__ DmaOff dma_offsets(int K, int N, int w, int lane) {
  DmaOff d;
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const int r = w * 32 + i * 16 + (lane >> 2);
    d.a[i] = r * K * 2 + (((lane & 3) ^ swz64(r)) << 4);
    if constexpr (C::NN) {
      const int k = 4 * w + 2 * i + (lane >> 5);
      const int c = (lane & 31) ^ swz_nn(k);
      d.b[i] = k * N * 2 + c * 16;
      d.bcol[i] = c * 8;
    } else {
      d.b[i] = d.a[i];
      d.bcol[i] = 0;
    }
  }
  return d;
}

// Queue the direct-to-LDS loads of K step kt into stage `st`: two 1 KB
// instructions per operand and wave.  N-contiguous weight columns past the
// tile's valid part get an out-of-range offset (they would otherwise wrap
// into the next K row, or past the end of the last group's weight).
template <class C>
__device__ __forceinline__ void dma_stage(const BigSrc& src, const DmaOff& off, int kt, int N, char* st, int w) {
  const __amdgpu_buffer_rsrc_t ra = uniform_rsrc(src.a, src.a_bytes);
  const __amdgpu_buffer_rsrc_t rb = uniform_rsrc(src.b, src.b_bytes);
  char* da = st + w * 2048;
  char* db = st + C::A_BYTES + w * 2048;
  const int sa = kt * C::ROW;
#pragma unroll
  for (int i = 0; i < 2; ++i)
    __builtin_amdgcn_raw_ptr_buffer_load_lds(ra, (lds_ptr_t)(da + i * 1024), 16, off.a[i], sa, 0, 0);
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    if constexpr (C::NN) {
      const int vo = off.bcol[i] < src.ncols ? off.b[i] + kt * C::BK * N * 2 : (int)0x80000000;
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rb, (lds_ptr_t)(db + i * 1024), 16, vo, 0, 0, 0);
    } else {
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rb, (lds_ptr_t)(db + i * 1024), 16, off.b[i], sa, 0, 0);
    }
  }
}

// The tile's bias row into an LDS slot: wave w copies bytes [256 w, 256 w + 256)
// (zeros past the row, or everywhere without a bias).
__device__ __forceinline__ void dma_bias(const BigSrc& src, char* slot, int w, int lane) {
  const __amdgpu_buffer_rsrc_t r = uniform_rsrc(src.bias, src.bias_bytes);
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_ptr_t)(slot + w * 256), 4, w * 256 + lane * 4, 0, 0, 0);
}

// Direct-to-LDS sources of one tile, built once per tile (scalar
// registers): buffer resources of both operands and of its bias row, and
// for an N-contiguous weight the lane offsets with columns past the tile's
// valid part out of range (they would otherwise wrap into the next K row,
// or past the end of the last group's weight).  A tile past the end of the
// workgroup's stream gets zero-size ranges: its loads still issue (and
// write zeros to stages nobody reads), so every K step issues the same
// number of memory operations.
template <class C>
struct TileDma {
  __amdgpu_buffer_rsrc_t ra, rb, rbias;
  int vb[2];
};

template <class C>
__device__ __forceinline__ TileDma<C> tile_dma(const BigSrc& src, const DmaOff& off, bool live) {
  TileDma<C> d;
  d.ra = uniform_rsrc(src.a, live ? src.a_bytes : 0);
  d.rb = uniform_rsrc(src.b, live ? src.b_bytes : 0);
  d.rbias = uniform_rsrc(src.bias, live ? src.bias_bytes : 0);
#pragma unroll
  for (int i = 0; i < 2; ++i) d.vb[i] = (C::NN && off.bcol[i] >= src.ncols) ? (int)0x80000000 : off.b[i];
  return d;
}

// Direct-to-LDS operation J of K step k into stage `st`: J = 0, 1 the lhs,
// J = 2, 3 the weight (1 KB each per wave), J = 4 this wave's 256-byte piece
// of the tile's bias row.
template <class C, int J>
__device__ __forceinline__ void dma_op(const TileDma<C>& d, const DmaOff& off, int k, int N, char* st,
                                       char* bias_slot, int w, int vbias) {
  if constexpr (J < 2) {
    __builtin_amdgcn_raw_ptr_buffer_load_lds(d.ra, (lds_ptr_t)(st + w * 2048 + J * 1024), 16, off.a[J],
                                             k * C::ROW, 0, 0);
  } else if constexpr (J < 4) {
    const int so = C::NN ? k * C::BK * N * 2 : k * C::ROW;
    __builtin_amdgcn_raw_ptr_buffer_load_lds(d.rb, (lds_ptr_t)(st + C::A_BYTES + w * 2048 + (J - 2) * 1024), 16,
                                             d.vb[J - 2], so, 0, 0);
  } else {
    __builtin_amdgcn_raw_ptr_buffer_load_lds(d.rbias, (lds_ptr_t)(bias_slot + w * 256), 4, vbias, 0, 0, 0);
  }
}

// s_waitcnt with only the vector-memory counter constrained (gfx9 encoding:
// vmcnt low bits [3:0], high bits [15:14]; expcnt [6:4] and lgkmcnt [11:8]
// left at their maxima).
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (0x7 << 4) | (0xF << 8));
}

// Workgroup barrier without a memory fence.  The K loop orders its LDS
// traffic itself: a wave's direct-to-LDS loads are complete once the explicit
// vmcnt wait before the barrier returns, and its fragment reads of a stage
// are complete once the MFMAs that consume them have issued.  A fence here
// would make the compiler drain every outstanding direct-to-LDS load before
// the next LDS read, i.e. all the steps in flight.  The clobber keeps the
// compiler from moving memory accesses across the barrier.
__device__ __forceinline__ void ring_barrier() { asm volatile("s_barrier" ::: "memory"); }

// 32x32x16 fragments of a K-contiguous operand: lane (kh = lane / 32,
// r32 = lane % 32) holds row base + 32 f + r32, K elements
// [16 h + 8 kh, 16 h + 8 kh + 8) of the stage, i.e. 16-byte chunk 2 h + kh.
// Fragment rows start at multiples of 32, so the swizzled chunk depends only
// on the lane, and fragment (f, h) is one base address plus an immediate.
__device__ __forceinline__ int frag_lane_off(int kh, int r32, int h) {
  return r32 * 64 + (((2 * h + kh) ^ swz64(r32)) << 4);
}

// Fragment of an N-contiguous weight for tile columns
// [cbase + 32 fn, cbase + 32 fn + 32) and K half h, from two LDS transpose
// reads.  In read t, lane l (group q = l / 16, j = l % 16) points at K row
// 16 h + 8 (q / 2) + 4 t + j / 4 and columns 16 (q % 2) + 4 (j % 4) + [0, 4)
// of the block; the read hands lane l column l % 32 at K rows
// 16 h + 8 (l / 32) + 4 t + [0, 4).  The lane part of the address is
// nn_lane_off(fn) for a block at column 0 of a 128-column half; the swizzle
// flips chunk bits 2 and 3, so a block at column 64 mod 128 XORs bit 3
// (byte 128) into the lane part.  The K half and read add 512 (16 h + 4 t).
__device__ __forceinline__ int nn_lane_off(int lane, int fn) {
  const int q = lane >> 4, j = lane & 15;
  const int krow = 8 * (q >> 1) + (j >> 2);
  const int chunk = (4 * fn + 2 * (q & 1) + ((j >> 1) & 1)) ^ swz_nn(j >> 2);
  return krow * 512 + chunk * 16 + (j & 1) * 8;
}

// LDS transpose reads are issued as inline assembly: the compiler does not
// know which LDS bytes the builtin reads and drains every outstanding
// direct-to-LDS load before it.  The memory clobber keeps the reads in
// program order with the compiler's own LDS reads, and the results are
// waited for explicitly (nn_frags_ready) since the compiler does not track
// them.
template <int OFF>
__device__ __forceinline__ i32x2 ds_read_tr16(unsigned addr) {
  i32x2 r;
  asm volatile("ds_read_b64_tr_b16 %0, %1 offset:%2" : "=v"(r) : "v"(addr), "i"(OFF) : "memory");
  return r;
}

template <int H>
__device__ __forceinline__ i32x4 nn_frag(unsigned addr) {
  const i32x2 lo = ds_read_tr16<H * 16 * 512>(addr);
  const i32x2 hi = ds_read_tr16<H * 16 * 512 + 4 * 512>(addr);
  return i32x4{lo[0], lo[1], hi[0], hi[1]};
}

// Per K half the refills issue eight LDS operations in a fixed order (four
// lhs fragments, then two weight fragments of two transpose reads each), so
// a K half's weight fragments have completed once at most the eight
// operations of the following half are outstanding.
__device__ __forceinline__ void nn_frags_ready() {
  __builtin_amdgcn_s_waitcnt(0xF | (0x7 << 4) | (8 << 8) | (0x3 << 14));
}

// Staging rows of the epilogue: 128 bytes (eight 16-byte chunks); chunk c
// of row r is stored at chunk c ^ swz_out(r), so that both the column-wise
// writes (one chunk of 16 or 32 consecutive rows per LDS cycle) and the
// row-wise reads (whole rows) hit distinct bank groups.
__device__ __forceinline__ int swz_out(int r) { return (r & 7) ^ ((r >> 3) & 1); }

// Epilogue of one tile.  Block (fm, fn) of the wave, before the exchange:
// lane (kh, r32) holds row rbase + 32 fm + r32 and, in register 4 g + i,
// column cbase + 32 fn + 8 g + 4 kh + i.  For each pair of groups (g, g+1)
// the permlane32 swap leaves lanes kh = 0 with columns 8 g + [0, 8) and
// lanes kh = 1 with 8 (g+1) + [0, 8), in order.  Each 32-row block (per
// column half for an f32 output) then passes through the wave's 4 KB
// staging slice so that a store writes 8 whole 128-byte row segments
// instead of 32 scattered 32-byte ones.  Stores outside the tile's valid
// rows and columns are dropped by the range check; a half tile pads to the
// full tile's store count E.  BIAS: add the bias row (without one, the
// accumulators are rounded as they are).
template <class C, int FMA, bool BIAS>
__device__ __forceinline__ void big_epilogue(const Params& p, const f32x16 (&acc)[C::FM][C::FN], const BigItem& it,
                                             const char* bias_slot, char* stg, int kh, int r32, int lane) {
  const int N = p.N;
  char* tile = reinterpret_cast<char*>(p.out) + ((long long)it.row0 * N + it.n0) * C::es_out;
  const int nrec = ((it.rows - 1) * N + it.ncols) * C::es_out;
  const __amdgpu_buffer_rsrc_t ro = uniform_rsrc(tile, nrec);
  const bool bias_f32 = p.bias_f32 != 0;
  const int srow = lane >> 3, schunk = lane & 7;  // store phase: row and chunk of this lane
  const int wr_row = r32 * 128;                   // write phase: this lane's staging row
  // columns cbase + 32 fn + 8 (gp + x) + 4 kh + [0, 4) of the bias row
  auto load_bias = [&](int fn, int gp, float (&bias)[2][4]) __attribute__((always_inline)) {
#pragma unroll
    for (int x = 0; x < 2; ++x) {
      const int c = it.cbase + fn * 32 + 8 * (gp + x) + 4 * kh;
      if (bias_f32) {
        const f32x4 v = *reinterpret_cast<const f32x4*>(bias_slot + c * 4);
        bias[x][0] = v[0];
        bias[x][1] = v[1];
        bias[x][2] = v[2];
        bias[x][3] = v[3];
      } else {
        const i32x2 v = *reinterpret_cast<const i32x2*>(bias_slot + c * 2);
        bias[x][0] = __uint_as_float((uint32_t)v[0] << 16);
        bias[x][1] = __uint_as_float((uint32_t)v[0] & 0xFFFF0000u);
        bias[x][2] = __uint_as_float((uint32_t)v[1] << 16);
        bias[x][3] = __uint_as_float((uint32_t)v[1] & 0xFFFF0000u);
      }
    }
  };
  // rows srow + 8 i of the staged block back out, as whole row segments;
  // col0: the block's first column in the tile, cw: columns per chunk
  auto drain = [&](int fm, int col0, int cw) __attribute__((always_inline)) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int row = srow + 8 * i;
      const i32x4 d = *reinterpret_cast<const i32x4*>(stg + row * 128 + ((schunk ^ swz_out(row)) << 4));
      const int col = col0 + cw * schunk;
      const int voff = col < it.ncols ? (it.rbase + fm * 32 + row) * N * C::es_out + col * C::es_out
                                      : (int)0x80000000;
      __builtin_amdgcn_raw_buffer_store_b128(d, ro, voff, 0, 0);
    }
  };
  auto stage_write = [&](int chunk, i32x4 v) __attribute__((always_inline)) {
    *reinterpret_cast<i32x4*>(stg + wr_row + ((chunk ^ swz_out(r32)) << 4)) = v;
  };
#pragma unroll
  for (int fm = 0; fm < FMA; ++fm) {
    if constexpr (C::OUT_F32) {
#pragma unroll
      for (int fn = 0; fn < C::FN; ++fn) {
#pragma unroll
        for (int gp = 0; gp < 4; gp += 2) {
          float v[2][4];
#pragma unroll
          for (int x = 0; x < 2; ++x)
#pragma unroll
            for (int i = 0; i < 4; ++i) v[x][i] = acc[fm][fn][4 * (gp + x) + i];
          if constexpr (BIAS) {
            float bias[2][4];
            load_bias(fn, gp, bias);
#pragma unroll
            for (int x = 0; x < 2; ++x)
#pragma unroll
              for (int i = 0; i < 4; ++i) v[x][i] += bias[x][i];
          }
          int lo[4], hi[4];
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v[0][i]), __float_as_uint(v[1][i]),
                                                            false, false);
            lo[i] = (int)r[0];
            hi[i] = (int)r[1];
          }
          // 32 columns of 4 bytes per staging row: chunks 2 (gp + kh) + {0, 1}
          stage_write(2 * (gp + kh), i32x4{lo[0], lo[1], lo[2], lo[3]});
          stage_write(2 * (gp + kh) + 1, i32x4{hi[0], hi[1], hi[2], hi[3]});
        }
        drain(fm, it.cbase + fn * 32, 4);
      }
    } else {
#pragma unroll
      for (int fn = 0; fn < C::FN; ++fn) {
#pragma unroll
        for (int gp = 0; gp < 4; gp += 2) {
          float v[2][4];
#pragma unroll
          for (int x = 0; x < 2; ++x)
#pragma unroll
            for (int i = 0; i < 4; ++i) v[x][i] = acc[fm][fn][4 * (gp + x) + i];
          if constexpr (BIAS) {
            float bias[2][4];
            load_bias(fn, gp, bias);
#pragma unroll
            for (int x = 0; x < 2; ++x)
#pragma unroll
              for (int i = 0; i < 4; ++i) v[x][i] += bias[x][i];
          }
          uint32_t x0[2], x1[2];
#pragma unroll
          for (int x = 0; x < 2; ++x) {
            x0[x] = pk_bf16_rne(v[x][0], v[x][1]);
            x1[x] = pk_bf16_rne(v[x][2], v[x][3]);
          }
          const auto r0 = __builtin_amdgcn_permlane32_swap(x0[0], x0[1], false, false);
          const auto r1 = __builtin_amdgcn_permlane32_swap(x1[0], x1[1], false, false);
          // 64 columns of 2 bytes per staging row: chunk 4 fn + gp + kh
          stage_write(4 * fn + gp + kh, i32x4{(int)r0[0], (int)r1[0], (int)r0[1], (int)r1[1]});
        }
      }
      drain(fm, it.cbase, 8);
    }
  }
  // a half tile pads to the full tile's store count with range-dropped
  // stores, each to an address of its own: the compiler deletes a store that
  // repeats an earlier one, and every dropped one would leave the K loop's
  // constant waits one operation short
#pragma unroll
  for (int i = FMA * C::FN * C::ST_BLOCK; i < C::E; ++i)
    __builtin_amdgcn_raw_buffer_store_b128(i32x4{0, 0, 0, 0}, ro, (int)0x80000000, 64 * i, 0);
}

template <class C>
__global__ __launch_bounds__(C::T) void gmm_big_kernel(Params p) {
  // One LDS array for the ring, the bias slots and the plan: with a second
  // LDS variable the compiler tags LDS accesses with alias scopes and then
  // drains every outstanding direct-to-LDS load before each fragment read.
  __shared__ __attribute__((aligned(1024))) char smem[C::LDS + sizeof(Plan)];
  Plan& pl = *reinterpret_cast<Plan*>(smem + C::LDS);
  if (threadIdx.x == 0) pl.flags = 0;
  __syncthreads();
  build_plan<C::T>(p, pl, C::BM);
  report_flags(p, pl);

  const int tid = threadIdx.x, lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int kh = lane >> 5, r32 = lane & 31;
  const int M = p.M, N = p.N, K = p.K;
  const int P = gridDim.x;
  const int slot = xcd_slot(blockIdx.x, P);

  // rows outside the active groups: fill them first (grid-stride)
  {
    const long long row_bytes = (long long)N * C::es_out;
    const int lo_row = pl.row_start[0], hi_row = pl.row_start[pl.ga];
    const long long z1 = fill_rows(p, lo_row) * row_bytes;
    const long long z2b = (long long)hi_row * row_bytes;
    const long long total = z1 + fill_rows(p, M - hi_row) * row_bytes;
    for (long long off = ((long long)slot * C::T + tid) * 16; off < total; off += (long long)P * C::T * 16)
      fill16(p, off < z1 ? off : z2b + (off - z1));
  }

  const int n_ntiles = (N + C::BN - 1) / C::BN;
  const int n_items = __builtin_amdgcn_readfirstlane(pl.n_mtiles) * n_ntiles;
  const int KT = K / C::BK;  // K steps per item; the launcher guarantees KT >= 5
  if (slot >= n_items) return;

  // This workgroup's items are slot, slot + P, ...; their K steps form one
  // stream.  Loads run three steps ahead of the multiplication and fragment
  // reads one step ahead -- within the current item or, near its end, in the
  // next one.
  BigItem cur = decode_big<C>(pl, slot, n_ntiles, N, w);
  BigItem nxt = cur;
  if (slot + P < n_items) nxt = decode_big<C>(pl, slot + P, n_ntiles, N, w);
  BigSrc cur_src = big_src<C>(p, cur), nxt_src = big_src<C>(p, nxt);
  const DmaOff doff = dma_offsets<C>(K, N, w, lane);
  char* const bias0 = smem + C::RING;

  // Prologue: the first tile's bias and steps 0..2; every older memory
  // operation (the zero fill) is complete after the wait, so the loop's
  // counts start from an empty queue.
  dma_bias(cur_src, bias0, w, lane);
#pragma unroll
  for (int s = 0; s < C::S - 1; ++s) dma_stage<C>(cur_src, doff, s, N, smem + s * C::STAGE, w);
  wait_vmcnt<0>();
  __syncthreads();

  const int alo0 = frag_lane_off(kh, r32, 0), alo1 = frag_lane_off(kh, r32, 1);
  const int blo0 = C::NN ? nn_lane_off(lane, 0) : alo0;
  const int blo1 = C::NN ? nn_lane_off(lane, 1) : alo1;

  // fragment (f, h) of the step in stage `st`, for the layout of `it`
  auto a_frag = [&](const char* st, const BigItem& it, int f, int h) __attribute__((always_inline)) {
    return *reinterpret_cast<const i32x4*>(st + it.rbase * C::ROW + f * 32 * C::ROW + (h ? alo1 : alo0));
  };
  auto b_frag = [&](const char* st, const BigItem& it, int f, int h) __attribute__((always_inline)) {
    const char* bb = st + C::A_BYTES;
    if constexpr (C::NN) {
      const int cb = it.cbase * 2;  // byte offset of the wave's first column in a K row
      const unsigned addr = (unsigned)(size_t)(lds_ptr_t)(bb + (cb & ~128) + ((f ? blo1 : blo0) ^ (cb & 128)));
      return h ? nn_frag<1>(addr) : nn_frag<0>(addr);
    } else {
      return *reinterpret_cast<const i32x4*>(bb + it.cbase * C::ROW + f * 32 * C::ROW + (h ? blo1 : blo0));
    }
  };

  i32x4 a[C::FM][2], b[C::FN][2];
#pragma unroll
  for (int h = 0; h < 2; ++h) {
#pragma unroll
    for (int f = 0; f < C::FM; ++f) a[f][h] = a_frag(smem, cur, f, h);
#pragma unroll
    for (int f = 0; f < C::FN; ++f) b[f][h] = b_frag(smem, cur, f, h);
  }

  f32x16 acc[C::FM][C::FN];
  int stage = 0;  // stage of the current step
  int L = slot;
  bool last_item = L + P >= n_items;
  int par = 0;  // bias slot of the current item
  TileDma<C> dcur = tile_dma<C>(cur_src, doff, true);
  TileDma<C> dnxt = tile_dma<C>(nxt_src, doff, !last_item);
  const int vbias = w * 256 + lane * 4;

  // One K step s.  The tile's K loop runs in phases so each step's wait
  // count and load source are constants: step s+1's operands are complete
  // (this wave's loads, then every wave's after the barrier) once at most
  // WAIT newer operations are outstanding -- step s+2's loads (four; five
  // for a tile's first step, which also brings its bias row) and, in a
  // tile's first two steps, the previous tile's E stores (after the
  // prologue's full wait the first tile's counts only wait longer).  The
  // barrier also frees the stage step s-1 used, which takes the loads of
  // step s+3 (this tile's step kd, or the next tile's when NEXT), spread
  // evenly over the MFMAs.  Each fragment is refilled with step s+1's --
  // the next tile's layout in a tile's last step -- right after its last
  // use (from an in-range stage even when no step follows).
  auto kstep = [&](auto full_tag, auto wait_tag, auto next_tag, auto bias_tag, auto last_tag, int kd)
      __attribute__((always_inline)) {
    constexpr bool FULL = decltype(full_tag)::value;
    constexpr int WAIT = decltype(wait_tag)::value;
    constexpr bool NEXT = decltype(next_tag)::value, BIAS = decltype(bias_tag)::value;
    constexpr bool LAST = decltype(last_tag)::value;
    constexpr int FMA = FULL ? C::FM : C::FM / 2;
    constexpr int NM = 2 * FMA * C::FN;  // MFMAs per step
    constexpr int NOPS = BIAS ? C::DMA_OPS : C::DMA_STEP;
    wait_vmcnt<WAIT>();
    // in a tile's last step every wave's reads of the current stage are
    // complete past the barrier: the epilogue stages its output there
    if constexpr (LAST) __builtin_amdgcn_s_waitcnt(0xF | (0x7 << 4) | (0x0 << 8) | (0x3 << 14));
    ring_barrier();
    const TileDma<C>& d = NEXT ? dnxt : dcur;
    char* st3 = smem + ((stage + 3) & (C::S - 1)) * C::STAGE;
    char* bslot = bias0 + (par ^ 1) * C::BIAS_SLOT;
    const char* st1 = smem + ((stage + 1) & (C::S - 1)) * C::STAGE;
    const BigItem& it1 = LAST ? nxt : cur;
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      if constexpr (C::NN) nn_frags_ready();
#pragma unroll
      for (int fm = 0; fm < FMA; ++fm) {
#pragma unroll
        for (int fn = 0; fn < C::FN; ++fn) {
          acc[fm][fn] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, b[fn][h]),
                                                                __builtin_bit_cast(bf16x8, a[fm][h]),
                                                                acc[fm][fn], 0, 0, 0);
          const int m = (h * FMA + fm) * C::FN + fn;
          // with the bias piece it goes first (older than the operands)
          if (m == 0 * NM / NOPS) { if constexpr (BIAS) dma_op<C, 4>(d, doff, kd, N, st3, bslot, w, vbias); else dma_op<C, 0>(d, doff, kd, N, st3, bslot, w, vbias); }
          if (m == 1 * NM / NOPS) { if constexpr (BIAS) dma_op<C, 0>(d, doff, kd, N, st3, bslot, w, vbias); else dma_op<C, 1>(d, doff, kd, N, st3, bslot, w, vbias); }
          if (m == 2 * NM / NOPS) { if constexpr (BIAS) dma_op<C, 1>(d, doff, kd, N, st3, bslot, w, vbias); else dma_op<C, 2>(d, doff, kd, N, st3, bslot, w, vbias); }
          if (m == 3 * NM / NOPS) { if constexpr (BIAS) dma_op<C, 2>(d, doff, kd, N, st3, bslot, w, vbias); else dma_op<C, 3>(d, doff, kd, N, st3, bslot, w, vbias); }
          if constexpr (BIAS) if (m == 4 * NM / NOPS) dma_op<C, 3>(d, doff, kd, N, st3, bslot, w, vbias);
          __builtin_amdgcn_sched_barrier(0);  // keep this order
        }
        a[fm][h] = a_frag(st1, it1, fm, h);
      }
#pragma unroll
      for (int fm = FMA; fm < C::FM; ++fm) a[fm][h] = a_frag(st1, it1, fm, h);
#pragma unroll
      for (int fn = 0; fn < C::FN; ++fn) b[fn][h] = b_frag(st1, it1, fn, h);
      __builtin_amdgcn_sched_barrier(0);
    }
    stage = (stage + 1) & (C::S - 1);
  };
  using T_ = std::true_type;
  using F_ = std::false_type;
  using W0 = std::integral_constant<int, C::DMA_STEP + C::E>;  // first two steps of a tile
  using W1 = std::integral_constant<int, C::DMA_STEP>;
  using W2 = std::integral_constant<int, C::DMA_STEP + 1>;  // step s+2 is the next tile's first
  // One tile: KT >= 5 steps (the launcher guarantees K >= 160).
  auto ktile = [&](auto full_tag) __attribute__((always_inline)) {
    constexpr bool FULL = decltype(full_tag)::value;
    constexpr int FMA = FULL ? C::FM : C::FM / 2;
    kstep(full_tag, W0{}, F_{}, F_{}, F_{}, 3);
    kstep(full_tag, W0{}, F_{}, F_{}, F_{}, 4);
    for (int kt = 2; kt + 3 < KT; ++kt) kstep(full_tag, W1{}, F_{}, F_{}, F_{}, kt + 3);
    kstep(full_tag, W1{}, T_{}, T_{}, F_{}, 0);  // kt = KT-3: the next tile's step 0 and bias row
    kstep(full_tag, W2{}, T_{}, F_{}, F_{}, 1);
    kstep(full_tag, W1{}, T_{}, F_{}, T_{}, 2);
    // The weight fragments of an [G,K,N] weight come from transpose reads,
    // whose registers are written when the data arrives; after the last tile
    // the refills have no later use, so the compiler could give their
    // registers to the epilogue while the reads are in flight.  Wait for
    // them and use them here first.
    if constexpr (C::NN) {
      __builtin_amdgcn_s_waitcnt(0xF | (0x7 << 4) | (0x0 << 8) | (0x3 << 14));
      asm volatile("" ::"v"(b[0][0]), "v"(b[0][1]), "v"(b[1][0]), "v"(b[1][1]));
    }
    // the last step's stage (the next tile's step 3 goes there after its
    // first barrier) holds the epilogue's staging slices, 4 KB per wave
    big_epilogue<C, FMA, C::BIAS>(p, acc, cur, bias0 + par * C::BIAS_SLOT,
                         smem + ((stage + 3) & (C::S - 1)) * C::STAGE + w * 4096, kh, r32, lane);
  };

  while (true) {
#pragma unroll
    for (int x = 0; x < C::FM; ++x)
#pragma unroll
      for (int y = 0; y < C::FN; ++y)
#pragma unroll
        for (int z = 0; z < 16; ++z) acc[x][y][z] = 0.f;
    if (!cur.half)
      ktile(std::true_type{});
    else
      ktile(std::false_type{});
    if (last_item) break;
    L += P;
    last_item = L + P >= n_items;
    cur = nxt;
    cur_src = nxt_src;
    dcur = dnxt;
    par ^= 1;
    if (!last_item) {
      nxt = decode_big<C>(pl, L + P, n_ntiles, N, w);
      nxt_src = big_src<C>(p, nxt);
    }
    dnxt = tile_dma<C>(nxt_src, doff, !last_item);
  }
}

}  // namespace gmmk
