// gmm_big.hpp -- the large-group kernel of the gfx950 grouped matmul (bf16
// operands, no scales; an optional bias).
//
// Output tiles are 256 x 256 (group-aligned in M, as in the general kernel),
// computed by eight waves (two per SIMD) of 128 x 64 each.  A group's last
// m-tile and the last n-tile of a row are usually partial; when the valid
// part is at most 128 rows or 128 columns the eight waves switch to 64 x 64
// each, laid out 2 x 4 or 4 x 2 over the valid half, so such a tile costs
// half a tile of MFMA work.
//
// K is consumed 32 at a time.  A K tile of both operands (256 rows x 64 bytes
// each, 32 KB) sits in one of four LDS stages that form a ring: while the
// waves multiply one stage, the next three -- of the same output tile, or the
// first ones of the workgroup's next output tile -- are in flight.  Operands
// reach LDS by direct-to-LDS buffer loads (no staging registers), except a
// [G,K,N] weight, which goes through registers to be transposed to the
// K-contiguous layout the MFMA operands need.
#pragma once

#include "gmm_device.hpp"

namespace gmmk {

template <bool NN_, bool OUT_F32_>
struct BigCfg {
  static constexpr bool NN = NN_;
  static constexpr bool OUT_F32 = OUT_F32_;
  static constexpr int BM = 256, BN = 256;
  static constexpr int WM = 2, WN = 4, NWAVES = WM * WN, T = 64 * NWAVES;
  static constexpr int TM = BM / WM, TN = BN / WN, FM = TM / 16, FN = TN / 16;
  static constexpr int BK = 32;          // K per stage (one 16x16x32 MFMA)
  static constexpr int ROW = BK * 2;     // bytes per LDS row
  static constexpr int A_BYTES = BM * ROW, B_BYTES = BN * ROW;
  static constexpr int STAGE = A_BYTES + B_BYTES;
  static constexpr int S = 4;            // stages in the ring
  static constexpr int LDS = S * STAGE;
  // direct-to-LDS instructions per wave per operand and stage (1 KB each)
  static constexpr int ROWS_PER_WAVE = BM / NWAVES;
  static constexpr int DMA_PER_OPERAND = ROWS_PER_WAVE * ROW / 1024;
  // NN weight tile per thread: 8 k rows x NWN n columns
  static constexpr int NWN = BN * BK / T / 8;
  static constexpr int NN_LOADS = 8;
  static_assert(DMA_PER_OPERAND >= 1 && ROWS_PER_WAVE % 16 == 0, "DMA split");
  static_assert(NWN == 2 || NWN == 4, "NN thread block");
};

typedef __attribute__((address_space(3))) void* lds_ptr_t;

// 64-byte LDS rows: 16-byte chunk c of row r is stored at chunk c ^ swz64(r).
// Sixteen consecutive rows read at one logical chunk land in sixteen distinct
// (row parity, chunk) bank groups.
__device__ __forceinline__ int swz64(int r) { return (r >> 1) & 3; }
__device__ __forceinline__ int lds_off64(int r, int c) { return r * 64 + ((c ^ swz64(r)) << 4); }

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
    it.rbase = (w / C::WN) * C::TM;
    it.cbase = (w % C::WN) * C::TN;
  } else if (half_m) {  // 2 x 4 waves of 64 x 64 over 128 x 256
    it.rbase = (w / C::WN) * (C::TM / 2);
    it.cbase = (w % C::WN) * C::TN;
  } else {  // 4 x 2 waves of 64 x 64 over 256 x 128
    it.rbase = (w / C::WM) * (C::TM / 2);
    it.cbase = (w % C::WM) * C::TN;
  }
  return it;
}

// Direct-to-LDS loads of 256 rows x 64 bytes (K columns [32 kt, 32 kt + 32))
// of a row-major operand.  One instruction fills 1 KB = 16 rows; wave w fills
// rows [w R, w R + R), R = 256 / waves.  Rows past the resource's end read as
// zero.
template <class C>
__device__ __forceinline__ void dma_rows(__amdgpu_buffer_rsrc_t rs, int row_bytes, int kt, char* dst) {
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
#pragma unroll
  for (int i = 0; i < C::DMA_PER_OPERAND; ++i) {
    const int r0 = w * C::ROWS_PER_WAVE + i * 16;
    const int r = r0 + (lane >> 2);
    const int c = (lane & 3) ^ swz64(r);
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (lds_ptr_t)(dst + r0 * C::ROW), 16, r * row_bytes + c * 16,
                                             kt * C::ROW, 0, 0);
  }
}

// NN weight tile: thread t holds 8 consecutive k rows x NWN consecutive n
// columns, to be written transposed into LDS.
template <class C>
__device__ __forceinline__ void nn_load(__amdgpu_buffer_rsrc_t rs, int N, int n0, int kt, int (&nb)[8 * C::NWN / 2]) {
  constexpr int NB = C::BN / C::NWN;
  const int tid = threadIdx.x;
  const int nbk = tid % NB, kb = tid / NB;
  const int nbase = n0 + nbk * C::NWN;
#pragma unroll
  for (int kr = 0; kr < 8; ++kr) {
    const int k = kt * C::BK + kb * 8 + kr;
    if constexpr (C::NWN == 2) {
      nb[kr] = __builtin_amdgcn_raw_buffer_load_b32(rs, (k * N + nbase) * 2, 0, 0);
    } else {
      i32x2 v = __builtin_amdgcn_raw_buffer_load_b64(rs, (k * N + nbase) * 2, 0, 0);
      nb[2 * kr] = v[0];
      nb[2 * kr + 1] = v[1];
    }
  }
}

template <class C>
__device__ __forceinline__ void nn_store(const int (&nb)[8 * C::NWN / 2], char* sb) {
  constexpr int NB = C::BN / C::NWN;
  constexpr int WPR = C::NWN / 2;  // 32-bit words per k row
  const int tid = threadIdx.x;
  const int nbk = tid % NB, kb = tid / NB;
#pragma unroll
  for (int j = 0; j < C::NWN; ++j) {
    i32x4 v;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const uint32_t w0 = (uint32_t)nb[(2 * q) * WPR + j / 2];
      const uint32_t w1 = (uint32_t)nb[(2 * q + 1) * WPR + j / 2];
      const uint32_t lo = (j & 1) ? (w0 >> 16) : (w0 & 0xFFFFu);
      const uint32_t hi = (j & 1) ? (w1 & 0xFFFF0000u) : (w1 << 16);
      v[q] = (int)(lo | hi);
    }
    *reinterpret_cast<i32x4*>(sb + lds_off64(nbk * C::NWN + j, kb)) = v;
  }
}

struct BigSrc {
  __amdgpu_buffer_rsrc_t a, b;
};

template <class C>
__device__ __forceinline__ BigSrc big_src(const Params& p, const BigItem& it) {
  const int K = p.K, N = p.N;
  BigSrc s;
  const char* lhs = reinterpret_cast<const char*>(p.lhs) + (long long)it.row0 * K * 2;
  s.a = make_rsrc(lhs, (long long)it.rows * K * 2);
  const char* rhs_h = reinterpret_cast<const char*>(p.rhs) + (long long)it.h * N * K * 2;
  if constexpr (C::NN)
    s.b = make_rsrc(rhs_h, (long long)K * N * 2);
  else
    s.b = make_rsrc(rhs_h + (long long)it.n0 * K * 2, (long long)it.ncols * K * 2);
  return s;
}

// s_waitcnt with only the vector-memory counter constrained (gfx9 encoding:
// vmcnt low bits [3:0], high bits [15:14]; expcnt [6:4] and lgkmcnt [11:8]
// left at their maxima).
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (0x7 << 4) | (0xF << 8));
}

// Wait until at most n vector-memory loads of this wave are outstanding,
// rounding n down to a supported immediate (waiting longer is always safe).
__device__ __forceinline__ void wait_loads_at_most(int n) {
  if (n >= 32)
    wait_vmcnt<32>();
  else if (n >= 24)
    wait_vmcnt<24>();
  else if (n >= 16)
    wait_vmcnt<16>();
  else if (n >= 12)
    wait_vmcnt<12>();
  else if (n >= 8)
    wait_vmcnt<8>();
  else if (n >= 4)
    wait_vmcnt<4>();
  else
    wait_vmcnt<0>();
}

// Position in a workgroup's stream of K steps: item L (linear tile index),
// its K tile kt, and the decoded item.
struct Cursor {
  int step;
  int L;
  int kt;
  BigItem it;
};

template <class C>
__device__ __forceinline__ void advance(Cursor& c, const Plan& pl, int KT, int P, int n_items, int n_ntiles,
                                        int N, int w) {
  ++c.step;
  if (++c.kt == KT) {
    c.kt = 0;
    c.L += P;
    if (c.L < n_items) c.it = decode_big<C>(pl, c.L, n_ntiles, N, w);
  }
}

template <class C>
__device__ __forceinline__ void read_frags(i32x4 (&a)[C::FM], i32x4 (&b)[C::FN], const char* stage,
                                           const BigItem& it, int q, int r16) {
  // Rows past a half tile's share are read too (wrapped into the tile; the
  // values are never used): unconditional reads keep the LDS queue full.
#pragma unroll
  for (int fm = 0; fm < C::FM; ++fm)
    a[fm] = *reinterpret_cast<const i32x4*>(stage + lds_off64((it.rbase + fm * 16 + r16) & (C::BM - 1), q));
  const char* sb = stage + C::A_BYTES;
#pragma unroll
  for (int fn = 0; fn < C::FN; ++fn)
    b[fn] = *reinterpret_cast<const i32x4*>(sb + lds_off64(it.cbase + fn * 16 + r16, q));
}

// acc[fm][fn] += a[fm] b[fn] for F0 <= fm < F1.  Half tiles run rows
// [0, FM/2) only; one conditional block for the upper rows keeps the
// accumulators in place (finer branching makes the register allocator copy
// them around).
template <class C, int F0, int F1>
__device__ __forceinline__ void mfma_rows(f32x4 (&acc)[C::FM][C::FN], const i32x4 (&a)[C::FM],
                                          const i32x4 (&b)[C::FN]) {
#pragma unroll
  for (int fm = F0; fm < F1; ++fm)
#pragma unroll
    for (int fn = 0; fn < C::FN; ++fn)
      acc[fm][fn] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a[fm]),
                                                            __builtin_bit_cast(bf16x8, b[fn]), acc[fm][fn], 0, 0,
                                                            0);
}

template <class C, int FMA>
__device__ __forceinline__ void big_epilogue(const Params& p, const f32x4 (&acc)[C::FM][C::FN],
                                             const BigItem& it, int q, int r16) {
  const int N = p.N;
  const int cl0 = it.cbase + r16;
  // bias of this lane's columns (added once, after the products)
  float bias[C::FN];
#pragma unroll
  for (int fn = 0; fn < C::FN; ++fn) {
    bias[fn] = 0.f;
    const int cl = cl0 + fn * 16;
    if (p.rhs_bias && cl < it.ncols) {
      const long long bi = (long long)it.h * N + it.n0 + cl;
      bias[fn] = p.bias_f32 ? reinterpret_cast<const float*>(p.rhs_bias)[bi]
                            : bf16_bits_to_f32(reinterpret_cast<const uint16_t*>(p.rhs_bias)[bi]);
    }
  }
#pragma unroll
  for (int fm = 0; fm < FMA; ++fm) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int rl = it.rbase + fm * 16 + 4 * q + i;
      if (rl >= it.rows) continue;
      const long long rbase = (long long)(it.row0 + rl) * N + it.n0 + cl0;
      if constexpr (C::OUT_F32) {
        float* op = reinterpret_cast<float*>(p.out) + rbase;
#pragma unroll
        for (int fn = 0; fn < C::FN; ++fn)
          if (cl0 + fn * 16 < it.ncols) op[fn * 16] = acc[fm][fn][i] + bias[fn];
      } else {
        uint16_t* op = reinterpret_cast<uint16_t*>(p.out) + rbase;
#pragma unroll
        for (int fn = 0; fn < C::FN; ++fn)
          if (cl0 + fn * 16 < it.ncols) op[fn * 16] = f32_to_bf16_rne(acc[fm][fn][i] + bias[fn]);
      }
    }
  }
}

template <class C>
__global__ __launch_bounds__(C::T) __attribute__((amdgpu_waves_per_eu(2, 2)))
void gmm_big_kernel(Params p) {
  __shared__ __attribute__((aligned(1024))) char smem[C::LDS];
  __shared__ Plan pl;
  if (threadIdx.x == 0) pl.flags = 0;
  __syncthreads();
  build_plan<C::T>(p, pl, C::BM);
  report_flags(p, pl);

  const int tid = threadIdx.x, lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int q = lane >> 4, r16 = lane & 15;
  const int M = p.M, N = p.N, K = p.K;
  const int P = gridDim.x;
  const int slot = xcd_slot(blockIdx.x, P);

  // rows outside the active groups: zero them first (grid-stride)
  {
    constexpr int out_es = C::OUT_F32 ? 4 : 2;
    const long long row_bytes = (long long)N * out_es;
    const int lo_row = pl.row_start[0], hi_row = pl.row_start[pl.ga];
    char* out = reinterpret_cast<char*>(p.out);
    const i32x4 z = {0, 0, 0, 0};
    const long long z1 = (long long)lo_row * row_bytes;
    const long long z2b = (long long)hi_row * row_bytes, z2e = (long long)M * row_bytes;
    const long long total = z1 + (z2e - z2b);
    for (long long off = ((long long)slot * C::T + tid) * 16; off < total; off += (long long)P * C::T * 16) {
      const long long o = off < z1 ? off : z2b + (off - z1);
      *reinterpret_cast<i32x4*>(out + o) = z;
    }
  }

  const int n_ntiles = (N + C::BN - 1) / C::BN;
  const int n_items = __builtin_amdgcn_readfirstlane(pl.n_mtiles) * n_ntiles;
  const int KT = K / C::BK;
  if (slot >= n_items) return;
  // This workgroup's items are slot, slot + P, ...; their K tiles form one
  // stream of `total` steps.
  const int total = (n_items - slot + P - 1) / P * KT;

  Cursor first;
  first.step = 0;
  first.L = slot;
  first.kt = 0;
  first.it = decode_big<C>(pl, slot, n_ntiles, N, w);

  // Loads per step and wave: DMA_A (+ DMA_B when NT) direct-to-LDS, plus 8
  // register loads of the weight when NN.  Loads retire in order, so "all
  // loads up to step x's have landed" is "at most <loads issued after
  // them> outstanding".
  constexpr int DMA_A = C::DMA_PER_OPERAND;
  constexpr int DMA_STEP = C::NN ? DMA_A : 2 * DMA_A;
  constexpr int NN_STEP = C::NN_LOADS;

  Cursor ld = first;  // next step whose operands go to LDS
  BigSrc ld_src = big_src<C>(p, ld.it);
  auto issue = [&]() __attribute__((always_inline)) {
    char* st = smem + (ld.step % C::S) * C::STAGE;
    dma_rows<C>(ld_src.a, K * 2, ld.kt, st);
    if constexpr (!C::NN) dma_rows<C>(ld_src.b, K * 2, ld.kt, st + C::A_BYTES);
    const int old_L = ld.L;
    advance<C>(ld, pl, KT, P, n_items, n_ntiles, N, w);
    if (ld.L != old_L && ld.step < total) ld_src = big_src<C>(p, ld.it);
  };

  // NN: the weight part of step x goes through registers: loaded in the
  // iteration of step x-1, written to LDS at its end.  nn_step is the next
  // such step; it is always cur.step + 1 once the loop runs.
  int nn_step = 0;
  int nb[8 * C::NWN / 2];
  auto nn_load_for = [&](const BigItem& it, int kt) __attribute__((always_inline)) {
    const char* rhs_h = reinterpret_cast<const char*>(p.rhs) + (long long)it.h * N * K * 2;
    nn_load<C>(make_rsrc(rhs_h, (long long)K * N * 2), N, it.n0, kt, nb);
  };
  auto nn_store_for = [&](int step) __attribute__((always_inline)) {
    nn_store<C>(nb, smem + (step % C::S) * C::STAGE + C::A_BYTES);
  };

  // Loads issued after the DMA of step x, as of the top of the iteration of
  // step x.  DMA(x) is issued in the prologue when x < S, else in the
  // iteration of step x-S+1 (refilling the stage read in step x-S), after
  // that iteration's NN loads.
  auto newer_than = [&](int x) __attribute__((always_inline)) {
    int n = DMA_STEP * (ld.step - x - 1);
    if constexpr (C::NN) {
      // NN loads of step y are issued in the iteration of step y-1 (step 0's
      // in the prologue, after its DMAs); those after DMA(x) are y >= y0.
      const int y0 = x < C::S ? 0 : x - C::S + 3;
      n += NN_STEP * (nn_step - y0 > 0 ? nn_step - y0 : 0);
    }
    return n;
  };

  // Prologue: S stages in flight; the NN weight of step 0 in LDS.
#pragma unroll
  for (int s = 0; s < C::S; ++s)
    if (ld.step < total) issue();
  if constexpr (C::NN) {
    nn_load_for(first.it, 0);
    nn_store_for(0);
    nn_step = 1;
  }
  wait_loads_at_most(newer_than(0));
  __syncthreads();

  Cursor cur = first;
  // the item after cur's (for the NN weight one step ahead)
  BigItem nxt = first.it;
  if (C::NN && slot + P < n_items) nxt = decode_big<C>(pl, slot + P, n_ntiles, N, w);
  f32x4 acc[C::FM][C::FN];
#pragma unroll
  for (int x = 0; x < C::FM; ++x)
#pragma unroll
    for (int y = 0; y < C::FN; ++y) acc[x][y] = f32x4{0.f, 0.f, 0.f, 0.f};

  while (cur.step < total) {
    const int s = cur.step;
    const char* st = smem + (s % C::S) * C::STAGE;
    if (s > 0) {
      // this step's operands: this wave's loads, then every wave's (the
      // barrier also frees the stage refilled below, read in step s-1)
      wait_loads_at_most(newer_than(s));
      __syncthreads();
    }
    i32x4 a[C::FM], b[C::FN];
    read_frags<C>(a, b, st, cur.it, q, r16);
    const bool nn_more = C::NN && nn_step < total;
    if constexpr (C::NN) {
      if (nn_more) {
        if (cur.kt + 1 < KT)
          nn_load_for(cur.it, cur.kt + 1);
        else
          nn_load_for(nxt, 0);
      }
    }
    if (s > 0 && ld.step < total) issue();
    const BigItem& it = cur.it;
    mfma_rows<C, 0, C::FM / 2>(acc, a, b);
    if (!it.half) mfma_rows<C, C::FM / 2, C::FM>(acc, a, b);
    if constexpr (C::NN) {
      if (nn_more) {
        nn_store_for(nn_step);
        ++nn_step;
      }
    }
    if (cur.kt == KT - 1) {
      if (!it.half)
        big_epilogue<C, C::FM>(p, acc, it, q, r16);
      else
        big_epilogue<C, C::FM / 2>(p, acc, it, q, r16);
#pragma unroll
      for (int x = 0; x < C::FM; ++x)
#pragma unroll
        for (int y = 0; y < C::FN; ++y) acc[x][y] = f32x4{0.f, 0.f, 0.f, 0.f};
    }
    const int old_L = cur.L;
    advance<C>(cur, pl, KT, P, n_items, n_ntiles, N, w);
    if (C::NN && cur.L != old_L && cur.L + P < n_items) nxt = decode_big<C>(pl, cur.L + P, n_ntiles, N, w);
  }
}

}  // namespace gmmk
