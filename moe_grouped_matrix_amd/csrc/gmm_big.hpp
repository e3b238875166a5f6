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
// each, 32 KB) sits in one of four LDS stages that form a ring.  While the
// waves multiply step s (fragments already in registers), they read step
// s+1's fragments from LDS, and steps s+2..s+4 -- of the same output tile, or
// the first ones of the workgroup's next output tile -- are in flight.  Operands
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

// Queue the direct-to-LDS loads of K step kt (both operands when NT, lhs
// only when NN) into LDS stage `st`; voff are this lane's row offsets.
template <class C>
__device__ __forceinline__ void dma_stage(const BigSrc& src, const int (&voff)[C::DMA_PER_OPERAND], int kt,
                                          char* st, int w) {
#pragma unroll
  for (int i = 0; i < C::DMA_PER_OPERAND; ++i) {
    char* dst = st + (w * C::ROWS_PER_WAVE + i * 16) * C::ROW;
    __builtin_amdgcn_raw_ptr_buffer_load_lds(src.a, (lds_ptr_t)dst, 16, voff[i], kt * C::ROW, 0, 0);
    if constexpr (!C::NN)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(src.b, (lds_ptr_t)(dst + C::A_BYTES), 16, voff[i], kt * C::ROW,
                                               0, 0);
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

// Fragment rows start at multiples of 16, so a fragment's swizzled chunk
// depends only on the lane: lane (q, r16) reads row base + r16, chunk
// q ^ swz64(r16).  Fragment f of a wave is then one base address plus an
// immediate f * 16 rows.  (Rows past a half tile's share may run into the B
// part of the stage: they are read, never used.)
__device__ __forceinline__ int frag_lane_off(int q, int r16) { return r16 * 64 + ((q ^ swz64(r16)) << 4); }

template <class C>
__device__ __forceinline__ void read_a_at(i32x4& a, const char* base, int fm) {
  a = *reinterpret_cast<const i32x4*>(base + fm * 16 * C::ROW);
}

template <class C>
__device__ __forceinline__ void read_b_at(i32x4 (&b)[C::FN], const char* base) {
#pragma unroll
  for (int fn = 0; fn < C::FN; ++fn) b[fn] = *reinterpret_cast<const i32x4*>(base + fn * 16 * C::ROW);
}

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
  const int KT = K / C::BK;  // K steps per item; the launcher guarantees KT >= S
  if (slot >= n_items) return;

  // This workgroup's items are slot, slot + P, ...; their K steps form one
  // stream.  Loads run S steps ahead of the multiplication, fragment reads
  // one step ahead, NN weight loads two steps ahead -- within the current
  // item or, near its end, in the next one.
  BigItem cur = decode_big<C>(pl, slot, n_ntiles, N, w);
  int cur_L = slot;
  BigItem nxt = cur;
  if (slot + P < n_items) nxt = decode_big<C>(pl, slot + P, n_ntiles, N, w);
  BigSrc cur_src = big_src<C>(p, cur), nxt_src = big_src<C>(p, nxt);

  // Per-lane byte offsets of this wave's direct-to-LDS rows (the K step adds
  // a scalar offset): operand rows r = 16 i + lane/4 of the wave's share.
  const int row_bytes = K * 2;
  int dma_voff[C::DMA_PER_OPERAND];
#pragma unroll
  for (int i = 0; i < C::DMA_PER_OPERAND; ++i) {
    const int r = w * C::ROWS_PER_WAVE + i * 16 + (lane >> 2);
    dma_voff[i] = r * row_bytes + (((lane & 3) ^ swz64(r)) << 4);
  }
  auto dma = [&](const BigSrc& src, int kt, int stage) __attribute__((always_inline)) {
    dma_stage<C>(src, dma_voff, kt, smem + stage * C::STAGE, w);
  };
  int nb[8 * C::NWN / 2];
  auto nn_load_for = [&](const BigItem& it, int kt) __attribute__((always_inline)) {
    const char* rhs_h = reinterpret_cast<const char*>(p.rhs) + (long long)it.h * N * K * 2;
    nn_load<C>(make_rsrc(rhs_h, (long long)K * N * 2), N, it.n0, kt, nb);
  };

  // Prologue: the first S steps in flight (the launcher guarantees the
  // first item has KT >= S steps); NN weights of steps 0 and 1 in LDS.
#pragma unroll
  for (int s = 0; s < C::S; ++s) dma(cur_src, s, s);
  if constexpr (C::NN) {
    nn_load_for(cur, 0);
    nn_store<C>(nb, smem + C::A_BYTES);
    nn_load_for(cur, 1);
    nn_store<C>(nb, smem + C::STAGE + C::A_BYTES);
  }
  wait_vmcnt<0>();
  __syncthreads();

  f32x4 acc[C::FM][C::FN];
#pragma unroll
  for (int x = 0; x < C::FM; ++x)
#pragma unroll
    for (int y = 0; y < C::FN; ++y) acc[x][y] = f32x4{0.f, 0.f, 0.f, 0.f};

  const int lane_off = frag_lane_off(q, r16);
  i32x4 a[C::FM], b0[C::FN], b1[C::FN];
  {
    const char* abase = smem + cur.rbase * C::ROW + lane_off;
#pragma unroll
    for (int fm = 0; fm < C::FM; ++fm) read_a_at<C>(a[fm], abase, fm);
    read_b_at<C>(b0, smem + C::A_BYTES + cur.cbase * C::ROW + lane_off);
  }

  // Loads issued per step and wave: DMA_STEP direct-to-LDS, plus (NN) 8
  // weight loads two steps ahead.  In steady state the loads of the next
  // step have completed once at most STEADY newer loads are outstanding
  // (loads retire in order; outstanding stores only make the wait longer).
  constexpr int DMA_STEP = C::NN ? C::DMA_PER_OPERAND : 2 * C::DMA_PER_OPERAND;
  constexpr int STEADY = C::NN ? 2 * DMA_STEP : (C::S - 2) * DMA_STEP;

  int stage = 0;  // stage of the current step
  for (int L = slot;;) {
    const bool last_item = L + P >= n_items;
    for (int kt = 0; kt < KT; ++kt) {
      const bool more = !(last_item && kt == KT - 1);  // a step follows
      const int st1 = (stage + 1) & (C::S - 1);
      if (more) {
        // step s+1's operands: this wave's loads, then every wave's; the
        // barrier also frees the current stage (its fragments are in
        // registers) for the refill below
        if (last_item && kt + C::S > KT)
          wait_vmcnt<0>();  // fewer newer loads near the end of the stream
        else
          wait_vmcnt<STEADY>();
        __syncthreads();
        const BigItem& it1 = kt + 1 < KT ? cur : nxt;
        read_b_at<C>(b1, smem + st1 * C::STAGE + C::A_BYTES + it1.cbase * C::ROW + lane_off);
        if constexpr (C::NN) {
          if (!(last_item && kt + 2 >= KT)) {
            if (kt + 2 < KT)
              nn_load_for(cur, kt + 2);
            else
              nn_load_for(nxt, kt + 2 - KT);
          }
        }
        // refill the current stage with step s+S
        if (kt + C::S < KT)
          dma(cur_src, kt + C::S, stage);
        else if (!last_item)
          dma(nxt_src, kt + C::S - KT, stage);
      }
      const BigItem& it1 = kt + 1 < KT ? cur : nxt;
      const char* abase = smem + st1 * C::STAGE + it1.rbase * C::ROW + lane_off;
      // rows [0, FM/2) always; the upper rows only for full tiles.  Each A
      // fragment is refilled with step s+1's right after its last use.
#pragma unroll
      for (int fm = 0; fm < C::FM / 2; ++fm) {
#pragma unroll
        for (int fn = 0; fn < C::FN; ++fn)
          acc[fm][fn] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a[fm]),
                                                                __builtin_bit_cast(bf16x8, b0[fn]),
                                                                acc[fm][fn], 0, 0, 0);
        read_a_at<C>(a[fm], abase, fm);
      }
      if (!cur.half) mfma_rows<C, C::FM / 2, C::FM>(acc, a, b0);
#pragma unroll
      for (int fm = C::FM / 2; fm < C::FM; ++fm) read_a_at<C>(a[fm], abase, fm);
      if constexpr (C::NN) {
        if (more && !(last_item && kt + 2 >= KT)) nn_store<C>(nb, smem + ((stage + 2) & (C::S - 1)) * C::STAGE + C::A_BYTES);
      }
#pragma unroll
      for (int fn = 0; fn < C::FN; ++fn) b0[fn] = b1[fn];
      stage = st1;
    }
    if (!cur.half)
      big_epilogue<C, C::FM>(p, acc, cur, q, r16);
    else
      big_epilogue<C, C::FM / 2>(p, acc, cur, q, r16);
    if (last_item) break;
#pragma unroll
    for (int x = 0; x < C::FM; ++x)
#pragma unroll
      for (int y = 0; y < C::FN; ++y) acc[x][y] = f32x4{0.f, 0.f, 0.f, 0.f};
    L += P;
    cur = nxt;
    cur_src = nxt_src;
    if (L + P < n_items) {
      nxt = decode_big<C>(pl, L + P, n_ntiles, N, w);
      nxt_src = big_src<C>(p, nxt);
    }
  }
}

}  // namespace gmmk
