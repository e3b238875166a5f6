// gmm_stream.hpp -- the weight-streaming kernel of the gfx950 grouped matmul:
// bf16 lhs x narrow weight [G,N,K] (e4m3fn, e5m2 or int8, or packed int4,
// uint4 or fp4 e2m1, widened exactly to bf16) with per-block rhs_scale and
// an optional bias, for problems with few rows per group (decode), where
// the run time is the time to read every active group's weight once from
// HBM.
//
// Output tiles are 64 rows (group-aligned) x 256 columns; a tile reads its
// group's 256 x K weight slab once, so a group of up to 64 rows reads its
// weight once.  K is consumed in stages of 128 (one quantisation block of
// the scale; without a scale every block counts 1), each stage holding in
// LDS the weight slab (256 rows of 128 bytes), the tile's lhs rows (64 rows
// of 256 bytes), the block's 256 scales and the tile's 256 bias values.
// Three stages form a ring filled by direct-to-LDS loads two stages ahead,
// across the workgroup's tiles, so the HBM stream never drains.  Eight
// waves, two per SIMD: wave w computes columns 32 w .. +32 for all 64 rows
// (two 32-row blocks) over the whole of K with 32x32x16 bf16 MFMAs, so no
// partial sums cross waves and each weight byte is widened by one wave
// only.  The weight fragment is the MFMA's first operand (a lane holds runs
// of four columns of one row), widened from its one-byte format to bf16 in
// registers and used for both row blocks, and each block's product is
// folded into fp32 totals with that block's scales.
//
// What sets the shape: the lhs rows share the LDS ring with the weights,
// and the widest tile moves the most weight per lhs byte (64-row tiles 32,
// 64, 128 and 256 columns wide ran a 128-K stage in 0.49, 0.67, 1.05 and
// 2.1 us; 32 x 64 tiles, which also read each expert's weight once per 32
// rows, took 38.9 us per decode call against 33.4 us).  A stage's own work
// (widening the weight, the scale fold, the MFMAs, the LDS reads) is what
// sets its time, not the HBM stream: with the weight loads dropped the call
// still took 27.0 of 31.3 us.  So each weight byte is widened by one wave
// (32.3 us, from 33.3 with two), two waves share each SIMD to hide each
// other's latencies (29.3 us, from 31.6 with one), and the wait for the next
// stage comes after the multiply (27.6 us).
//
// Every wave issues the same loads in every stage (four weight and two
// lhs; wave 0 also the scales, wave 1 the bias; loads past a range return
// zeros and still count) and the same stores per tile, so the vmcnt waits
// are constants (one set for waves 0 and 1, one for the others).
#pragma once

#include "gmm_big.hpp"

namespace gmmk {

// FB_: the weight's format: one byte (0 e4m3fn, 1 e5m2, 2 int8) or four
// bits, two to a byte with the even element in the low nibble (3 int4,
// 4 uint4, 5 fp4 e2m1).
template <bool OUT_F32_, int FB_ = 0>
struct StreamCfg {
  static constexpr bool OUT_F32 = OUT_F32_;
  static constexpr int FB = FB_;
  static constexpr int BM = 64, BN = 256, BKS = 128;  // tile rows, tile columns, K per stage
  static constexpr int NWAVES = 8, T = 64 * NWAVES;
  static constexpr bool NIB = FB >= 3;  // four-bit weights
  static constexpr int W_ROW = NIB ? BKS / 2 : BKS, A_ROW = BKS * 2;  // bytes per weight / lhs row in a stage
  static constexpr int W_CHUNKS = W_ROW / 16;  // 16-byte chunks per weight row (8, or 4 for four bits)
  static constexpr int W_BYTES = BN * W_ROW, A_BYTES = BM * A_ROW;
  // the block's scales (256 f32) and the tile's bias (256 values): one
  // 16-byte-per-lane load each, whose 64 lanes all write the slot
  static constexpr int SLOT = 1024;
  static constexpr int SC_OFF = W_BYTES + A_BYTES, BI_OFF = SC_OFF + SLOT;
  static constexpr int STAGE = BI_OFF + SLOT;
  static constexpr int S = 3;
  static constexpr int RING = S * STAGE;
  static constexpr int LDS = RING;
  static constexpr int W_OPS = W_BYTES / 1024 / NWAVES, A_OPS = A_BYTES / 1024 / NWAVES;
  // loads per stage: waves 0 and 1 one more (the scales, the bias)
  static constexpr int OPS_LO = W_OPS + A_OPS, OPS_HI = OPS_LO + 1;
  static constexpr int FM = 2, FN = 1;  // 32-row and 32-column blocks per wave
  static constexpr int WCOLS = 32 * FN;  // columns per wave
  static constexpr int es_out = OUT_F32 ? 4 : 2;
  static constexpr int E = FM * FN * (OUT_F32 ? 4 : 2);  // 16-byte stores per wave and tile
  static_assert(W_OPS * NWAVES * 1024 == W_BYTES && A_OPS * NWAVES == 16, "load split");
  static_assert(WCOLS * NWAVES == BN, "the waves cover the tile's columns");
};

// 128-byte weight rows: chunk c of row n at c ^ swz_w(n); 64-byte (four-bit)
// weight rows: at c ^ swz_w4(n); 256-byte lhs rows: chunk c of row r at
// c ^ (r & 15).  Sixteen consecutive weight or lhs rows read at one logical
// chunk then land in distinct 16-byte bank groups.
__device__ __forceinline__ int swz_w(int n) { return (n & 7) ^ ((n >> 3) & 1); }
__device__ __forceinline__ int swz_w4(int n) { return (n >> 2) & 3; }
template <class C>
__device__ __forceinline__ int swz_row(int n) { return C::NIB ? swz_w4(n) : swz_w(n); }
__device__ __forceinline__ int swz_a(int r) { return r & 15; }

struct StreamItem {
  int h, row0, rows, n0, ncols;
};

template <class C>
__device__ __forceinline__ StreamItem decode_stream(const Plan& pl, int L, int n_ntiles, int N) {
  StreamItem it;
  const int t = L / n_ntiles;
  const int j = L % n_ntiles;
  const int h = find_group(pl, t);
  const int row0 = pl.row_start[h] + (t - pl.tile_start[h]) * C::BM;
  const int left = pl.row_start[h + 1] - row0;
  it.h = __builtin_amdgcn_readfirstlane(h);
  it.row0 = __builtin_amdgcn_readfirstlane(row0);
  it.rows = __builtin_amdgcn_readfirstlane(left < C::BM ? left : C::BM);
  it.n0 = j * C::BN;
  it.ncols = N - it.n0 < C::BN ? N - it.n0 : C::BN;
  return it;
}

// Buffer resources of one tile's four sources (zero-size when `live` is
// false: past the end of the stream).
struct StreamSrc {
  __amdgpu_buffer_rsrc_t ra, rw, rs, rb;
  int ncols;
};

template <class C>
__device__ __forceinline__ StreamSrc stream_src(const Params& p, const StreamItem& it, bool live) {
  const int K = p.K, N = p.N;
  StreamSrc s;
  const char* a = reinterpret_cast<const char*>(p.lhs) + (long long)it.row0 * K * 2;
  const int wrow = C::NIB ? K / 2 : K;  // weight bytes per row
  const char* w = reinterpret_cast<const char*>(p.rhs) + ((long long)it.h * N + it.n0) * wrow;
  s.ra = uniform_rsrc(a, live ? it.rows * K * 2 : 0);
  s.rw = uniform_rsrc(w, live ? it.ncols * wrow : 0);
  if (p.rhs_scale) {
    const char* sc = reinterpret_cast<const char*>(p.rhs_scale) + ((long long)it.h * p.nb * N + it.n0) * 4;
    s.rs = uniform_rsrc(sc, live ? p.nb * N * 4 - it.n0 * 4 : 0);
  } else {
    s.rs = uniform_rsrc(a, 0);
  }
  const int bes = p.bias_f32 ? 4 : 2;
  if (p.rhs_bias) {
    const char* b = reinterpret_cast<const char*>(p.rhs_bias) + ((long long)it.h * N + it.n0) * bes;
    s.rb = uniform_rsrc(b, live ? it.ncols * bes : 0);
  } else {
    s.rb = uniform_rsrc(a, 0);
  }
  s.ncols = it.ncols;
  return s;
}

// Per-lane offsets of this wave's loads.  Its weight load i is load
// j = 8 i + w of the stage: rows 8 j + lane/8, chunk lane%8 (four-bit
// weights: rows 16 j + lane/4, chunk lane%4).  Its lhs load i is load
// j = 8 i + w: rows 4 j + lane/16, chunk lane%16.  Wave 0 also
// loads the block's scales (lane: columns 4 lane .. +4) and wave 1 the bias
// (lane: columns 8 lane .. +8 for bf16, lanes < 32; 4 lane .. +4 for f32).
// The column test is made per tile (stream_stage).
struct StreamOff {
  int w[8], a[4], xcols;  // xcols: the first column of this lane's scale / bias chunk, or 1 << 20
};

template <class C>
__device__ __forceinline__ StreamOff stream_offsets(int K, int w, int lane, bool bias_f32) {
  StreamOff o;
#pragma unroll
  for (int i = 0; i < C::W_OPS; ++i) {
    if constexpr (C::NIB) {
      const int n = 16 * (C::NWAVES * i + w) + (lane >> 2);
      o.w[i] = n * (K / 2) + (((lane & 3) ^ swz_w4(n)) << 4);
    } else {
      const int n = 8 * (C::NWAVES * i + w) + (lane >> 3);
      o.w[i] = n * K + (((lane & 7) ^ swz_w(n)) << 4);
    }
  }
#pragma unroll
  for (int i = 0; i < C::A_OPS; ++i) {
    const int r = 4 * (C::NWAVES * i + w) + (lane >> 4);
    o.a[i] = r * K * 2 + (((lane & 15) ^ swz_a(r)) << 4);
  }
  if (w == 1 && !bias_f32)
    o.xcols = lane < 32 ? 8 * lane : 1 << 20;
  else
    o.xcols = 4 * lane;
  return o;
}

// The loads of stage k (K elements [128 k, 128 k + 128), scale block k) of
// a tile into LDS stage `st`: every wave its weight and lhs rows, wave 0 the
// block's scales, wave 1 the tile's bias.  N is a multiple of 8, so a
// lane's 16-byte scale or bias chunk is all inside the tile's columns or
// all outside.
template <class C>
__device__ __forceinline__ void stream_stage(const StreamSrc& s, const StreamOff& o, int k, int N, char* st, int w) {
#pragma unroll
  for (int i = 0; i < C::W_OPS; ++i)
    __builtin_amdgcn_raw_ptr_buffer_load_lds(s.rw, (lds_ptr_t)(st + (C::NWAVES * i + w) * 1024), 16, o.w[i],
                                             k * C::W_ROW, 0, 0);
#pragma unroll
  for (int i = 0; i < C::A_OPS; ++i)
    __builtin_amdgcn_raw_ptr_buffer_load_lds(s.ra, (lds_ptr_t)(st + C::W_BYTES + (C::NWAVES * i + w) * 1024), 16,
                                             o.a[i], k * C::A_ROW, 0, 0);
  const int xv = o.xcols < s.ncols ? (int)(threadIdx.x & 63) * 16 : (int)0x80000000;
  if (w == 0)
    __builtin_amdgcn_raw_ptr_buffer_load_lds(s.rs, (lds_ptr_t)(st + C::SC_OFF), 16, xv, k * N * 4, 0, 0);
  else if (w == 1)
    __builtin_amdgcn_raw_ptr_buffer_load_lds(s.rb, (lds_ptr_t)(st + C::BI_OFF), 16, xv, 0, 0, 0);
}

// s_waitcnt vmcnt for this wave: waves 0 and 1 issue one load more per stage.
template <int N_LO, int N_HI>
__device__ __forceinline__ void wait_stream(int w) {
  if (w < 2)
    wait_vmcnt<N_HI>();
  else
    wait_vmcnt<N_LO>();
}

template <class C>
__global__ __launch_bounds__(C::T) void gmm_stream_kernel(Params p) {
  // one LDS array (a second LDS variable would make the compiler drain the
  // direct-to-LDS loads in flight before every LDS read)
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
  const int n_ntiles = (N + C::BN - 1) / C::BN;
  const int n_items = __builtin_amdgcn_readfirstlane(pl.n_mtiles) * n_ntiles;
  const int KT = K / C::BKS;  // stages per tile; the launcher guarantees KT >= S
  const bool scaled = p.rhs_scale != nullptr;  // in blocks of 128 (one stage) when present
  const bool bias_f32 = p.bias_f32 != 0;

  if (slot < n_items) {
    StreamItem cur = decode_stream<C>(pl, slot, n_ntiles, N);
    StreamItem nxt = cur;
    int L = slot;
    bool last_item = L + P >= n_items;
    if (!last_item) nxt = decode_stream<C>(pl, L + P, n_ntiles, N);
    StreamSrc scur = stream_src<C>(p, cur, true), snxt = stream_src<C>(p, nxt, !last_item);
    const StreamOff off = stream_offsets<C>(K, w, lane, bias_f32);

    // prologue: stages 0 .. S-2 of the first tile, then E range-dropped
    // stores (each to an address of its own, so none is merged away) in
    // place of a previous tile's epilogue stores, so that the first tile
    // finds the same operations outstanding as every later one and the
    // loop's constant waits hold for it too.  Only stage 0 is waited for:
    // all workgroups ask for their first S-1 stages at once, and the last of
    // those arrive several microseconds after the first.
#pragma unroll
    for (int st = 0; st < C::S - 1; ++st) stream_stage<C>(scur, off, st, N, smem + st * C::STAGE, w);
    {
      const __amdgpu_buffer_rsrc_t rz = uniform_rsrc(reinterpret_cast<const char*>(p.out), 0);
#pragma unroll
      for (int e = 0; e < C::E; ++e)
        __builtin_amdgcn_raw_buffer_store_b128(i32x4{0, 0, 0, 0}, rz, (int)0x80000000, 64 * e, 0);
    }
    wait_stream<(C::S - 2) * C::OPS_LO + C::E, (C::S - 2) * C::OPS_HI + C::E>(w);
    // a bare barrier, as in the loop: __syncthreads() carries a workgroup
    // fence, which the compiler meets by draining every load in flight
    ring_barrier();

    // lane parts of the fragment addresses (stage-relative).  32x32x16 K
    // step j of a stage (j = 0..7), lane half kh: K elements 64 kh + 8 j +
    // [0, 8) of the stage -- weight bytes 8 j .. of the lane's 64-byte run
    // (16-byte chunks 4 kh .. 4 kh + 3 of its column's 128-byte row; four-bit
    // weights: bytes 4 j .. of a 32-byte run, chunks 2 kh, 2 kh + 1 of a
    // 64-byte row), lhs chunk 8 kh + j of its row's 256-byte row.
    constexpr int WC = C::W_CHUNKS / 2;  // 16-byte weight chunks per lane and stage
    int w_off[C::FN][WC];
#pragma unroll
    for (int fb = 0; fb < C::FN; ++fb) {
      const int wn = C::WCOLS * w + 32 * fb + r32;  // weight row = tile column
#pragma unroll
      for (int c = 0; c < WC; ++c) w_off[fb][c] = wn * C::W_ROW + (((WC * kh + c) ^ swz_row<C>(wn)) << 4);
    }
    // lhs rows 32 fm + r32 (fm = 0, 1), the same swizzle
    const int a_base = C::W_BYTES + r32 * C::A_ROW;
    const int a_swz = swz_a(r32);
    // this lane's columns of block fb: WCOLS w + 32 fb + 8 g + 4 kh + [0, 4), g = 0..3
    const int col_l = C::WCOLS * w + 4 * kh;

    // a stage's fragments: the weight runs (64 one-byte values per column
    // block), the lhs rows (eight 16-byte chunks per row block), the
    // block's scales of the lane's columns
    i32x4 fw[C::FN][WC], fa[C::FM][8];
    f32x4 fsc[C::FN][4];
    auto read_frags = [&](const char* st) __attribute__((always_inline)) {
#pragma unroll
      for (int fb = 0; fb < C::FN; ++fb)
#pragma unroll
        for (int c = 0; c < WC; ++c) fw[fb][c] = *reinterpret_cast<const i32x4*>(st + w_off[fb][c]);
#pragma unroll
      for (int fm = 0; fm < C::FM; ++fm)
#pragma unroll
        for (int j = 0; j < 8; ++j)
          fa[fm][j] =
              *reinterpret_cast<const i32x4*>(st + a_base + fm * 32 * C::A_ROW + (((8 * kh + j) ^ a_swz) << 4));
#pragma unroll
      for (int fb = 0; fb < C::FN; ++fb)
#pragma unroll
        for (int g = 0; g < 4; ++g)
          fsc[fb][g] = scaled ? *reinterpret_cast<const f32x4*>(st + C::SC_OFF + (col_l + 32 * fb + 8 * g) * 4)
                              : f32x4{1.f, 1.f, 1.f, 1.f};
    };

    int stage = 0;
    read_frags(smem);  // stage 0 of the first tile
    f32x16 tot[C::FM * C::FN];  // block (fm, fb) at fm * FN + fb
#pragma unroll
    for (int b = 0; b < C::FM * C::FN; ++b)
#pragma unroll
      for (int i = 0; i < 16; ++i) tot[b][i] = 0.f;

    // One stage kt of the current tile.  The barrier at the end of the
    // previous stage freed the slot of stage kt-1 (every wave had read its
    // fragments), which now takes stage kt+S-1 (of this tile, or stage kd of
    // the next one when NEXT).  Stage kt's fragments, read into registers at
    // the end of the previous stage, are multiplied and folded with its
    // scales and, in a tile's last stage, the outputs stored.  Then stage
    // kt+1's loads are complete (this wave's, then every wave's after the
    // barrier) once at most the S-2 stages issued after it and, at a tile
    // boundary (WITH_E), the E stores between them are outstanding, and the
    // registers are refilled with stage kt+1's fragments.  Waiting there
    // rather than before the multiply keeps two stages' loads in flight
    // while a stage is multiplied (27.6 against 29.3 us per decode call).
    auto kstage = [&](auto wait_tag, auto next_tag, int kt, int kd) __attribute__((always_inline)) {
      constexpr bool WITH_E = decltype(wait_tag)::value;
      constexpr bool NEXT = decltype(next_tag)::value;
      stream_stage<C>(NEXT ? snxt : scur, off, kd, N, smem + ((stage + C::S - 1) % C::S) * C::STAGE, w);
      const char* st = smem + stage * C::STAGE;
#pragma unroll
      for (int fb = 0; fb < C::FN; ++fb) {
        f32x16 acc[C::FM];
#pragma unroll
        for (int fm = 0; fm < C::FM; ++fm)
#pragma unroll
          for (int i = 0; i < 16; ++i) acc[fm][i] = 0.f;
        if constexpr (C::NIB) {
#pragma unroll
          for (int j = 0; j < 8; ++j) {
            // word j % 4 of chunk j / 4 of the run: K step j's eight
            // nibbles, widened once for both row blocks
            const i32x4 bw = nib8_to_bf16x8<C::FB>((unsigned)fw[fb][j >> 2][j & 3]);
#pragma unroll
            for (int fm = 0; fm < C::FM; ++fm)
              acc[fm] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
                  __builtin_bit_cast(bf16x8, bw), __builtin_bit_cast(bf16x8, fa[fm][j]), acc[fm], 0, 0, 0);
          }
        } else {
#pragma unroll
          for (int c = 0; c < 4; ++c) {
            // weight bytes 16 c .. 16 c + 15 of the run: K steps 2 c, 2 c + 1,
            // widened once for both row blocks
            const i32x4 bw0 = fp8x8_to_bf16x8<C::FB>(i32x2{fw[fb][c][0], fw[fb][c][1]});
            const i32x4 bw1 = fp8x8_to_bf16x8<C::FB>(i32x2{fw[fb][c][2], fw[fb][c][3]});
#pragma unroll
            for (int fm = 0; fm < C::FM; ++fm) {
              acc[fm] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
                  __builtin_bit_cast(bf16x8, bw0), __builtin_bit_cast(bf16x8, fa[fm][2 * c]), acc[fm], 0, 0, 0);
              acc[fm] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
                  __builtin_bit_cast(bf16x8, bw1), __builtin_bit_cast(bf16x8, fa[fm][2 * c + 1]), acc[fm], 0, 0, 0);
            }
          }
        }
        // register 4 g + i holds column 8 g + 4 kh + i of the block for the lane's row
#pragma unroll
        for (int fm = 0; fm < C::FM; ++fm)
#pragma unroll
          for (int g = 0; g < 4; ++g)
#pragma unroll
            for (int i = 0; i < 4; ++i)
              tot[fm * C::FN + fb][4 * g + i] += acc[fm][4 * g + i] * fsc[fb][g][i];
      }
      if (kt == KT - 1) {
        // epilogue: bias from this stage's slot (its next use is past the
        // barrier below), round, and a permlane32 swap per pair of column
        // groups so that each lane stores eight consecutive columns of its
        // row with one 16-byte store (two for an f32 output); out-of-range
        // rows and columns drop
        char* tile = reinterpret_cast<char*>(p.out) + ((long long)cur.row0 * N + cur.n0) * C::es_out;
        const __amdgpu_buffer_rsrc_t ro = uniform_rsrc(tile, ((cur.rows - 1) * N + cur.ncols) * C::es_out);
#pragma unroll
        for (int b = 0; b < C::FM * C::FN; ++b) {
          const int row = 32 * (b / C::FN) + r32, fb = b % C::FN;
          float v[16];
#pragma unroll
          for (int g = 0; g < 4; ++g) {
            float bi[4] = {0.f, 0.f, 0.f, 0.f};
            const int cb = col_l + 32 * fb + 8 * g;  // first of the lane's four columns
            if (p.rhs_bias) {
              if (bias_f32) {
                const f32x4 b4 = *reinterpret_cast<const f32x4*>(st + C::BI_OFF + cb * 4);
                bi[0] = b4[0];
                bi[1] = b4[1];
                bi[2] = b4[2];
                bi[3] = b4[3];
              } else {
                const i32x2 b2 = *reinterpret_cast<const i32x2*>(st + C::BI_OFF + cb * 2);
                bi[0] = __uint_as_float((uint32_t)b2[0] << 16);
                bi[1] = __uint_as_float((uint32_t)b2[0] & 0xFFFF0000u);
                bi[2] = __uint_as_float((uint32_t)b2[1] << 16);
                bi[3] = __uint_as_float((uint32_t)b2[1] & 0xFFFF0000u);
              }
            }
#pragma unroll
            for (int i = 0; i < 4; ++i) v[4 * g + i] = tot[b][4 * g + i] + bi[i];
          }
#pragma unroll
          for (int gp = 0; gp < 4; gp += 2) {
            // after the swap: kh = 0 holds columns 8 gp + [0, 8) of the
            // block, kh = 1 holds 8 (gp + 1) + [0, 8)
            const int col = C::WCOLS * w + 32 * fb + 8 * (gp + kh);
            const int voff = col < cur.ncols ? (row * N + col) * C::es_out : (int)0x80000000;
            if constexpr (C::OUT_F32) {
              int lo[4], hi[4];
#pragma unroll
              for (int i = 0; i < 4; ++i) {
                const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v[4 * gp + i]),
                                                                __float_as_uint(v[4 * gp + 4 + i]), false, false);
                lo[i] = (int)r[0];
                hi[i] = (int)r[1];
              }
              __builtin_amdgcn_raw_buffer_store_b128(i32x4{lo[0], lo[1], lo[2], lo[3]}, ro, voff, 0, 0);
              __builtin_amdgcn_raw_buffer_store_b128(i32x4{hi[0], hi[1], hi[2], hi[3]}, ro, voff, 16, 0);
            } else {
              const uint32_t x00 = pk_bf16_rne(v[4 * gp], v[4 * gp + 1]);
              const uint32_t x01 = pk_bf16_rne(v[4 * gp + 2], v[4 * gp + 3]);
              const uint32_t x10 = pk_bf16_rne(v[4 * gp + 4], v[4 * gp + 5]);
              const uint32_t x11 = pk_bf16_rne(v[4 * gp + 6], v[4 * gp + 7]);
              const auto r0 = __builtin_amdgcn_permlane32_swap(x00, x10, false, false);
              const auto r1 = __builtin_amdgcn_permlane32_swap(x01, x11, false, false);
              __builtin_amdgcn_raw_buffer_store_b128(i32x4{(int)r0[0], (int)r1[0], (int)r0[1], (int)r1[1]}, ro,
                                                     voff, 0, 0);
            }
          }
#pragma unroll
          for (int i = 0; i < 16; ++i) tot[b][i] = 0.f;
        }
      }
      wait_stream<(C::S - 2) * C::OPS_LO + (WITH_E ? C::E : 0), (C::S - 2) * C::OPS_HI + (WITH_E ? C::E : 0)>(w);
      ring_barrier();
      const int stage1 = stage + 1 == C::S ? 0 : stage + 1;
      read_frags(smem + stage1 * C::STAGE);
      stage = stage1;
    };
    using WE = std::true_type;   // a tile boundary's stores are among the newer operations
    using WN = std::false_type;
    using CUR = std::false_type;
    using NXT = std::true_type;
    // With S = 3 (KT >= 3): the stores sit between stage 1 and stage 2 of a
    // tile, so the waits of its stage 0 (for stage 1) and of the previous
    // tile's last stage (for stage 0) count them; stages KT-2 and KT-1 load
    // the next tile's stages 0 and 1.
    static_assert(C::S == 3, "the tile loop below is written for a three-stage ring");

    while (true) {
      kstage(WE{}, CUR{}, 0, 2);
      for (int kt = 1; kt < KT - 2; ++kt) kstage(WN{}, CUR{}, kt, kt + 2);
      kstage(WN{}, NXT{}, KT - 2, 0);
      kstage(WE{}, NXT{}, KT - 1, 1);
      if (last_item) break;
      L += P;
      last_item = L + P >= n_items;
      cur = nxt;
      scur = snxt;
      if (!last_item) nxt = decode_stream<C>(pl, L + P, n_ntiles, N);
      snxt = stream_src<C>(p, nxt, !last_item);
    }
  }

  // rows outside the active groups: fill them last, after this workgroup's
  // tiles (grid-stride over the whole grid)
  {
    const long long row_bytes = (long long)N * C::es_out;
    const int lo_row = pl.row_start[0], hi_row = pl.row_start[pl.ga];
    const long long z1 = fill_rows(p, lo_row) * row_bytes;
    const long long z2b = (long long)hi_row * row_bytes;
    const long long total = z1 + fill_rows(p, M - hi_row) * row_bytes;
    for (long long o = ((long long)slot * C::T + tid) * 16; o < total; o += (long long)P * C::T * 16)
      fill16(p, o < z1 ? o : z2b + (o - z1));
  }
}

}  // namespace gmmk
