// gmm_stream.hpp -- the weight-streaming kernel of the gfx950 grouped matmul:
// bf16 lhs x e4m3 weight [G,N,K] with per-block rhs_scale and an optional
// bias, for problems with few rows per group (decode), where the run time is
// the time to read every active group's weight once from HBM.
//
// Output tiles are 32 rows (group-aligned) x 64 columns; a tile reads its
// group's 64 x K weight slab once.  K is consumed in stages of 128 (one
// quantisation block of the scale; without a scale every block counts 1),
// each stage holding in LDS the weight slab
// (64 rows of 128 bytes), the tile's lhs rows (32 rows of 256 bytes), the
// block's 64 scales and the tile's 64 bias values.  Six stages form a ring
// filled by direct-to-LDS loads five stages ahead, across the workgroup's
// tiles, so the HBM stream never drains.  Eight waves, two per SIMD: wave w
// takes K half w / 4 of every stage and columns 16 (w % 4) .. +16 of the
// tile for all 32 rows, with 16x16x32 bf16 MFMAs after widening its e4m3
// weight fragment to bf16 (so no weight byte is widened twice), and folds
// each block's product into fp32 totals with that block's scales (the weight
// fragment is the MFMA's first operand, so a lane holds four consecutive
// columns of a row and their four scales).  At the end of a tile the two K
// halves add their totals through LDS and each stores one 16-row half.
//
// Every wave issues the same four loads per stage (weight, lhs, scale, bias;
// loads past a range return zeros and still count) and one store per tile,
// so the vmcnt waits are constants.
#pragma once

#include "gmm_big.hpp"

namespace gmmk {

// FB_: the weight's fp8 format (0 e4m3fn, 1 e5m2).
template <bool OUT_F32_, int FB_ = 0>
struct StreamCfg {
  static constexpr bool OUT_F32 = OUT_F32_;
  static constexpr int FB = FB_;
  static constexpr int BM = 32, BN = 64, BKS = 128;  // tile rows, tile columns, K per stage
  static constexpr int NWAVES = 8, T = 64 * NWAVES;
  static constexpr int W_ROW = BKS, A_ROW = BKS * 2;  // bytes per weight / lhs row in a stage
  static constexpr int W_BYTES = BN * W_ROW, A_BYTES = BM * A_ROW;
  static constexpr int SLOT = 256;                    // per-wave scale / bias slot
  static constexpr int SC_OFF = W_BYTES + A_BYTES, BI_OFF = SC_OFF + NWAVES * SLOT;
  static constexpr int STAGE = BI_OFF + NWAVES * SLOT;
  static constexpr int S = 6;
  static constexpr int RING = S * STAGE;
  static constexpr int XCHG = 4 * 2 * 64 * 16;  // partial totals passed between the two K halves
  static constexpr int LDS = RING + XCHG;
  static constexpr int OPS = 4;  // loads per wave and stage
  static constexpr int E = 1;    // stores per wave and tile
  static constexpr int es_out = OUT_F32 ? 4 : 2;
  static_assert(W_BYTES == NWAVES * 1024 && A_BYTES == NWAVES * 1024, "one 1 KB load per wave and operand");
};

// 128-byte weight rows: chunk c of row n at c ^ swz_w(n); 256-byte lhs rows:
// chunk c of row r at c ^ (r & 15).  Sixteen consecutive rows read at one
// logical chunk then land in distinct bank groups.
__device__ __forceinline__ int swz_w(int n) { return (n & 7) ^ ((n >> 3) & 1); }
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
  const char* w = reinterpret_cast<const char*>(p.rhs) + ((long long)it.h * N + it.n0) * K;
  s.ra = uniform_rsrc(a, live ? it.rows * K * 2 : 0);
  s.rw = uniform_rsrc(w, live ? it.ncols * K : 0);
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

// Per-lane offsets of this wave's loads.  Weight: rows 8 w + lane/8, chunk
// lane%8.  Lhs: rows 4 w + lane/16, chunk lane%16.  Scale: column
// 16 (w%4) + lane for lanes < 16.  Bias: columns 16 (w%4) + 2 lane, +1 (bf16,
// lanes < 8) or 16 (w%4) + lane (f32, lanes < 16).
struct StreamOff {
  int w, a, scol, bcol, bbyte;
};

template <class C>
__device__ __forceinline__ StreamOff stream_offsets(int K, int w, int lane, bool bias_f32) {
  StreamOff o;
  const int n = 8 * w + (lane >> 3);
  o.w = n * K + (((lane & 7) ^ swz_w(n)) << 4);
  const int r = 4 * w + (lane >> 4);
  o.a = r * K * 2 + (((lane & 15) ^ swz_a(r)) << 4);
  o.scol = lane < 16 ? 16 * (w & 3) + lane : 1 << 20;
  if (bias_f32) {
    o.bcol = lane < 16 ? 16 * (w & 3) + lane : 1 << 20;
    o.bbyte = o.bcol * 4;
  } else {
    o.bcol = lane < 8 ? 16 * (w & 3) + 2 * lane : 1 << 20;
    o.bbyte = o.bcol * 2;
  }
  return o;
}

// The four loads of stage k (K elements [128 k, 128 k + 128), scale block
// k) of a tile into LDS stage `st`.
template <class C>
__device__ __forceinline__ void stream_stage(const StreamSrc& s, const StreamOff& o, int k, int N, char* st, int w) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(s.rw, (lds_ptr_t)(st + w * 1024), 16, o.w, k * C::W_ROW, 0, 0);
  __builtin_amdgcn_raw_ptr_buffer_load_lds(s.ra, (lds_ptr_t)(st + C::W_BYTES + w * 1024), 16, o.a, k * C::A_ROW,
                                           0, 0);
  const int sv = o.scol < s.ncols ? o.scol * 4 : (int)0x80000000;
  __builtin_amdgcn_raw_ptr_buffer_load_lds(s.rs, (lds_ptr_t)(st + C::SC_OFF + w * C::SLOT), 4, sv, k * N * 4, 0,
                                           0);
  const int bv = o.bcol < s.ncols ? o.bbyte : (int)0x80000000;
  __builtin_amdgcn_raw_ptr_buffer_load_lds(s.rb, (lds_ptr_t)(st + C::BI_OFF + w * C::SLOT), 4, bv, 0, 0, 0);
}

template <int F>
__device__ __forceinline__ i32x4 fp8x8_to_bf16x8_pk(uint32_t lo, uint32_t hi) {
  return fp8x8_to_bf16x8<F>(i32x2{(int)lo, (int)hi});
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
  const int wk = w >> 2, wc = w & 3;
  const int r16 = lane & 15, q = lane >> 4;
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

    // prologue: stages 0 .. S-2 of the first tile, then one range-dropped
    // store in place of a previous tile's epilogue store, so that the first
    // tile finds the same operations outstanding as every later one and the
    // loop's constant waits hold for it too.  Only stage 0 is waited for:
    // all workgroups ask for their first S-1 stages at once, and the last of
    // those arrive several microseconds after the first.
#pragma unroll
    for (int st = 0; st < C::S - 1; ++st) stream_stage<C>(scur, off, st, N, smem + st * C::STAGE, w);
    __builtin_amdgcn_raw_buffer_store_b32(0, uniform_rsrc(reinterpret_cast<const char*>(p.out), 0), (int)0x80000000,
                                          0, 0);
    wait_vmcnt<(C::S - 2) * C::OPS + C::E>();
    // a bare barrier, as in the loop: __syncthreads() carries a workgroup
    // fence, which the compiler meets by draining every load in flight
    ring_barrier();

    // lane parts of the fragment addresses (stage-relative): weight row
    // (output column) wn, K half wk -> 16-byte chunk 4 wk + q of the row;
    // lhs rows 16 ch + r16, chunks 8 wk + 2 q + jj
    const int wn = 16 * wc + r16;
    const int w_off = wn * C::W_ROW + (((4 * wk + q) ^ swz_w(wn)) << 4);
    int a_off[2][2];
#pragma unroll
    for (int ch = 0; ch < 2; ++ch)
#pragma unroll
      for (int jj = 0; jj < 2; ++jj) {
        const int r = 16 * ch + r16;
        a_off[ch][jj] = C::W_BYTES + r * C::A_ROW + (((8 * wk + 2 * q + jj) ^ swz_a(r)) << 4);
      }
    const int sc_off = C::SC_OFF + w * C::SLOT + 16 * q;
    const int bi_off = C::BI_OFF + w * C::SLOT + (bias_f32 ? 16 * q : 8 * q);
    // exchange slots: this wave's partial of the other half's rows, and the
    // partner's partial of this wave's rows
    char* const x_put = smem + C::RING + ((wc * 2 + (1 - wk)) * 64 + lane) * 16;
    const char* const x_get = smem + C::RING + ((wc * 2 + wk) * 64 + lane) * 16;

    // a stage's fragments: the weight run (16 e4m3 = two K steps), lhs
    // (two row chunks x two K steps), the block's scales of the lane's
    // four columns
    i32x4 fw, fa[2][2];
    f32x4 fsc;
    auto read_frags = [&](const char* st) __attribute__((always_inline)) {
      fw = *reinterpret_cast<const i32x4*>(st + w_off);
#pragma unroll
      for (int ch = 0; ch < 2; ++ch)
#pragma unroll
        for (int jj = 0; jj < 2; ++jj) fa[ch][jj] = *reinterpret_cast<const i32x4*>(st + a_off[ch][jj]);
      fsc = scaled ? *reinterpret_cast<const f32x4*>(st + sc_off) : f32x4{1.f, 1.f, 1.f, 1.f};
    };

    int stage = 0;
    read_frags(smem);  // stage 0 of the first tile
    f32x4 tot[2] = {{0.f, 0.f, 0.f, 0.f}, {0.f, 0.f, 0.f, 0.f}};

    // One stage kt of the current tile.  Stage kt+1's loads are complete
    // (this wave's, then every wave's after the barrier) once at most WAIT
    // newer operations are outstanding: stages kt+2 .. kt+S-2 (OPS each) and,
    // in a tile's first S-2 stages, the previous tile's store.  The barrier
    // also frees the stage kt-1 used, which takes stage kt+S-1 (of this tile,
    // or kd of the next one when NEXT).  Stage kt's fragments (read during
    // the previous stage) are multiplied, then the registers are refilled
    // with stage kt+1's.
    auto kstage = [&](auto wait_tag, auto next_tag, int kt, int kd) __attribute__((always_inline)) {
      constexpr int WAIT = decltype(wait_tag)::value;
      constexpr bool NEXT = decltype(next_tag)::value;
      wait_vmcnt<WAIT>();
      ring_barrier();
      stream_stage<C>(NEXT ? snxt : scur, off, kd, N, smem + ((stage + C::S - 1) % C::S) * C::STAGE, w);
      // K step jj uses bytes 8 jj .. 8 jj + 7 of the lane's weight run
      const i32x4 bw[2] = {fp8x8_to_bf16x8_pk<C::FB>((uint32_t)fw[0], (uint32_t)fw[1]),
                           fp8x8_to_bf16x8_pk<C::FB>((uint32_t)fw[2], (uint32_t)fw[3])};
#pragma unroll
      for (int ch = 0; ch < 2; ++ch) {
        f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int jj = 0; jj < 2; ++jj)
          acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, bw[jj]),
                                                        __builtin_bit_cast(bf16x8, fa[ch][jj]), acc, 0, 0, 0);
#pragma unroll
        for (int i = 0; i < 4; ++i) tot[ch][i] += acc[i] * fsc[i];
      }
      const char* st = smem + stage * C::STAGE;
      const int stage1 = stage + 1 == C::S ? 0 : stage + 1;
      if (kt == KT - 1) {
        // epilogue: the two K halves add their totals (each keeps rows
        // 16 wk .. +16), then bias from this stage's slot, round, one store of
        // the lane's four columns (out of range rows / columns drop)
        *reinterpret_cast<f32x4*>(x_put) = tot[1 - wk];
        __builtin_amdgcn_s_waitcnt(0xF | (0x7 << 4) | (0x0 << 8) | (0x3 << 14));  // lgkmcnt(0)
        ring_barrier();
        const f32x4 other = *reinterpret_cast<const f32x4*>(x_get);
        const f32x4 mine = wk ? tot[1] : tot[0];
        float v[4];
        float bias[4] = {0.f, 0.f, 0.f, 0.f};
        if (p.rhs_bias) {
          if (bias_f32) {
            const f32x4 b4 = *reinterpret_cast<const f32x4*>(st + bi_off);
            bias[0] = b4[0];
            bias[1] = b4[1];
            bias[2] = b4[2];
            bias[3] = b4[3];
          } else {
            const i32x2 b2 = *reinterpret_cast<const i32x2*>(st + bi_off);
            bias[0] = __uint_as_float((uint32_t)b2[0] << 16);
            bias[1] = __uint_as_float((uint32_t)b2[0] & 0xFFFF0000u);
            bias[2] = __uint_as_float((uint32_t)b2[1] << 16);
            bias[3] = __uint_as_float((uint32_t)b2[1] & 0xFFFF0000u);
          }
        }
#pragma unroll
        for (int i = 0; i < 4; ++i) v[i] = mine[i] + other[i] + bias[i];
        char* tile = reinterpret_cast<char*>(p.out) + ((long long)cur.row0 * N + cur.n0) * C::es_out;
        const __amdgpu_buffer_rsrc_t ro = uniform_rsrc(tile, ((cur.rows - 1) * N + cur.ncols) * C::es_out);
        const int col = 16 * wc + 4 * q;
        const int row = 16 * wk + r16;
        const int voff = col < cur.ncols ? (row * N + col) * C::es_out : (int)0x80000000;
        if constexpr (C::OUT_F32) {
          __builtin_amdgcn_raw_buffer_store_b128(
              i32x4{__float_as_int(v[0]), __float_as_int(v[1]), __float_as_int(v[2]), __float_as_int(v[3])}, ro,
              voff, 0, 0);
        } else {
          const uint32_t x0 = pk_bf16_rne(v[0], v[1]);
          const uint32_t x1 = pk_bf16_rne(v[2], v[3]);
          __builtin_amdgcn_raw_buffer_store_b64(i32x2{(int)x0, (int)x1}, ro, voff, 0, 0);
        }
        tot[0] = f32x4{0.f, 0.f, 0.f, 0.f};
        tot[1] = f32x4{0.f, 0.f, 0.f, 0.f};
      }
      read_frags(smem + stage1 * C::STAGE);
      stage = stage1;
    };
    using WE = std::integral_constant<int, (C::S - 3) * C::OPS + C::E>;
    using WN = std::integral_constant<int, (C::S - 3) * C::OPS>;
    using CUR = std::false_type;
    using NXT = std::true_type;
    // stages kt < S-2 wait for the previous tile's store too; stages
    // kt >= KT-S+1 load the next tile's first stages
    const int e_end = C::S - 2, n_beg = KT - C::S + 1;

    while (true) {
      const int a1 = e_end < n_beg ? e_end : n_beg;
      for (int kt = 0; kt < a1; ++kt) kstage(WE{}, CUR{}, kt, kt + C::S - 1);
      for (int kt = a1; kt < e_end; ++kt) kstage(WE{}, NXT{}, kt, kt + C::S - 1 - KT);
      for (int kt = e_end; kt < n_beg; ++kt) kstage(WN{}, CUR{}, kt, kt + C::S - 1);
      for (int kt = (e_end > n_beg ? e_end : n_beg); kt < KT; ++kt) kstage(WN{}, NXT{}, kt, kt + C::S - 1 - KT);
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
