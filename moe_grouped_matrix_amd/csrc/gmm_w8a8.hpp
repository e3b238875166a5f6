// gmm_w8a8.hpp -- the block-scaled fp8 x fp8 grouped matmul (W8A8) for large
// problems whose scale blocks are one K step of 128 elements:
//
//   out[r, n] = bias[h, n] + sum_b ls[r, b] rs[h, b, n] sum_{k in block b} x[r, k] w[h, n, k]
//
// (the quantised matmul of the Megablox gmm with per-token activation and
// per-channel weight scales, one pair per K block).
//
// Per K step and 16 x 16 output block the work is one 16x16x128 f8f6f4 MFMA
// (32 cycles of the matrix core) and the fold tot += acc * (ls * rs) -- a
// multiply and an FMA for each of the block's 256 values, 8 VALU
// instructions of 4 cycles each on a wave64.  The two units cost the same,
// so the kernel is built to run them side by side: one wave per SIMD, and
// within the wave each row block's four MFMAs issue between the fold of the
// previous row block, while the next K step's fragments stream from LDS into
// a second register set.
//
// Layout: output tiles of 256 tokens x 128 columns (group-aligned in M, as
// in the general kernel); four waves of 128 x 64 (FM = 8 token blocks by
// FN = 4 column blocks).  The MFMA's first operand is the weight fragment,
// so a lane's four results are four consecutive columns of one token and
// the epilogue stores them straight from registers (8 or 16 bytes per lane
// and block; an L2 line collects the four 32-byte pieces of a row segment
// before it is written back).
//
// Staging: a K step of both operands (32 KB tokens + 16 KB weights) fills
// one of three LDS stages by direct-to-LDS buffer loads; its scales (256 row
// and 128 column scales) one of four scale slots; the tile's bias row one of
// two bias slots.  The loads of global step g + 3 (across the workgroup's
// tiles) are issued at step g into stage g % 3, which the waves finished
// reading into registers during step g - 1 -- the registers are the ring's
// fourth stage.  Per wave and step that is 14 loads: 8 token-row loads and
// 4 weight-row loads of 1 KB, one load of 64 row scales, and one of 64
// column scales (waves 0-1) or of half the tile's bias row (waves 2-3),
// spread over the step's MFMAs.  Every wave issues the same operations in
// every step (loads of a missing tile or scale are dropped by the range
// check), and every tile's epilogue issues the same number of stores (16
// for bf16 output, 32 for f32), so the waits are constants: at the top of step
// g the loads of step g + 1 are complete once only those of step g + 2 are
// outstanding, and in a tile's first two steps also the previous tile's
// stores.
#pragma once

#include "gmm_big.hpp"

namespace gmmk {

template <int FA_, int FB_, bool OUT_F32_>
struct W8Cfg {
  static constexpr int FA = FA_, FB = FB_;  // f8f6f4 format codes: 0 e4m3fn, 1 e5m2
  static constexpr bool OUT_F32 = OUT_F32_;
  static constexpr int BM = 256, BN = 128, BK = 128;
  static constexpr int NWAVES = 4, T = 64 * NWAVES;
  static constexpr int TM = 128, TN = 64;  // wave tile: tokens x columns
  static constexpr int FM = TM / 16, FN = TN / 16;
  static constexpr int X_BYTES = BM * 128, W_BYTES = BN * 128;
  static constexpr int STAGE = X_BYTES + W_BYTES;
  static constexpr int S = 3;                  // operand stages
  static constexpr int SS = 4;                 // scale slots
  static constexpr int SLOT = (BM + BN) * 4;   // row scales, then column scales
  static constexpr int BIAS_SLOT = BN * 4;     // a tile's bias row (f32 or bf16)
  static constexpr int SCALES = S * STAGE;
  static constexpr int BIASES = SCALES + SS * SLOT;
  static constexpr int LDS = BIASES + 2 * BIAS_SLOT;
  static constexpr int X_OPS = X_BYTES / 1024 / NWAVES, W_OPS = W_BYTES / 1024 / NWAVES;
  static constexpr int OPS = X_OPS + W_OPS + 2;  // + row scales + column scales or bias
  static constexpr int E = OUT_F32 ? FM * FN : FM * FN / 2;  // epilogue stores per wave and tile
  static constexpr int es_out = OUT_F32 ? 4 : 2;
  static_assert(X_OPS == 8 && W_OPS == 4, "load split");
  static_assert(2 * OPS + E < 64, "vmcnt range");
  static_assert(LDS + (int)sizeof(Plan) <= 160 * 1024, "LDS");
};

// 128-byte operand rows in the stages: chunk c of row r at chunk c ^ (r % 8).
// The fragment reads (lane q * 16 + r16 reads row base + r16 at chunk q, and
// at chunk q + 4) then run without bank conflicts; the general kernel's
// swizzle (r ^ r / 8) % 8 costs four conflict cycles per read in this lane
// order (both measured on gfx950 with the LDS bank-conflict counter).
__device__ __forceinline__ int w8_swz(int r) { return r & 7; }
__device__ __forceinline__ int w8_off(int r, int c) { return r * 128 + ((c ^ w8_swz(r)) << 4); }

struct W8Tile {
  int h, row0, rows, n0, ncols;
};

template <class C>
__device__ __forceinline__ W8Tile w8_tile(const Plan& pl, int L, int n_ntiles, int N) {
  W8Tile t;
  const int mt = L / n_ntiles, j = L % n_ntiles;
  const int h = find_group(pl, mt);
  const int row0 = pl.row_start[h] + (mt - pl.tile_start[h]) * C::BM;
  const int left = pl.row_start[h + 1] - row0;
  t.h = __builtin_amdgcn_readfirstlane(h);
  t.row0 = __builtin_amdgcn_readfirstlane(row0);
  t.rows = __builtin_amdgcn_readfirstlane(left < C::BM ? left : C::BM);
  t.n0 = __builtin_amdgcn_readfirstlane(j * C::BN);
  t.ncols = __builtin_amdgcn_readfirstlane(N - t.n0 < C::BN ? N - t.n0 : C::BN);
  return t;
}

// Buffer resources of one tile's loads; a tile that does not exist (past the
// workgroup's last) has empty ranges, so its loads are dropped.
struct W8Src {
  __amdgpu_buffer_rsrc_t x, w, ls, rs_or_bias;
};

// Per-lane parts of this wave's load offsets (the K step and the load's row
// group add a scalar).  Token-row load j fills stage rows 8 (8 w + j) +
// lane / 8, weight-row load j rows 8 (4 w + j) + lane / 8; lane position
// lane % 8 of a row holds logical chunk (lane % 8) ^ w8_swz(row), which does
// not depend on j, so load j is load 0 moved by 8 j rows (a scalar).  The
// row-scale load puts token t(p) at position p = 64 w + lane of the slot,
// t(p) = 128 (p / 128) + 16 (p % 8) + (p % 128) / 8, so that a lane's eight
// row scales (its token in each of the wave's eight row blocks) are 32
// contiguous bytes.  Four VGPRs: with one per load the offsets do not stay
// in VGPRs, and each is read back from an accumulation register before use.
struct W8Off {
  int x, w;       // token-row and weight-row loads (j = 0)
  int ls, small;  // row scale; column scale (waves 0-1) or bias (waves 2-3)
};

template <class C>
__device__ __forceinline__ W8Off w8_offsets(int K, int nb, int w, int lane) {
  W8Off o;
  const int rx = 8 * C::X_OPS * w + (lane >> 3), rw = 8 * C::W_OPS * w + (lane >> 3);
  o.x = rx * K + (((lane & 7) ^ w8_swz(rx)) << 4);
  o.w = rw * K + (((lane & 7) ^ w8_swz(rw)) << 4);
  const int p = 64 * w + lane;
  const int t = 128 * (p >> 7) + 16 * (p & 7) + ((p & 127) >> 3);
  o.ls = t * nb * 4;
  o.small = w < 2 ? (64 * w + lane) * 4 : (w - 2) * 256 + lane * 4;
  return o;
}

template <class C>
__device__ __forceinline__ W8Src w8_src(const Params& p, const W8Tile& t, bool live, int w) {
  W8Src s;
  const int K = p.K, N = p.N, nb = p.nb;
  s.x = uniform_rsrc(reinterpret_cast<const char*>(p.lhs) + (long long)t.row0 * K, live ? t.rows * K : 0);
  s.w = uniform_rsrc(reinterpret_cast<const char*>(p.rhs) + ((long long)t.h * N + t.n0) * K, live ? t.ncols * K : 0);
  const char* lsb = p.lhs_scale ? reinterpret_cast<const char*>(p.lhs_scale) + (long long)t.row0 * nb * 4
                                : reinterpret_cast<const char*>(p.lhs);
  s.ls = uniform_rsrc(lsb, live && p.lhs_scale ? t.rows * nb * 4 : 0);
  if (w < 2) {
    const char* b = p.rhs_scale ? reinterpret_cast<const char*>(p.rhs_scale) + ((long long)t.h * nb * N + t.n0) * 4
                                : reinterpret_cast<const char*>(p.lhs);
    s.rs_or_bias = uniform_rsrc(b, live && p.rhs_scale ? (nb * N - t.n0) * 4 : 0);
  } else {
    const int es = p.bias_f32 ? 4 : 2;
    const char* b = p.rhs_bias ? reinterpret_cast<const char*>(p.rhs_bias) + ((long long)t.h * N + t.n0) * es
                               : reinterpret_cast<const char*>(p.lhs);
    s.rs_or_bias = uniform_rsrc(b, live && p.rhs_bias ? (N - t.n0) * es : 0);
  }
  return s;
}

// Load J (0..13) of K step kd of a tile into stage `st`, scale slot `sc`
// and bias slot `bs`: J < 8 token rows, J < 12 weight rows, 12 row scales,
// 13 column scales (waves 0-1) or bias (waves 2-3).  A device function, not
// a lambda in the kernel: a lambda there is also compiled for the host,
// where these builtins do not exist.
template <class C>
__device__ __forceinline__ void w8_load(const W8Src& s, const W8Off& o, int kd, int K, int N, char* st, char* sc,
                                        char* bs, int w, int J) {
  if (J < C::X_OPS) {
    __builtin_amdgcn_raw_ptr_buffer_load_lds(s.x, (lds_ptr_t)(st + (C::X_OPS * w + J) * 1024), 16, o.x,
                                             kd * C::BK + 8 * J * K, 0, 0);
  } else if (J < C::X_OPS + C::W_OPS) {
    const int j = J - C::X_OPS;
    __builtin_amdgcn_raw_ptr_buffer_load_lds(s.w, (lds_ptr_t)(st + C::X_BYTES + (C::W_OPS * w + j) * 1024), 16,
                                             o.w, kd * C::BK + 8 * j * K, 0, 0);
  } else if (J == C::X_OPS + C::W_OPS) {
    __builtin_amdgcn_raw_ptr_buffer_load_lds(s.ls, (lds_ptr_t)(sc + 256 * w), 4, o.ls, kd * 4, 0, 0);
  } else {
    // column scales (waves 0-1) or bias (waves 2-3), chosen without a branch
    // (a branch here would split the MFMA loop into blocks, and the
    // compiler then sinks the folds out of the loop)
    const bool cs = w < 2;
    char* dst = cs ? sc + C::BM * 4 + 256 * w : bs + 256 * (w - 2);
    __builtin_amdgcn_raw_ptr_buffer_load_lds(s.rs_or_bias, (lds_ptr_t)dst, 4, o.small, cs ? kd * N * 4 : 0, 0, 0);
  }
}

template <class C>
struct W8Frags {
  i32x8 x[C::FM];
  i32x8 w[C::FN];
};

template <class C>
__global__ __launch_bounds__(C::T) void gmm_w8a8_kernel(Params p) {
  // one LDS array for the ring, the scale and bias slots and the plan: with
  // a second LDS variable the compiler tags LDS accesses with alias scopes
  // and then drains the direct-to-LDS loads in flight before every LDS read
  __shared__ __attribute__((aligned(1024))) char smem[C::LDS + sizeof(Plan)];
  Plan& pl = *reinterpret_cast<Plan*>(smem + C::LDS);
  if (threadIdx.x == 0) pl.flags = 0;
  __syncthreads();
  build_plan<C::T>(p, pl, C::BM);
  report_flags(p, pl);

  const int tid = threadIdx.x, lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = w >> 1, wn = w & 1;
  const int q = lane >> 4, r16 = lane & 15;
  const int M = p.M, N = p.N, K = p.K;
  const int P = gridDim.x;
  const int slot = xcd_slot(blockIdx.x, P);

  // rows outside the active groups first (grid-stride)
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
  if (slot >= n_items) return;
  const int KT = K / C::BK;  // K steps per tile (the launcher guarantees KT >= 3)
  const int my_tiles = (n_items - slot + P - 1) / P;
  const int steps = my_tiles * KT;
  const bool has_bias = p.rhs_bias != nullptr;
  const W8Off off = w8_offsets<C>(K, p.nb, w, lane);

  // load cursor: the tile and step of global step g + 3
  int ld_tile = 0, ld_kd = 0;
  W8Tile ldt = w8_tile<C>(pl, slot, n_ntiles, N);
  W8Src lsrc = w8_src<C>(p, ldt, true, w);
  // compute cursor: the tile of the current step and the step within it
  int ct = 0, kt = 0;
  W8Tile cur = ldt;
  // load J of global step g, then (after the last) the cursor's next step
  auto load = [&](int g, int J) __attribute__((always_inline)) {
    w8_load<C>(lsrc, off, ld_kd, K, N, smem + (g % C::S) * C::STAGE, smem + C::SCALES + (g % C::SS) * C::SLOT,
               smem + C::BIASES + (ld_tile & 1) * C::BIAS_SLOT, w, J);
  };
  auto advance = [&]() __attribute__((always_inline)) {
    if (++ld_kd == KT) {
      ld_kd = 0;
      ++ld_tile;
      const bool live = ld_tile < my_tiles;
      if (live) ldt = w8_tile<C>(pl, slot + ld_tile * P, n_ntiles, N);
      lsrc = w8_src<C>(p, ldt, live, w);
    }
  };

  // prologue: steps 0, 1, 2 (every older memory operation -- the fill -- is
  // complete after the wait, so the loop's counts start from an empty queue)
  for (int g = 0; g < 3; ++g) {
    if (g > 0) advance();
#pragma unroll
    for (int J = 0; J < C::OPS; ++J) load(g, J);
  }
  wait_vmcnt<0>();
  __syncthreads();

  // Fragment addresses.  A lane's row in token block fm is
  // 128 wm + 16 fm + r16, whose swizzle does not depend on fm: one lane
  // pattern per 16-byte half of the fragment, the block adding 2048 fm as an
  // immediate (the weight side likewise, per column block).
  int xo[4][2], wo[4][2];
#pragma unroll
  for (int f = 0; f < 4; ++f)
#pragma unroll
    for (int hh = 0; hh < 2; ++hh) {
      xo[f][hh] = w8_off(wm * C::TM + f * 16 + r16, q + 4 * hh) - f * 2048;
      wo[f][hh] = w8_off(wn * C::TN + f * 16 + r16, q + 4 * hh);
    }
  const int ls_lane = (wm * C::TM + r16 * 8) * 4, rs_lane = C::BM * 4 + (wn * C::TN + 4 * q) * 4;
  auto frag = [&](const char* base, int o, int imm) __attribute__((always_inline)) {
    return *reinterpret_cast<const i32x4*>(base + o + imm);
  };
  auto read_x = [&](const char* st, int fm) __attribute__((always_inline)) {
    const i32x4 lo = frag(st, xo[fm & 3][0], fm * 2048), hi = frag(st, xo[fm & 3][1], fm * 2048);
    return i32x8{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
  };
  auto read_w = [&](const char* st, int fn) __attribute__((always_inline)) {
    const i32x4 lo = frag(st, wo[fn][0], C::X_BYTES), hi = frag(st, wo[fn][1], C::X_BYTES);
    return i32x8{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
  };

  W8Frags<C> f;
#pragma unroll
  for (int fm = 0; fm < C::FM; ++fm) f.x[fm] = read_x(smem, fm);
#pragma unroll
  for (int fn = 0; fn < C::FN; ++fn) f.w[fn] = read_w(smem, fn);

  f32x4 tot[C::FM][C::FN];
#pragma unroll
  for (int a = 0; a < C::FM; ++a)
#pragma unroll
    for (int b = 0; b < C::FN; ++b) tot[a][b] = f32x4{0.f, 0.f, 0.f, 0.f};

  // Epilogue of a tile: bias, rounding, stores straight from registers.  A
  // lane holds columns 4q + [0, 4) of each 16-column block for its token.
  // bf16 output: the permlane16 swap of blocks 2p and 2p + 1 hands lanes
  // q = 0, 2 eight consecutive columns of block 2p and lanes q = 1, 3 eight
  // of block 2p + 1, so each store writes 16 bytes per lane (16 per tile);
  // f32 output: the lane's four columns are 16 bytes already (32 per tile).
  // Stores outside the tile's valid rows and columns are dropped.
  auto epilogue = [&]() __attribute__((always_inline)) {
    char* tile = reinterpret_cast<char*>(p.out) + ((long long)cur.row0 * N + cur.n0) * C::es_out;
    const int nrec = ((cur.rows - 1) * N + cur.ncols) * C::es_out;
    const __amdgpu_buffer_rsrc_t ro = uniform_rsrc(tile, nrec);
    const char* bslot = smem + C::BIASES + (ct & 1) * C::BIAS_SLOT;
    float bias[C::FN][4];
#pragma unroll
    for (int fn = 0; fn < C::FN; ++fn) {
      const int cl = wn * C::TN + fn * 16 + 4 * q;  // this lane's first column of block fn
#pragma unroll
      for (int i = 0; i < 4; ++i) bias[fn][i] = 0.f;
      if (has_bias) {
        if (p.bias_f32) {
          const f32x4 v = *reinterpret_cast<const f32x4*>(bslot + cl * 4);
#pragma unroll
          for (int i = 0; i < 4; ++i) bias[fn][i] = v[i];
        } else {
          const i32x2 v = *reinterpret_cast<const i32x2*>(bslot + cl * 2);
          bias[fn][0] = __uint_as_float((uint32_t)v[0] << 16);
          bias[fn][1] = __uint_as_float((uint32_t)v[0] & 0xFFFF0000u);
          bias[fn][2] = __uint_as_float((uint32_t)v[1] << 16);
          bias[fn][3] = __uint_as_float((uint32_t)v[1] & 0xFFFF0000u);
        }
      }
    }
#pragma unroll
    for (int fm = 0; fm < C::FM; ++fm) {
      const int rl = wm * C::TM + fm * 16 + r16;
      if constexpr (C::OUT_F32) {
#pragma unroll
        for (int fn = 0; fn < C::FN; ++fn) {
          const int cl = wn * C::TN + fn * 16 + 4 * q;
          const int voff = rl < cur.rows && cl < cur.ncols ? (rl * N + cl) * 4 : (int)0x80000000;
          const f32x4 v = tot[fm][fn];
          __builtin_amdgcn_raw_buffer_store_b128(
              i32x4{__float_as_int(v[0] + bias[fn][0]), __float_as_int(v[1] + bias[fn][1]),
                    __float_as_int(v[2] + bias[fn][2]), __float_as_int(v[3] + bias[fn][3])},
              ro, voff, 0, 0);
        }
      } else {
#pragma unroll
        for (int pr = 0; pr < C::FN / 2; ++pr) {
          uint32_t a[2], b[2];
#pragma unroll
          for (int x = 0; x < 2; ++x) {
            const f32x4 va = tot[fm][2 * pr], vb = tot[fm][2 * pr + 1];
            a[x] = pk_bf16_rne(va[2 * x] + bias[2 * pr][2 * x], va[2 * x + 1] + bias[2 * pr][2 * x + 1]);
            b[x] = pk_bf16_rne(vb[2 * x] + bias[2 * pr + 1][2 * x], vb[2 * x + 1] + bias[2 * pr + 1][2 * x + 1]);
          }
          const auto s0 = __builtin_amdgcn_permlane16_swap(a[0], b[0], false, false);
          const auto s1 = __builtin_amdgcn_permlane16_swap(a[1], b[1], false, false);
          const int cl = wn * C::TN + (2 * pr + (q & 1)) * 16 + (q >> 1) * 8;
          const int voff = rl < cur.rows && cl < cur.ncols ? (rl * N + cl) * 2 : (int)0x80000000;
          __builtin_amdgcn_raw_buffer_store_b128(i32x4{(int)s0[0], (int)s1[0], (int)s0[1], (int)s1[1]}, ro, voff, 0,
                                                 0);
        }
      }
#pragma unroll
      for (int fn = 0; fn < C::FN; ++fn) tot[fm][fn] = f32x4{0.f, 0.f, 0.f, 0.f};
    }
  };

  // One K step g: its fragments are in `f`; each is refilled with step
  // g + 1's from stage (g + 1) % 3 right after its last MFMA.  In a tile's
  // first two steps the previous tile's stores are newer than the loads
  // waited for.
  auto kstep = [&](int g) __attribute__((always_inline)) {
    // the load cursor to step g + 3 first: its branch (a new tile every KT
    // steps) placed after the MFMA loop lets the compiler sink the folds
    // out of the loop, past it
    advance();
    // this step's scales: complete and visible since the last step's barrier
    // (its loads were waited for then), and their slot is not reloaded
    // before the next step -- read them while the waits below run
    const char* sc = smem + C::SCALES + (g % C::SS) * C::SLOT;
    const f32x4 ls0 = *reinterpret_cast<const f32x4*>(sc + ls_lane);
    const f32x4 ls1 = *reinterpret_cast<const f32x4*>(sc + ls_lane + 16);
    f32x4 rs[C::FN];
#pragma unroll
    for (int fn = 0; fn < C::FN; ++fn) rs[fn] = *reinterpret_cast<const f32x4*>(sc + rs_lane + fn * 64);
    if (kt < 2)
      wait_vmcnt<C::OPS + C::E>();
    else
      wait_vmcnt<C::OPS>();
    // this wave's reads of stage g % 3 (last step's fragment refills) and of
    // the scale slot of step g - 1 are complete before the barrier frees them
    __builtin_amdgcn_s_waitcnt(0xF | (0x7 << 4) | (0x0 << 8) | (0x3 << 14));
    ring_barrier();
    const char* stn = smem + ((g + 1) % C::S) * C::STAGE;
    // Row block fm: its four MFMAs, each followed by a quarter of the fold of
    // row block fm - 1 (whose MFMAs finished a row block ago) and one of the
    // next step's fragment reads.  The fold's quarters are eight independent
    // VALU instructions each -- the products l * rs of column blocks 0-1,
    // of 2-3, then the FMAs of 0-1, of 2-3 -- so that no instruction waits
    // on the one before it.
    f32x4 acc[2][C::FN];
    float sc8[2][8];
#pragma unroll
    for (int fm = 0; fm <= C::FM; ++fm) {
#pragma unroll
      for (int fn = 0; fn < C::FN; ++fn) {
        if (fm < C::FM)
          acc[fm & 1][fn] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(
              f.w[fn], f.x[fm], f32x4{0.f, 0.f, 0.f, 0.f}, C::FB, C::FA, 0, 0, 0, 0);
        if (fm > 0) {
          const int pm = fm - 1;
          const float l = pm < 4 ? ls0[pm] : ls1[pm - 4];
          if (fn < 2) {
#pragma unroll
            for (int i = 0; i < 8; ++i) sc8[fn][i] = l * rs[2 * fn + i / 4][i % 4];
          } else {
#pragma unroll
            for (int i = 0; i < 8; ++i) {
              const int cb = 2 * (fn - 2) + i / 4;
              tot[pm][cb][i % 4] += acc[pm & 1][cb][i % 4] * sc8[fn - 2][i];
            }
          }
        }
        // step g + 3's loads, one after every other MFMA: issued in one
        // burst they queue at the texture unit and hold up the wave
        if (fm < C::FM && (fm * C::FN + fn) % 2 == 0 && (fm * C::FN + fn) / 2 < C::OPS)
          load(g + 3, (fm * C::FN + fn) / 2);
        // refill each fragment with the next step's right after its last use
        if (fm < C::FM && fn == C::FN - 1) f.x[fm] = read_x(stn, fm);
        if (fm == C::FM - 1) f.w[fn] = read_w(stn, fn);
        // in this order: the MFMA, then the VALU work that runs beside it,
        // then the memory operations (left to itself the scheduler puts
        // two groups' MFMAs back to back, and the second waits for the first)
        if (fm < C::FM) __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
        __builtin_amdgcn_sched_group_barrier(0x002, 16, 0);
        __builtin_amdgcn_sched_group_barrier(0x100, 4, 0);
        __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);
        __builtin_amdgcn_sched_barrier(0);
      }
    }
    if (++kt == KT) {
      epilogue();
      kt = 0;
      if (++ct < my_tiles) cur = w8_tile<C>(pl, slot + ct * P, n_ntiles, N);
    }
  };

  for (int g = 0; g < steps; ++g) kstep(g);
  // the loads issued for steps past the last are dropped, but they still
  // write their LDS destination: let them land before the workgroup ends
  wait_vmcnt<0>();
}

}  // namespace gmmk
