// gmm_tgmm_tiles.hpp -- the output tiles of one group of the transposed
// grouped matmul when a group's tiles all run at once, one per workgroup of
// an XCD ("gang" schedule).  Plain integer code, built for the device and
// for a host-side coverage check.
//
// A group's output is K x N.  Tiles hold at most 65536 accumulators and read
// at most 512 operand columns per contraction row (four 128-column LDS
// areas per stage), so the shapes are 256 x 256 (full), 384 x 128 (tall:
// three lhs areas, one rhs area) and 128 x 384 (wide: one and three).
//
// With K = kf + ek and N = nf + en, where kf and nf are multiples of 256 and
// the edges ek, en are at most 128 (an edge above 128 is rounded up into a
// partial full tile instead):
//  - full tiles cover [0, kf) x [0, nf);
//  - without an L tile: tall tiles cover [0, min(kf, K)) x [nf, N) in
//    k-steps of 384, wide tiles [kf, K) x [0, N) in n-steps of 384 (the
//    corner too);
//  - with an L tile (both edges, kf, nf > 0): a full-shape tile at
//    (K - 256, N - 256) whose part [K - 256, kf) x [N - 256, nf) is the
//    last full tile's and is not stored, tall tiles over [0, K - 256) x
//    [nf, N), wide tiles over [kf, K) x [0, N - 256).
// The variant with fewer tiles is used (K = N = 1408: 25 + 1 + 3 + 3 = 32
// tiles with the L tile, 33 without).
#pragma once

#ifndef GMM_HD
#define GMM_HD __host__ __device__
#endif

namespace gmmk {

// tile shapes (the dynamic schedule also uses kTgHalf: a 256 x 256 tile
// with at most 128 valid rows or columns, computed as 64 x 64 per wave)
enum TgShape { kTgFull = 0, kTgHalf = 1, kTgTall = 2, kTgWide = 3 };

struct TgTile {
  int shape;
  int k0, n0;          // origin in the group's K x N output
  int rows, ncols;     // valid rows / columns from the origin
  int skip_r, skip_c;  // [0, skip_r) x [0, skip_c) of the tile is another tile's (0: none)
};

struct TgGang {
  int kf, nf, ek, en;
  int L;               // 1: the L tile is used
  int nfn;             // full tiles along n
  int nfull, ntall, nwide;
  int klim, nlim;      // extents of the tall strip (k) and the wide strip (n)
  int T;               // tiles per group
};

// X = xf + ex with xf a multiple of 256 and 0 <= ex <= 128 (ex = 0 when the
// last 256-block has more than 128 valid columns: xf then exceeds X)
GMM_HD inline void tg_split_extent(int X, int& xf, int& ex) {
  const int r = X % 256;
  if (X <= 128) {
    xf = 0;
    ex = X;
  } else if (r == 0) {
    xf = X;
    ex = 0;
  } else if (r <= 128 && X > 256) {
    xf = X - r;
    ex = r;
  } else {
    xf = X - r + 256;
    ex = 0;
  }
}

GMM_HD inline int tg_ceil384(int x) { return x > 0 ? (x + 383) / 384 : 0; }

GMM_HD inline TgGang tg_gang_plan(int K, int N) {
  TgGang g;
  tg_split_extent(K, g.kf, g.ek);
  tg_split_extent(N, g.nf, g.en);
  g.nfn = g.nf / 256;
  g.nfull = (g.kf / 256) * g.nfn;
  const int kcov = g.kf < K ? g.kf : K;  // kf exceeds K when the last 256-block is partial
  const int t_plain = g.nfull + (g.en > 0 ? tg_ceil384(kcov) : 0) + (g.ek > 0 ? tg_ceil384(N) : 0);
  const bool l_ok = g.ek > 0 && g.en > 0 && g.kf > 0 && g.nf > 0;
  const int t_l = l_ok ? g.nfull + 1 + tg_ceil384(K - 256) + tg_ceil384(N - 256) : t_plain + 1;
  g.L = t_l < t_plain ? 1 : 0;
  g.klim = g.L ? K - 256 : kcov;
  g.nlim = g.L ? N - 256 : N;
  g.ntall = g.en > 0 ? tg_ceil384(g.klim) : 0;
  g.nwide = g.ek > 0 ? tg_ceil384(g.nlim) : 0;
  g.T = g.nfull + g.L + g.ntall + g.nwide;
  return g;
}

// tile j (0 <= j < g.T) of a group
GMM_HD inline TgTile tg_gang_tile(const TgGang& g, int K, int N, int j) {
  TgTile t;
  t.skip_r = 0;
  t.skip_c = 0;
  if (j < g.nfull) {
    t.shape = kTgFull;
    t.k0 = 256 * (j / g.nfn);
    t.n0 = 256 * (j % g.nfn);
    t.rows = K - t.k0 < 256 ? K - t.k0 : 256;
    t.ncols = N - t.n0 < 256 ? N - t.n0 : 256;
    return t;
  }
  j -= g.nfull;
  if (j < g.L) {
    t.shape = kTgFull;
    t.k0 = K - 256;
    t.n0 = N - 256;
    t.rows = 256;
    t.ncols = 256;
    t.skip_r = g.kf - t.k0;
    t.skip_c = g.nf - t.n0;
    return t;
  }
  j -= g.L;
  if (j < g.ntall) {
    t.shape = kTgTall;
    t.k0 = 384 * j;
    t.n0 = g.nf;
    t.rows = g.klim - t.k0 < 384 ? g.klim - t.k0 : 384;
    t.ncols = N - g.nf;
    return t;
  }
  j -= g.ntall;
  t.shape = kTgWide;
  t.k0 = g.kf;
  t.n0 = 384 * j;
  t.rows = K - g.kf;
  t.ncols = g.nlim - t.n0 < 384 ? g.nlim - t.n0 : 384;
  return t;
}

}  // namespace gmmk
