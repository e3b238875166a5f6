"""The gang schedule's tiles of one tgmm group (gmm_tgmm_tiles.hpp), checked
on the CPU: the header's plain integer code is compiled for the host with
g++ and, for every K and N that are multiples of 8 up to 1536 (and the
model's 1408 x 1408), the tiles' stored parts must cover the group's K x N
output exactly once, within the limits the kernel relies on (at most 65536
accumulators, at most 512 operand columns per contraction row, a shape's
valid part inside its extent, 8-aligned origins), and the 1408 x 1408 grid
must take exactly 32 tiles (one per workgroup of an XCD)."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "moe_grouped_matrix_amd", "csrc", "gmm_tgmm_tiles.hpp")

CHECK = r"""
#include <cstdio>
#include <cstdlib>
#include <vector>
#include "gmm_tgmm_tiles.hpp"
using namespace gmmk;
// the shape's extent: rows x columns
static void extent(int shape, int& r, int& c) {
  if (shape == kTgTall) { r = 384; c = 128; }
  else if (shape == kTgWide) { r = 128; c = 384; }
  else { r = 256; c = 256; }
}
int main(int argc, char** argv) {
  long long shapes = 0;
  int t1408 = -1;
  std::vector<unsigned char> cov;
  auto check = [&](int K, int N) {
    const TgGang g = tg_gang_plan(K, N);
    if (K == 1408 && N == 1408) t1408 = g.T;
    // coverage on an 8 x 8 grid of cells (every origin and extent is a multiple of 8)
    const int kc = K / 8, nc = N / 8;
    cov.assign((size_t)kc * nc, 0);
    for (int j = 0; j < g.T; ++j) {
      const TgTile t = tg_gang_tile(g, K, N, j);
      int er, ec;
      extent(t.shape, er, ec);
      if (t.shape == kTgHalf) { std::printf("half tile in a gang plan K=%d N=%d\n", K, N); return false; }
      if (t.rows <= 0 || t.ncols <= 0 || t.rows > er || t.ncols > ec || t.k0 % 8 || t.n0 % 8 ||
          t.k0 < 0 || t.n0 < 0 || t.k0 + t.rows > K || t.n0 + t.ncols > N || er * ec > 65536 || er + ec > 512 ||
          t.skip_r < 0 || t.skip_c < 0 || t.skip_r % 8 || t.skip_c % 8) {
        std::printf("bad tile K=%d N=%d j=%d shape=%d k0=%d n0=%d rows=%d ncols=%d skip=%d,%d\n", K, N, j,
                    t.shape, t.k0, t.n0, t.rows, t.ncols, t.skip_r, t.skip_c);
        return false;
      }
      for (int r = 0; r < t.rows; r += 8)
        for (int c = 0; c < t.ncols; c += 8) {
          if (r < t.skip_r && c < t.skip_c) continue;
          unsigned char& v = cov[(size_t)((t.k0 + r) / 8) * nc + (t.n0 + c) / 8];
          if (v) { std::printf("cell stored twice K=%d N=%d at %d,%d (tile %d)\n", K, N, t.k0 + r, t.n0 + c, j); return false; }
          v = 1;
        }
    }
    for (size_t i = 0; i < cov.size(); ++i)
      if (!cov[i]) { std::printf("cell not stored K=%d N=%d at %d,%d\n", K, N, (int)(i / nc) * 8, (int)(i % nc) * 8); return false; }
    ++shapes;
    return true;
  };
  for (int K = 8; K <= 1536; K += 8)
    for (int N = 8; N <= 1536; N += 8)
      if (!check(K, N)) return 1;
  if (!check(1408, 1408) || !check(4096, 1408) || !check(1408, 4104)) return 1;
  std::printf("shapes %lld T1408 %d\n", shapes, t1408);
  return 0;
}
"""


def test_gang_tiles_cover_each_output_once(tmp_path):
    gxx = shutil.which("g++")
    if not gxx:
        pytest.skip("g++ not available")
    src = tmp_path / "check.cpp"
    src.write_text(CHECK)
    exe = tmp_path / "check"
    res = subprocess.run([gxx, "-O2", "-std=c++17", "-DGMM_HD=", "-I" + os.path.dirname(HEADER), str(src), "-o",
                          str(exe)], capture_output=True, text=True)
    assert res.returncode == 0, res.stderr[-2000:]
    run = subprocess.run([str(exe)], capture_output=True, text=True, timeout=300)
    assert run.returncode == 0, run.stdout[-2000:]
    words = run.stdout.split()
    assert words[0] == "shapes" and int(words[1]) == 192 * 192 + 3
    assert words[2] == "T1408" and int(words[3]) == 32, run.stdout
