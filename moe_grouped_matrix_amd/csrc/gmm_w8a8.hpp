// gmm_w8a8.hpp -- the block-scaled fp8 x fp8 grouped matmul (W8A8) with a
// direct-to-LDS operand ring, for large problems whose scale blocks are one
// K step (128 elements).
//
// The arithmetic is the general kernel's for the same configuration
// (gmm_device.hpp, Cfg<FP8, NT, ..., 256, 128, 4, 2, scaled>): 256 x 128
// group-aligned tiles, eight waves of 64 x 64, v_mfma_scale_f32_16x16x128
// with unit scales, and after each K step (one quantisation block) the fold
// tot += part * rhs_scale[col] * lhs_scale[row]; bias, rounding and the
// staged epilogue are the same code.  What differs is how operands reach
// LDS.  The general kernel loads a step into registers and writes them to
// LDS after the multiply, so a step's loads have one step of multiplies to
// arrive.  Here three LDS stages form a ring filled by direct-to-LDS buffer
// loads two steps ahead, with the block's scales in the same stage:
//
//   per wave and step: 4 lhs loads (1 KB each: 8 rows of 128 bytes), 2
//   weight loads, and 1 scale load (waves 0-3: 64 row scales each, waves
//   4-5: 64 column scales each, waves 6-7: a range-dropped load into a slot
//   nobody reads, so that every wave counts the same 7 operations).
//
// At the top of step kt each wave waits until only step kt+1's 7 loads are
// outstanding (or none, in a tile's last step), then a bare barrier makes
// every wave's loads of stage kt visible and frees the stage step kt-1 read,
// which takes step kt+2's loads.  Each lane loads the global chunk that the
// LDS swizzle puts at its position (a load writes 64 lanes x 16 bytes in
// lane order), so the stage has the layout the multiply reads.
#pragma once

#include "gmm_big.hpp"

namespace gmmk {

template <class C>
struct W8A8Ring {
  static_assert(C::op == Op::FP8 && !C::NN && C::SCALED && C::T == 512 && C::BM == 256 && C::BN == 128,
                "the W8A8 ring serves the large scaled fp8 configuration");
  static constexpr int A_OPS = C::A_BYTES / 1024 / 8, B_OPS = C::B_BYTES / 1024 / 8;
  static constexpr int OPS = A_OPS + B_OPS + 1;  // + one scale load
  static constexpr int LSC = C::A_BYTES + C::B_BYTES;  // 256 row scales
  static constexpr int RSC = LSC + C::BM * 4;          // 128 column scales
  static constexpr int DUMMY = RSC + C::BN * 4;        // the range-dropped loads' slot
  static constexpr int STAGE = DUMMY + 256;
  static constexpr int S = 3;
  static constexpr int LDS = S * STAGE;
  static_assert(A_OPS == 4 && B_OPS == 2, "DMA split");
  static_assert(C::T / 64 * kStageSlice<C> <= LDS, "epilogue staging fits the ring");
};

// The loads of K step k into stage `st`: A_OPS lhs, B_OPS weight and one
// scale load (row scales step by one block, 4 bytes; column scales by N of
// them).  A device function, not a lambda in the kernel: a lambda there is
// also compiled for the host, where these builtins do not exist, and the
// kernel's host-side launch stub would silently not be emitted.
template <class C>
__device__ __forceinline__ void w8a8_issue(char* st, __amdgpu_buffer_rsrc_t ra, __amdgpu_buffer_rsrc_t rb,
                                           __amdgpu_buffer_rsrc_t rsc, const int (&aoff)[W8A8Ring<C>::A_OPS],
                                           const int (&boff)[W8A8Ring<C>::B_OPS], int soff, int sdst, int k, int w,
                                           int N) {
  using R = W8A8Ring<C>;
#pragma unroll
  for (int jj = 0; jj < R::A_OPS; ++jj)
    __builtin_amdgcn_raw_ptr_buffer_load_lds(ra, (lds_ptr_t)(st + (R::A_OPS * w + jj) * 1024), 16, aoff[jj],
                                             k * C::BK, 0, 0);
#pragma unroll
  for (int jj = 0; jj < R::B_OPS; ++jj)
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rb, (lds_ptr_t)(st + C::A_BYTES + (R::B_OPS * w + jj) * 1024), 16,
                                             boff[jj], k * C::BK, 0, 0);
  __builtin_amdgcn_raw_ptr_buffer_load_lds(rsc, (lds_ptr_t)(st + sdst), 4, soff, w < 4 ? k * 4 : k * N * 4, 0, 0);
}

template <class C>
__global__ __launch_bounds__(C::T) void gmm_w8a8_kernel(Params p) {
  static_assert(C::op == Op::FP8 && C::FA <= 1 && C::FB <= 1, "one-byte fp8 operands (e4m3fn or e5m2)");
  using R = W8A8Ring<C>;
  // one LDS array for the ring and the plan: with a second LDS variable the
  // compiler tags LDS accesses with alias scopes and then drains the
  // direct-to-LDS loads in flight before every LDS read
  __shared__ __attribute__((aligned(1024))) char smem[R::LDS + sizeof(Plan)];
  Plan& pl = *reinterpret_cast<Plan*>(smem + R::LDS);
  if (threadIdx.x == 0) pl.flags = 0;
  __syncthreads();
  build_plan<C::T>(p, pl, C::BM);
  report_flags(p, pl);

  const int tid = threadIdx.x, lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = w / C::WN, wn = w % C::WN;
  const int q = lane >> 4, r16 = lane & 15;
  const int M = p.M, N = p.N, K = p.K;
  const int out_es = p.out_f32 ? 4 : 2;
  const long long row_bytes = (long long)N * out_es;
  const int n_ntiles = (N + C::BN - 1) / C::BN;
  const long long n_gemm = (long long)pl.n_mtiles * n_ntiles;
  const int lo_row = pl.row_start[0], hi_row = pl.row_start[pl.ga];
  const long long z1_bytes = fill_rows(p, lo_row) * row_bytes;
  const long long z2_bytes = fill_rows(p, M - hi_row) * row_bytes;
  const long long z1 = (z1_bytes + kZeroChunk - 1) / kZeroChunk;
  const long long z2 = (z2_bytes + kZeroChunk - 1) / kZeroChunk;
  const long long n_items = n_gemm + z1 + z2;
  const int KT = K / C::BK;  // K steps = scale blocks (the launcher checks blk == BK)
  const int P = gridDim.x;
  const int slot = xcd_slot(blockIdx.x, P);
  const bool has_ls = p.lhs_scale != nullptr, has_rs = p.rhs_scale != nullptr;

  // per-lane load offsets (K step 0): lhs load j fills LDS rows
  // 8 (4 w + j) + lane/8 of the stage, weight load j rows 8 (2 w + j) +
  // lane/8; lane position lane%8 of a row holds logical chunk
  // (lane%8) ^ swz(row)
  int aoff[R::A_OPS], boff[R::B_OPS];
#pragma unroll
  for (int j = 0; j < R::A_OPS; ++j) {
    const int r = 8 * (R::A_OPS * w + j) + (lane >> 3);
    aoff[j] = r * K + (((lane & 7) ^ swz(r)) << 4);
  }
#pragma unroll
  for (int j = 0; j < R::B_OPS; ++j) {
    const int r = 8 * (R::B_OPS * w + j) + (lane >> 3);
    boff[j] = r * K + (((lane & 7) ^ swz(r)) << 4);
  }

  for (long long L = slot; L < n_items; L += P) {
    if (L >= n_gemm) {
      long long z = L - n_gemm;
      if (z < z1) {
        long long b = z * kZeroChunk;
        fill_item<C>(p, b, b + kZeroChunk < z1_bytes ? b + kZeroChunk : z1_bytes);
      } else {
        z -= z1;
        long long base = (long long)hi_row * row_bytes;
        long long b = base + z * kZeroChunk;
        long long e = b + kZeroChunk;
        long long end = base + z2_bytes;
        fill_item<C>(p, b, e < end ? e : end);
      }
      continue;
    }
    const int t = (int)(L / n_ntiles);
    const int j = (int)(L % n_ntiles);
    const int h = __builtin_amdgcn_readfirstlane(find_group(pl, t));
    const int row0 = __builtin_amdgcn_readfirstlane(pl.row_start[h] + (t - pl.tile_start[h]) * C::BM);
    const int rows_left = pl.row_start[h + 1] - row0;
    const int rows = __builtin_amdgcn_readfirstlane(rows_left < C::BM ? rows_left : C::BM);
    const int n0 = j * C::BN;
    const int ncols = N - n0 < C::BN ? N - n0 : C::BN;

    // buffer resources of the tile: lhs rows, the weight's n-tile rows, the
    // tile rows' scales, the group's column scales from n0
    const __amdgpu_buffer_rsrc_t ra =
        uniform_rsrc(reinterpret_cast<const char*>(p.lhs) + (long long)row0 * K, rows * K);
    const __amdgpu_buffer_rsrc_t rb = uniform_rsrc(
        reinterpret_cast<const char*>(p.rhs) + ((long long)h * N + n0) * K, ncols * K);
    // this wave's scale load: row scales of rows 64 w + lane (waves 0-3;
    // the tile rows' scales), column scales of columns 64 (w - 4) + lane
    // (waves 4-5; the group's scales from column n0), or nothing
    const char* sbase = reinterpret_cast<const char*>(p.lhs);
    int sbytes = 0;
    if (w < 4) {
      if (has_ls) {
        sbase = reinterpret_cast<const char*>(p.lhs_scale) + (long long)row0 * p.nb * 4;
        sbytes = rows * p.nb * 4;
      }
    } else if (has_rs) {
      sbase = reinterpret_cast<const char*>(p.rhs_scale) + ((long long)h * p.nb * N + n0) * 4;
      sbytes = (p.nb * N - n0) * 4;
    }
    const __amdgpu_buffer_rsrc_t rsc = uniform_rsrc(sbase, sbytes);
    const int srow = 64 * w + lane, scol = 64 * (w - 4) + lane;
    const int soff = w < 4 ? srow * p.nb * 4 : (w < 6 && scol < ncols ? scol * 4 : (int)0x80000000);
    const int sdst = w < 4 ? R::LSC + 256 * w : (w < 6 ? R::RSC + 256 * (w - 4) : R::DUMMY);

    auto issue = [&](int k) __attribute__((always_inline)) {
      w8a8_issue<C>(smem + (k % R::S) * R::STAGE, ra, rb, rsc, aoff, boff, soff, sdst, k, w, N);
    };

    f32x4 acc[C::FM][C::FN], tot[C::FM][C::FN];
#pragma unroll
    for (int a = 0; a < C::FM; ++a)
#pragma unroll
      for (int b = 0; b < C::FN; ++b) {
        acc[a][b] = f32x4{0.f, 0.f, 0.f, 0.f};
        tot[a][b] = f32x4{0.f, 0.f, 0.f, 0.f};
      }

    issue(0);
    if (KT > 1) issue(1);
    for (int kt = 0; kt < KT; ++kt) {
      // step kt's loads are complete once only step kt+1's are outstanding
      // (older operations -- the previous tile's stores -- finish first)
      if (kt + 1 < KT)
        wait_vmcnt<R::OPS>();
      else
        wait_vmcnt<0>();
      ring_barrier();
      if (kt + 2 < KT) issue(kt + 2);
      const char* st = smem + (kt % R::S) * R::STAGE;
      mma_tile<C>(acc, st, st + C::A_BYTES);
      // fold this block: tot += part * rhs_scale[col] * lhs_scale[row]
      const float* lsc = reinterpret_cast<const float*>(st + R::LSC);
      const float* rsc_l = reinterpret_cast<const float*>(st + R::RSC);
      float rs[C::FN];
      f32x4 ls[C::FM];
#pragma unroll
      for (int fn = 0; fn < C::FN; ++fn) rs[fn] = has_rs ? rsc_l[wn * C::TN + fn * 16 + r16] : 1.f;
#pragma unroll
      for (int fm = 0; fm < C::FM; ++fm)
        ls[fm] = has_ls ? *reinterpret_cast<const f32x4*>(lsc + wm * C::TM + fm * 16 + 4 * q)
                        : f32x4{1.f, 1.f, 1.f, 1.f};
#pragma unroll
      for (int fm = 0; fm < C::FM; ++fm)
#pragma unroll
        for (int fn = 0; fn < C::FN; ++fn) {
#pragma unroll
          for (int i = 0; i < 4; ++i) tot[fm][fn][i] += acc[fm][fn][i] * (rs[fn] * ls[fm][i]);
          acc[fm][fn] = f32x4{0.f, 0.f, 0.f, 0.f};
        }
    }
    // every wave's reads of the last stages are done before the epilogue
    // stages its output there
    ring_barrier();

    // epilogue (as the general kernel's): bias, round, and each 16-row block
    // of the wave's tile through the wave's staging slice, stored as 16-byte
    // chunks of output rows
    {
      const int es = out_es;
      const int pitch = C::TN * es + 16;
      char* const stg = smem + w * kStageSlice<C>;
      const int cpr = C::TN * es / 16;
      float bias[C::FN];
#pragma unroll
      for (int fn = 0; fn < C::FN; ++fn) {
        const int cl = wn * C::TN + fn * 16 + r16;
        bias[fn] = 0.f;
        if (p.rhs_bias && cl < ncols) {
          const long long bi = (long long)h * N + n0 + cl;
          bias[fn] = p.bias_f32 ? reinterpret_cast<const float*>(p.rhs_bias)[bi]
                                : bf16_bits_to_f32(reinterpret_cast<const uint16_t*>(p.rhs_bias)[bi]);
        }
      }
#pragma unroll
      for (int fm = 0; fm < C::FM; ++fm) {
#pragma unroll
        for (int fn = 0; fn < C::FN; ++fn)
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const float v = tot[fm][fn][i] + bias[fn];
            char* d = stg + (4 * q + i) * pitch + (fn * 16 + r16) * es;
            if (p.out_f32)
              *reinterpret_cast<float*>(d) = v;
            else
              *reinterpret_cast<uint16_t*>(d) = f32_to_bf16_rne(v);
          }
        for (int c = lane; c < 16 * cpr; c += 64) {
          const int r = c / cpr, cb = c % cpr;
          const i32x4 d = *reinterpret_cast<const i32x4*>(stg + r * pitch + cb * 16);
          const int rl = wm * C::TM + fm * 16 + r;
          const int cl = wn * C::TN + cb * (16 / es);
          if (rl < rows && cl < ncols)
            *reinterpret_cast<i32x4*>(reinterpret_cast<char*>(p.out) +
                                      ((long long)(row0 + rl) * N + n0 + cl) * es) = d;
        }
      }
    }
    // the next tile's first loads overwrite the staging slices
    __syncthreads();
  }
}

}  // namespace gmmk
