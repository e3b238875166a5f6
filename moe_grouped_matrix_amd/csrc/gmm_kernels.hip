// gmm_kernels.hip -- instantiations of the gfx950 grouped-matmul kernel
// family and their launchers.
#include <atomic>

#include "gmm_big.hpp"
#include "gmm_device.hpp"
#include "gmm_tgmm.hpp"
#include "gmm_launch.hpp"

namespace gmmk {

// The scratch of gmm_tgmm_run_noalloc (kStaticScratchBytes, zero at load).
// Host code never passes `scratch` itself to a kernel: on the host the name
// stands for a host-side shadow, not the device array.  The device address
// comes from static_scratch_address, called once per device with that
// device current.
static __device__ __align__(256) int32_t scratch[kStaticScratchBytes / 4];

hipError_t static_scratch_address(void** ptr) {
  return hipGetSymbolAddress(ptr, HIP_SYMBOL(scratch));
}

__global__ void clear_ints_kernel(int32_t* p, int n) {
  if ((int)threadIdx.x < n) p[threadIdx.x] = 0;
}

hipError_t launch_clear_ints(int32_t* p, int n, hipStream_t stream) {
  if (n < 0 || n > 64) return hipErrorInvalidValue;
  hipLaunchKernelGGL(clear_ints_kernel, dim3(1), dim3(64), 0, stream, p, n);
  return hipGetLastError();
}

namespace {

// Tile shapes.  Big: 256 x 128 output tile, four waves of 128 x 64 (for
// large groups); with scales, eight waves of 64 x 64, since the per-block
// partial and the running total both stay in registers.  Small: 32 x 64,
// four waves of 32 x 16 (decode-sized groups).  F32 uses 64 x 64 tiles of
// four 32 x 32 waves.
template <Op OP, bool NN, bool BF8, bool SC, SizeClass SZ, int FMT, bool MX = false>
struct Pick {
  using type = Cfg<OP, NN, BF8, 256, 128, SC ? 4 : 2, 2, SC, FMT, MX>;
};
template <Op OP, bool NN, bool BF8, bool SC, int FMT, bool MX>
struct Pick<OP, NN, BF8, SC, SizeClass::Small, FMT, MX> {
  using type = Cfg<OP, NN, BF8, 32, 64, 1, 4, SC, FMT, MX>;
};

// Every kernel below walks its work items with a grid stride, so any grid
// size is correct; a positive cap (a test hook) makes each workgroup run
// many tiles, with the operand streams carried from one tile to the next.
inline long long apply_cap(long long grid, int cap) { return cap > 0 && grid > cap ? cap : grid; }

template <class C>
hipError_t launch_cfg(const Params& p, int cu_count, int cap, hipStream_t stream) {
  static std::atomic<int> occ_cache{0};
  int occ = occ_cache.load();
  if (occ <= 0) {
    hipError_t e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&occ, gmm_kernel<C>, C::T, 0);
    if (e != hipSuccess) return e;
    if (occ < 1) occ = 1;
    occ_cache.store(occ);
  }
  // Upper bound on work items: group-aligned m-tiles are at most
  // ceil(M/BM) + Ga, times the n-tiles, plus the zero-fill chunks.
  const long long n_tiles = (p.N + C::BN - 1) / C::BN;
  const long long m_tiles = (p.M + C::BM - 1) / C::BM + p.Ga;
  const long long row_bytes = (long long)p.N * (p.out_f32 ? 4 : 2);
  const long long zero_items = ((long long)p.M * row_bytes + kZeroChunk - 1) / kZeroChunk + 2;
  const long long bound = m_tiles * n_tiles + zero_items;
  long long grid = (long long)cu_count * occ;
  if (grid > bound) grid = bound;
  if (grid >= 8) grid -= grid % 8;
  if (grid < 1) grid = 1;
  grid = apply_cap(grid, cap);
  hipLaunchKernelGGL(gmm_kernel<C>, dim3((unsigned)grid), dim3(C::T), 0, stream, p);
  return hipGetLastError();
}

template <class C>
hipError_t launch_big(const Params& p, int cu_count, int cap, hipStream_t stream) {
  const long long n_tiles = (p.N + C::BN - 1) / C::BN;
  const long long m_tiles = (p.M + C::BM - 1) / C::BM + p.Ga;
  long long grid = cu_count;  // one workgroup per CU (LDS-bound)
  if (grid > m_tiles * n_tiles && m_tiles * n_tiles >= 8) grid = m_tiles * n_tiles;
  if (grid >= 8) grid -= grid % 8;
  if (grid < 1) grid = 1;
  grid = apply_cap(grid, cap);
  hipLaunchKernelGGL(gmm_big_kernel<C>, dim3((unsigned)grid), dim3(C::T), 0, stream, p);
  return hipGetLastError();
}

// One workgroup per CU (LDS-bound), at most one per tile.
template <class C>
hipError_t launch_tgmm_cfg(const Params& p, int cu_count, int cap, hipStream_t stream) {
  const long long items = (long long)p.Ga * ((p.K + C::BM - 1) / C::BM) * ((p.N + C::BN - 1) / C::BN);
  long long grid = cu_count;
  if (grid > items && items >= 8) grid = items;
  if (grid >= 8) grid -= grid % 8;
  if (grid < 1) grid = 1;
  grid = apply_cap(grid, cap);
  hipLaunchKernelGGL(gmm_tgmm_kernel<C>, dim3((unsigned)grid), dim3(C::T), 0, stream, p);
  return hipGetLastError();
}

// FMT: the fp8 formats (bit 0 lhs, bit 1 rhs; 0 e4m3fn, 1 e5m2).
template <Op OP, bool NN, bool BF8, bool SC, int FMT>
hipError_t by_size(const Params& p, const KernelChoice& kc, int cu, hipStream_t st) {
  const SizeClass sz = kc.size;
  const int cap = kc.grid_cap;
  if constexpr (OP == Op::F32) return launch_cfg<Cfg<Op::F32, NN, false, 64, 64, 2, 2, SC>>(p, cu, cap, st);
  if constexpr (OP == Op::BF16 && !BF8 && !SC) {
    // the big kernel runs a tile in five phases of K steps of 32: K >= 160
    if (sz == SizeClass::Big && p.K >= 5 * 32) {
      const bool bias = p.rhs_bias != nullptr;
      if (p.out_f32)
        return bias ? launch_big<BigCfg<NN, true, true>>(p, cu, cap, st) : launch_big<BigCfg<NN, true, false>>(p, cu, cap, st);
      return bias ? launch_big<BigCfg<NN, false, true>>(p, cu, cap, st) : launch_big<BigCfg<NN, false, false>>(p, cu, cap, st);
    }
  }
  if constexpr (OP == Op::BF16 && BF8 && !NN && (FMT >> 3) < 6) {  // one-byte and four-bit weights
    if (sz == SizeClass::Small && stream_fits(p)) return launch_stream(p, FMT >> 3, cu, cap, st);
  }
  // W8A8 (one-byte fp8 operands) with scale blocks of one K step
  if constexpr (OP == Op::FP8 && !NN && SC && (FMT & 7) <= 1 && (FMT >> 3) <= 1) {
    if (sz == SizeClass::Big && w8a8_fits(p)) return launch_w8a8(p, FMT & 7, FMT >> 3, cu, cap, st);
  }
  if (sz == SizeClass::Big)
    return launch_cfg<typename Pick<OP, NN, BF8, SC, SizeClass::Big, FMT>::type>(p, cu, cap, st);
  return launch_cfg<typename Pick<OP, NN, BF8, SC, SizeClass::Small, FMT>::type>(p, cu, cap, st);
}

// E8M0 block scales on the scaled f8f6f4 instruction (general kernel).
template <int FMT>
hipError_t by_size_mx(const Params& p, const KernelChoice& kc, int cu, hipStream_t st) {
  if (kc.size == SizeClass::Big)
    return launch_cfg<typename Pick<Op::FP8, false, false, false, SizeClass::Big, FMT, true>::type>(
        p, cu, kc.grid_cap, st);
  return launch_cfg<typename Pick<Op::FP8, false, false, false, SizeClass::Small, FMT, true>::type>(
      p, cu, kc.grid_cap, st);
}

template <Op OP, bool NN, bool BF8, int FMT = 0>
hipError_t by_scaled(const Params& p, const KernelChoice& c, int cu, hipStream_t st) {
  if (c.scaled) return by_size<OP, NN, BF8, true, FMT>(p, c, cu, st);
  return by_size<OP, NN, BF8, false, FMT>(p, c, cu, st);
}

}  // namespace

int tile_m(const KernelChoice& c) {
  if (c.op == Op::F32) return 64;
  return c.size == SizeClass::Big ? 256 : 32;
}

hipError_t launch_gmm(const Params& p, const KernelChoice& c, int cu, hipStream_t st) {
  switch (c.op) {
    case Op::F32:
      if (c.b_fp8 || c.fmt) return hipErrorInvalidValue;
      return c.nn ? by_scaled<Op::F32, true, false>(p, c, cu, st)
                  : by_scaled<Op::F32, false, false>(p, c, cu, st);
    case Op::BF16:
      if (c.b_fp8) {  // widened weights: the rhs format in bits 3..5
        if (c.nn || (c.fmt & 7)) return hipErrorInvalidValue;
        switch (c.fmt >> 3) {
          case 0: return by_scaled<Op::BF16, false, true, 0 << 3>(p, c, cu, st);
          case 1: return by_scaled<Op::BF16, false, true, 1 << 3>(p, c, cu, st);
          case 2: return by_scaled<Op::BF16, false, true, 2 << 3>(p, c, cu, st);
          case 3: return by_scaled<Op::BF16, false, true, 3 << 3>(p, c, cu, st);
          case 4: return by_scaled<Op::BF16, false, true, 4 << 3>(p, c, cu, st);
          case 5: return by_scaled<Op::BF16, false, true, 5 << 3>(p, c, cu, st);
        }
        return hipErrorInvalidValue;
      }
      if (c.fmt) return hipErrorInvalidValue;
      return c.nn ? by_scaled<Op::BF16, true, false>(p, c, cu, st)
                  : by_scaled<Op::BF16, false, false>(p, c, cu, st);
    case Op::FP8:  // lhs and rhs format codes 0 e4m3fn, 1 e5m2, 4 fp4 e2m1
      if (c.nn || c.b_fp8) return hipErrorInvalidValue;
      if (c.mx) {
        if (c.scaled) return hipErrorInvalidValue;
        switch (c.fmt) {
          case 0 | 0 << 3: return by_size_mx<0 | 0 << 3>(p, c, cu, st);
          case 1 | 0 << 3: return by_size_mx<1 | 0 << 3>(p, c, cu, st);
          case 4 | 0 << 3: return by_size_mx<4 | 0 << 3>(p, c, cu, st);
          case 0 | 1 << 3: return by_size_mx<0 | 1 << 3>(p, c, cu, st);
          case 1 | 1 << 3: return by_size_mx<1 | 1 << 3>(p, c, cu, st);
          case 4 | 1 << 3: return by_size_mx<4 | 1 << 3>(p, c, cu, st);
          case 0 | 4 << 3: return by_size_mx<0 | 4 << 3>(p, c, cu, st);
          case 1 | 4 << 3: return by_size_mx<1 | 4 << 3>(p, c, cu, st);
          case 4 | 4 << 3: return by_size_mx<4 | 4 << 3>(p, c, cu, st);
        }
        return hipErrorInvalidValue;
      }
      switch (c.fmt) {
        case 0 | 0 << 3: return by_scaled<Op::FP8, false, false, 0 | 0 << 3>(p, c, cu, st);
        case 1 | 0 << 3: return by_scaled<Op::FP8, false, false, 1 | 0 << 3>(p, c, cu, st);
        case 4 | 0 << 3: return by_scaled<Op::FP8, false, false, 4 | 0 << 3>(p, c, cu, st);
        case 0 | 1 << 3: return by_scaled<Op::FP8, false, false, 0 | 1 << 3>(p, c, cu, st);
        case 1 | 1 << 3: return by_scaled<Op::FP8, false, false, 1 | 1 << 3>(p, c, cu, st);
        case 4 | 1 << 3: return by_scaled<Op::FP8, false, false, 4 | 1 << 3>(p, c, cu, st);
        case 0 | 4 << 3: return by_scaled<Op::FP8, false, false, 0 | 4 << 3>(p, c, cu, st);
        case 1 | 4 << 3: return by_scaled<Op::FP8, false, false, 1 | 4 << 3>(p, c, cu, st);
        case 4 | 4 << 3: return by_scaled<Op::FP8, false, false, 4 | 4 << 3>(p, c, cu, st);
      }
      return hipErrorInvalidValue;
    case Op::I8:  // lhs and rhs format codes 0 int8, 3 int4, 4 uint4
      if (c.nn || c.b_fp8) return hipErrorInvalidValue;
      switch (c.fmt) {
        case 0 | 0 << 3: return by_scaled<Op::I8, false, false, 0 | 0 << 3>(p, c, cu, st);
        case 3 | 0 << 3: return by_scaled<Op::I8, false, false, 3 | 0 << 3>(p, c, cu, st);
        case 4 | 0 << 3: return by_scaled<Op::I8, false, false, 4 | 0 << 3>(p, c, cu, st);
        case 0 | 3 << 3: return by_scaled<Op::I8, false, false, 0 | 3 << 3>(p, c, cu, st);
        case 3 | 3 << 3: return by_scaled<Op::I8, false, false, 3 | 3 << 3>(p, c, cu, st);
        case 4 | 3 << 3: return by_scaled<Op::I8, false, false, 4 | 3 << 3>(p, c, cu, st);
        case 0 | 4 << 3: return by_scaled<Op::I8, false, false, 0 | 4 << 3>(p, c, cu, st);
        case 3 | 4 << 3: return by_scaled<Op::I8, false, false, 3 | 4 << 3>(p, c, cu, st);
        case 4 | 4 << 3: return by_scaled<Op::I8, false, false, 4 | 4 << 3>(p, c, cu, st);
      }
      return hipErrorInvalidValue;
  }
  return hipErrorInvalidValue;
}

hipError_t launch_tgmm(const Params& p, int cu, int cap, hipStream_t st) {
  if (p.out_f32) return launch_tgmm_cfg<TgCfg<true>>(p, cu, cap, st);
  return launch_tgmm_cfg<TgCfg<false>>(p, cu, cap, st);
}

// The plan-building device code of the kernels, run on its own to export
// the tiles.
__global__ __launch_bounds__(256) void worklist_kernel(Params p, int tm, int32_t* tiles,
                                                       long long capacity, int32_t* count) {
  __shared__ Plan pl;
  if (threadIdx.x == 0) pl.flags = 0;
  __syncthreads();
  build_plan<256>(p, pl, tm);
  for (int t = threadIdx.x; t < pl.n_mtiles; t += 256) {
    if (t >= capacity) break;
    const int h = find_group(pl, t);
    const int row0 = pl.row_start[h] + (t - pl.tile_start[h]) * tm;
    const int left = pl.row_start[h + 1] - row0;
    tiles[3 * t + 0] = pl.s + h;
    tiles[3 * t + 1] = row0;
    tiles[3 * t + 2] = left < tm ? left : tm;
  }
  if (threadIdx.x == 0) {
    count[0] = pl.n_mtiles;
    count[1] = pl.row_start[0];
    count[2] = pl.row_start[pl.ga];
    count[3] = (int)pl.flags;
  }
}

hipError_t launch_worklist(const Params& p, int tm, int32_t* tiles, long long capacity,
                           int32_t* count, hipStream_t stream) {
  hipLaunchKernelGGL(worklist_kernel, dim3(1), dim3(256), 0, stream, p, tm, tiles, capacity, count);
  return hipGetLastError();
}

}  // namespace gmmk
