// gmm_quant.hip -- the activation quantiser on gfx950: bf16 x [M,K] to
// e4m3fn q [M,K] and an f32 scale per 128-element block of each row, the
// per_token_group_quant_fp8 launcher of the metrale gemm_quant.rs page (its
// scale is the activation scale that page's fp8_gemm_t_blockscaled applies,
// x ~ q * scale).  The page states the shapes only; the arithmetic is
//   scale = amax / 448 in binary32 (448 the largest finite e4m3fn value;
//           1 for an all-zero block),
//   q     = the nearest e4m3fn value to clamp(x / scale, -448, 448), with
//           x / scale one correctly rounded binary32 division and ties to
//           the even mantissa.
//
// The pass is HBM-bound (2 bytes read, 1 written per element).  Because K is
// a multiple of 128 the matrix is a flat run of 256-byte blocks: block j is
// bytes [256 j, 256 j + 256) of x, [128 j, 128 j + 128) of q and word j of
// scale.  Eight lanes (half a DPP row) take one block, 32 bytes (16 values)
// per lane, so every lane reads two whole 16-byte words, writes one 16-byte
// word of codes, and the block's amax is three lane permutations away.
// Loads and stores are non-temporal: nothing is read twice.  (On this part
// the pass runs at the rate of a plain device copy of the same bytes.)
//
// The quotients come from the block's reciprocal: with y = 1/s correctly
// rounded, q0 = x*y rounded is within an ulp of x/s, the remainder
// r = x - q0*s is exact in one fma, and q0 + r*y rounded to nearest is the
// correctly rounded quotient (Markstein's theorem on division by a
// correctly rounded reciprocal) -- three operations instead of a division.
// The remainder is exact when ulp(q0) * ulp(s) >= 2^-149; for the quotients
// that can decide a code (>= 2^-11: smaller ones round to zero) that holds
// once s >= 2^-92.  A block with a smaller scale divides.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "gmm_launch.hpp"

namespace gmmk {

namespace {

constexpr int kQuantT = 256;  // threads per workgroup: 32 groups of 8 lanes
constexpr int kGroupsPerWg = kQuantT / 8;
constexpr int kWgPerCu = 4;

typedef short short2_t __attribute__((ext_vector_type(2)));
typedef unsigned u32x4 __attribute__((ext_vector_type(4)));

// max over each group of 8 lanes (half a DPP row): swap neighbours, swap
// pairs, then mirror the half-row.  The values are bit patterns of
// non-negative floats, whose integer order is their order.
__device__ __forceinline__ unsigned group_max(unsigned v) {
  v = max(v, (unsigned)__builtin_amdgcn_mov_dpp((int)v, 0xB1, 0xF, 0xF, false));   // quad_perm [1,0,3,2]
  v = max(v, (unsigned)__builtin_amdgcn_mov_dpp((int)v, 0x4E, 0xF, 0xF, false));   // quad_perm [2,3,0,1]
  v = max(v, (unsigned)__builtin_amdgcn_mov_dpp((int)v, 0x141, 0xF, 0xF, false));  // row_half_mirror
  return v;
}

__device__ __forceinline__ float clamp448(float t) { return fminf(fmaxf(t, -448.0f), 448.0f); }

// x / s correctly rounded, given y = 1/s correctly rounded and s >= 2^-92.
// The quotient has x's sign (s > 0); the fmas alone would turn a -0 (or a
// negative quotient that underflows) into +0, hence the copysign.
__device__ __forceinline__ float quotient(float x, float s, float y) {
#pragma clang fp contract(off)
  const float q0 = x * y;
  const float r = __builtin_fmaf(-q0, s, x);
  return __builtin_copysignf(__builtin_fmaf(r, y, q0), x);
}

__global__ __launch_bounds__(kQuantT) void quant_fp8_kernel(QuantParams p) {
  const int r8 = threadIdx.x & 7;
  const long long groups = (long long)gridDim.x * kGroupsPerWg;  // lane groups of the grid
  const long long B = p.blocks;
  const char* const x = reinterpret_cast<const char*>(p.x);
  // a group's blocks are g, g + groups, ...; its 8 lanes share the trip
  // count, so the permutations always see the whole group active
  for (long long j = (long long)blockIdx.x * kGroupsPerWg + (threadIdx.x >> 3); j < B; j += groups) {
    const u32x4* src = reinterpret_cast<const u32x4*>(x + j * 256 + r8 * 32);
    const u32x4 a = __builtin_nontemporal_load(src), b = __builtin_nontemporal_load(src + 1);
    const unsigned w[8] = {a.x, a.y, a.z, a.w, b.x, b.y, b.z, b.w};
    float v[16];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      v[2 * i] = __uint_as_float(w[i] << 16);  // bf16 -> f32 is exact
      v[2 * i + 1] = __uint_as_float(w[i] & 0xFFFF0000u);
    }
    unsigned am = 0;
#pragma unroll
    for (int i = 0; i < 16; ++i) am = max(am, __float_as_uint(v[i]) & 0x7FFFFFFFu);
    const float amax = __uint_as_float(group_max(am));
    const float s = amax == 0.0f ? 1.0f : amax / 448.0f;
    float t[16];
    if (s >= 0x1p-92f) {
      const float y = 1.0f / s;
#pragma unroll
      for (int i = 0; i < 16; ++i) t[i] = clamp448(quotient(v[i], s, y));
    } else {
#pragma unroll
      for (int i = 0; i < 16; ++i) t[i] = clamp448(v[i] / s);
    }
    u32x4 codes;
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      short2_t c = {0, 0};
      c = __builtin_amdgcn_cvt_scalef32_pk_fp8_f32(c, t[4 * k], t[4 * k + 1], 1.0f, false);
      c = __builtin_amdgcn_cvt_scalef32_pk_fp8_f32(c, t[4 * k + 2], t[4 * k + 3], 1.0f, true);
      codes[k] = __builtin_bit_cast(unsigned, c);
    }
    __builtin_nontemporal_store(codes, reinterpret_cast<u32x4*>(reinterpret_cast<char*>(p.q) + j * 128 + r8 * 16));
    if (r8 == 0) __builtin_nontemporal_store(s, p.scale + j);
  }
}

// Block scales widened to binary32 (widen_block_scale_f32 of the metrale
// gemm_quant.rs page): bf16 exactly, f32 as is, and an E8M0 byte e as the
// binary32 with bit pattern e << 23 (2^(e - 127)), except 2^-127 for e = 0
// and 0.0 for e = 255, as the page states.  Scale tensors are small; one
// element per thread, grid-stride.
__global__ __launch_bounds__(256) void widen_scales_kernel(WidenParams p) {
  const long long stride = (long long)gridDim.x * 256;
  for (long long i = (long long)blockIdx.x * 256 + threadIdx.x; i < p.n; i += stride) {
    float v;
    if (p.dtype == kScaleBf16) {
      v = __uint_as_float((uint32_t) reinterpret_cast<const uint16_t*>(p.src)[i] << 16);
    } else if (p.dtype == kScaleF32) {
      v = reinterpret_cast<const float*>(p.src)[i];
    } else {
      const uint32_t e = reinterpret_cast<const uint8_t*>(p.src)[i];
      v = __uint_as_float(e == 0 ? 0x00400000u : (e == 255 ? 0u : e << 23));
    }
    p.dst[i] = v;
  }
}

}  // namespace

hipError_t launch_widen_scales(const WidenParams& p, int cu_count, hipStream_t stream) {
  long long grid = (p.n + 255) / 256;
  if (grid > (long long)cu_count * 8) grid = (long long)cu_count * 8;
  if (grid < 1) grid = 1;
  hipLaunchKernelGGL(widen_scales_kernel, dim3((unsigned)grid), dim3(256), 0, stream, p);
  return hipGetLastError();
}

hipError_t launch_quant_fp8(const QuantParams& p, int cu_count, hipStream_t stream) {
  long long grid = (p.blocks + kGroupsPerWg - 1) / kGroupsPerWg;
  const long long cap = (long long)cu_count * kWgPerCu;
  if (grid > cap) grid = cap;
  if (grid < 1) grid = 1;
  hipLaunchKernelGGL(quant_fp8_kernel, dim3((unsigned)grid), dim3(kQuantT), 0, stream, p);
  return hipGetLastError();
}

}  // namespace gmmk
