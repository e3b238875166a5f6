// gmm_device.hpp -- device code of the gfx950 grouped matmul.
//
// One persistent kernel family computes the whole operation in a single
// launch:
//   1. every workgroup turns group_sizes and the group offset into group
//      offsets and a table of group-aligned m-tiles, in LDS (the group
//      offsets of make_group_metadata on the tpu-inference 0.13.2 wheel diff
//      page, megablox/gmm.py; tiles start at each group's first row, so no
//      tile holds rows of two groups);
//   2. it then takes work items in turn: an item is an (m-tile, n-tile) pair
//      computed with MFMA from LDS-staged, double-buffered K tiles, or a
//      slice of the rows outside the active groups, which it zeroes
//      (_zero_uninitialized_memory on the same page) or, given an existing
//      output, copies from it or leaves alone when it is the output itself
//      (gmm's existing_out there: each output tile starts from it and only
//      the group's rows are stored over it).
// The contraction, the per-block scale fold and the bias follow the kernel
// body of gmm() on that page (_accum); the per-token lhs scale follows the
// block-scaled W8A8 GEMM of the metrale gemm_quant.rs page
// (fp8_gemm_t_blockscaled); the in-place [G,K,N] weight read follows the
// MaxText PR "Megablox: transposed-RHS gmm_v2 kernel for the backward dlhs".
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "gmm_params.hpp"

namespace gmmk {

typedef int i32x2 __attribute__((ext_vector_type(2)));
typedef int i32x4 __attribute__((ext_vector_type(4)));
typedef int i32x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

// Group plan kept in LDS for the whole life of a workgroup.
struct Plan {
  int32_t tile_start[kMaxGroups + 1];  // first m-tile of active group h
  int32_t row_start[kMaxGroups + 1];   // o[s + h], clamped to [0, M]
  long long wave_tot[16];
  int32_t s, ga, n_mtiles;
  unsigned int flags;
};

// ---------------------------------------------------------------------------
// prologue: group offsets and m-tile table

// Exclusive prefix sum of one value per thread over the workgroup.
template <int T>
__device__ inline long long block_excl_scan(long long v, long long* wave_tot, long long* total) {
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  long long incl = v;
#pragma unroll
  for (int d = 1; d < 64; d <<= 1) {
    long long y = __shfl_up(incl, d, 64);
    if (lane >= d) incl += y;
  }
  if (lane == 63) wave_tot[w] = incl;
  __syncthreads();
  long long base = 0, tot = 0;
#pragma unroll
  for (int i = 0; i < T / 64; ++i) {
    long long x = wave_tot[i];
    if (i < w) base += x;
    tot += x;
  }
  __syncthreads();
  *total = tot;
  return base + incl - v;
}

// Builds the plan for m-tiles of height bm.  Values outside the contract are
// clamped so that every later access stays in bounds, and reported in flags:
// negative sizes count as 0, offsets beyond M are cut to M, an offset outside
// [0, G-Ga] is clamped into [0, G] with Ga cut to G - s.
template <int T>
__device__ void build_plan(const Params& p, Plan& pl, int bm) {
  constexpr int EMAX = (kMaxGroups + T - 1) / T;
  const int tid = threadIdx.x;
  uint32_t flags = 0;

  // o[g+1] for the groups this thread owns (a contiguous run of E groups).
  // The sizes and the offset come in through range-checked buffer loads, all
  // issued before the first use: sizes past G (and the offset when there is
  // none) read as 0, so no branch stands between the loads, and the plan
  // waits for memory once instead of once per load.
  const int E = (p.G + T - 1) / T;
  const __amdgpu_buffer_rsrc_t rsz = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<int32_t*>(p.group_sizes), (short)0, p.G * 4, kBufferRsrcWord3);
  const __amdgpu_buffer_rsrc_t rof = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<int32_t*>(p.group_offset), (short)0, p.group_offset ? 4 : 0, kBufferRsrcWord3);
  int raw[EMAX];
#pragma unroll
  for (int e = 0; e < EMAX; ++e) raw[e] = __builtin_amdgcn_raw_buffer_load_b32(rsz, (tid * E + e) * 4, 0, 0);
  int s = __builtin_amdgcn_raw_buffer_load_b32(rof, 0, 0, 0);
  long long loc[EMAX];
  long long sum = 0;
#pragma unroll
  for (int e = 0; e < EMAX; ++e) {
    // entries e >= E belong to the next thread's run
    int x = e < E ? raw[e] : 0;
    if (x < 0) {
      flags |= kFlagNegative;
      x = 0;
    }
    sum += x;
    loc[e] = sum;
  }
  if (s < 0 || s > p.G - p.Ga) {
    flags |= kFlagBadOffset;
    s = s < 0 ? 0 : (s > p.G ? p.G : s);
  }
  const int ga = p.Ga < p.G - s ? p.Ga : p.G - s;
  long long total;
  const long long excl = block_excl_scan<T>(sum, pl.wave_tot, &total);
  if (total > p.M) flags |= kFlagExceed;
#pragma unroll
  for (int e = 0; e < EMAX; ++e) {
    const int g = tid * E + e;
    if (e < E && g < p.G) {
      const int h = g + 1 - s;
      if (h >= 0 && h <= ga) {
        long long o = excl + loc[e];
        pl.row_start[h] = (int)(o < p.M ? o : p.M);
      }
    }
  }
  if (tid == 0 && s == 0) pl.row_start[0] = 0;
  __syncthreads();

  // m-tiles per active group, then their prefix sum.
  const int E2 = (ga + T - 1) / T;
  long long loc2[EMAX];
  long long sum2 = 0;
#pragma unroll
  for (int e = 0; e < EMAX; ++e) {
    const int h = tid * E2 + e;
    long long c = 0;
    if (e < E2 && h < ga) c = (pl.row_start[h + 1] - pl.row_start[h] + bm - 1) / bm;
    sum2 += c;
    loc2[e] = sum2;
  }
  long long total2;
  const long long excl2 = block_excl_scan<T>(sum2, pl.wave_tot, &total2);
#pragma unroll
  for (int e = 0; e < EMAX; ++e) {
    const int h = tid * E2 + e;
    if (e < E2 && h < ga) pl.tile_start[h + 1] = (int)(excl2 + loc2[e]);
  }
  if (tid == 0) {
    pl.tile_start[0] = 0;
    pl.s = s;
    pl.ga = ga;
    pl.n_mtiles = (int)total2;
  }
  // Block-wide OR of the flags (only workgroup 0 reports them).
  if (flags) atomicOr(&pl.flags, flags);
  __syncthreads();
}

// Active group (relative index h) that holds m-tile t, 0 <= t < n_mtiles:
// the largest h with tile_start[h] <= t.  Empty groups own no tile and are
// never returned.
__device__ inline int find_group(const Plan& pl, int t) {
  int lo = 0, hi = pl.ga;
  while (hi - lo > 1) {
    const int mid = (lo + hi) >> 1;
    if (pl.tile_start[mid] <= t)
      lo = mid;
    else
      hi = mid;
  }
  return lo;
}

__device__ inline void report_flags(const Params& p, const Plan& pl) {
  if (blockIdx.x == 0 && threadIdx.x == 0 && pl.flags) atomicOr(p.flags, (uint32_t)pl.flags);
}

// Position of a logical work item among the workgroups of one round: the
// hardware hands workgroups to the 8 XCDs in turn, so workgroup b runs on
// XCD b % 8; giving each XCD a contiguous run of items keeps the operands
// those items share in that XCD's L2.
__device__ inline int xcd_slot(int b, int P) {
  if (P % 8) return b;
  return (b % 8) * (P / 8) + b / 8;
}

// ---------------------------------------------------------------------------
// element helpers

__device__ inline __amdgpu_buffer_rsrc_t make_rsrc(const void* base, long long bytes) {
  int n = bytes > 0x7FFFFFF0LL ? 0x7FFFFFF0 : (int)(bytes < 0 ? 0 : bytes);
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, n, kBufferRsrcWord3);
}

// Two one-byte values (bytes 0-1 or 2-3 of w) widened to two bf16: format
// F = 0 e4m3fn, 1 e5m2, 2 int8.  Exact: every finite value of each is a
// bf16 (an int8 has at most 8 significant bits, so the low half of its
// binary32 is zero).
template <int F>
__device__ __forceinline__ bf16x2 fp8x2_to_bf16x2(unsigned w, bool hi) {
  if constexpr (F == 0) {
    return hi ? __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w, 1.0f, true)
              : __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w, 1.0f, false);
  } else if constexpr (F == 1) {
    return hi ? __builtin_amdgcn_cvt_scalef32_pk_bf16_bf8(w, 1.0f, true)
              : __builtin_amdgcn_cvt_scalef32_pk_bf16_bf8(w, 1.0f, false);
  } else {
    const unsigned h = hi ? w >> 16 : w;
    const float f0 = (float)(int)(int8_t)(h & 0xFF), f1 = (float)(int)(int8_t)((h >> 8) & 0xFF);
    const unsigned bits = (__float_as_uint(f0) >> 16) | (__float_as_uint(f1) & 0xFFFF0000u);
    return __builtin_bit_cast(bf16x2, bits);
  }
}

// 8 four-bit values (the nibbles of w, the low nibble of each byte first)
// of format F = 3 int4, 4 uint4, 5 fp4 e2m1 widened to 8 bf16 (exact: each
// value has at most 3 significant bits).
template <int F>
__device__ inline i32x4 nib8_to_bf16x8(unsigned w) {
  i32x4 r;
  if constexpr (F == 5) {
    r[0] = __builtin_bit_cast(int, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, 1.0f, 0));
    r[1] = __builtin_bit_cast(int, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, 1.0f, 1));
    r[2] = __builtin_bit_cast(int, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, 1.0f, 2));
    r[3] = __builtin_bit_cast(int, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, 1.0f, 3));
  } else {
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      int lo = (w >> (8 * j)) & 15, hi = (w >> (8 * j + 4)) & 15;
      if constexpr (F == 3) {
        lo = (lo ^ 8) - 8;
        hi = (hi ^ 8) - 8;
      }
      r[j] = (int)((__float_as_uint((float)lo) >> 16) | (__float_as_uint((float)hi) & 0xFFFF0000u));
    }
  }
  return r;
}

// 8 one-byte values of format F widened to 8 bf16.
template <int F>
__device__ inline i32x4 fp8x8_to_bf16x8(i32x2 v) {
  i32x4 r;
  r[0] = __builtin_bit_cast(int, fp8x2_to_bf16x2<F>((unsigned)v[0], false));
  r[1] = __builtin_bit_cast(int, fp8x2_to_bf16x2<F>((unsigned)v[0], true));
  r[2] = __builtin_bit_cast(int, fp8x2_to_bf16x2<F>((unsigned)v[1], false));
  r[3] = __builtin_bit_cast(int, fp8x2_to_bf16x2<F>((unsigned)v[1], true));
  return r;
}

__device__ inline float bf16_bits_to_f32(uint16_t b) { return __uint_as_float((uint32_t)b << 16); }

__device__ inline uint16_t f32_to_bf16_rne(float f) {
  __bf16 b = (__bf16)f;
  return __builtin_bit_cast(uint16_t, b);
}

// Two values rounded the same way and packed, lo in bits 0-15: one
// v_cvt_pk_bf16_f32 for the pair (converting each value on its own costs one
// conversion per value plus the shifts and ors that pack them).
__device__ __forceinline__ uint32_t pk_bf16_rne(float lo, float hi) {
  typedef float f32x2_t __attribute__((ext_vector_type(2)));
  typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2_t{lo, hi}, bf16x2_t));
}

// 16-byte chunk c (0..7) of a 128-byte LDS row r is stored at chunk
// c ^ swz(r).  Sixteen consecutive rows read at one logical chunk hit sixteen
// distinct 16-byte bank groups, with 32 or 64 banks.
__device__ inline int swz(int r) { return (r ^ (r >> 3)) & 7; }
__device__ inline int lds_off(int r, int c) { return r * 128 + ((c ^ swz(r)) << 4); }

// ---------------------------------------------------------------------------
// tile configurations

// FMT_: the narrow formats, FMT_ & 7 for lhs (FA) and FMT_ >> 3 for rhs
// (FB).  fp8 x fp8 products (Op::FP8): 0 e4m3fn, 1 e5m2, 4 fp4 e2m1 -- the
// format codes of the f8f6f4 matrix instructions.  int8 products (Op::I8):
// 0 int8, 3 int4, 4 uint4.  bf16 products with narrow weights widened to
// bf16 (B_FP8): FB 0 e4m3fn, 1 e5m2, 2 int8, 3 int4, 4 uint4, 5 fp4 e2m1.
// The four-bit types are packed two to a byte.
// MX_: E8M0 block scales of 32 K elements applied by the scaled f8f6f4
// instruction itself (no fold; SCALED_ is false).
template <Op OP, bool NN_, bool BFP8_, int BM_, int BN_, int WM_, int WN_, bool SCALED_, int FMT_ = 0,
          bool MX_ = false>
struct Cfg {
  static constexpr Op op = OP;
  static constexpr bool NN = NN_;        // rhs is [Ga,K,N]
  static constexpr bool B_FP8 = BFP8_;   // fp8 rhs widened to bf16 operands
  static constexpr bool SCALED = SCALED_;
  static constexpr bool MX = MX_;
  static constexpr int FA = FMT_ & 7, FB = FMT_ >> 3;
  static constexpr int BM = BM_, BN = BN_, WM = WM_, WN = WN_;
  static constexpr int T = 64 * WM * WN;
  static constexpr int ES = OP == Op::F32 ? 4 : (OP == Op::BF16 ? 2 : 1);  // operand bytes
  static constexpr int BK = 128 / ES;       // K elements per 128-byte LDS row
  static constexpr int TM = BM / WM, TN = BN / WN;
  static constexpr int FM = TM / 16, FN = TN / 16;
  static constexpr int A_CH = BM * 8 / T;   // 16-byte A chunks per thread
  static constexpr int B_CH = BN * 8 / T;   // 16-byte B operand chunks per thread
  static constexpr int KB = 16 / ES;        // K elements per 16-byte chunk
  static constexpr int NW = BN * 8 / T;     // NN: n-columns per thread block
  static constexpr int A_BYTES = BM * 128, B_BYTES = BN * 128;
  static constexpr int LDS = 2 * (A_BYTES + B_BYTES);
  static constexpr int BSB = B_FP8 ? 1 : ES;  // rhs storage bytes per element (four-bit: half)
  static constexpr bool B_NIB = B_FP8 && FB >= 3;  // four-bit weights widened to bf16
  // four-bit operands of a one-byte product (fp4 e2m1 on the f8f6f4
  // instruction as it is; int4 / uint4 widened to int8 in LDS): a K step of
  // 128 elements is 64 bytes of a row, loaded 8 bytes a chunk
  static constexpr bool A_Q4 = (OP == Op::FP8 && FA == 4) || (OP == Op::I8 && FA >= 3);
  static constexpr bool B_Q4 = (OP == Op::FP8 && FB == 4) || (OP == Op::I8 && FB >= 3);
  // bytes of `elems` consecutive rhs / lhs elements (an even count when four-bit)
  __device__ static constexpr long long rhs_bytes(long long elems) {
    return (B_NIB || B_Q4) ? elems / 2 : elems * BSB;
  }
  __device__ static constexpr long long lhs_bytes(long long elems) { return A_Q4 ? elems / 2 : elems * ES; }
  static_assert(TM % 16 == 0 && TN % 16 == 0, "wave tile must be a multiple of 16");
  static_assert(A_CH >= 1 && A_CH * T == BM * 8, "A tile must split evenly");
  static_assert(B_CH >= 1 && B_CH * T == BN * 8, "B tile must split evenly");
  static_assert(!NN || (!B_FP8 && OP != Op::FP8), "NN needs f32 or bf16 weights");
  static_assert(!NN || NW == 2 || NW == 4 || NW == 8, "NN thread block width");
  static_assert(!B_FP8 || OP == Op::BF16, "fp8 weights widen to bf16");
  static_assert(OP == Op::FP8 || OP == Op::I8 || FA == 0, "an lhs format only for one-byte products");
  static_assert(OP == Op::FP8 || OP == Op::I8 || B_FP8 || FB == 0, "an rhs format only for narrow weights");
  static_assert(OP != Op::FP8 || ((FA <= 1 || FA == 4) && (FB <= 1 || FB == 4)),
                "f8f6f4 formats: e4m3fn, e5m2 or fp4 e2m1");
  static_assert(OP != Op::I8 || ((FA == 0 || FA == 3 || FA == 4) && (FB == 0 || FB == 3 || FB == 4)),
                "int8 products: int8, int4 or uint4 operands");
  static_assert(!NN || OP != Op::I8, "NN needs f32 or bf16 weights");
  static_assert(!MX || (OP == Op::FP8 && !SCALED), "E8M0 block scales on the f8f6f4 instruction");
};

// 16 nibbles (two words, the low nibble of each byte first) widened to 16
// int8: F = 3 int4 (sign-extended), 4 uint4.  Byte 2j of the result is the
// low nibble of input byte j and byte 2j+1 its high nibble.
template <int F>
__device__ inline i32x4 nib16_to_i8x16(i32x2 v) {
  i32x4 r;
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    const uint32_t x = (uint32_t)v[h];
    const uint32_t lo = x & 0x0F0F0F0Fu, hi = (x >> 4) & 0x0F0F0F0Fu;
    // interleave: bytes (lo.b0, hi.b0, lo.b1, hi.b1), then (lo.b2, hi.b2, lo.b3, hi.b3)
    uint32_t w0 = __builtin_amdgcn_perm(hi, lo, 0x05010400u);
    uint32_t w1 = __builtin_amdgcn_perm(hi, lo, 0x07030602u);
    if constexpr (F == 3) {  // bit 3 of a nibble set: its byte gets 0xF0 (the sign extension)
      w0 |= (w0 & 0x08080808u) * 0x1Eu;
      w1 |= (w1 & 0x08080808u) * 0x1Eu;
    }
    r[2 * h] = (int)w0;
    r[2 * h + 1] = (int)w1;
  }
  return r;
}

// Staged operand chunk into its 16-byte LDS slot.  A four-bit chunk (Q4,
// 16 values in v[0..1]) of an int8 product is widened to 16 int8; of an
// f8f6f4 product (fp4 e2m1) it stays packed in the slot's first 8 bytes.
template <Op OP, bool Q4, int F>
__device__ __forceinline__ void store_q(char* slot, i32x4 v) {
  if constexpr (!Q4) {
    *reinterpret_cast<i32x4*>(slot) = v;
  } else if constexpr (OP == Op::I8) {
    *reinterpret_cast<i32x4*>(slot) = nib16_to_i8x16<F>(i32x2{v[0], v[1]});
  } else {
    *reinterpret_cast<i32x2*>(slot) = i32x2{v[0], v[1]};
  }
}

// One operand of the 16x16x128 f8f6f4 instruction for the K step in a row
// (lane quarter q).  The instruction's lane layouts differ by width (read
// off gfx950 with a one-hot probe): a one-byte operand's lane quarter q
// holds K elements 16 q + [0,16) in its first four registers and
// 64 + 16 q + [0,16) in the next four -- 16 bytes from slots q and q + 4;
// an fp4 e2m1 operand's holds K elements 32 q + [0,32), packed in four
// registers -- the 8 bytes of slots 2 q and 2 q + 1.  Each side in its own
// layout, mixed products pair the same K elements.
template <int F>
__device__ __forceinline__ i32x8 f8f6f4_operand(const char* base, int r, int q) {
  if constexpr (F == 4) {
    const i32x2 lo = *reinterpret_cast<const i32x2*>(base + lds_off(r, 2 * q));
    const i32x2 hi = *reinterpret_cast<const i32x2*>(base + lds_off(r, 2 * q + 1));
    return i32x8{lo[0], lo[1], hi[0], hi[1], 0, 0, 0, 0};
  } else {
    const i32x4 lo = *reinterpret_cast<const i32x4*>(base + lds_off(r, q));
    const i32x4 hi = *reinterpret_cast<const i32x4*>(base + lds_off(r, q + 4));
    return i32x8{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
  }
}

// ---------------------------------------------------------------------------
// the kernel

template <class C>
struct Stage {
  i32x4 a[C::A_CH];
  // NT: B_CH chunks of operand (or fp8 half-chunks in .x/.y when B_FP8);
  // NN: KB rows of NW elements, packed into B_CH chunks.
  i32x4 b[C::B_CH];
};

template <class C>
__device__ inline void load_tile(const C&, Stage<C>& st, __amdgpu_buffer_rsrc_t ar,
                                 __amdgpu_buffer_rsrc_t br, int kt, int K, int N, int n0) {
  const int tid = threadIdx.x;
  const int arow_bytes = K * C::ES;
#pragma unroll
  for (int i = 0; i < C::A_CH; ++i) {
    const int c = tid + i * C::T;
    const int r = c >> 3, cc = c & 7;
    if constexpr (C::A_Q4) {
      const i32x2 v = __builtin_amdgcn_raw_buffer_load_b64(ar, r * (K / 2) + kt * 64 + cc * 8, 0, 0);
      st.a[i] = i32x4{v[0], v[1], 0, 0};
    } else {
      st.a[i] = __builtin_amdgcn_raw_buffer_load_b128(ar, r * arow_bytes + kt * 128 + cc * 16, 0, 0);
    }
  }
  if constexpr (!C::NN) {
#pragma unroll
    for (int i = 0; i < C::B_CH; ++i) {
      const int c = tid + i * C::T;
      const int r = c >> 3, cc = c & 7;
      if constexpr (C::B_Q4) {
        const i32x2 v = __builtin_amdgcn_raw_buffer_load_b64(br, r * (K / 2) + kt * 64 + cc * 8, 0, 0);
        st.b[i] = i32x4{v[0], v[1], 0, 0};
      } else if constexpr (C::B_NIB) {
        st.b[i][0] = __builtin_amdgcn_raw_buffer_load_b32(br, r * (K / 2) + kt * 32 + cc * 4, 0, 0);
        st.b[i][1] = 0;
      } else if constexpr (C::B_FP8) {
        i32x2 v = __builtin_amdgcn_raw_buffer_load_b64(br, r * K + kt * 64 + cc * 8, 0, 0);
        st.b[i][0] = v[0];
        st.b[i][1] = v[1];
      } else {
        st.b[i] = __builtin_amdgcn_raw_buffer_load_b128(br, r * K * C::ES + kt * 128 + cc * 16, 0, 0);
      }
    }
  } else {
    // Thread block: KB consecutive k rows x NW consecutive n columns.
    constexpr int NBLK = C::BN / C::NW;
    const int nb = tid % NBLK, kb = tid / NBLK;
    const int nbase = n0 + nb * C::NW;
    const int kbase = kt * C::BK + kb * C::KB;
    constexpr int RB = C::NW * C::ES;  // bytes per row piece: 4, 8 or 16
    int* words = reinterpret_cast<int*>(&st.b[0]);
#pragma unroll
    for (int kr = 0; kr < C::KB; ++kr) {
      const int off = ((kbase + kr) * N + nbase) * C::ES;
      if constexpr (RB == 4) {
        words[kr] = __builtin_amdgcn_raw_buffer_load_b32(br, off, 0, 0);
      } else if constexpr (RB == 8) {
        i32x2 v = __builtin_amdgcn_raw_buffer_load_b64(br, off, 0, 0);
        words[2 * kr] = v[0];
        words[2 * kr + 1] = v[1];
      } else {
        i32x4 v = __builtin_amdgcn_raw_buffer_load_b128(br, off, 0, 0);
        words[4 * kr + 0] = v[0];
        words[4 * kr + 1] = v[1];
        words[4 * kr + 2] = v[2];
        words[4 * kr + 3] = v[3];
      }
    }
  }
}

template <class C>
__device__ inline void store_tile(const C&, const Stage<C>& st, char* sa, char* sb) {
  const int tid = threadIdx.x;
#pragma unroll
  for (int i = 0; i < C::A_CH; ++i) {
    const int c = tid + i * C::T;
    store_q<C::op, C::A_Q4, C::FA>(sa + lds_off(c >> 3, c & 7), st.a[i]);
  }
  if constexpr (!C::NN) {
#pragma unroll
    for (int i = 0; i < C::B_CH; ++i) {
      const int c = tid + i * C::T;
      i32x4 v = st.b[i];
      if constexpr (C::B_NIB)
        v = nib8_to_bf16x8<C::FB>((unsigned)st.b[i][0]);
      else if constexpr (C::B_FP8)
        v = fp8x8_to_bf16x8<C::FB>(i32x2{st.b[i][0], st.b[i][1]});
      store_q<C::op, C::B_Q4, C::FB>(sb + lds_off(c >> 3, c & 7), v);
    }
  } else {
    constexpr int NBLK = C::BN / C::NW;
    const int nb = tid % NBLK, kb = tid / NBLK;
    const int* words = reinterpret_cast<const int*>(&st.b[0]);
#pragma unroll
    for (int j = 0; j < C::NW; ++j) {
      i32x4 v;
      if constexpr (C::ES == 2) {
        // element (kr, j) is the 16-bit half j&1 of word kr*NW/2 + j/2
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const uint32_t w0 = (uint32_t)words[(2 * q) * (C::NW / 2) + j / 2];
          const uint32_t w1 = (uint32_t)words[(2 * q + 1) * (C::NW / 2) + j / 2];
          const uint32_t lo = (j & 1) ? (w0 >> 16) : (w0 & 0xFFFFu);
          const uint32_t hi = (j & 1) ? (w1 & 0xFFFF0000u) : (w1 << 16);
          v[q] = (int)(lo | hi);
        }
      } else {
#pragma unroll
        for (int q = 0; q < 4; ++q) v[q] = words[q * C::NW + j];
      }
      const int r = nb * C::NW + j;
      *reinterpret_cast<i32x4*>(sb + lds_off(r, kb)) = v;
    }
  }
}

// The value of one accumulator element: int8 x int8 tiles accumulate exact
// int32 sums in the same registers (their bits), the others binary32.
template <class C>
__device__ __forceinline__ float acc_value(float a) {
  if constexpr (C::op == Op::I8)
    return (float)__float_as_int(a);
  else
    return a;
}

// acc[fm][fn] += A(wave rows fm) * B(wave cols fn) over one 128-byte K row.
template <class C>
__device__ inline void mma_tile(f32x4 (&acc)[C::FM][C::FN], const char* sa, const char* sb) {
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int wm = w / C::WN, wn = w % C::WN;
  const int q = lane >> 4, r16 = lane & 15;
  if constexpr (C::op == Op::I8) {
    // two 16x16x64 int8 products per 128-byte row: lane quarter q takes K
    // bytes 16q .. 16q+15, then 64 + 16q .. (the same K order in A and B)
#pragma unroll
    for (int kk = 0; kk < 2; ++kk) {
      i32x4 bfr[C::FN];
#pragma unroll
      for (int fn = 0; fn < C::FN; ++fn)
        bfr[fn] = *reinterpret_cast<const i32x4*>(sb + lds_off(wn * C::TN + fn * 16 + r16, q + 4 * kk));
#pragma unroll
      for (int fm = 0; fm < C::FM; ++fm) {
        const i32x4 af = *reinterpret_cast<const i32x4*>(sa + lds_off(wm * C::TM + fm * 16 + r16, q + 4 * kk));
#pragma unroll
        for (int fn = 0; fn < C::FN; ++fn)
          acc[fm][fn] = __builtin_bit_cast(
              f32x4, __builtin_amdgcn_mfma_i32_16x16x64_i8(af, bfr[fn], __builtin_bit_cast(i32x4, acc[fm][fn]), 0, 0, 0));
      }
    }
  } else if constexpr (C::op == Op::FP8) {
    i32x8 bf[C::FN];
#pragma unroll
    for (int fn = 0; fn < C::FN; ++fn) bf[fn] = f8f6f4_operand<C::FB>(sb, wn * C::TN + fn * 16 + r16, q);
#pragma unroll
    for (int fm = 0; fm < C::FM; ++fm) {
      const i32x8 af = f8f6f4_operand<C::FA>(sa, wm * C::TM + fm * 16 + r16, q);
#pragma unroll
      for (int fn = 0; fn < C::FN; ++fn)
        acc[fm][fn] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(af, bf[fn], acc[fm][fn],
                                                                       C::FA, C::FB, 0, 0, 0, 0);
    }
  } else {
#pragma unroll
    for (int kk = 0; kk < 2; ++kk) {
      i32x4 bfr[C::FN];
#pragma unroll
      for (int fn = 0; fn < C::FN; ++fn) {
        const int r = wn * C::TN + fn * 16 + r16;
        bfr[fn] = *reinterpret_cast<const i32x4*>(sb + lds_off(r, q + 4 * kk));
      }
#pragma unroll
      for (int fm = 0; fm < C::FM; ++fm) {
        const int r = wm * C::TM + fm * 16 + r16;
        const i32x4 af = *reinterpret_cast<const i32x4*>(sa + lds_off(r, q + 4 * kk));
#pragma unroll
        for (int fn = 0; fn < C::FN; ++fn) {
          if constexpr (C::op == Op::BF16) {
            acc[fm][fn] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
                __builtin_bit_cast(bf16x8, af), __builtin_bit_cast(bf16x8, bfr[fn]), acc[fm][fn],
                0, 0, 0);
          } else {
#pragma unroll
            for (int j = 0; j < 4; ++j)
              acc[fm][fn] = __builtin_amdgcn_mfma_f32_16x16x4f32(
                  __int_as_float(af[j]), __int_as_float(bfr[fn][j]), acc[fm][fn], 0, 0, 0);
          }
        }
      }
    }
  }
}

// acc[fm][fn] += A * B over one K step with the instruction's E8M0 block
// scales: sca[fm] the scale byte of this lane's tile row (wave row block
// fm) and K block q of the step, scb[fn] that of its tile column.  The
// scale a lane quarter q supplies covers the instruction's K elements
// 32 q + [0,32) whichever lanes hold them (measured on gfx950: with the
// operands in the layouts of f8f6f4_operand, where the step's K element k
// is the instruction's element k in either width, the products match
// block-scaled sums exactly; with a one-byte operand's lane quarter given
// its own 32 consecutive elements instead, they do not).  So each operand
// keeps its unscaled layout and any pair of widths takes E8M0 scales.
template <class C>
__device__ inline void mma_tile_mx(f32x4 (&acc)[C::FM][C::FN], const char* sa, const char* sb,
                                   const int (&sca)[C::FM], const int (&scb)[C::FN]) {
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int wm = w / C::WN, wn = w % C::WN;
  const int q = lane >> 4, r16 = lane & 15;
  i32x8 bf[C::FN];
#pragma unroll
  for (int fn = 0; fn < C::FN; ++fn) bf[fn] = f8f6f4_operand<C::FB>(sb, wn * C::TN + fn * 16 + r16, q);
#pragma unroll
  for (int fm = 0; fm < C::FM; ++fm) {
    const i32x8 af = f8f6f4_operand<C::FA>(sa, wm * C::TM + fm * 16 + r16, q);
#pragma unroll
    for (int fn = 0; fn < C::FN; ++fn)
      acc[fm][fn] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(af, bf[fn], acc[fm][fn], C::FA, C::FB, 0,
                                                                     sca[fm], 0, scb[fn]);
  }
}

// Bytes [off, off + 16) of a row outside the active groups: zeros, or the
// same bytes of the existing output.  (With kFillKeep nothing is written;
// the callers then have no such bytes to fill.)
__device__ __forceinline__ void fill16(const Params& p, long long off) {
  i32x4 v = {0, 0, 0, 0};
  if (p.fill == kFillCopy) v = *reinterpret_cast<const i32x4*>(reinterpret_cast<const char*>(p.existing) + off);
  *reinterpret_cast<i32x4*>(reinterpret_cast<char*>(p.out) + off) = v;
}

// Bytes of the rows before the active ones and after them that the fill
// writes (none when the existing output is the output itself).
__device__ __forceinline__ long long fill_rows(const Params& p, int rows) {
  return p.fill == kFillKeep ? 0 : (long long)rows;
}

template <class C>
__device__ inline void fill_item(const Params& p, long long begin, long long end) {
  for (long long off = begin + (long long)threadIdx.x * 16; off < end; off += (long long)C::T * 16) fill16(p, off);
}

// Bytes of one wave's epilogue staging slice: 16 rows of TN values of up to
// 4 bytes, each row padded by 16 bytes.  The slices of all waves fit in the
// operand stages.
template <class C>
constexpr int kStageSlice = 16 * (C::TN * 4 + 16);

template <class C>
__global__ __launch_bounds__(C::T) void gmm_kernel(Params p) {
  // operand stages, then (scaled problems) two buffers of one block's row
  // and column scales
  constexpr int SC_BYTES = C::SCALED ? 2 * (C::BM + C::BN) * 4 : 0;
  static_assert(C::T / 64 * kStageSlice<C> <= C::LDS, "epilogue staging fits the operand stages");
  __shared__ __attribute__((aligned(16))) char smem[C::LDS + SC_BYTES];
  __shared__ Plan pl;
  if (threadIdx.x == 0) pl.flags = 0;
  __syncthreads();
  build_plan<C::T>(p, pl, C::BM);
  report_flags(p, pl);

  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
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
  const int KT = K / C::BK;
  const int P = gridDim.x;
  const int slot = xcd_slot(blockIdx.x, P);

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
    const int h = find_group(pl, t);
    const int row0 = pl.row_start[h] + (t - pl.tile_start[h]) * C::BM;
    const int rows_left = pl.row_start[h + 1] - row0;
    const int rows = rows_left < C::BM ? rows_left : C::BM;
    const int n0 = j * C::BN;
    const int ncols = N - n0 < C::BN ? N - n0 : C::BN;

    const char* lhs = reinterpret_cast<const char*>(p.lhs) + C::lhs_bytes((long long)row0 * K);
    const __amdgpu_buffer_rsrc_t ar = make_rsrc(lhs, C::lhs_bytes((long long)rows * K));
    const char* rhs_h = reinterpret_cast<const char*>(p.rhs) + C::rhs_bytes((long long)h * N * K);
    __amdgpu_buffer_rsrc_t br;
    if constexpr (C::NN)
      br = make_rsrc(rhs_h, C::rhs_bytes((long long)K * N));
    else
      br = make_rsrc(rhs_h + C::rhs_bytes((long long)n0 * K), C::rhs_bytes((long long)ncols * K));

    f32x4 acc[C::FM][C::FN];
    f32x4 tot[C::SCALED ? C::FM : 1][C::SCALED ? C::FN : 1];
#pragma unroll
    for (int a = 0; a < C::FM; ++a)
#pragma unroll
      for (int b = 0; b < C::FN; ++b) acc[a][b] = f32x4{0.f, 0.f, 0.f, 0.f};
    if constexpr (C::SCALED) {
#pragma unroll
      for (int a = 0; a < C::FM; ++a)
#pragma unroll
        for (int b = 0; b < C::FN; ++b) tot[a][b] = f32x4{0.f, 0.f, 0.f, 0.f};
    }

    const C cfg{};
    Stage<C> st;
    load_tile(cfg, st, ar, br, 0, K, N, n0);
    store_tile(cfg, st, smem, smem + C::A_BYTES);

    // Block scales pass through LDS one block ahead, like the operands: in
    // the first step of block b thread i loads the row scale of tile row i
    // and the column scale of tile column i for block b+1 before the
    // multiply and writes them to buffer (b+1) & 1 after it; block b's fold
    // reads buffer b & 1.  (Loading each lane's 20 scales from memory at
    // the block's start and waiting for them at its end cost more than the
    // multiplies.)  Rows and columns outside the tile, and an absent scale,
    // count 1.
    const int kt_per_blk = C::SCALED ? p.blk / C::BK : 0;
    constexpr int SL = C::SCALED ? (C::BM + C::T - 1) / C::T : 1, SR = C::SCALED ? (C::BN + C::T - 1) / C::T : 1;
    float* const lsc = reinterpret_cast<float*>(smem + C::LDS);  // [2][BM]
    float* const rsc = lsc + 2 * C::BM;                          // [2][BN]
    float sl[SL], sr[SR];
    auto load_scales = [&](int b) __attribute__((always_inline)) {
#pragma unroll
      for (int i = 0; i < SL; ++i) {
        const int r = tid + i * C::T;
        sl[i] = (p.lhs_scale && r < rows) ? p.lhs_scale[(long long)(row0 + r) * p.nb + b] : 1.f;
      }
#pragma unroll
      for (int i = 0; i < SR; ++i) {
        const int c = tid + i * C::T;
        sr[i] = (p.rhs_scale && c < ncols) ? p.rhs_scale[((long long)h * p.nb + b) * N + n0 + c] : 1.f;
      }
    };
    auto store_scales = [&](int buf) __attribute__((always_inline)) {
#pragma unroll
      for (int i = 0; i < SL; ++i)
        if (tid + i * C::T < C::BM) lsc[buf * C::BM + tid + i * C::T] = sl[i];
#pragma unroll
      for (int i = 0; i < SR; ++i)
        if (tid + i * C::T < C::BN) rsc[buf * C::BN + tid + i * C::T] = sr[i];
    };
    if constexpr (C::SCALED) {
      load_scales(0);
      store_scales(0);
    }
    // E8M0 block scales for the instruction (MX): the bytes of this lane's
    // rows and columns for K block 4 kt + q, one K step ahead in registers.
    // Rows and columns outside the tile read 0 (their outputs are dropped);
    // an absent scale is 127 (1.0).
    constexpr int XA = C::MX ? C::FM : 1, XB = C::MX ? C::FN : 1;
    int sca[XA], scb[XB], nsca[XA], nscb[XB];
    const uint8_t* ls8 = reinterpret_cast<const uint8_t*>(p.lhs_scale);
    const uint8_t* rs8 = reinterpret_cast<const uint8_t*>(p.rhs_scale);
    const __amdgpu_buffer_rsrc_t lsr =
        C::MX && ls8 ? make_rsrc(ls8 + (long long)row0 * p.nb, (long long)rows * p.nb) : make_rsrc(p.lhs, 0);
    const __amdgpu_buffer_rsrc_t rsr =
        C::MX && rs8 ? make_rsrc(rs8 + (long long)h * p.nb * N + n0, (long long)(p.nb - 1) * N + ncols)
                     : make_rsrc(p.lhs, 0);
    auto load_mx = [&](int kt, int (&xa)[XA], int (&xb)[XB]) __attribute__((always_inline)) {
      const int b = kt * 4 + q;
#pragma unroll
      for (int fm = 0; fm < XA; ++fm)
        xa[fm] = p.lhs_scale ? (int)__builtin_amdgcn_raw_buffer_load_b8(
                                   lsr, (wm * C::TM + fm * 16 + r16) * p.nb + b, 0, 0)
                             : 127;
#pragma unroll
      for (int fn = 0; fn < XB; ++fn)
        xb[fn] = p.rhs_scale ? (int)__builtin_amdgcn_raw_buffer_load_b8(rsr, b * N + wn * C::TN + fn * 16 + r16, 0, 0)
                             : 127;
    };
    if constexpr (C::MX) load_mx(0, sca, scb);
    __syncthreads();

    for (int kt = 0; kt < KT; ++kt) {
      char* sa = smem + (kt & 1) * (C::A_BYTES + C::B_BYTES);
      char* sb = sa + C::A_BYTES;
      bool next_scales = false;
      if constexpr (C::SCALED) {
        next_scales = kt % kt_per_blk == 0 && kt / kt_per_blk + 1 < p.nb;
        if (next_scales) load_scales(kt / kt_per_blk + 1);
      }
      if (kt + 1 < KT) load_tile(cfg, st, ar, br, kt + 1, K, N, n0);
      if constexpr (C::MX) {
        if (kt + 1 < KT) load_mx(kt + 1, nsca, nscb);
        mma_tile_mx<C>(acc, sa, sb, sca, scb);
#pragma unroll
        for (int fm = 0; fm < XA; ++fm) sca[fm] = nsca[fm];
#pragma unroll
        for (int fn = 0; fn < XB; ++fn) scb[fn] = nscb[fn];
      } else {
        mma_tile<C>(acc, sa, sb);
      }
      if constexpr (C::SCALED) {
        if ((kt + 1) % kt_per_blk == 0) {
          const int bb = (kt / kt_per_blk) & 1;
          float rs[C::FN];
          f32x4 ls[C::FM];
#pragma unroll
          for (int fn = 0; fn < C::FN; ++fn) rs[fn] = rsc[bb * C::BN + wn * C::TN + fn * 16 + r16];
#pragma unroll
          for (int fm = 0; fm < C::FM; ++fm)
            ls[fm] = *reinterpret_cast<const f32x4*>(lsc + bb * C::BM + wm * C::TM + fm * 16 + 4 * q);
#pragma unroll
          for (int fm = 0; fm < C::FM; ++fm)
#pragma unroll
            for (int fn = 0; fn < C::FN; ++fn) {
#pragma unroll
              for (int i = 0; i < 4; ++i) tot[fm][fn][i] += acc_value<C>(acc[fm][fn][i]) * (rs[fn] * ls[fm][i]);
              acc[fm][fn] = f32x4{0.f, 0.f, 0.f, 0.f};
            }
        }
        if (next_scales) store_scales((kt / kt_per_blk + 1) & 1);
      }
      if (kt + 1 < KT) {
        char* na = smem + ((kt + 1) & 1) * (C::A_BYTES + C::B_BYTES);
        store_tile(cfg, st, na, na + C::A_BYTES);
      }
      __syncthreads();
    }

    // epilogue: bias, round, store.  Each 16-row block of the wave's tile
    // passes through the wave's staging slice (the operand stages are free
    // once every wave is past the K loop's last barrier), so that each store
    // writes a whole 16-byte chunk of an output row instead of one value.
    // Chunks outside the tile's valid rows and columns are skipped: N is a
    // multiple of 8 and the output 16-byte aligned, so a chunk is either
    // all inside or all outside.
    {
      const int es = out_es;
      const int pitch = C::TN * es + 16;  // staged row bytes; the extra 16 spread the rows over the banks
      char* const stg = smem + w * kStageSlice<C>;
      const int cpr = C::TN * es / 16;  // 16-byte chunks per staged row
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
        // lane (q, r16) holds rows 4 q + i of the block, column 16 fn + r16
#pragma unroll
        for (int fn = 0; fn < C::FN; ++fn)
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            float v;
            if constexpr (C::SCALED)
              v = tot[fm][fn][i];
            else
              v = acc_value<C>(acc[fm][fn][i]);
            v += bias[fn];
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
    // the next tile's first stage overwrites the staging slices
    __syncthreads();
  }
}

}  // namespace gmmk
