// gmm_launch.hpp -- host-side launch entry points of the gfx950 kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "gmm_params.hpp"

namespace gmmk {

enum class SizeClass { Small = 0, Big = 1 };

struct KernelChoice {
  Op op;
  bool nn;      // rhs [Ga,K,N]
  bool b_fp8;   // fp8 rhs widened to bf16 operands
  int fmt;      // narrow formats: fmt & 7 lhs, fmt >> 3 rhs.  FP8 products: 0 e4m3fn, 1 e5m2,
                // 4 fp4 e2m1; I8 products: 0 int8, 3 int4, 4 uint4; widened bf16 weights
                // (b_fp8): rhs 0 e4m3fn, 1 e5m2, 2 int8, 3 int4, 4 uint4, 5 fp4 e2m1
  bool scaled;  // f32 rhs_scale and/or lhs_scale present (folded per block)
  bool mx;      // E8M0 scales of 32-element blocks, applied by the scaled instruction
  SizeClass size;
  int grid_cap;  // > 0: at most this many workgroups (a test hook)
};

// K elements of one K tile for an operand type (the K granularity).
inline int k_tile(Op op) { return op == Op::F32 ? 32 : (op == Op::BF16 ? 64 : 128); }

// int8 x int8 sums are exact int32 as long as a run of int32 accumulation
// (K, or the scale block) has at most 2^17 products of at most 2^14.
constexpr long long kMaxInt8Run = 1LL << 17;

// m-tile height the kernel uses for this choice.
int tile_m(const KernelChoice& c);

// Queue the gmm kernel.  Returns hipSuccess or the launch error.
hipError_t launch_gmm(const Params& p, const KernelChoice& c, int cu_count, hipStream_t stream);

// The block-scaled fp8 x fp8 kernel (gmm_w8a8.hip) takes scale blocks of
// one K step of 128 with both scales given, at least three K steps (its
// cross-tile load pipeline runs three steps ahead) and N a multiple of 4 (a
// lane stores four consecutive columns).
inline bool w8a8_fits(const Params& p) {
  return p.lhs_scale && p.rhs_scale && p.blk == 128 && p.K >= 3 * 128 && p.K % 128 == 0 && p.N % 4 == 0;
}

// Queue it for lhs format fa and rhs format fb (0 e4m3fn, 1 e5m2).
hipError_t launch_w8a8(const Params& p, int fa, int fb, int cu_count, int grid_cap, hipStream_t stream);

// The weight-streaming kernel (gmm_stream.hip) takes bf16 x narrow-weight
// NT problems with few rows per group: K a multiple of 128 with at least S
// stages of 128 per tile (S: the depth of its LDS ring), no lhs scale, and
// rhs scale blocks of exactly one stage (or no rhs scale).
bool stream_fits(const Params& p);

// Queue it for weight format fb (0 e4m3fn, 1 e5m2, 2 int8, 3 int4, 4 uint4,
// 5 fp4 e2m1).
hipError_t launch_stream(const Params& p, int fb, int cu_count, int grid_cap, hipStream_t stream);

// Queue the transposed grouped matmul (out [Ga,K,N]); grid_cap > 0 limits
// the workgroups.
hipError_t launch_tgmm(const Params& p, int cu_count, int grid_cap, hipStream_t stream);

// Activation quantiser arguments: x bf16 [M,K], q e4m3fn [M,K], scale f32
// [M,K/128], blocks = M * K / 128 (K % 128 == 0).
struct QuantParams {
  const uint16_t* x;
  uint8_t* q;
  float* scale;
  long long blocks;
};

// Queue the activation quantiser (gmm_quant.hip).
hipError_t launch_quant_fp8(const QuantParams& p, int cu_count, hipStream_t stream);

// Block-scale widening arguments: src [n] of kScaleBf16 / kScaleF32 /
// kScaleE8m0 elements, dst [n] f32.
enum ScaleDtype : int32_t { kScaleBf16 = 0, kScaleF32 = 1, kScaleE8m0 = 2 };
struct WidenParams {
  const void* src;
  float* dst;
  long long n;
  int32_t dtype;
};

// Queue the block-scale widening (gmm_quant.hip).
hipError_t launch_widen_scales(const WidenParams& p, int cu_count, hipStream_t stream);

// Device scratch for callers that cannot allocate (gmm_tgmm_run_noalloc):
// a file-scope array in gmm_kernels.hip, one copy per device, holding the
// transposed product's work-queue counters.
constexpr int kStaticScratchBytes = 256;
static_assert(kQueueWords * 4 <= kStaticScratchBytes && kQueueWords <= 64, "work-queue counters fit the scratch");

// The device address of the current device's scratch (hipGetSymbolAddress).
hipError_t static_scratch_address(void** ptr);

// Queue a one-workgroup kernel that writes n zero int32 at p (n <= 64).
hipError_t launch_clear_ints(int32_t* p, int n, hipStream_t stream);

// Queue the worklist export kernel (one workgroup).
hipError_t launch_worklist(const Params& p, int tm, int32_t* tiles, long long capacity,
                           int32_t* count, hipStream_t stream);

}  // namespace gmmk
