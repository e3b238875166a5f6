// gmm_stream.hip -- instantiations and launcher of the weight-streaming
// kernel (gmm_stream.hpp).  A translation unit of its own because it is
// built with the MFMA results in ordinary VGPRs (-amdgpu-mfma-vgpr-form):
// the scale fold reads every result with VALU instructions, and results left
// in accumulation registers cost one copy instruction per value (measured
// on the decode call: 31.4 against 32.5 us).
#include "gmm_stream.hpp"
#include "gmm_launch.hpp"

namespace gmmk {

namespace {

// One workgroup per CU (LDS-bound), even when there are fewer tiles:
// workgroups without a tile still take their share of the rows outside the
// active groups, which can be most of the output (an expert shard of a
// decode batch).
template <class C>
hipError_t launch(const Params& p, int cu_count, int cap, hipStream_t stream) {
  long long grid = cu_count;
  if (grid >= 8) grid -= grid % 8;
  if (grid < 1) grid = 1;
  if (cap > 0 && grid > cap) grid = cap;
  hipLaunchKernelGGL(gmm_stream_kernel<C>, dim3((unsigned)grid), dim3(C::T), 0, stream, p);
  return hipGetLastError();
}

template <int FB>
hipError_t launch_out(const Params& p, int cu, int cap, hipStream_t st) {
  if (p.out_f32) return launch<StreamCfg<true, FB>>(p, cu, cap, st);
  return launch<StreamCfg<false, FB>>(p, cu, cap, st);
}

}  // namespace

bool stream_fits(const Params& p) {
  return p.K % 128 == 0 && p.K >= StreamCfg<false>::S * StreamCfg<false>::BKS && p.lhs_scale == nullptr &&
         (p.rhs_scale == nullptr || p.blk == StreamCfg<false>::BKS);
}

hipError_t launch_stream(const Params& p, int fb, int cu, int cap, hipStream_t st) {
  if (!stream_fits(p)) return hipErrorInvalidValue;
  switch (fb) {
    case 0: return launch_out<0>(p, cu, cap, st);
    case 1: return launch_out<1>(p, cu, cap, st);
    case 2: return launch_out<2>(p, cu, cap, st);
    case 3: return launch_out<3>(p, cu, cap, st);
    case 4: return launch_out<4>(p, cu, cap, st);
    case 5: return launch_out<5>(p, cu, cap, st);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace gmmk
