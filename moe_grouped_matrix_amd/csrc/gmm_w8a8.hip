// gmm_w8a8.hip -- instantiations and launcher of the block-scaled fp8 x fp8
// kernel (gmm_w8a8.hpp).  A translation unit of its own because it is built
// with the MFMA results in ordinary VGPRs (-amdgpu-mfma-vgpr-form): the fold
// reads every result with VALU instructions, and results left in
// accumulation registers cost one copy instruction per value.
#include "gmm_w8a8.hpp"
#include "gmm_launch.hpp"

namespace gmmk {

namespace {

// One workgroup per CU (the ring takes most of the LDS), at most one per
// output tile.
template <class C>
hipError_t launch(const Params& p, int cu_count, int cap, hipStream_t stream) {
  const long long n_tiles = (p.N + C::BN - 1) / C::BN;
  const long long m_tiles = (p.M + C::BM - 1) / C::BM + p.Ga;
  long long grid = cu_count;
  if (grid > m_tiles * n_tiles && m_tiles * n_tiles >= 8) grid = m_tiles * n_tiles;
  if (grid >= 8) grid -= grid % 8;
  if (grid < 1) grid = 1;
  if (cap > 0 && grid > cap) grid = cap;
  hipLaunchKernelGGL(gmm_w8a8_kernel<C>, dim3((unsigned)grid), dim3(C::T), 0, stream, p);
  return hipGetLastError();
}

template <int FA, int FB>
hipError_t launch_out(const Params& p, int cu, int cap, hipStream_t st) {
  if (p.out_f32) return launch<W8Cfg<FA, FB, true>>(p, cu, cap, st);
  return launch<W8Cfg<FA, FB, false>>(p, cu, cap, st);
}

}  // namespace

hipError_t launch_w8a8(const Params& p, int fa, int fb, int cu, int cap, hipStream_t st) {
  if (!w8a8_fits(p) || fa < 0 || fa > 1 || fb < 0 || fb > 1) return hipErrorInvalidValue;
  if (fa == 0) return fb == 0 ? launch_out<0, 0>(p, cu, cap, st) : launch_out<0, 1>(p, cu, cap, st);
  return fb == 0 ? launch_out<1, 0>(p, cu, cap, st) : launch_out<1, 1>(p, cu, cap, st);
}

}  // namespace gmmk
