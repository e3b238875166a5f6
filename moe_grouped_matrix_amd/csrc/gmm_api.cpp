// gmm_api.cpp -- the C ABI of libgmm.so (declared in include/gmm.h).
//
// Argument checks mirror the shape and dtype validation of the Megablox gmm
// (tpu-inference 0.13.2 wheel diff page, megablox/gmm.py, _validate_args and
// the checks at the top of gmm()); everything they reject returns
// GMM_E_INVALID before any work is queued.  The kernels themselves live in
// gmm_kernels.hip.
#include <hip/hip_runtime.h>

#include <cstdio>
#include <cstring>
#include <map>
#include <mutex>
#include <string>

#include "gmm.h"
#include "gmm_launch.hpp"

constexpr size_t kDeviceBlock = 16;  // the data-error flag word
static_assert(gmmk::kFlagNegative == GMM_FLAG_NEGATIVE_SIZE && gmmk::kFlagExceed == GMM_FLAG_SIZES_EXCEED_M &&
                  gmmk::kFlagBadOffset == GMM_FLAG_BAD_OFFSET && gmmk::kFlagSchedule == GMM_FLAG_SCHEDULE_TIMEOUT,
              "the kernels' flag bits are the header's");
constexpr size_t kQueueBlock = gmmk::kQueueWords * sizeof(int32_t);

struct gmm_handle {
  int device = 0;
  int cu_count = 0;
  uint32_t* flags = nullptr;  // device word of data-error flags (kDeviceBlock bytes)
  // the transposed product's work-queue counters (kQueueWords int32, zero
  // between calls), one block per stream: calls on one stream run in order,
  // so each call finds its stream's counters reset by the previous one;
  // calls on different streams never share counters
  std::map<void*, int32_t*> queues;
  int tile_policy = 0;        // 0 auto, 1 small tiles, 2 big tiles
  int grid_limit = 0;         // > 0: at most this many workgroups per launch
  void* scratch = nullptr;    // device address of the device's static scratch
  std::string err;
};

// Device addresses of the static scratch (gmmk::static_scratch_address), one
// per device, looked up by the first gmm_create on that device.
static std::mutex g_scratch_mu;
static std::map<int, void*> g_scratch;

namespace {

struct DeviceGuard {
  int prev = -1;
  explicit DeviceGuard(int dev) {
    if (hipGetDevice(&prev) != hipSuccess) prev = -1;
    if (prev != dev) (void)hipSetDevice(dev);
  }
  ~DeviceGuard() {
    int cur = -1;
    if (prev >= 0 && hipGetDevice(&cur) == hipSuccess && cur != prev) (void)hipSetDevice(prev);
  }
};

gmm_status fail(gmm_handle* h, gmm_status st, const std::string& msg) {
  if (h) h->err = msg;
  return st;
}

std::string shape_str(const gmm_tensor* t) {
  std::string s = "(";
  for (int i = 0; i < t->ndim && i < 4; ++i) {
    if (i) s += ",";
    s += std::to_string(t->shape[i]);
  }
  return s + ")";
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

int elem_size(int dtype) {
  switch (dtype) {
    case GMM_F32: return 4;
    case GMM_BF16: return 2;
    case GMM_F8E4M3FN: return 1;
    case GMM_F8E5M2: return 1;
    case GMM_E8M0: return 1;
    case GMM_I8: return 1;
    case GMM_I32: return 4;
    default: return 0;
  }
}

long long numel(const gmm_tensor* t) {
  long long n = 1;
  for (int i = 0; i < t->ndim; ++i) n *= t->shape[i];
  return n;
}

bool four_bit(int dtype) { return dtype == GMM_I4 || dtype == GMM_U4 || dtype == GMM_F4E2M1; }

// bytes of a tensor's data (four-bit types: two elements to a byte)
long long tensor_bytes(const gmm_tensor* t) {
  return four_bit(t->dtype) ? (numel(t) + 1) / 2 : numel(t) * elem_size(t->dtype);
}

bool overlaps(const gmm_tensor* a, const gmm_tensor* b) {
  if (!a || !b || !a->data || !b->data) return false;
  const char* a0 = static_cast<const char*>(a->data);
  const char* b0 = static_cast<const char*>(b->data);
  const char* a1 = a0 + tensor_bytes(a);
  const char* b1 = b0 + tensor_bytes(b);
  return a0 < b1 && b0 < a1;
}

}  // namespace

extern "C" {

gmm_status gmm_create(gmm_handle** out, int device) {
  if (!out) return GMM_E_INVALID;
  *out = nullptr;
  int n = 0;
  if (hipGetDeviceCount(&n) != hipSuccess || device < 0 || device >= n) return GMM_E_HIP;
  hipDeviceProp_t prop;
  if (hipGetDeviceProperties(&prop, device) != hipSuccess) return GMM_E_HIP;
  if (std::strncmp(prop.gcnArchName, "gfx950", 6) != 0) return GMM_E_UNSUPPORTED;
  gmm_handle* h = new gmm_handle();
  h->device = device;
  h->cu_count = prop.multiProcessorCount;
  DeviceGuard g(device);
  if (hipMalloc(&h->flags, kDeviceBlock) != hipSuccess) {
    delete h;
    return GMM_E_HIP;
  }
  if (hipMemset(h->flags, 0, kDeviceBlock) != hipSuccess) {
    (void)hipFree(h->flags);
    delete h;
    return GMM_E_HIP;
  }
  {
    std::lock_guard<std::mutex> lk(g_scratch_mu);
    auto it = g_scratch.find(device);
    if (it == g_scratch.end()) {
      void* ptr = nullptr;
      if (gmmk::static_scratch_address(&ptr) != hipSuccess || !ptr) {
        (void)hipFree(h->flags);
        delete h;
        return GMM_E_HIP;
      }
      it = g_scratch.emplace(device, ptr).first;
    }
    h->scratch = it->second;
  }
  *out = h;
  return GMM_OK;
}

gmm_status gmm_destroy(gmm_handle* h) {
  if (!h) return GMM_OK;
  {
    DeviceGuard g(h->device);
    // work queued on the handle's streams must not outlive the handle
    if (h->flags) (void)hipFree(h->flags);
    for (auto& kv : h->queues) (void)hipFree(kv.second);
  }
  delete h;
  return GMM_OK;
}

const char* gmm_last_error(const gmm_handle* h) { return h ? h->err.c_str() : "null handle"; }

// Test hook: 0 chooses tiles from the problem shape, 1 forces the small
// (decode) tiles, 2 the big tiles.  Results differ only in fp32 summation
// order.
gmm_status gmm_set_tile_policy(gmm_handle* h, int policy) {
  if (!h || policy < 0 || policy > 2) return GMM_E_INVALID;
  h->tile_policy = policy;
  return GMM_OK;
}

// Test hook: at most `limit` workgroups per launch of the gmm and tgmm
// kernels (0 = as many as the kernel's own choice).  Every kernel walks its
// tiles with a grid stride, so the result is unchanged; with few workgroups
// each one runs many tiles back to back.
gmm_status gmm_set_grid_limit(gmm_handle* h, int limit) {
  if (!h || limit < 0) return GMM_E_INVALID;
  h->grid_limit = limit;
  return GMM_OK;
}

}  // extern "C"

namespace {

gmm_status run_gmm(gmm_handle* h, const gmm_tensor* lhs, const gmm_tensor* rhs, const gmm_tensor* group_sizes,
                   const gmm_tensor* rhs_scale, const gmm_tensor* rhs_bias, const gmm_tensor* lhs_scale,
                   const int32_t* group_offset, int transpose_rhs, const gmm_tensor* existing_out,
                   const gmm_tensor* out, void* stream) {
  if (!h) return GMM_E_INVALID;
  h->err.clear();
  if (!lhs || !rhs || !group_sizes || !out) return fail(h, GMM_E_INVALID, "lhs, rhs, group_sizes and out are required");
  if (lhs->ndim != 2) return fail(h, GMM_E_INVALID, "expected a 2-tensor for lhs, got ndim=" + std::to_string(lhs->ndim));
  if (rhs->ndim != 3) return fail(h, GMM_E_INVALID, "expected a 3-tensor for rhs, got ndim=" + std::to_string(rhs->ndim));
  if (group_sizes->ndim != 1 || group_sizes->dtype != GMM_I32)
    return fail(h, GMM_E_INVALID, "expected a 1-d int32 group_sizes");
  if (out->ndim != 2) return fail(h, GMM_E_INVALID, "expected a 2-tensor for out");

  const long long M = lhs->shape[0], K = lhs->shape[1];
  const long long Ga = rhs->shape[0];
  const long long N = transpose_rhs ? rhs->shape[2] : rhs->shape[1];
  const long long Kr = transpose_rhs ? rhs->shape[1] : rhs->shape[2];
  const long long G = group_sizes->shape[0];
  if (Kr != K)
    return fail(h, GMM_E_INVALID, "lhs and rhs disagree on the contraction size: lhs " + shape_str(lhs) +
                                      ", rhs " + shape_str(rhs));
  if (M < 0 || K <= 0 || N <= 0 || Ga < 0) return fail(h, GMM_E_INVALID, "negative or zero extent");
  if (out->shape[0] != M || out->shape[1] != N)
    return fail(h, GMM_E_INVALID, "out must be [M,N] = [" + std::to_string(M) + "," + std::to_string(N) + "], got " + shape_str(out));
  if (out->dtype != GMM_F32 && out->dtype != GMM_BF16) return fail(h, GMM_E_INVALID, "out must be f32 or bf16");
  if (G < 1) return fail(h, GMM_E_INVALID, "group_sizes must hold at least one group");
  if (Ga > G) return fail(h, GMM_E_INVALID, "rhs holds more groups than group_sizes");

  gmmk::KernelChoice kc{};
  const int ld = lhs->dtype, rd = rhs->dtype;
  // operand format codes of the int8 products (0 int8, 3 int4, 4 uint4) and
  // of the f8f6f4 products (0 e4m3fn, 1 e5m2, 4 fp4 e2m1); -1 for another type
  auto int_code = [](int d) { return d == GMM_I8 ? 0 : d == GMM_I4 ? 3 : d == GMM_U4 ? 4 : -1; };
  auto f8_code = [](int d) { return d == GMM_F8E4M3FN ? 0 : d == GMM_F8E5M2 ? 1 : d == GMM_F4E2M1 ? 4 : -1; };
  if (ld == GMM_F32 && rd == GMM_F32) {
    kc.op = gmmk::Op::F32;
  } else if (ld == GMM_BF16 && rd == GMM_BF16) {
    kc.op = gmmk::Op::BF16;
  } else if (ld == GMM_BF16 && (rd == GMM_F8E4M3FN || rd == GMM_F8E5M2 || rd == GMM_I8)) {
    kc.op = gmmk::Op::BF16;
    kc.b_fp8 = true;
    kc.fmt = (rd == GMM_F8E5M2 ? 1 : (rd == GMM_I8 ? 2 : 0)) << 3;
  } else if (ld == GMM_BF16 && four_bit(rd)) {
    kc.op = gmmk::Op::BF16;
    kc.b_fp8 = true;
    kc.fmt = (rd == GMM_I4 ? 3 : (rd == GMM_U4 ? 4 : 5)) << 3;
  } else if (int_code(ld) >= 0 && int_code(rd) >= 0) {
    kc.op = gmmk::Op::I8;
    kc.fmt = int_code(ld) | int_code(rd) << 3;
  } else if (f8_code(ld) >= 0 && f8_code(rd) >= 0) {
    kc.op = gmmk::Op::FP8;
    kc.fmt = f8_code(ld) | f8_code(rd) << 3;
  } else {
    const bool known_l = elem_size(ld) > 0 || four_bit(ld), known_r = elem_size(rd) > 0 || four_bit(rd);
    if (!known_l || !known_r || ld == GMM_I32 || rd == GMM_I32 || ld == GMM_E8M0 || rd == GMM_E8M0)
      return fail(h, GMM_E_INVALID, "unsupported lhs / rhs dtype");
    return fail(h, GMM_E_UNSUPPORTED, "unsupported (lhs, rhs) dtype pair");
  }
  kc.nn = transpose_rhs != 0;
  if (kc.nn && (kc.b_fp8 || kc.op == gmmk::Op::FP8))
    return fail(h, GMM_E_UNSUPPORTED, "fp8, int8 and four-bit weights are read in the [G,N,K] layout only");
  if (kc.nn && kc.op == gmmk::Op::I8) return fail(h, GMM_E_UNSUPPORTED, "int8 weights are read in the [G,N,K] layout only");

  long long nb = 1;
  // block scales: f32 (folded per block), or E8M0 bytes of 32-element blocks
  // for the scaled matrix instruction -- then every given scale is E8M0
  const bool mx = (rhs_scale && rhs_scale->dtype == GMM_E8M0) || (lhs_scale && lhs_scale->dtype == GMM_E8M0);
  const int scale_dtype = mx ? GMM_E8M0 : GMM_F32;
  if (rhs_scale) {
    if (rhs_scale->ndim != 4 || rhs_scale->dtype != scale_dtype)
      return fail(h, GMM_E_INVALID, "expected an f32 (or, with E8M0 scales on both sides, E8M0) 4-tensor for rhs_scale");
    nb = rhs_scale->shape[1];
    if (rhs_scale->shape[0] != Ga || rhs_scale->shape[2] != 1 || rhs_scale->shape[3] != N || nb < 1)
      return fail(h, GMM_E_INVALID, "expected rhs_scale of shape (Ga, nb, 1, N), got " + shape_str(rhs_scale));
  }
  if (lhs_scale) {
    if (lhs_scale->ndim != 2 || lhs_scale->dtype != scale_dtype || lhs_scale->shape[0] != M || lhs_scale->shape[1] < 1)
      return fail(h, GMM_E_INVALID, "expected lhs_scale of shape (M, nb), of rhs_scale's dtype (f32 or E8M0)");
    if (rhs_scale && lhs_scale->shape[1] != nb)
      return fail(h, GMM_E_INVALID, "lhs_scale and rhs_scale disagree on the number of blocks");
    nb = lhs_scale->shape[1];
  }
  if (K % nb) return fail(h, GMM_E_INVALID, "K must be a multiple of the number of quantisation blocks");
  if (rhs_bias) {
    if (rhs_bias->ndim != 3 || rhs_bias->shape[0] != Ga || rhs_bias->shape[1] != 1 || rhs_bias->shape[2] != N)
      return fail(h, GMM_E_INVALID, "expected rhs_bias of shape (Ga, 1, N), got " + shape_str(rhs_bias));
    if (rhs_bias->dtype != GMM_F32 && rhs_bias->dtype != GMM_BF16)
      return fail(h, GMM_E_INVALID, "rhs_bias must be f32 or bf16");
  }
  kc.scaled = !mx && (rhs_scale != nullptr || lhs_scale != nullptr);
  kc.mx = mx;
  if (mx) {
    if (kc.op != gmmk::Op::FP8)
      return fail(h, GMM_E_UNSUPPORTED, "E8M0 block scales need e4m3fn, e5m2 or fp4 e2m1 operands on both sides");
    if (K != 32 * nb) return fail(h, GMM_E_UNSUPPORTED, "E8M0 block scales cover blocks of 32 K elements (nb = K/32)");
  }

  // Limits of the kernels (valid problems outside them are unsupported).
  const int kt = gmmk::k_tile(kc.op);
  const long long blk = K / nb;
  if (G > gmmk::kMaxGroups) return fail(h, GMM_E_UNSUPPORTED, "more than 1024 groups");
  if (M >= (1LL << 31) || N >= (1LL << 31) || K >= (1LL << 31))
    return fail(h, GMM_E_UNSUPPORTED, "extent beyond 2^31");
  if (N % 8) return fail(h, GMM_E_UNSUPPORTED, "N must be a multiple of 8");
  if (K % kt) return fail(h, GMM_E_UNSUPPORTED, "K must be a multiple of " + std::to_string(kt) + " for this dtype");
  if (kc.scaled && blk % kt)
    return fail(h, GMM_E_UNSUPPORTED, "the quantisation block K/nb must be a multiple of " + std::to_string(kt));
  if (kc.op == gmmk::Op::I8 && (kc.scaled ? blk : K) > gmmk::kMaxInt8Run)
    return fail(h, GMM_E_UNSUPPORTED, "int8 x int8: at most 2^17 products per int32 sum (K, or K/nb with scales)");
  const long long wbytes = four_bit(rd) ? K * N / 2 : K * N * elem_size(rd);
  if (wbytes >= 0x7FFFFFF0LL || 256LL * K * elem_size(ld) >= 0x7FFFFFF0LL)
    return fail(h, GMM_E_UNSUPPORTED, "one group's weight (or a 256-row lhs tile) exceeds 2 GiB");
  // the epilogues address a 256-row output tile with 32-bit byte offsets
  if (256LL * N * elem_size(out->dtype) >= 0x7FFFFFF0LL)
    return fail(h, GMM_E_UNSUPPORTED, "a 256-row output tile exceeds 2 GiB");

  const gmm_tensor* ins[] = {lhs, rhs, group_sizes, rhs_scale, rhs_bias, lhs_scale};
  for (const gmm_tensor* t : ins) {
    if (!t) continue;
    if (numel(t) > 0 && !t->data) return fail(h, GMM_E_INVALID, "null data pointer");
    if (!aligned16(t->data)) return fail(h, GMM_E_INVALID, "tensor data must be 16-byte aligned");
    if (overlaps(t, out)) return fail(h, GMM_E_INVALID, "out overlaps an input");
  }
  if (M > 0 && !out->data) return fail(h, GMM_E_INVALID, "null out pointer");
  if (!aligned16(out->data) || !aligned16(group_offset))
    return fail(h, GMM_E_INVALID, "out and group_offset must be 16-byte aligned");
  int32_t fill = gmmk::kFillZero;
  if (existing_out) {
    if (existing_out->ndim != 2 || existing_out->shape[0] != M || existing_out->shape[1] != N)
      return fail(h, GMM_E_INVALID, "existing_out must be [M,N] like out, got " + shape_str(existing_out));
    if (existing_out->dtype != out->dtype)
      return fail(h, GMM_E_INVALID, "existing_out dtype must match the output dtype");
    if (M > 0 && !existing_out->data) return fail(h, GMM_E_INVALID, "null existing_out pointer");
    if (!aligned16(existing_out->data)) return fail(h, GMM_E_INVALID, "existing_out must be 16-byte aligned");
    if (existing_out->data == out->data)
      fill = gmmk::kFillKeep;
    else if (overlaps(existing_out, out))
      return fail(h, GMM_E_INVALID, "existing_out must be out itself or not overlap it");
    else
      fill = gmmk::kFillCopy;
  }
  if (M == 0) return GMM_OK;

  kc.grid_cap = h->grid_limit;
  if (h->tile_policy == 1)
    kc.size = gmmk::SizeClass::Small;
  else if (h->tile_policy == 2)
    kc.size = gmmk::SizeClass::Big;
  else
    kc.size = (M >= 8192 && M >= 512 * (Ga > 0 ? Ga : 1)) ? gmmk::SizeClass::Big : gmmk::SizeClass::Small;

  gmmk::Params p{};
  p.lhs = lhs->data;
  p.rhs = rhs->data;
  p.group_sizes = static_cast<const int32_t*>(group_sizes->data);
  p.group_offset = group_offset;
  p.rhs_scale = rhs_scale ? static_cast<const float*>(rhs_scale->data) : nullptr;
  p.rhs_bias = rhs_bias ? rhs_bias->data : nullptr;
  p.lhs_scale = lhs_scale ? static_cast<const float*>(lhs_scale->data) : nullptr;
  p.out = const_cast<void*>(out->data);
  p.existing = existing_out ? existing_out->data : nullptr;
  p.fill = fill;
  p.flags = h->flags;
  p.M = (int32_t)M;
  p.K = (int32_t)K;
  p.N = (int32_t)N;
  p.G = (int32_t)G;
  p.Ga = (int32_t)Ga;
  p.nb = (int32_t)nb;
  p.blk = (int32_t)blk;
  p.bias_f32 = rhs_bias && rhs_bias->dtype == GMM_F32;
  p.out_f32 = out->dtype == GMM_F32;

  DeviceGuard g(h->device);
  hipError_t e = gmmk::launch_gmm(p, kc, h->cu_count, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return fail(h, GMM_E_HIP, std::string("kernel launch failed: ") + hipGetErrorString(e));
  return GMM_OK;
}

}  // namespace

extern "C" {

gmm_status gmm_run(gmm_handle* h, const gmm_tensor* lhs, const gmm_tensor* rhs,
                   const gmm_tensor* group_sizes, const gmm_tensor* rhs_scale,
                   const gmm_tensor* rhs_bias, const gmm_tensor* lhs_scale,
                   const int32_t* group_offset, int transpose_rhs, const gmm_tensor* out,
                   void* stream) {
  return run_gmm(h, lhs, rhs, group_sizes, rhs_scale, rhs_bias, lhs_scale, group_offset, transpose_rhs, nullptr,
                 out, stream);
}

gmm_status gmm_run_existing_out(gmm_handle* h, const gmm_tensor* lhs, const gmm_tensor* rhs,
                                const gmm_tensor* group_sizes, const gmm_tensor* rhs_scale,
                                const gmm_tensor* rhs_bias, const gmm_tensor* lhs_scale,
                                const int32_t* group_offset, int transpose_rhs,
                                const gmm_tensor* existing_out, const gmm_tensor* out, void* stream) {
  if (!h) return GMM_E_INVALID;
  h->err.clear();
  if (!existing_out) return fail(h, GMM_E_INVALID, "existing_out is required (gmm_run writes zeros instead)");
  return run_gmm(h, lhs, rhs, group_sizes, rhs_scale, rhs_bias, lhs_scale, group_offset, transpose_rhs,
                 existing_out, out, stream);
}

gmm_status gmm_widen_scales_run(gmm_handle* h, const gmm_tensor* src, const gmm_tensor* dst, void* stream) {
  if (!h) return GMM_E_INVALID;
  h->err.clear();
  if (!src || !dst) return fail(h, GMM_E_INVALID, "src and dst are required");
  int32_t dt;
  switch (src->dtype) {
    case GMM_BF16: dt = gmmk::kScaleBf16; break;
    case GMM_F32: dt = gmmk::kScaleF32; break;
    case GMM_E8M0: dt = gmmk::kScaleE8m0; break;
    default: return fail(h, GMM_E_INVALID, "src must be bf16, f32 or e8m0");
  }
  if (dst->dtype != GMM_F32) return fail(h, GMM_E_INVALID, "dst must be f32");
  if (src->ndim < 0 || src->ndim > 4 || dst->ndim < 0 || dst->ndim > 4)
    return fail(h, GMM_E_INVALID, "tensors of rank 0 to 4");
  const long long n = numel(src);
  if (n < 0 || numel(dst) != n) return fail(h, GMM_E_INVALID, "dst must hold as many elements as src");
  if (n > 0 && (!src->data || !dst->data)) return fail(h, GMM_E_INVALID, "null data pointer");
  if (!aligned16(src->data) || !aligned16(dst->data)) return fail(h, GMM_E_INVALID, "tensor data must be 16-byte aligned");
  if (overlaps(src, dst)) return fail(h, GMM_E_INVALID, "src and dst must not overlap");
  if (n == 0) return GMM_OK;
  gmmk::WidenParams p{};
  p.src = src->data;
  p.dst = static_cast<float*>(const_cast<void*>(dst->data));
  p.n = n;
  p.dtype = dt;
  DeviceGuard g(h->device);
  hipError_t e = gmmk::launch_widen_scales(p, h->cu_count, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return fail(h, GMM_E_HIP, std::string("kernel launch failed: ") + hipGetErrorString(e));
  return GMM_OK;
}

gmm_status gmm_quant_fp8_run(gmm_handle* h, const gmm_tensor* x, const gmm_tensor* q, const gmm_tensor* scale,
                             void* stream) {
  if (!h) return GMM_E_INVALID;
  h->err.clear();
  if (!x || !q || !scale) return fail(h, GMM_E_INVALID, "x, q and scale are required");
  if (x->ndim != 2 || x->dtype != GMM_BF16) return fail(h, GMM_E_INVALID, "x must be a bf16 2-tensor");
  const long long M = x->shape[0], K = x->shape[1];
  if (M < 0 || K <= 0) return fail(h, GMM_E_INVALID, "negative or zero extent");
  if (K % 128) return fail(h, GMM_E_INVALID, "K must be a multiple of the 128-element block");
  if (q->ndim != 2 || q->dtype != GMM_F8E4M3FN || q->shape[0] != M || q->shape[1] != K)
    return fail(h, GMM_E_INVALID, "q must be e4m3fn [M,K] like x, got " + shape_str(q));
  if (scale->ndim != 2 || scale->dtype != GMM_F32 || scale->shape[0] != M || scale->shape[1] != K / 128)
    return fail(h, GMM_E_INVALID, "scale must be f32 [M,K/128], got " + shape_str(scale));
  const gmm_tensor* ts[] = {x, q, scale};
  for (const gmm_tensor* t : ts) {
    if (M > 0 && !t->data) return fail(h, GMM_E_INVALID, "null data pointer");
    if (!aligned16(t->data)) return fail(h, GMM_E_INVALID, "tensor data must be 16-byte aligned");
  }
  if (overlaps(x, q) || overlaps(x, scale) || overlaps(q, scale))
    return fail(h, GMM_E_INVALID, "x, q and scale must not overlap");
  if (M == 0) return GMM_OK;
  gmmk::QuantParams p{};
  p.x = static_cast<const uint16_t*>(x->data);
  p.q = static_cast<uint8_t*>(const_cast<void*>(q->data));
  p.scale = static_cast<float*>(const_cast<void*>(scale->data));
  p.blocks = M * (K / 128);
  DeviceGuard g(h->device);
  hipError_t e = gmmk::launch_quant_fp8(p, h->cu_count, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return fail(h, GMM_E_HIP, std::string("kernel launch failed: ") + hipGetErrorString(e));
  return GMM_OK;
}

// The transposed product: validation, then the launch with the work-queue
// counters of the handle's block for this stream, or (no_alloc) of the
// device's static scratch, cleared first.
static gmm_status run_tgmm(gmm_handle* h, const gmm_tensor* lhs, const gmm_tensor* rhs,
                           const gmm_tensor* group_sizes, const int32_t* group_offset, const gmm_tensor* out,
                           void* stream, bool no_alloc) {
  if (!h) return GMM_E_INVALID;
  h->err.clear();
  if (!lhs || !rhs || !group_sizes || !out) return fail(h, GMM_E_INVALID, "lhs, rhs, group_sizes and out are required");
  if (lhs->ndim != 2 || rhs->ndim != 2) return fail(h, GMM_E_INVALID, "expected 2-tensors for lhs and rhs");
  if (group_sizes->ndim != 1 || group_sizes->dtype != GMM_I32)
    return fail(h, GMM_E_INVALID, "expected a 1-d int32 group_sizes");
  if (out->ndim != 3) return fail(h, GMM_E_INVALID, "expected a 3-tensor [Ga,K,N] for out");
  const long long M = lhs->shape[0], K = lhs->shape[1], N = rhs->shape[1];
  const long long G = group_sizes->shape[0], Ga = out->shape[0];
  if (rhs->shape[0] != M)
    return fail(h, GMM_E_INVALID, "lhs and rhs must have the same rows: lhs " + shape_str(lhs) + ", rhs " + shape_str(rhs));
  if (M < 0 || K <= 0 || N <= 0 || Ga < 0) return fail(h, GMM_E_INVALID, "negative or zero extent");
  if (out->shape[1] != K || out->shape[2] != N)
    return fail(h, GMM_E_INVALID, "out must be [Ga," + std::to_string(K) + "," + std::to_string(N) + "], got " + shape_str(out));
  if (lhs->dtype != GMM_BF16 || rhs->dtype != GMM_BF16) {
    if (elem_size(lhs->dtype) == 0 || elem_size(rhs->dtype) == 0 || lhs->dtype == GMM_I32 || rhs->dtype == GMM_I32)
      return fail(h, GMM_E_INVALID, "unsupported lhs / rhs dtype");
    return fail(h, GMM_E_UNSUPPORTED, "tgmm takes bf16 lhs and rhs");
  }
  if (out->dtype != GMM_F32 && out->dtype != GMM_BF16) return fail(h, GMM_E_INVALID, "out must be f32 or bf16");
  if (G < 1) return fail(h, GMM_E_INVALID, "group_sizes must hold at least one group");
  if (Ga > G) return fail(h, GMM_E_INVALID, "out holds more groups than group_sizes");
  if (G > gmmk::kMaxGroups) return fail(h, GMM_E_UNSUPPORTED, "more than 1024 groups");
  if (K % 8 || N % 8) return fail(h, GMM_E_UNSUPPORTED, "K and N must be multiples of 8");
  if (M * K * 2 >= 0x7FFFFFF0LL || M * N * 2 >= 0x7FFFFFF0LL || Ga * K >= (1LL << 31))
    return fail(h, GMM_E_UNSUPPORTED, "an operand beyond 2 GiB or Ga*K beyond 2^31");
  // the epilogue addresses an output tile of up to 384 rows with 32-bit byte offsets
  if (384LL * N * elem_size(out->dtype) >= 0x7FFFFFF0LL)
    return fail(h, GMM_E_UNSUPPORTED, "a 384-row output tile exceeds 2 GiB");
  const gmm_tensor* ins[] = {lhs, rhs, group_sizes};
  for (const gmm_tensor* t : ins) {
    if (numel(t) > 0 && !t->data) return fail(h, GMM_E_INVALID, "null data pointer");
    if (!aligned16(t->data)) return fail(h, GMM_E_INVALID, "tensor data must be 16-byte aligned");
    if (overlaps(t, out)) return fail(h, GMM_E_INVALID, "out overlaps an input");
  }
  if (Ga > 0 && !out->data) return fail(h, GMM_E_INVALID, "null out pointer");
  if (!aligned16(out->data) || !aligned16(group_offset))
    return fail(h, GMM_E_INVALID, "out and group_offset must be 16-byte aligned");
  if (Ga == 0) return GMM_OK;

  DeviceGuard g(h->device);
  int32_t* queue = nullptr;
  if (no_alloc) {
    // the device's scratch keeps the last call's contents: clear the
    // counters in stream order (a kernel, not a memset)
    queue = static_cast<int32_t*>(h->scratch);
    hipError_t e = gmmk::launch_clear_ints(queue, (int)(kQueueBlock / sizeof(int32_t)),
                                           static_cast<hipStream_t>(stream));
    if (e != hipSuccess) return fail(h, GMM_E_HIP, std::string("kernel launch failed: ") + hipGetErrorString(e));
  } else {
    int32_t*& q = h->queues[stream];
    if (!q) {  // first call on this stream: its counters, zeroed
      if (hipMalloc(&q, kQueueBlock) != hipSuccess || hipMemset(q, 0, kQueueBlock) != hipSuccess) {
        if (q) (void)hipFree(q);
        h->queues.erase(stream);
        return fail(h, GMM_E_HIP, "allocating the work-queue counters failed");
      }
    }
    queue = q;
  }
  gmmk::Params p{};
  p.lhs = lhs->data;
  p.rhs = rhs->data;
  p.group_sizes = static_cast<const int32_t*>(group_sizes->data);
  p.group_offset = group_offset;
  p.out = const_cast<void*>(out->data);
  p.flags = h->flags;
  p.queue = queue;
  p.M = (int32_t)M;
  p.K = (int32_t)K;
  p.N = (int32_t)N;
  p.G = (int32_t)G;
  p.Ga = (int32_t)Ga;
  p.nb = 1;
  p.blk = (int32_t)K;
  p.out_f32 = out->dtype == GMM_F32;
  hipError_t e = gmmk::launch_tgmm(p, h->cu_count, h->grid_limit, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return fail(h, GMM_E_HIP, std::string("kernel launch failed: ") + hipGetErrorString(e));
  return GMM_OK;
}

gmm_status gmm_tgmm_run(gmm_handle* h, const gmm_tensor* lhs, const gmm_tensor* rhs,
                        const gmm_tensor* group_sizes, const int32_t* group_offset, const gmm_tensor* out,
                        void* stream) {
  return run_tgmm(h, lhs, rhs, group_sizes, group_offset, out, stream, false);
}

gmm_status gmm_tgmm_run_noalloc(gmm_handle* h, const gmm_tensor* lhs, const gmm_tensor* rhs,
                                const gmm_tensor* group_sizes, const int32_t* group_offset,
                                const gmm_tensor* out, void* stream) {
  return run_tgmm(h, lhs, rhs, group_sizes, group_offset, out, stream, true);
}

gmm_status gmm_device_flags(gmm_handle* h, void* stream, uint32_t* flags) {
  if (!h || !flags) return GMM_E_INVALID;
  DeviceGuard g(h->device);
  hipStream_t st = static_cast<hipStream_t>(stream);
  uint32_t v = 0;
  if (hipStreamSynchronize(st) != hipSuccess ||
      hipMemcpy(&v, h->flags, sizeof v, hipMemcpyDeviceToHost) != hipSuccess ||
      hipMemset(h->flags, 0, sizeof v) != hipSuccess)
    return fail(h, GMM_E_HIP, "reading the device flags failed");
  *flags = v;
  if (v) return fail(h, GMM_E_DEVICE_DATA, "invalid device-resident group_sizes or group offset (flags " + std::to_string(v) + ")");
  return GMM_OK;
}

gmm_status gmm_debug_worklist(gmm_handle* h, const gmm_tensor* group_sizes, const int32_t* group_offset,
                              int64_t num_active, int64_t M, int32_t tm, int32_t* tiles, int64_t capacity,
                              int32_t* count, void* stream) {
  if (!h) return GMM_E_INVALID;
  h->err.clear();
  if (!group_sizes || group_sizes->ndim != 1 || group_sizes->dtype != GMM_I32 || !group_sizes->data)
    return fail(h, GMM_E_INVALID, "expected a 1-d int32 group_sizes");
  const long long G = group_sizes->shape[0];
  if (G < 1 || G > gmmk::kMaxGroups) return fail(h, GMM_E_UNSUPPORTED, "1 <= G <= 1024 required");
  if (num_active < 0 || num_active > G) return fail(h, GMM_E_INVALID, "num_active must be in [0, G]");
  if (M < 0 || M >= (1LL << 31)) return fail(h, GMM_E_INVALID, "M out of range");
  if (tm < 1 || tm > 4096) return fail(h, GMM_E_INVALID, "tm must be in [1, 4096]");
  if (!count || (capacity > 0 && !tiles) || capacity < 0) return fail(h, GMM_E_INVALID, "bad output buffers");
  gmmk::Params p{};
  p.group_sizes = static_cast<const int32_t*>(group_sizes->data);
  p.group_offset = group_offset;
  p.flags = h->flags;
  p.M = (int32_t)M;
  p.G = (int32_t)G;
  p.Ga = (int32_t)num_active;
  DeviceGuard g(h->device);
  hipError_t e = gmmk::launch_worklist(p, tm, tiles, capacity, count, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return fail(h, GMM_E_HIP, std::string("kernel launch failed: ") + hipGetErrorString(e));
  return GMM_OK;
}

}  // extern "C"
