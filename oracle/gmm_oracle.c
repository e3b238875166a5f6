/*
 * gmm_oracle.c -- plain CPU reference for grouped matrix multiplication.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing in the product library links, loads or
 * calls this file; only the tests, the smoke check and the benchmark's CPU
 * baseline leg do.  It shares no code, header or table with the HIP path.
 *
 * What it computes is the plain definition of the Megablox grouped matmul
 * (tpu-inference 0.13.2 wheel diff page, megablox/gmm.py, docstring of gmm():
 * each group's contiguous block of lhs rows is multiplied by that group's
 * slice of rhs), with the extras the same function's kernel body applies:
 *
 *   rows of group g are  [o[g], o[g+1])  with  o[0] = 0,
 *                        o[g+1] = o[g] + group_sizes[g]
 *       (make_group_metadata: group offsets are the cumulative sum of the
 *        group sizes, like CSR row offsets)
 *   only groups s .. s+Ga-1 are computed, Ga = rhs.shape[0], and rhs, scale
 *   and bias are indexed by g - s
 *       (gmm(): group_offset argument; kernel index maps subtract the offset)
 *   out[r, n] = sum_b scale[g-s, b, 0, n] * lscale[r, b] *
 *                     (sum over k in block b of lhs[r, k] * W(g-s, n, k))
 *               + bias[g-s, 0, n]
 *       (kernel _accum: the accumulator is reset per quantisation block,
 *        multiplied by that block's rhs_scale, and the bias is added once;
 *        the per-token lhs scale is the activation scale of the block-scaled
 *        W8A8 GEMM on the metrale gemm_quant.rs page, doc comment of
 *        fp8_gemm_t_blockscaled)
 *   W(h, n, k) = rhs[h, n, k]   when transpose_rhs == 0  (NT, rhs [Ga,N,K])
 *              = rhs[h, k, n]   when transpose_rhs == 1  (NN, rhs [Ga,K,N],
 *                the forward weight read in place as in the MaxText PR
 *                "transposed-RHS gmm_v2 kernel for the backward dlhs")
 *   every row outside [o[s], o[s+Ga]) is 0
 *       (gmm(): _zero_uninitialized_memory; applied to every such row)
 *
 * Arithmetic: every input element is decoded exactly to double; products and
 * sums are formed in double with k ascending; the result is returned in
 * double, before any rounding to the output type.  Rounding to the output
 * type is left to the caller.
 *
 * Element decoders are written from the format definitions:
 *   f32      IEEE-754 binary32.
 *   bf16     the upper 16 bits of a binary32.
 *   e4m3fn   1 sign bit, 4 exponent bits (bias 7), 3 mantissa bits; exponent
 *            field 0 encodes subnormals m/8 * 2^-6; S.1111.111 is NaN; there
 *            are no infinities (OCP 8-bit floating point specification).
 *   e5m2     1 sign bit, 5 exponent bits (bias 15), 2 mantissa bits; exponent
 *            field 0 encodes subnormals m/4 * 2^-14; exponent field 31 is
 *            infinity (m = 0) or NaN (same specification; one of the dtypes
 *            the Megablox gmm accepts, assert_is_supported_dtype on the
 *            tpu-inference wheel diff page).
 *   int8     two's-complement integer, -128 .. 127 (also on that list).
 *   int4, uint4, fp4 e2m1 (also on that list): four bits, two to a byte,
 *            element i in the low nibble of byte i/2 when i is even and in
 *            the high nibble when odd.  int4 is two's complement (-8 .. 7),
 *            uint4 0 .. 15; e2m1 has 1 sign, 2 exponent (bias 1) and 1
 *            mantissa bit: exponent field 0 encodes m/2, else
 *            (1 + m/2) * 2^(e-1), so the magnitudes are 0, 0.5, 1, 1.5, 2,
 *            3, 4 and 6 (OCP microscaling formats specification).
 */
#include <math.h>
#include <omp.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

/* Threads the parallel loops below use (the benchmark times the oracle on
 * one thread as well as on all of them).  n <= 0 leaves the count as it is.
 * Returns the count in force.  No arithmetic depends on it: every output
 * element is summed by one thread in k order. */
int oracle_set_threads(int n) {
  if (n > 0) omp_set_num_threads(n);
  return omp_get_max_threads();
}

#define OR_F32 0
#define OR_BF16 1
#define OR_E4M3FN 2
#define OR_E5M2 3
#define OR_I8 4
#define OR_I4 5
#define OR_U4 6
#define OR_F4E2M1 7

#define OR_OK 0
#define OR_E_ARG (-1)
#define OR_E_DATA (-4)
#define OR_E_NOMEM (-5)

double oracle_decode_bf16(uint16_t bits) {
  uint32_t u = (uint32_t)bits << 16;
  float f;
  memcpy(&f, &u, sizeof f);
  return (double)f;
}

double oracle_decode_e4m3fn(uint8_t code) {
  int sign = (code >> 7) & 1;
  int e = (code >> 3) & 0xF;
  int m = code & 0x7;
  double v;
  if (e == 0xF && m == 0x7) return NAN;
  if (e == 0)
    v = ldexp((double)m / 8.0, -6);
  else
    v = ldexp(1.0 + (double)m / 8.0, e - 7);
  return sign ? -v : v;
}

double oracle_decode_e5m2(uint8_t code) {
  int sign = (code >> 7) & 1;
  int e = (code >> 2) & 0x1F;
  int m = code & 0x3;
  double v;
  if (e == 0x1F) v = m ? NAN : INFINITY;
  else if (e == 0)
    v = ldexp((double)m / 4.0, -14);
  else
    v = ldexp(1.0 + (double)m / 4.0, e - 15);
  return sign ? -v : v;
}

/*
 * Round a double once to bfloat16, to nearest with ties to even (the cast of
 * the fp32 accumulator to the output type in the kernel body of gmm();
 * the rounding mode is not stated there, nearest-even is read in).
 * bfloat16 keeps 8 significant bits over binary32's exponent range:
 * quantum 2^(e-7) for |x| in [2^e, 2^(e+1)), e >= -126, and 2^-133 below.
 * Overflow gives infinity.
 */
uint16_t oracle_round_bf16(double x) {
  float f;
  uint32_t u;
  if (x != x) return 0x7FC0;
  if (x == 0.0 || isinf(x)) {
    f = (float)x;
  } else {
    int e;
    frexp(x, &e);            /* x = m * 2^e, 0.5 <= |m| < 1 */
    e -= 1;                  /* now |x| in [2^e, 2^(e+1)) */
    if (e < -126) e = -126;
    double q = ldexp(1.0, e - 7);
    double r = nearbyint(x / q) * q;  /* default rounding: nearest, ties to even */
    if (fabs(r) >= ldexp(1.0, 128)) r = x > 0 ? INFINITY : -INFINITY;
    f = (float)r;            /* exact: r has at most 8 significant bits */
  }
  memcpy(&u, &f, sizeof u);
  return (uint16_t)(u >> 16);
}

void oracle_round_bf16_array(const double* x, int64_t n, uint16_t* out) {
  for (int64_t i = 0; i < n; ++i) out[i] = oracle_round_bf16(x[i]);
}

double oracle_decode_e2m1(uint8_t nibble) {
  const int sign = (nibble >> 3) & 1, e = (nibble >> 1) & 3, m = nibble & 1;
  const double v = e == 0 ? m * 0.5 : (1.0 + m * 0.5) * ldexp(1.0, e - 1);
  return sign ? -v : v;
}

static int nibble_at(const void* base, int64_t idx) {
  const uint8_t b = ((const uint8_t*)base)[idx >> 1];
  return (idx & 1) ? b >> 4 : b & 0xF;
}

static double load_elem(const void* base, int dtype, int64_t idx) {
  switch (dtype) {
    case OR_F32: return (double)((const float*)base)[idx];
    case OR_BF16: return oracle_decode_bf16(((const uint16_t*)base)[idx]);
    case OR_E4M3FN: return oracle_decode_e4m3fn(((const uint8_t*)base)[idx]);
    case OR_E5M2: return oracle_decode_e5m2(((const uint8_t*)base)[idx]);
    case OR_I8: return (double)((const int8_t*)base)[idx];
    case OR_I4: {
      const int n = nibble_at(base, idx);
      return (double)(n >= 8 ? n - 16 : n);
    }
    case OR_U4: return (double)nibble_at(base, idx);
    case OR_F4E2M1: return oracle_decode_e2m1((uint8_t)nibble_at(base, idx));
    default: return NAN;
  }
}

static int dtype_ok(int d) { return d >= OR_F32 && d <= OR_F4E2M1; }

/*
 * Group offsets o[0..G] (int64, so no overflow) from group_sizes.
 * Returns OR_E_DATA for a negative size or a total beyond M.
 */
int oracle_group_offsets(const int32_t* group_sizes, int64_t G, int64_t M, int64_t* o) {
  o[0] = 0;
  for (int64_t g = 0; g < G; ++g) {
    if (group_sizes[g] < 0) return OR_E_DATA;
    o[g + 1] = o[g] + group_sizes[g];
  }
  if (o[G] > M) return OR_E_DATA;
  return OR_OK;
}

/*
 * oracle_gmm: reference values for a set of output rows.
 *
 *   lhs          [M, K] of lhs_dtype, row-major.
 *   rhs          [Ga, N, K] (transpose_rhs == 0) or [Ga, K, N] (== 1).
 *   group_sizes  [G] int32.
 *   group_offset s; groups s .. s+Ga-1 are active.  Requires 0 <= s and
 *                s + Ga <= G.
 *   rhs_scale    NULL or f32 [Ga, nb, 1, N]; K % nb == 0.
 *   rhs_bias     NULL or [Ga, 1, N] of bias_dtype.
 *   lhs_scale    NULL or f32 [M, nb].
 *   nb           number of quantisation blocks (1 when no scale is given).
 *   rows         NULL (all M rows, in order) or n_rows row indices.
 *   out          [n_rows, N] double: reference value of each requested row.
 *   row_group    NULL or [n_rows] int64: the group of each row, -1 if none.
 *
 * Returns OR_OK, OR_E_ARG for inconsistent arguments, OR_E_DATA for invalid
 * group sizes or group offset, OR_E_NOMEM.
 */
int oracle_gmm(const void* lhs, int lhs_dtype, int64_t M, int64_t K,
               const void* rhs, int rhs_dtype, int64_t Ga, int64_t N, int transpose_rhs,
               const int32_t* group_sizes, int64_t G, int64_t group_offset,
               const float* rhs_scale, const void* rhs_bias, int bias_dtype,
               const float* lhs_scale, int64_t nb,
               const int64_t* rows, int64_t n_rows,
               double* out, int64_t* row_group) {
  if (M < 0 || K <= 0 || N <= 0 || Ga < 0 || G < 0 || nb <= 0) return OR_E_ARG;
  if (!dtype_ok(lhs_dtype) || !dtype_ok(rhs_dtype)) return OR_E_ARG;
  if (rhs_bias && !dtype_ok(bias_dtype)) return OR_E_ARG;
  if (K % nb != 0) return OR_E_ARG;
  if (!rhs_scale && !lhs_scale && nb != 1) return OR_E_ARG;
  if (rows == NULL) n_rows = M;
  for (int64_t i = 0; i < n_rows; ++i) {
    int64_t r = rows ? rows[i] : i;
    if (r < 0 || r >= M) return OR_E_ARG;
  }
  const int64_t s = group_offset;
  if (s < 0 || s + Ga > G) return OR_E_DATA;

  int64_t* o = (int64_t*)malloc(sizeof(int64_t) * (size_t)(G + 1));
  if (!o) return OR_E_NOMEM;
  int rc = oracle_group_offsets(group_sizes, G, M, o);
  if (rc != OR_OK) { free(o); return rc; }

  /* Rows that belong to no active group are zero. */
  for (int64_t i = 0; i < n_rows; ++i) {
    for (int64_t n = 0; n < N; ++n) out[i * N + n] = 0.0;
    if (row_group) row_group[i] = -1;
  }

  const int64_t blk = K / nb;
  double* w = (double*)malloc(sizeof(double) * (size_t)(N * K));
  if (!w) { free(o); return OR_E_NOMEM; }

  for (int64_t g = s; g < s + Ga; ++g) {
    const int64_t lo = o[g], hi = o[g + 1];
    if (hi == lo) continue;
    int any = 0;
    for (int64_t i = 0; i < n_rows && !any; ++i) {
      int64_t r = rows ? rows[i] : i;
      any = (r >= lo && r < hi);
    }
    if (!any) continue;
    const int64_t h = g - s;

    /* This group's weight, decoded exactly, as W(n, k). */
    for (int64_t n = 0; n < N; ++n)
      for (int64_t k = 0; k < K; ++k) {
        int64_t idx = transpose_rhs ? (h * K + k) * N + n : (h * N + n) * K + k;
        w[n * K + k] = load_elem(rhs, rhs_dtype, idx);
      }

#pragma omp parallel for schedule(dynamic, 1)
    for (int64_t i = 0; i < n_rows; ++i) {
      const int64_t r = rows ? rows[i] : i;
      if (r < lo || r >= hi) continue;
      if (row_group) row_group[i] = g;
      for (int64_t n = 0; n < N; ++n) {
        double t = 0.0;
        for (int64_t b = 0; b < nb; ++b) {
          double p = 0.0;
          for (int64_t k = b * blk; k < (b + 1) * blk; ++k)
            p += load_elem(lhs, lhs_dtype, r * K + k) * w[n * K + k];
          if (rhs_scale) p *= (double)rhs_scale[(h * nb + b) * N + n];
          if (lhs_scale) p *= (double)lhs_scale[r * nb + b];
          t += p;
        }
        if (rhs_bias) t += load_elem(rhs_bias, bias_dtype, h * N + n);
        out[i * N + n] = t;
      }
    }
  }
  free(w);
  free(o);
  return OR_OK;
}

/*
 * oracle_tgmm: reference values of the transposed grouped matmul, the weight
 * gradient of gmm.  The Megablox metadata builder (tpu-inference wheel diff
 * page, megablox/gmm.py, make_group_metadata, argument visit_empty_groups)
 * keeps a tile for every empty group because this operation must still write
 * that group's output; the MaxText PR page "transposed-RHS gmm_v2 kernel for
 * the backward dlhs" keeps it as the weight-gradient step of gmm's custom VJP.
 * For the forward out_g = lhs_g . W_g (W_g [K, N], rows of group g), the
 * gradient of sum(out . rhs) with respect to W_g is lhs_g^T . rhs_g:
 *
 *   out[h, k, n] = sum over r in [o[g], o[g+1]) of lhs[r, k] * rhs[r, n],
 *                  g = s + h, r ascending, in double;
 *   out[h] = 0 when group g is empty.
 *
 *   lhs          [M, K] of lhs_dtype, row-major.
 *   rhs          [M, N] of rhs_dtype, row-major.
 *   group_sizes  [G] int32; groups s .. s+Ga-1 are active (0 <= s,
 *                s + Ga <= G).
 *   sel_h, sel_k NULL (every (h, k), h-major) or n_sel pairs: output row k
 *                of active group h.
 *   out          [n_sel, N] double (n_sel = Ga * K when no selection).
 *
 * Returns OR_OK, OR_E_ARG, OR_E_DATA (invalid sizes or offset), OR_E_NOMEM.
 */
int oracle_tgmm(const void* lhs, int lhs_dtype, int64_t M, int64_t K,
                const void* rhs, int rhs_dtype, int64_t N,
                const int32_t* group_sizes, int64_t G, int64_t group_offset, int64_t Ga,
                const int64_t* sel_h, const int64_t* sel_k, int64_t n_sel, double* out) {
  if (M < 0 || K <= 0 || N <= 0 || Ga < 0 || G < 0) return OR_E_ARG;
  if (!dtype_ok(lhs_dtype) || !dtype_ok(rhs_dtype)) return OR_E_ARG;
  if ((sel_h == NULL) != (sel_k == NULL)) return OR_E_ARG;
  if (sel_h == NULL) n_sel = Ga * K;
  for (int64_t i = 0; i < n_sel && sel_h; ++i)
    if (sel_h[i] < 0 || sel_h[i] >= Ga || sel_k[i] < 0 || sel_k[i] >= K) return OR_E_ARG;
  const int64_t s = group_offset;
  if (s < 0 || s + Ga > G) return OR_E_DATA;

  int64_t* o = (int64_t*)malloc(sizeof(int64_t) * (size_t)(G + 1));
  if (!o) return OR_E_NOMEM;
  int rc = oracle_group_offsets(group_sizes, G, M, o);
  if (rc != OR_OK) { free(o); return rc; }

#pragma omp parallel for schedule(dynamic, 1)
  for (int64_t i = 0; i < n_sel; ++i) {
    const int64_t h = sel_h ? sel_h[i] : i / K;
    const int64_t k = sel_k ? sel_k[i] : i % K;
    const int64_t lo = o[s + h], hi = o[s + h + 1];
    double* row = out + i * N;
    for (int64_t n = 0; n < N; ++n) row[n] = 0.0;
    for (int64_t r = lo; r < hi; ++r) {
      const double a = load_elem(lhs, lhs_dtype, r * K + k);
      for (int64_t n = 0; n < N; ++n) row[n] += a * load_elem(rhs, rhs_dtype, r * N + n);
    }
  }
  free(o);
  return OR_OK;
}

/*
 * Per-token activation quantisation to e4m3fn over blocks of `blk` elements
 * of each row: the per_token_group_quant_fp8 launcher on the metrale
 * gemm_quant.rs page (bf16 input [M,K] -> A_fp8 [M,K] e4m3 and a_scale
 * [M,K/128] f32 over 128-element K groups; the scale is the activation
 * scale of fp8_gemm_t_blockscaled on the same page, so x ~ q * scale).  The
 * page gives shapes only; the arithmetic read in for both this oracle and
 * the device kernel:
 *   amax  = max |x| over the block (exact in binary32: x is bf16)
 *   scale = amax / 448 in binary32, rounded to nearest (448 is the largest
 *           finite e4m3fn value); 1 when amax is 0
 *   q     = the e4m3fn value nearest to clamp(x / scale, -448, 448), where
 *           x / scale is one binary32 division rounded to nearest; ties go to
 *           the even mantissa; the sign of x is kept, so a negative value
 *           that rounds to zero (and -0) gives the code 0x80
 */

/* e4m3fn code nearest to v, |v| <= 448 (ties to the even mantissa). */
uint8_t oracle_round_e4m3fn(double v) {
  const uint8_t sign = signbit(v) ? 0x80 : 0x00;
  const double a = fabs(v);
  if (a == 0.0) return sign;
  int e;
  frexp(a, &e);
  e -= 1;                  /* a in [2^e, 2^(e+1)) */
  if (e < -6) e = -6;      /* below 2^-6 the spacing is the subnormal one, 2^-9 */
  const double quantum = ldexp(1.0, e - 3);
  const double r = nearbyint(a / quantum) * quantum;  /* nearest; ties to an even multiple */
  if (r == 0.0) return sign;
  if (r < ldexp(1.0, -6)) return (uint8_t)(sign | (uint8_t)(r / ldexp(1.0, -9)));  /* subnormal m/8 * 2^-6 */
  int er;
  const double m = frexp(r, &er);                     /* r = m * 2^er, m in [0.5, 1) */
  const int biased = er - 1 + 7;
  const int mant = (int)(m * 16.0) - 8;               /* r / 2^(er-1) = 1 + mant/8 */
  return (uint8_t)(sign | (uint8_t)(biased << 3) | (uint8_t)mant);
}

int oracle_quant_fp8(const uint16_t* x, int64_t M, int64_t K, int64_t blk, uint8_t* q, float* scale) {
  if (M < 0 || K <= 0 || blk <= 0 || K % blk) return OR_E_ARG;
  const int64_t nb = K / blk;
#pragma omp parallel for schedule(static)
  for (int64_t r = 0; r < M; ++r) {
    for (int64_t b = 0; b < nb; ++b) {
      const uint16_t* xb = x + r * K + b * blk;
      float amax = 0.0f;
      for (int64_t k = 0; k < blk; ++k) {
        const float a = fabsf((float)oracle_decode_bf16(xb[k]));
        if (a > amax) amax = a;
      }
      volatile float s = amax / 448.0f;
      if (amax == 0.0f) s = 1.0f;
      scale[r * nb + b] = s;
      for (int64_t k = 0; k < blk; ++k) {
        volatile float t = (float)oracle_decode_bf16(xb[k]) / s;
        float c = t;
        if (c > 448.0f) c = 448.0f;
        if (c < -448.0f) c = -448.0f;
        q[r * K + b * blk + k] = oracle_round_e4m3fn((double)c);
      }
    }
  }
  return OR_OK;
}

/*
 * Block-scale widening to binary32: widen_block_scale_f32 on the metrale
 * gemm_quant.rs page, which lets the block-scaled kernels read f32 scales.
 * The source is bf16 (dtype 0), f32 (1) or E8M0 (2).  An E8M0 byte e is
 * 2^(e - 127), the binary32 whose bit pattern is e << 23, except as the page
 * states for its ends: e = 0 is 2^-127 and e = 255 is 0.0.
 */
float oracle_widen_scale(const void* src, int dtype, int64_t i) {
  switch (dtype) {
    case 0: return (float)oracle_decode_bf16(((const uint16_t*)src)[i]);
    case 1: return ((const float*)src)[i];
    case 2: {
      const int e = ((const uint8_t*)src)[i];
      if (e == 0) return ldexpf(1.0f, -127);
      if (e == 255) return 0.0f;
      return ldexpf(1.0f, e - 127);
    }
    default: return NAN;
  }
}

int oracle_widen_scales(const void* src, int dtype, int64_t n, float* dst) {
  if (n < 0 || dtype < 0 || dtype > 2) return OR_E_ARG;
  for (int64_t i = 0; i < n; ++i) dst[i] = oracle_widen_scale(src, dtype, i);
  return OR_OK;
}
