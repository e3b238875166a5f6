"""The C oracle under the host sanitizers (CPU only).

oracle/gmm_oracle.c is compiled with gcc's AddressSanitizer and
UndefinedBehaviorSanitizer (any report is fatal) together with a small C
driver that calls every entry point: the element decoders and rounders over
all their codes (each finite e4m3fn code must round back to itself), gmm
over every operand type (the four-bit ones packed two to a byte), NT and NN
layouts, scales, f32 and bf16 bias, a group offset, row selections, empty
groups and rows outside the groups, tgmm over full outputs and selections,
the activation quantiser and the scale widening, and the argument and data
errors each documents.  The driver checks each call's return code; the
sanitizers check every access and every integer and float conversion on
the way.  (A host-only gcc build: nothing here runs on a GPU.)"""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = os.path.join(ROOT, "oracle", "gmm_oracle.c")

DRIVER = r"""
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

int oracle_set_threads(int n);
double oracle_decode_bf16(uint16_t bits);
double oracle_decode_e4m3fn(uint8_t code);
double oracle_decode_e5m2(uint8_t code);
double oracle_decode_e2m1(uint8_t nibble);
uint16_t oracle_round_bf16(double x);
void oracle_round_bf16_array(const double* x, int64_t n, uint16_t* out);
uint8_t oracle_round_e4m3fn(double v);
int oracle_group_offsets(const int32_t* group_sizes, int64_t G, int64_t M, int64_t* o);
int oracle_gmm(const void* lhs, int lhs_dtype, int64_t M, int64_t K, const void* rhs, int rhs_dtype, int64_t Ga,
               int64_t N, int transpose_rhs, const int32_t* group_sizes, int64_t G, int64_t group_offset,
               const float* rhs_scale, const void* rhs_bias, int bias_dtype, const float* lhs_scale, int64_t nb,
               const int64_t* rows, int64_t n_rows, double* out, int64_t* row_group);
int oracle_tgmm(const void* lhs, int lhs_dtype, int64_t M, int64_t K, const void* rhs, int rhs_dtype, int64_t N,
                const int32_t* group_sizes, int64_t G, int64_t group_offset, int64_t Ga, const int64_t* sel_h,
                const int64_t* sel_k, int64_t n_sel, double* out);
int oracle_quant_fp8(const uint16_t* x, int64_t M, int64_t K, int64_t blk, uint8_t* q, float* scale);
float oracle_widen_scale(const void* src, int dtype, int64_t i);
int oracle_widen_scales(const void* src, int dtype, int64_t n, float* dst);

enum { F32, BF16, E4M3FN, E5M2, I8, I4, U4, F4E2M1 };
static int fails = 0;
#define EXPECT(call, want) do { int rc_ = (call); if (rc_ != (want)) { \
  printf("line %d: %s returned %d, expected %d\n", __LINE__, #call, rc_, (want)); ++fails; } } while (0)

static size_t esize(int dt) { return dt == F32 ? 4 : dt == BF16 ? 2 : 1; }
static int packed(int dt) { return dt == I4 || dt == U4 || dt == F4E2M1; }
/* a buffer of n elements of dt with a seeded pattern of small finite values */
static void* fill(int dt, int64_t n, unsigned seed) {
  size_t bytes = packed(dt) ? (size_t)(n + 1) / 2 : (size_t)n * esize(dt);
  unsigned char* p = malloc(bytes ? bytes : 1);
  for (size_t i = 0; i < bytes; ++i) {
    seed = seed * 1103515245u + 12345u;
    p[i] = (unsigned char)(seed >> 16);
  }
  if (dt == F32) for (int64_t i = 0; i < n; ++i) ((float*)p)[i] = (float)((int)(p[4 * i] % 7) - 3);
  if (dt == BF16) for (int64_t i = 0; i < n; ++i) ((uint16_t*)p)[i] = (uint16_t)(0x3f80 + (p[2 * i] & 0x3f));
  if (dt == E4M3FN) for (int64_t i = 0; i < n; ++i) p[i] &= 0x77;  /* no NaN codes */
  if (dt == E5M2) for (int64_t i = 0; i < n; ++i) p[i] &= 0x3f;
  return p;
}

int main(void) {
  oracle_set_threads(2);
  for (int c = 0; c < 65536; ++c) (void)oracle_round_bf16(oracle_decode_bf16((uint16_t)c));
  for (int c = 0; c < 256; ++c) {
    /* the rounder takes |v| <= 448: every code but the two NaNs */
    if ((c & 0x7f) != 0x7f && oracle_round_e4m3fn(oracle_decode_e4m3fn((uint8_t)c)) != c) {
      printf("e4m3fn code %d does not round-trip\n", c);
      ++fails;
    }
    (void)oracle_decode_e5m2((uint8_t)c);
  }
  for (int c = 0; c < 16; ++c) (void)oracle_decode_e2m1((uint8_t)c);
  double xs[5] = {0.0, -0.0, 1e300, -1e-300, 3.5};
  uint16_t r16[5];
  oracle_round_bf16_array(xs, 5, r16);

  const int32_t sizes[6] = {7, 0, 33, 1, 0, 20};
  const int64_t G = 6, M = 64, K = 256, N = 24, nb = 2;
  int64_t o[7];
  EXPECT(oracle_group_offsets(sizes, G, M, o), 0);
  const int32_t bad[2] = {5, -1};
  EXPECT(oracle_group_offsets(bad, 2, M, o), -4);

  const int lhs_types[] = {F32, BF16, E4M3FN, E5M2, I8, I4, U4, F4E2M1};
  const int rhs_types[] = {F32, BF16, E4M3FN, E5M2, I8, I4, U4, F4E2M1};
  float* rs = (float*)fill(F32, G * nb * N, 11);
  float* ls = (float*)fill(F32, M * nb, 12);
  void* bias_f = fill(F32, G * N, 13);
  void* bias_b = fill(BF16, G * N, 14);
  int64_t rows[4] = {0, 6, 40, 63};
  double* out = malloc(sizeof(double) * M * N);
  int64_t* rg = malloc(sizeof(int64_t) * M);
  for (int a = 0; a < 8; ++a)
    for (int b = 0; b < 8; ++b)
      for (int t = 0; t < 2; ++t) {
        void* lhs = fill(lhs_types[a], M * K, 100 + a);
        void* rhs = fill(rhs_types[b], G * N * K, 200 + b);
        EXPECT(oracle_gmm(lhs, lhs_types[a], M, K, rhs, rhs_types[b], G, N, t, sizes, G, 0, NULL, NULL, 0, NULL,
                          1, NULL, 0, out, rg), 0);
        EXPECT(oracle_gmm(lhs, lhs_types[a], M, K, rhs, rhs_types[b], 4, N, t, sizes, G, 2, rs, bias_f, F32, ls,
                          nb, rows, 4, out, rg), 0);
        EXPECT(oracle_gmm(lhs, lhs_types[a], M, K, rhs, rhs_types[b], 3, N, t, sizes, G, 1, rs, bias_b, BF16,
                          NULL, nb, NULL, 0, out, NULL), 0);
        free(lhs);
        free(rhs);
      }
  void* lhs = fill(BF16, M * K, 7);
  void* rhs = fill(BF16, G * N * K, 8);
  int64_t out_of_range[1] = {M};
  EXPECT(oracle_gmm(lhs, BF16, M, K, rhs, BF16, G, N, 0, sizes, G, 0, NULL, NULL, 0, NULL, 1, out_of_range, 1, out,
                    rg), -1);
  EXPECT(oracle_gmm(lhs, BF16, M, K, rhs, BF16, G, N, 0, sizes, G, 1, NULL, NULL, 0, NULL, 1, NULL, 0, out, rg), -4);
  EXPECT(oracle_gmm(lhs, BF16, M, K, rhs, BF16, G, N, 0, sizes, G, 0, NULL, NULL, 0, NULL, 3, NULL, 0, out, rg), -1);
  EXPECT(oracle_gmm(lhs, BF16, M, K, rhs, 99, G, N, 0, sizes, G, 0, NULL, NULL, 0, NULL, 1, NULL, 0, out, rg), -1);

  /* tgmm: rhs [M, N] */
  void* trhs = fill(BF16, M * N, 9);
  double* tout = malloc(sizeof(double) * G * K * N);
  EXPECT(oracle_tgmm(lhs, BF16, M, K, trhs, BF16, N, sizes, G, 0, G, NULL, NULL, 0, tout), 0);
  int64_t sh[3] = {0, 2, 3}, sk[3] = {0, 255, 17};
  EXPECT(oracle_tgmm(lhs, BF16, M, K, trhs, BF16, N, sizes, G, 1, 4, sh, sk, 3, tout), 0);
  int64_t bad_k[1] = {K};
  EXPECT(oracle_tgmm(lhs, BF16, M, K, trhs, BF16, N, sizes, G, 0, G, sh, bad_k, 1, tout), -1);
  EXPECT(oracle_tgmm(lhs, BF16, M, K, trhs, BF16, N, sizes, G, 3, G, NULL, NULL, 0, tout), -4);

  /* the activation quantiser and the scale widening */
  uint8_t* q = malloc((size_t)(M * K));
  float* sc = malloc(sizeof(float) * M * (K / 128));
  EXPECT(oracle_quant_fp8((const uint16_t*)lhs, M, K, 128, q, sc), 0);
  EXPECT(oracle_quant_fp8((const uint16_t*)lhs, M, K, 100, q, sc), -1);
  /* the widening's source codes: bf16 0, f32 1, E8M0 2 (every byte) */
  float wide[256];
  uint8_t* e8 = malloc(256);
  for (int c = 0; c < 256; ++c) e8[c] = (uint8_t)c;
  EXPECT(oracle_widen_scales(e8, 2, 256, wide), 0);
  EXPECT(oracle_widen_scales(bias_b, 0, 64, wide), 0);
  EXPECT(oracle_widen_scales(rs, 1, 64, wide), 0);
  (void)oracle_widen_scale(e8, 2, 255);

  free(q); free(sc); free(e8); free(lhs); free(rhs); free(trhs); free(tout); free(out); free(rg);
  free(rs); free(ls); free(bias_f); free(bias_b);
  printf("fails %d\n", fails);
  return fails != 0;
}
"""


def test_oracle_under_address_and_undefined_behaviour_sanitizers(tmp_path):
    gcc = shutil.which("gcc")
    if not gcc:
        pytest.skip("gcc not available")
    drv = tmp_path / "driver.c"
    drv.write_text(DRIVER)
    exe = tmp_path / "oracle_sanitized"
    flags = ["-O1", "-g", "-std=c99", "-fopenmp", "-fsanitize=address,undefined", "-fno-sanitize-recover=all",
             "-fno-omit-frame-pointer"]
    res = subprocess.run([gcc] + flags + [SRC, str(drv), "-o", str(exe), "-lm"], capture_output=True, text=True)
    if res.returncode != 0 and "asan" in res.stderr.lower():
        pytest.skip("the sanitizer runtimes are not installed: " + res.stderr[-300:])
    assert res.returncode == 0, res.stderr[-3000:]
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=0", UBSAN_OPTIONS="print_stacktrace=1")
    run = subprocess.run([str(exe)], capture_output=True, text=True, timeout=600, env=env)
    assert run.returncode == 0, (run.stdout[-3000:], run.stderr[-3000:])
    assert "fails 0" in run.stdout
