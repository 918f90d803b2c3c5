"""Host builds under the address and undefined-behaviour sanitizers.

* The oracle (oracle/oracle.c) is compiled with gcc -fsanitize=address,undefined
  together with a small driver that calls every exported function on small
  inputs, including the corner cases the tests rely on (all-zero rows, rows
  whose scale is subnormal or underflows to zero, row subsets, out-of-range
  embedding ids, both gradient paths and the LoRA branch).
* The C ABI's argument checks (w8a8_rotated_int8_amd/csrc/validate.h, plain C++
  with no HIP call) are compiled with g++ under the same sanitizers and driven
  with null, misaligned, empty, oversized and valid arguments for every entry
  point.

Any sanitizer report aborts the program (-fno-sanitize-recover=all) and fails
the test.
"""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SAN = ["-fsanitize=address,undefined", "-fno-sanitize-recover=all", "-fno-omit-frame-pointer",
       "-g", "-O1"]

pytestmark = pytest.mark.skipif(shutil.which("gcc") is None or shutil.which("g++") is None,
                                reason="gcc/g++ not available")

ORACLE_DRIVER = r"""
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

int oracle_hadamard(int n, int8_t* H);
double oracle_norm_const(int block);
int oracle_rotate_rows(const uint16_t*, int64_t, int64_t, int, float*, int64_t*);
int oracle_quantize_rows(const float*, int64_t, int64_t, int8_t*, float*);
int oracle_rotate_quantize(const uint16_t*, int64_t, int64_t, int, int64_t, int8_t*, float*, int64_t*);
int oracle_gemm_i8_i32(const int8_t*, const int8_t*, int64_t, int64_t, int64_t, const int64_t*, int64_t, int32_t*);
int oracle_dequant_epilogue(const int32_t*, int64_t, int64_t, const float*, const int64_t*, const float*, const uint16_t*, uint16_t*);
int oracle_bwd_quant_dy(const uint16_t*, int64_t, int64_t, const float*, int8_t*, float*);
int oracle_gemm_i8_i32_rows_of_b(const int8_t*, const int8_t*, int64_t, int64_t, int64_t, const int64_t*, int64_t, int32_t*);
int oracle_bwd_int8_epilogue(const int32_t*, int64_t, int64_t, const float*, const int64_t*, int, uint16_t*);
int oracle_dequant_weight(const int8_t*, const float*, int64_t, int64_t, int, uint16_t*);
int oracle_bf16_gemm_dx(const uint16_t*, const uint16_t*, int64_t, int64_t, int64_t, const int64_t*, int64_t, uint16_t*);
int oracle_embedding_lookup(const int32_t*, int64_t, const int8_t*, const float*, int64_t, int64_t, int, uint16_t*, int64_t*);
int oracle_lora_down(const uint16_t*, int64_t, int64_t, const uint16_t*, int64_t, const int64_t*, int64_t, uint16_t*);
int oracle_lora_epilogue(const int32_t*, int64_t, int64_t, const float*, const int64_t*, const float*, const uint16_t*, const uint16_t*, const uint16_t*, int64_t, double, uint16_t*);
uint16_t oracle_double_to_bf16(double);

#define CHECK(c) do { if (!(c)) { printf("FAIL %s:%d %s\n", __FILE__, __LINE__, #c); return 1; } } while (0)

static uint16_t bf(float f) { return oracle_double_to_bf16((double)f); }

int main(void) {
  enum { M = 9, K = 256, N = 128, R = 16, V = 20, T = 7 };
  uint16_t* x = malloc(sizeof(uint16_t) * M * K);
  uint16_t* w = malloc(sizeof(uint16_t) * N * K);
  uint16_t* dy = malloc(sizeof(uint16_t) * M * N);
  srand(7);
  for (int i = 0; i < M * K; ++i) x[i] = bf((float)(rand() % 2001 - 1000) / 100.0f);
  for (int i = 0; i < N * K; ++i) w[i] = bf((float)(rand() % 2001 - 1000) / 50000.0f);
  for (int i = 0; i < M * N; ++i) dy[i] = bf((float)(rand() % 2001 - 1000) * 1e-6f);
  memset(x, 0, sizeof(uint16_t) * K);                         /* all-zero row */
  for (int i = 0; i < N; ++i) dy[N + i] = bf(ldexpf(1.0f, -120)); /* subnormal scale after fold */
  for (int i = 0; i < N; ++i) dy[2 * N + i] = bf(ldexpf(1.0f, -124)); /* scale underflows */
  float* sw_tiny = malloc(sizeof(float) * N);
  for (int i = 0; i < N; ++i) sw_tiny[i] = ldexpf(1.0f, -20);

  int8_t H[128 * 128];
  CHECK(oracle_hadamard(128, H) == 0);
  CHECK(oracle_norm_const(128) > 0.0);
  float* r = malloc(sizeof(float) * M * K);
  int64_t bad = -1;
  CHECK(oracle_rotate_rows(x, M, K, 128, r, &bad) == 0);
  int8_t* qr = malloc(M * K); float* sr = malloc(sizeof(float) * M);
  CHECK(oracle_quantize_rows(r, M, K, qr, sr) == 0);
  int8_t* qx = malloc(M * K); float* sx = malloc(sizeof(float) * M);
  int8_t* qw = malloc(N * K); float* sw = malloc(sizeof(float) * N);
  CHECK(oracle_rotate_quantize(x, M, K, 128, 4, qx, sx, &bad) == 0);
  CHECK(memcmp(qx, qr, M * K) == 0 && sx[0] == 0.0f);
  CHECK(oracle_rotate_quantize(w, N, K, 128, 0, qw, sw, &bad) == 0);
  int64_t rows[3] = {0, 4, M - 1};
  int32_t* acc = malloc(sizeof(int32_t) * M * N);
  CHECK(oracle_gemm_i8_i32(qx, qw, M, N, K, NULL, 0, acc) == 0);
  CHECK(oracle_gemm_i8_i32(qx, qw, M, N, K, rows, 3, acc) == 0);
  uint16_t* y = malloc(sizeof(uint16_t) * M * N);
  CHECK(oracle_dequant_epilogue(acc, 3, N, sx, rows, sw, w, y) == 0);
  int8_t* qg = malloc(M * N); float* sg = malloc(sizeof(float) * M);
  CHECK(oracle_bwd_quant_dy(dy, M, N, sw_tiny, qg, sg) == 0);
  CHECK(sg[1] == ldexpf(1.0f, -147) && qg[N] == 127 && sg[2] == 0.0f && qg[2 * N] == 0);
  CHECK(oracle_bwd_quant_dy(dy, M, N, sw, qg, sg) == 0);
  int32_t* acc2 = malloc(sizeof(int32_t) * M * K);
  CHECK(oracle_gemm_i8_i32_rows_of_b(qg, qw, M, N, K, rows, 3, acc2) == 0);
  uint16_t* dx = malloc(sizeof(uint16_t) * M * K);
  CHECK(oracle_bwd_int8_epilogue(acc2, 3, K, sg, rows, 128, dx) == 0);
  uint16_t* what = malloc(sizeof(uint16_t) * N * K);
  CHECK(oracle_dequant_weight(qw, sw, N, K, 128, what) == 0);
  CHECK(oracle_bf16_gemm_dx(dy, what, M, N, K, rows, 3, dx) == 0);
  int32_t ids[T] = {0, 5, -1, 19, 20, 3, 1 << 30};
  uint16_t* out = malloc(sizeof(uint16_t) * T * K);
  int64_t oob = 0;
  CHECK(oracle_embedding_lookup(ids, T, qw, sw, V, K, 128, out, &oob) == 0 && oob == 3);
  uint16_t* la = malloc(sizeof(uint16_t) * R * K);
  uint16_t* lb = malloc(sizeof(uint16_t) * N * R);
  for (int i = 0; i < R * K; ++i) la[i] = bf(0.01f * (float)(i % 7));
  for (int i = 0; i < N * R; ++i) lb[i] = bf(0.02f * (float)(i % 5));
  uint16_t* xa = malloc(sizeof(uint16_t) * M * R);
  CHECK(oracle_lora_down(x, M, K, la, R, rows, 3, xa) == 0);
  CHECK(oracle_lora_epilogue(acc, 3, N, sx, rows, sw, NULL, xa, lb, R, 0.5, y) == 0);
  /* rejected arguments */
  CHECK(oracle_rotate_rows(x, M, 100, 128, r, &bad) != 0);
  CHECK(oracle_hadamard(100, H) != 0);
  free(x); free(w); free(dy); free(sw_tiny); free(r); free(qr); free(sr); free(qx); free(sx);
  free(qw); free(sw); free(acc); free(y); free(qg); free(sg); free(acc2); free(dx); free(what);
  free(out); free(la); free(lb); free(xa);
  printf("ok\n");
  return 0;
}
"""

VALIDATE_DRIVER = r"""
#include <stdio.h>
#include "validate.h"

using namespace convrot::check;

static int failures = 0;
#define EXPECT(call, want) do { int got_ = (call); if (got_ != (want)) { \
    printf("FAIL line %d: %s = %d, want %d\n", __LINE__, #call, got_, (want)); ++failures; } } while (0)

static const void* P(unsigned long v) { return reinterpret_cast<const void*>(v); }

int main() {
  const void* a = P(1ul << 20); const void* b = P(2ul << 20); const void* y = P(3ul << 20);
  const void* ws = P(4ul << 20); const void* odd = P((1ul << 20) + 4);
  const int64_t big = 1ll << 31, huge = 1ll << 62;
  // quantizers
  EXPECT(quantize_weight(a, 64, 4096, 128, 0, b, y), CONVROT_OK);
  EXPECT(quantize_weight(a, 64, 4096, 64, 0, b, y), CONVROT_ESHAPE);
  EXPECT(quantize_weight(nullptr, 64, 4096, 64, 0, b, y), CONVROT_EINVAL);
  EXPECT(quantize_weight(nullptr, 0, 4096, 128, 0, nullptr, nullptr), kNoOp);
  EXPECT(quantize_rows(a, 64, 4096, b, y, 0, nullptr, true), CONVROT_EINVAL);
  EXPECT(quantize_rows(a, 64, 4096, b, odd, 0, nullptr, false), CONVROT_EINVAL);
  EXPECT(quantize_rows(a, 64, 100, b, y, 0, nullptr, false), CONVROT_ESHAPE);
  EXPECT(quantize_rows(a, 64, 65536, b, y, 0, nullptr, false), CONVROT_ESHAPE);
  EXPECT(quantize_rows(a, big, 128, b, y, 0, nullptr, false), CONVROT_ESHAPE);
  EXPECT(quantize_rows(a, huge, 4096, b, y, 0, nullptr, false), CONVROT_ESHAPE);
  EXPECT(quantize_rows(a, -huge, 4096, b, y, 0, nullptr, false), CONVROT_EINVAL);
  EXPECT(quantize_rows(a, 64, 4096, b, y, -1, nullptr, false), CONVROT_EINVAL);
  // GEMMs
  EXPECT(gemm_i8_bf16(a, b, a, b, 64, 256, 256, nullptr, y), CONVROT_OK);
  EXPECT(gemm_i8_bf16(a, b, a, b, 64, 256, 256, odd, y), CONVROT_EINVAL);
  EXPECT(gemm_i8_bf16(a, b, a, b, huge, huge, 256, nullptr, y), CONVROT_ESHAPE);
  EXPECT(gemm_i8_bf16(nullptr, nullptr, nullptr, nullptr, 0, 256, 256, nullptr, nullptr), kNoOp);
  EXPECT(gemm_i8_i32(a, b, 64, 256, 256, 0, y), CONVROT_OK);
  EXPECT(gemm_i8_i32(a, b, 64, 200, 256, 1, y), CONVROT_ESHAPE);
  EXPECT(gemm_i8_i32(a, b, 64, 256, 256, 2, y), CONVROT_EINVAL);
  EXPECT(gemm_i8_i32(a, b, 1ll << 30, 1ll << 30, 128, 0, y), CONVROT_ESHAPE);
  // forward, LoRA forward, LoRA down projection
  EXPECT(linear_fwd(a, 64, 4096, b, b, 4096, nullptr, y, ws), CONVROT_OK);
  EXPECT(linear_fwd(a, 64, 4096, b, b, 4096, nullptr, y, P((4ul << 20) + 16)), CONVROT_EINVAL);
  EXPECT(linear_fwd(a, 64, 4096, b, odd, 4096, nullptr, y, ws), CONVROT_EINVAL);
  EXPECT(linear_fwd(a, 64, 4096, b, b, big, nullptr, y, ws), CONVROT_ESHAPE);
  EXPECT(linear_fwd(a, huge, 4096, b, b, 4096, nullptr, y, ws), CONVROT_ESHAPE);
  EXPECT(linear_fwd(nullptr, 0, 4096, nullptr, nullptr, 4096, nullptr, nullptr, nullptr), kNoOp);
  EXPECT(linear_fwd(nullptr, 0, 4000, nullptr, nullptr, 4096, nullptr, nullptr, nullptr), CONVROT_ESHAPE);
  EXPECT(linear_fwd_lora(a, 64, 4096, b, b, 4096, nullptr, a, b, 16, y, ws), CONVROT_OK);
  EXPECT(linear_fwd_lora(a, 64, 4096, b, b, 4096, nullptr, a, b, 8, y, ws), CONVROT_ESHAPE);
  EXPECT(linear_fwd_lora(a, 64, 4096, b, b, 4096, nullptr, odd, b, 16, y, ws), CONVROT_EINVAL);
  EXPECT(lora_down(a, 64, 4096, b, 32, y), CONVROT_OK);
  EXPECT(lora_down(a, 64, 4096, b, 32, odd), CONVROT_EINVAL);
  EXPECT(lora_down(nullptr, 0, 4096, nullptr, 32, nullptr), kNoOp);
  // input gradient, transient dequantization
  EXPECT(linear_bwd_dx(a, 64, 4096, b, b, 4096, CONVROT_BWD_INT8, y, ws), CONVROT_OK);
  EXPECT(linear_bwd_dx(a, 64, 65536, b, b, 4096, CONVROT_BWD_INT8, y, ws), CONVROT_ESHAPE);
  EXPECT(linear_bwd_dx(a, 64, 65536, b, b, 4096, CONVROT_BWD_BF16, y, ws), CONVROT_OK);
  EXPECT(linear_bwd_dx(a, 64, 4096, b, b, 4096, 2, y, ws), CONVROT_EINVAL);
  EXPECT(linear_bwd_dx(a, huge, 4096, b, b, 4096, CONVROT_BWD_BF16, y, ws), CONVROT_ESHAPE);
  EXPECT(linear_bwd_dx(nullptr, 0, 4096, nullptr, nullptr, 4096, 1, nullptr, nullptr), kNoOp);
  EXPECT(dequant_weight_t(a, b, 4096, 4096, y), CONVROT_OK);
  EXPECT(dequant_weight_t(a, odd, 4096, 4096, y), CONVROT_EINVAL);
  EXPECT(dequant_weight_t(a, b, huge, 4096, y), CONVROT_ESHAPE);
  // embedding lookup
  EXPECT(embedding_lookup(a, 64, b, b, 1000, 4096, y, nullptr), CONVROT_OK);
  EXPECT(embedding_lookup(a, 64, b, b, 1000, 4096, y, P((3ul << 20) + 4)), CONVROT_OK);
  EXPECT(embedding_lookup(a, 64, b, b, 1000, 4096, y, P((3ul << 20) + 2)), CONVROT_EINVAL);
  EXPECT(embedding_lookup(odd, 64, b, b, 1000, 4096, y, nullptr), CONVROT_EINVAL);
  EXPECT(embedding_lookup(a, big, b, b, 1000, 4096, y, nullptr), CONVROT_ESHAPE);
  EXPECT(embedding_lookup(nullptr, 0, nullptr, nullptr, 10, 96, nullptr, nullptr), CONVROT_ESHAPE);
  if (failures) return 1;
  printf("ok\n");
  return 0;
}
"""


def _run(cmd, cwd):
    r = subprocess.run(cmd, cwd=cwd, capture_output=True, text=True, timeout=300)
    assert r.returncode == 0, f"{' '.join(map(str, cmd))}\n{r.stdout}\n{r.stderr}"
    return r


def test_oracle_under_asan_ubsan(tmp_path):
    drv = tmp_path / "drv.c"
    exe = tmp_path / "oracle_san"
    drv.write_text(ORACLE_DRIVER)
    _run(["gcc", *SAN, "-std=c11", "-fopenmp", "-fno-fast-math", "-ffp-contract=off",
          os.path.join(ROOT, "oracle", "oracle.c"), str(drv), "-o", str(exe), "-lm"], tmp_path)
    env = dict(os.environ, OMP_NUM_THREADS="4", ASAN_OPTIONS="detect_leaks=1:abort_on_error=1")
    r = subprocess.run([str(exe)], capture_output=True, text=True, timeout=300, env=env)
    assert r.returncode == 0 and r.stdout.strip().endswith("ok"), r.stdout + r.stderr


def test_abi_checks_under_asan_ubsan(tmp_path):
    drv = tmp_path / "drv.cpp"
    exe = tmp_path / "validate_san"
    drv.write_text(VALIDATE_DRIVER)
    _run(["g++", *SAN, "-std=c++17", "-D__HIP_PLATFORM_AMD__", "-I/opt/rocm/include",
          "-I", os.path.join(ROOT, "w8a8_rotated_int8_amd", "csrc"), str(drv), "-o", str(exe)],
         tmp_path)
    r = subprocess.run([str(exe)], capture_output=True, text=True, timeout=120,
                       env=dict(os.environ, ASAN_OPTIONS="abort_on_error=1"))
    assert r.returncode == 0 and r.stdout.strip() == "ok", r.stdout + r.stderr
