"""The oracle's C code under AddressSanitizer and UndefinedBehaviorSanitizer
(host code only; CPU).

A small C driver calls every function of oracle/f8ref.c on edge shapes --
empty, single-element, odd lengths, ragged rectangles -- with buffers of
exactly the size each function may touch, so an out-of-bounds read or write,
a signed overflow, or a shift past the width aborts the run.  The driver
also checks a few results that the format definitions fix (the OCP OFP8
maxima, the sign of zero, saturation of infinities, exact amax), so that a
sanitized build that computes nonsense fails too.
"""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = os.path.join(ROOT, "oracle", "f8ref.c")

DRIVER = r"""
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

float oracle_bf16_to_f32(uint16_t b);
double oracle_fp8_decode(uint8_t code, int fmt);
uint8_t oracle_fp8_encode(float v, int fmt);
float oracle_amax(const uint16_t *x, int64_t n);
void oracle_scale(float amax, int fmt, float *scale, float *inv_scale);
int64_t oracle_cast(const uint16_t *x, int64_t rows, int64_t cols, int fmt, float scale, uint8_t *q, uint8_t *qt);
void oracle_encode_f32(const float *v, int64_t n, int fmt, uint8_t *q);
void oracle_encode_bits_range(uint32_t lo, uint32_t count, int fmt, uint8_t *q);
float oracle_history_amax(const float *hist);
void oracle_history_push(float *hist, int32_t *count, int32_t *pos, float amax_now);

#define CHECK(c) do { if (!(c)) { fprintf(stderr, "check failed line %d: %s\n", __LINE__, #c); return 1; } } while (0)

static uint16_t *bf16_buf(int64_t n, unsigned seed) {
  uint16_t *x = (uint16_t *)malloc((size_t)(n > 0 ? n : 1) * sizeof(uint16_t));
  for (int64_t i = 0; i < n; ++i) {
    seed = seed * 1103515245u + 12345u;
    uint16_t b = (uint16_t)(seed >> 16);
    if ((b & 0x7F80u) == 0x7F80u) b &= 0xBFFFu; /* keep it finite */
    x[i] = b;
  }
  return x;
}

int main(void) {
  for (int fmt = 0; fmt < 2; ++fmt)
    for (int c = 0; c < 256; ++c) (void)oracle_fp8_decode((uint8_t)c, fmt);
  CHECK(oracle_fp8_decode(0x7E, 0) == 448.0);
  CHECK(oracle_fp8_decode(0x7B, 1) == 57344.0);
  CHECK(oracle_fp8_encode(INFINITY, 0) == 0x7E && oracle_fp8_encode(-INFINITY, 1) == 0xFB);
  CHECK(oracle_fp8_encode(-0.0f, 0) == 0x80 && oracle_fp8_encode(0.0f, 1) == 0x00);
  CHECK(oracle_fp8_encode(1e-30f, 0) == 0x00);
  {
    const float sp[] = {NAN, -NAN, 1e38f, -1e38f, 1.4e-45f, 2e-3f, 448.0f, 464.0f, 57344.0f, 61440.0f};
    uint8_t q[sizeof sp / sizeof sp[0]];
    for (int fmt = 0; fmt < 2; ++fmt) oracle_encode_f32(sp, (int64_t)(sizeof sp / sizeof sp[0]), fmt, q);
    oracle_encode_f32(sp, 0, 0, q);
  }
  {
    uint8_t *q = (uint8_t *)malloc(4096);
    oracle_encode_bits_range(0xFFFFF000u, 4096u, 0, q); /* the last patterns, up to 0xFFFFFFFF */
    oracle_encode_bits_range(0x7F7FF800u, 4096u, 1, q);
    free(q);
  }
  {
    CHECK(oracle_amax(NULL, 0) == 0.0f);
    const int64_t ns[] = {1, 2, 7, 8, 9, 1023, 4097};
    for (size_t k = 0; k < sizeof ns / sizeof ns[0]; ++k) {
      uint16_t *x = bf16_buf(ns[k], (unsigned)k + 1u);
      float want = 0.0f;
      for (int64_t i = 0; i < ns[k]; ++i) want = fmaxf(want, fabsf(oracle_bf16_to_f32(x[i])));
      CHECK(oracle_amax(x, ns[k]) == want);
      x[ns[k] - 1] = 0x7FC0u; /* NaN at the last index */
      CHECK(isnan(oracle_amax(x, ns[k])));
      free(x);
    }
  }
  {
    const float am[] = {0.0f, 1e-30f, 1.0f, 448.0f, 3e38f, INFINITY, NAN};
    for (size_t k = 0; k < sizeof am / sizeof am[0]; ++k)
      for (int fmt = 0; fmt < 2; ++fmt) {
        float s = 0.0f, inv = 0.0f;
        oracle_scale(am[k], fmt, &s, &inv);
      }
    float s = 0.0f, inv = 0.0f;
    oracle_scale(448.0f, 0, &s, &inv);
    CHECK(s == 1.0f && inv == 1.0f);
  }
  {
    const int64_t shapes[][2] = {{0, 5}, {5, 0}, {1, 1}, {3, 5}, {17, 33}, {128, 129}, {130, 16}};
    for (size_t k = 0; k < sizeof shapes / sizeof shapes[0]; ++k) {
      const int64_t r = shapes[k][0], c = shapes[k][1], n = r * c;
      uint16_t *x = bf16_buf(n, 99u + (unsigned)k);
      uint8_t *q = (uint8_t *)malloc((size_t)(n > 0 ? n : 1));
      uint8_t *qt = (uint8_t *)malloc((size_t)(n > 0 ? n : 1));
      for (int fmt = 0; fmt < 2; ++fmt) {
        float s = 0.0f, inv = 0.0f;
        oracle_scale(oracle_amax(x, n), fmt, &s, &inv);
        CHECK(oracle_cast(x, r, c, fmt, s, q, qt) == 0); /* s from the tensor's own amax: nothing saturates */
        for (int64_t i = 0; i < r; ++i)
          for (int64_t j = 0; j < c; ++j) CHECK(qt[j * r + i] == q[i * c + j]);
        (void)oracle_cast(x, r, c, fmt, s * 4.0f, q, NULL);
      }
      free(x);
      free(q);
      free(qt);
    }
  }
  {
    float hist[16] = {0};
    int32_t count = 0, pos = 0;
    for (int t = 0; t < 40; ++t) {
      oracle_history_push(hist, &count, &pos, (float)(t + 1));
      CHECK(count == (t + 1 < 16 ? t + 1 : 16) && pos == (t + 1) % 16);
    }
    CHECK(oracle_history_amax(hist) == 40.0f);
    hist[3] = NAN;
    CHECK(isnan(oracle_history_amax(hist)));
  }
  printf("ok\n");
  return 0;
}
"""


@pytest.mark.skipif(shutil.which("gcc") is None, reason="needs gcc")
def test_oracle_c_under_asan_and_ubsan(tmp_path):
    drv = tmp_path / "driver.c"
    drv.write_text(DRIVER)
    exe = tmp_path / "driver"
    cmd = ["gcc", "-std=c99", "-O1", "-g", "-fno-omit-frame-pointer", "-ffp-contract=off",
           "-fsanitize=address,undefined", "-fno-sanitize-recover=all",
           "-Wall", "-Wno-unknown-pragmas", "-o", str(exe), str(drv), SRC, "-lm"]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0 and "asan" in r.stderr.lower():
        pytest.skip("the sanitizer runtimes are not installed: " + r.stderr[-300:])
    assert r.returncode == 0, r.stderr
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=0",
               UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1")
    r = subprocess.run([str(exe)], capture_output=True, text=True, env=env, timeout=120)
    assert r.returncode == 0 and r.stdout.strip() == "ok", (r.stdout, r.stderr)
    assert "runtime error" not in r.stderr, r.stderr
