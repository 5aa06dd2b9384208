/*
 * sanitize_driver.c — drives every entry point of the oracle (lq_oracle.c) over
 * every descriptor combination on small seeded inputs, so that a build with
 * the address and undefined-behaviour sanitizers can check the oracle's host
 * code. TEST INFRASTRUCTURE ONLY, like the oracle itself.
 *
 * Prints one line, "digest <hex> nonfinite <hex> calls <n>": FNV-1a hashes
 * over every output byte, so a sanitized build and a plain one can be
 * compared. The first covers the number formats and a pass over inputs that
 * mix normal values, zeros of both signs, subnormals and large magnitudes.
 * The second covers a pass that adds NaN and infinities: outside the
 * quantizer's contract, they must still not reach undefined behaviour, but
 * which NaN a binary32 operation propagates (payload, sign) may follow the
 * compiler's operand order, so that hash need not match across builds.
 *
 *   gcc -O1 -g -fsanitize=address,undefined,float-cast-overflow \
 *       -fno-sanitize-recover=all oracle/sanitize_driver.c oracle/lq_oracle.c -lm
 */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include "lq_oracle.h"

static uint64_t g_hash = 1469598103934665603ull;
static long g_calls = 0;

static void mix(const void* p, size_t n) {
  const unsigned char* b = (const unsigned char*)p;
  for (size_t i = 0; i < n; i++) {
    g_hash ^= b[i];
    g_hash *= 1099511628211ull;
  }
}

/* xorshift64*: a fixed, seeded stream of test values */
static uint64_t g_state = 0x9E3779B97F4A7C15ull;
static uint64_t next_u64(void) {
  g_state ^= g_state >> 12;
  g_state ^= g_state << 25;
  g_state ^= g_state >> 27;
  return g_state * 2685821657736338717ull;
}
static float next_value(int with_nonfinite) {
  const uint64_t r = next_u64();
  const int pick = (int)(r % 16);
  const float u = (float)((r >> 11) & 0xFFFFF) / (float)0x100000 - 0.5f;   /* [-0.5, 0.5) */
  switch (pick) {
    case 0: return 0.0f;
    case 1: return -0.0f;
    case 2: return 1e-40f * (u + 0.75f);                 /* subnormal */
    case 3: return ldexpf(u, 100);                        /* large */
    case 4: return ldexpf(u, -60);                        /* tiny */
    case 5: return with_nonfinite ? NAN : 2.5f;
    case 6: return with_nonfinite ? (u < 0 ? -INFINITY : INFINITY) : -3.5f;
    default: return ldexpf(u, (int)(r >> 60) - 4);
  }
}

static void run_variant(const or_desc* d, const float* x, int64_t rows, int64_t cols) {
  const int64_t n = rows * cols;
  uint8_t* codes = calloc((size_t)n + 16, 1);
  uint8_t* scales = calloc((size_t)n * 4 + 64, 1);
  uint8_t* zeros = calloc((size_t)n * 4 + 64, 1);
  float* xhat = calloc((size_t)n, sizeof(float));
  uint32_t* y = calloc((size_t)n, 4);
  uint32_t* y2 = calloc((size_t)n, 4);
  float tstat[3], ts = 1.0f;
  double e2 = 0.0, s2 = 0.0;
  or_tensor_stat(d, x, rows, cols, tstat);
  const int rc = or_fake_quant_rows(d, x, rows, cols, tstat, &ts, codes, scales, zeros, xhat, y, &e2, &s2);
  g_calls++;
  mix(&rc, sizeof rc);
  if (rc == 0) {
    mix(codes, (size_t)n);
    mix(scales, (size_t)n * 4);
    mix(zeros, (size_t)n * 4);
    mix(xhat, (size_t)n * sizeof(float));
    mix(y, (size_t)n * 4);
    mix(&e2, sizeof e2);
    mix(&s2, sizeof s2);
    mix(&ts, sizeof ts);
    /* the stored codes and scales back through the dequantizer, and once more
       through the quantizer as given scales */
    or_desc g = *d;
    g.given_scales = 1;
    mix(&rc, sizeof rc);
    if (or_dequant_rows(&g, codes, scales, zeros, ts, rows, cols, y2) == 0) mix(y2, (size_t)n * 4);
    double e3 = 0.0, s3 = 0.0;
    if (or_fake_quant_rows(&g, x, rows, cols, tstat, &ts, codes, scales, zeros, xhat, y2, &e3, &s3) == 0)
      mix(&e3, sizeof e3);
    g_calls += 2;
  }
  free(codes);
  free(scales);
  free(zeros);
  free(xhat);
  free(y);
  free(y2);
}

int main(void) {
  /* number formats: every code of every kind, encodes around each code */
  for (int k = ORK_E4M3; k <= ORK_E3M2; k++) {
    const uint32_t ncodes = (k == ORK_FP16 || k == ORK_BF16) ? 65536u : 256u;
    for (uint32_t c = 0; c < ncodes; c++) {
      const double v = or_fp_decode(k, c);
      const uint32_t e0 = or_fp_encode(k, v, 1), e1 = or_fp_encode(k, v * 1.0625, 0);
      mix(&v, sizeof v);
      mix(&e0, sizeof e0);
      mix(&e1, sizeof e1);
    }
    const double m = or_fp_max(k);
    mix(&m, sizeof m);
  }
  for (int i = -300; i <= 300; i++) {
    const int e = or_ue8m0_exponent(ldexp(1.3, i), 127.0);
    const double r0 = or_round_int(i * 0.5, OR_RNE), r1 = or_round_int(i * 0.5, OR_RNA);
    mix(&e, sizeof e);
    mix(&r0, sizeof r0);
    mix(&r1, sizeof r1);
  }
  uint32_t signs[64];
  for (int i = 0; i < 64; i++) signs[i] = (uint32_t)next_u64();
  for (int n = 16; n <= 1024; n *= 2) {
    float v[1024];
    for (int i = 0; i < n; i++) v[i] = next_value(0);
    or_rotate(v, n, signs, 1024);
    or_unrotate(v, n, signs, 1024);
    mix(v, sizeof(float) * (size_t)n);
  }
  double table[3 * 25];
  for (int i = 0; i < 3 * 25; i++) table[i] = 20.0 + (double)(next_u64() % 1000) * 0.001;
  table[7] = NAN;
  table[8] = INFINITY;
  int32_t counts[60];
  if (or_sweep_tally(table, 3, 0.01, 0.002, counts) == 0) mix(counts, sizeof counts);

  /* the quantizer: every descriptor combination, valid or not */
  static const int hads[] = {0, 16, 64, 1024};
  static const int tile_rows[] = {1, 3};
  uint64_t finite_hash = 0;
  for (int pass = 0; pass < 2; pass++) {
    const int64_t rows = 3, cols = 1024;
    float* x = malloc(sizeof(float) * (size_t)(rows * cols));
    for (int64_t i = 0; i < rows * cols; i++) x[i] = next_value(pass);
    for (int fmt = OR_INT8; fmt <= OR_E3M2; fmt++)
      for (int gran = OR_TENSOR; gran <= OR_TILE; gran++)
        for (int sf = OR_S_F32; sf <= OR_S_E4M3; sf++)
          for (int sym = 0; sym <= 1; sym++)
            for (int rnd = OR_RNE; rnd <= OR_RNA; rnd++)
              for (int h = 0; h < 4; h++)
                for (int two = 0; two <= 1; two++)
                  for (int tr = 0; tr < (gran == OR_TILE ? 2 : 1); tr++) {
                    or_desc d;
                    memset(&d, 0, sizeof d);
                    d.fmt = fmt;
                    d.gran = gran;
                    d.block = (gran == OR_BLOCK || gran == OR_TILE) ? 32 : 0;
                    d.scale_fmt = sf;
                    d.symmetric = sym;
                    d.rounding = rnd;
                    d.out_dtype = (fmt + sf + h) % 3;
                    d.hadamard = hads[h];
                    d.unrotate_y = h & 1;
                    d.two_level = two;
                    d.tile_rows = tile_rows[tr];
                    d.signs = (h == 3) ? signs : NULL;
                    run_variant(&d, x, rows, cols);
                  }
    free(x);
    if (pass == 0) {
      finite_hash = g_hash;
      g_hash = 1469598103934665603ull;
    }
  }
  printf("digest %016llx nonfinite %016llx calls %ld\n", (unsigned long long)finite_hash,
         (unsigned long long)g_hash, g_calls);
  return 0;
}
