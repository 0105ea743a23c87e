/* The C oracle (oracle/liboracle.c) under AddressSanitizer and
 * UndefinedBehaviorSanitizer on the CPU: every routine on small inputs with
 * the edge cases the tests feed it (all-zero groups, signed zeros, subnormal
 * and near-maximal bf16 values, tables with far-apart and equal levels, +inf
 * magnitudes, k a multiple of 32 only), plus a few exact results.  Test
 * infrastructure: built together with liboracle.c and run by
 * tests/test_sanitize.py. */
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

int oracle_dyadic_quantize(const uint16_t* w, int64_t n, int64_t k, uint8_t* idx, uint16_t* scales);
int oracle_dyadic_dequant(const uint8_t* idx, const uint16_t* scales, int64_t n, int64_t k,
                          uint16_t* out);
int oracle_dyadic_matmul(const uint8_t* packed, const uint16_t* scales, const uint16_t* x,
                         int64_t n, int64_t k, int64_t m, double* y);
int oracle_lut16_indices(const uint16_t* w, const uint16_t* scales, const uint16_t* lut, int64_t n,
                         int64_t k, uint8_t* idx);
int oracle_signmag8_indices(const uint16_t* w, const uint16_t* cb, int64_t n, int64_t k,
                            uint8_t* nib);
int oracle_lut16_fit(const uint16_t* w, int64_t n, int64_t k, int iters, uint16_t* scales,
                     uint16_t* lut);
int oracle_signmag8_fit(const uint16_t* w, int64_t n, int64_t k, int iters, uint16_t* cb);
int oracle_num_threads(void);
void oracle_set_num_threads(int n);

static int failures = 0;
#define EXPECT(c)                                                    \
  do {                                                               \
    if (!(c)) {                                                      \
      fprintf(stderr, "FAIL line %d: %s\n", __LINE__, #c);           \
      ++failures;                                                    \
    }                                                                \
  } while (0)

static uint32_t rng = 12345u;
static uint16_t rand16(void) {
  rng = rng * 1103515245u + 12345u;
  return (uint16_t)(rng >> 8);
}

int main(void) {
  enum { N = 5, K = 256 };
  uint16_t w[N * K], s[N * K / 64], s16[N * K / 64], lut[N * K / 64 * 16], cb[N * K / 32 * 8];
  uint16_t deq[N * K], x[3 * K];
  uint8_t idx[N * K], packed[N * K / 2], nib[N * K];
  double y[3 * N];
  for (int i = 0; i < N * K; ++i) {
    uint16_t b = rand16();
    if (((b >> 7) & 0xFF) == 0xFF) b &= 0x807F; /* keep finite */
    w[i] = b;
  }
  memset(w, 0, 64 * sizeof(uint16_t));                 /* all-zero group */
  for (int i = 64; i < 128; ++i) w[i] = 0x8000;        /* -0.0 group */
  for (int i = 128; i < 192; ++i) w[i] = (uint16_t)(1 + i % 127);  /* subnormals */
  w[200] = 0x7F7F;                                     /* largest finite */
  for (int i = 0; i < 3 * K; ++i) x[i] = (uint16_t)(0x3C00 + rand16() % 0x800);

  EXPECT(oracle_dyadic_quantize(w, N, K, idx, s) == 0);
  for (int i = 0; i < 64; ++i) EXPECT(idx[i] == 8 && idx[64 + i] == 8);
  EXPECT(s[0] == 0 && s[1] == 0);
  EXPECT(oracle_dyadic_dequant(idx, s, N, K, deq) == 0);
  for (int i = 0; i < 128; ++i) EXPECT(deq[i] == 0);
  for (int i = 0; i < N * K / 2; ++i) packed[i] = (uint8_t)(idx[2 * i] | (idx[2 * i + 1] << 4));
  EXPECT(oracle_dyadic_matmul(packed, s, x, N, K, 3, y) == 0);
  EXPECT(oracle_dyadic_quantize(w, N, 96, idx, s) == -1);

  for (int i = 0; i < N * K / 64; ++i) s16[i] = (uint16_t)(i % 2 ? 0x3F80 : 0x0001);
  for (int i = 0; i < N * K / 64 * 16; ++i) lut[i] = rand16() & 0xBFFF;
  for (int g = 0; g < N * K / 64; ++g) lut[g * 16 + 3] = lut[g * 16 + 4]; /* equal levels */
  EXPECT(oracle_lut16_indices(w, s16, lut, N, K, idx) == 0);
  for (int i = 0; i < N * K; ++i) EXPECT(idx[i] < 16);

  for (int i = 0; i < N * K / 32 * 8; ++i) cb[i] = rand16() & 0x7FFF;
  for (int i = 0; i < 8; ++i) cb[i] = 0x7C00;          /* a group of only +inf */
  cb[8 + 5] = 0x7C00;
  EXPECT(oracle_signmag8_indices(w, cb, N, K, nib) == 0);
  for (int i = 0; i < 32; ++i) EXPECT((nib[i] & 7) == 0);
  EXPECT(oracle_signmag8_indices(w, cb, N, 96, nib) == 0); /* k a multiple of 32 */
  EXPECT(oracle_signmag8_indices(w, cb, N, 80, nib) == -1);

  for (int iters = 0; iters <= 25; iters += 25) {
    EXPECT(oracle_lut16_fit(w, N, K, iters, s, lut) == 0);
    for (int q = 0; q < 16; ++q) EXPECT(lut[q] == 0); /* all-zero group */
    EXPECT(oracle_signmag8_fit(w, N, K, iters, cb) == 0);
  }
  EXPECT(oracle_signmag8_fit(w, N, 96, 25, cb) == 0);
  oracle_set_num_threads(1);
  EXPECT(oracle_num_threads() == 1);
  EXPECT(oracle_dyadic_quantize(w, N, K, idx, s) == 0);

  if (failures) {
    fprintf(stderr, "%d failures\n", failures);
    return 1;
  }
  printf("oracle_check ok\n");
  return 0;
}
