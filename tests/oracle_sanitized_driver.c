/* oracle_sanitized_driver.c — drives every entry of the CPU oracle (oracle/mx_oracle.c) on
 * seeded inputs of ragged sizes, for a build of the oracle with the host AddressSanitizer and
 * UndefinedBehaviorSanitizer (tests/test_oracle_sanitized.py builds and runs it).  Test
 * infrastructure: it checks memory safety and defined behaviour of the oracle, plus a few
 * round trips; the oracle's arithmetic is pinned by the other oracle tests.
 * Exit status 0 when every call returned success and every round trip held. */
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

double orc_bf16_to_double(uint16_t b);
uint16_t orc_double_to_bf16(double v);
double orc_decode(int code, int fmt);
int orc_encode(double v, int fmt);
int orc_encode_many(const double* v, int64_t n, int fmt, uint8_t* out);
int orc_scale_byte(double amax, int fmt);
double orc_scale_value(int byte);
int orc_quantize(const uint16_t* x, int64_t rows, int64_t K, int64_t ldx, int fmt,
                 uint8_t* codes, uint8_t* scales);
int orc_dequantize(const uint8_t* codes, const uint8_t* scales, int64_t rows, int64_t K,
                   int fmt, double* out);
int orc_fp6_pack(const uint8_t* codes, int64_t rows, int64_t K, uint8_t* packed);
int orc_fp6_unpack(const uint8_t* packed, int64_t rows, int64_t K, uint8_t* codes);
int orc_shuffle16(const uint8_t* w, int64_t N, int64_t K, uint8_t* out);
int orc_unshuffle16(const uint8_t* s, int64_t N, int64_t K, uint8_t* w);
void orc_matmul_nt(const double* xd, const double* wd, const double* bias, int64_t M, int64_t N,
                   int64_t K, double* y);
int orc_linear_entries_fmt(const uint8_t* xq, const uint8_t* xs, int xfmt, int64_t K,
                           const uint8_t* wq, const uint8_t* ws, int wfmt, const double* bias,
                           const int64_t* rows, const int64_t* cols, int64_t count, double* out);
int orc_rmsnorm(const uint16_t* x, int64_t rows, int64_t K, int64_t ldx, const uint16_t* gamma,
                double eps, uint16_t* y, double* pre);

static uint64_t g_state = 0x9E3779B97F4A7C15ull;
static uint32_t rnd(void) {   /* xorshift64* */
  g_state ^= g_state >> 12;
  g_state ^= g_state << 25;
  g_state ^= g_state >> 27;
  return (uint32_t)((g_state * 0x2545F4914F6CDD1Dull) >> 32);
}
/* a finite bf16 bit pattern, mostly moderate magnitudes, some zeros and tiny values */
static uint16_t rnd_bf16(void) {
  uint32_t r = rnd();
  if ((r & 31) == 0) return (uint16_t)(r & 0x8000);                 /* signed zero */
  uint32_t e = 100 + (r >> 8) % 60;                                 /* exponents 2^-27 .. 2^32 */
  return (uint16_t)((r & 0x8000) | (e << 7) | ((r >> 16) & 0x7F));
}

static void* xmalloc(size_t n) {
  void* p = malloc(n ? n : 1);
  if (!p) { fprintf(stderr, "out of memory\n"); exit(2); }
  return p;
}

#define CHECK(c) do { if (!(c)) { fprintf(stderr, "check failed line %d: %s\n", __LINE__, #c); return 1; } } while (0)

static int run_case(int64_t M, int64_t N, int64_t K, int64_t pad, int wfmt, int xfmt) {
  const int64_t KB = K / 32, ldx = K + pad;
  uint16_t* x = xmalloc(sizeof(uint16_t) * M * ldx);
  uint16_t* w = xmalloc(sizeof(uint16_t) * N * K);
  uint16_t* gamma = xmalloc(sizeof(uint16_t) * K);
  for (int64_t i = 0; i < M * ldx; ++i) x[i] = rnd_bf16();
  for (int64_t i = 0; i < N * K; ++i) w[i] = rnd_bf16();
  for (int64_t i = 0; i < K; ++i) gamma[i] = rnd_bf16();
  uint8_t *xq = xmalloc(M * K), *xs = xmalloc(M * KB), *wq = xmalloc(N * K), *ws = xmalloc(N * KB);
  CHECK(orc_quantize(x, M, K, ldx, xfmt, xq, xs) == 0);
  CHECK(orc_quantize(w, N, K, K, wfmt, wq, ws) == 0);
  double *xd = xmalloc(sizeof(double) * M * K), *wd = xmalloc(sizeof(double) * N * K);
  CHECK(orc_dequantize(xq, xs, M, K, xfmt, xd) == 0);
  CHECK(orc_dequantize(wq, ws, N, K, wfmt, wd) == 0);
  double* bias = xmalloc(sizeof(double) * N);
  for (int64_t n = 0; n < N; ++n) bias[n] = orc_bf16_to_double(rnd_bf16());
  double* y = xmalloc(sizeof(double) * M * N);
  orc_matmul_nt(xd, wd, bias, M, N, K, y);
  /* sampled entries from the codes equal the full product's */
  int64_t rows[4] = {0, M - 1, M / 2, 0}, cols[4] = {0, N - 1, N / 3, N - 1};
  double e[4];
  CHECK(orc_linear_entries_fmt(xq, xs, xfmt, K, wq, ws, wfmt, bias, rows, cols, 4, e) == 0);
  for (int i = 0; i < 4; ++i) {
    const double ref = y[rows[i] * N + cols[i]];
    CHECK(e[i] == ref || (e[i] - ref) * (e[i] - ref) <= 1e-18 * (ref * ref + 1e-300));
  }
  /* FP6 pack / unpack round trip */
  if (wfmt != 0) {
    uint8_t *pk = xmalloc(N * K / 4 * 3), *back = xmalloc(N * K);
    CHECK(orc_fp6_pack(wq, N, K, pk) == 0);
    CHECK(orc_fp6_unpack(pk, N, K, back) == 0);
    CHECK(memcmp(back, wq, N * K) == 0);
    free(pk);
    free(back);
  }
  /* the pages' (16, 16) shuffle round trip (E4M3 bytes; N % 16 == 0) */
  if (wfmt == 0 && N % 16 == 0) {
    uint8_t *sh = xmalloc(N * K), *back = xmalloc(N * K);
    CHECK(orc_shuffle16(wq, N, K, sh) == 0);
    CHECK(orc_unshuffle16(sh, N, K, back) == 0);
    CHECK(memcmp(back, wq, N * K) == 0);
    free(sh);
    free(back);
  }
  /* the RMS-norm producer, with and without its pre-rounding output */
  uint16_t* yn = xmalloc(sizeof(uint16_t) * M * K);
  double* pre = xmalloc(sizeof(double) * M * K);
  CHECK(orc_rmsnorm(x, M, K, ldx, gamma, 1e-6, yn, pre) == 0);
  CHECK(orc_rmsnorm(x, M, K, ldx, gamma, 0.0, yn, NULL) == 0);
  free(x); free(w); free(gamma); free(xq); free(xs); free(wq); free(ws); free(xd); free(wd);
  free(bias); free(y); free(yn); free(pre);
  return 0;
}

int main(void) {
  /* codec entries over every code and many values */
  for (int fmt = 0; fmt <= 3; ++fmt) {
    if (fmt == 1) continue;
    for (int c = 0; c < 256; ++c) (void)orc_decode(c, fmt);
    double v[1000];
    uint8_t out[1000];
    for (int i = 0; i < 1000; ++i) v[i] = orc_bf16_to_double(rnd_bf16()) * orc_scale_value((int)(rnd() % 255));
    CHECK(orc_encode_many(v, 1000, fmt, out) == 0);
    for (int i = 0; i < 1000; ++i) CHECK(orc_encode(v[i], fmt) == out[i]);
  }
  for (int b = 0; b < 256; ++b) (void)orc_scale_value(b);
  for (uint32_t u = 0; u < 65536; u += 7) {
    const double d = orc_bf16_to_double((uint16_t)u);
    if (d == d) CHECK(orc_double_to_bf16(d) == (uint16_t)u || (d == 0.0));
    (void)orc_scale_byte(d < 0 ? -d : d, 0);
  }
  /* layers of ragged sizes, every weight format, a padded activation stride */
  const int64_t shapes[][4] = {{1, 16, 32, 0}, {3, 48, 96, 8}, {17, 80, 160, 16}, {5, 32, 544, 0}};
  for (size_t s = 0; s < sizeof shapes / sizeof shapes[0]; ++s)
    for (int wfmt = 0; wfmt <= 3; ++wfmt) {
      if (wfmt == 1) continue;
      const int xfmt = (wfmt != 0 && s % 2 == 1) ? wfmt : 0;   /* FP6 activations too */
      if (run_case(shapes[s][0], shapes[s][1], shapes[s][2], shapes[s][3], wfmt, xfmt)) return 1;
    }
  printf("oracle sanitized run ok\n");
  return 0;
}
