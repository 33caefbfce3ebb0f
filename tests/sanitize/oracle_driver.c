/* Drives every entry point of oracle/oracle.c under AddressSanitizer and
 * UndefinedBehaviorSanitizer (built by tests/test_sanitizers.py with gcc, on
 * the CPU).  Exits 0 and prints "ok" when every check holds and the
 * sanitizers report nothing (they abort the program on the first report). */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

float oracle_f16_to_f32(uint16_t h);
uint16_t oracle_f32_to_f16(float f);
int64_t oracle_quantize_q8(const float *x, int64_t n, int32_t qa, int8_t *q, float *d);
int64_t oracle_quantize_q8_f16(const float *x, int64_t n, int32_t qa, int8_t *q, float *d);
float oracle_q1_0_row(const uint8_t *blocks, int64_t nb, const int8_t *q, const float *d, int32_t qa);
float oracle_q2_0_row(const uint8_t *blocks, int64_t nb, const int8_t *q, const float *d, int32_t qa);
int oracle_matvec(int fmt, const uint8_t *canon, int64_t rows, int64_t cols, const int8_t *q, const float *d,
                  int32_t qa, int32_t ncols, int64_t ld_q, int64_t ld_d, float *y, int threads);
int oracle_cover_rows(int64_t rows, int threads, int *counts);

static uint64_t st = 0x243F6A8885A308D3ull;
static uint32_t rnd(void)
{
    st = st * 6364136223846793005ull + 1442695040888963407ull;
    return (uint32_t)(st >> 33);
}
static float rnd_normalish(void) { return ((float)(rnd() % 20001) - 10000.0f) / 2500.0f; }

#define CHECK(c)                                                          \
    do {                                                                  \
        if (!(c)) {                                                       \
            fprintf(stderr, "check failed at line %d: %s\n", __LINE__, #c); \
            return 1;                                                     \
        }                                                                 \
    } while (0)

int main(void)
{
    /* f16 widening and narrowing: every non-NaN pattern round-trips */
    for (uint32_t h = 0; h < 65536; ++h) {
        float f = oracle_f16_to_f32((uint16_t)h);
        if (!isnan(f))
            CHECK(oracle_f32_to_f16(f) == (uint16_t)h);
    }
    const int qas[3] = {32, 64, 128};
    const int64_t n = 4096 + 384;
    float *x = malloc(sizeof(float) * n);
    int8_t *q = malloc(n);
    float *d = malloc(sizeof(float) * n / 32);
    for (int64_t i = 0; i < n; ++i)
        x[i] = rnd_normalish();
    for (int i = 0; i < 128; ++i)
        x[i] = 0.0f; /* an all-zero block at every qa */
    for (int k = 0; k < 3; ++k) {
        CHECK(oracle_quantize_q8(x, n, qas[k], q, d) == 0);
        CHECK(d[0] == 0.0f && q[0] == 0);
        oracle_quantize_q8_f16(x, n, qas[k], q, d);
    }
    /* products: every format, ragged shapes, one and several threads agree */
    const int64_t shapes[5][2] = {{1, 1}, {3, 2}, {17, 5}, {100, 10}, {65, 33}};
    for (int fmt = 1; fmt <= 2; ++fmt) {
        const int64_t qk = fmt == 1 ? 128 : 64;
        for (int s = 0; s < 5; ++s) {
            const int64_t rows = shapes[s][0], nb = shapes[s][1], cols = nb * qk;
            uint8_t *w = malloc((size_t)(rows * nb * 18));
            for (int64_t i = 0; i < rows * nb * 18; ++i)
                w[i] = (uint8_t)rnd();
            for (int64_t i = 0; i < rows * nb; ++i) {
                uint16_t h = (uint16_t)(rnd() % 0x7C00); /* finite scales */
                w[i * 18] = (uint8_t)h;
                w[i * 18 + 1] = (uint8_t)(h >> 8);
            }
            const int ncols = 3;
            int8_t *qq = malloc((size_t)(ncols * cols));
            float *dd = malloc(sizeof(float) * (size_t)(ncols * cols / 32));
            for (int64_t i = 0; i < ncols * cols; ++i)
                qq[i] = (int8_t)(rnd() & 0xFF); /* includes -128 */
            for (int64_t i = 0; i < ncols * cols / 32; ++i)
                dd[i] = oracle_f16_to_f32((uint16_t)(rnd() % 0x5C00));
            float *y1 = malloc(sizeof(float) * (size_t)(ncols * rows));
            float *y3 = malloc(sizeof(float) * (size_t)(ncols * rows));
            for (int k = 0; k < 3; ++k) {
                if (cols % qas[k])
                    continue;
                CHECK(oracle_matvec(fmt, w, rows, cols, qq, dd, qas[k], ncols, cols, cols / 32, y1, 1) == 0);
                CHECK(oracle_matvec(fmt, w, rows, cols, qq, dd, qas[k], ncols, cols, cols / 32, y3, 3) == 0);
                CHECK(memcmp(y1, y3, sizeof(float) * (size_t)(ncols * rows)) == 0);
                float r0 = fmt == 1 ? oracle_q1_0_row(w, nb, qq, dd, qas[k]) : oracle_q2_0_row(w, nb, qq, dd, qas[k]);
                CHECK(memcmp(&r0, &y1[0], sizeof r0) == 0);
            }
            CHECK(oracle_matvec(fmt, w, rows, cols + 1, qq, dd, 32, 1, cols, cols / 32, y1, 1) == -1);
            free(w); free(qq); free(dd); free(y1); free(y3);
        }
    }
    /* the row scheduler visits every row once */
    for (int threads = 1; threads <= 5; threads += 2) {
        int counts[1000];
        memset(counts, 0, sizeof counts);
        oracle_cover_rows(1000, threads, counts);
        for (int r = 0; r < 1000; ++r)
            CHECK(counts[r] == 1);
    }
    free(x); free(q); free(d);
    printf("ok\n");
    return 0;
}
