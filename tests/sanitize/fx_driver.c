/* Driver of the seeded input generator for a sanitizer build (address and undefined
 * behaviour): every entry point on odd sizes, offsets and the edge values of the e4m3 and
 * bf16 encoders, with results checked against the whole-array calls they must equal. */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

void fx_normal_f32(uint64_t seed, uint32_t tid, uint64_t start, uint64_t n, float sigma, float* out);
void fx_normal_bf16(uint64_t seed, uint32_t tid, uint64_t start, uint64_t n, float sigma, uint16_t* out);
void fx_uniform_ids(uint64_t seed, uint32_t tid, uint64_t start, uint64_t n, uint32_t vocab, int32_t* out);
void fx_quant_e4m3_cols(const float* w, int64_t rows, int64_t cols, uint8_t* codes, float* scales);
uint8_t fx_e4m3_encode(float x);
uint16_t fx_bf16_encode(float x);

static int fails = 0;
#define CHECK(c) do { if (!(c)) { fprintf(stderr, "check failed: %s (line %d)\n", #c, __LINE__); ++fails; } } while (0)

int main(void) {
    const uint64_t n = 1001;                       /* odd: the last Box-Muller pair is split */
    float* a = malloc(n * sizeof(float));
    float* b = malloc(n * sizeof(float));
    fx_normal_f32(7, 3, 0, n, 1.0f, a);
    fx_normal_f32(7, 3, 1, n - 1, 1.0f, b);        /* an odd start: same values, shifted */
    CHECK(memcmp(a + 1, b, (n - 1) * sizeof(float)) == 0);
    uint16_t* h = malloc(n * sizeof(uint16_t));
    fx_normal_bf16(7, 3, 0, n, 1.0f, h);
    for (uint64_t i = 0; i < n; ++i) CHECK(h[i] == fx_bf16_encode(a[i]));
    int32_t* ids = malloc(n * sizeof(int32_t));
    fx_uniform_ids(1, 2, 5, n, 1000, ids);
    for (uint64_t i = 0; i < n; ++i) CHECK(ids[i] >= 0 && ids[i] < 1000);
    fx_uniform_ids(1, 2, 0, 0, 1000, ids);          /* empty range */
    /* e4m3 per-column quantisation of a ragged matrix, zero columns included */
    const int64_t rows = 37, cols = 13;
    float* w = calloc(rows * cols, sizeof(float));
    fx_normal_f32(9, 4, 0, rows * (cols - 1), 1.0f, w);   /* last column stays zero */
    uint8_t* q = malloc(rows * cols);
    float* s = malloc(cols * sizeof(float));
    fx_quant_e4m3_cols(w, rows, cols, q, s);
    for (int64_t c = 0; c < cols; ++c) CHECK(s[c] >= 0.0f && isfinite(s[c]));
    /* encoder edge values */
    CHECK(fx_e4m3_encode(0.0f) == 0x00);
    CHECK(fx_e4m3_encode(448.0f) == 0x7E);
    CHECK(fx_e4m3_encode(1e9f) == 0x7E);           /* saturates */
    CHECK(fx_e4m3_encode(-1e9f) == 0xFE);
    CHECK((fx_e4m3_encode(NAN) & 0x7F) == 0x7F);
    CHECK(fx_bf16_encode(1.0f) == 0x3F80);
    CHECK((fx_bf16_encode(NAN) & 0x7FC0) == 0x7FC0);
    free(a); free(b); free(h); free(ids); free(w); free(q); free(s);
    if (fails) return 1;
    printf("fixture generator driver ok\n");
    return 0;
}
