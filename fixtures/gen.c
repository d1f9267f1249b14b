/*
 * Seeded synthetic-input generator.  Shared by the CPU oracle and by the
 * GPU library's callers (tests, bench); it holds none of the denoiser's
 * arithmetic, only the recipe for the random-init weights and inputs.
 *
 * Every value is a pure function of (seed, tensor id, flat index), so any
 * slice of any tensor can be produced on its own, in any order, by any
 * number of threads.
 *
 *   hash   : SplitMix64 output function (Steele, Lea & Flood, OOPSLA 2014)
 *            applied to  seed + (tid * 2^40 + index + 1) * golden-gamma.
 *   normal : Box-Muller on two 24-bit uniforms taken from one 64-bit hash,
 *            single precision (glibc logf / sinf / cosf), element 2j takes
 *            the cosine branch of pair j, element 2j+1 the sine branch.
 *   ids    : multiply-high of the upper 32 hash bits by the vocabulary size.
 *   bf16   : round-to-nearest-even of the float value.
 *   e4m3   : OCP FP8 E4M3 (bias 7, max 448, no infinities), per output
 *            column scale = amax / 448, round-to-nearest-even, saturating.
 */
#include <math.h>
#include <stdint.h>
#include <string.h>

static inline uint64_t fx_hash(uint64_t seed, uint32_t tid, uint64_t index) {
    uint64_t z = seed + (((uint64_t)tid << 40) + index + 1ull) * 0x9E3779B97F4A7C15ull;
    z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
    z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
    return z ^ (z >> 31);
}

static inline float fx_normal_at(uint64_t seed, uint32_t tid, uint64_t idx) {
    uint64_t h = fx_hash(seed, tid, idx >> 1);
    /* (2m+1) * 2^-24 with m < 2^23: exact in float, strictly inside (0,1) */
    float u1 = (float)(((h >> 41) << 1) | 1ull) * 0x1p-24f;
    float u2 = (float)((h >> 8) & 0xFFFFFFull) * 0x1p-24f;
    float r = sqrtf(-2.0f * logf(u1));
    float th = 6.28318530717958647692f * u2;
    return (idx & 1) ? r * sinf(th) : r * cosf(th);
}

static inline uint16_t fx_f32_to_bf16(float f) {
    uint32_t u;
    memcpy(&u, &f, 4);
    if ((u & 0x7fffffffu) > 0x7f800000u) return (uint16_t)((u >> 16) | 0x40u);
    u += 0x7fffu + ((u >> 16) & 1u);
    return (uint16_t)(u >> 16);
}

/* Both Box-Muller branches of one pair share the hash, log and square root. */
static inline void fx_normal_pair(uint64_t seed, uint32_t tid, uint64_t pair, float* c, float* s) {
    uint64_t h = fx_hash(seed, tid, pair);
    float u1 = (float)(((h >> 41) << 1) | 1ull) * 0x1p-24f;
    float u2 = (float)((h >> 8) & 0xFFFFFFull) * 0x1p-24f;
    float r = sqrtf(-2.0f * logf(u1));
    float th = 6.28318530717958647692f * u2;
    *c = r * cosf(th);
    *s = r * sinf(th);
}

#define FX_NORMAL_BODY(STORE)                                                      \
    int64_t i0 = 0;                                                                \
    if ((start & 1) && n > 0) { STORE(0, sigma * fx_normal_at(seed, tid, start)); i0 = 1; } \
    int64_t npairs = ((int64_t)n - i0) / 2;                                        \
    _Pragma("omp parallel for schedule(static)")                                   \
    for (int64_t q = 0; q < npairs; ++q) {                                         \
        float c, sn;                                                               \
        fx_normal_pair(seed, tid, (start + (uint64_t)i0) / 2 + (uint64_t)q, &c, &sn); \
        STORE(i0 + 2 * q, sigma * c);                                              \
        STORE(i0 + 2 * q + 1, sigma * sn);                                         \
    }                                                                              \
    if (i0 + 2 * npairs < (int64_t)n)                                              \
        STORE((int64_t)n - 1, sigma * fx_normal_at(seed, tid, start + n - 1));

void fx_normal_f32(uint64_t seed, uint32_t tid, uint64_t start, uint64_t n, float sigma,
                   float* out) {
#define ST_F32(i, v) (out[(i)] = (v))
    FX_NORMAL_BODY(ST_F32)
#undef ST_F32
}

void fx_normal_bf16(uint64_t seed, uint32_t tid, uint64_t start, uint64_t n, float sigma,
                    uint16_t* out) {
#define ST_BF16(i, v) (out[(i)] = fx_f32_to_bf16(v))
    FX_NORMAL_BODY(ST_BF16)
#undef ST_BF16
}

void fx_uniform_ids(uint64_t seed, uint32_t tid, uint64_t start, uint64_t n, uint32_t vocab,
                    int32_t* out) {
    #pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < (int64_t)n; ++i) {
        uint64_t h = fx_hash(seed, tid, start + (uint64_t)i);
        out[i] = (int32_t)(((h >> 32) * (uint64_t)vocab) >> 32);
    }
}

/* float -> OCP e4m3 code, round-to-nearest-even, saturating to +-448. */
static inline uint8_t fx_f32_to_e4m3(float x) {
    uint8_t sign = signbit(x) ? 0x80 : 0x00;
    float a = fabsf(x);
    if (isnan(x)) return 0x7f;
    if (a >= 0x1p-6f) {
        int e;
        frexpf(a, &e);           /* a = f * 2^e, f in [0.5, 1) */
        e -= 1;                  /* a = 1.m * 2^e */
        float q = nearbyintf(ldexpf(a, 3 - e));   /* in [8, 16] */
        if (q >= 16.0f) { q = 8.0f; e += 1; }
        if (e > 8 || (e == 8 && q > 14.0f)) return (uint8_t)(sign | 0x7e); /* 448 */
        return (uint8_t)(sign | ((e + 7) << 3) | ((int)q - 8));
    }
    float q = nearbyintf(ldexpf(a, 9));           /* subnormal steps of 2^-9 */
    return (uint8_t)(sign | (int)q);              /* q == 8 is the smallest normal */
}

/* Per output column quantisation of a row-major [rows, cols] float matrix. */
void fx_quant_e4m3_cols(const float* w, int64_t rows, int64_t cols, uint8_t* q,
                        float* scales) {
    #pragma omp parallel for schedule(static)
    for (int64_t c = 0; c < cols; ++c) {
        float amax = 0.0f;
        for (int64_t r = 0; r < rows; ++r) amax = fmaxf(amax, fabsf(w[r * cols + c]));
        scales[c] = amax > 0.0f ? amax / 448.0f : 1.0f;
    }
    #pragma omp parallel for schedule(static)
    for (int64_t r = 0; r < rows; ++r)
        for (int64_t c = 0; c < cols; ++c) q[r * cols + c] = fx_f32_to_e4m3(w[r * cols + c] / scales[c]);
}

/* OCP Microscaling (MX) FP4 storage of a [rows][cols] matrix whose rows are the
 * contraction dimension: elements E2M1 (sign, 2 exponent bits with bias 1, 1 mantissa
 * bit; magnitudes 0, 0.5, 1, 1.5, 2, 3, 4, 6), one E8M0 scale 2^(s - 127) per 32
 * consecutive rows of a column.  Per block: X = 2^(floor(log2 amax) - 2) (2 is the largest
 * E2M1 exponent), elements rounded to the nearest E2M1 value of v / X, ties to the even
 * mantissa, saturating at 6; an all-zero block gets s = 0.  codes: [rows][cols / 2], the
 * even column in the low nibble; scales: [rows / 32][cols]. */
static inline uint8_t fx_f32_to_e2m1(float x) {
    static const float mag[8] = {0.0f, 0.5f, 1.0f, 1.5f, 2.0f, 3.0f, 4.0f, 6.0f};
    const uint8_t sign = signbit(x) ? 8 : 0;
    const float a = fabsf(x);
    if (!(a < 6.0f)) return (uint8_t)(7 | sign);          /* saturate (and NaN) */
    int best = 0;
    for (int c = 1; c < 8; ++c) {
        const float dc = fabsf(a - mag[c]), db = fabsf(a - mag[best]);
        if (dc < db || (dc == db && (c & 1) == 0)) best = c;  /* ties: even mantissa */
    }
    return (uint8_t)(best | sign);
}

/* One block of 32 rows of column c: its scale byte, and the exponent e of X = 2^e. */
static inline int fx_mx_block_scale(const float* w, int64_t cols, int64_t b, int64_t c, int* e_out) {
    float amax = 0.0f;
    for (int r = 0; r < 32; ++r) amax = fmaxf(amax, fabsf(w[(b * 32 + r) * cols + c]));
    if (!(amax > 0.0f)) { *e_out = 0; return 0; }
    int ex;
    frexpf(amax, &ex);                                  /* amax = m 2^ex, m in [0.5, 1) */
    int e = ex - 1 - 2;
    if (e < -126) e = -126;
    if (e > 127) e = 127;
    *e_out = e;
    return e + 127;
}

void fx_quant_mxfp4(const float* w, int64_t rows, int64_t cols, uint8_t* codes,
                    uint8_t* scales) {
    const int64_t nb = rows / 32;
    #pragma omp parallel for schedule(static)
    for (int64_t c2 = 0; c2 < cols / 2; ++c2) {
        for (int64_t b = 0; b < nb; ++b) {
            int e[2], sb[2];
            for (int h = 0; h < 2; ++h) {
                sb[h] = fx_mx_block_scale(w, cols, b, 2 * c2 + h, &e[h]);
                scales[b * cols + 2 * c2 + h] = (uint8_t)sb[h];
            }
            for (int r = 0; r < 32; ++r) {
                const int64_t k = b * 32 + r;
                uint8_t q[2];
                for (int h = 0; h < 2; ++h)
                    q[h] = sb[h] ? fx_f32_to_e2m1(ldexpf(w[k * cols + 2 * c2 + h], -e[h])) : 0;
                codes[k * (cols / 2) + c2] = (uint8_t)(q[0] | (q[1] << 4));
            }
        }
    }
}

/* Exposed for the generator's own unit tests. */
uint8_t fx_e4m3_encode(float x) { return fx_f32_to_e4m3(x); }
uint16_t fx_bf16_encode(float x) { return fx_f32_to_bf16(x); }
uint8_t fx_e2m1_encode(float x) { return fx_f32_to_e2m1(x); }
