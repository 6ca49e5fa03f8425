/*
 * Seeded synthetic-input generator, host side (plain C, OpenMP).
 *
 * This module holds no arithmetic of the decode layer. It turns
 * (seed, tensor tag, layer, sub-stream, element index) into a value through
 * a counter-based hash, so any element can be regenerated on its own and the
 * device-side twin (gen_dev.hip) produces identical bits.
 *
 * Hash: the SplitMix64 output mix of Steele, Lea and Flood ("Fast splittable
 * pseudorandom number generators", OOPSLA 2014), applied to a Weyl sequence.
 * Normal draws: Irwin-Hall sum of the four 16-bit fields of one 64-bit hash,
 * centred and scaled to unit variance (support truncated at +-2*sqrt(3)).
 * The fp32 value is an exact integer times one fp32 scale: a single IEEE
 * multiply, bit-identical on any conforming CPU or GPU.
 */
#include <stdint.h>
#include <string.h>
#include <math.h>

#define SPA_GOLDEN 0x9E3779B97F4A7C15ULL

static inline uint64_t spa_mix64(uint64_t z) {
    z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ULL;
    z = (z ^ (z >> 27)) * 0x94D049BB133111EBULL;
    return z ^ (z >> 31);
}

uint64_t spa_gen_stream_key(uint64_t seed, uint32_t tag, uint32_t layer, uint32_t sub) {
    uint64_t k = spa_mix64(seed + SPA_GOLDEN);
    k = spa_mix64(k ^ (((uint64_t)tag << 32) | (uint64_t)layer));
    k = spa_mix64(k ^ ((uint64_t)sub + SPA_GOLDEN));
    return k;
}

static inline uint64_t spa_elem(uint64_t key, uint64_t i) {
    return spa_mix64(key + (i + 1ULL) * SPA_GOLDEN);
}

static inline int32_t spa_ih4(uint64_t h) {
    uint32_t s = (uint32_t)(h & 0xFFFFu) + (uint32_t)((h >> 16) & 0xFFFFu) +
                 (uint32_t)((h >> 32) & 0xFFFFu) + (uint32_t)(h >> 48);
    return (int32_t)s - 131070;
}

/* fp32 -> bf16 bits, round to nearest even (inputs here are finite). */
static inline uint16_t spa_f32_to_bf16_rne(float f) {
    uint32_t u;
    memcpy(&u, &f, 4);
    u += 0x7FFFu + ((u >> 16) & 1u);
    return (uint16_t)(u >> 16);
}

/* scale that maps an Irwin-Hall(4) integer to a unit-variance draw times std */
float spa_gen_normal_scale(double std_dev) {
    return (float)(std_dev * sqrt(3.0) / 65536.0);
}

void spa_gen_normal_f32(float* out, int64_t n, uint64_t key, int64_t i0, float scale) {
    #pragma omp parallel for schedule(static)
    for (int64_t j = 0; j < n; ++j)
        out[j] = (float)spa_ih4(spa_elem(key, (uint64_t)(i0 + j))) * scale;
}

void spa_gen_normal_bf16(uint16_t* out, int64_t n, uint64_t key, int64_t i0, float scale) {
    #pragma omp parallel for schedule(static)
    for (int64_t j = 0; j < n; ++j)
        out[j] = spa_f32_to_bf16_rne((float)spa_ih4(spa_elem(key, (uint64_t)(i0 + j))) * scale);
}

/* integers uniform in [lo, hi] (modulo reduction of the 64-bit hash) */
void spa_gen_uniform_int(int32_t* out, int64_t n, uint64_t key, int64_t i0, int32_t lo, int32_t hi) {
    uint64_t span = (uint64_t)((int64_t)hi - (int64_t)lo + 1);
    for (int64_t j = 0; j < n; ++j)
        out[j] = lo + (int32_t)(spa_elem(key, (uint64_t)(i0 + j)) % span);
}

/*
 * OCP FP8 E4M3 (bias 7, max finite 448, no infinities, S.1111.111 = NaN):
 * round-to-nearest-even of a finite fp32, saturating to +-448. Used only to
 * prepare fp8 weight inputs offline.
 */
static uint8_t spa_f32_to_e4m3_rne_sat(float f) {
    uint32_t u;
    memcpy(&u, &f, 4);
    uint8_t sign = (uint8_t)((u >> 24) & 0x80u);
    float a = fabsf(f);
    if (a >= 448.0f) return sign | 0x7Eu;
    if (a < 0.0009765625f) {          /* below half the smallest subnormal 2^-9: */
        /* subnormal range handled below; exact zero region */
    }
    /* find the quantum for a: normal exponent e = floor(log2 a), min normal 2^-6 */
    int e;
    frexpf(a, &e);                    /* a = m * 2^e, m in [0.5, 1) */
    e -= 1;                           /* a in [2^e, 2^(e+1)) */
    if (e < -6) e = -6;               /* subnormals share the 2^-9 quantum */
    float q = ldexpf(1.0f, e - 3);    /* 3 mantissa bits */
    float r = a / q;                  /* exact: q is a power of two */
    float fl = floorf(r);
    float rem = r - fl;
    float n;
    if (rem > 0.5f) n = fl + 1.0f;
    else if (rem < 0.5f) n = fl;
    else n = (fmodf(fl, 2.0f) == 0.0f) ? fl : fl + 1.0f;
    float v = n * q;
    if (v >= 448.0f) return sign | 0x7Eu;
    if (v == 0.0f) return sign;
    /* encode v */
    int ev;
    frexpf(v, &ev);
    ev -= 1;
    if (ev < -6) {                    /* subnormal: v = mant * 2^-9 */
        int mant = (int)(v / ldexpf(1.0f, -9));
        return sign | (uint8_t)mant;
    }
    int mant = (int)(v / ldexpf(1.0f, ev - 3)) - 8;
    return sign | (uint8_t)(((ev + 7) << 3) | mant);
}

static float spa_e4m3_to_f32(uint8_t c) {
    int s = c >> 7, e = (c >> 3) & 15, m = c & 7;
    float v = (e == 0) ? ldexpf((float)m, -9) : ldexpf((float)(8 + m), e - 10);
    return s ? -v : v;
}

/*
 * Per-output-channel fp8 weights: for each of `rows` rows of length `cols`
 * (fp32 input), scale = amax/448 and code = E4M3(w / scale).
 */
void spa_quant_rows_e4m3(const float* w, int64_t rows, int64_t cols, uint8_t* codes, float* scales) {
    #pragma omp parallel for schedule(static)
    for (int64_t r = 0; r < rows; ++r) {
        const float* wr = w + r * cols;
        float amax = 0.0f;
        for (int64_t c = 0; c < cols; ++c) { float a = fabsf(wr[c]); if (a > amax) amax = a; }
        float sc = amax > 0.0f ? amax / 448.0f : 1.0f;
        scales[r] = sc;
        for (int64_t c = 0; c < cols; ++c) codes[r * cols + c] = spa_f32_to_e4m3_rne_sat(wr[c] / sc);
    }
}

/* decode helper exposed for the generator's own self-check */
void spa_e4m3_decode(const uint8_t* codes, int64_t n, float* out) {
    for (int64_t i = 0; i < n; ++i) out[i] = spa_e4m3_to_f32(codes[i]);
}
