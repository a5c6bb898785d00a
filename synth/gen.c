/*
 * Seeded synthetic inputs for the W4A16 verify linear.
 *
 * This file produces the *inputs* that both the CPU oracle and the GPU
 * library consume: Gaussian weights quantised to the canonical packed uint4
 * format, and Gaussian activations rounded to bf16.  It contains none of the
 * verify GEMM's arithmetic (no unpacking, no dequantisation, no products).
 *
 * Random numbers: Philox4x64-10, the counter-based generator of Salmon,
 * Moraes, Dror and Shaw, "Parallel Random Numbers: As Easy as 1, 2, 3"
 * (SC 2011).  Block b of a stream keyed by `key` is Philox4x64-10 applied to
 * the counter (b, 0, 0, 0); numpy.random.Philox with the same key and counter
 * b-1 returns the same four words (numpy increments before it generates),
 * which the generator tests check.  Every output element is a pure function
 * of (key, element index), so the thread decomposition never changes values.
 *
 * Normals: Box-Muller on two 24-bit uniforms taken from one 64-bit word
 * (u1 from bits 40..63, shifted by half an ulp so it is never 0; u2 from
 * bits 8..31).  Word w of block b gives elements 8b+2w (cosine branch) and
 * 8b+2w+1 (sine branch).
 *
 * Quantiser (per output column n and group G of `group` consecutive k):
 *   wmin, wmax over the group (fp32); s = fp16_rne((wmax - wmin) / 15),
 *   widened back to fp32; s == 0 -> s = 2^-14;
 *   z = clamp(rint(-wmin / s), 0, 15); q = clamp(rint(w / s) + z, 0, 15),
 *   rint = round half to even, all in fp32.
 *
 * Canonical packed format (the library's and the oracle's input):
 *   qweight int32 [K/8][N]: bits [4i, 4i+4) of word (j, n) hold q[8j+i][n];
 *   scales  uint16 [K/g][N]: fp16 bit patterns;
 *   zeros   int32 [K/g][N/8]: bits [4i, 4i+4) of word (G, j) hold z[G][8j+i].
 *
 * Built with gcc into libw4synth.so; called from synth/__init__.py.
 */
#include <math.h>
#include <pthread.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

/* ---------------- Philox4x64-10 ---------------- */

#define PHILOX_M0 0xD2E7470EE14C6C93ULL
#define PHILOX_M1 0xCA5A826395121157ULL
#define PHILOX_W0 0x9E3779B97F4A7C15ULL
#define PHILOX_W1 0xBB67AE8584CAA73BULL

static inline void mulhilo64(uint64_t a, uint64_t b, uint64_t* hi, uint64_t* lo) {
    __uint128_t p = (__uint128_t)a * (__uint128_t)b;
    *hi = (uint64_t)(p >> 64);
    *lo = (uint64_t)p;
}

static inline void philox4x64_10(const uint64_t ctr_in[4], const uint64_t key_in[2], uint64_t out[4]) {
    uint64_t c0 = ctr_in[0], c1 = ctr_in[1], c2 = ctr_in[2], c3 = ctr_in[3];
    uint64_t k0 = key_in[0], k1 = key_in[1];
    for (int r = 0; r < 10; ++r) {
        if (r > 0) {
            k0 += PHILOX_W0;
            k1 += PHILOX_W1;
        }
        uint64_t hi0, lo0, hi1, lo1;
        mulhilo64(PHILOX_M0, c0, &hi0, &lo0);
        mulhilo64(PHILOX_M1, c2, &hi1, &lo1);
        uint64_t n0 = hi1 ^ c1 ^ k0;
        uint64_t n1 = lo1;
        uint64_t n2 = hi0 ^ c3 ^ k1;
        uint64_t n3 = lo0;
        c0 = n0; c1 = n1; c2 = n2; c3 = n3;
    }
    out[0] = c0; out[1] = c1; out[2] = c2; out[3] = c3;
}

/* Raw Philox block, exposed so the generator can be checked against numpy. */
void w4s_philox_block(uint64_t key0, uint64_t key1, uint64_t block, uint64_t out[4]) {
    uint64_t ctr[4] = {block, 0, 0, 0};
    uint64_t key[2] = {key0, key1};
    philox4x64_10(ctr, key, out);
}

/* Key of the stream for a user seed: the seed and a fixed tag word. */
#define STREAM_TAG 0x57344131364D4131ULL

static inline void box_muller_pair(uint64_t r, float* z0, float* z1) {
    const float two_m24 = 5.9604644775390625e-08f; /* 2^-24 */
    float u1 = ((float)(uint32_t)(r >> 40) + 0.5f) * two_m24;
    float u2 = (float)(uint32_t)((r >> 8) & 0xFFFFFFu) * two_m24;
    float rad = sqrtf(-2.0f * logf(u1));
    float th = 6.28318530717958647692f * u2;
    *z0 = rad * cosf(th);
    *z1 = rad * sinf(th);
}

/* Normals for elements [e0, e0 + count) of the stream `seed`, times `scale`. */
static void normals_range(uint64_t seed, uint64_t e0, size_t count, float scale, float* out) {
    uint64_t key[2] = {seed, STREAM_TAG};
    size_t i = 0;
    while (i < count) {
        uint64_t e = e0 + i;
        uint64_t b = e >> 3;
        uint64_t ctr[4] = {b, 0, 0, 0};
        uint64_t r[4];
        philox4x64_10(ctr, key, r);
        float z[8];
        for (int w = 0; w < 4; ++w) box_muller_pair(r[w], &z[2 * w], &z[2 * w + 1]);
        for (unsigned t = (unsigned)(e & 7); t < 8 && i < count; ++t, ++i) out[i] = z[t] * scale;
    }
}

void w4s_normals(uint64_t seed, uint64_t e0, size_t count, float scale, float* out) {
    normals_range(seed, e0, count, scale, out);
}

/* ---------------- fp16 / bf16 rounding (round to nearest even) ---------------- */

/* fp32 -> fp16 bit pattern, round to nearest even; finite inputs only
 * (overflow saturates to infinity, which the quantiser never reaches). */
static uint16_t f32_to_f16_rne(float f) {
    uint32_t u;
    memcpy(&u, &f, 4);
    uint32_t sign = (u >> 16) & 0x8000u;
    uint32_t absu = u & 0x7FFFFFFFu;
    if (absu >= 0x477FF000u) return (uint16_t)(sign | 0x7C00u); /* rounds to >= 65520 -> inf */
    if (absu < 0x38800000u) {                                   /* below 2^-14: subnormal fp16 */
        /* value = absf; fp16 subnormal unit is 2^-24 */
        float a;
        memcpy(&a, &absu, 4);
        float scaled = a * 16777216.0f; /* exact: multiply by 2^24 */
        float r = rintf(scaled);        /* round half even in the default mode */
        return (uint16_t)(sign | (uint32_t)r);
    }
    uint32_t mant = absu & 0x7FFFFFu;
    int32_t exp = (int32_t)(absu >> 23) - 127 + 15;
    uint32_t half = ((uint32_t)exp << 10) | (mant >> 13);
    uint32_t rem = mant & 0x1FFFu;
    if (rem > 0x1000u || (rem == 0x1000u && (half & 1u))) half += 1; /* carry may bump exponent: fine */
    return (uint16_t)(sign | half);
}

static float f16_to_f32(uint16_t h) {
    uint32_t sign = ((uint32_t)h & 0x8000u) << 16;
    uint32_t e = (h >> 10) & 0x1Fu;
    uint32_t m = h & 0x3FFu;
    float r;
    if (e == 0) {
        r = (float)m * 5.9604644775390625e-08f; /* m * 2^-24, exact */
        uint32_t u;
        memcpy(&u, &r, 4);
        u |= sign;
        memcpy(&r, &u, 4);
        return r;
    }
    uint32_t u = sign | ((e - 15 + 127) << 23) | (m << 13);
    memcpy(&r, &u, 4);
    return r;
}

uint16_t w4s_f32_to_f16(float f) { return f32_to_f16_rne(f); }
float w4s_f16_to_f32(uint16_t h) { return f16_to_f32(h); }

/* fp32 -> bf16 bits, round to nearest even (no NaNs occur). */
static inline uint16_t f32_to_bf16_rne(float f) {
    uint32_t u;
    memcpy(&u, &f, 4);
    u += 0x7FFFu + ((u >> 16) & 1u);
    return (uint16_t)(u >> 16);
}

/* ---------------- quantiser ---------------- */

static inline float clamp15(float v) { return v < 0.0f ? 0.0f : (v > 15.0f ? 15.0f : v); }

/* Quantise one group of `g` weights: writes q[0..g) and returns (s bits, z). */
static void quantize_group(const float* w, int g, uint8_t* q, uint16_t* s_bits, uint8_t* zq) {
    float wmin = w[0], wmax = w[0];
    for (int i = 1; i < g; ++i) {
        if (w[i] < wmin) wmin = w[i];
        if (w[i] > wmax) wmax = w[i];
    }
    uint16_t sb = f32_to_f16_rne((wmax - wmin) / 15.0f);
    float s = f16_to_f32(sb);
    if (s == 0.0f) {
        sb = 0x0400u; /* 2^-14 */
        s = f16_to_f32(sb);
    }
    float z = clamp15(rintf(-wmin / s));
    for (int i = 0; i < g; ++i) q[i] = (uint8_t)clamp15(rintf(w[i] / s) + z);
    *s_bits = sb;
    *zq = (uint8_t)z;
}

/* Quantise rows [n0, n1) of W (fp32 [N][K] row-major, or generated on the fly
 * when W == NULL) and write them into the canonical packed arrays. n0 and n1
 * are multiples of 8 so that no zeros word is shared between callers. */
static void quantize_rows(const float* W, uint64_t seed, float stddev, int N, int K, int g, int n0, int n1,
                          int32_t* qweight, uint16_t* scales, int32_t* zeros) {
    const int KG = K / g;
    float* row = (float*)malloc(sizeof(float) * (size_t)K * 8);
    uint8_t* qrow = (uint8_t*)malloc((size_t)K * 8);
    uint8_t* zrow = (uint8_t*)malloc((size_t)KG * 8);
    for (int nb = n0; nb < n1; nb += 8) {
        int rows = (n1 - nb) < 8 ? (n1 - nb) : 8;
        for (int r = 0; r < rows; ++r) {
            int n = nb + r;
            float* wr = row + (size_t)r * K;
            if (W)
                memcpy(wr, W + (size_t)n * K, sizeof(float) * (size_t)K);
            else
                normals_range(seed, (uint64_t)n * (uint64_t)K, (size_t)K, stddev, wr);
            for (int G = 0; G < KG; ++G) {
                uint16_t sb;
                quantize_group(wr + (size_t)G * g, g, qrow + (size_t)r * K + (size_t)G * g, &sb,
                               zrow + (size_t)r * KG + G);
                scales[(size_t)G * N + n] = sb;
            }
        }
        /* pack q along K: word (j, n), nibble i <- q[8j+i][n] */
        for (int r = 0; r < rows; ++r) {
            int n = nb + r;
            const uint8_t* qr = qrow + (size_t)r * K;
            for (int j = 0; j < K / 8; ++j) {
                uint32_t word = 0;
                for (int i = 0; i < 8; ++i) word |= (uint32_t)qr[8 * j + i] << (4 * i);
                qweight[(size_t)j * N + n] = (int32_t)word;
            }
        }
        /* pack z along N: word (G, nb/8), nibble i <- z[G][nb+i] */
        for (int G = 0; G < KG; ++G) {
            uint32_t word = 0;
            for (int r = 0; r < rows; ++r) word |= (uint32_t)zrow[(size_t)r * KG + G] << (4 * r);
            zeros[(size_t)G * (N / 8) + nb / 8] = (int32_t)word;
        }
    }
    free(row);
    free(qrow);
    free(zrow);
}

typedef struct {
    const float* W;
    uint64_t seed;
    float stddev;
    int N, K, g, n0, n1;
    int32_t* qweight;
    uint16_t* scales;
    int32_t* zeros;
} qjob_t;

static void* qjob_run(void* p) {
    qjob_t* j = (qjob_t*)p;
    quantize_rows(j->W, j->seed, j->stddev, j->N, j->K, j->g, j->n0, j->n1, j->qweight, j->scales, j->zeros);
    return NULL;
}

static int run_quant(const float* W, uint64_t seed, float stddev, int N, int K, int g, int32_t* qweight,
                     uint16_t* scales, int32_t* zeros, int nthreads) {
    if (N <= 0 || K <= 0 || g <= 0 || K % g != 0 || K % 8 != 0 || N % 8 != 0) return 1;
    if (nthreads < 1) nthreads = 1;
    int blocks = N / 8;
    if (nthreads > blocks) nthreads = blocks;
    if (nthreads > 256) nthreads = 256;
    pthread_t th[256];
    qjob_t jobs[256];
    int per = blocks / nthreads, extra = blocks % nthreads, b = 0;
    for (int t = 0; t < nthreads; ++t) {
        int nb = per + (t < extra ? 1 : 0);
        jobs[t] = (qjob_t){W, seed, stddev, N, K, g, b * 8, (b + nb) * 8, qweight, scales, zeros};
        b += nb;
    }
    int started = 0;
    for (int t = 1; t < nthreads; ++t) {
        if (pthread_create(&th[t], NULL, qjob_run, &jobs[t]) != 0) break;
        started = t;
    }
    qjob_run(&jobs[0]);
    for (int t = 1; t <= started; ++t) pthread_join(th[t], NULL);
    for (int t = started + 1; t < nthreads; ++t) qjob_run(&jobs[t]); /* threads that failed to start */
    return 0;
}

/* W ~ N(0, stddev^2) drawn from stream `seed` (element (n, k) is stream
 * element n*K + k), quantised and packed. Returns 0 on success. */
int w4s_gen_linear(uint64_t seed, float stddev, int N, int K, int group, int32_t* qweight, uint16_t* scales,
                   int32_t* zeros, int nthreads) {
    return run_quant(NULL, seed, stddev, N, K, group, qweight, scales, zeros, nthreads);
}

/* Quantise and pack a caller-supplied fp32 W [N][K] (row-major). */
int w4s_quantize(const float* W, int N, int K, int group, int32_t* qweight, uint16_t* scales, int32_t* zeros,
                 int nthreads) {
    return run_quant(W, 0, 0.0f, N, K, group, qweight, scales, zeros, nthreads);
}

/* Activation rows: row i of the [M][K] table is stream (seed_base + row0 + i),
 * x ~ N(0, 1) rounded to bf16 (bits). */
void w4s_gen_x(uint64_t seed_base, int row0, int M, int K, uint16_t* out) {
    float* tmp = (float*)malloc(sizeof(float) * (size_t)K);
    for (int i = 0; i < M; ++i) {
        normals_range(seed_base + (uint64_t)(row0 + i), 0, (size_t)K, 1.0f, tmp);
        for (int k = 0; k < K; ++k) out[(size_t)i * K + k] = f32_to_bf16_rne(tmp[k]);
    }
    free(tmp);
}
