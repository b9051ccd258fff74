/*
 * Seeded synthetic inputs for the CSA / HCA hot path.
 *
 * This file produces INPUTS only: random draws and their encoding into the
 * storage formats the library's callers hand in (bf16 tokens and queries,
 * MXFP4 indexer queries/keys, FP8-E4M3 + bf16 cache entries for decode
 * workloads whose cache exists before the step).  It holds none of the
 * method's arithmetic: no compression weights, no RoPE, no scoring, no
 * selection, no attention.  Both the fp64 oracle and the HIP path consume
 * the bytes written here.
 *
 * Random numbers are counter based: value i of stream s under seed S is a
 * pure function of (S, s, i), so any row can be regenerated on its own.
 *   h(S, s, i) = mix64(mix64(S + s * G) + i * G),  G = 0x9E3779B97F4A7C15,
 * where mix64 is the SplitMix64 output finaliser (Steele, Lea, Flood,
 * "Fast splittable pseudorandom number generators", OOPSLA 2014).
 * Normals use the Box-Muller transform on counters 2i and 2i+1.
 */
#include <math.h>
#include <stdint.h>
#include <string.h>

#define GOLDEN 0x9E3779B97F4A7C15ULL

static inline uint64_t mix64(uint64_t z) {
    z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ULL;
    z = (z ^ (z >> 27)) * 0x94D049BB133111EBULL;
    return z ^ (z >> 31);
}

uint64_t gen_u64(uint64_t seed, uint64_t stream, uint64_t i) {
    return mix64(mix64(seed + stream * GOLDEN) + i * GOLDEN);
}

/* uniform in [0, 1) with 53 random bits */
double gen_uniform(uint64_t seed, uint64_t stream, uint64_t i) {
    return (double)(gen_u64(seed, stream, i) >> 11) * 0x1.0p-53;
}

double gen_normal(uint64_t seed, uint64_t stream, uint64_t i) {
    double u1 = ((double)(gen_u64(seed, stream, 2 * i) >> 11) + 0.5) * 0x1.0p-53;
    double u2 = (double)(gen_u64(seed, stream, 2 * i + 1) >> 11) * 0x1.0p-53;
    return sqrt(-2.0 * log(u1)) * cos(6.283185307179586476925 * u2);
}

/* ---- storage-format encoders used to build inputs ---------------------- */

/* float -> bf16, round to nearest even (inputs are finite) */
static inline uint16_t enc_bf16(float f) {
    uint32_t b;
    memcpy(&b, &f, 4);
    uint32_t lsb = (b >> 16) & 1u;
    b += 0x7FFFu + lsb;
    return (uint16_t)(b >> 16);
}

/* |a| -> OCP E4M3FN magnitude code, nearest-even, saturating at 448 */
static uint8_t enc_e4m3_mag(double a) {
    if (!(a < 464.0)) return 0x7E;
    if (a < 0x1.0p-6) {
        double q = nearbyint(a * 512.0); /* subnormal step 2^-9 */
        return (uint8_t)q;               /* q == 8 is the smallest normal */
    }
    int e;
    double f = frexp(a, &e); /* a = f * 2^e, f in [0.5, 1) */
    int ex = e - 1;           /* a = (2f) * 2^ex, 2f in [1, 2) */
    double q = nearbyint((2.0 * f - 1.0) * 8.0);
    if (q >= 8.0) { q = 0.0; ex += 1; }
    int be = ex + 7;
    if (be > 15 || (be == 15 && q >= 7.0)) return 0x7E;
    return (uint8_t)((be << 3) | (int)q);
}

static inline uint8_t enc_e4m3(double v) {
    uint8_t m = enc_e4m3_mag(fabs(v));
    return (v < 0 && m != 0) ? (uint8_t)(m | 0x80) : m;
}

/* |a| (already divided by the block scale) -> E2M1 magnitude code, nearest-even,
   saturating at 6.  Grid: 0, .5, 1, 1.5, 2, 3, 4, 6. */
static inline uint8_t enc_e2m1_mag(double a) {
    if (a <= 0.25) return 0;
    if (a < 0.75) return 1;
    if (a <= 1.25) return 2;
    if (a < 1.75) return 3;
    if (a <= 2.5) return 4;
    if (a < 3.5) return 5;
    if (a <= 5.0) return 6;
    return 7;
}

/* ---- bulk generators --------------------------------------------------- */

void gen_fill_normal_f32(uint64_t seed, uint64_t stream, int64_t n, double mean, double sigma, float* out) {
#pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < n; ++i) out[i] = (float)(mean + sigma * gen_normal(seed, stream, (uint64_t)i));
}

void gen_fill_normal_bf16(uint64_t seed, uint64_t stream, int64_t n, double sigma, uint16_t* out) {
#pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < n; ++i) out[i] = enc_bf16((float)(sigma * gen_normal(seed, stream, (uint64_t)i)));
}

/* Head weights w = 2^-u, u uniform in {0, 1, 2}. */
void gen_fill_pow2_weights(uint64_t seed, uint64_t stream, int64_t n, float* out) {
#pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < n; ++i) {
        uint64_t u = gen_u64(seed, stream, (uint64_t)i) % 3u;
        out[i] = ldexpf(1.0f, -(int)u);
    }
}

/*
 * MXFP4 rows: rows x dim values (dim a multiple of 32), value (r, c) drawn
 * as N(0,1) from counter r*dim + c, plus an optional planted offset:
 * row r is planted when uniform(seed, stream + 1, r) < plant_frac, and then
 * gets + plant_sigma * dir[c] on every component, dir[c] in {-1, +1} drawn
 * from stream + 2 (one direction per call).  Encoding follows the OCP MX
 * rule: per 32-element block, shared exponent floor(log2(amax)) - 2 stored
 * as E8M0 (bias 127), elements E2M1 nearest-even, saturating; packed two per
 * byte, element 2i in the low nibble.  An all-zero block gets exponent 0.
 * row0 offsets the counter so a slice of a larger tensor can be generated.
 */
void gen_fill_mxfp4(uint64_t seed, uint64_t stream, int64_t row0, int64_t rows, int32_t dim,
                    double plant_frac, double plant_sigma, uint8_t* data, uint8_t* scale, uint8_t* planted) {
    const int nb = dim / 32;
#pragma omp parallel for schedule(static)
    for (int64_t rr = 0; rr < rows; ++rr) {
        int64_t r = row0 + rr;
        int plant = plant_frac > 0.0 && gen_uniform(seed, stream + 1, (uint64_t)r) < plant_frac;
        if (planted) planted[rr] = (uint8_t)plant;
        double v[32];
        for (int b = 0; b < nb; ++b) {
            double amax = 0.0;
            for (int i = 0; i < 32; ++i) {
                int c = b * 32 + i;
                double x = gen_normal(seed, stream, (uint64_t)(r * dim + c));
                if (plant) {
                    double dir = (gen_u64(seed, stream + 2, (uint64_t)c) & 1u) ? 1.0 : -1.0;
                    x += plant_sigma * dir;
                }
                v[i] = x;
                if (fabs(x) > amax) amax = fabs(x);
            }
            int se = 0;
            if (amax > 0.0) {
                int e;
                frexp(amax, &e);  /* floor(log2(amax)) = e - 1 */
                se = (e - 1) - 2;
            }
            if (se < -127) se = -127;
            if (se > 127) se = 127;
            scale[rr * nb + b] = (uint8_t)(se + 127);
            double inv = ldexp(1.0, -se);
            for (int i = 0; i < 32; i += 2) {
                uint8_t lo = enc_e2m1_mag(fabs(v[i] * inv)) | (v[i] < 0 ? 8 : 0);
                uint8_t hi = enc_e2m1_mag(fabs(v[i + 1] * inv)) | (v[i + 1] < 0 ? 8 : 0);
                if ((lo & 7) == 0) lo = 0; /* no negative zero */
                if ((hi & 7) == 0) hi = 0;
                data[rr * (dim / 2) + b * 16 + i / 2] = (uint8_t)(lo | (hi << 4));
            }
        }
    }
}

/*
 * Cache entries in the storage format (d = d_nope + 64): N(0,1) values,
 * the first d_nope as E4M3 codes under a per-entry fp32 scale amax/448
 * (1 when amax is 0), the last 64 as bf16.  Used for decode workloads whose
 * compressed cache and window ring exist before the step.
 */
void gen_fill_entries(uint64_t seed, uint64_t stream, int64_t row0, int64_t rows, int32_t d_nope,
                      uint8_t* nope, uint16_t* rope, float* scale) {
    const int d = d_nope + 64;
#pragma omp parallel for schedule(static)
    for (int64_t rr = 0; rr < rows; ++rr) {
        int64_t r = row0 + rr;
        double v[1024];
        double amax = 0.0;
        for (int c = 0; c < d; ++c) {
            v[c] = gen_normal(seed, stream, (uint64_t)(r * d + c));
            if (c < d_nope && fabs(v[c]) > amax) amax = fabs(v[c]);
        }
        float s = amax > 0.0 ? (float)(amax / 448.0) : 1.0f;
        scale[rr] = s;
        for (int c = 0; c < d_nope; ++c) nope[rr * d_nope + c] = enc_e4m3(v[c] / (double)s);
        for (int c = 0; c < 64; ++c) rope[rr * 64 + c] = enc_bf16((float)v[d_nope + c]);
    }
}

/* Random selection lists: for each of T rows, k distinct ascending indices
   below n[t] (fewer if n[t] < k; -1 padded).  Partial Fisher-Yates on a
   scratch array supplied by the caller (size >= max n). */
void gen_fill_random_idx(uint64_t seed, uint64_t stream, int64_t T, const int64_t* n, int32_t k,
                         int32_t* idx, int32_t* scratch) {
    for (int64_t t = 0; t < T; ++t) {
        int64_t nt = n[t];
        int32_t take = nt < k ? (int32_t)nt : k;
        for (int64_t j = 0; j < nt; ++j) scratch[j] = (int32_t)j;
        for (int32_t a = 0; a < take; ++a) {
            uint64_t r = gen_u64(seed, stream, (uint64_t)(t * 1000003 + a));
            int64_t b = a + (int64_t)(r % (uint64_t)(nt - a));
            int32_t tmp = scratch[a];
            scratch[a] = scratch[b];
            scratch[b] = tmp;
        }
        /* sort the chosen prefix ascending (insertion sort on <= 2048 items) */
        for (int32_t a = 1; a < take; ++a) {
            int32_t x = scratch[a];
            int32_t b = a - 1;
            while (b >= 0 && scratch[b] > x) { scratch[b + 1] = scratch[b]; --b; }
            scratch[b + 1] = x;
        }
        for (int32_t a = 0; a < k; ++a) idx[t * k + a] = a < take ? scratch[a] : -1;
    }
}
