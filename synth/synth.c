/*
 * Seeded synthetic inputs for the routed low-bit expert FFN.
 *
 * This module only draws numbers: random code bytes, fp16 block scales,
 * activations and router logits.  It contains none of the method's arithmetic
 * (no dequantisation, no routing, no projection), so both the float64 oracle
 * and the GPU path can take their inputs from it without sharing any of the
 * computation they are compared on.
 *
 * Generator.  Every value is a pure function of (seed, stream, index):
 *     key(seed, stream) = mix64(mix64(seed) ^ stream)
 *     word(seed, stream, i) = mix64(key + (i + 1) * 0x9E3779B97F4A7C15)
 * where mix64 is the SplitMix64 output function (Steele, Lea and Flood,
 * "Fast splittable pseudorandom number generators", OOPSLA 2014).  The word
 * sequence of one stream is exactly the SplitMix64 sequence started at state
 * `key`, so any element of any tensor can be regenerated on its own.
 *
 * Distributions.
 *   uniform bytes      : the eight little-endian bytes of consecutive words;
 *                        uniform bytes give uniform, independent 2-bit and
 *                        4-bit codes in every field.
 *   normal N(0,1)      : Box-Muller on the pair j = i / 2:
 *                        u1 = (w[2j] >> 11 + 0.5) 2^-53, u2 = (w[2j+1] >> 11) 2^-53,
 *                        r = sqrt(-2 ln u1); element 2j is r cos(2 pi u2) and
 *                        element 2j+1 is r sin(2 pi u2).
 *   fp16 / bf16        : the double value rounded once, to nearest-even, into
 *                        the target format (subnormals kept).
 *   Zipf-skewed logits : per layer a random permutation gives each expert a
 *                        popularity rank r (0 = most popular);
 *                        logit[t][e] = -s ln(r_e + 1) + G[t][e] with G standard
 *                        Gumbel, -ln(-ln u).  The top-k of such logits is a
 *                        k-sample without replacement from p_e ~ (r_e + 1)^-s
 *                        (the Gumbel-top-k construction), so tokens share
 *                        experts through popularity skew alone.  s = 0 gives
 *                        plain N(0,1) logits instead.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define GAMMA 0x9E3779B97F4A7C15ull

static inline uint64_t mix64(uint64_t z) {
    z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
    z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
    return z ^ (z >> 31);
}

static inline uint64_t stream_key(uint64_t seed, uint64_t stream) {
    return mix64(mix64(seed) ^ stream);
}

static inline uint64_t word_at(uint64_t key, uint64_t i) { return mix64(key + (i + 1) * GAMMA); }

/* Stream identifiers: kind in the top byte, then three fields. */
enum { K_CODES = 1, K_SCALES = 2, K_X = 3, K_LOGITS = 4, K_PERM = 5 };

uint64_t synth_stream(uint32_t kind, uint32_t a, uint32_t b, uint32_t c) {
    return ((uint64_t)(kind & 0xFF) << 56) | ((uint64_t)(a & 0xFFFFFF) << 32) |
           ((uint64_t)(b & 0xFFFFFF) << 8) | (uint64_t)(c & 0xFF);
}

uint64_t synth_word(uint64_t seed, uint64_t stream, uint64_t i) {
    return word_at(stream_key(seed, stream), i);
}

static inline double unit_open(uint64_t w) { return ((double)(w >> 11) + 0.5) * 0x1p-53; }
static inline double unit_closed_open(uint64_t w) { return (double)(w >> 11) * 0x1p-53; }

static inline void normal_pair(uint64_t key, uint64_t j, double* z0, double* z1) {
    double u1 = unit_open(word_at(key, 2 * j));
    double u2 = unit_closed_open(word_at(key, 2 * j + 1));
    double r = sqrt(-2.0 * log(u1));
    double a = 6.283185307179586476925 * u2;
    *z0 = r * cos(a);
    *z1 = r * sin(a);
}


/* out[i] = f(i-th normal of the stream) for i < n, drawing each Box-Muller pair once. */
#define FILL_NORMALS(key, n, EXPR_OF_Z, out)                           \
    do {                                                               \
        for (size_t j_ = 0; 2 * j_ < (n); ++j_) {                      \
            double z0_, z1_;                                           \
            normal_pair((key), j_, &z0_, &z1_);                        \
            { double z = z0_; (out)[2 * j_] = (EXPR_OF_Z); }           \
            if (2 * j_ + 1 < (n)) { double z = z1_; (out)[2 * j_ + 1] = (EXPR_OF_Z); } \
        }                                                              \
    } while (0)

/* Round a double once, to nearest with ties to even, into a binary format
 * with mbits explicit mantissa bits, exponent bias `bias` and an exponent
 * field of ebits bits; subnormals are kept, overflow gives infinity.
 * Works on the double's bit pattern so there is no intermediate rounding. */
static uint16_t double_to_small(double v, int mbits, int ebits) {
    uint64_t b;
    memcpy(&b, &v, 8);
    uint16_t sign = (uint16_t)((b >> 63) << (mbits + ebits));
    int exp = (int)((b >> 52) & 0x7FF);
    uint64_t man = b & ((1ull << 52) - 1);
    int bias = (1 << (ebits - 1)) - 1;
    int emin = 1 - bias;
    uint16_t inf_bits = (uint16_t)(((1u << ebits) - 1) << mbits);
    if (exp == 0x7FF) return (uint16_t)(sign | inf_bits | (man ? 1u : 0u));
    if (exp == 0) return sign;        /* zero or double subnormal: below every target */
    int e = exp - 1023;
    uint64_t M = man | (1ull << 52);  /* value = M * 2^(e - 52) */
    int qe = (e > emin ? e : emin) - mbits;
    int shift = 52 + qe - e;          /* >= 52 - mbits */
    uint64_t r;
    if (shift >= 64) {
        r = 0;
    } else {
        r = M >> shift;
        uint64_t rem = M & ((1ull << shift) - 1);
        uint64_t half = 1ull << (shift - 1);
        if (rem > half || (rem == half && (r & 1))) ++r;
    }
    uint64_t bits;
    if (e < emin) bits = r;           /* subnormal, or rounded up to the least normal */
    else bits = ((uint64_t)(e + bias) << mbits) + (r - (1ull << mbits));
    if (bits >= inf_bits) return (uint16_t)(sign | inf_bits);
    return (uint16_t)(sign | bits);
}

uint16_t synth_double_to_f16(double v) { return double_to_small(v, 10, 5); }

uint16_t synth_double_to_bf16(double v) { return double_to_small(v, 7, 8); }

/* n uniform random bytes of one stream. */
void synth_bytes(uint64_t seed, uint64_t stream, uint8_t* out, size_t n) {
    uint64_t key = stream_key(seed, stream);
    size_t nw = n / 8;
    for (size_t i = 0; i < nw; ++i) {
        uint64_t w = word_at(key, i);
        memcpy(out + 8 * i, &w, 8);
    }
    if (n % 8) {
        uint64_t w = word_at(key, nw);
        memcpy(out + 8 * nw, &w, n % 8);
    }
}

/* |N(0, sigma)| (absolute = 1) or N(0, sigma) rounded to fp16, as raw bits. */
void synth_f16_normal(uint64_t seed, uint64_t stream, double sigma, int absolute, uint16_t* out, size_t n) {
    uint64_t key = stream_key(seed, stream);
    FILL_NORMALS(key, n, synth_double_to_f16(absolute ? fabs(sigma * z) : sigma * z), out);
}

/* N(0,1) rounded to bf16, as raw bits. */
void synth_bf16_normal(uint64_t seed, uint64_t stream, uint16_t* out, size_t n) {
    uint64_t key = stream_key(seed, stream);
    FILL_NORMALS(key, n, synth_double_to_bf16(z), out);
}

/* N(0,1) rounded to fp32. */
void synth_f32_normal(uint64_t seed, uint64_t stream, float* out, size_t n) {
    uint64_t key = stream_key(seed, stream);
    FILL_NORMALS(key, n, (float)z, out);
}

/* Activations of one layer and step: T x H values, bf16 bits (dtype 1) or fp32
 * (dtype 0).  Element i of the stream is the i-th normal; threads fill
 * disjoint, pair-aligned ranges, so the values do not depend on the thread count. */
void synth_activations(uint64_t seed, uint32_t layer, uint32_t step, int64_t T, int64_t H, int dtype, void* out) {
    uint64_t key = stream_key(seed, synth_stream(K_X, layer, step, 0));
    int64_t n = T * H;
    int64_t npairs = (n + 1) / 2;
    const int64_t chunk = 1 << 15;
#pragma omp parallel for schedule(static)
    for (int64_t c = 0; c < (npairs + chunk - 1) / chunk; ++c) {
        int64_t j1 = (c + 1) * chunk < npairs ? (c + 1) * chunk : npairs;
        for (int64_t j = c * chunk; j < j1; ++j) {
            double z0, z1;
            normal_pair(key, (uint64_t)j, &z0, &z1);
            if (dtype == 1) {
                uint16_t* o = (uint16_t*)out;
                o[2 * j] = synth_double_to_bf16(z0);
                if (2 * j + 1 < n) o[2 * j + 1] = synth_double_to_bf16(z1);
            } else {
                float* o = (float*)out;
                o[2 * j] = (float)z0;
                if (2 * j + 1 < n) o[2 * j + 1] = (float)z1;
            }
        }
    }
}

typedef struct { uint64_t key; int32_t idx; } perm_item;
static int perm_cmp(const void* a, const void* b) {
    const perm_item* x = (const perm_item*)a;
    const perm_item* y = (const perm_item*)b;
    if (x->key != y->key) return x->key < y->key ? -1 : 1;
    return x->idx - y->idx;
}

/* Popularity rank of every expert of one layer (a random permutation). */
void synth_popularity_rank(uint64_t seed, uint32_t layer, int32_t E, int32_t* rank) {
    uint64_t key = stream_key(seed, synth_stream(K_PERM, layer, 0, 0));
    perm_item* it = (perm_item*)malloc(sizeof(perm_item) * (size_t)E);
    for (int32_t e = 0; e < E; ++e) { it[e].key = word_at(key, (uint64_t)e); it[e].idx = e; }
    qsort(it, (size_t)E, sizeof(perm_item), perm_cmp);
    for (int32_t r = 0; r < E; ++r) rank[it[r].idx] = r;
    free(it);
}

/* Router logits of one layer and step, T x E fp32.  s > 0: Zipf-skewed
 * (popularity exponent s, per-layer permutation); s == 0: N(0,1). */
void synth_logits(uint64_t seed, uint32_t layer, uint32_t step, int64_t T, int32_t E, double s, float* out) {
    uint64_t st = synth_stream(K_LOGITS, layer, step, 0);
    if (s == 0.0) { synth_f32_normal(seed, st, out, (size_t)(T * E)); return; }
    int32_t* rank = (int32_t*)malloc(sizeof(int32_t) * (size_t)E);
    synth_popularity_rank(seed, layer, E, rank);
    uint64_t key = stream_key(seed, st);
    for (int64_t t = 0; t < T; ++t)
        for (int32_t e = 0; e < E; ++e) {
            double u = unit_open(word_at(key, (uint64_t)(t * E + e)));
            double g = -log(-log(u));
            out[t * E + e] = (float)(-s * log((double)rank[e] + 1.0) + g);
        }
    free(rank);
}

/* Byte size of one expert blob: gate [FF][H], up [FF][H], down [H][FF], each
 * quantized in blocks of qk weights along its input dimension; every block
 * is 16 bytes of codes plus a 2-byte fp16 scale. */
int64_t synth_blob_bytes(int32_t qk, int64_t H, int64_t FF) { return 3 * (H * FF / qk) * 18; }

/* Fill one expert blob.  Per matrix: codes plane (rows x nblk x 16 B, uniform
 * random bytes) followed by the scales plane (rows x nblk fp16, |N(0,sigma)|).
 * expert = 0xFFFFFF names the layer's shared expert. */
void synth_expert_blob(uint64_t seed, uint32_t layer, uint32_t expert, int32_t qk, int64_t H, int64_t FF,
                       double sigma, uint8_t* out) {
    int64_t rows[3] = {FF, FF, H};
    int64_t cols[3] = {H, H, FF};
    uint8_t* p = out;
    for (int m = 0; m < 3; ++m) {
        int64_t nb = rows[m] * (cols[m] / qk);
        synth_bytes(seed, synth_stream(K_CODES, layer, expert, (uint32_t)m), p, (size_t)(nb * 16));
        p += nb * 16;
        synth_f16_normal(seed, synth_stream(K_SCALES, layer, expert, (uint32_t)m), sigma, 1, (uint16_t*)p, (size_t)nb);
        p += nb * 2;
    }
}

/* Fill n_exp consecutive experts' blobs [e_first, e_first + n_exp) of one
 * layer, blob i at out + i * stride; threads split the experts. */
void synth_expert_blobs(uint64_t seed, uint32_t layer, uint32_t e_first, int32_t n_exp, int32_t qk, int64_t H,
                        int64_t FF, double sigma, uint8_t* out, int64_t stride) {
#pragma omp parallel for schedule(dynamic, 1)
    for (int32_t i = 0; i < n_exp; ++i)
        synth_expert_blob(seed, layer, e_first + (uint32_t)i, qk, H, FF, sigma, out + (int64_t)i * stride);
}
