/*
 * ORACLE for the routed low-bit expert FFN -- test infrastructure only.
 *
 * A plain, slow, single-threaded float64 implementation of what one routed
 * mixture-of-experts FFN layer computes.  It is the reference the GPU library
 * is checked against and is never part of the product path: only the tests,
 * the smoke check and the benchmark's CPU-baseline leg load it.  It shares no
 * source, header, table or helper with the GPU library; it reads the blob
 * bytes with its own decoding written from the format definition below.
 *
 * Sources (the pages these functions follow):
 *   [Strata]  "Strata in the source: one verify window, three workers and a
 *             cache that learns" -- sections "The byte budget, in code"
 *             (Q2_0: 64 weights = 16 bytes of 2-bit codes + one fp16 scale;
 *             each expert has gate, up and down of 2,560 x 640) and "The CPU
 *             kernels" (codes {0,1,2,3} are integer offsets times the scale;
 *             64 codes unpack from 8 little-endian 16-bit words, 8 codes per
 *             word, two bits each, lowest bits first).
 *   [Krasis]  Krasis white paper, section 5.3 "Per-token routed expert
 *             execution" (route -> top-k ids and weights -> expert
 *             projections -> activation/gating -> weighted reduction) and
 *             section 7.1 (the layer output is the router-weighted sum of the
 *             selected experts' outputs).
 *   [kairos]  kairos-engine README, "The MoE forward" (normalise, router GEMM
 *             to logits, top-k; the router reads its input through its own
 *             weightless norm and a per-input-dim scale; the down projection's
 *             scale is per expert; the shared expert is summed with the routed
 *             experts, not sequenced), "The memory problem, and the expert
 *             arena" (4-bit expert file; ~12.85 GB of experts) and "Decode,
 *             2026-09-28/29: the hybrid, and the host thread" (the model's
 *             GELU is the tanh form).
 *   [Krasis]  section 7.5 "Preserving the native execution shape": a fixed
 *             top-k shape in which an omitted route is a slot with a dummy
 *             expert and a zero router weight, for which no expert work is
 *             done.
 *
 * Readings where the pages leave a step open (each is also a descriptor
 * field or documented choice of the library):
 *   - Block decoding: weight = scale * (code - z).  The Strata page maps codes
 *     {0,1,2,3} to {-1,0,1,2} (z = 1); the measured 2-bit configurations use
 *     z = 1.5 and the 4-bit ones z = 7.5 (32 codes per fp16 scale).  z is an
 *     argument here.
 *   - Byte order inside a block: 2-bit code i sits in byte i/4 at bit
 *     2*(i%4) (the unpack order of the Strata CPU kernel); 4-bit code i sits
 *     in byte i/2, low nibble for even i.
 *   - Blob: gate [FF][H], up [FF][H], down [H][FF] in this order; each matrix
 *     is a codes plane [rows][nblk][16 B] followed by a scales plane
 *     [rows][nblk] of little-endian fp16, blocks running along the matrix's
 *     input dimension.
 *   - Routing order: logit descending, expert index ascending on ties
 *     (-0 == +0; a NaN logit ranks below every number).  Weights are the
 *     softmax over the k selected logits (renormalize = 1) or the full softmax
 *     over all E logits taken at the selected experts (renormalize = 0).
 *   - Activation: SwiGLU, a = silu(gate x) * (up x), silu(v) = v / (1 + e^-v);
 *     or GeGLU with the tanh form of GELU, a = gelu(gate x) * (up x),
 *     gelu(v) = v/2 (1 + tanh(sqrt(2/pi) (v + 0.044715 v^3))).
 *   - Per-expert down scale: expert e's output is s_e * (W_down a).
 *   - Router: logits = W_r x' with bf16 W_r [E][H]; x' = x, or with the
 *     weightless norm x / sqrt(mean(x^2) + eps), then times the per-input-dim
 *     scale when one is given.
 *   - Caller-supplied routing: the given ids and weights are used as they are;
 *     a slot whose weight is 0 contributes nothing and its expert is not read.
 *   - Output: y = shared(x) + sum_j w_j expert_{id_j}(x), shared first, then
 *     slots in rank order.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

/* qtype 1: 64 two-bit codes per block; qtype 2: 32 four-bit codes per block. */
static int codes_per_block(int qtype) { return qtype == 1 ? 64 : (qtype == 2 ? 32 : 0); }
static int bits_per_code(int qtype) { return qtype == 1 ? 2 : (qtype == 2 ? 4 : 0); }

/* Every block is 16 bytes of codes and a 2-byte scale, whatever the qtype. */
int64_t oracle_blob_bytes(int qtype, int64_t H, int64_t FF) {
    int qk = codes_per_block(qtype);
    if (qk == 0) return -1;
    return 3 * (H * FF / qk) * (16 + 2);
}

/* IEEE 754 binary16 -> double, from the format's definition (exact). */
static double half_to_double(uint16_t h) {
    int s = h >> 15, e = (h >> 10) & 31, m = h & 1023;
    double v;
    if (e == 0) v = ldexp((double)m, -24);                 /* subnormal: m * 2^-24 */
    else if (e == 31) v = m ? NAN : INFINITY;
    else v = ldexp((double)(1024 + m), e - 25);            /* (1 + m/1024) * 2^(e-15) */
    return s ? -v : v;
}

/* bfloat16 bits are the upper half of a binary32 (exact widening). */
static double bf16_to_double(uint16_t b) {
    uint32_t u = (uint32_t)b << 16;
    float f;
    memcpy(&f, &u, 4);
    return (double)f;
}

typedef struct {
    const uint8_t* codes;   /* [rows][nblk][16] */
    const uint8_t* scales;  /* [rows][nblk] fp16 little-endian */
    int64_t rows, cols, nblk;
    int qk, bits;
    double z;
} omat;

/* Matrix m (0 = gate, 1 = up, 2 = down) of an expert blob. */
static omat matrix_of(const uint8_t* blob, int qtype, double z, int64_t H, int64_t FF, int m) {
    omat M;
    int64_t rows[3] = {FF, FF, H};
    int64_t cols[3] = {H, H, FF};
    M.qk = codes_per_block(qtype);
    M.bits = bits_per_code(qtype);
    M.z = z;
    const uint8_t* p = blob;
    for (int i = 0; i < m; ++i) p += rows[i] * (cols[i] / M.qk) * 18;
    M.rows = rows[m];
    M.cols = cols[m];
    M.nblk = M.cols / M.qk;
    M.codes = p;
    M.scales = p + M.rows * M.nblk * 16;
    return M;
}

/* The integer code of weight i (0 <= i < qk) of a 16-byte block. */
static int code_of(const uint8_t* blk, int bits, int i) {
    if (bits == 2) return (blk[i / 4] >> (2 * (i % 4))) & 3;
    return (blk[i / 2] >> (4 * (i % 2))) & 15;
}

/* The qk weights of block b of row r, dequantized: scale * (code - z). */
static void block_weights(const omat* M, int64_t r, int64_t b, double* w) {
    int64_t idx = r * M->nblk + b;
    const uint8_t* blk = M->codes + idx * 16;
    uint16_t sb = (uint16_t)(M->scales[2 * idx] | (M->scales[2 * idx + 1] << 8));
    double s = half_to_double(sb);
    for (int i = 0; i < M->qk; ++i) w[i] = s * ((double)code_of(blk, M->bits, i) - M->z);
}

/* Dense dequantized matrix m of a blob: out[rows][cols]. */
void oracle_dequant_matrix(const uint8_t* blob, int qtype, double z, int64_t H, int64_t FF, int m, double* out) {
    omat M = matrix_of(blob, qtype, z, H, FF, m);
    double w[64];
    for (int64_t r = 0; r < M.rows; ++r)
        for (int64_t b = 0; b < M.nblk; ++b) {
            block_weights(&M, r, b, w);
            for (int i = 0; i < M.qk; ++i) out[r * M.cols + b * M.qk + i] = w[i];
        }
}

/* out[r] = sum_k W[r][k] v[k] for every row of matrix M. */
static void matvec(const omat* M, const double* v, double* out) {
    double w[64];
    for (int64_t r = 0; r < M->rows; ++r) {
        double acc = 0.0;
        for (int64_t b = 0; b < M->nblk; ++b) {
            block_weights(M, r, b, w);
            for (int i = 0; i < M->qk; ++i) acc += w[i] * v[b * M->qk + i];
        }
        out[r] = acc;
    }
}

static double silu(double v) { return v / (1.0 + exp(-v)); }

/* GELU, tanh form: v/2 (1 + tanh(sqrt(2/pi) (v + 0.044715 v^3))). */
static double gelu_tanh(double v) {
    const double c = sqrt(2.0 / 3.14159265358979323846);
    return 0.5 * v * (1.0 + tanh(c * (v + 0.044715 * v * v * v)));
}

/* The gate's activation: 0 = SiLU (SwiGLU), 1 = tanh GELU (GeGLU). */
static double gate_act(double g, int act) { return act == 1 ? gelu_tanh(g) : silu(g); }

/* Activations as exact doubles: x_dtype 0 = fp32, 1 = bf16 raw bits. */
static void load_x(const void* x, int x_dtype, int64_t n, double* out) {
    if (x_dtype == 1) {
        const uint16_t* b = (const uint16_t*)x;
        for (int64_t i = 0; i < n; ++i) out[i] = bf16_to_double(b[i]);
    } else {
        const float* f = (const float*)x;
        for (int64_t i = 0; i < n; ++i) out[i] = (double)f[i];
    }
}

/* One expert's gated FFN on one token: y = W_down (act(W_gate x) * (W_up x)). */
static void ffn_token_act(const uint8_t* blob, int qtype, double z, int64_t H, int64_t FF, int act, const double* x,
                          double* y, double* g, double* u) {
    omat Mg = matrix_of(blob, qtype, z, H, FF, 0);
    omat Mu = matrix_of(blob, qtype, z, H, FF, 1);
    omat Md = matrix_of(blob, qtype, z, H, FF, 2);
    matvec(&Mg, x, g);
    matvec(&Mu, x, u);
    for (int64_t f = 0; f < FF; ++f) g[f] = gate_act(g[f], act) * u[f];
    matvec(&Md, g, y);
}

/* SwiGLU. */
static void ffn_token(const uint8_t* blob, int qtype, double z, int64_t H, int64_t FF, const double* x, double* y,
                      double* g, double* u) {
    ffn_token_act(blob, qtype, z, H, FF, 0, x, y, g, u);
}

/* gelu_tanh of n values (exported for the pins). */
void oracle_gelu_tanh(const double* v, int64_t n, double* out) {
    for (int64_t i = 0; i < n; ++i) out[i] = gelu_tanh(v[i]);
}

/* y[T][H] = expert FFN with activation act (0 SwiGLU, 1 GeGLU-tanh) of each token. */
int oracle_expert_ffn_act(const uint8_t* blob, int qtype, double z, int64_t H, int64_t FF, int act, const void* x,
                          int x_dtype, int64_t T, double* y) {
    if (codes_per_block(qtype) == 0 || H % codes_per_block(qtype) || FF % codes_per_block(qtype)) return 1;
    if (act != 0 && act != 1) return 1;
    double* xt = (double*)malloc(sizeof(double) * (size_t)H);
    double* g = (double*)malloc(sizeof(double) * (size_t)FF);
    double* u = (double*)malloc(sizeof(double) * (size_t)FF);
    for (int64_t t = 0; t < T; ++t) {
        load_x((const uint8_t*)x + (size_t)(t * H) * (x_dtype == 1 ? 2 : 4), x_dtype, H, xt);
        ffn_token_act(blob, qtype, z, H, FF, act, xt, y + t * H, g, u);
    }
    free(xt);
    free(g);
    free(u);
    return 0;
}

/* y[T][H] = expert FFN of each token; x is T x H (fp32 or bf16 bits). */
int oracle_expert_ffn(const uint8_t* blob, int qtype, double z, int64_t H, int64_t FF, const void* x, int x_dtype,
                      int64_t T, double* y) {
    if (codes_per_block(qtype) == 0 || H % codes_per_block(qtype) || FF % codes_per_block(qtype)) return 1;
    double* xt = (double*)malloc(sizeof(double) * (size_t)H);
    double* g = (double*)malloc(sizeof(double) * (size_t)FF);
    double* u = (double*)malloc(sizeof(double) * (size_t)FF);
    for (int64_t t = 0; t < T; ++t) {
        load_x((const uint8_t*)x + (size_t)(t * H) * (x_dtype == 1 ? 2 : 4), x_dtype, H, xt);
        ffn_token(blob, qtype, z, H, FF, xt, y + t * H, g, u);
    }
    free(xt);
    free(g);
    free(u);
    return 0;
}

/* Expert a ranks before expert b: larger logit first, NaN below every number,
 * equal logits (including -0 and +0) broken toward the lower index. */
static const float* g_rank_logits;
static int rank_cmp(const void* pa, const void* pb) {
    int a = *(const int*)pa, b = *(const int*)pb;
    float la = g_rank_logits[a], lb = g_rank_logits[b];
    int na = isnan(la), nb = isnan(lb);
    if (na != nb) return na ? 1 : -1;
    if (!na && la != lb) return la > lb ? -1 : 1;
    return a - b;
}

/* Top-k of each token's E logits and the routing weights. */
int oracle_route_topk(const float* logits, int64_t T, int32_t E, int32_t k, int32_t renormalize, int32_t* ids,
                      double* w) {
    if (k < 1 || k > E) return 1;
    int* order = (int*)malloc(sizeof(int) * (size_t)E);
    for (int64_t t = 0; t < T; ++t) {
        const float* l = logits + t * E;
        for (int e = 0; e < E; ++e) order[e] = e;
        g_rank_logits = l;
        qsort(order, (size_t)E, sizeof(int), rank_cmp);  /* a total order: the result is unique */
        for (int j = 0; j < k; ++j) ids[t * k + j] = order[j];
        double top = (double)l[order[0]];
        double denom = 0.0;
        if (renormalize) {
            /* softmax over the k selected logits; an all -inf selection gets equal weights */
            for (int j = 0; j < k; ++j) denom += isinf(top) && top < 0 ? 1.0 : exp((double)l[order[j]] - top);
            for (int j = 0; j < k; ++j)
                w[t * k + j] = (isinf(top) && top < 0 ? 1.0 : exp((double)l[order[j]] - top)) / denom;
        } else {
            /* full softmax over all E logits, read at the selected experts */
            for (int e = 0; e < E; ++e) denom += isinf(top) && top < 0 ? 1.0 : exp((double)l[e] - top);
            for (int j = 0; j < k; ++j)
                w[t * k + j] = (isinf(top) && top < 0 ? 1.0 : exp((double)l[order[j]] - top)) / denom;
        }
    }
    free(order);
    return 0;
}

/* One routed MoE FFN layer.
 *   blobs[E]  : host pointers to each expert's blob (qtype, z, H, FF)
 *   shared    : the shared expert's blob (FF = shared_ff) or NULL
 *   x         : T x H activations (fp32 or bf16 bits); logits : T x E fp32
 *   y         : T x H output; ids, w : T x k routing (outputs) */
int oracle_layer_forward(const uint8_t* const* blobs, int32_t E, int32_t k, int32_t renormalize, int qtype, double z,
                         int64_t H, int64_t FF, const uint8_t* shared, int64_t shared_ff, const void* x, int x_dtype,
                         const float* logits, int64_t T, double* y, int32_t* ids, double* w) {
    int qk = codes_per_block(qtype);
    if (qk == 0 || H % qk || FF % qk || (shared && shared_ff % qk)) return 1;
    if (oracle_route_topk(logits, T, E, k, renormalize, ids, w)) return 1;
    int64_t ffmax = shared && shared_ff > FF ? shared_ff : FF;
    double* xt = (double*)malloc(sizeof(double) * (size_t)H);
    double* ye = (double*)malloc(sizeof(double) * (size_t)H);
    double* g = (double*)malloc(sizeof(double) * (size_t)ffmax);
    double* u = (double*)malloc(sizeof(double) * (size_t)ffmax);
    for (int64_t t = 0; t < T; ++t) {
        double* yt = y + t * H;
        load_x((const uint8_t*)x + (size_t)(t * H) * (x_dtype == 1 ? 2 : 4), x_dtype, H, xt);
        for (int64_t h = 0; h < H; ++h) yt[h] = 0.0;
        if (shared) {
            ffn_token(shared, qtype, z, H, shared_ff, xt, ye, g, u);
            for (int64_t h = 0; h < H; ++h) yt[h] += ye[h];
        }
        for (int j = 0; j < k; ++j) {
            ffn_token(blobs[ids[t * k + j]], qtype, z, H, FF, xt, ye, g, u);
            for (int64_t h = 0; h < H; ++h) yt[h] += w[t * k + j] * ye[h];
        }
    }
    free(xt);
    free(ye);
    free(g);
    free(u);
    return 0;
}

/* Router: logits[t][e] = sum_h W_r[e][h] x'[t][h], W_r bf16 bits [E][H];
 * x' = x, or with norm = 1 the weightless norm x / sqrt(mean_h x^2 + eps);
 * then times in_scale[h] when in_scale is not NULL. */
int oracle_router_logits(const uint16_t* wr, int32_t E, int64_t H, const void* x, int x_dtype, int64_t T, int norm,
                         double eps, const float* in_scale, double* logits) {
    if (E < 1 || H < 1) return 1;
    double* xt = (double*)malloc(sizeof(double) * (size_t)H);
    for (int64_t t = 0; t < T; ++t) {
        load_x((const uint8_t*)x + (size_t)(t * H) * (x_dtype == 1 ? 2 : 4), x_dtype, H, xt);
        if (norm) {
            double ss = 0.0;
            for (int64_t h = 0; h < H; ++h) ss += xt[h] * xt[h];
            const double r = 1.0 / sqrt(ss / (double)H + eps);
            for (int64_t h = 0; h < H; ++h) xt[h] *= r;
        }
        if (in_scale)
            for (int64_t h = 0; h < H; ++h) xt[h] *= (double)in_scale[h];
        for (int32_t e = 0; e < E; ++e) {
            double acc = 0.0;
            for (int64_t h = 0; h < H; ++h) acc += bf16_to_double(wr[(size_t)e * H + h]) * xt[h];
            logits[t * E + e] = acc;
        }
    }
    free(xt);
    return 0;
}

/* One routed MoE FFN layer with the options of the extended call:
 *   act        : 0 SwiGLU, 1 GeGLU-tanh (routed and shared experts alike)
 *   down_scale : NULL, or [E]: routed expert e's output is down_scale[e] * (W_down a)
 *   ids_in/w_in: NULL, or caller-supplied routing [T][k]; a slot whose weight is 0 is
 *                skipped (its id is not read); a nonzero weight with an id outside
 *                [0, E) is an error (returns 2).  Otherwise routing from logits.
 *   ids, w     : the routing used (outputs). */
int oracle_layer_forward_ex(const uint8_t* const* blobs, int32_t E, int32_t k, int32_t renormalize, int qtype,
                            double z, int64_t H, int64_t FF, int act, const uint8_t* shared, int64_t shared_ff,
                            const float* down_scale, const void* x, int x_dtype, const float* logits,
                            const int32_t* ids_in, const float* w_in, int64_t T, double* y, int32_t* ids, double* w) {
    int qk = codes_per_block(qtype);
    if (qk == 0 || H % qk || FF % qk || (shared && shared_ff % qk) || (act != 0 && act != 1)) return 1;
    if (ids_in) {
        for (int64_t q = 0; q < T * k; ++q) {
            if (w_in[q] != 0.0f && (ids_in[q] < 0 || ids_in[q] >= E)) return 2;
            ids[q] = ids_in[q];
            w[q] = (double)w_in[q];
        }
    } else if (oracle_route_topk(logits, T, E, k, renormalize, ids, w)) {
        return 1;
    }
    int64_t ffmax = shared && shared_ff > FF ? shared_ff : FF;
    double* xt = (double*)malloc(sizeof(double) * (size_t)H);
    double* ye = (double*)malloc(sizeof(double) * (size_t)H);
    double* g = (double*)malloc(sizeof(double) * (size_t)ffmax);
    double* u = (double*)malloc(sizeof(double) * (size_t)ffmax);
    for (int64_t t = 0; t < T; ++t) {
        double* yt = y + t * H;
        load_x((const uint8_t*)x + (size_t)(t * H) * (x_dtype == 1 ? 2 : 4), x_dtype, H, xt);
        for (int64_t h = 0; h < H; ++h) yt[h] = 0.0;
        if (shared) {
            ffn_token_act(shared, qtype, z, H, shared_ff, act, xt, ye, g, u);
            for (int64_t h = 0; h < H; ++h) yt[h] += ye[h];
        }
        for (int j = 0; j < k; ++j) {
            const double wj = w[t * k + j];
            if (ids_in && wj == 0.0) continue;   /* an omitted route: no expert work */
            const int e = ids[t * k + j];
            ffn_token_act(blobs[e], qtype, z, H, FF, act, xt, ye, g, u);
            const double s = down_scale ? (double)down_scale[e] : 1.0;
            for (int64_t h = 0; h < H; ++h) yt[h] += wj * (s * ye[h]);
        }
    }
    free(xt);
    free(ye);
    free(g);
    free(u);
    return 0;
}
