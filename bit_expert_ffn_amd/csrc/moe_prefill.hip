// Prefill path (T > 8 tokens): expert-major grouped GEMMs on the matrix cores.
//
// What is computed is the same layer as on the decode path (Krasis white paper
// 5.3; kairos-engine README "The MoE forward": the batch is bucketed by expert
// and each expert runs one GEMM over every token that chose it; "Prefill and
// decode are different machines": prefill dequantises and feeds the tensor
// cores).  Steps, each one kernel on the caller's stream:
//   1. route    : top-k per token (the decode path's wave top-k).
//   2. count    : per-expert counts, offsets and a list of row tiles (<= 128
//                 (token, slot) rows of one expert each).
//   3. place    : one wave per expert scans the pairs in (token, slot) order and
//                 writes the sorted position of each (a stable counting sort).
//   4. gate/up  : per row tile and 64 FF features, G = X W_g^T and U = X W_u^T
//                 on MFMA, then a = silu(G) * U, stored as bf16 hi + lo.
//   5. down     : per row tile and 64 H features, Y = a W_d^T on MFMA.
//   6. combine  : y[t] = shared(t) + sum_j w[t][j] * Y[pair(t, j)], fixed order.
//
// Exactness on bf16 MFMA.  A dequantised weight w = s * (c - z) (fp16 scale,
// code offset of at most 5 significant bits) has at most 16 significant bits,
// so w = hi + lo with hi = its bf16 truncation and lo = w - hi, both exact
// bf16.  Activations are exact bf16 (fp32 inputs and the SwiGLU output are
// split into hi + lo the same way, relative error <= 2^-17).  Gate/up take two
// MFMAs per tile (x * w_hi + x * w_lo), down three (a_hi w_hi + a_hi w_lo +
// a_lo w_hi; the dropped a_lo w_lo is below 2^-16 relative).  Products are
// exact and accumulate in fp32 inside the MFMA across the whole K loop, so no
// per-block scaling pass is needed.
//
// MFMA v_mfma_f32_16x16x32_bf16, lane l: A row l%16 and B column l%16 hold
// K elements 8*(l/16) .. +7; D column l%16 holds rows 4*(l/16) .. +3.
#include "moe_device.h"
#include "moe_internal.h"

namespace moe {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));

constexpr int kRowsPerTile = 128;          // (token, slot) rows per tile
constexpr int kRowTiles = kRowsPerTile / 16;
constexpr int kPrefillThreads = 256;       // 4 waves, 16 output features each

LargeLayout large_layout(int T, int k, int E, int H, int FF, int FFs, int qtype) {
    LargeLayout L{};
    size_t off = 0;
    auto take = [&](size_t b) {
        size_t o = off;
        off = (off + b + 255) & ~(size_t)255;
        return o;
    };
    const int qk = codes_per_block(qtype);
    const size_t n = (size_t)T * k;
    const size_t P = n + (FFs ? (size_t)T : 0);
    const int ffmax = FFs > FF ? FFs : FF;
    const size_t max_tiles = (n + kRowsPerTile - 1) / kRowsPerTile + E + (FFs ? (T + kRowsPerTile - 1) / kRowsPerTile : 0);
    L.ids = take(n * 4);
    L.w = take(n * 4);
    L.counts = take((size_t)(E + 1) * 4);
    L.offsets = take((size_t)(E + 2) * 4);
    L.tiles = take(max_tiles * 3 * 4);   // expert, first row, rows
    L.ntiles = take(4);
    L.perm = take(P * 4);                // sorted row -> token
    L.inv = take(n * 4);                 // (token, slot) -> sorted row
    L.a = take(P * ffmax * 2 * 2);       // a_hi then a_lo planes, bf16
    L.ypair = take(P * (size_t)H * 4);
    L.max_tiles = max_tiles;
    L.total = off;
    (void)qk;
    return L;
}

struct PrefillParams {
    const void* const* table;
    const uint8_t* single;
    const uint8_t* shared;
    const void* x;            // [T][H]
    int T, E, k, H, FF, FFs, ffmax;
    float z;
    const int* ids;
    const float* w;
    int* counts;
    int* offsets;
    int* tiles;               // [max_tiles][3]
    int* ntiles;
    int* perm;
    int* inv;
    uint16_t* a_hi;
    uint16_t* a_lo;
    float* ypair;
    float* y;
    int max_tiles;
};

// ---------------------------------------------------------------------------------------------
// Bucketing: counts, offsets, tile list (one workgroup).
// ---------------------------------------------------------------------------------------------
__global__ void __launch_bounds__(1024) prefill_count_kernel(PrefillParams p) {
    __shared__ int hist[kMaxE + 1];
    __shared__ int tbase[kMaxE + 2];
    const int tid = threadIdx.x;
    const int n = p.T * p.k;
    for (int e = tid; e < p.E; e += blockDim.x) hist[e] = 0;
    __syncthreads();
    for (int i = tid; i < n; i += blockDim.x) atomicAdd(&hist[p.ids[i]], 1);   // counts: order-free
    __syncthreads();
    if (tid == 0) {
        int off = 0, tb = 0;
        for (int e = 0; e < p.E; ++e) {
            p.counts[e] = hist[e];
            p.offsets[e] = off;
            tbase[e] = tb;
            off += hist[e];
            tb += (hist[e] + kRowsPerTile - 1) / kRowsPerTile;
        }
        p.offsets[p.E] = off;
        tbase[p.E] = tb;
        int nt = tb;
        if (p.shared) nt += (p.T + kRowsPerTile - 1) / kRowsPerTile;
        *p.ntiles = nt;
    }
    __syncthreads();
    for (int e = tid; e < p.E; e += blockDim.x) {
        const int cnt = hist[e], o = p.offsets[e];
        for (int i = 0; i * kRowsPerTile < cnt; ++i) {
            int* t = p.tiles + 3 * (tbase[e] + i);
            t[0] = e;
            t[1] = o + i * kRowsPerTile;
            t[2] = min(kRowsPerTile, cnt - i * kRowsPerTile);
        }
    }
    if (p.shared) {
        const int base = tbase[p.E];
        for (int i = tid; i * kRowsPerTile < p.T; i += blockDim.x) {
            int* t = p.tiles + 3 * (base + i);
            t[0] = p.E;   // the shared expert
            t[1] = n + i * kRowsPerTile;
            t[2] = min(kRowsPerTile, p.T - i * kRowsPerTile);
        }
    }
}

// One wave per expert writes its pairs in (token, slot) order: a stable counting sort.
__global__ void __launch_bounds__(256) prefill_place_kernel(PrefillParams p) {
    const int lane = threadIdx.x & 63;
    const int e = blockIdx.x * 4 + (threadIdx.x >> 6);
    const int n = p.T * p.k;
    if (e < p.E) {
        int pos = p.offsets[e];
        for (int c = 0; c < n; c += 64) {
            const int q = c + lane;
            const bool match = q < n && p.ids[q] == e;
            const uint64_t m = __ballot(match);
            if (match) {
                const int r = pos + __popcll(m & ((1ull << lane) - 1));
                p.perm[r] = q / p.k;
                p.inv[q] = r;
            }
            pos += __popcll(m);
        }
    }
    if (p.shared)
        for (int t = blockIdx.x * blockDim.x + threadIdx.x; t < p.T; t += gridDim.x * blockDim.x) p.perm[n + t] = t;
}

// Identity routing for one expert's FFN: every token, expert 0, weight 1.
__global__ void prefill_identity_kernel(int* ids, float* w, int T) {
    const int t = blockIdx.x * blockDim.x + threadIdx.x;
    if (t < T) {
        ids[t] = 0;
        w[t] = 1.f;
    }
}

// ---------------------------------------------------------------------------------------------
// Operand helpers.
// ---------------------------------------------------------------------------------------------
__device__ __forceinline__ uint32_t pack_hi16(uint32_t a, uint32_t b) { return __builtin_amdgcn_perm(b, a, 0x07060302u); }

// 8 dequantised weights w_j = s * (c_j - z) as two exact bf16 terms (hi = the
// truncation, lo = the rest), K order j = 0..7.
__device__ __forceinline__ void weights_hi_lo(const float (&c)[8], float s, float zs, bf16x8_t& hi, bf16x8_t& lo) {
    uint32_t wb[8], lb[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) {
        const float w = __builtin_fmaf(c[j], s, -zs);                 // exact: <= 16 significant bits
        wb[j] = __float_as_uint(w);
        lb[j] = __float_as_uint(w - __uint_as_float(wb[j] & 0xFFFF0000u));   // exact remainder, <= 8 bits
    }
    uint32_t h[4], l[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        h[i] = pack_hi16(wb[2 * i], wb[2 * i + 1]);
        l[i] = pack_hi16(lb[2 * i], lb[2 * i + 1]);
    }
    hi = __builtin_bit_cast(bf16x8_t, *reinterpret_cast<const uint4*>(h));
    lo = __builtin_bit_cast(bf16x8_t, *reinterpret_cast<const uint4*>(l));
}

// Codes k = 8*kq .. 8*kq+7 of one 32-wide K step of a block, as floats.
template <int QT>
__device__ __forceinline__ void codes8(const uint8_t* chunk, int step, int kq, float (&c)[8]) {
    if constexpr (QT == 2) {   // 4-bit: one block = one K step; dword kq holds codes 8kq .. 8kq+7
        const uint32_t d = *reinterpret_cast<const uint32_t*>(chunk + 4 * kq);
#pragma unroll
        for (int j = 0; j < 8; ++j) c[j] = (float)((d >> (4 * j)) & 15u);
    } else {                   // 2-bit: 64 codes = two K steps; codes 32*step + 8*kq .. in dword 2*step + kq/2
        const uint32_t d = *reinterpret_cast<const uint32_t*>(chunk + 4 * (2 * step + kq / 2));
        const int sh = 16 * (kq & 1);
#pragma unroll
        for (int j = 0; j < 8; ++j) c[j] = (float)((d >> (sh + 2 * j)) & 3u);
    }
}

__device__ __forceinline__ float half_to_f32(uint16_t h) { return (float)__builtin_bit_cast(_Float16, h); }

__device__ __forceinline__ uint32_t f32_to_bf16_rne(float f) {
    const uint32_t u = __float_as_uint(f);
    return (u + 0x7FFFu + ((u >> 16) & 1u)) >> 16;
}

// ---------------------------------------------------------------------------------------------
// Gate/up + SwiGLU.
// grid.x: row tiles, grid.y: groups of 64 FF features (16 per wave).
// ---------------------------------------------------------------------------------------------
template <int QT, int NTERM>
__global__ void __launch_bounds__(kPrefillThreads, 2) prefill_gateup_kernel(PrefillParams p) {
    constexpr int QK = QT == 1 ? 64 : 32;
    constexpr int STEPS = QK / 32;   // 32-wide K steps per block
    const int tile = blockIdx.x;
    if (tile >= *p.ntiles) return;
    const int* td = p.tiles + 3 * tile;
    const int e = td[0], row0 = td[1], nrows = td[2];
    const bool sh = e == p.E;
    const int FFe = sh ? p.FFs : p.FF;
    const int f0 = blockIdx.y * 64;
    if (f0 >= FFe) return;
    const uint8_t* blob = sh ? p.shared : (p.table ? (const uint8_t*)p.table[e] : p.single);
    const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
    const int col = lane & 15, kq = lane >> 4;
    const int f = min(f0 + 16 * wv + col, FFe - 1);
    const int nblk = p.H / QK;
    const size_t plane = (size_t)FFe * nblk;
    const uint8_t* gcode = blob + (size_t)f * nblk * 16;
    const uint8_t* gscale = blob + plane * 16 + (size_t)f * nblk * 2;
    const uint8_t* ucode = blob + plane * 18 + (size_t)f * nblk * 16;
    const uint8_t* uscale = blob + plane * 18 + plane * 16 + (size_t)f * nblk * 2;
    const int nrt = (nrows + 15) / 16;

    // Tokens of this lane's A rows (row tile r, row l%16); rows past the tile repeat its last row.
    int tok[kRowTiles];
#pragma unroll
    for (int r = 0; r < kRowTiles; ++r) tok[r] = p.perm[row0 + min(16 * r + col, nrows - 1)];

    f32x4_t accg[kRowTiles], accu[kRowTiles];
#pragma unroll
    for (int r = 0; r < kRowTiles; ++r) {
        accg[r] = f32x4_t{0.f, 0.f, 0.f, 0.f};
        accu[r] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    }

    for (int b = 0; b < nblk; ++b) {
        const float sg = half_to_f32(*reinterpret_cast<const uint16_t*>(gscale + 2 * b));
        const float su = half_to_f32(*reinterpret_cast<const uint16_t*>(uscale + 2 * b));
#pragma unroll
        for (int st = 0; st < STEPS; ++st) {
            float cg[8], cu[8];
            codes8<QT>(gcode + 16 * b, st, kq, cg);
            codes8<QT>(ucode + 16 * b, st, kq, cu);
            bf16x8_t bgh, bgl, buh, bul;
            weights_hi_lo(cg, sg, p.z * sg, bgh, bgl);
            weights_hi_lo(cu, su, p.z * su, buh, bul);
            const int k0 = QK * b + 32 * st + 8 * kq;
#pragma unroll
            for (int r = 0; r < kRowTiles; ++r) {
                if (r < nrt) {
                    if constexpr (NTERM == 1) {
                        const uint4 xv = *reinterpret_cast<const uint4*>((const uint16_t*)p.x + (size_t)tok[r] * p.H + k0);
                        const bf16x8_t a = __builtin_bit_cast(bf16x8_t, xv);
                        accg[r] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, bgh, accg[r], 0, 0, 0);
                        accg[r] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, bgl, accg[r], 0, 0, 0);
                        accu[r] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, buh, accu[r], 0, 0, 0);
                        accu[r] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, bul, accu[r], 0, 0, 0);
                    } else {
                        // fp32 activations: two bf16 terms (hi + lo); x_lo * w_lo is dropped (< 2^-16).
                        const float* xs = (const float*)p.x + (size_t)tok[r] * p.H + k0;
                        const float4 v0 = *reinterpret_cast<const float4*>(xs);
                        const float4 v1 = *reinterpret_cast<const float4*>(xs + 4);
                        const float xv[8] = {v0.x, v0.y, v0.z, v0.w, v1.x, v1.y, v1.z, v1.w};
                        uint32_t hb[8], lb[8];
#pragma unroll
                        for (int j = 0; j < 8; ++j) {
                            hb[j] = __float_as_uint(xv[j]) & 0xFFFF0000u;
                            lb[j] = __float_as_uint(xv[j] - __uint_as_float(hb[j]));
                        }
                        uint32_t h4[4], l4[4];
#pragma unroll
                        for (int i = 0; i < 4; ++i) {
                            h4[i] = pack_hi16(hb[2 * i], hb[2 * i + 1]);
                            l4[i] = pack_hi16(lb[2 * i], lb[2 * i + 1]);
                        }
                        const bf16x8_t ah = __builtin_bit_cast(bf16x8_t, *reinterpret_cast<const uint4*>(h4));
                        const bf16x8_t al = __builtin_bit_cast(bf16x8_t, *reinterpret_cast<const uint4*>(l4));
                        accg[r] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ah, bgh, accg[r], 0, 0, 0);
                        accg[r] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ah, bgl, accg[r], 0, 0, 0);
                        accg[r] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(al, bgh, accg[r], 0, 0, 0);
                        accu[r] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ah, buh, accu[r], 0, 0, 0);
                        accu[r] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ah, bul, accu[r], 0, 0, 0);
                        accu[r] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(al, buh, accu[r], 0, 0, 0);
                    }
                }
            }
        }
    }
    // a = silu(g) * u as bf16 hi + lo, at [sorted row][feature].
    const int fo = f0 + 16 * wv + col;
    if (fo < FFe) {
#pragma unroll
        for (int r = 0; r < kRowTiles; ++r) {
            if (r < nrt) {
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const int rr = 16 * r + 4 * kq + i;
                    if (rr < nrows) {
                        const float g = accg[r][i], u = accu[r][i];
                        const float a = g / (1.f + expf(-g)) * u;
                        const uint32_t hi = f32_to_bf16_rne(a);
                        const uint32_t lo = f32_to_bf16_rne(a - __uint_as_float(hi << 16));
                        const size_t o = (size_t)(row0 + rr) * p.ffmax + fo;
                        p.a_hi[o] = (uint16_t)hi;
                        p.a_lo[o] = (uint16_t)lo;
                    }
                }
            }
        }
    }
}

// ---------------------------------------------------------------------------------------------
// Down projection: Y[row][h] = sum_f a[row][f] W_d[h][f].
// grid.x: row tiles, grid.y: groups of 64 H features.
// ---------------------------------------------------------------------------------------------
template <int QT>
__global__ void __launch_bounds__(kPrefillThreads, 2) prefill_down_kernel(PrefillParams p) {
    constexpr int QK = QT == 1 ? 64 : 32;
    constexpr int STEPS = QK / 32;
    const int tile = blockIdx.x;
    if (tile >= *p.ntiles) return;
    const int* td = p.tiles + 3 * tile;
    const int e = td[0], row0 = td[1], nrows = td[2];
    const bool sh = e == p.E;
    const int FFe = sh ? p.FFs : p.FF;
    const int h0 = blockIdx.y * 64;
    if (h0 >= p.H) return;
    const uint8_t* blob = sh ? p.shared : (p.table ? (const uint8_t*)p.table[e] : p.single);
    const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
    const int col = lane & 15, kq = lane >> 4;
    const int h = min(h0 + 16 * wv + col, p.H - 1);
    const int nblk = FFe / QK;
    const uint8_t* dcode = blob + (size_t)2 * FFe * (p.H / QK) * 18;
    const uint8_t* dscale = dcode + (size_t)p.H * nblk * 16;
    const uint8_t* hcode = dcode + (size_t)h * nblk * 16;
    const uint8_t* hscale = dscale + (size_t)h * nblk * 2;
    const int nrt = (nrows + 15) / 16;

    int arow[kRowTiles];
#pragma unroll
    for (int r = 0; r < kRowTiles; ++r) arow[r] = row0 + min(16 * r + col, nrows - 1);

    f32x4_t acc[kRowTiles];
#pragma unroll
    for (int r = 0; r < kRowTiles; ++r) acc[r] = f32x4_t{0.f, 0.f, 0.f, 0.f};

    for (int b = 0; b < nblk; ++b) {
        const float s = half_to_f32(*reinterpret_cast<const uint16_t*>(hscale + 2 * b));
#pragma unroll
        for (int st = 0; st < STEPS; ++st) {
            float c[8];
            codes8<QT>(hcode + 16 * b, st, kq, c);
            bf16x8_t bh, bl;
            weights_hi_lo(c, s, p.z * s, bh, bl);
            const int k0 = QK * b + 32 * st + 8 * kq;
#pragma unroll
            for (int r = 0; r < kRowTiles; ++r) {
                if (r < nrt) {
                    const size_t o = (size_t)arow[r] * p.ffmax + k0;
                    const bf16x8_t ah = __builtin_bit_cast(bf16x8_t, *reinterpret_cast<const uint4*>(p.a_hi + o));
                    const bf16x8_t al = __builtin_bit_cast(bf16x8_t, *reinterpret_cast<const uint4*>(p.a_lo + o));
                    acc[r] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ah, bh, acc[r], 0, 0, 0);
                    acc[r] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ah, bl, acc[r], 0, 0, 0);
                    acc[r] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(al, bh, acc[r], 0, 0, 0);
                }
            }
        }
    }
    const int ho = h0 + 16 * wv + col;
    if (ho < p.H) {
#pragma unroll
        for (int r = 0; r < kRowTiles; ++r) {
            if (r < nrt) {
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const int rr = 16 * r + 4 * kq + i;
                    if (rr < nrows) p.ypair[(size_t)(row0 + rr) * p.H + ho] = acc[r][i];
                }
            }
        }
    }
}

// y[t][h] = shared(t)[h] + sum_j w[t][j] * Y[pair(t, j)][h], in this order.
__global__ void __launch_bounds__(256) prefill_combine_kernel(PrefillParams p) {
    const size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
    const size_t n4 = (size_t)p.T * p.H / 4;
    if (i >= n4) return;
    const int t = (int)(i * 4 / p.H), h = (int)(i * 4 - (size_t)t * p.H);
    float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
    if (p.shared) acc = *reinterpret_cast<const float4*>(p.ypair + (size_t)(p.T * p.k + t) * p.H + h);
    for (int j = 0; j < p.k; ++j) {
        const float wt = p.w[t * p.k + j];
        const float4 v = *reinterpret_cast<const float4*>(p.ypair + (size_t)p.inv[t * p.k + j] * p.H + h);
        acc.x = __builtin_fmaf(wt, v.x, acc.x);
        acc.y = __builtin_fmaf(wt, v.y, acc.y);
        acc.z = __builtin_fmaf(wt, v.z, acc.z);
        acc.w = __builtin_fmaf(wt, v.w, acc.w);
    }
    *reinterpret_cast<float4*>(p.y + (size_t)t * p.H + h) = acc;
}

// ---------------------------------------------------------------------------------------------
// Host orchestration.
// ---------------------------------------------------------------------------------------------
hipError_t launch_prefill_layer(const void* const* table, const void* single, const void* shared, int qtype, float z,
                                int H, int FF, int FFs, const void* x, int x_dtype, const float* logits, int T, int E,
                                int k, int renorm, int identity, int* ids_out, float* w_out, const LargeLayout& L,
                                char* ws, float* y, hipStream_t s, StageMarks* marks) {
    PrefillParams p{};
    p.table = table;
    p.single = (const uint8_t*)single;
    p.shared = (const uint8_t*)shared;
    p.x = x;
    p.T = T;
    p.E = E;
    p.k = k;
    p.H = H;
    p.FF = FF;
    p.FFs = FFs;
    p.ffmax = FFs > FF ? FFs : FF;
    p.z = z;
    int* ids = ids_out ? ids_out : (int*)(ws + L.ids);
    float* w = w_out ? w_out : (float*)(ws + L.w);
    p.ids = ids;
    p.w = w;
    p.counts = (int*)(ws + L.counts);
    p.offsets = (int*)(ws + L.offsets);
    p.tiles = (int*)(ws + L.tiles);
    p.ntiles = (int*)(ws + L.ntiles);
    p.perm = (int*)(ws + L.perm);
    p.inv = (int*)(ws + L.inv);
    const size_t P = (size_t)T * k + (FFs ? (size_t)T : 0);
    p.a_hi = (uint16_t*)(ws + L.a);
    p.a_lo = p.a_hi + P * p.ffmax;
    p.ypair = (float*)(ws + L.ypair);
    p.y = y;
    p.max_tiles = (int)L.max_tiles;

    stage_mark(marks, s);
    if (identity)
        hipLaunchKernelGGL(prefill_identity_kernel, dim3((T + 255) / 256), dim3(256), 0, s, ids, w, T);
    else
        launch_route_topk(logits, T, E, k, renorm, ids, w, s);
    stage_mark(marks, s);
    hipLaunchKernelGGL(prefill_count_kernel, dim3(1), dim3(1024), 0, s, p);
    stage_mark(marks, s);
    hipLaunchKernelGGL(prefill_place_kernel, dim3((E + 3) / 4), dim3(256), 0, s, p);
    stage_mark(marks, s);
    const dim3 g_gu(p.max_tiles, (p.ffmax + 63) / 64), g_dn(p.max_tiles, (H + 63) / 64);
    if (qtype == 2) {
        if (x_dtype == 1)
            hipLaunchKernelGGL((prefill_gateup_kernel<2, 1>), g_gu, dim3(kPrefillThreads), 0, s, p);
        else
            hipLaunchKernelGGL((prefill_gateup_kernel<2, 2>), g_gu, dim3(kPrefillThreads), 0, s, p);
        stage_mark(marks, s);
        hipLaunchKernelGGL((prefill_down_kernel<2>), g_dn, dim3(kPrefillThreads), 0, s, p);
    } else {
        if (x_dtype == 1)
            hipLaunchKernelGGL((prefill_gateup_kernel<1, 1>), g_gu, dim3(kPrefillThreads), 0, s, p);
        else
            hipLaunchKernelGGL((prefill_gateup_kernel<1, 2>), g_gu, dim3(kPrefillThreads), 0, s, p);
        stage_mark(marks, s);
        hipLaunchKernelGGL((prefill_down_kernel<1>), g_dn, dim3(kPrefillThreads), 0, s, p);
    }
    stage_mark(marks, s);
    const size_t n4 = (size_t)T * H / 4;
    hipLaunchKernelGGL(prefill_combine_kernel, dim3((unsigned)((n4 + 255) / 256)), dim3(256), 0, s, p);
    stage_mark(marks, s);
    return hipGetLastError();
}

}  // namespace moe
