// Prefill path (T > 8 tokens): expert-major grouped GEMMs on the matrix cores.
//
// What is computed is the same layer as on the decode path (Krasis white paper
// 5.3; kairos-engine README "The MoE forward": the batch is bucketed by expert
// and each expert runs one GEMM over every token that chose it; "Prefill and
// decode are different machines": prefill dequantises and feeds the tensor
// cores).  Stages on the caller's stream:
//   1. route    : top-k per token (the decode path's wave top-k), or the
//                 caller-supplied routing copied and checked.
//   2. count    : per-expert counts, offsets and a list of row tiles (<= 128
//                 (token, slot) rows of one expert each).
//   3. place    : the sorted position of every pair, a stable counting sort in
//                 two launches over blocks of pairs (block counts, then
//                 positions); then the activations are converted (3b).
//   3b. xprep   : each token's activations as fp16 times a power of two.
//   4. gate/up  : per row tile and 256 features, G = X W_g^T and U = X W_u^T
//                 on MFMA, then a = act(G) * U, stored as bf16 hi + lo.
//   5. down     : per row tile and 256 outputs, Y = a W_d^T on MFMA.
//   6. combine  : y[t] = shared(t) + sum_j w[t][j] * Y[pair(t, j)], fixed order.
//
// Exact operands.  A weight is w = s * (c - z): an fp16 block scale s times a
// small half-integer c - z.  The matrix cores multiply by 2(c - z), an exact
// small integer, and the scale is applied once per block and output element in
// fp32 (acc += (s / 2) * P_block), so no weight is ever rounded.
//   gate/up: fp16 MFMA.  x * 2^-e (one e per token, 0 unless |x| >= 2^15) is
//     exact in fp16 for bf16 input (fp32 input: hi + lo, two MFMA passes); the
//     weight operand 2c - 2z comes from OR-ing the code into the mantissa of
//     1024.0 and one packed fp16 subtraction per two weights.
//   down: bf16 MFMA.  a is split into bf16 hi + lo (16 significant bits, two
//     MFMA passes); the weight operand c - z is converted through fp32.
// Products are exact and accumulate in fp32 inside each block.
//
// MFMA v_mfma_f32_32x32x16_{f16,bf16}, lane l: A row l%32 and B column l%32
// hold K elements 8*(l/32) .. +7; D column l%32 holds rows 8*(i/4) + 4*(l/32)
// + i%4 in register i.  Within a block, lane half h and K step s take codes
// QK/2*h + 8s .. +7 (any K order works when A and B agree on it).
//
// Tiles are mapped to workgroups so that each XCD (8 of them, workgroups
// dealt round-robin) runs a contiguous run of (row tile, column group) pairs:
// the column groups of one row tile share its activation rows in that XCD's L2.
#include <string.h>

#include <type_traits>

#include "moe_device.h"
#include "moe_internal.h"

namespace moe {

typedef _Float16 f16x8_t __attribute__((ext_vector_type(8)));
typedef _Float16 f16x2_t __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));

constexpr int kRowsPerTile = 128;          // (token, slot) rows per tile
constexpr int kGuThreads = 512;            // gate/up workgroup: 8 waves
constexpr int kGuFeatures = 256;           // features per gate/up workgroup (32 per wave)
constexpr int kDnThreads = 512;            // down workgroup: 8 waves
constexpr int kDnCols = 512;               // outputs per down workgroup (64 per wave)
constexpr int kPlaceBlock = 1024;          // (token, slot) pairs per placement block

LargeLayout large_layout(int T, int k, int E, int H, int FF, int FFs, int qtype) {
    LargeLayout L{};
    size_t off = small_fixed_bytes(k, H, FF, FFs, qtype);   // the decode path's sync words and `a` stay untouched
    auto take = [&](size_t b) {
        size_t o = off;
        off = (off + b + 255) & ~(size_t)255;
        return o;
    };
    (void)qtype;
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
    L.bcount = take(((n + kPlaceBlock - 1) / kPlaceBlock) * (size_t)E * 4);   // per block of pairs, per expert
    L.xq = take((size_t)2 * T * H * 2 + 256);   // + slack: the last chunk of the last row reads past H
    L.xe = take((size_t)T * 4);
    L.a = take(P * ffmax * 2 * 2 + 256); // a_hi then a_lo planes, bf16 (+ slack as for xq)
    L.ypair = take(P * (size_t)H * 4);
    L.logits = take((size_t)T * E * 4);
    L.max_tiles = max_tiles;
    L.total = off;
    return L;
}

struct PrefillParams {
    const void* const* table;
    const uint8_t* single;
    const uint8_t* shared;
    const void* x;            // [T][H]
    int T, E, k, H, FF, FFs, ffmax;
    float z;
    uint32_t zc16;            // fp16 pair (-(1024 + 2z), -(1024 + 2z))
    int act;                  // gate activation (kActSilu / kActGeluTanh)
    int routed;               // caller-supplied routing: zero-weight pairs are skipped
    const float* down_scale;  // [E] per routed expert, or null
    const int* ids;
    const float* w;
    int* counts;
    int* offsets;
    int* tiles;               // [max_tiles][3]
    int* ntiles;
    int* perm;
    int* inv;
    int* bcount;              // [blocks][E] pairs of each expert in each block of kPlaceBlock pairs
    uint16_t* xq;             // [2][T][H] fp16
    int* xe;                  // [T]
    uint16_t* a_hi;
    uint16_t* a_lo;
    float* ypair;
    float* y;
    const int* err;           // the workspace's error word
    int max_tiles;
};

// A (token, slot) pair takes part: always with routing from logits; with
// caller-supplied routing (Krasis white paper 7.5: an omitted route is a
// zero-weight slot) when its weight is nonzero and its id in [0, E) (an id
// outside it was flagged by prefill_routed_kernel and fails the call).
__device__ __forceinline__ bool pair_on(const PrefillParams& p, int q) {
    if (!p.routed) return true;
    const int e = p.ids[q];
    return p.w[q] != 0.f && e >= 0 && e < p.E;
}

// ---------------------------------------------------------------------------------------------
// Bucketing: a stable counting sort of the (token, slot) pairs by expert, over
// blocks of kPlaceBlock pairs (the pairs of one expert stay in (token, slot)
// order).  Three launches: each block's count of every expert; the totals,
// offsets and tile list, and each block's base per expert; each pair's
// position.
// ---------------------------------------------------------------------------------------------
__global__ void __launch_bounds__(256) prefill_blockcount_kernel(PrefillParams p) {
    __shared__ int h[kMaxE];
    const int tid = threadIdx.x, b = blockIdx.x;
    const int n = p.T * p.k, q0 = b * kPlaceBlock, q1 = min(n, q0 + kPlaceBlock);
    for (int e = tid; e < p.E; e += 256) h[e] = 0;
    __syncthreads();
    for (int q = q0 + tid; q < q1; q += 256)
        if (pair_on(p, q)) atomicAdd(&h[p.ids[q]], 1);   // counts: order-free
    __syncthreads();
    for (int e = tid; e < p.E; e += 256) p.bcount[(size_t)b * p.E + e] = h[e];
}

// One workgroup: each expert's total over the blocks, the offsets (in expert
// order) and the tile list; then each block's count of an expert is replaced
// by that block's base for it, offset + the expert's pairs in earlier blocks.
__global__ void __launch_bounds__(1024) prefill_count_kernel(PrefillParams p) {
    static_assert(kMaxE <= 1024, "one thread per expert in the scan");
    __shared__ int hist[kMaxE + 1];
    __shared__ int off_l[kMaxE + 1];
    __shared__ int tbase[kMaxE + 2];
    const int tid = threadIdx.x;
    const int n = p.T * p.k;
    const int nb = (n + kPlaceBlock - 1) / kPlaceBlock;
    int cnt = 0, nt_e = 0;   // thread e: expert e's pairs and row tiles
    if (tid < p.E) {
        for (int b0 = 0; b0 < nb; b0 += 8) {   // eight block counts in flight at a time
            int c[8];
#pragma unroll
            for (int u = 0; u < 8; ++u) c[u] = b0 + u < nb ? p.bcount[(size_t)(b0 + u) * p.E + tid] : 0;
#pragma unroll
            for (int u = 0; u < 8; ++u) cnt += c[u];
        }
        nt_e = (cnt + kRowsPerTile - 1) / kRowsPerTile;
        hist[tid] = cnt;
        off_l[tid] = cnt;
        tbase[tid] = nt_e;
    }
    __syncthreads();
    // Inclusive scans of the pair and tile counts over the experts (integer
    // sums: exact in any order), then the exclusive offsets.
    for (int d = 1; d < p.E; d <<= 1) {
        int a = 0, t = 0;
        if (tid < p.E && tid >= d) {
            a = off_l[tid - d];
            t = tbase[tid - d];
        }
        __syncthreads();
        if (tid < p.E && tid >= d) {
            off_l[tid] += a;
            tbase[tid] += t;
        }
        __syncthreads();
    }
    int incl = 0, tincl = 0;
    if (tid < p.E) {
        incl = off_l[tid];
        tincl = tbase[tid];
    }
    __syncthreads();
    if (tid < p.E) {
        off_l[tid] = incl - cnt;
        tbase[tid] = tincl - nt_e;
        p.counts[tid] = cnt;
        p.offsets[tid] = incl - cnt;
        if (tid == p.E - 1) {
            off_l[p.E] = incl;
            tbase[p.E] = tincl;
            p.offsets[p.E] = incl;
            *p.ntiles = tincl + (p.shared ? (p.T + kRowsPerTile - 1) / kRowsPerTile : 0);
        }
    }
    __syncthreads();
    for (int e = tid; e < p.E; e += blockDim.x) {
        const int ce = hist[e], o = off_l[e];
        for (int i = 0; i * kRowsPerTile < ce; ++i) {
            int* t = p.tiles + 3 * (tbase[e] + i);
            t[0] = e;
            t[1] = o + i * kRowsPerTile;
            t[2] = min(kRowsPerTile, ce - i * kRowsPerTile);
        }
        int run = o;
        for (int b0 = 0; b0 < nb; b0 += 8) {
            int c[8];
#pragma unroll
            for (int u = 0; u < 8; ++u) c[u] = b0 + u < nb ? p.bcount[(size_t)(b0 + u) * p.E + e] : 0;
#pragma unroll
            for (int u = 0; u < 8; ++u) {
                if (b0 + u < nb) p.bcount[(size_t)(b0 + u) * p.E + e] = run;
                run += c[u];
            }
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

// A pair's position: its block's base for its expert, plus the pairs of that
// expert earlier in the block.  The block goes by in chunks of 256 pairs (one
// a thread); within a wave, the lanes holding the same expert are found with
// one ballot per bit of the expert id, and a lane's rank among them is the
// count of those below it; a wave's count per expert goes to LDS, where the
// later waves of the chunk, and then the running count of the block, take it.
__global__ void __launch_bounds__(256) prefill_place_kernel(PrefillParams p) {
    __shared__ int run[kMaxE];        // the block's base + its pairs in earlier chunks, per expert
    __shared__ int wc[4][kMaxE];      // this chunk: each wave's pairs of each expert
    const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6, b = blockIdx.x;
    const int n = p.T * p.k, q0 = b * kPlaceBlock, len = min(kPlaceBlock, n - q0);
    for (int e = tid; e < p.E; e += 256) {
        run[e] = p.bcount[(size_t)b * p.E + e];
#pragma unroll
        for (int w = 0; w < 4; ++w) wc[w][e] = 0;
    }
    const int nbits = p.E > 1 ? 32 - __clz(p.E - 1) : 0;
    __syncthreads();
    for (int c0 = 0; c0 < len; c0 += 256) {
        const int i = c0 + tid;
        const int e = (i < len && pair_on(p, q0 + i)) ? p.ids[q0 + i] : -1;
        uint64_t m = __ballot(e >= 0);   // every lane votes in each ballot
        for (int bit = 0; bit < nbits; ++bit) {
            const bool v = e >= 0 && ((e >> bit) & 1);
            const uint64_t bb = __ballot(v);
            m &= v ? bb : ~bb;
        }
        const int rw = lanes_below(m);   // for e >= 0: m holds the lanes whose expert is e
        if (e >= 0 && rw == 0) wc[wv][e] = __popcll(m);
        __syncthreads();
        if (e >= 0) {
            int pos = run[e] + rw;
            for (int w = 0; w < wv; ++w) pos += wc[w][e];
            p.perm[pos] = (q0 + i) / p.k;
            p.inv[q0 + i] = pos;
        }
        __syncthreads();
        if (e >= 0 && rw == 0) {
            atomicAdd(&run[e], __popcll(m));   // integer sums: order-free
            wc[wv][e] = 0;
        }
        __syncthreads();
    }
    if (p.shared && b == 0)
        for (int t = tid; t < p.T; t += 256) p.perm[n + t] = t;
}

// Caller-supplied routing: copied to the routing buffers the later stages
// read (and the caller's optional outputs); a nonzero weight on an id outside
// [0, E) flags kErrBadId in the workspace's error word, so the combine writes
// NaN.
__global__ void prefill_routed_kernel(const int* ids_in, const float* w_in, int n, int E, int* ids, float* w,
                                      int* err) {
    const int q = blockIdx.x * blockDim.x + threadIdx.x;
    if (q >= n) return;
    const int e = ids_in[q];
    const float wt = w_in[q];
    ids[q] = e;
    w[q] = wt;
    if (wt != 0.f && (e < 0 || e >= E)) flag_error(err, kErrBadId);
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
// Activations to fp16.  One workgroup per token: e = max(0, floor(log2 max|x|) - 14)
// keeps x * 2^-e below 2^15.  Within each group of G = 8 (4-bit) or 16 (2-bit)
// values, position 2q + r holds value q + r*G/2: the order in which the
// dequantised weight pairs come out of one code word.
// ---------------------------------------------------------------------------------------------
// The values of one 16-byte word of activations (8 bf16 or 4 fp32), widened.
template <int XDT>
__device__ __forceinline__ void word_values(const uint4 u, float* v) {
    const uint32_t w[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        if constexpr (XDT == 1) {
            v[2 * j] = __uint_as_float(w[j] << 16);
            v[2 * j + 1] = __uint_as_float(w[j] & 0xFFFF0000u);
        } else {
            v[j] = __uint_as_float(w[j]);
        }
    }
}

template <int QT, int XDT>
__global__ void __launch_bounds__(256) prefill_xprep_kernel(PrefillParams p) {
    constexpr int G = QT == 1 ? 16 : 8;
    constexpr int VPW = XDT == 1 ? 8 : 4;   // values per 16-byte word
    constexpr int WPG = G / VPW;             // words per group
    __shared__ uint32_t red[4];
    const int t = blockIdx.x;
    const int H = p.H;
    const size_t base = (size_t)t * H;
    // The row in 16-byte words (rows are 64-byte multiples, x is 16-byte aligned).
    const uint4* xr = reinterpret_cast<const uint4*>((const uint8_t*)p.x + base * (XDT == 1 ? 2 : 4));
    uint32_t mx = 0;   // |x| bit patterns order like their values (NaN above every number)
    for (int i = threadIdx.x; i < H / VPW; i += 256) {
        float v[VPW];
        word_values<XDT>(xr[i], v);
#pragma unroll
        for (int j = 0; j < VPW; ++j) {
            const uint32_t b = __float_as_uint(v[j]) & 0x7FFFFFFFu;
            mx = b > mx ? b : mx;
        }
    }
    mx = wave_max_u32(mx);
    if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = mx;
    __syncthreads();
    mx = max(max(red[0], red[1]), max(red[2], red[3]));
    const int eb = (int)(mx >> 23);
    const int e = (mx < 0x7F800000u && eb > 141) ? eb - 141 : 0;
    if (threadIdx.x == 0) p.xe[t] = e;
    _Float16* hi = (_Float16*)p.xq + base;
    _Float16* lo = (_Float16*)p.xq + (size_t)p.T * H + base;
    for (int g = threadIdx.x; g < H / G; g += 256) {
        float v[G];
#pragma unroll
        for (int q = 0; q < WPG; ++q) word_values<XDT>(xr[(size_t)g * WPG + q], v + q * VPW);
#pragma unroll
        for (int i = 0; i < G; ++i) v[i] = __builtin_ldexpf(v[i], -e);
        _Float16 oh[G], ol[G];
#pragma unroll
        for (int q = 0; q < G / 2; ++q) {
#pragma unroll
            for (int r = 0; r < 2; ++r) {
                const float f = v[q + r * (G / 2)];
                const _Float16 h = (_Float16)f;
                oh[2 * q + r] = h;
                ol[2 * q + r] = (_Float16)(f - (float)h);
            }
        }
#pragma unroll
        for (int i = 0; i < G; i += 8) {
            *reinterpret_cast<f16x8_t*>(hi + (size_t)g * G + i) =
                f16x8_t{oh[i], oh[i + 1], oh[i + 2], oh[i + 3], oh[i + 4], oh[i + 5], oh[i + 6], oh[i + 7]};
            if constexpr (XDT == 0)
                *reinterpret_cast<f16x8_t*>(lo + (size_t)g * G + i) =
                    f16x8_t{ol[i], ol[i + 1], ol[i + 2], ol[i + 3], ol[i + 4], ol[i + 5], ol[i + 6], ol[i + 7]};
        }
    }
}

// ---------------------------------------------------------------------------------------------
// Shared pieces of the two GEMM kernels.
// ---------------------------------------------------------------------------------------------
__device__ __forceinline__ float half_to_f32(uint16_t h) { return (float)__builtin_bit_cast(_Float16, h); }

__device__ __forceinline__ uint32_t f32_to_bf16_rne(float f) {
    const uint32_t u = __float_as_uint(f);
    return (u + 0x7FFFu + ((u >> 16) & 1u)) >> 16;
}


// Direct global -> LDS copy of 16 bytes per lane; lane i lands at dst + 16 i.
__device__ __forceinline__ void load_lds16(const void* src, uint8_t* dst_wave) {
    __builtin_amdgcn_global_load_lds(src, (__attribute__((address_space(3))) void*)dst_wave, 16, 0, 0);
}

// A load the compiler knows reads global memory (a pointer taken from the
// expert table is otherwise generic, and a generic load could read LDS, which
// would make it wait for the LDS copies in flight).
__device__ __forceinline__ uint32_t ldg_u16(const uint8_t* base, uint32_t off) {
    return *(const __attribute__((address_space(1))) uint16_t*)(base + off);
}

typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
__device__ __forceinline__ uint4 ldg_u128(const uint8_t* base, uint32_t off) {
    const u32x4_t v = *(const __attribute__((address_space(1))) u32x4_t*)(base + off);
    return uint4{v[0], v[1], v[2], v[3]};
}

__device__ __forceinline__ void wait_loads() { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); }

// XCD-contiguous mapping of the 1-D grid onto n logical work items; -1 = no work.
__device__ __forceinline__ int xcd_item(int n) {
    const int per = (n + 7) >> 3;
    const int j = (int)(blockIdx.x >> 3);
    if (j >= per) return -1;
    const int L = (int)(blockIdx.x & 7) * per + j;
    return L < n ? L : -1;
}

// fp16 weight operand 2(c - z) of one K step from one 32-bit code word.
//   4-bit: word = codes 0..7; pairs (q, q + 4), q = 0..3.
//   2-bit: word = codes 0..15; step half u takes pairs (q, q + 8), q = 4u .. 4u + 3.
template <int QT>
__device__ __forceinline__ f16x8_t weights_f16(uint32_t d, int u, uint32_t magic_v, f16x2_t zc) {
    uint32_t w[4];
    if constexpr (QT == 2) {
        w[0] = and_or(d << 1, 0x001E001Eu, magic_v);
        w[1] = and_or(d >> 3, 0x001E001Eu, magic_v);
        w[2] = and_or(d >> 7, 0x001E001Eu, magic_v);
        w[3] = and_or(d >> 11, 0x001E001Eu, magic_v);
        (void)u;
    } else {
        if (u == 0) {
            w[0] = and_or(d << 1, 0x00060006u, magic_v);
            w[1] = and_or(d >> 1, 0x00060006u, magic_v);
            w[2] = and_or(d >> 3, 0x00060006u, magic_v);
            w[3] = and_or(d >> 5, 0x00060006u, magic_v);
        } else {
            w[0] = and_or(d >> 7, 0x00060006u, magic_v);
            w[1] = and_or(d >> 9, 0x00060006u, magic_v);
            w[2] = and_or(d >> 11, 0x00060006u, magic_v);
            w[3] = and_or(d >> 13, 0x00060006u, magic_v);
        }
    }
    f16x2_t h[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) h[i] = __builtin_bit_cast(f16x2_t, w[i]) + zc;   // exact: small integers
    return f16x8_t{h[0][0], h[0][1], h[1][0], h[1][1], h[2][0], h[2][1], h[3][0], h[3][1]};
}

// bf16 weight operand c - z of one K step, natural code order: 8 codes at bits
// 4j (4-bit) or 2j + shift (2-bit).
template <int QT>
__device__ __forceinline__ bf16x8_t weights_bf16(uint32_t d, int u, float z) {
    float c[8];
    if constexpr (QT == 2) {
        const uint32_t lo = d & 0x0F0F0F0Fu, hi = (d >> 4) & 0x0F0F0F0Fu;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            c[2 * i] = (float)((lo >> (8 * i)) & 0xFFu);
            c[2 * i + 1] = (float)((hi >> (8 * i)) & 0xFFu);
        }
    } else {
        const uint32_t t = d >> (16 * u);
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            const uint32_t m = (t >> (2 * k)) & 0x03030303u;   // byte i: code 4i + k
            c[k] = (float)(m & 0xFFu);
            c[4 + k] = (float)((m >> 8) & 0xFFu);
        }
    }
    uint32_t w[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const float a = c[2 * i] - z, b = c[2 * i + 1] - z;   // exact half-integers
        w[i] = __builtin_amdgcn_perm(__float_as_uint(b), __float_as_uint(a), 0x07060302u);
    }
    return __builtin_bit_cast(bf16x8_t, *reinterpret_cast<const uint4*>(w));
}

// ---------------------------------------------------------------------------------------------
// LDS tiles of one K chunk, filled by direct global -> LDS copies (lane i of a
// copy instruction lands 16 i bytes after the instruction's base):
//   A: 128 rows of 16 pieces of 16 bytes (K chunk of NTERM planes), row pitch 17
//      pieces.  16 consecutive rows reading the same piece then start 68 dwords
//      apart, i.e. on 16 distinct 4-bank groups of the 64 banks.
//   B: weight rows of BPC code blocks (16 bytes each, a contiguous run in the
//      blob), row pitch BPITCH pieces (BPC + 1, or 3 for BPC = 1) for the same
//      reason.  Consecutive lanes copy one row's run.
// The padding pieces are filled with valid (unused) data, so every lane of every
// copy instruction is active.  Reads past a row's end in the last, partial
// chunk stay inside the buffers (slack after the activation planes, the scales
// plane after the codes) and are never used.
// ---------------------------------------------------------------------------------------------
constexpr int kApitch = 17;                           // pieces per A row in LDS
constexpr int kAbytes = kRowsPerTile * kApitch * 16;  // 34,816
constexpr int kAcopies = kRowsPerTile * kApitch / 64; // 34 copy instructions per chunk
static_assert(kRowsPerTile * kApitch % 64 == 0, "A copies cover whole instructions");

__host__ __device__ constexpr int bpitch(int bpc) { return bpc == 1 ? 3 : bpc + 1; }

// Gate/up + SwiGLU.  Workgroup (8 waves, one per CU): one row tile x 256
// features; wave w owns features 32w .. 32w + 31 of both matrices (NR row
// sub-tiles x {gate, up} MFMA tiles).  K chunk: 128 / NTERM activations per row
// (NTERM fp16 planes) and the matching BPC code blocks of the 512 weight rows
// (gate rows, then up rows); two buffers, one barrier per chunk.
template <int QT, int NTERM>
__global__ void __launch_bounds__(kGuThreads, 1) prefill_gateup_kernel(PrefillParams p) {
    constexpr int QK = QT == 1 ? 64 : 32;
    constexpr int KC = 128 / NTERM;          // activations per row per chunk
    constexpr int BPC = KC / QK;             // blocks per chunk
    constexpr int SPB = QK / 16;             // MFMA K steps per block
    constexpr int PPP = 16 / NTERM;          // A pieces per plane
    constexpr int BP = bpitch(BPC);
    constexpr int BROWS = 2 * kGuFeatures;
    constexpr int BUF = kAbytes + BROWS * BP * 16;
    // Two separately declared buffers: the compiler can then tell that reads of
    // one do not depend on the copies still landing in the other.
    __shared__ __attribute__((aligned(16))) uint8_t buf0[BUF];
    __shared__ __attribute__((aligned(16))) uint8_t buf1[BUF];
    __shared__ __attribute__((aligned(16))) int s_e[kRowsPerTile];
    const int nft = (p.ffmax + kGuFeatures - 1) / kGuFeatures;
    const int item = xcd_item(*p.ntiles * nft);
    if (item < 0) return;
    const int tile = item / nft, ft = item - tile * nft;
    const int* td = p.tiles + 3 * tile;
    const int e = td[0], row0 = td[1], nrows = td[2];
    const bool sh = e == p.E;
    const int FFe = sh ? p.FFs : p.FF;
    const int f0 = ft * kGuFeatures;
    if (f0 >= FFe) return;
    const uint8_t* blob = sh ? p.shared : (p.table ? (const uint8_t*)p.table[e] : p.single);
    const int H = p.H;
    const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
    const int col = lane & 31, hh = lane >> 5;
    const int nblk = H / QK;
    const size_t plane = (size_t)FFe * nblk;
    if (tid < kRowsPerTile) s_e[tid] = p.xe[p.perm[row0 + min(tid, nrows - 1)]];

    // A copies: wave w issues copies g = w + 8 j (g < 34); piece 64 g + lane is
    // row / 17, piece % 17 (piece 16: padding, copies piece 0 again).
    constexpr int AJ = (kAcopies + 7) / 8;
    uint32_t xoff[AJ];
#pragma unroll
    for (int j = 0; j < AJ; ++j) {
        const int P = 64 * (wv + 8 * j) + lane;
        const int row = min(P / kApitch, kRowsPerTile - 1), pc = P % kApitch;
        const int q = pc == 16 ? 0 : pc;
        xoff[j] = (uint32_t)((q / PPP) * p.T * H + p.perm[row0 + min(row, nrows - 1)] * H + 8 * (q % PPP));
    }
    // B copies: wave w fills rows 64 w .. 64 w + 63 with BP copies; piece 64 j + lane
    // of the wave is row 64 w + (64 j + lane) / BP, piece (64 j + lane) % BP.
    uint32_t boff[BP];
#pragma unroll
    for (int j = 0; j < BP; ++j) {
        const int L = 64 * j + lane;
        const int row = 64 * wv + L / BP, pc = L % BP;
        const int m = row / kGuFeatures, fr = min(f0 + row % kGuFeatures, FFe - 1);
        boff[j] = (uint32_t)(m * plane * 18 + ((size_t)fr * nblk + (pc < BPC ? pc : 0)) * 16);
    }
    const uint8_t* xq = (const uint8_t*)p.xq;
    // Copies j0 .. j1 - 1 of chunk c's weight codes (B) and activations (A), so
    // that they can spread over the previous chunk's blocks.
    auto issue_b = [&](int c, uint8_t* buf, int j0, int j1) {
        const uint32_t kb = (uint32_t)(c * BPC * 16);
#pragma unroll
        for (int j = 0; j < BP; ++j)
            if (j >= j0 && j < j1) load_lds16(blob + (boff[j] + kb), buf + kAbytes + (64 * wv * BP + 64 * j) * 16);
    };
    auto issue_a = [&](int c, uint8_t* buf, int j0, int j1) {
        const uint32_t k0 = (uint32_t)(c * KC);
#pragma unroll
        for (int j = 0; j < AJ; ++j)
            if (j >= j0 && j < j1 && wv + 8 * j < kAcopies) load_lds16(xq + 2 * (xoff[j] + k0), buf + 1024 * (wv + 8 * j));
    };
    // Scales of this lane's gate and up rows in registers, 8 blocks (16 bytes,
    // CPL chunks) at a time: one 16-byte load per row when a row's scales are
    // 16-byte aligned (nblk a multiple of 8; the chunk count is then a multiple
    // of CPL), else 2-byte loads clamped to the row.
    constexpr int CPL = 8 / BPC;
    const int fl = min(f0 + 32 * wv + col, FFe - 1);
    const uint32_t gsoff = (uint32_t)(plane * 16 + (size_t)fl * nblk * 2);
    const uint32_t usoff = gsoff + (uint32_t)(plane * 18);
    const bool s16 = (nblk & 7) == 0;
    uint4 svg, svu;
    auto load_s8 = [&](int q) {
        if (s16) {
            svg = ldg_u128(blob, gsoff + 16u * (uint32_t)q);
            svu = ldg_u128(blob, usoff + 16u * (uint32_t)q);
        } else {
            uint32_t hg[8], hu[8];
#pragma unroll
            for (int j = 0; j < 8; ++j) {
                const uint32_t blk = (uint32_t)min(8 * q + j, nblk - 1);
                hg[j] = ldg_u16(blob, gsoff + 2 * blk);
                hu[j] = ldg_u16(blob, usoff + 2 * blk);
            }
            svg = uint4{hg[0] | hg[1] << 16, hg[2] | hg[3] << 16, hg[4] | hg[5] << 16, hg[6] | hg[7] << 16};
            svu = uint4{hu[0] | hu[1] << 16, hu[2] | hu[3] << 16, hu[4] | hu[5] << 16, hu[6] | hu[7] << 16};
        }
    };
    // This lane's LDS read bases: A row col (+ 32 r rows), B rows of its features.
    const uint32_t a_base = (uint32_t)(col * kApitch * 16 + (QK / 2) * hh * 2);
    // (B: this lane's half of each 16-byte block, bytes 8 hh .. 8 hh + 7)
    const uint32_t g_base = (uint32_t)(kAbytes + (32 * wv + col) * BP * 16 + 8 * hh);
    const uint32_t u_base = g_base + (uint32_t)(kGuFeatures * BP * 16);

    // The chunk loop and epilogue, specialised on the number NR of 32-row MFMA
    // sub-tiles that hold rows (a tile of n rows needs ceil(n / 32)).
    auto run = [&](auto nr_c) {
        constexpr int NR = decltype(nr_c)::value;
        f32x16_t accg[NR], accu[NR];
#pragma unroll
        for (int r = 0; r < NR; ++r)
#pragma unroll
            for (int i = 0; i < 16; ++i) {
                accg[r][i] = 0.f;
                accu[r][i] = 0.f;
            }
        const uint32_t magic_v = [] {
            uint32_t m;
            asm volatile("v_mov_b32 %0, 0x64006400" : "=v"(m));
            return m;
        }();
        const f16x2_t zc = __builtin_bit_cast(f16x2_t, p.zc16);
        const f32x16_t zero = {};
        const int nchunks = (H + KC - 1) / KC;
        auto chunk = [&](int c, const uint8_t* buf, uint8_t* next) {
            wait_loads();
            __syncthreads();
            // This chunk's block scales s / 2 (the weight operands are 2(c - z)),
            // taken from the 8-block registers before the group's last chunk
            // refills them.
            const int cq = c % CPL;
            float fg[BPC], fu[BPC];
#pragma unroll
            for (int i = 0; i < BPC; ++i) {
                const int bi = cq * BPC + i, wsel = bi >> 1, sh = 16 * (bi & 1);
                const uint32_t wg = wsel == 0 ? svg.x : wsel == 1 ? svg.y : wsel == 2 ? svg.z : svg.w;
                const uint32_t wu = wsel == 0 ? svu.x : wsel == 1 ? svu.y : wsel == 2 ? svu.z : svu.w;
                fg[i] = 0.5f * half_to_f32((uint16_t)(wg >> sh));
                fu[i] = 0.5f * half_to_f32((uint16_t)(wu >> sh));
            }
            if (cq == CPL - 1 && c + 1 < nchunks) load_s8((c + 1) / CPL);
            // Chunk c + 1's copies go out two or three at a time at the starts of
            // this chunk's blocks (codes first: they come from HBM), so that no
            // wave stalls behind a burst of them; every chunk but a row's last
            // has all its blocks.  (Copies issued between a block's LDS reads
            // would make the compiler wait for them before those reads.)
            const bool more = c + 1 < nchunks;
            // Each block's products summed from zero, then scaled by s / 2 once per
            // output element, in fp32.
#pragma unroll
            for (int i = 0; i < BPC; ++i) {
                if (c * BPC + i >= nblk) break;
                if constexpr (BPC == 4) {
                    if (more && i == 0) issue_b(c + 1, next, 0, 3);
                    if (more && i == 1) issue_b(c + 1, next, 3, BP);
                    if (more && i == 2) issue_a(c + 1, next, 0, 3);
                    if (more && i == 3) issue_a(c + 1, next, 3, AJ);
                } else {
                    if (more && i == 0) issue_b(c + 1, next, 0, BP);
                    if (more && i == (BPC > 1 ? 1 : 0)) issue_a(c + 1, next, 0, AJ);
                }
                const uint2 g2 = *reinterpret_cast<const uint2*>(buf + g_base + i * 16);
                const uint2 u2 = *reinterpret_cast<const uint2*>(buf + u_base + i * 16);
                const uint32_t gw[2] = {g2.x, g2.y};
                const uint32_t uw[2] = {u2.x, u2.y};
                f16x8_t wg[SPB], wu[SPB];
#pragma unroll
                for (int s = 0; s < SPB; ++s) {
                    const int wd = (QT == 2) ? s : (s >> 1);
                    wg[s] = weights_f16<QT>(gw[wd], s & 1, magic_v, zc);
                    wu[s] = weights_f16<QT>(uw[wd], s & 1, magic_v, zc);
                }
#pragma unroll
                for (int r = 0; r < NR; ++r) {
                    f32x16_t pg = zero, pu = zero;
#pragma unroll
                    for (int s = 0; s < SPB; ++s) {
#pragma unroll
                        for (int t = 0; t < NTERM; ++t) {
                            // activations K = QK i + QK/2 hh + 8 s of plane t (hh is in a_base)
                            const int off = 32 * r * kApitch * 16 + (PPP * t + (i * QK + 8 * s) / 8) * 16;
                            const f16x8_t av = *reinterpret_cast<const f16x8_t*>(buf + a_base + off);
                            pg = __builtin_amdgcn_mfma_f32_32x32x16_f16(av, wg[s], pg, 0, 0, 0);
                            pu = __builtin_amdgcn_mfma_f32_32x32x16_f16(av, wu[s], pu, 0, 0, 0);
                        }
                    }
#pragma unroll
                    for (int k = 0; k < 16; ++k) {
                        accg[r][k] = __builtin_fmaf(fg[i], pg[k], accg[r][k]);
                        accu[r][k] = __builtin_fmaf(fu[i], pu[k], accu[r][k]);
                    }
                }
            }
        };
        issue_b(0, buf0, 0, BP);
        issue_a(0, buf0, 0, AJ);
        load_s8(0);
        for (int c = 0; c < nchunks; c += 2) {
            chunk(c, buf0, buf1);
            if (c + 1 < nchunks) chunk(c + 1, buf1, buf0);
        }

        // a = silu(g) * u with g, u rescaled by the token's 2^e; stored as bf16 hi + lo.
        // The row exponents are read before any store (an LDS read here waits for
        // all outstanding memory operations, stores included).
        int ex[NR][16];
#pragma unroll
        for (int r = 0; r < NR; ++r)
#pragma unroll
            for (int kk = 0; kk < 4; ++kk) {
                const int4 e4 = *reinterpret_cast<const int4*>(s_e + 32 * r + 8 * kk + 4 * hh);
                ex[r][4 * kk] = e4.x;
                ex[r][4 * kk + 1] = e4.y;
                ex[r][4 * kk + 2] = e4.z;
                ex[r][4 * kk + 3] = e4.w;
            }
        const int fo = f0 + 32 * wv + col;
        if (fo < FFe) {
#pragma unroll
            for (int r = 0; r < NR; ++r) {
#pragma unroll
                for (int k = 0; k < 16; ++k) {
                    const int rr = 32 * r + 8 * (k >> 2) + 4 * hh + (k & 3);
                    if (rr < nrows) {
                        const float g = __builtin_ldexpf(accg[r][k], ex[r][k]);
                        const float u = __builtin_ldexpf(accu[r][k], ex[r][k]);
                        // act(g) = g / (1 + e^-b) (b = g for SiLU; see gate_arg) with the
                        // hardware exp2 and reciprocal (~1 ulp each)
                        const float a = g * __builtin_amdgcn_rcpf(1.f + __builtin_amdgcn_exp2f(-1.44269504088896341f *
                                                                                               gate_arg(g, p.act))) * u;
                        const uint32_t ah = f32_to_bf16_rne(a);
                        const uint32_t al = f32_to_bf16_rne(a - __uint_as_float(ah << 16));
                        const size_t o = (size_t)(row0 + rr) * p.ffmax + fo;
                        p.a_hi[o] = (uint16_t)ah;
                        p.a_lo[o] = (uint16_t)al;
                    }
                }
            }
        }
    };
    switch ((nrows + 31) >> 5) {
        case 1: run(std::integral_constant<int, 1>{}); break;
        case 2: run(std::integral_constant<int, 2>{}); break;
        case 3: run(std::integral_constant<int, 3>{}); break;
        default: run(std::integral_constant<int, 4>{}); break;
    }
}

// ---------------------------------------------------------------------------------------------
// Down projection: Y[row][h] = sum_f a[row][f] W_d[h][f].  Workgroup (8 waves,
// one per CU): one row tile x 512 outputs; wave w owns outputs 64w .. 64w + 63
// (NR row sub-tiles x 2 column sub-tiles).  K chunk: 64 features of a_hi
// (pieces 0..7 of an A row) and a_lo (pieces 8..15), and the matching BPC code
// blocks of the 512 weight rows.
// ---------------------------------------------------------------------------------------------
template <int QT>
__global__ void __launch_bounds__(kDnThreads, 1) prefill_down_kernel(PrefillParams p) {
    constexpr int QK = QT == 1 ? 64 : 32;
    constexpr int KC = 64;
    constexpr int BPC = KC / QK;
    constexpr int SPB = QK / 16;
    constexpr int BP = bpitch(BPC);
    constexpr int BUF = kAbytes + kDnCols * BP * 16;
    __shared__ __attribute__((aligned(16))) uint8_t buf0[BUF];
    __shared__ __attribute__((aligned(16))) uint8_t buf1[BUF];
    const int H = p.H;
    const int nht = (H + kDnCols - 1) / kDnCols;
    const int item = xcd_item(*p.ntiles * nht);
    if (item < 0) return;
    const int tile = item / nht, ht = item - tile * nht;
    const int* td = p.tiles + 3 * tile;
    const int e = td[0], row0 = td[1], nrows = td[2];
    const bool sh = e == p.E;
    const int FFe = sh ? p.FFs : p.FF;
    const uint8_t* blob = sh ? p.shared : (p.table ? (const uint8_t*)p.table[e] : p.single);
    const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
    const int col = lane & 31, hh = lane >> 5;
    const int nblk = FFe / QK;
    const uint32_t dco = (uint32_t)((size_t)2 * FFe * (H / QK) * 18);   // down codes plane
    const uint32_t dso = dco + (uint32_t)((size_t)H * nblk * 16);       // down scales plane
    const int hbase = ht * kDnCols;

    constexpr int AJ = (kAcopies + 7) / 8;
    const uint8_t* abase = (const uint8_t*)p.a_hi;   // a_lo follows at a fixed distance
    const uint32_t aplane = (uint32_t)((const uint8_t*)p.a_lo - abase);
    uint32_t aoff[AJ];
#pragma unroll
    for (int j = 0; j < AJ; ++j) {
        const int P = 64 * (wv + 8 * j) + lane;
        const int row = min(P / kApitch, kRowsPerTile - 1), pc = P % kApitch;
        const int q = pc == 16 ? 0 : pc;
        aoff[j] = (q >> 3 ? aplane : 0u) + 2u * (uint32_t)((row0 + min(row, nrows - 1)) * p.ffmax + 8 * (q & 7));
    }
    uint32_t boff[BP];
#pragma unroll
    for (int j = 0; j < BP; ++j) {
        const int L = 64 * j + lane;
        const int hr = min(hbase + 64 * wv + L / BP, H - 1), pc = L % BP;
        boff[j] = dco + (uint32_t)(((size_t)hr * nblk + (pc < BPC ? pc : 0)) * 16);
    }
    // The copies of chunk c, weight codes (B) and `a` (A), issued separately so
    // that they spread over the previous chunk's blocks.
    auto issue_b = [&](int c, uint8_t* buf) {
        const uint32_t kb = (uint32_t)(c * BPC * 16);
#pragma unroll
        for (int j = 0; j < BP; ++j) load_lds16(blob + (boff[j] + kb), buf + kAbytes + (64 * wv * BP + 64 * j) * 16);
    };
    auto issue_a = [&](int c, uint8_t* buf) {
        const uint32_t k0 = (uint32_t)(c * KC * 2);
#pragma unroll
        for (int j = 0; j < AJ; ++j)
            if (wv + 8 * j < kAcopies) load_lds16(abase + (aoff[j] + k0), buf + 1024 * (wv + 8 * j));
    };
    // Scales of this lane's two output rows in registers, 8 blocks (CPL chunks)
    // at a time, as in the gate/up kernel.
    constexpr int CPL = 8 / BPC;
    uint32_t soff[2];
#pragma unroll
    for (int n = 0; n < 2; ++n)
        soff[n] = dso + (uint32_t)((size_t)min(hbase + 64 * wv + 32 * n + col, H - 1) * nblk * 2);
    const bool s16 = (nblk & 7) == 0;
    uint4 sv[2];
    auto load_s8 = [&](int q) {
#pragma unroll
        for (int n = 0; n < 2; ++n) {
            if (s16) {
                sv[n] = ldg_u128(blob, soff[n] + 16u * (uint32_t)q);
            } else {
                uint32_t h[8];
#pragma unroll
                for (int j = 0; j < 8; ++j) h[j] = ldg_u16(blob, soff[n] + 2u * (uint32_t)min(8 * q + j, nblk - 1));
                sv[n] = uint4{h[0] | h[1] << 16, h[2] | h[3] << 16, h[4] | h[5] << 16, h[6] | h[7] << 16};
            }
        }
    };
    const uint32_t a_base = (uint32_t)(col * kApitch * 16 + (QK / 2) * hh * 2);
    const uint32_t b_base = (uint32_t)(kAbytes + (64 * wv + col) * BP * 16 + 8 * hh);   // this lane's half-blocks

    auto run = [&](auto nr_c) {
        constexpr int NR = decltype(nr_c)::value;
        f32x16_t acc[NR][2];
#pragma unroll
        for (int r = 0; r < NR; ++r)
#pragma unroll
            for (int n = 0; n < 2; ++n)
#pragma unroll
                for (int i = 0; i < 16; ++i) acc[r][n][i] = 0.f;
        const f32x16_t zero = {};
        const float z = p.z;
        const int nchunks = (FFe + KC - 1) / KC;
        auto chunk = [&](int c, const uint8_t* buf, uint8_t* next) {
            wait_loads();
            __syncthreads();
            const int cq = c % CPL;
            float fs[2][BPC];
#pragma unroll
            for (int n = 0; n < 2; ++n)
#pragma unroll
                for (int i = 0; i < BPC; ++i) {
                    const int bi = cq * BPC + i, wsel = bi >> 1, sh = 16 * (bi & 1);
                    const uint32_t w = wsel == 0 ? sv[n].x : wsel == 1 ? sv[n].y : wsel == 2 ? sv[n].z : sv[n].w;
                    fs[n][i] = half_to_f32((uint16_t)(w >> sh));
                }
            if (cq == CPL - 1 && c + 1 < nchunks) load_s8((c + 1) / CPL);
            const bool more = c + 1 < nchunks;
#pragma unroll
            for (int i = 0; i < BPC; ++i) {
                if (c * BPC + i >= nblk) break;
                if (more && i == 0) issue_b(c + 1, next);
                if (more && i == (BPC > 1 ? 1 : 0)) issue_a(c + 1, next);
                bf16x8_t wb[2][SPB];
#pragma unroll
                for (int n = 0; n < 2; ++n) {
                    const uint2 d2 = *reinterpret_cast<const uint2*>(buf + b_base + (32 * n * BP + i) * 16);
                    const uint32_t dw[2] = {d2.x, d2.y};
#pragma unroll
                    for (int s = 0; s < SPB; ++s) wb[n][s] = weights_bf16<QT>(dw[(QT == 2) ? s : (s >> 1)], s & 1, z);
                }
#pragma unroll
                for (int r = 0; r < NR; ++r) {
                    bf16x8_t ah[SPB], al[SPB];
#pragma unroll
                    for (int s = 0; s < SPB; ++s) {
                        const int off = 32 * r * kApitch * 16 + ((i * QK + 8 * s) / 8) * 16;
                        ah[s] = *reinterpret_cast<const bf16x8_t*>(buf + a_base + off);
                        al[s] = *reinterpret_cast<const bf16x8_t*>(buf + a_base + off + 8 * 16);
                    }
#pragma unroll
                    for (int n = 0; n < 2; ++n) {
                        f32x16_t pp = zero;
#pragma unroll
                        for (int s = 0; s < SPB; ++s) {
                            pp = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ah[s], wb[n][s], pp, 0, 0, 0);
                            pp = __builtin_amdgcn_mfma_f32_32x32x16_bf16(al[s], wb[n][s], pp, 0, 0, 0);
                        }
#pragma unroll
                        for (int k = 0; k < 16; ++k) acc[r][n][k] = __builtin_fmaf(fs[n][i], pp[k], acc[r][n][k]);
                    }
                }
            }
        };
        issue_b(0, buf0);
        issue_a(0, buf0);
        load_s8(0);
        for (int c = 0; c < nchunks; c += 2) {
            chunk(c, buf0, buf1);
            if (c + 1 < nchunks) chunk(c + 1, buf1, buf0);
        }
#pragma unroll
        for (int n = 0; n < 2; ++n) {
            const int ho = hbase + 64 * wv + 32 * n + col;
            if (ho < H) {
#pragma unroll
                for (int r = 0; r < NR; ++r)
#pragma unroll
                    for (int k = 0; k < 16; ++k) {
                        const int rr = 32 * r + 8 * (k >> 2) + 4 * hh + (k & 3);
                        if (rr < nrows) p.ypair[(size_t)(row0 + rr) * H + ho] = acc[r][n][k];
                    }
            }
        }
    };
    switch ((nrows + 31) >> 5) {
        case 1: run(std::integral_constant<int, 1>{}); break;
        case 2: run(std::integral_constant<int, 2>{}); break;
        case 3: run(std::integral_constant<int, 3>{}); break;
        default: run(std::integral_constant<int, 4>{}); break;
    }
}

// y[t][h] = shared(t)[h] + sum_j w[t][j] * Y[pair(t, j)][h], in this order.
// While the workspace's error word is set, every output is NaN.
typedef float f32x4 __attribute__((ext_vector_type(4)));

__global__ void __launch_bounds__(256) prefill_combine_kernel(PrefillParams p) {
    const size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
    const size_t n4 = (size_t)p.T * p.H / 4;
    if (i >= n4) return;
    if (load_error(p.err) != 0) {
        const float nan = __uint_as_float(0x7FC00000u);
        *reinterpret_cast<float4*>(p.y + i * 4) = make_float4(nan, nan, nan, nan);
        return;
    }
    const int t = (int)(i * 4 / p.H), h = (int)(i * 4 - (size_t)t * p.H);
    float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
    if (p.shared) acc = *reinterpret_cast<const float4*>(p.ypair + (size_t)(p.T * p.k + t) * p.H + h);
    // Eight slots at a time: their rows and weights, then all eight row loads,
    // then the sums in slot order (a skipped slot loads nothing and adds
    // nothing).
    constexpr int G = 8;
    for (int j0 = 0; j0 < p.k; j0 += G) {
        bool on[G];
        float wt[G];
        int row[G];
#pragma unroll
        for (int u = 0; u < G; ++u) {
            const int q = t * p.k + j0 + u;
            on[u] = j0 + u < p.k && pair_on(p, q);
            wt[u] = on[u] ? p.w[q] * (p.down_scale ? p.down_scale[p.ids[q]] : 1.f) : 0.f;
            row[u] = on[u] ? p.inv[q] : 0;
        }
        float4 v[G];
#pragma unroll
        for (int u = 0; u < G; ++u)
            if (on[u]) {   // rows read once: non-temporal
                const f32x4 q = __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(p.ypair + (size_t)row[u] * p.H + h));
                v[u] = make_float4(q[0], q[1], q[2], q[3]);
            } else {
                v[u] = make_float4(0.f, 0.f, 0.f, 0.f);
            }
#pragma unroll
        for (int u = 0; u < G; ++u) {
            if (!on[u]) continue;
            acc.x = __builtin_fmaf(wt[u], v[u].x, acc.x);
            acc.y = __builtin_fmaf(wt[u], v[u].y, acc.y);
            acc.z = __builtin_fmaf(wt[u], v[u].z, acc.z);
            acc.w = __builtin_fmaf(wt[u], v[u].w, acc.w);
        }
    }
    const f32x4 o = {acc.x, acc.y, acc.z, acc.w};
    __builtin_nontemporal_store(o, reinterpret_cast<f32x4*>(p.y + (size_t)t * p.H + h));
}

// ---------------------------------------------------------------------------------------------
// Host orchestration.
// ---------------------------------------------------------------------------------------------
static uint32_t f16_bits(float v) {   // exact for the values used here (integers below 2048)
    const _Float16 h = (_Float16)v;
    uint16_t b;
    memcpy(&b, &h, 2);
    return b;
}

template <int QT>
static void launch_gemms(const PrefillParams& p, int x_dtype, hipStream_t s, StageMarks* marks) {
    const int nft = (p.ffmax + kGuFeatures - 1) / kGuFeatures, nht = (p.H + kDnCols - 1) / kDnCols;
    const unsigned g_gu = (unsigned)((p.max_tiles * nft + 7) & ~7), g_dn = (unsigned)((p.max_tiles * nht + 7) & ~7);
    if (x_dtype == 1)
        hipLaunchKernelGGL((prefill_gateup_kernel<QT, 1>), dim3(g_gu), dim3(kGuThreads), 0, s, p);
    else
        hipLaunchKernelGGL((prefill_gateup_kernel<QT, 2>), dim3(g_gu), dim3(kGuThreads), 0, s, p);
    stage_mark(marks, s);
    hipLaunchKernelGGL((prefill_down_kernel<QT>), dim3(g_dn), dim3(kDnThreads), 0, s, p);
}

hipError_t launch_prefill_layer(const void* const* table, const void* single, const void* shared, int qtype, float z,
                                int H, int FF, int FFs, const void* x, int x_dtype, const float* logits, int T, int E,
                                int k, int renorm, int identity, const LayerOpts& o, int* ids_out, float* w_out,
                                const LargeLayout& L, char* ws, float* y, hipStream_t s, StageMarks* marks) {
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
    const uint32_t zb = f16_bits(-(1024.f + 2.f * z));
    p.zc16 = zb | (zb << 16);
    int* ids = ids_out ? ids_out : (int*)(ws + L.ids);
    float* w = w_out ? w_out : (float*)(ws + L.w);
    p.ids = ids;
    p.act = o.act;
    p.routed = o.ids_in != nullptr;
    p.down_scale = o.down_scale;
    p.w = w;
    p.counts = (int*)(ws + L.counts);
    p.offsets = (int*)(ws + L.offsets);
    p.tiles = (int*)(ws + L.tiles);
    p.ntiles = (int*)(ws + L.ntiles);
    p.perm = (int*)(ws + L.perm);
    p.inv = (int*)(ws + L.inv);
    p.bcount = (int*)(ws + L.bcount);
    p.xq = (uint16_t*)(ws + L.xq);
    p.xe = (int*)(ws + L.xe);
    const size_t P = (size_t)T * k + (FFs ? (size_t)T : 0);
    p.a_hi = (uint16_t*)(ws + L.a);
    p.a_lo = p.a_hi + P * p.ffmax;
    p.ypair = (float*)(ws + L.ypair);
    p.y = y;
    p.err = (const int*)ws + kErrWord;   // the GEMV path's synchronisation area starts every workspace
    p.max_tiles = (int)L.max_tiles;

    stage_mark(marks, s);
    if (identity)
        hipLaunchKernelGGL(prefill_identity_kernel, dim3((T + 255) / 256), dim3(256), 0, s, ids, w, T);
    else if (o.ids_in)
        hipLaunchKernelGGL(prefill_routed_kernel, dim3((T * k + 255) / 256), dim3(256), 0, s, o.ids_in, o.w_in, T * k,
                           E, ids, w, (int*)ws + kErrWord);
    else
        (void)launch_route_topk(logits, T, E, k, renorm, ids, w, s);
    stage_mark(marks, s);
    const unsigned n_pb = (unsigned)((T * k + kPlaceBlock - 1) / kPlaceBlock);
    hipLaunchKernelGGL(prefill_blockcount_kernel, dim3(n_pb), dim3(256), 0, s, p);
    hipLaunchKernelGGL(prefill_count_kernel, dim3(1), dim3(1024), 0, s, p);
    stage_mark(marks, s);
    hipLaunchKernelGGL(prefill_place_kernel, dim3(n_pb), dim3(256), 0, s, p);
    if (qtype == 2) {
        if (x_dtype == 1) hipLaunchKernelGGL((prefill_xprep_kernel<2, 1>), dim3(T), dim3(256), 0, s, p);
        else hipLaunchKernelGGL((prefill_xprep_kernel<2, 0>), dim3(T), dim3(256), 0, s, p);
    } else {
        if (x_dtype == 1) hipLaunchKernelGGL((prefill_xprep_kernel<1, 1>), dim3(T), dim3(256), 0, s, p);
        else hipLaunchKernelGGL((prefill_xprep_kernel<1, 0>), dim3(T), dim3(256), 0, s, p);
    }
    stage_mark(marks, s);
    if (qtype == 2) launch_gemms<2>(p, x_dtype, s, marks);
    else launch_gemms<1>(p, x_dtype, s, marks);
    stage_mark(marks, s);
    const size_t n4 = (size_t)T * H / 4;
    hipLaunchKernelGGL(prefill_combine_kernel, dim3((unsigned)((n4 + 255) / 256)), dim3(256), 0, s, p);
    stage_mark(marks, s);
    return hipGetLastError();
}

}  // namespace moe
