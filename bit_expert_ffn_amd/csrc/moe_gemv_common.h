// Shared device code of the GEMV kernels (one-token decode and verify
// windows): block dequantisation in registers, activation slices, the packed
// SwiGLU output words and column sums.
//
// Decode / verify path (T <= 8 tokens): dequant-fused GEMV over the selected
// experts' block-quantized gate/up/down matrices.
//
// What is computed (Krasis white paper 5.3; kairos-engine README "The MoE
// forward" and "Prefill and decode are different machines"): for every
// distinct selected expert e and the tokens routed to it,
//     a = silu(W_gate x) * (W_up x),   d = W_down a,
// then y[t] = shared(x[t]) + sum_j w[t][j] d_{ids[t][j]}[t].  The codes are
// read straight from HBM and dequantized in registers (the kairos README's
// "fused GEMV reads the codes straight from VRAM"); each distinct expert is
// read once for all the tokens of the window that chose it (Strata, "The plan:
// three destinations per expert").
//
// Layout of the work.  A workgroup of 256 threads owns a tile of output rows
// of one matrix.  Thread (rp, b) owns block column b (the same 16-byte code
// chunk position in every row) and row rp of each pass of P = 256 / nblk rows,
// so one pass reads P * nblk consecutive chunks: every wavefront load is a
// contiguous, 16-byte-per-lane read of the codes plane and a contiguous 2-byte
// read of the scales plane.  The thread keeps its slice of the activations
// (qk values per token) in registers for all its rows.  Partial dot products
// go through LDS and are summed per row in block order by one thread, so the
// summation order of every output is fixed (deterministic, and independent of
// which other tokens share the expert).
//
// Dequantisation in registers.  weight = s * (c - z) and
//     sum_i (c_i - z) x_i = sum_i c_i x_i - z sum_i x_i.
// The codes become bf16 pairs by OR-ing them into the mantissa of 128.0
// (bf16 0x4300): a 2-bit code c at mantissa bit 2q reads as 128 + c * 4^q, so
// no shift is needed for q = 0, 1, 2 and the dword needs only two shifts for
// its 16 codes.  v_dot2_f32_bf16 multiplies a code pair by an activation pair
// (products exact in fp32) and accumulates in fp32 into one accumulator per q,
// started at -128 * sum(x over that q's positions); then
//     sum c x = acc0 + acc1 / 4 + acc2 / 16.
// 4-bit codes use q = 0 only (one shift per code pair).  fp32 activations
// (and the SwiGLU output feeding the down projection) are split into two bf16
// terms hi + lo (relative error <= 2^-17) that share the accumulators.
#pragma once

#include "moe_device.h"
#include "moe_internal.h"

namespace moe {

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));

__device__ __forceinline__ float dot2(uint32_t a, uint32_t b, float c) {
    return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, a), __builtin_bit_cast(bf16x2_t, b), c,
                                           false);
}

__device__ __forceinline__ uint32_t bf16_rne(float f) {
    uint32_t u = __float_as_uint(f);
    return (u + 0x7FFFu + ((u >> 16) & 1u)) >> 16;
}

__device__ __forceinline__ float bf16_to_f32(uint32_t h) { return __uint_as_float(h << 16); }

constexpr uint32_t kMagic = 0x43004300u;   // bf16 pair (128.0, 128.0)

// Loads through global-address-space pointers: the expert blobs and the
// activations come as generic pointers, and generic (flat) loads would make
// every wait for one of them also wait for LDS traffic and for all other loads.
__device__ __forceinline__ uint4 ldg_u4(const void* p) {
    typedef uint32_t v4u __attribute__((ext_vector_type(4)));
    const v4u v = *(const __attribute__((address_space(1))) v4u*)p;
    return make_uint4(v[0], v[1], v[2], v[3]);
}
__device__ __forceinline__ uint16_t ldg_u16(const void* p) {
    return *(const __attribute__((address_space(1))) uint16_t*)p;
}
// Weight codes of a routed expert: non-temporal.  Each is read once a call,
// and a layer's next call selects other experts; the shared expert's codes,
// read by every call, keep the ordinary loads (they can stay in the memory-
// side cache from one call of the layer to the next).
__device__ __forceinline__ uint4 ldg_u4_nt(const void* p) {
    typedef uint32_t v4u __attribute__((ext_vector_type(4)));
    const v4u v = __builtin_nontemporal_load((const __attribute__((address_space(1))) v4u*)p);
    return make_uint4(v[0], v[1], v[2], v[3]);
}



__device__ __forceinline__ uint32_t magic_vgpr() {
    uint32_t m;
    asm volatile("v_mov_b32 %0, %1" : "=v"(m) : "i"(kMagic));
    return m;
}

// Bytes 0-1 of a and of b -> (a.lo16, b.lo16); bytes 2-3 -> (a.hi16, b.hi16).
__device__ __forceinline__ uint32_t pair_lo(uint32_t a, uint32_t b) { return __builtin_amdgcn_perm(b, a, 0x05040100u); }
__device__ __forceinline__ uint32_t pair_hi(uint32_t a, uint32_t b) { return __builtin_amdgcn_perm(b, a, 0x07060302u); }
constexpr uint32_t kOnes = 0x3F803F80u;    // bf16 pair (1.0, 1.0)
constexpr int kCpolSc1 = 16;               // cache policy bits of a buffer load: sc1 (agent coherence)
constexpr int kRsrcWord3 = 0x00020000;     // buffer resource word 3: 32-bit data format, raw access
constexpr int kMaxPass = 8;    // gate/up passes per tile (tile rows = P * passes)
constexpr int kMaxPassPair = 5;   // the same with two block columns a lane (twice the codes a pass)

template <int QT>
struct QTraits;
template <>
struct QTraits<1> {                 // 64 two-bit codes per block
    static constexpr int QK = 64;
    static constexpr int NPAIR = 32;  // dot pairs per block
    static constexpr int NQ = 3;      // mantissa positions q used
};
template <>
struct QTraits<2> {                 // 32 four-bit codes per block
    static constexpr int QK = 32;
    static constexpr int NPAIR = 16;
    static constexpr int NQ = 1;
};

// Activation slice of one token for one block column: NPAIR dot pairs per term,
// and the per-q offsets (-128 * sum of x over those positions) and z * sum(x).
template <int QT, int NTERM>
struct XSlice {
    uint32_t pr[NTERM][QTraits<QT>::NPAIR];
    float neg_c[QTraits<QT>::NQ];
    float zx;
};

// Position class q of dot pair i within a dword (2-bit codes): pairs 0,3,6 at
// q=0; 1,4,7 at q=1; 2,5 at q=2.
__device__ __forceinline__ constexpr int q_of_pair(int i) { return i % 3; }

// Arrange qk natural-order bf16 values (words nat[j] = (v[2j], v[2j+1])) into
// dot pairs matching the code pairs of each dword.
template <int QT>
__device__ __forceinline__ void arrange_pairs(const uint32_t* nat, uint32_t* pr) {
    if constexpr (QT == 1) {
        // dword d: pair i = (v[16d + i], v[16d + i + 8])
#pragma unroll
        for (int d = 0; d < 4; ++d)
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                uint32_t a = nat[8 * d + i / 2], b = nat[8 * d + 4 + i / 2];
                pr[8 * d + i] = (i & 1) ? pair_hi(a, b) : pair_lo(a, b);
            }
    } else {
        // dword d: pair i = (v[8d + i], v[8d + i + 4])
#pragma unroll
        for (int d = 0; d < 4; ++d)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                uint32_t a = nat[4 * d + i / 2], b = nat[4 * d + 2 + i / 2];
                pr[4 * d + i] = (i & 1) ? pair_hi(a, b) : pair_lo(a, b);
            }
    }
}

template <int QT, int NTERM>
__device__ __forceinline__ void finish_slice(XSlice<QT, NTERM>& s, float z) {
    constexpr int NP = QTraits<QT>::NPAIR;
    float xq[3] = {0.f, 0.f, 0.f};
#pragma unroll
    for (int tm = 0; tm < NTERM; ++tm)
#pragma unroll
        for (int i = 0; i < NP; ++i) {
            const int q = (QT == 1) ? q_of_pair(i % 8) : 0;
            xq[q] = dot2(kOnes, s.pr[tm][i], xq[q]);
        }
    float xs = 0.f;
#pragma unroll
    for (int q = 0; q < QTraits<QT>::NQ; ++q) {
        s.neg_c[q] = -128.f * xq[q];
        xs += xq[q];
    }
    s.zx = z * xs;
}

// Load one token's slice from bf16 activations (NTERM 1) or from two bf16
// planes hi/lo (NTERM 2).  `src` points at the first value of the block column.
template <int QT, int NTERM>
__device__ __forceinline__ void load_slice_bf16(XSlice<QT, NTERM>& s, const uint16_t* hi, const uint16_t* lo,
                                                float z) {
    constexpr int NW = QTraits<QT>::QK / 2;   // natural words
    uint32_t nat[NW];
#pragma unroll
    for (int tm = 0; tm < NTERM; ++tm) {
        const uint4* p = reinterpret_cast<const uint4*>(tm == 0 ? hi : lo);
#pragma unroll
        for (int v = 0; v < NW / 4; ++v) {
            uint4 u = ldg_u4(p + v);
            nat[4 * v + 0] = u.x;
            nat[4 * v + 1] = u.y;
            nat[4 * v + 2] = u.z;
            nat[4 * v + 3] = u.w;
        }
        arrange_pairs<QT>(nat, s.pr[tm]);
    }
    finish_slice<QT, NTERM>(s, z);
}

// fp32 activations: split each value into hi = bf16(v), lo = bf16(v - hi).
template <int QT>
__device__ __forceinline__ void load_slice_f32(XSlice<QT, 2>& s, const float* src, float z) {
    constexpr int QK = QTraits<QT>::QK;
    uint32_t nhi[QK / 2], nlo[QK / 2];
#pragma unroll
    for (int v = 0; v < QK / 4; ++v) {
        const uint4 fu = ldg_u4(reinterpret_cast<const float4*>(src) + v);
        float4 f = make_float4(__uint_as_float(fu.x), __uint_as_float(fu.y), __uint_as_float(fu.z), __uint_as_float(fu.w));
        float vals[4] = {f.x, f.y, f.z, f.w};
        uint32_t h[4], l[4];
#pragma unroll
        for (int c = 0; c < 4; ++c) {
            h[c] = bf16_rne(vals[c]);
            l[c] = bf16_rne(vals[c] - bf16_to_f32(h[c]));
        }
        nhi[2 * v] = h[0] | (h[1] << 16);
        nhi[2 * v + 1] = h[2] | (h[3] << 16);
        nlo[2 * v] = l[0] | (l[1] << 16);
        nlo[2 * v + 1] = l[2] | (l[3] << 16);
    }
    arrange_pairs<QT>(nhi, s.pr[0]);
    arrange_pairs<QT>(nlo, s.pr[1]);
    finish_slice<QT, 2>(s, z);
}

// A slice stored as packed words w[j] = bf16 hi(v_j) | bf16 lo(v_j) << 16 (the
// SwiGLU output as the gate/up stage publishes it).  `a` is read with
// agent-coherent (sc1) buffer loads: it is written by other workgroups,
// possibly on other XCDs, and these loads see it without invalidating this
// XCD's L2.  Returns whether every word has been written (is non-zero).
template <int QT>
__device__ __forceinline__ bool load_packed_words(uint32_t (&w)[QTraits<QT>::QK], __amdgpu_buffer_rsrc_t rsrc,
                                                  uint32_t byte_off) {
    constexpr int QK = QTraits<QT>::QK;
    typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
#pragma unroll
    for (int v = 0; v < QK / 4; ++v) {
        const u32x4 u = __builtin_amdgcn_raw_buffer_load_b128(rsrc, (int)(byte_off + 16 * v), 0, kCpolSc1);
        w[4 * v + 0] = u[0];
        w[4 * v + 1] = u[1];
        w[4 * v + 2] = u[2];
        w[4 * v + 3] = u[3];
    }
    uint32_t m = w[0];
#pragma unroll
    for (int i = 1; i < QK; ++i) m = w[i] < m ? w[i] : m;
    return m != 0u;
}

// De-interleave packed words into the two terms' dot pairs.
template <int QT>
__device__ __forceinline__ void slice_from_packed(XSlice<QT, 2>& s, const uint32_t (&w)[QTraits<QT>::QK], float z) {
    constexpr int HALF = QT == 1 ? 8 : 4;   // pair (v, v + HALF) within a dword's codes
    constexpr int PER = QT == 1 ? 16 : 8;   // values per code dword
#pragma unroll
    for (int d = 0; d < 4; ++d)
#pragma unroll
        for (int i = 0; i < HALF; ++i) {
            const uint32_t a = w[PER * d + i], b = w[PER * d + i + HALF];
            s.pr[0][HALF * d + i] = pair_lo(a, b);
            s.pr[1][HALF * d + i] = pair_hi(a, b);
        }
    finish_slice<QT, 2>(s, z);
}

// An arranged activation slice in LDS: the dot pairs, then the per-q offsets
// and z * sum x, padded to a multiple of 4 words.
template <int QT, int NTERM>
struct SliceWords {
    static constexpr int N = (NTERM * QTraits<QT>::NPAIR + QTraits<QT>::NQ + 1 + 3) & ~3;
};

template <int QT, int NTERM>
__device__ __forceinline__ void slice_to_lds(const XSlice<QT, NTERM>& s, uint32_t* d) {
    constexpr int NP = QTraits<QT>::NPAIR, NQ = QTraits<QT>::NQ;
#pragma unroll
    for (int tm = 0; tm < NTERM; ++tm)
#pragma unroll
        for (int i = 0; i < NP; ++i) d[tm * NP + i] = s.pr[tm][i];
#pragma unroll
    for (int q = 0; q < NQ; ++q) d[NTERM * NP + q] = __float_as_uint(s.neg_c[q]);
    d[NTERM * NP + NQ] = __float_as_uint(s.zx);
}

template <int QT, int NTERM>
__device__ __forceinline__ void slice_from_lds(XSlice<QT, NTERM>& s, const uint32_t* d) {
    constexpr int NP = QTraits<QT>::NPAIR, NQ = QTraits<QT>::NQ, SW = SliceWords<QT, NTERM>::N;
    uint32_t w[SW];
#pragma unroll
    for (int v = 0; v < SW / 4; ++v) {
        const uint4 u = reinterpret_cast<const uint4*>(d)[v];
        w[4 * v + 0] = u.x;
        w[4 * v + 1] = u.y;
        w[4 * v + 2] = u.z;
        w[4 * v + 3] = u.w;
    }
#pragma unroll
    for (int tm = 0; tm < NTERM; ++tm)
#pragma unroll
        for (int i = 0; i < NP; ++i) s.pr[tm][i] = w[tm * NP + i];
#pragma unroll
    for (int q = 0; q < NQ; ++q) s.neg_c[q] = __uint_as_float(w[NTERM * NP + q]);
    s.zx = __uint_as_float(w[NTERM * NP + NQ]);
}

// A SwiGLU output as the gate/up stage publishes it: two bf16 terms hi + lo
// (relative error <= 2^-17) in one word, hi | lo << 16.  The word is never 0:
// a value that rounds to +0 is stored as -0 (0x8000), a NaN as the canonical
// quiet NaN, so 0 marks a word not yet written.
__device__ __forceinline__ uint32_t pack_a(float a) {
    if (a != a) a = __uint_as_float(0x7FC00000u);
    const uint32_t hi = bf16_rne(a);
    const uint32_t lo = bf16_rne(a - bf16_to_f32(hi));
    const uint32_t w = hi | (lo << 16);
    return w == 0u ? 0x8000u : w;
}

// sum_i s * (c_i - z) x_i of one block for NT tokens (ntok valid; one token
// needs no check, which keeps the code free of branches).
template <int QT, int NTERM, int NT>
__device__ __forceinline__ void block_dot(const uint4 codes, float scale, const XSlice<QT, NTERM> (&xs)[NT],
                                          int ntok, float (&out)[NT]) {
    constexpr int NQ = QTraits<QT>::NQ;
    float acc[NT][NQ];
#pragma unroll
    for (int t = 0; t < NT; ++t)
#pragma unroll
        for (int q = 0; q < NQ; ++q) acc[t][q] = xs[t].neg_c[q];
    const uint32_t dw[4] = {codes.x, codes.y, codes.z, codes.w};
    const uint32_t mg = magic_vgpr();
#pragma unroll
    for (int d = 0; d < 4; ++d) {
        const uint32_t D = dw[d];
        if constexpr (QT == 1) {
            uint32_t p[8];
            const uint32_t D6 = D >> 6, D12 = D >> 12;
            p[0] = and_or(D, 0x00030003u, mg);
            p[1] = and_or(D, 0x000C000Cu, mg);
            p[2] = and_or(D, 0x00300030u, mg);
            p[3] = and_or(D6, 0x00030003u, mg);
            p[4] = and_or(D6, 0x000C000Cu, mg);
            p[5] = and_or(D6, 0x00300030u, mg);
            p[6] = and_or(D12, 0x00030003u, mg);
            p[7] = and_or(D12, 0x000C000Cu, mg);
#pragma unroll
            for (int t = 0; t < NT; ++t) {
                if (NT == 1 || t < ntok) {
#pragma unroll
                    for (int tm = 0; tm < NTERM; ++tm)
#pragma unroll
                        for (int i = 0; i < 8; ++i)
                            acc[t][q_of_pair(i)] = dot2(p[i], xs[t].pr[tm][8 * d + i], acc[t][q_of_pair(i)]);
                }
            }
        } else {
            uint32_t p[4];
            p[0] = and_or(D, 0x000F000Fu, mg);
            p[1] = and_or(D >> 4, 0x000F000Fu, mg);
            p[2] = and_or(D >> 8, 0x000F000Fu, mg);
            p[3] = and_or(D >> 12, 0x000F000Fu, mg);
#pragma unroll
            for (int t = 0; t < NT; ++t) {
                if (NT == 1 || t < ntok) {
#pragma unroll
                    for (int tm = 0; tm < NTERM; ++tm)
#pragma unroll
                        for (int i = 0; i < 4; ++i) acc[t][0] = dot2(p[i], xs[t].pr[tm][4 * d + i], acc[t][0]);
                }
            }
        }
    }
#pragma unroll
    for (int t = 0; t < NT; ++t) {
        float cx;
        if constexpr (QT == 1) cx = __builtin_fmaf(acc[t][2], 0.0625f, __builtin_fmaf(acc[t][1], 0.25f, acc[t][0]));
        else cx = acc[t][0];
        out[t] = scale * (cx - xs[t].zx);
    }
}

// Two blocks against the same activation slices (gate and up of one row, or
// two rows of one block column): the arithmetic of two block_dot calls, each
// accumulation in the same order, with the two blocks' dot products
// interleaved so that twice as many accumulation chains are in flight.
template <int QT, int NTERM, int NT>
__device__ __forceinline__ void block_dot_pair(const uint4 ca, float sa, const uint4 cb, float sb,
                                               const XSlice<QT, NTERM> (&xs)[NT], int ntok, float (&oa)[NT],
                                               float (&ob)[NT]) {
    constexpr int NQ = QTraits<QT>::NQ;
    float acc[2][NT][NQ];
#pragma unroll
    for (int t = 0; t < NT; ++t)
#pragma unroll
        for (int q = 0; q < NQ; ++q) acc[0][t][q] = acc[1][t][q] = xs[t].neg_c[q];
    const uint32_t dw[2][4] = {{ca.x, ca.y, ca.z, ca.w}, {cb.x, cb.y, cb.z, cb.w}};
    const uint32_t mg = magic_vgpr();
#pragma unroll
    for (int d = 0; d < 4; ++d) {
        if constexpr (QT == 1) {
            uint32_t p[2][8];
#pragma unroll
            for (int h = 0; h < 2; ++h) {
                const uint32_t D = dw[h][d], D6 = D >> 6, D12 = D >> 12;
                p[h][0] = and_or(D, 0x00030003u, mg);
                p[h][1] = and_or(D, 0x000C000Cu, mg);
                p[h][2] = and_or(D, 0x00300030u, mg);
                p[h][3] = and_or(D6, 0x00030003u, mg);
                p[h][4] = and_or(D6, 0x000C000Cu, mg);
                p[h][5] = and_or(D6, 0x00300030u, mg);
                p[h][6] = and_or(D12, 0x00030003u, mg);
                p[h][7] = and_or(D12, 0x000C000Cu, mg);
            }
#pragma unroll
            for (int t = 0; t < NT; ++t) {
                if (NT == 1 || t < ntok) {
#pragma unroll
                    for (int tm = 0; tm < NTERM; ++tm)
#pragma unroll
                        for (int i = 0; i < 8; ++i)
#pragma unroll
                            for (int h = 0; h < 2; ++h)
                                acc[h][t][q_of_pair(i)] = dot2(p[h][i], xs[t].pr[tm][8 * d + i], acc[h][t][q_of_pair(i)]);
                }
            }
        } else {
            uint32_t p[2][4];
#pragma unroll
            for (int h = 0; h < 2; ++h) {
                const uint32_t D = dw[h][d];
                p[h][0] = and_or(D, 0x000F000Fu, mg);
                p[h][1] = and_or(D >> 4, 0x000F000Fu, mg);
                p[h][2] = and_or(D >> 8, 0x000F000Fu, mg);
                p[h][3] = and_or(D >> 12, 0x000F000Fu, mg);
            }
#pragma unroll
            for (int t = 0; t < NT; ++t) {
                if (NT == 1 || t < ntok) {
#pragma unroll
                    for (int tm = 0; tm < NTERM; ++tm)
#pragma unroll
                        for (int i = 0; i < 4; ++i)
#pragma unroll
                            for (int h = 0; h < 2; ++h)
                                acc[h][t][0] = dot2(p[h][i], xs[t].pr[tm][4 * d + i], acc[h][t][0]);
                }
            }
        }
    }
#pragma unroll
    for (int t = 0; t < NT; ++t) {
        float cx[2];
#pragma unroll
        for (int h = 0; h < 2; ++h) {
            if constexpr (QT == 1)
                cx[h] = __builtin_fmaf(acc[h][t][2], 0.0625f, __builtin_fmaf(acc[h][t][1], 0.25f, acc[h][t][0]));
            else
                cx[h] = acc[h][t][0];
        }
        oa[t] = sa * (cx[0] - xs[t].zx);
        ob[t] = sb * (cx[1] - xs[t].zx);
    }
}

__device__ __forceinline__ float half_bits_to_f32(uint16_t h) {
    return (float)__builtin_bit_cast(_Float16, h);   // exact, subnormals included
}


// A block scale converted where it is used: the empty asm keeps the
// conversion (and so the wait for its load) from being moved up to the load,
// where it would hold back the loads issued after it.
__device__ __forceinline__ float scale_at_use(uint16_t bits) {
    uint32_t b = bits;
    asm volatile("" : "+v"(b));
    return half_bits_to_f32((uint16_t)b);
}

// LDS DMA of 16 bytes per lane with an agent-coherent (sc1) read: lane i's
// chunk lands at dst_wave + 16 i.
__device__ __forceinline__ void load_lds16_sc1(const void* src, uint8_t* dst_wave) {
    __builtin_amdgcn_global_load_lds(src, (__attribute__((address_space(3))) void*)dst_wave, 16, 0, kCpolSc1);
}

// Expert e's blob from a device table of blob addresses (a global load of
// one pointer).
__device__ __forceinline__ const uint8_t* table_blob(const void* const* table, int e) {
    return (const uint8_t*)((const __attribute__((address_space(1))) uint64_t*)table)[e];
}

// A value whose bits are never 0: +0 becomes -0 (equal in every use), so 0
// marks a word not yet written.
__device__ __forceinline__ uint32_t nonzero_bits(float v) {
    const uint32_t u = __float_as_uint(v);
    return u == 0u ? 0x80000000u : u;
}

// Makes v opaque to the compiler at this point (no code is emitted).
__device__ __forceinline__ void pin_u4(uint4& v) { asm volatile("" : "+v"(v.x), "+v"(v.y), "+v"(v.z), "+v"(v.w)); }

// v + v of the neighbouring lane (lanes 2i and 2i + 1 exchange).
__device__ __forceinline__ float dpp_xor1_f32(float v) {
    return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), kDppXor1, 0xF, 0xF, false));
}

// q[0] + q[1] + ... + q[n - 1], added in that order; q is 16-byte aligned LDS.
__device__ __forceinline__ float sum_columns(const float* q, int n) {
    const float4* q4 = reinterpret_cast<const float4*>(q);
    float acc = 0.f;
    int b = 0;
#pragma unroll 2
    for (; b + 4 <= n; b += 4) {
        const float4 v = q4[b / 4];
        acc += v.x;
        acc += v.y;
        acc += v.z;
        acc += v.w;
    }
    if (b < n) {
        const float4 v = q4[b / 4];
        acc += v.x;
        if (b + 1 < n) acc += v.y;
        if (b + 2 < n) acc += v.z;
    }
    return acc;
}

// The same sum in four interleaved chains (column j in chain j % 4), combined
// as (c0 + c1) + (c2 + c3).
__device__ __forceinline__ float sum_columns4(const float* q, int n) {
    const float4* q4 = reinterpret_cast<const float4*>(q);
    float c0 = 0.f, c1 = 0.f, c2 = 0.f, c3 = 0.f;
    int b = 0;
#pragma unroll 4
    for (; b + 4 <= n; b += 4) {
        const float4 v = q4[b / 4];
        c0 += v.x;
        c1 += v.y;
        c2 += v.z;
        c3 += v.w;
    }
    if (b < n) {
        const float4 v = q4[b / 4];
        c0 += v.x;
        if (b + 1 < n) c1 += v.y;
        if (b + 2 < n) c2 += v.z;
    }
    return (c0 + c1) + (c2 + c3);
}

}  // namespace moe
