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
constexpr uint32_t kOnes = 0x3F803F80u;    // bf16 pair (1.0, 1.0)

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
                pr[8 * d + i] = (i & 1) ? ((a >> 16) | (b & 0xFFFF0000u)) : ((a & 0xFFFFu) | (b << 16));
            }
    } else {
        // dword d: pair i = (v[8d + i], v[8d + i + 4])
#pragma unroll
        for (int d = 0; d < 4; ++d)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                uint32_t a = nat[4 * d + i / 2], b = nat[4 * d + 2 + i / 2];
                pr[4 * d + i] = (i & 1) ? ((a >> 16) | (b & 0xFFFF0000u)) : ((a & 0xFFFFu) | (b << 16));
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
            uint4 u = p[v];
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
        float4 f = reinterpret_cast<const float4*>(src)[v];
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

// sum_i s * (c_i - z) x_i of one block for NT tokens (ntok valid).
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
#pragma unroll
    for (int d = 0; d < 4; ++d) {
        const uint32_t D = dw[d];
        if constexpr (QT == 1) {
            uint32_t p[8];
            const uint32_t D6 = D >> 6, D12 = D >> 12;
            p[0] = (D & 0x00030003u) | kMagic;
            p[1] = (D & 0x000C000Cu) | kMagic;
            p[2] = (D & 0x00300030u) | kMagic;
            p[3] = (D6 & 0x00030003u) | kMagic;
            p[4] = (D6 & 0x000C000Cu) | kMagic;
            p[5] = (D6 & 0x00300030u) | kMagic;
            p[6] = (D12 & 0x00030003u) | kMagic;
            p[7] = (D12 & 0x000C000Cu) | kMagic;
#pragma unroll
            for (int t = 0; t < NT; ++t) {
                if (t < ntok) {
#pragma unroll
                    for (int tm = 0; tm < NTERM; ++tm)
#pragma unroll
                        for (int i = 0; i < 8; ++i)
                            acc[t][q_of_pair(i)] = dot2(p[i], xs[t].pr[tm][8 * d + i], acc[t][q_of_pair(i)]);
                }
            }
        } else {
            uint32_t p[4];
            p[0] = (D & 0x000F000Fu) | kMagic;
            p[1] = ((D >> 4) & 0x000F000Fu) | kMagic;
            p[2] = ((D >> 8) & 0x000F000Fu) | kMagic;
            p[3] = ((D >> 12) & 0x000F000Fu) | kMagic;
#pragma unroll
            for (int t = 0; t < NT; ++t) {
                if (t < ntok) {
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

__device__ __forceinline__ float half_bits_to_f32(uint16_t h) {
    return (float)__builtin_bit_cast(_Float16, h);   // exact, subnormals included
}

// ---------------------------------------------------------------------------------------------
// Gate/up + SwiGLU.
// ---------------------------------------------------------------------------------------------
struct GateUpParams {
    const void* const* table;
    const uint8_t* single;     // used instead of table[e] when table == nullptr
    const uint8_t* shared;
    const void* x;             // [T][H]
    int H, FF, FFs, T;
    float z;
    const SmallMeta* meta;
    const int* pair_tok;
    const int* pair_exp;
    const int* group_first;
    const int* group_n;
    uint16_t *a_hi, *a_lo;     // [pairs][FF]
    uint16_t *as_hi, *as_lo;   // [T][FFs]
    int passes;                // M: passes per tile (tile rows = P * M)
    int tiles, tiles_s, max_groups;
};

constexpr int kMaxPass = 8;

template <int QT, int NT, int NTERM>
__global__ void __launch_bounds__(kGemvThreads) gateup_kernel(GateUpParams p) {
    constexpr int QK = QTraits<QT>::QK;
    extern __shared__ float lds[];
    const int tid = threadIdx.x;
    int idx = blockIdx.x;

    const uint8_t* blob;
    int rows, tile, ntok, toks[NT], outrow[NT];
    uint16_t *ohi, *olo;
    if (idx < p.max_groups * p.tiles) {
        const int g = idx / p.tiles;
        tile = idx - g * p.tiles;
        if (g >= p.meta->n_groups) return;
        const int first = p.group_first[g];
        ntok = p.group_n[g];
        const int e = p.pair_exp[first];
        blob = p.table ? (const uint8_t*)p.table[e] : p.single;
        rows = p.FF;
#pragma unroll
        for (int t = 0; t < NT; ++t) {
            toks[t] = t < ntok ? p.pair_tok[first + t] : 0;
            outrow[t] = first + t;
        }
        ohi = p.a_hi;
        olo = p.a_lo;
    } else {
        idx -= p.max_groups * p.tiles;
        const int sg = idx / p.tiles_s;
        tile = idx - sg * p.tiles_s;
        blob = p.shared;
        rows = p.FFs;
        ntok = min(NT, p.T - sg * NT);
#pragma unroll
        for (int t = 0; t < NT; ++t) {
            toks[t] = t < ntok ? sg * NT + t : 0;
            outrow[t] = sg * NT + t;
        }
        ohi = p.as_hi;
        olo = p.as_lo;
    }

    const int nblk = p.H / QK;
    const int P = kGemvThreads / nblk;
    const bool active = tid < P * nblk;
    const int rp = tid / nblk, b = tid - (tid / nblk) * nblk;
    const int R = P * p.passes;
    const int f0 = tile * R;
    const size_t plane = (size_t)rows * nblk;        // blocks per matrix
    const uint8_t* gcode = blob;
    const uint8_t* gscale = blob + plane * 16;
    const uint8_t* ucode = blob + plane * 18;
    const uint8_t* uscale = ucode + plane * 16;

    // Issue every code and scale load of the tile first.
    uint4 cg[kMaxPass], cu[kMaxPass];
    uint16_t sg_[kMaxPass], su_[kMaxPass];
#pragma unroll
    for (int m = 0; m < kMaxPass; ++m) {
        const int f = f0 + m * P + rp;
        if (m < p.passes && active && f < rows) {
            const size_t blk = (size_t)f * nblk + b;
            cg[m] = *reinterpret_cast<const uint4*>(gcode + blk * 16);
            cu[m] = *reinterpret_cast<const uint4*>(ucode + blk * 16);
            sg_[m] = *reinterpret_cast<const uint16_t*>(gscale + blk * 2);
            su_[m] = *reinterpret_cast<const uint16_t*>(uscale + blk * 2);
        }
    }

    XSlice<QT, NTERM> xs[NT];
    if (active) {
#pragma unroll
        for (int t = 0; t < NT; ++t) {
            if (t < ntok) {
                if constexpr (NTERM == 1) {
                    const uint16_t* src = (const uint16_t*)p.x + (size_t)toks[t] * p.H + b * QK;
                    load_slice_bf16<QT, 1>(xs[t], src, nullptr, p.z);
                } else {
                    const float* src = (const float*)p.x + (size_t)toks[t] * p.H + b * QK;
                    load_slice_f32<QT>(xs[t], src, p.z);
                }
            }
        }
    }

    // part[mat][row][b][t]
    float* part = lds;
#pragma unroll
    for (int m = 0; m < kMaxPass; ++m) {
        const int f = f0 + m * P + rp;
        if (m < p.passes && active && f < rows) {
            float og[NT], ou[NT];
            block_dot<QT, NTERM, NT>(cg[m], half_bits_to_f32(sg_[m]), xs, ntok, og);
            block_dot<QT, NTERM, NT>(cu[m], half_bits_to_f32(su_[m]), xs, ntok, ou);
            const int rr = m * P + rp;
#pragma unroll
            for (int t = 0; t < NT; ++t) {
                part[((0 * R + rr) * nblk + b) * NT + t] = og[t];
                part[((1 * R + rr) * nblk + b) * NT + t] = ou[t];
            }
        }
    }
    __syncthreads();

    for (int i = tid; i < R * NT; i += kGemvThreads) {
        const int rr = i / NT, t = i - (i / NT) * NT;
        const int f = f0 + rr;
        if (f >= rows || t >= ntok) continue;
        float g = 0.f, u = 0.f;
        for (int bb = 0; bb < nblk; ++bb) {
            g += part[((0 * R + rr) * nblk + bb) * NT + t];
            u += part[((1 * R + rr) * nblk + bb) * NT + t];
        }
        const float a = g / (1.f + expf(-g)) * u;
        const uint32_t hi = bf16_rne(a);
        const uint32_t lo = bf16_rne(a - bf16_to_f32(hi));
        const size_t o = (size_t)outrow[t] * rows + f;
        ohi[o] = (uint16_t)hi;
        olo[o] = (uint16_t)lo;
    }
}

// ---------------------------------------------------------------------------------------------
// Down projection + deterministic combine.
// ---------------------------------------------------------------------------------------------
struct DownParams {
    const void* const* table;
    const uint8_t* single;
    const uint8_t* shared;
    int H, FF, FFs, T, k;
    float z;
    const SmallMeta* meta;
    const int* pair_tok;
    const int* pair_exp;
    const int* group_first;
    const int* group_n;
    const int* slot_pair;
    const float* w;              // [T][k]
    const uint16_t *a_hi, *a_lo;
    const uint16_t *as_hi, *as_lo;
    float* d;                    // [pairs][H]
    float* ds;                   // [T][H]
    float* y;                    // [T][H]
    int* tile_cnt;
    int tile_rows;               // R: H rows per tile
    int tiles, max_groups, shared_groups;
};

template <int QT, int NT>
__global__ void __launch_bounds__(kGemvThreads) down_kernel(DownParams p) {
    constexpr int QK = QTraits<QT>::QK;
    extern __shared__ float lds[];
    __shared__ int s_last;
    const int tid = threadIdx.x;
    int idx = blockIdx.x;

    const uint8_t* blob;
    int K, tile, ntok, arow[NT];
    const uint16_t *ahi, *alo;
    float* out;
    if (idx < p.max_groups * p.tiles) {
        const int g = idx / p.tiles;
        tile = idx - g * p.tiles;
        if (g >= p.meta->n_groups) return;
        const int first = p.group_first[g];
        ntok = p.group_n[g];
        const int e = p.pair_exp[first];
        blob = p.table ? (const uint8_t*)p.table[e] : p.single;
        K = p.FF;
#pragma unroll
        for (int t = 0; t < NT; ++t) arow[t] = first + t;
        ahi = p.a_hi;
        alo = p.a_lo;
        out = p.d;
    } else {
        idx -= p.max_groups * p.tiles;
        const int sg = idx / p.tiles;
        tile = idx - sg * p.tiles;
        blob = p.shared;
        K = p.FFs;
        ntok = min(NT, p.T - sg * NT);
#pragma unroll
        for (int t = 0; t < NT; ++t) arow[t] = sg * NT + t;
        ahi = p.as_hi;
        alo = p.as_lo;
        out = p.ds;
    }

    const int nblk = K / QK;
    const int P = kGemvThreads / nblk;
    const bool active = tid < P * nblk;
    const int rp = tid / nblk, b = tid - (tid / nblk) * nblk;
    const int R = p.tile_rows;
    const int h0 = tile * R;
    const int hend = min(p.H, h0 + R);
    // The gate and up planes come first: 2 * FF * (H / qk) blocks of 18 bytes.
    const size_t gu_bytes = (size_t)2 * K * (p.H / QK) * 18;
    const uint8_t* dcode = blob + gu_bytes;
    const uint8_t* dscale = dcode + (size_t)p.H * nblk * 16;

    XSlice<QT, 2> xs[NT];
    if (active) {
#pragma unroll
        for (int t = 0; t < NT; ++t)
            if (t < ntok)
                load_slice_bf16<QT, 2>(xs[t], ahi + (size_t)arow[t] * K + b * QK, alo + (size_t)arow[t] * K + b * QK,
                                       p.z);
    }

    float* part = lds;
    for (int base = h0; base < hend; base += P * kMaxPass) {
        uint4 c[kMaxPass];
        uint16_t sc[kMaxPass];
#pragma unroll
        for (int m = 0; m < kMaxPass; ++m) {
            const int h = base + m * P + rp;
            if (active && h < hend) {
                const size_t blk = (size_t)h * nblk + b;
                c[m] = *reinterpret_cast<const uint4*>(dcode + blk * 16);
                sc[m] = *reinterpret_cast<const uint16_t*>(dscale + blk * 2);
            }
        }
#pragma unroll
        for (int m = 0; m < kMaxPass; ++m) {
            const int h = base + m * P + rp;
            if (active && h < hend) {
                float o[NT];
                block_dot<QT, 2, NT>(c[m], half_bits_to_f32(sc[m]), xs, ntok, o);
#pragma unroll
                for (int t = 0; t < NT; ++t) part[((m * P + rp) * nblk + b) * NT + t] = o[t];
            }
        }
        __syncthreads();
        const int rows_here = min(P * kMaxPass, hend - base);
        for (int i = tid; i < rows_here * NT; i += kGemvThreads) {
            const int rr = i / NT, t = i - (i / NT) * NT;
            if (t >= ntok) continue;
            float acc = 0.f;
            for (int bb = 0; bb < nblk; ++bb) acc += part[(rr * nblk + bb) * NT + t];
            out[(size_t)arow[t] * p.H + base + rr] = acc;
        }
        __syncthreads();
    }

    // The last workgroup to finish this tile of H rows combines it.
    __threadfence();
    __syncthreads();
    if (tid == 0) {
        const int expected = p.meta->n_groups + p.shared_groups;
        const int old = atomicAdd(&p.tile_cnt[tile], 1);
        s_last = (old == expected - 1);
    }
    __syncthreads();
    if (!s_last) return;
    __threadfence();
    const int rows_tile = hend - h0;
    for (int i = tid; i < p.T * rows_tile; i += kGemvThreads) {
        const int t = i / rows_tile, h = h0 + (i - (i / rows_tile) * rows_tile);
        float acc = p.shared ? p.ds[(size_t)t * p.H + h] : 0.f;
        for (int j = 0; j < p.k; ++j) {
            const int pr = p.slot_pair[t * p.k + j];
            acc = __builtin_fmaf(p.w[t * p.k + j], p.d[(size_t)pr * p.H + h], acc);
        }
        p.y[(size_t)t * p.H + h] = acc;
    }
}

// ---------------------------------------------------------------------------------------------
// Host side.
// ---------------------------------------------------------------------------------------------
GemvShape gemv_shape(int H, int FF, int FFs, int qtype, float z) {
    GemvShape g{};
    const int qk = codes_per_block(qtype);
    g.H = H;
    g.FF = FF;
    g.FFs = FFs;
    g.qtype = qtype;
    g.z = z;
    const int nblk_gu = H / qk;
    const int P = kGemvThreads / nblk_gu;
    const int passes = 2;
    g.tile_rows_gu = P * passes;
    g.tiles_gu = (FF + g.tile_rows_gu - 1) / g.tile_rows_gu;
    g.tiles_gu_s = FFs ? (FFs + g.tile_rows_gu - 1) / g.tile_rows_gu : 0;
    const int nblk_dn = FF / qk;
    const int Pd = kGemvThreads / nblk_dn;
    g.tile_rows_dn = Pd * 4;
    g.tiles_dn = (H + g.tile_rows_dn - 1) / g.tile_rows_dn;
    return g;
}

template <int QT, int NT>
static hipError_t launch_for(const GemvShape& g, const void* const* table, const void* single, const void* shared,
                             const void* x, int x_dtype, int T, int k, int max_groups, const float* w,
                             const SmallLayout& L, char* ws, float* y, hipStream_t s) {
    constexpr int QK = QTraits<QT>::QK;
    const int shared_groups = shared ? (T + NT - 1) / NT : 0;
    GateUpParams gp{};
    gp.table = table;
    gp.single = (const uint8_t*)single;
    gp.shared = (const uint8_t*)shared;
    gp.x = x;
    gp.H = g.H;
    gp.FF = g.FF;
    gp.FFs = g.FFs;
    gp.T = T;
    gp.z = g.z;
    gp.meta = (const SmallMeta*)(ws + L.meta);
    gp.pair_tok = (const int*)(ws + L.pair_tok);
    gp.pair_exp = (const int*)(ws + L.pair_exp);
    gp.group_first = (const int*)(ws + L.group_first);
    gp.group_n = (const int*)(ws + L.group_n);
    gp.a_hi = (uint16_t*)(ws + L.a_hi);
    gp.a_lo = (uint16_t*)(ws + L.a_lo);
    gp.as_hi = (uint16_t*)(ws + L.as_hi);
    gp.as_lo = (uint16_t*)(ws + L.as_lo);
    const int nblk = g.H / QK;
    const int P = kGemvThreads / nblk;
    gp.passes = g.tile_rows_gu / P;
    gp.tiles = g.tiles_gu;
    gp.tiles_s = g.tiles_gu_s;
    gp.max_groups = max_groups;
    const size_t lds_gu = (size_t)2 * g.tile_rows_gu * nblk * NT * sizeof(float);
    const int grid_gu = max_groups * g.tiles_gu + shared_groups * g.tiles_gu_s;
    if (x_dtype == 1)
        hipLaunchKernelGGL((gateup_kernel<QT, NT, 1>), dim3(grid_gu), dim3(kGemvThreads), lds_gu, s, gp);
    else
        hipLaunchKernelGGL((gateup_kernel<QT, NT, 2>), dim3(grid_gu), dim3(kGemvThreads), lds_gu, s, gp);
    hipError_t err = hipGetLastError();
    if (err != hipSuccess) return err;

    DownParams dp{};
    dp.table = table;
    dp.single = (const uint8_t*)single;
    dp.shared = (const uint8_t*)shared;
    dp.H = g.H;
    dp.FF = g.FF;
    dp.FFs = g.FFs;
    dp.T = T;
    dp.k = k;
    dp.z = g.z;
    dp.meta = gp.meta;
    dp.pair_tok = gp.pair_tok;
    dp.pair_exp = gp.pair_exp;
    dp.group_first = gp.group_first;
    dp.group_n = gp.group_n;
    dp.slot_pair = (const int*)(ws + L.slot_pair);
    dp.w = w;
    dp.a_hi = gp.a_hi;
    dp.a_lo = gp.a_lo;
    dp.as_hi = gp.as_hi;
    dp.as_lo = gp.as_lo;
    dp.d = (float*)(ws + L.d);
    dp.ds = (float*)(ws + L.ds);
    dp.y = y;
    dp.tile_cnt = (int*)(ws + L.tile_cnt);
    dp.tile_rows = g.tile_rows_dn;
    dp.tiles = g.tiles_dn;
    dp.max_groups = max_groups;
    dp.shared_groups = shared_groups;
    const int nb_r = g.FF / QK;
    const int nb_s = g.FFs ? g.FFs / QK : nb_r;
    const int nb_max = nb_r > nb_s ? nb_r : nb_s;
    size_t lds_dn = 0;
    for (int nb : {nb_r, nb_s}) {
        const size_t need = (size_t)(kGemvThreads / nb) * kMaxPass * nb * NT * sizeof(float);
        if (need > lds_dn) lds_dn = need;
    }
    (void)nb_max;
    const int grid_dn = (max_groups + shared_groups) * g.tiles_dn;
    hipLaunchKernelGGL((down_kernel<QT, NT>), dim3(grid_dn), dim3(kGemvThreads), lds_dn, s, dp);
    return hipGetLastError();
}

hipError_t launch_gemv_layer(const GemvShape& g, const void* const* table, const void* single_blob,
                             const void* shared, const void* x, int x_dtype, int T, int k, int max_groups,
                             const int* /*ids*/, const float* w, const SmallLayout& L, char* ws, float* y,
                             hipStream_t s) {
    const bool one = (T == 1);
    if (g.qtype == 1)
        return one ? launch_for<1, 1>(g, table, single_blob, shared, x, x_dtype, T, k, max_groups, w, L, ws, y, s)
                   : launch_for<1, kGroup>(g, table, single_blob, shared, x, x_dtype, T, k, max_groups, w, L, ws, y,
                                           s);
    return one ? launch_for<2, 1>(g, table, single_blob, shared, x, x_dtype, T, k, max_groups, w, L, ws, y, s)
               : launch_for<2, kGroup>(g, table, single_blob, shared, x, x_dtype, T, k, max_groups, w, L, ws, y, s);
}

// ---------------------------------------------------------------------------------------------
// Debug dequantisation of one matrix to fp32 (one thread per weight).
// ---------------------------------------------------------------------------------------------
__global__ void dequant_kernel(const uint8_t* __restrict__ mat, int qtype, float z, int rows, int cols,
                               float* __restrict__ out) {
    const size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (i >= (size_t)rows * cols) return;
    const int qk = qtype == 1 ? 64 : 32;
    const int r = (int)(i / cols), c = (int)(i % cols);
    const int nblk = cols / qk;
    const size_t blk = (size_t)r * nblk + c / qk;
    const int j = c % qk;
    const uint8_t byte = mat[blk * 16 + (qtype == 1 ? j / 4 : j / 2)];
    const int code = qtype == 1 ? (byte >> (2 * (j % 4))) & 3 : (byte >> (4 * (j % 2))) & 15;
    const uint16_t sb = *reinterpret_cast<const uint16_t*>(mat + (size_t)rows * nblk * 16 + blk * 2);
    out[i] = half_bits_to_f32(sb) * ((float)code - z);
}

hipError_t launch_dequant(const void* blob, int qtype, float z, int rows, int cols, size_t plane_offset, float* out,
                          hipStream_t s) {
    const size_t n = (size_t)rows * cols;
    if (n == 0) return hipSuccess;
    hipLaunchKernelGGL(dequant_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s,
                       (const uint8_t*)blob + plane_offset, qtype, z, rows, cols, out);
    return hipGetLastError();
}

}  // namespace moe
