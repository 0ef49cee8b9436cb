// Device helpers shared by the HIP kernels of libmoe_ffn: orderable routing
// keys, DPP wavefront reductions and the one-wave top-k.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "moe_internal.h"

namespace moe {

// Routing order (Krasis white paper 5.3: the k highest-scoring experts; ties
// toward the lower index).  A 32-bit key orders floats like `>` with
// -0 == +0: a non-negative value sets its sign bit, a negative one takes its
// two's complement (-0 and +0 both give 0x80000000, with no compare).  NaN
// maps to 1, below every number (-inf maps to 0x00800000), and 0 marks an
// empty or already-selected slot.
__device__ __forceinline__ uint32_t order_bits(float f) {
    const uint32_t u = __float_as_uint(f);
    const uint32_t neg = (uint32_t)((int32_t)u >> 31);
    const uint32_t key = (u ^ (neg | 0x80000000u)) + (u >> 31);
    return f != f ? 1u : key;
}

__device__ __forceinline__ float from_order_bits(uint32_t k) {
    if (k <= 1u) return __uint_as_float(0x7FC00000u);
    const uint32_t u = (k & 0x80000000u) ? (k & 0x7FFFFFFFu) : 0u - k;
    return __uint_as_float(u);
}

// DPP controls (gfx9 encoding): quad_perm [1,0,3,2] and [2,3,0,1], row_half_mirror,
// row_mirror, and the broadcasts of lane 15 of each row to the next row and of
// lane 31 to rows 2 and 3.
constexpr int kDppXor1 = 0xB1;
constexpr int kDppXor2 = 0x4E;
constexpr int kDppHalfMirror = 0x141;
constexpr int kDppMirror = 0x140;
constexpr int kDppBcast15 = 0x142;
constexpr int kDppBcast31 = 0x143;

template <int CTRL>
__device__ __forceinline__ uint32_t dpp_u32(uint32_t v) {
    return (uint32_t)__builtin_amdgcn_update_dpp((int)v, (int)v, CTRL, 0xF, 0xF, false);
}

// max(v, v from the DPP source lane).  Lanes of rows outside ROWM, and lanes
// without a source, see the identity 0, so the compiler can fold the DPP move
// into the v_max (one instruction per step).
template <int CTRL, int ROWM = 0xF>
__device__ __forceinline__ uint32_t dpp_max_u32(uint32_t v) {
    const uint32_t o = (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, CTRL, ROWM, 0xF, false);
    return o > v ? o : v;
}

template <int CTRL, int ROWM = 0xF>
__device__ __forceinline__ uint32_t dpp_min_u32(uint32_t v) {
    const uint32_t o = (uint32_t)__builtin_amdgcn_update_dpp(-1, (int)v, CTRL, ROWM, 0xF, false);
    return o < v ? o : v;
}

// (d & mask) | v in one v_and_or_b32.  gfx9 VOP3 encodings take no literal
// operands, so the mask goes in an SGPR and the OR value in a VGPR; written as
// plain C the compiler splits it into two instructions.
__device__ __forceinline__ uint32_t and_or(uint32_t d, uint32_t mask, uint32_t v) {
    uint32_t r;
    asm("v_and_or_b32 %0, %1, %2, %3" : "=v"(r) : "v"(d), "s"(mask), "v"(v));
    return r;
}

// Workgroup barrier for LDS traffic: waits for this wave's LDS operations
// only, so that an outstanding global atomic whose result is not needed does
// not hold the workgroup (a __syncthreads also waits for every global memory
// operation).  The memory clobber keeps the compiler from moving memory
// accesses across it.
__device__ __forceinline__ void lds_barrier() { asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory"); }

// Relaxed device-scope atomic add whose result is not needed, issued so that
// the compiler's wait tracking does not see it: later waits for unrelated
// loads then do not wait for this atomic's round trip.  The expcnt wait
// covers the hardware's reading of the operand registers before they are
// reused.
__device__ __forceinline__ void atomic_add_detached(int* p, int v) {
    asm volatile("global_atomic_add %0, %1, off\n\ts_waitcnt expcnt(0)" ::"v"(p), "v"(v) : "memory");
}

// Error bits of a workspace (see kErrWord), set with a relaxed device-scope OR.
__device__ __forceinline__ void flag_error(int* err, int bits) {
    __hip_atomic_fetch_or(err, bits, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ int load_error(const int* err) {
    return __hip_atomic_load(err, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// A bounded wait: polls ready() (sleeping between polls) until it holds or
// `polls` polls have failed; then flags kErrTimeout and returns false.  A
// bound of 0 gives up at once, whether or not ready() holds (the debug mode
// that exercises every failure path without a real stall).
template <int SLEEP = 1, class F>
__device__ __forceinline__ bool bounded_wait(F ready, long polls, int* err) {
    if (polls == 0) {
        flag_error(err, kErrTimeout);
        return false;
    }
    long n = 0;
    while (!ready()) {
        if (++n > polls) {
            flag_error(err, kErrTimeout);
            return false;
        }
        __builtin_amdgcn_s_sleep(SLEEP);
    }
    return true;
}

// The gate's activation of a gated expert FFN: SiLU (SwiGLU), or the tanh
// form of GELU (GeGLU; kairos-engine README, "Decode, 2026-09-28/29").  Both
// are v / (1 + e^(-b)): b = v for SiLU, and since (1 + tanh u) / 2 =
// 1 / (1 + e^(-2u)), b = 2 sqrt(2/pi) (v + 0.044715 v^3) for GELU.
constexpr int kActSilu = 0;
constexpr int kActGeluTanh = 1;
__device__ __forceinline__ float gate_arg(float v, int act) {
    return act == kActGeluTanh ? 1.5957691216057308f * (v + 0.044715f * (v * v * v)) : v;
}
__device__ __forceinline__ float act_gate(float v, int act) { return v / (1.f + expf(-gate_arg(v, act))); }

__device__ __forceinline__ uint32_t readlane_u32(uint32_t v, int lane) {
    return (uint32_t)__builtin_amdgcn_readlane((int)v, lane);
}

// Maximum / minimum over the 64 lanes of a wave (every lane active); uniform
// result.  Four DPP steps give each row of 16 lanes its extremum; two row
// broadcasts carry it up to lane 63, which is read once.
__device__ __forceinline__ uint32_t wave_max_u32(uint32_t v) {
    v = dpp_max_u32<kDppXor1>(v);
    v = dpp_max_u32<kDppXor2>(v);
    v = dpp_max_u32<kDppHalfMirror>(v);
    v = dpp_max_u32<kDppMirror>(v);
    v = dpp_max_u32<kDppBcast15, 0xA>(v);
    v = dpp_max_u32<kDppBcast31, 0xC>(v);
    return readlane_u32(v, 63);
}

__device__ __forceinline__ uint32_t wave_min_u32(uint32_t v) {
    v = dpp_min_u32<kDppXor1>(v);
    v = dpp_min_u32<kDppXor2>(v);
    v = dpp_min_u32<kDppHalfMirror>(v);
    v = dpp_min_u32<kDppMirror>(v);
    v = dpp_min_u32<kDppBcast15, 0xA>(v);
    v = dpp_min_u32<kDppBcast31, 0xC>(v);
    return readlane_u32(v, 63);
}

template <int CTRL>
__device__ __forceinline__ float dpp_add_f32(float v) {
    return v + __uint_as_float(dpp_u32<CTRL>(__float_as_uint(v)));
}

// Sum over each row of 16 lanes in a fixed order (deterministic); every lane
// of the row gets the row's sum.
__device__ __forceinline__ float row_sum_f32(float v) {
    v = dpp_add_f32<kDppXor1>(v);
    v = dpp_add_f32<kDppXor2>(v);
    v = dpp_add_f32<kDppHalfMirror>(v);
    v = dpp_add_f32<kDppMirror>(v);
    return v;
}

// Sum over the 64 lanes of a wave in a fixed order (deterministic); uniform result.
__device__ __forceinline__ float wave_sum_f32(float v) {
    v = dpp_add_f32<kDppXor1>(v);
    v = dpp_add_f32<kDppXor2>(v);
    v = dpp_add_f32<kDppHalfMirror>(v);
    v = dpp_add_f32<kDppMirror>(v);
    const float r0 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__float_as_int(v), 0));
    const float r1 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__float_as_int(v), 16));
    const float r2 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__float_as_int(v), 32));
    const float r3 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__float_as_int(v), 48));
    return (r0 + r1) + (r2 + r3);
}

// One wave: top-k of one token's E <= 64 * KPL logits (every lane active).
// Lane l holds logits l, l + 64, ... (KPL slots) as 64-bit keys
// order_bits(logit) << 32 | ~index, so that a larger key ranks first (higher
// logit, then lower expert index) and no two keys are equal.  Lane j < k
// returns the j-th selected expert and its routing weight: softmax over the k
// selected logits (renorm) or the full softmax over E read at the selected
// experts; an all -inf selection gets equal weights.
//
// Selection goes by threshold (topk_threshold): few elements lie at or above
// the k-th largest lane maximum, and only those are ranked.  When more than 64
// do (heavy ties near the top), k rounds of a wave maximum over per-lane sorted
// lists pick the winners one by one instead (topk_rounds).  Both give the same
// keys: the k largest, in descending order.

__device__ __forceinline__ uint64_t readlane_u64(uint64_t v, int lane) {
    const uint32_t lo = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)v, lane);
    const uint32_t hi = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)(v >> 32), lane);
    return (uint64_t)hi << 32 | lo;
}

// Number of lanes below this one whose bit is set in `mask`.
__device__ __forceinline__ int lanes_below(uint64_t mask) {
    return (int)__builtin_amdgcn_mbcnt_hi((uint32_t)(mask >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)mask, 0u));
}

// Threshold selection.  P = the largest 16-bit value that at least k of the
// 64 lane maxima reach in their top 16 bits (a search one bit at a time: one
// ballot count per step, the fewest instructions for a lone wave, which issues
// about one every six cycles); thr = P << 16.  The k lanes whose maxima reach
// thr hold k distinct elements >= thr, so the k-th largest element is >= thr
// and every selected element is among those >= thr.  When at most 64 are, they
// are gathered one per lane through `scratch` (128 keys of LDS owned by this
// wave, 16-byte aligned; slots 64.. take the writes of lanes with nothing to
// store, and slots past the last candidate are cleared first), each counts the
// larger keys among them (16 at a time from broadcast LDS reads: the cleared
// slots hold 0, below every key), and the k of rank < k are written back at
// their ranks.  Returns false (nothing selected) when more than 64 elements
// reach thr; the outcome is uniform across the wave.
template <int KPL>
__device__ __forceinline__ bool topk_threshold(const uint64_t (&key)[KPL], int k, int lane, uint64_t* scratch,
                                               uint64_t* sel) {
    uint32_t hi[KPL];
    uint32_t lmax = 0;
#pragma unroll
    for (int i = 0; i < KPL; ++i) {
        hi[i] = (uint32_t)(key[i] >> 32);
        lmax = hi[i] > lmax ? hi[i] : lmax;
    }
    const uint32_t l16 = lmax >> 16;
    uint32_t p = 0;
#pragma unroll
    for (int sh = 15; sh >= 0; --sh) {
        const uint32_t c = p | (1u << sh);
        p = __popcll(__ballot(l16 >= c)) >= k ? c : p;
    }
    const uint32_t thr = p << 16;
    uint64_t mask[KPL];
    int base[KPL];
    int n = 0;
#pragma unroll
    for (int i = 0; i < KPL; ++i) {
        mask[i] = __ballot(hi[i] >= thr);
        base[i] = n;
        n += __popcll(mask[i]);
    }
    if (n > 64) return false;
    scratch[lane] = 0ull;
#pragma unroll
    for (int i = 0; i < KPL; ++i) {
        // Position base[i] + (lanes below with a candidate in slot i), computed
        // on every lane (no branch) and used where this lane has one.
        const int pos = (int)__builtin_amdgcn_mbcnt_hi((uint32_t)(mask[i] >> 32),
                                                       __builtin_amdgcn_mbcnt_lo((uint32_t)mask[i], (uint32_t)base[i]));
        scratch[hi[i] >= thr ? pos : 64 + lane] = key[i];
    }
    // LDS accesses of one wave complete in program order; the barrier keeps the
    // compiler from moving them across each other.
    __builtin_amdgcn_wave_barrier();
    const uint64_t mine = scratch[lane];
    // Slots u0 .. u0 + 15 < 64 (n <= 64), the same address in every lane.
    int rank = 0;
    for (int u0 = 0; u0 < n; u0 += 16) {
        const ulonglong2* q = (const ulonglong2*)(scratch + u0);
        ulonglong2 c[8];
#pragma unroll
        for (int j = 0; j < 8; ++j) c[j] = q[j];
#pragma unroll
        for (int j = 0; j < 8; ++j) rank += (int)(c[j].x > mine) + (int)(c[j].y > mine);
    }
    __builtin_amdgcn_wave_barrier();
    scratch[lane < n && rank < k ? rank : 64 + lane] = mine;
    __builtin_amdgcn_wave_barrier();
    *sel = lane < k ? scratch[lane] : 0ull;
    __builtin_amdgcn_wave_barrier();
    return true;
}

// Batcher odd-even merge sort networks (compare-exchange index pairs) for
// 2, 4, 8 and 16 keys, listed as constants so every index is static.
template <int KPL> struct SortNet;
template <> struct SortNet<2> {
    static constexpr int N = 1;
    static constexpr int P[1][2] = {{0, 1}};
};
template <> struct SortNet<4> {
    static constexpr int N = 5;
    static constexpr int P[5][2] = {{0, 1}, {2, 3}, {0, 2}, {1, 3}, {1, 2}};
};
template <> struct SortNet<8> {
    static constexpr int N = 19;
    static constexpr int P[19][2] = {{0, 1}, {2, 3}, {4, 5}, {6, 7}, {0, 2}, {1, 3}, {4, 6}, {5, 7}, {1, 2}, {5, 6}, {0, 4}, {1, 5}, {2, 6}, {3, 7}, {2, 4}, {3, 5}, {1, 2}, {3, 4}, {5, 6}};
};
template <> struct SortNet<16> {
    static constexpr int N = 63;
    static constexpr int P[63][2] = {{0, 1}, {2, 3}, {4, 5}, {6, 7}, {8, 9}, {10, 11}, {12, 13}, {14, 15}, {0, 2}, {1, 3}, {4, 6}, {5, 7}, {8, 10}, {9, 11}, {12, 14}, {13, 15}, {1, 2}, {5, 6}, {9, 10}, {13, 14}, {0, 4}, {1, 5}, {2, 6}, {3, 7}, {8, 12}, {9, 13}, {10, 14}, {11, 15}, {2, 4}, {3, 5}, {10, 12}, {11, 13}, {1, 2}, {3, 4}, {5, 6}, {9, 10}, {11, 12}, {13, 14}, {0, 8}, {1, 9}, {2, 10}, {3, 11}, {4, 12}, {5, 13}, {6, 14}, {7, 15}, {4, 8}, {5, 9}, {6, 10}, {7, 11}, {2, 4}, {3, 5}, {6, 8}, {7, 9}, {10, 12}, {11, 13}, {1, 2}, {3, 4}, {5, 6}, {7, 8}, {9, 10}, {11, 12}, {13, 14}};
};

// Sort a lane's packed keys descending: key64 = order_bits(logit) << 32 | ~index,
// so that a larger key64 ranks first (higher logit, then lower index).  Each
// compare-exchange is one 64-bit compare and two selects, with no branches.
template <int KPL>
__device__ __forceinline__ void sort_desc(uint64_t (&key)[KPL]) {
#pragma unroll
    for (int c = 0; c < SortNet<KPL>::N; ++c) {
        const int i = SortNet<KPL>::P[c][0], j = SortNet<KPL>::P[c][1];
        const uint64_t a = key[i], b = key[j];
        const bool sw = b > a;
        key[i] = sw ? b : a;
        key[j] = sw ? a : b;
    }
}

// Rounds selection: each lane sorts its keys (descending); each round takes
// the wave maximum of the lanes' heads, whose owner (a single lane: keys are
// distinct) shifts its list by one.  Lane r < k gets the round-r key.
template <int KPL>
__device__ __forceinline__ uint64_t topk_rounds(uint64_t (&key)[KPL], int k, int lane) {
    sort_desc<KPL>(key);
    uint64_t sel = 0;
    for (int r = 0; r < k; ++r) {
        const uint32_t head = (uint32_t)(key[0] >> 32);
        const uint32_t m = wave_max_u32(head);
        const uint64_t cand = __ballot(head == m);
        int owner;
        if (__popcll(cand) == 1) {
            owner = __ffsll((unsigned long long)cand) - 1;
        } else {   // equal logits: the lowest expert index among the candidates
            const uint32_t ix = 0xFFFFFFFFu - (uint32_t)key[0];
            owner = (int)(wave_min_u32(head == m ? ix : 0xFFFFFFFFu) & 63u);
        }
        const uint64_t won = readlane_u64(key[0], owner);
        if (lane == r) sel = won;
        if (lane == owner) {
#pragma unroll
            for (int i = 0; i + 1 < KPL; ++i) key[i] = key[i + 1];
            key[KPL - 1] = 0ull;
        }
    }
    return sel;
}

// A row's logits as this lane holds them (l, l + 64, ...).  Every load is
// unconditional (clamped address) so that all of them are in flight together;
// out-of-range slots are masked afterwards, branch-free.
template <int KPL>
__device__ __forceinline__ void topk_load(const float* __restrict__ row, int E, int lane, float (&lv)[KPL]) {
#pragma unroll
    for (int i = 0; i < KPL; ++i) {
        const int e = lane + 64 * i;
        lv[i] = row[e < E ? e : E - 1];
    }
}

// want_w false: only the ids (rank order); *out_w is left unset.
template <int KPL>
__device__ __forceinline__ void topk_of_values(const float (&lv)[KPL], int E, int k, int renorm, int lane,
                                               uint64_t* scratch, int* out_id, float* out_w, bool want_w = true) {
    uint64_t key[KPL];
#pragma unroll
    for (int i = 0; i < KPL; ++i) {
        const uint32_t e = (uint32_t)(lane + 64 * i);
        const uint64_t valid = 0ull - (uint64_t)(e < (uint32_t)E);
        key[i] = (((uint64_t)order_bits(lv[i]) << 32) | (uint64_t)(0xFFFFFFFFu - e)) & valid;
    }
    uint64_t sel;
    if (!topk_threshold<KPL>(key, k, lane, scratch, &sel)) sel = topk_rounds<KPL>(key, k, lane);
    const uint32_t my_key = (uint32_t)(sel >> 32);
    const int my_id = lane < k ? (int)(0xFFFFFFFFu - (uint32_t)sel) : -1;
    if (!want_w) {
        *out_id = my_id;
        return;
    }
    const uint32_t top_key = readlane_u32(my_key, 0);
    const float top = from_order_bits(top_key);
    const float my_logit = from_order_bits(my_key);
    const bool all_neg_inf = (top == -INFINITY);
    float e_sel = 0.f;
    if (lane < k) e_sel = all_neg_inf ? 1.f : expf(my_logit - top);
    float denom;
    if (renorm) {
        denom = wave_sum_f32(e_sel);
    } else {
        float part = 0.f;
#pragma unroll
        for (int i = 0; i < KPL; ++i) {
            const int e = lane + 64 * i;
            if (e < E) part += all_neg_inf ? 1.f : expf(lv[i] - top);
        }
        denom = wave_sum_f32(part);
    }
    *out_id = my_id;
    *out_w = e_sel / denom;
}

template <int KPL>
__device__ __forceinline__ void wave_topk_kpl(const float* __restrict__ row, int E, int k, int renorm, int lane,
                                              uint64_t* scratch, int* out_id, float* out_w, bool want_w) {
    float lv[KPL];
    topk_load<KPL>(row, E, lane, lv);
    topk_of_values<KPL>(lv, E, k, renorm, lane, scratch, out_id, out_w, want_w);
}

// Two rows by one wave, one after the other, with both rows' loads issued
// first: the second row's logits arrive while the first is ranked.  With
// `two` false only row0 is ranked (its loads are issued twice).
template <int KPL>
__device__ __forceinline__ void wave_topk2_kpl(const float* __restrict__ row0, const float* __restrict__ row1,
                                               bool two, int E, int k, int renorm, int lane, uint64_t* scratch,
                                               int (&out_id)[2], float (&out_w)[2]) {
    float l0[KPL], l1[KPL];
    topk_load<KPL>(row0, E, lane, l0);
    topk_load<KPL>(two ? row1 : row0, E, lane, l1);
    topk_of_values<KPL>(l0, E, k, renorm, lane, scratch, &out_id[0], &out_w[0]);
    if (two) topk_of_values<KPL>(l1, E, k, renorm, lane, scratch, &out_id[1], &out_w[1]);
}

// `scratch`: 128 keys of LDS owned by the calling wave.  want_w false: the ids
// only (no softmax), for callers that never read the weights.
__device__ __forceinline__ void wave_topk(const float* __restrict__ row, int E, int k, int renorm, int lane,
                                          uint64_t* scratch, int* out_id, float* out_w, bool want_w = true) {
    if (E <= 128) wave_topk_kpl<2>(row, E, k, renorm, lane, scratch, out_id, out_w, want_w);
    else if (E <= 256) wave_topk_kpl<4>(row, E, k, renorm, lane, scratch, out_id, out_w, want_w);
    else if (E <= 512) wave_topk_kpl<8>(row, E, k, renorm, lane, scratch, out_id, out_w, want_w);
    else wave_topk_kpl<16>(row, E, k, renorm, lane, scratch, out_id, out_w, want_w);
}

__device__ __forceinline__ void wave_topk2(const float* __restrict__ row0, const float* __restrict__ row1, bool two,
                                           int E, int k, int renorm, int lane, uint64_t* scratch, int (&out_id)[2],
                                           float (&out_w)[2]) {
    if (E <= 128) wave_topk2_kpl<2>(row0, row1, two, E, k, renorm, lane, scratch, out_id, out_w);
    else if (E <= 256) wave_topk2_kpl<4>(row0, row1, two, E, k, renorm, lane, scratch, out_id, out_w);
    else if (E <= 512) wave_topk2_kpl<8>(row0, row1, two, E, k, renorm, lane, scratch, out_id, out_w);
    else wave_topk2_kpl<16>(row0, row1, two, E, k, renorm, lane, scratch, out_id, out_w);
}

}  // namespace moe
