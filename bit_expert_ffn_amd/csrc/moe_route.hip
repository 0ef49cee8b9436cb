// Top-k routing and the expert-major bucketing of the decode / verify path.
//
// Routing follows Krasis white paper 5.3 ("select top-k expert IDs and
// weights") and kairos-engine README "The MoE forward" (top-k over the router
// logits).  Order: logit descending, expert index ascending on ties; -0 == +0;
// NaN below every number.  One wavefront owns one token: each lane holds up to
// 16 logits as 64-bit keys (orderable float bits << 32 | ~index), and k rounds
// of a wave-wide max pick the experts in rank order.  Every comparison is on
// integers derived from the same fp32 values the oracle sorts, so ids are
// exact.  Weights are the softmax over the k selected logits (or, without
// renormalisation, the full softmax read at the selected experts).
//
// Bucketing follows the Strata page, "The plan: three destinations per
// expert" (a window's routed ids are de-duplicated so an expert chosen by two
// tokens is computed once for both) and the kairos README (expert-major
// buckets).  Pairs (token, slot) are sorted by (expert, token); consecutive
// pairs of one expert form groups of at most kGroup tokens that the GEMV
// kernels process together.
#include "moe_internal.h"

namespace moe {

__device__ __forceinline__ uint32_t order_bits(float f) {
    uint32_t u = __float_as_uint(f);
    if (f != f) return 0u;                       // NaN ranks below -inf
    if ((u & 0x7FFFFFFFu) == 0u) u = 0u;         // -0 and +0 compare equal
    return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

__device__ __forceinline__ float from_order_bits(uint32_t k) {
    if (k == 0u) return __uint_as_float(0x7FC00000u);
    uint32_t u = (k & 0x80000000u) ? (k & 0x7FFFFFFFu) : ~k;
    return __uint_as_float(u);
}

__device__ __forceinline__ uint64_t wave_max_u64(uint64_t v) {
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) {
        uint64_t o = __shfl_xor(v, off, 64);
        v = o > v ? o : v;
    }
    return v;
}

__device__ __forceinline__ float wave_sum_f32(float v) {
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) v += __shfl_xor(v, off, 64);
    return v;
}

// One wave: top-k of one token's E logits.  Lane j < k returns (id_j, w_j).
__device__ void wave_topk(const float* __restrict__ row, int E, int k, int renorm, int lane, int* out_id,
                          float* out_w) {
    uint64_t key[16];
    const int nk = (E + 63) >> 6;
#pragma unroll
    for (int i = 0; i < 16; ++i) {
        int e = lane + 64 * i;
        key[i] = 0;
        if (i < nk && e < E)
            key[i] = ((uint64_t)order_bits(row[e]) << 32) | (uint64_t)(0xFFFFFFFFu - (uint32_t)e);
    }
    uint64_t best = 0;
#pragma unroll
    for (int i = 0; i < 16; ++i) best = key[i] > best ? key[i] : best;

    int my_id = -1;
    float my_logit = 0.f;
    float top = 0.f;
    for (int r = 0; r < k; ++r) {
        uint64_t m = wave_max_u64(best);
        if (lane == r) {
            my_id = (int)(0xFFFFFFFFu - (uint32_t)(m & 0xFFFFFFFFu));
            my_logit = from_order_bits((uint32_t)(m >> 32));
        }
        if (r == 0) top = from_order_bits((uint32_t)(m >> 32));
        if (best == m) {  // keys are unique: exactly one lane owns m
            best = 0;
#pragma unroll
            for (int i = 0; i < 16; ++i) {
                if (key[i] == m) key[i] = 0;
                best = key[i] > best ? key[i] : best;
            }
        }
    }
    const bool all_neg_inf = (top == -INFINITY);
    float e_sel = 0.f;
    if (lane < k) e_sel = all_neg_inf ? 1.f : expf(my_logit - top);
    float denom;
    if (renorm) {
        denom = wave_sum_f32(e_sel);
    } else {
        float part = 0.f;
        for (int i = 0; i < nk; ++i) {
            int e = lane + 64 * i;
            if (e < E) part += all_neg_inf ? 1.f : expf(row[e] - top);
        }
        denom = wave_sum_f32(part);
    }
    *out_id = my_id;
    *out_w = e_sel / denom;
}

// Routing only: one wave per token, 4 tokens per workgroup.
__global__ void __launch_bounds__(256) route_topk_kernel(const float* __restrict__ logits, int T, int E, int k,
                                                         int renorm, int* __restrict__ ids,
                                                         float* __restrict__ w) {
    const int lane = threadIdx.x & 63;
    const int t = blockIdx.x * 4 + (threadIdx.x >> 6);
    if (t >= T) return;
    int id;
    float wt;
    wave_topk(logits + (size_t)t * E, E, k, renorm, lane, &id, &wt);
    if (lane < k) {
        ids[(size_t)t * k + lane] = id;
        w[(size_t)t * k + lane] = wt;
    }
}

hipError_t launch_route_topk(const float* logits, int T, int E, int k, int renorm, int* ids, float* w,
                             hipStream_t s) {
    if (T == 0) return hipSuccess;
    hipLaunchKernelGGL(route_topk_kernel, dim3((T + 3) / 4), dim3(256), 0, s, logits, T, E, k, renorm, ids, w);
    return hipGetLastError();
}

// Routing + bucketing for T <= kSmallT tokens in one workgroup of 512 threads
// (wave t routes token t).  identity != 0 skips routing: every token uses
// expert 0 with weight 1 (a single expert's FFN).
__global__ void __launch_bounds__(512) route_bucket_small_kernel(
    const float* __restrict__ logits, int T, int E, int k, int renorm, int identity, int* __restrict__ ids,
    float* __restrict__ w, SmallMeta* __restrict__ meta, int* __restrict__ pair_tok, int* __restrict__ pair_slot,
    int* __restrict__ pair_exp, int* __restrict__ slot_pair, int* __restrict__ group_first,
    int* __restrict__ group_n, int* __restrict__ active, int* __restrict__ counters, int n_counters) {
    __shared__ int s_id[kSmallT * kMaxK];
    __shared__ int s_rank[kSmallT * kMaxK];
    __shared__ int s_pos[kSmallT * kMaxK];
    __shared__ int s_cnt[kSmallT * kMaxK];
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wv = tid >> 6;

    for (int i = tid; i < n_counters; i += blockDim.x) counters[i] = 0;

    if (identity) {
        for (int t = tid; t < T; t += blockDim.x) {
            s_id[t] = 0;
            ids[t] = 0;
            w[t] = 1.f;
        }
    } else if (wv < T) {
        int id;
        float wt;
        wave_topk(logits + (size_t)wv * E, E, k, renorm, lane, &id, &wt);
        if (lane < k) {
            s_id[wv * k + lane] = id;
            ids[wv * k + lane] = id;
            w[wv * k + lane] = wt;
        }
    }
    __syncthreads();

    const int n = T * k;
    for (int p = tid; p < n; p += blockDim.x) {
        const int e = s_id[p], t = p / k, j = p % k;
        int rank = 0, pos = 0, cnt = 0;
        for (int q = 0; q < n; ++q) {
            const int eq = s_id[q], tq = q / k;
            rank += (eq < e) || (eq == e && tq < t);
            pos += (eq == e && tq < t);
            cnt += (eq == e);
        }
        s_rank[p] = rank;
        s_pos[p] = pos;
        s_cnt[p] = cnt;
        pair_tok[rank] = t;
        pair_slot[rank] = j;
        pair_exp[rank] = e;
        slot_pair[p] = rank;
    }
    __syncthreads();

    for (int p = tid; p < n; p += blockDim.x) {
        const int pos = s_pos[p];
        if (pos % kGroup == 0) {
            int g = 0;
            for (int q = 0; q < n; ++q) g += (s_pos[q] % kGroup == 0) && (s_rank[q] < s_rank[p]);
            group_first[g] = s_rank[p];
            group_n[g] = min(kGroup, s_cnt[p] - pos);
        }
        if (pos == 0) {
            int a = 0;
            for (int q = 0; q < n; ++q) a += (s_pos[q] == 0) && (s_id[q] < s_id[p]);
            active[a] = s_id[p];
        }
    }
    if (tid == 0) {
        int ng = 0, na = 0;
        for (int q = 0; q < n; ++q) {
            ng += (s_pos[q] % kGroup == 0);
            na += (s_pos[q] == 0);
        }
        meta->n_pairs = n;
        meta->n_groups = ng;
        meta->n_active = na;
        meta->pad = 0;
    }
}

hipError_t launch_route_bucket_small(const float* logits, int T, int E, int k, int renorm, int identity,
                                     int* ids, float* w, const SmallLayout& L, char* ws, int n_counters,
                                     hipStream_t s) {
    hipLaunchKernelGGL(route_bucket_small_kernel, dim3(1), dim3(512), 0, s, logits, T, E, k, renorm, identity, ids,
                       w, (SmallMeta*)(ws + L.meta), (int*)(ws + L.pair_tok), (int*)(ws + L.pair_slot),
                       (int*)(ws + L.pair_exp), (int*)(ws + L.slot_pair), (int*)(ws + L.group_first),
                       (int*)(ws + L.group_n), (int*)(ws + L.active), (int*)(ws + L.tile_cnt), n_counters);
    return hipGetLastError();
}

}  // namespace moe
