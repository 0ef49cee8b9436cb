// Top-k routing (Krasis white paper 5.3 "select top-k expert IDs and
// weights"; kairos-engine README "The MoE forward": top-k over the router
// logits).  Order: logit descending, expert index ascending on ties; -0 == +0;
// NaN below every number.  One wavefront owns one token: each lane holds up to
// 16 logits as 64-bit keys; the few at or above a ballot-searched threshold are
// ranked against each other (k rounds of a DPP wave maximum when ties leave too
// many).  Every comparison is on integers derived from the same fp32
// values the oracle sorts, so ids are exact.  Weights: softmax over the k
// selected logits, or the full softmax read at the selected experts.
#include "moe_device.h"
#include "moe_internal.h"

namespace moe {

// Routing only: one wave per token, 4 tokens per workgroup.
__global__ void __launch_bounds__(256) route_topk_kernel(const float* __restrict__ logits, int T, int E, int k,
                                                         int renorm, int* __restrict__ ids,
                                                         float* __restrict__ w) {
    __shared__ __align__(16) uint64_t scratch[4][128];
    const int lane = threadIdx.x & 63;
    const int t = blockIdx.x * 4 + (threadIdx.x >> 6);
    if (t >= T) return;
    int id;
    float wt;
    wave_topk(logits + (size_t)t * E, E, k, renorm, lane, scratch[threadIdx.x >> 6], &id, &wt);
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

}  // namespace moe
