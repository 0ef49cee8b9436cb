// Router front end: logits[t][e] = sum_h W_r[e][h] x'[t][h] with bf16 router
// weights W_r [E][H] and fp32 accumulation.  x' is the activation row x, or
// (kairos-engine README, "The MoE forward": the router reads its input through
// its own weightless norm, and its scale is per input dimension)
//     x' = x / sqrt(mean_h x^2 + eps)   (norm), then   x'_h *= in_scale[h].
// Every product of a bf16 weight and an fp32 x' is formed in fp32 and summed
// in fp32.
//
// T <= 8 (decode, verify windows): router_gemv_kernel, one wave per expert
// row (4 per workgroup).  Each workgroup first computes the norm factor of
// every token (one wave per token, a fixed-order sum).  Lane l reads the
// 16-byte chunks l, l + 64, ... of the weight row (coalesced) and the same
// chunks of each token's row; per token it accumulates in that order and a
// fixed DPP tree sums the lanes.  A token's logits are therefore bitwise the
// same whatever the other tokens of the window.
// T > 8 (prefill): router_gemm_kernel computes 64 x 64 tiles of (tokens x
// experts) from 32-wide slices of x' and W_r staged in LDS; each tile first
// computes its tokens' norm factors (one wave per token, the same arithmetic).
#include "moe_device.h"
#include "moe_internal.h"

namespace moe {

constexpr int kRtTileT = 64;   // tokens per GEMM tile
constexpr int kRtTileE = 64;   // experts per GEMM tile
constexpr int kRtK = 32;       // input dimensions per LDS slice

struct RouterParams {
    const uint16_t* wr;        // [E][H] bf16 bits
    const float* in_scale;     // [H] or null
    const void* x;             // [T][H] bf16 bits or fp32
    float* logits;             // [T][E]
    int E, H, T, norm;
    float eps;
};

template <int XDT>
__device__ __forceinline__ float x_at(const void* x, size_t i) {
    if constexpr (XDT == 1) return __uint_as_float((uint32_t)((const uint16_t*)x)[i] << 16);
    else return ((const float*)x)[i];
}

// 1 / sqrt(mean of x^2 + eps) of token t's row, by one wave: lane l sums
// positions l, l + 64, ... in order, then a fixed DPP tree.
template <int XDT>
__device__ __forceinline__ float row_rinv(const RouterParams& p, int t, int lane) {
    float ss = 0.f;
    const size_t base = (size_t)t * p.H;
    for (int h = lane; h < p.H; h += 64) {
        const float v = x_at<XDT>(p.x, base + h);
        ss = __builtin_fmaf(v, v, ss);
    }
    ss = wave_sum_f32(ss);
    return 1.f / sqrtf(ss / (float)p.H + p.eps);
}

// x'[t][h0 .. h0 + 7] from the activations (8 consecutive values).
template <int XDT>
__device__ __forceinline__ void x_chunk(const RouterParams& p, int t, int h0, float r, float (&v)[8]) {
    const size_t base = (size_t)t * p.H + h0;
    if constexpr (XDT == 1) {
        const uint4 u = *reinterpret_cast<const uint4*>((const uint16_t*)p.x + base);
        const uint32_t w[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            v[2 * i] = __uint_as_float(w[i] << 16);
            v[2 * i + 1] = __uint_as_float(w[i] & 0xFFFF0000u);
        }
    } else {
        const float4 a = *reinterpret_cast<const float4*>((const float*)p.x + base);
        const float4 b = *reinterpret_cast<const float4*>((const float*)p.x + base + 4);
        v[0] = a.x; v[1] = a.y; v[2] = a.z; v[3] = a.w;
        v[4] = b.x; v[5] = b.y; v[6] = b.z; v[7] = b.w;
    }
    if (p.norm) {
#pragma unroll
        for (int i = 0; i < 8; ++i) v[i] = v[i] * r;
    }
    if (p.in_scale) {
        const float4 a = *reinterpret_cast<const float4*>(p.in_scale + h0);
        const float4 b = *reinterpret_cast<const float4*>(p.in_scale + h0 + 4);
        const float s[8] = {a.x, a.y, a.z, a.w, b.x, b.y, b.z, b.w};
#pragma unroll
        for (int i = 0; i < 8; ++i) v[i] = v[i] * s[i];
    }
}

template <int XDT>
__global__ void __launch_bounds__(256) router_gemv_kernel(RouterParams p) {
    __shared__ float rinv[kSmallT];
    const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
    if (p.norm)
        for (int t = wv; t < p.T; t += 4) {
            const float r = row_rinv<XDT>(p, t, lane);
            if (lane == 0) rinv[t] = r;
        }
    __syncthreads();
    const int e = blockIdx.x * 4 + wv;
    if (e >= p.E) return;
    float acc[kSmallT];
#pragma unroll
    for (int t = 0; t < kSmallT; ++t) acc[t] = 0.f;
    const uint16_t* row = p.wr + (size_t)e * p.H;
    for (int h0 = 8 * lane; h0 < p.H; h0 += 8 * 64) {
        const uint4 u = *reinterpret_cast<const uint4*>(row + h0);
        const uint32_t w2[4] = {u.x, u.y, u.z, u.w};
        float w[8];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            w[2 * i] = __uint_as_float(w2[i] << 16);
            w[2 * i + 1] = __uint_as_float(w2[i] & 0xFFFF0000u);
        }
#pragma unroll
        for (int t = 0; t < kSmallT; ++t) {
            if (t < p.T) {
                float v[8];
                x_chunk<XDT>(p, t, h0, p.norm ? rinv[t] : 1.f, v);
#pragma unroll
                for (int i = 0; i < 8; ++i) acc[t] = __builtin_fmaf(w[i], v[i], acc[t]);
            }
        }
    }
#pragma unroll
    for (int t = 0; t < kSmallT; ++t) {
        if (t < p.T) {
            const float s = wave_sum_f32(acc[t]);
            if (lane == 0) p.logits[(size_t)t * p.E + e] = s;
        }
    }
}

// One 64 x 64 tile of (tokens, experts); thread (ty, tx) owns tokens
// 4 ty .. 4 ty + 3 and experts 4 tx .. 4 tx + 3 and sums over h in slice
// order, each slice in h order.
template <int XDT>
__global__ void __launch_bounds__(256) router_gemm_kernel(RouterParams p) {
    __shared__ __align__(16) float xs[kRtK][kRtTileT + 4];
    __shared__ __align__(16) float wsl[kRtK][kRtTileE + 4];
    __shared__ float rinv[kRtTileT];
    const int tid = threadIdx.x;
    const int t0 = blockIdx.x * kRtTileT, e0 = blockIdx.y * kRtTileE;
    if (p.norm)
        for (int r = tid >> 6; r < kRtTileT; r += 4) {
            const float v = t0 + r < p.T ? row_rinv<XDT>(p, t0 + r, tid & 63) : 0.f;
            if ((tid & 63) == 0) rinv[r] = v;
        }
    __syncthreads();
    const int tx = tid & 15, ty = tid >> 4;
    float acc[4][4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = 0.f;
    for (int h0 = 0; h0 < p.H; h0 += kRtK) {
        // 64 x 32 values of x' and of W_r, 8 per thread: thread i takes
        // column i % 32 of rows i / 32 (+ 8 per step).
#pragma unroll
        for (int s = 0; s < 8; ++s) {
            const int idx = tid + 256 * s, r = idx >> 5, c = idx & 31, h = h0 + c;
            const int t = t0 + r;
            float xv = 0.f;
            if (t < p.T) {
                xv = x_at<XDT>(p.x, (size_t)t * p.H + h);
                if (p.norm) xv = xv * rinv[r];
                if (p.in_scale) xv = xv * p.in_scale[h];
            }
            xs[c][r] = xv;
            const int e = e0 + r;
            wsl[c][r] = e < p.E ? __uint_as_float((uint32_t)p.wr[(size_t)e * p.H + h] << 16) : 0.f;
        }
        __syncthreads();
#pragma unroll 8
        for (int c = 0; c < kRtK; ++c) {
            const float4 a = *reinterpret_cast<const float4*>(&xs[c][4 * ty]);
            const float4 b = *reinterpret_cast<const float4*>(&wsl[c][4 * tx]);
            const float av[4] = {a.x, a.y, a.z, a.w}, bv[4] = {b.x, b.y, b.z, b.w};
#pragma unroll
            for (int i = 0; i < 4; ++i)
#pragma unroll
                for (int j = 0; j < 4; ++j) acc[i][j] = __builtin_fmaf(bv[j], av[i], acc[i][j]);
        }
        __syncthreads();
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int t = t0 + 4 * ty + i;
        if (t >= p.T) continue;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int e = e0 + 4 * tx + j;
            if (e < p.E) p.logits[(size_t)t * p.E + e] = acc[i][j];
        }
    }
}

hipError_t launch_router(const void* wr, const float* in_scale, int norm, float eps, int E, int H, const void* x,
                         int x_dtype, int T, float* logits, hipStream_t s) {
    RouterParams p{};
    p.wr = (const uint16_t*)wr;
    p.in_scale = in_scale;
    p.x = x;
    p.logits = logits;
    p.E = E;
    p.H = H;
    p.T = T;
    p.norm = norm;
    p.eps = eps;
    const bool bf = x_dtype == 1;
    if (T <= kSmallT) {
        const dim3 grid((E + 3) / 4);
        if (bf) hipLaunchKernelGGL(router_gemv_kernel<1>, grid, dim3(256), 0, s, p);
        else hipLaunchKernelGGL(router_gemv_kernel<0>, grid, dim3(256), 0, s, p);
        return hipGetLastError();
    }
    const dim3 grid((T + kRtTileT - 1) / kRtTileT, (E + kRtTileE - 1) / kRtTileE);
    if (bf) hipLaunchKernelGGL(router_gemm_kernel<1>, grid, dim3(256), 0, s, p);
    else hipLaunchKernelGGL(router_gemm_kernel<0>, grid, dim3(256), 0, s, p);
    return hipGetLastError();
}

}  // namespace moe
