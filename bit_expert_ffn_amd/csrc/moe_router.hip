// Router front end: logits[t][e] = sum_h W_r[e][h] x'[t][h] with bf16 router
// weights W_r [E][H] and fp32 accumulation.  x' is the activation row x, or
// (kairos-engine README, "The MoE forward": the router reads its input through
// its own weightless norm, and its scale is per input dimension)
//     x' = x / sqrt(mean_h x^2 + eps)   (norm), then   x'_h *= in_scale[h].
// Every product of a bf16 weight and an fp32 x' is formed in fp32 and summed
// in fp32.
//
// T <= 8 (decode, verify windows): router_gemv_kernel, one workgroup per
// expert row, its 256 threads splitting the row's 16-byte chunks; each thread
// issues the loads of its chunks of the weight row and of the matching
// activations (and scale) at once; then, per token, it accumulates
// w * (x * scale) over its chunks in order, and, for the norm, x * x; a fixed
// DPP tree sums each wave, the four waves' sums are added in wave order, and
// the norm factor 1 / sqrt(mean x^2 + eps) multiplies the sum (a per-token
// scalar: W (x r s) = r W (x s)).  A token's logits are therefore bitwise the
// same whatever the other tokens of the window, and a call waits for one
// round trip to memory.
// T > 8 (prefill): router_gemm_kernel computes 64 x 64 tiles of (tokens x
// experts) from 32-wide slices of x' and W_r staged in LDS; each tile first
// computes its tokens' norm factors (one wave per token).
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

constexpr int kRtCPT = 2;   // 16-byte weight chunks (8 weights) a thread takes per round

// One workgroup per expert row e; thread i of the 256 takes the row's 16-byte
// chunks i, i + 256, ... (two per round), and every load of a round (the
// weights, each token's 8 matching activations, the scale) is issued before
// any product, straight from memory (the activations are read by every
// workgroup, so from L2).  Per token, a thread accumulates w * (x * scale)
// over its chunks in order (and x * x for the norm); a fixed DPP tree sums
// each wave and the four waves' sums are added in wave order.
template <int XDT>
__global__ void __launch_bounds__(256) router_gemv_kernel(RouterParams p) {
    constexpr int XW = XDT == 1 ? 1 : 2;       // 16-byte words of 8 activations
    __shared__ float part[4][kSmallT][2];
    const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
    const int e = blockIdx.x;
    const int T = p.T;
    const int n_ch = p.H / 8;
    const uint16_t* row = p.wr + (size_t)e * p.H;
    const uint8_t* xb = (const uint8_t*)p.x;
    float acc[kSmallT], ss[kSmallT];
#pragma unroll
    for (int t = 0; t < kSmallT; ++t) acc[t] = ss[t] = 0.f;
    for (int c0 = 0; c0 < n_ch; c0 += 256 * kRtCPT) {
        uint4 wch[kRtCPT], xv[kRtCPT][kSmallT][XW];
        float4 sv[kRtCPT][2];
#pragma unroll
        for (int i = 0; i < kRtCPT; ++i) {
            const int c = c0 + tid + 256 * i;
            const int cc = c < n_ch ? c : n_ch - 1;   // clamped: every load unconditional
            wch[i] = *reinterpret_cast<const uint4*>(row + 8 * cc);
#pragma unroll
            for (int t = 0; t < kSmallT; ++t)
                if (t < T)
#pragma unroll
                    for (int q = 0; q < XW; ++q)
                        xv[i][t][q] = *reinterpret_cast<const uint4*>(xb + ((size_t)t * p.H + 8 * cc) * (XDT == 1 ? 2 : 4) + 16 * q);
            if (p.in_scale) {
                sv[i][0] = reinterpret_cast<const float4*>(p.in_scale)[2 * cc];
                sv[i][1] = reinterpret_cast<const float4*>(p.in_scale)[2 * cc + 1];
            }
        }
#pragma unroll
        for (int i = 0; i < kRtCPT; ++i) {
            if (c0 + tid + 256 * i >= n_ch) continue;
            const uint32_t w2[4] = {wch[i].x, wch[i].y, wch[i].z, wch[i].w};
            float w[8];
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                w[2 * j] = __uint_as_float(w2[j] << 16);
                w[2 * j + 1] = __uint_as_float(w2[j] & 0xFFFF0000u);
            }
            const float sc[8] = {sv[i][0].x, sv[i][0].y, sv[i][0].z, sv[i][0].w,
                                 sv[i][1].x, sv[i][1].y, sv[i][1].z, sv[i][1].w};
#pragma unroll
            for (int t = 0; t < kSmallT; ++t) {
                if (t >= T) continue;
                float v[8];
                if constexpr (XDT == 1) {
                    const uint32_t x2[4] = {xv[i][t][0].x, xv[i][t][0].y, xv[i][t][0].z, xv[i][t][0].w};
#pragma unroll
                    for (int j = 0; j < 4; ++j) {
                        v[2 * j] = __uint_as_float(x2[j] << 16);
                        v[2 * j + 1] = __uint_as_float(x2[j] & 0xFFFF0000u);
                    }
                } else {
                    const uint4 a = xv[i][t][0], b = xv[i][t][XW - 1];
                    v[0] = __uint_as_float(a.x); v[1] = __uint_as_float(a.y);
                    v[2] = __uint_as_float(a.z); v[3] = __uint_as_float(a.w);
                    v[4] = __uint_as_float(b.x); v[5] = __uint_as_float(b.y);
                    v[6] = __uint_as_float(b.z); v[7] = __uint_as_float(b.w);
                }
#pragma unroll
                for (int j = 0; j < 8; ++j) {
                    if (p.norm) ss[t] = __builtin_fmaf(v[j], v[j], ss[t]);
                    const float xs = p.in_scale ? v[j] * sc[j] : v[j];
                    acc[t] = __builtin_fmaf(w[j], xs, acc[t]);
                }
            }
        }
    }
#pragma unroll
    for (int t = 0; t < kSmallT; ++t) {
        if (t < T) {
            const float a = wave_sum_f32(acc[t]);
            const float q = p.norm ? wave_sum_f32(ss[t]) : 0.f;
            if (lane == 0) {
                part[wv][t][0] = a;
                part[wv][t][1] = q;
            }
        }
    }
    __syncthreads();
    if (tid < T) {
        float sum = (part[0][tid][0] + part[1][tid][0]) + (part[2][tid][0] + part[3][tid][0]);
        if (p.norm) {
            const float q = (part[0][tid][1] + part[1][tid][1]) + (part[2][tid][1] + part[3][tid][1]);
            sum = sum * (1.f / sqrtf(q / (float)p.H + p.eps));
        }
        p.logits[(size_t)tid * p.E + e] = sum;
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
        if (bf) hipLaunchKernelGGL(router_gemv_kernel<1>, dim3(E), dim3(256), 0, s, p);
        else hipLaunchKernelGGL(router_gemv_kernel<0>, dim3(E), dim3(256), 0, s, p);
        return hipGetLastError();
    }
    const dim3 grid((T + kRtTileT - 1) / kRtTileT, (E + kRtTileE - 1) / kRtTileE);
    if (bf) hipLaunchKernelGGL(router_gemm_kernel<1>, grid, dim3(256), 0, s, p);
    else hipLaunchKernelGGL(router_gemm_kernel<0>, grid, dim3(256), 0, s, p);
    return hipGetLastError();
}

}  // namespace moe
