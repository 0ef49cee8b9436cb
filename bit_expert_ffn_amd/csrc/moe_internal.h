// Internal declarations shared by the HIP translation units of libmoe_ffn.
// Nothing here is part of the C ABI (include/moe_ffn.h).
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace moe {

constexpr int kMaxE = 1024;        // logits per token held by one wave (16 per lane)
constexpr int kMaxK = 32;          // selected experts per token
constexpr int kSmallT = 8;         // decode / verify window limit of the GEMV path
constexpr int kGroup = 2;          // tokens of one expert processed together on the GEMV path
constexpr int kGemvThreads = 256;  // workgroup size of the GEMV kernels
constexpr int kMaxBlocksPerRow = 256;

// Bytes of one block: 16 code bytes + one fp16 scale.
constexpr int kBlockCodeBytes = 16;
constexpr int kBlockBytes = 18;

inline int codes_per_block(int qtype) { return qtype == 1 ? 64 : (qtype == 2 ? 32 : 0); }

// Routing / bucketing results of the GEMV path, written by the route kernel.
struct SmallMeta {
    int n_pairs;    // T * k (token, slot) pairs
    int n_groups;   // expert-major groups of <= kGroup pairs
    int n_active;   // distinct experts
    int pad;
};

// Workspace layout for the GEMV path (T <= kSmallT), byte offsets.
struct SmallLayout {
    size_t ids, w, meta, pair_tok, pair_slot, pair_exp, slot_pair, group_first, group_n, active;
    size_t a_hi, a_lo;       // [pairs][FF] bf16: SwiGLU output split into two bf16 terms
    size_t as_hi, as_lo;     // [T][FFs] shared expert's
    size_t d;                // [pairs][H] fp32: per-pair down projection
    size_t ds;               // [T][H] fp32: shared expert's down projection
    size_t tile_cnt;         // [tiles] arrival counters of the combine
    size_t total;
};

// Workspace layout for the matrix-core path (T > kSmallT), byte offsets.
struct LargeLayout {
    size_t ids, w, counts, offsets, perm, inv, tiles, ntiles;
    size_t a;                // [pairs][FF] bf16 hi/lo interleaved in 2 planes
    size_t as;               // [T][FFs] shared
    size_t ypair;            // [pairs][H] fp32
    size_t ys;               // [T][H] fp32 shared output
    size_t total;
};

struct GemvShape {
    int H, FF, FFs, qtype;
    float z;
    int tile_rows_gu;   // rows of FF per gate/up workgroup
    int tile_rows_dn;   // rows of H per down workgroup
    int tiles_gu, tiles_gu_s, tiles_dn;
};

SmallLayout small_layout(int T, int k, int H, int FF, int FFs, int qtype);
LargeLayout large_layout(int T, int k, int E, int H, int FF, int FFs, int qtype);
GemvShape gemv_shape(int H, int FF, int FFs, int qtype, float z);

// Launchers (return hipError_t of the launch).
hipError_t launch_route_topk(const float* logits, int T, int E, int k, int renorm, int* ids, float* w,
                             hipStream_t s);
hipError_t launch_route_bucket_small(const float* logits, int T, int E, int k, int renorm, int identity,
                                     int* ids, float* w, const SmallLayout& L, char* ws, int n_counters,
                                     hipStream_t s);
hipError_t launch_gemv_layer(const GemvShape& g, const void* const* table, const void* single_blob,
                             const void* shared, const void* x, int x_dtype, int T, int k, int max_groups,
                             const int* ids, const float* w, const SmallLayout& L, char* ws, float* y,
                             hipStream_t s);
hipError_t launch_dequant(const void* blob, int qtype, float z, int rows, int cols, size_t plane_offset,
                          float* out, hipStream_t s);

}  // namespace moe
