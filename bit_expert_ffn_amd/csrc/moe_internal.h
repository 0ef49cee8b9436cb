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
constexpr int kGemvThreads = 256;  // workgroup size of the GEMV kernels
constexpr int kMaxBlocksPerRow = 256;

// Bytes of one block: 16 code bytes + one fp16 scale.
constexpr int kBlockCodeBytes = 16;
constexpr int kBlockBytes = 18;

inline int codes_per_block(int qtype) { return qtype == 1 ? 64 : (qtype == 2 ? 32 : 0); }

// Error word of a workspace: the int kErrWord ints into the synchronisation
// area (the first word of its second 64-byte line), in every layout.  Kernels
// OR cause bits into it; moe_workspace_check reads it and returns the area to
// zero.  While it is non-zero, every layer call on the workspace writes NaN
// into its output rows and does no other work.
constexpr int kErrWord = 16;
constexpr int kErrTimeout = 1;     // a bounded wait gave up
constexpr int kErrBadId = 2;       // a caller-supplied expert id outside [0, E) (its slot was skipped)
// Polls of a bounded wait before it gives up (each poll sleeps about 64
// cycles after a coherent load); the debug override moe_debug_set_wait_limit
// replaces it, and a bound of 0 makes every wait give up at its first check.
constexpr long kDefaultWaitPolls = 1l << 22;
long wait_polls();

// Synchronisation area of the one-token decode kernel: 4 + groups + 16 lines
// of 64 bytes (flags, per-group counters, load counters), then kReadyReplicas
// replicas of the per-group ready flags, kReadyStride bytes apart.  The
// verify-window kernel lays out its own lines over the same area
// (window_sync_bytes).  The area must be zero before the first call on a
// workspace; every call leaves it zero again.
constexpr int kReadyReplicas = 16;
constexpr int kReadyStride = 4096;
__host__ __device__ inline size_t decode_sync_lines_bytes(int max_groups_total) { return (size_t)64 * (4 + max_groups_total + 16); }
__host__ __device__ inline size_t decode_sync_bytes(int max_groups_total) {
    const size_t lines = (decode_sync_lines_bytes(max_groups_total) + kReadyStride - 1) / kReadyStride * kReadyStride;
    return lines + (size_t)kReadyReplicas * kReadyStride;
}

// Workspace layout for the GEMV path (T <= kSmallT), byte offsets.
struct SmallLayout {
    // The first four regions sit at the same offsets for every T <= kSmallT
    // (sized for kSmallT tokens), and the matrix-core layout starts after
    // them, so that calls of any size can share one workspace: the sync
    // words, `a` and d, whose words are never 0 once written and are
    // returned to 0 by each call that wrote them.
    size_t sync;
    size_t a;                // [T*k][FF] SwiGLU output per (expert, token) pair, packed bf16 hi | lo << 16
    size_t as;               // [T][FFs] the shared expert's
    size_t d;                // [8k + 8][H] verify windows: down output per slot, then per token of the shared expert
    size_t ids, w;           // [T][k] routing when the caller passes no output
    size_t logits;           // [T][E] router output when the router runs inside the call
    size_t total;
};

// Workspace layout for the matrix-core path (T > kSmallT), byte offsets.
struct LargeLayout {
    size_t ids, w;           // [T][k] routing when the caller passes no output
    size_t counts, offsets;  // per expert
    size_t tiles, ntiles;    // row tiles: (expert, first sorted row, rows)
    size_t perm, inv;        // sorted row -> token; (token, slot) -> sorted row
    size_t bcount;           // [blocks of pairs][E] counts of the placement sort
    size_t xq, xe;           // [2][T][H] fp16 activation planes (hi, lo); [T] power-of-two exponents
    size_t a;                // [rows][FFmax] bf16 hi plane, then the lo plane
    size_t ypair;            // [rows][H] fp32 down projection per sorted row
    size_t logits;           // [T][E] router output when the router runs inside the call
    size_t max_tiles;
    size_t total;
};

// Options of a layer call beyond its descriptor (moe_layer_forward_ex).
struct LayerOpts {
    int act = 0;                       // 0 SwiGLU, 1 GeGLU (tanh GELU)
    const float* down_scale = nullptr; // [E] per routed expert, or none
    const int* ids_in = nullptr;       // [T][k] caller-supplied routing, or none (route from logits)
    const float* w_in = nullptr;       // [T][k]; a zero weight skips its slot
};

struct GemvShape {
    int H, FF, FFs, qtype;
    float z;
    int gu_passes, tile_rows_gu, tiles_gu, tiles_gu_s;
    int gu_pair;              // gate/up lanes take two adjacent block columns each
    int max_groups, shared_groups, n_gu;
    int tile_rows_dn, tiles_dn;
    int stage_words;          // `a` words each down workgroup stages in LDS (one token), else 0
    int x_off;                // one token: LDS word offset of the gate/up activation slices, else -1
    size_t lds_bytes;
    int grid;
};

// Verify windows (2 <= T <= kSmallT): work items of the window kernel (its
// grid is set at launch from the GPU's capacity).
struct WindowShape {
    int gu_passes, tiles_gu, tiles_gu_s;     // gate/up: passes per tile; tiles per routed / shared expert
    int dn_passes, chunk_rows, n_chunks;     // down: passes per routed item; H rows per chunk; chunks
    int sh_passes, sh_rows, sh_items;        // down of the shared expert: passes, rows and items per chunk
    int max_items;           // the larger of the gate/up and down item counts, at most
    int x_off, stage_words;
    size_t lds_bytes;
    int grid;
};
WindowShape window_shape(int H, int FF, int FFs, int qtype, int x_dtype, int T, int k);
size_t window_sync_bytes(int k, int n_chunks);

SmallLayout small_layout(int T, int k, int E, int H, int FF, int FFs, int qtype);
size_t small_fixed_bytes(int k, int H, int FF, int FFs, int qtype);   // sync + a + as + d: where every layout's own regions start
LargeLayout large_layout(int T, int k, int E, int H, int FF, int FFs, int qtype);
// n_cu: compute units of the device the call runs on (0: 256).
GemvShape gemv_shape(int H, int FF, int FFs, int qtype, float z, int T, int k, int n_cu);

// Caller-owned HIP events recorded on the launch stream at kernel boundaries
// (measurement entry point): boundary 0 before the first kernel, boundary i
// after the i-th.  Boundaries beyond n are counted but not recorded.
struct StageMarks {
    const hipEvent_t* ev = nullptr;
    int n = 0;
    int next = 0;
    hipError_t err = hipSuccess;
};

inline void stage_mark(StageMarks* m, hipStream_t s) {
    if (!m) return;
    if (m->next < m->n && m->err == hipSuccess) m->err = hipEventRecord(m->ev[m->next], s);
    ++m->next;
}

// Launchers (return hipError_t of the launch).
hipError_t launch_route_topk(const float* logits, int T, int E, int k, int renorm, int* ids, float* w,
                             hipStream_t s);
hipError_t launch_decode_layer(const GemvShape& g, const void* const* table, const void* single, const void* shared,
                               const void* x, int x_dtype, const float* logits, int T, int E, int k, int renorm,
                               int identity, const LayerOpts& o, int* ids_out, float* w_out, const SmallLayout& L,
                               char* ws, float* y, hipStream_t s, StageMarks* marks = nullptr);
hipError_t launch_window_layer(const WindowShape& g, const void* const* table, const void* single,
                               const void* shared, const void* x, int x_dtype, const float* logits, int T, int E,
                               int k, int renorm, int identity, const LayerOpts& o, int qtype, float z, int H, int FF,
                               int FFs, int* ids_out, float* w_out, const SmallLayout& L, char* ws, float* y,
                               hipStream_t s, StageMarks* marks = nullptr);
hipError_t launch_prefill_layer(const void* const* table, const void* single, const void* shared, int qtype, float z,
                                int H, int FF, int FFs, const void* x, int x_dtype, const float* logits, int T, int E,
                                int k, int renorm, int identity, const LayerOpts& o, int* ids_out, float* w_out,
                                const LargeLayout& L, char* ws, float* y, hipStream_t s, StageMarks* marks = nullptr);
// Router logits [T][E] = W_r x' (bf16 W_r [E][H]; x' = x, optionally through
// the weightless RMS norm and a per-input-dim scale): one launch (a GEMV for
// T <= kSmallT, a tiled GEMM above).
hipError_t launch_router(const void* wr, const float* in_scale, int norm, float eps, int E, int H, const void* x,
                         int x_dtype, int T, float* logits, hipStream_t s);
hipError_t launch_dequant(const void* blob, int qtype, float z, int rows, int cols, size_t plane_offset,
                          float* out, hipStream_t s);

}  // namespace moe
