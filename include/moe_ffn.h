/*
 * moe_ffn.h -- C ABI of the routed low-bit expert FFN library for MI355X (gfx950).
 *
 * One routed mixture-of-experts FFN layer per call: top-k routing over the
 * router logits, the selected experts' block-quantized gate/up/down weights
 * dequantized inside the kernels, SwiGLU, and the router-weighted combine plus
 * an optional shared expert.
 *
 * Sources of what is computed (page titles; section names in quotes):
 *   Krasis white paper, 5.3 "Per-token routed expert execution": route, select
 *     top-k ids and weights, look experts up in a flat device pointer table,
 *     run the expert projections, apply the activation, reduce the weighted
 *     expert outputs.  7.1: the layer output is the router-weighted sum.
 *   "Strata in the source: one verify window, three workers and a cache that
 *     learns", "The byte budget, in code": 64 weights per fp16 scale in 16
 *     bytes of 2-bit codes; gate, up and down per expert.  "The CPU kernels":
 *     the code bit order.  "The plan: three destinations per expert": a verify
 *     window's routed ids are de-duplicated so an expert chosen by several
 *     tokens is read once.
 *   kairos-engine README, "The MoE forward": top-k over the logits, experts
 *     processed expert-major over buckets of tokens, shared expert summed with
 *     the routed ones.  "Prefill and decode are different machines": fused
 *     dequant GEMV for a few tokens, dequant then matrix-core GEMM for many.
 *
 * Conventions for every entry point:
 *   - Every data pointer is a DEVICE pointer owned by the caller; the library
 *     keeps no reference after the call returns and allocates no device memory.
 *   - `stream` is a hipStream_t passed as void* (NULL = the null stream); all
 *     work is enqueued on it and the call returns without synchronising.
 *   - Shapes and pointers are checked on the host before anything is enqueued;
 *     on failure a non-OK status is returned, nothing is launched and
 *     moe_last_error() describes the problem.  A launch failure returns
 *     MOE_ERR_DEVICE.  Faults inside kernels surface at the caller's next
 *     synchronisation.
 *   - Results are deterministic: the same inputs give bitwise identical outputs
 *     from run to run (no atomics on any value path).  On the decode/verify path
 *     (T <= 8) a token's output is also bitwise independent of the other tokens
 *     in the batch.
 *   - Concurrency.  The decode and verify-window kernels rely on all of their
 *     workgroups being resident on the GPU at once (their work items wait on
 *     each other).  Layer calls on one device must therefore not overlap each
 *     other, whatever their workspaces, nor other long-running kernels on
 *     other streams: order them on one stream, or with events.  Calls on
 *     different devices are independent.  The library's host state (launch
 *     caches) is per device and thread-safe.
 *   - Failures inside a call.  Every wait inside a kernel is bounded.  A wait
 *     that gives up sets a cause bit in the workspace's error word and the
 *     output rows it served are NaN.  While the word is set, every later layer
 *     call on that workspace writes NaN into all of its output rows and does
 *     nothing else, so stale shared state can never give a finite wrong
 *     result.  moe_workspace_check reports and clears it.
 *   - Workspace: a device buffer of at least the *_workspace_bytes size,
 *     256-byte aligned, ZERO-FILLED ONCE after allocation (and after a failure
 *     that moe_workspace_check reported, which zero-fills it itself).  Its leading bytes
 *     hold the decode kernel's state (synchronisation words and the hand-off
 *     buffer between its gate/up and down stages), which every call returns
 *     to zero; the rest is scratch.  One workspace may serve calls of any T,
 *     decode and prefill alike (size it for the largest).
 */
#ifndef MOE_FFN_H
#define MOE_FFN_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    MOE_OK = 0,
    MOE_ERR_INVALID_ARG = 1,   /* null pointer, bad shape, k out of range, ... */
    MOE_ERR_UNSUPPORTED = 2,   /* valid request outside what the kernels cover */
    MOE_ERR_WORKSPACE = 3,     /* ws_bytes smaller than the *_workspace_bytes size */
    MOE_ERR_DEVICE = 4         /* a HIP call or kernel launch failed */
} moe_status;

/* Block formats.  Every block is 16 bytes of codes followed (in the scales
 * plane) by one IEEE fp16 scale; weight = scale * (code - zero_point).
 *   MOE_Q2_64: 64 two-bit codes; code i in byte i/4 at bit 2*(i%4)
 *              (Strata "The byte budget, in code" and "The CPU kernels").
 *   MOE_Q4_32: 32 four-bit codes; code i in byte i/2, low nibble for even i. */
typedef enum { MOE_Q2_64 = 1, MOE_Q4_32 = 2 } moe_qtype;

/* Activation dtypes: fp32, or bfloat16 stored as raw 16-bit words. */
typedef enum { MOE_F32 = 0, MOE_BF16 = 1 } moe_dtype;

/* Gated activation of an expert (routed and shared alike):
 *   MOE_ACT_SWIGLU     a = silu(gate x) * (up x), silu(v) = v / (1 + e^-v);
 *   MOE_ACT_GEGLU_TANH a = gelu(gate x) * (up x) with the tanh form
 *                      gelu(v) = v/2 (1 + tanh(sqrt(2/pi) (v + 0.044715 v^3)))
 *                      (kairos-engine README, "Decode, 2026-09-28/29": the
 *                      Gemma model's GELU is the tanh form). */
typedef enum { MOE_ACT_SWIGLU = 0, MOE_ACT_GEGLU_TANH = 1 } moe_act;

typedef struct {
    int32_t hidden;      /* H: model width = input and output length */
    int32_t ff;          /* FF: expert intermediate width */
    int32_t qtype;       /* moe_qtype */
    float zero_point;    /* z: 1.5 (2-bit) / 7.5 (4-bit) in the measured shapes; 1.0 is the Strata mapping.
                            Must be a multiple of 0.5 in [-64, 64] (MOE_ERR_UNSUPPORTED otherwise): the
                            matrix-core path multiplies by 2(c - z), which is then an exact small integer */
    int32_t act;         /* moe_act */
} moe_expert_desc;

typedef struct {
    moe_expert_desc expert;  /* shape and format of every routed expert (and of the shared one, but ff) */
    int32_t n_experts;       /* E */
    int32_t top_k;           /* k, 1 <= k <= min(E, 32) */
    int32_t renormalize;     /* 1: softmax over the k selected logits; 0: full softmax over E, read at the selected */
    int32_t shared_ff;       /* FF of the always-on shared expert; 0 = none */
} moe_layer_desc;

/*
 * Expert blob layout (bytes).  gate [FF][H], up [FF][H], down [H][FF], in this
 * order; each matrix is quantized in blocks along its input dimension and
 * stored as a codes plane [rows][nblk][16] followed by a scales plane
 * [rows][nblk] of little-endian fp16.  Total = 3 * H * FF / qk * 18 bytes
 * (1,382,400 for H=2560, FF=640, 2-bit: "The byte budget, in code").
 * H and FF must be multiples of qk (64 for MOE_Q2_64, 32 for MOE_Q4_32).
 * Blobs should be 16-byte aligned; the planes then are too.
 */
size_t moe_expert_blob_bytes(const moe_expert_desc* desc);   /* 0 if desc is invalid */

/* Device workspace the calls below need for T tokens (bytes, 256-aligned
 * sub-buffers).  0 if the descriptor is invalid. */
size_t moe_expert_workspace_bytes(const moe_expert_desc* desc, int32_t T);
size_t moe_layer_workspace_bytes(const moe_layer_desc* desc, int32_t T);

/*
 * Top-k routing (Krasis 5.3; kairos "The MoE forward").
 *   logits  : [T][E] fp32, row-major.
 *   ids     : [T][k] int32 out -- the k largest logits of each token in rank
 *             order: logit descending, expert index ascending on ties
 *             (-0 and +0 are equal; a NaN logit ranks below every number).
 *   weights : [T][k] fp32 out -- renormalize=1: exp(l_j - l_0) / sum_{i<k}
 *             exp(l_i - l_0) (sums to 1); renormalize=0: the full softmax over
 *             all E logits at the selected experts.  An all -inf selection
 *             gets equal weights.
 * Limits: 1 <= E <= 1024, 1 <= k <= min(E, 32), T >= 0 (T = 0 is a no-op).
 */
moe_status moe_route_topk(const float* logits, int32_t T, int32_t E, int32_t k, int32_t renormalize,
                          int32_t* ids, float* weights, void* stream);

/*
 * One expert's SwiGLU FFN on T tokens: y[t] = W_down (silu(W_gate x[t]) * (W_up x[t])).
 *   blob : one expert blob (layout above).
 *   x    : [T][H] activations, dtype x_dtype (moe_dtype).
 *   y    : [T][H] fp32 out.
 *   ws   : device workspace of at least moe_expert_workspace_bytes(desc, T) bytes.
 * T <= 8 runs the dequant-fused GEMV path; larger T the matrix-core path.
 */
moe_status moe_expert_ffn(const moe_expert_desc* desc, const void* blob, const void* x, int32_t x_dtype,
                          int32_t T, float* y, void* ws, size_t ws_bytes, void* stream);

/*
 * One routed MoE FFN layer on T tokens.
 *   expert_table : device array of E device pointers, entry e = expert e's blob
 *                  (Krasis 5.3: a flat device pointer table lets captured graphs
 *                  follow changing expert addresses).  Entries are not checked
 *                  on the hot path; a null entry that gets selected is undefined
 *                  behaviour (use moe_validate_table to check a table).
 *   shared_blob  : the shared expert (ff = desc->shared_ff), NULL iff shared_ff == 0.
 *   x            : [T][H] activations (x_dtype); logits : [T][E] fp32.
 *   y            : [T][H] fp32 out: y[t] = shared(x[t]) + sum_j w[t][j] * expert_{ids[t][j]}(x[t]),
 *                  accumulated in that fixed order (shared first, then rank order).
 *   ids_out, w_out : optional [T][k] copies of the routing (NULL to skip).
 *   ws           : device workspace of at least moe_layer_workspace_bytes(desc, T) bytes.
 * T <= 8 (decode, verify windows) runs the GEMV path: routing, expert-major
 * de-duplicated buckets, dequant-fused gate/up + SwiGLU, down, combine.
 * Larger T (prefill) sorts token slots by expert and runs grouped matrix-core
 * GEMMs over ragged per-expert token counts; T above moe_max_tokens(desc)
 * returns MOE_ERR_UNSUPPORTED.
 */
moe_status moe_layer_forward(const moe_layer_desc* desc, const void* const* expert_table, const void* shared_blob,
                             const void* x, int32_t x_dtype, const float* logits, int32_t T, float* y,
                             int32_t* ids_out, float* w_out, void* ws, size_t ws_bytes, void* stream);

/*
 * Router front end (kairos-engine README, "The MoE forward": normalise, run the
 * router GEMM to get the logits, take the top-k; the router reads its input
 * through its own weightless norm, and its scale is per input dimension):
 *   logits[t][e] = sum_h W[e][h] x'[t][h],  x' = x, or x / sqrt(mean_h x^2 + eps)
 *   when norm = 1, then times in_scale[h] when in_scale is not NULL.
 * W is bf16 [E][H] (raw 16-bit words); products and sums in fp32.  For T <= 8
 * a token's logits are bitwise independent of the other tokens.
 */
typedef struct {
    const void* weight;      /* [E][H] bf16 router weights, device, 16-byte aligned */
    const float* in_scale;   /* [H] fp32 per-input-dim scale, device, 16-byte aligned; or NULL */
    int32_t norm;            /* 1: weightless RMS norm of x first; 0: none */
    float eps;               /* the norm's epsilon (>= 0) */
} moe_router;

/*
 * The router alone: logits [T][E] fp32 (device) from x [T][H] (x_dtype).
 * H must be a multiple of 32.  No workspace.
 */
moe_status moe_router_logits(const moe_router* router, int32_t E, int32_t H, const void* x, int32_t x_dtype,
                             int32_t T, float* logits, void* stream);

/*
 * Options of moe_layer_forward_ex; a NULL options pointer, or all fields NULL,
 * is moe_layer_forward.
 *   router     : the logits are computed from x by the router above, inside the
 *                call (one more launch before the layer's); `logits` must then be
 *                NULL.  They go to logits_out [T][E] if given, else to the
 *                workspace.
 *   down_scale : [E] fp32 per routed expert: expert e's output is
 *                down_scale[e] * (W_down a) (kairos-engine README, "The MoE
 *                forward": the down projection's scale is per expert).  The
 *                shared expert is not scaled.  In the combine the weight and the
 *                scale are multiplied first: (w_j * s_e) * (W_down a).
 *   ids_in, w_in: [T][k] routing supplied by the caller instead of logits (a
 *                fixed top-k shape: Krasis white paper 7.5, "Preserving the native
 *                execution shape").  A slot whose weight is exactly 0 (+0 or -0)
 *                is skipped: its expert is never read and its id may be anything
 *                (a dummy).  A nonzero weight on an id outside [0, E) is an error:
 *                the call's outputs are NaN and moe_workspace_check reports it
 *                (cause bit 2).  Weights are used as given (not renormalised).
 *                Exclusive with router; `logits` is ignored.
 * The activation is the descriptor's `act`.  All pointers are device pointers,
 * 4-byte aligned.
 */
typedef struct {
    const moe_router* router;
    float* logits_out;
    const float* down_scale;
    const int32_t* ids_in;
    const float* w_in;
} moe_layer_opts;

moe_status moe_layer_forward_ex(const moe_layer_desc* desc, const moe_layer_opts* opts,
                                const void* const* expert_table, const void* shared_blob, const void* x,
                                int32_t x_dtype, const float* logits, int32_t T, float* y, int32_t* ids_out,
                                float* w_out, void* ws, size_t ws_bytes, void* stream);

/*
 * Measurement variant of moe_layer_forward: the same checks and the same work,
 * plus caller-created HIP events (hipEvent_t passed as void*, timing enabled)
 * recorded on `stream` at the boundaries of the kernels the call launches:
 * events[0] before the first stage, events[i] after the i-th.  Boundaries
 * past n_events are not recorded.  *n_kernels (if not NULL) receives the
 * number of stages: 1 on the decode/verify path (the fused layer kernel); 6 on
 * the prefill path (routing, expert histogram, slot placement, gate/up +
 * SwiGLU, down, combine).  Each stage is one kernel except the expert
 * histogram (two launches: per-block counts, then the totals, offsets, tile
 * list and per-block bases) and slot placement (two: the placement, then the
 * activations' conversion to the matrix-core operand planes).  Events are not
 * owned by the library.
 * A failing hipEventRecord returns MOE_ERR_DEVICE after the work is enqueued.
 */
moe_status moe_layer_forward_timed(const moe_layer_desc* desc, const void* const* expert_table,
                                   const void* shared_blob, const void* x, int32_t x_dtype, const float* logits,
                                   int32_t T, float* y, int32_t* ids_out, float* w_out, void* ws, size_t ws_bytes,
                                   void* stream, void* const* events, int32_t n_events, int32_t* n_kernels);

/*
 * Debug: dequantize matrix m (0 gate [FF][H], 1 up [FF][H], 2 down [H][FF]) of
 * a blob to fp32 (exact: an fp16 scale times a small integer offset), row-major.
 */
moe_status moe_dequant_matrix(const moe_expert_desc* desc, const void* blob, int32_t m, float* out, void* stream);

/*
 * Debug: copy the device table to the host and check that its first E entries
 * are non-null.  Synchronises `stream`.  Returns MOE_ERR_INVALID_ARG naming the
 * first null entry.
 */
moe_status moe_validate_table(const void* const* expert_table, int32_t E, void* stream);

/*
 * moe_layer_forward for callers that cannot allocate device memory: code under
 * HIP graph capture, tight serving loops, harnesses that forbid hipMalloc.  The
 * same checks, kernels and results (bitwise) as moe_layer_forward for T <= 8,
 * but the workspace is a library-owned device array of 4 MiB per GPU (a
 * file-scope __device__ array, held until the process ends), so the caller
 * passes none.  Each call first clears the array's shared region with a fill
 * kernel (no memset node, so a captured graph replays it correctly) and calls
 * no hipMalloc, hipFree or allocating routine.
 *   T > 8 (the matrix-core path, whose workspace is far larger) returns
 *   MOE_ERR_UNSUPPORTED; a shape whose T = 8 workspace exceeds 4 MiB returns
 *   MOE_ERR_WORKSPACE (the Strata and Gemma decode shapes need about 1.2 MB).
 * Every call on a GPU shares that GPU's array: calls that overlap on one GPU
 * race (they must be ordered, as every layer call on a device must be).  A
 * failure shows as NaN outputs (the next call's clear resets the array).
 */
moe_status moe_layer_forward_noalloc(const moe_layer_desc* desc, const void* const* expert_table,
                                     const void* shared_blob, const void* x, int32_t x_dtype, const float* logits,
                                     int32_t T, float* y, int32_t* ids_out, float* w_out, void* stream);

/*
 * The largest T a layer call accepts for this descriptor (0 if it is
 * invalid): the matrix-core path addresses its activation planes [2][T][H] and
 * its SwiGLU planes [2][rows][max(FF, shared_ff)] (rows = T*k, plus T with a
 * shared expert) with 32-bit byte offsets, so
 *   T_max = min((2^32 - 4096) / (4 H), (2^32 - 4096) / (4 max(FF, shared_ff) (k + [shared_ff > 0]))).
 * For H 7168, FF 2048, k 8 this is 65,535.
 */
int64_t moe_max_tokens(const moe_layer_desc* desc);

/*
 * Reports and clears a failure of earlier layer calls on a workspace (see
 * "Failures inside a call" above).  Synchronises `stream`, reads the
 * workspace's error word and returns MOE_OK if it is clear.  Otherwise it
 * zero-fills the workspace's shared region (the part every call leaves zero),
 * synchronises again and returns MOE_ERR_DEVICE; moe_last_error() names the
 * cause bits (1: a bounded wait gave up; 2: a caller-supplied expert id outside
 * [0, E), whose slot was skipped).  `desc` is the descriptor the workspace
 * serves (it sizes the shared region).  Not for use inside graph capture.
 */
moe_status moe_workspace_check(const moe_layer_desc* desc, void* ws, size_t ws_bytes, void* stream);

/*
 * Debug and testing: the bound of every wait inside the layer kernels, in
 * polls (each a coherent load and a short sleep).  A negative value restores
 * the default (2^22).  0 makes every bounded wait give up at its first check,
 * whether or not it would have ended: every kernel still exits normally, and
 * the failure path (error word, NaN outputs, moe_workspace_check) can be tested
 * without a real stall.  Process-wide; takes effect at the next call.
 */
void moe_debug_set_wait_limit(int64_t polls);

const char* moe_status_str(moe_status s);
/* Detail of the last non-OK status returned on the calling thread. */
const char* moe_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* MOE_FFN_H */
