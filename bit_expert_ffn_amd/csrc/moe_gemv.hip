// Fused one-token decode layer (see moe_gemv_common.h for the GEMV scheme).
#include <algorithm>
#include <mutex>
#include <set>

#include "moe_gemv_common.h"

namespace moe {
// ---------------------------------------------------------------------------------------------
// Fused one-token decode layer: one kernel per layer.
//
// Every workgroup first recomputes the routing of the token from its logits
// (a few KB, served from L2); the token's k slots are the groups, in rank
// order.  Workgroups [0, n_gu) run gate/up + SwiGLU tiles and publish their
// rows of `a` as never-zero packed words with agent-coherent stores; each
// tile then bumps its group's counter, and the tile that completes a group
// raises the group's ready flag in each of n_ready replicas (4 KB apart).
// Workgroups [n_gu, n_gu + tiles_dn) own a tile of H output rows: they issue
// the loads of their down-projection weights for every selected expert once
// the first gate/up tile is done, wait until every group's flag in their
// replica (tile % n_ready) is raised, copy `a` into LDS (reading again any word
// still 0), and finish the down projection and the weighted combine for their
// rows.  Polling one replica per 16 workgroups keeps the pollers off the lines
// that the counters and flags are written on.  Workgroups are dispatched in
// index order, so every gate/up workgroup is running or done before any down
// workgroup starts waiting; the wait is bounded anyway and flags an error if
// the bound is ever reached.  The last workgroup waits until every down
// workgroup holds its `a` and returns the counters, flags and `a` words to
// zero for the next call.
//
// Failures.  A bounded wait that gives up ORs kErrTimeout into the
// workspace's error word, and the down workgroup it belongs to writes NaN
// into its output rows.  The down and janitor workgroups read the error word
// before their first wait (not earlier: an agent-coherent load in flight
// holds every barrier of its workgroup): if a failure that
// moe_workspace_check has not cleared is there, they write NaN rows and do
// nothing else, so no wait runs on stale shared state.
// ---------------------------------------------------------------------------------------------
constexpr size_t kDecodeLdsBudget = 112 * 1024;   // dynamic LDS of the fused decode kernel
constexpr size_t kDecodeStaticLds = 6 * 1024;      // its static LDS (the routing state), rounded up
constexpr int kMaxRowsDn = 12;               // H rows per down workgroup
// Down rows one thread prefetches: as many as the registers hold without
// spilling (2-bit blocks decode into more registers than 4-bit ones).
__host__ __device__ constexpr int rows_per_thread(int qtype) { return qtype == 1 ? 6 : 10; }
constexpr int kLoadFan = 16;                 // counters of the down workgroups done loading `a`

struct DecodeParams {
    const void* const* table;
    const uint8_t* single;       // one expert's blob when table == nullptr (moe_expert_ffn)
    const uint8_t* shared;
    const void* x;               // [T][H] bf16 or fp32
    const float* logits;         // [T][E]
    int T, E, k, renorm, identity;
    int H, FF, FFs;
    float z;
    int act;                     // gate activation (kActSilu / kActGeluTanh)
    const float* down_scale;     // [E] per routed expert, or null
    const int* ids_in;           // [T][k] caller-supplied routing, or null
    const float* w_in;           // [T][k]
    int* ids_out;                // [T][k] or null
    float* w_out;                // [T][k] or null
    uint32_t* a;                 // [T*k][FF] packed bf16 hi | lo << 16, agent-coherent
    uint32_t* as;                // [T][FFs] the same for the shared expert
    float* y;                    // [T][H]
    int* sync;                   // DecodeSync words, see sync_* below
    int* err;                    // the workspace's error word (sync + kErrWord)
    long polls;                  // bound of every wait
    int gu_passes, tiles_gu, tiles_gu_s, max_groups, shared_groups, n_gu;
    int dn_rows, tiles_dn;
    int n_ready;                 // ready-flag replicas in use: min(kReadyReplicas, tiles_dn)
    int stage_words;             // `a` words each down workgroup copies to LDS first (one token), else 0
    int x_off;                   // one token: LDS word offset of the arranged activation slices (gate/up), else -1
};

// Word offsets inside the synchronisation area (ints; 16 ints = one 64-byte line).
__device__ __forceinline__ int* sync_group(int* s, int g) { return s + 16 * (4 + g); }
// Count i of the down workgroups done loading `a` (workgroup tile counts in i = tile % kLoadFan).
__device__ __forceinline__ int* sync_loaded(int* s, int i, int n_ctr) { return s + 16 * (4 + n_ctr + i); }
// Ready flag of group g in replica r (replicas kReadyStride bytes apart, after the lines above).
__device__ __forceinline__ int* sync_ready(int* s, int r, int g, int n_ctr) {
    const size_t lines = (decode_sync_lines_bytes(n_ctr) + kReadyStride - 1) / kReadyStride * kReadyStride;
    return s + (lines + (size_t)r * kReadyStride) / 4 + g;
}

// floor(x / d) for 0 <= x < 2^20 and 1 <= d < 2^24, in single precision (the
// decode shapes stay below both: at most 33 groups of 2^14 tiles).
// (x + 0.5) / d lies at least 0.5 / d from every integer; the reciprocal (1 ulp)
// and the rounded product leave a relative error below 2^-22, so the error
// stays below (x + 0.5) / d * 2^-22 < 0.5 / d and the truncation is exact.
// A few instructions where an integer division takes about twenty.
__device__ __forceinline__ int small_div(int x, int d) {
    return (int)(((float)x + 0.5f) * __builtin_amdgcn_rcpf((float)d));
}

struct RouteLDS {
    int id[kMaxK];
    float w[kMaxK];
    int pair_tok[kMaxK], pair_exp[kMaxK], slot_pair[kMaxK];
    int group_first[kMaxK], group_n[kMaxK], group_of_pair[kMaxK];
    int slot_src[kMaxK];   // slot j -> group * NT + token-in-group of its pair; -1: a skipped slot
    alignas(16) uint64_t topk[kGemvThreads / 64][128];   // each wave's top-k scratch
    int n_groups;
    int fail;              // this workgroup's output is NaN: an earlier failure, or one of its waits gave up
    int bad;               // a caller-supplied id outside [0, E) with a nonzero weight
};

// Routing of the token: its k slots are its pairs and groups, in rank order
// (group numbering changes no arithmetic).  With caller-supplied routing
// (Krasis white paper 7.5: a fixed top-k shape in which an omitted route is
// a zero-weight slot), the slots of nonzero weight become the groups, in slot
// order; a zero-weight slot has no group and its expert is never read.  A
// nonzero weight on an id outside [0, E) flags kErrBadId and fails the call.
// want_w false: the slot weights are not computed (R.w is left unset), for a
// workgroup that never reads them.
__device__ void route_and_bucket(const DecodeParams& p, RouteLDS& R, bool want_w) {
    const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
    const int k = p.k;
    if (tid == 0) R.fail = 0;
    if (wv == 0 && p.ids_in) {
        const int id = lane < k ? p.ids_in[lane] : 0;
        const float wt = lane < k ? p.w_in[lane] : 0.f;
        const bool on = lane < k && wt != 0.f;
        const bool bad = on && (id < 0 || id >= p.E);
        if (bad) flag_error(p.err, kErrBadId);
        const uint64_t live = __ballot(on && !bad);
        const int pos = lanes_below(live);
        if (lane < k) {
            R.id[lane] = id;
            R.w[lane] = wt;
            R.slot_src[lane] = (on && !bad) ? pos : -1;
        }
        if (on && !bad) {
            R.slot_pair[pos] = pos;
            R.pair_tok[pos] = 0;
            R.pair_exp[pos] = id;
            R.group_first[pos] = pos;
            R.group_n[pos] = 1;
            R.group_of_pair[pos] = pos;
        }
        const bool any_bad = __ballot(bad) != 0;   // every lane votes
        if (lane == 0) {
            R.n_groups = __popcll(live);
            R.bad = any_bad;
        }
    } else if (wv == 0) {
        int id = 0;
        float wt = 1.f;
        if (!p.identity) wave_topk(p.logits, p.E, k, p.renorm, lane, R.topk[0], &id, &wt, want_w);
        if (lane < k) {
            R.id[lane] = id;
            R.w[lane] = wt;
            R.slot_pair[lane] = lane;
            R.pair_tok[lane] = 0;
            R.pair_exp[lane] = id;
            R.group_first[lane] = lane;
            R.group_n[lane] = 1;
            R.group_of_pair[lane] = lane;
            R.slot_src[lane] = lane;
        }
        if (lane == 0) {
            R.n_groups = k;
            R.bad = 0;
        }
    }
    __syncthreads();
}

// PAIR: each lane takes two adjacent block columns of its row (used where that
// puts more of the 256 lanes to work, e.g. 88 columns: 220 lanes against 176)
// and adds their two sums itself, in the order the lane pairs of the default
// mapping add them (even column first), so the partials are the same bits.
template <int QT, int NT, int NTERM, bool PAIR>
__device__ void gateup_role(const DecodeParams& p, RouteLDS& R, int item, float* lds) {
    constexpr int QK = QTraits<QT>::QK;
    const int tid = threadIdx.x;
    const uint8_t* blob;
    int rows, tile, ntok, grp, toks[NT], outrow[NT];
    uint32_t* out;
    if (item < p.max_groups * p.tiles_gu) {
        const int g = small_div(item, p.tiles_gu);
        tile = item - g * p.tiles_gu;
        if (g >= R.n_groups) return;
        grp = g;
        const int first = R.group_first[g];
        ntok = R.group_n[g];
        blob = p.table ? table_blob(p.table, R.pair_exp[first]) : p.single;
        rows = p.FF;
#pragma unroll
        for (int t = 0; t < NT; ++t) {
            toks[t] = R.pair_tok[first + (t < ntok ? t : 0)];
            outrow[t] = first + t;
        }
        out = p.a;
    } else {
        const int i2 = item - p.max_groups * p.tiles_gu;
        const int sg = small_div(i2, p.tiles_gu_s);
        tile = i2 - sg * p.tiles_gu_s;
        grp = p.max_groups + sg;
        blob = p.shared;
        rows = p.FFs;
        ntok = min(NT, p.T - sg * NT);
#pragma unroll
        for (int t = 0; t < NT; ++t) {
            toks[t] = sg * NT + (t < ntok ? t : 0);
            outrow[t] = sg * NT + t;
        }
        out = p.as;
    }

    const int nblk = p.H / QK;
    constexpr int BPL = PAIR ? 2 : 1;   // block columns per lane
    const int cols = nblk / BPL;
    const int P = small_div(kGemvThreads, cols);
    const bool active = tid < P * cols;
    const int rq = small_div(tid, cols);
    const int rp = active ? rq : 0, lc = active ? tid - rq * cols : 0;
    const int b = lc * BPL;             // the lane's (first) block column
    const int Rr = P * p.gu_passes;
    const int f0 = tile * Rr;
    const size_t plane = (size_t)rows * nblk;
    const uint8_t* gcode = blob;
    const uint8_t* gscale = blob + plane * 16;
    const uint8_t* ucode = blob + plane * 18;
    const uint8_t* uscale = ucode + plane * 16;

    // Loads of every pass first, from clamped rows (the last tile's overhang
    // re-reads its last row), so that all of them are in flight at once; the
    // pass count is uniform across the workgroup.
    constexpr int MP = PAIR ? kMaxPassPair : kMaxPass;
    uint4 cg[MP][BPL], cu[MP][BPL];
    uint16_t sg_[MP][BPL], su_[MP][BPL];
#pragma unroll
    for (int m = 0; m < MP; ++m) {
        if (m < p.gu_passes) {
            const int f = min(f0 + m * P + rp, rows - 1);
            const size_t blk = (size_t)f * nblk + b;
#pragma unroll
            for (int j = 0; j < BPL; ++j) {
                if (out == p.as) {   // the shared expert: read every call
                    cg[m][j] = ldg_u4(gcode + (blk + j) * 16);
                    cu[m][j] = ldg_u4(ucode + (blk + j) * 16);
                } else {
                    cg[m][j] = ldg_u4_nt(gcode + (blk + j) * 16);
                    cu[m][j] = ldg_u4_nt(ucode + (blk + j) * 16);
                }
                sg_[m][j] = ldg_u16(gscale + (blk + j) * 2);
                su_[m][j] = ldg_u16(uscale + (blk + j) * 2);
            }
        }
    }
    XSlice<QT, NTERM> xs[BPL][NT];
#pragma unroll
    for (int j = 0; j < BPL; ++j) {
        if (NT == 1 && p.x_off >= 0) {   // arranged while the routing ran
            slice_from_lds<QT, NTERM>(xs[j][0], reinterpret_cast<const uint32_t*>(lds) + p.x_off +
                                                    (b + j) * SliceWords<QT, NTERM>::N);
        } else {
#pragma unroll
            for (int t = 0; t < NT; ++t) {
                if constexpr (NTERM == 1)
                    load_slice_bf16<QT, 1>(xs[j][t], (const uint16_t*)p.x + (size_t)toks[t] * p.H + (b + j) * QK,
                                           nullptr, p.z);
                else
                    load_slice_f32<QT>(xs[j][t], (const float*)p.x + (size_t)toks[t] * p.H + (b + j) * QK, p.z);
            }
        }
    }
    // Partials part[((mat * Rr + rr) * NT + t) * ncp + col]: a row's columns
    // are contiguous, padded to a multiple of 4.  With an even count of block
    // columns, lanes 2i and 2i + 1 (columns b and b + 1 of one row) add their
    // partials first, and the row has nblk / 2 columns.
    const bool pairs = (nblk & 1) == 0;
    const int ncol = pairs ? nblk / 2 : nblk;
    const int ncp = (ncol + 3) & ~3;
    const int col = pairs ? b >> 1 : b;
#pragma unroll
    for (int m = 0; m < MP; ++m) {
        const int f = f0 + m * P + rp;
        if (m < p.gu_passes && active && f < rows) {
            float og[NT], ou[NT];
            block_dot_pair<QT, NTERM, NT>(cg[m][0], scale_at_use(sg_[m][0]), cu[m][0], scale_at_use(su_[m][0]), xs[0],
                                          ntok, og, ou);
            if constexpr (PAIR) {
                float og1[NT], ou1[NT];
                block_dot_pair<QT, NTERM, NT>(cg[m][BPL - 1], scale_at_use(sg_[m][BPL - 1]), cu[m][BPL - 1],
                                              scale_at_use(su_[m][BPL - 1]), xs[BPL - 1], ntok, og1, ou1);
#pragma unroll
                for (int t = 0; t < NT; ++t) {
                    og[t] = og[t] + og1[t];
                    ou[t] = ou[t] + ou1[t];
                }
            } else if (pairs) {
#pragma unroll
                for (int t = 0; t < NT; ++t) {
                    og[t] += dpp_xor1_f32(og[t]);
                    ou[t] += dpp_xor1_f32(ou[t]);
                }
            }
            const int rr = m * P + rp;
            if (PAIR || !pairs || (b & 1) == 0) {
#pragma unroll
                for (int t = 0; t < NT; ++t) {
                    lds[((0 * Rr + rr) * NT + t) * ncp + col] = og[t];
                    lds[((1 * Rr + rr) * NT + t) * ncp + col] = ou[t];
                }
            }
        }
    }
    __syncthreads();
    // One thread per (row, token): both row sums, SwiGLU, the store; waves
    // 1-3 take the rows when they suffice, so that the count below (wave 0)
    // waits for no store of its own.
    const int off = Rr * NT <= kGemvThreads - 64 ? 64 : 0;
    for (int i = tid - off; i >= 0 && i < Rr * NT; i += kGemvThreads) {
        const int rr = i / NT, t = i - rr * NT;
        const int f = f0 + rr;
        if (f >= rows || t >= ntok) continue;
        const float g = sum_columns4(lds + ((0 * Rr + rr) * NT + t) * ncp, ncol);
        const float u = sum_columns4(lds + ((1 * Rr + rr) * NT + t) * ncp, ncol);
        const float a = act_gate(g, p.act) * u;
        __hip_atomic_store(out + (size_t)outrow[t] * rows + f, pack_a(a), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
    // Every store above has been issued, not necessarily completed (the
    // barrier does not wait for them): a flag raised after this count can be
    // seen before a word has landed.  Readers check each word (see pack_a)
    // and read again one still 0, so that costs a reload, not a wrong value.
    lds_barrier();
    // Count this tile; the tile that completes its group raises the group's
    // ready flag in every replica (down workgroups each poll one replica).
    if (tid < 64) {
        int old = 0;
        if (tid == 0)
            old = __hip_atomic_fetch_add(sync_group(p.sync, grp), 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        old = __builtin_amdgcn_readfirstlane(old);
        const int need = grp < p.max_groups ? p.tiles_gu : p.tiles_gu_s;
        const int n_ctr = p.max_groups + p.shared_groups;
        if (old == need - 1 && tid < p.n_ready)
            __hip_atomic_store(sync_ready(p.sync, tid, grp, n_ctr), 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        // The first tile of each group to finish also counts the group in the
        // prefetch hint (slot n_ctr of every replica): from the first count on,
        // the down weights may be loaded.  The janitor clears the hint only
        // once it counts every group, so no count lands after the clear.
        if (old == 0 && tid < p.n_ready)
            __hip_atomic_fetch_add(sync_ready(p.sync, tid, n_ctr, n_ctr), 1, __ATOMIC_RELAXED,
                                   __HIP_MEMORY_SCOPE_AGENT);
    }
}

// One token: the down workgroup copies every `a` word it reads (the routed
// rows 0..ng-1, then the shared row) into LDS once, with LDS DMA (no
// registers held), instead of each thread loading its own slices (which would
// read the same words several times).  The 16-byte chunks of a slice of QK
// words are stored in XOR-swizzled order, chunk v of slice s at position
// v ^ (s % CPS), so that the slice reads of a wave spread over every LDS bank.
// Each thread then checks the chunks its lane brought in and reads again any
// with a word still 0.
constexpr int kStagePasses = 8;                             // 16-byte chunks per thread
constexpr int kStageMaxWords = kStagePasses * kGemvThreads * 4;

__host__ __device__ constexpr int stage_bytes(int words) {   // whole passes of 256 chunks
    return (words / 4 + kGemvThreads - 1) / kGemvThreads * kGemvThreads * 16;
}

template <int QK>
__device__ __forceinline__ uint32_t stage_src_off(int q, int routed_words, uint32_t as_off) {
    constexpr int CPS = QK / 4;
    const int sl = q / CPS, v = (q % CPS) ^ (sl % CPS);
    const int wd = sl * QK + 4 * v;
    return wd < routed_words ? 4u * (uint32_t)wd : as_off + 4u * (uint32_t)(wd - routed_words);
}

// Copies this call's `a` words: routed_words (the routed groups' rows) then
// the shared expert's row; p.stage_words sizes the largest call (every slot a
// group), and with caller-supplied routing fewer slots may have groups.
template <int QK>
__device__ __forceinline__ void stage_a(const DecodeParams& p, __amdgpu_buffer_rsrc_t rsrc, const uint8_t* a_base,
                                        uint32_t as_off, int routed_words, uint8_t* dst, int* fail) {
    typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
    const int tid = threadIdx.x, wv = tid >> 6;
    int lane = tid & 63;
    // The addresses below are computed here, not hoisted to the start of the
    // caller (where holding them would spill registers).
    asm volatile("" : "+v"(lane));
    const int n_chunks = (routed_words + (p.shared ? p.T * p.FFs : 0)) / 4;
    // Pass j of wave wv fills LDS chunks [64 (4 j + wv), +64): lane i the i-th.
    // Positions past the last chunk (inside the last pass) take a copy of it.
#pragma unroll
    for (int j = 0; j < kStagePasses; ++j) {
        const int q0 = 64 * (4 * j + wv);
        if (q0 < n_chunks) {
            const int q = min(q0 + lane, n_chunks - 1);
            load_lds16_sc1(a_base + stage_src_off<QK>(q, routed_words, as_off), dst + 16 * q0);
        }
    }
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    // Check every chunk this lane brought in (one LDS read each, all issued
    // together); the rare chunk with a word still 0 is read again.
    uint32_t m = 0xFFFFFFFFu;
#pragma unroll
    for (int j = 0; j < kStagePasses; ++j) {
        const u32x4 v = *reinterpret_cast<const u32x4*>(dst + 16 * min(64 * (4 * j + wv) + lane, n_chunks - 1));
        m = min(m, min(min(v[0], v[1]), min(v[2], v[3])));
    }
    if (m == 0u) {
        for (int j = 0; j < kStagePasses; ++j) {
            const int q = 64 * (4 * j + wv) + lane;
            if (q >= n_chunks) break;
            u32x4* slot = reinterpret_cast<u32x4*>(dst + 16 * q);
            u32x4 v = *slot;
            long n = 0;
            while (p.polls == 0 || min(min(v[0], v[1]), min(v[2], v[3])) == 0u) {
                if (++n > p.polls) {   // a bound of 0 gives up at once
                    flag_error(p.err, kErrTimeout);
                    *fail = 1;
                    break;
                }
                __builtin_amdgcn_s_sleep(1);
                v = __builtin_amdgcn_raw_buffer_load_b128(rsrc, (int)stage_src_off<QK>(q, routed_words, as_off), 0,
                                                          kCpolSc1);
            }
            *slot = v;
        }
    }
}

template <int QT, int NT>
__device__ void down_role(const DecodeParams& p, RouteLDS& R, int tile, float* lds) {
    constexpr int QK = QTraits<QT>::QK;
    const int tid = threadIdx.x;
    const int h0 = tile * p.dn_rows;
    const int nrows = min(p.dn_rows, p.H - h0);
    const int nb_r = p.FF / QK;
    const int nb_s = p.FFs / QK;
    const int ng = R.n_groups;
    const int n_units = ng * nb_r + p.shared_groups * nb_s;
    // Combine weight of slot j = tid % JS (the lane that adds slot j's term
    // below): its routing weight times its expert's down scale, if any.
    const int JS = p.k <= 16 ? 16 : 32;
    float cw = 0.f;
    {
        const int j = tid % JS;
        if (j < p.k && R.slot_src[j] >= 0)
            cw = R.w[j] * (p.down_scale ? p.down_scale[R.id[j]] : 1.f);
    }
    if (n_units == 0) {
        // Every slot skipped and no shared expert: y = 0.  Still counted as
        // loaded, which the janitor waits for.
        if (tid == 0) atomic_add_detached(sync_loaded(p.sync, tile % kLoadFan, p.max_groups + p.shared_groups), 1);
        const bool failed = load_error(p.err) != 0;   // an unchecked earlier failure
        for (int i = tid; i < p.T * nrows; i += kGemvThreads)
            p.y[(size_t)(i / nrows) * p.H + h0 + i % nrows] = failed ? __uint_as_float(0x7FC00000u) : 0.f;
        return;
    }
    // Units (group, block column); with few units, S threads split a unit's rows.
    int S = kGemvThreads / n_units;
    S = S < 1 ? 1 : (S > nrows ? nrows : S);
    const int per_round = kGemvThreads / S;
    const size_t gu_r = (size_t)2 * p.FF * (p.H / QK) * 18, gu_s = (size_t)2 * p.FFs * (p.H / QK) * 18;

    // One buffer resource over `a` and the shared expert's rows after it.
    const uint32_t as_off = (uint32_t)((const char*)p.as - (const char*)p.a);
    const uint32_t a_bytes = as_off + (uint32_t)((size_t)p.T * p.FFs * 4);
    const __amdgpu_buffer_rsrc_t a_rsrc = __builtin_amdgcn_make_buffer_rsrc((void*)p.a, 0, (int)a_bytes, kRsrcWord3);

    // The down weights are prefetched only once a first gate/up tile is done:
    // until then the gate/up weight loads, which are on the critical path, have
    // the memory system to themselves.
    {
        const int rep = tile % p.n_ready;
        const int n_ctr = p.max_groups + p.shared_groups;
        const int* hint = sync_ready(p.sync, rep, n_ctr, n_ctr);
        if (!bounded_wait([&]() __attribute__((always_inline)) { return __hip_atomic_load(hint, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) != 0; },
                          p.polls, p.err))
            R.fail = 1;
    }

    // Partials part[((group * dn_rows + r) * NT + t) * nbp + b]: a (group, row,
    // token)'s block columns are contiguous, padded to a multiple of 4.  Routed
    // groups first, then shared groups from sh_off on.
    const int D = p.dn_rows * NT;
    const int nbp_r = (nb_r + 3) & ~3, nbp_s = (nb_s + 3) & ~3;
    const int sh_off = ng * D * nbp_r;
    float* part = lds + (p.stage_words ? stage_bytes(p.stage_words) / 4 : 0);   // after the staged `a`, if any
    bool waited = false;
    for (int u0 = 0; u0 < n_units; u0 += per_round) {
        const int uu = u0 + tid / S, rs = tid - (tid / S) * S;
        const bool act = (tid / S) < per_round && uu < n_units;
        const int u = act ? uu : 0;
        int g, b, K, nb, ntok;
        const uint8_t* dcode;
        if (u < ng * nb_r) {
            g = u / nb_r;
            b = u - g * nb_r;
            K = p.FF;
            nb = nb_r;
            const int first = R.group_first[g];
            ntok = R.group_n[g];
            dcode = (p.table ? table_blob(p.table, R.pair_exp[first]) : p.single) + gu_r;
        } else {
            const int us = u - ng * nb_r;
            g = us / nb_s;            // shared group
            b = us - g * nb_s;
            K = p.FFs;
            nb = nb_s;
            ntok = min(NT, p.T - g * NT);
            dcode = p.shared + gu_s;
        }
        const uint8_t* dscale = dcode + (size_t)p.H * nb * 16;
        constexpr int RPT = rows_per_thread(QT);
        uint4 c[RPT];
        uint16_t sc[RPT];
#pragma unroll
        for (int i = 0; i < RPT; ++i) {
            const int r = min(rs + i * S, nrows - 1);
            const size_t blk = (size_t)(h0 + r) * nb + b;
            c[i] = u >= ng * nb_r ? ldg_u4(dcode + blk * 16) : ldg_u4_nt(dcode + blk * 16);
            sc[i] = ldg_u16(dscale + blk * 2);
        }
        if (!waited) {
            // The error word, loaded behind this unit's weights (whose arrival
            // the first poll below waits for anyway): an unchecked earlier
            // failure means NaN rows, and no wait on the stale state.
            if (load_error(p.err) != 0) {
                for (int i = tid; i < p.T * nrows; i += kGemvThreads)
                    p.y[(size_t)(i / nrows) * p.H + h0 + i % nrows] = __uint_as_float(0x7FC00000u);
                return;
            }
            // Thread g of the first wave watches group g's ready flag (routed
            // groups, then shared groups) in this workgroup's replica; the wave
            // continues when all are raised.
            if (tid < 64) {
                const int rep = tile % p.n_ready;
                const int n_ctr = p.max_groups + p.shared_groups;
                for (int g0 = 0; g0 < ng + p.shared_groups; g0 += 64) {
                    const int gi = g0 + tid;
                    const bool mine = gi < ng + p.shared_groups;
                    const int ctr = gi < ng ? gi : p.max_groups + (gi - ng);
                    const bool ok = bounded_wait(
                        [&]() __attribute__((always_inline)) {
                            const bool ready = !mine || __hip_atomic_load(sync_ready(p.sync, rep, ctr, n_ctr),
                                                                          __ATOMIC_RELAXED,
                                                                          __HIP_MEMORY_SCOPE_AGENT) != 0;
                            return (bool)__all(ready);
                        },
                        p.polls, p.err);
                    if (!ok) R.fail = 1;
                }
            }
            __syncthreads();
            waited = true;
            if (p.stage_words) {
                stage_a<QK>(p, a_rsrc, reinterpret_cast<const uint8_t*>(p.a), as_off, ng * p.FF,
                            reinterpret_cast<uint8_t*>(lds), &R.fail);
                // Every load has landed; saying so leaves the compiler no load
                // to wait for after the atomic below.
                __builtin_amdgcn_s_waitcnt(0);
                lds_barrier();
                // Every `a` word this workgroup reads is in LDS: count the
                // workgroup (without waiting for the atomic).
                if (tid == 0)
                    atomic_add_detached(sync_loaded(p.sync, tile % kLoadFan, p.max_groups + p.shared_groups), 1);
            }
        }
        XSlice<QT, 2> xs[NT];
        const bool sh = u >= ng * nb_r;
        if (act) {
            const uint32_t base = sh ? as_off : 0u;   // byte offset of this unit's `a` rows
#pragma unroll
            for (int t = 0; t < NT; ++t) {
                const int tt = t < ntok ? t : 0;
                const int row = sh ? g * NT + tt : R.group_first[g] + tt;
                const uint32_t off = base + 4u * (uint32_t)(row * K + b * QK);
                uint32_t w[QK];
                if (p.stage_words) {
                    const int slice = ((sh ? ng * p.FF : 0) + row * K) / QK + b;
                    const uint4* src = reinterpret_cast<const uint4*>(lds) + slice * (QK / 4);
#pragma unroll
                    for (int v = 0; v < QK / 4; ++v) {
                        const uint4 q = src[v ^ (slice % (QK / 4))];
                        w[4 * v + 0] = q.x;
                        w[4 * v + 1] = q.y;
                        w[4 * v + 2] = q.z;
                        w[4 * v + 3] = q.w;
                    }
                } else {
                    // A word still 0 has not landed yet: read the slice again.
                    // (A plain loop: a lambda holding w by reference spills it.)
                    long n = 0;
                    while (!load_packed_words<QT>(w, a_rsrc, off) || p.polls == 0) {
                        if (++n > p.polls) {   // a bound of 0 gives up at once
                            flag_error(p.err, kErrTimeout);
                            R.fail = 1;
                            break;
                        }
                        __builtin_amdgcn_s_sleep(1);
                    }
                }
                slice_from_packed<QT>(xs[t], w, p.z);
            }
        }
        if (act) {
#pragma unroll
            for (int i = 0; i < RPT; ++i) {
                const int r = rs + i * S;
                if (r < nrows) {
                    float o[NT];
                    block_dot<QT, 2, NT>(c[i], scale_at_use(sc[i]), xs, ntok, o);
                    const int nbp = sh ? nbp_s : nbp_r;
                    float* dst = part + (sh ? sh_off : 0) + ((g * p.dn_rows + r) * NT) * nbp + b;
#pragma unroll
                    for (int t = 0; t < NT; ++t) dst[t * nbp] = o[t];
                }
            }
        }
    }
    if (!p.stage_words) {
        // Every load of this workgroup has landed (its results are used); saying
        // so leaves the compiler no load to wait for after the atomic below.
        __builtin_amdgcn_s_waitcnt(0);
        lds_barrier();
        // Every `a` word this workgroup reads has been used: count the workgroup
        // (without waiting for the atomic).
        if (tid == 0) atomic_add_detached(sync_loaded(p.sync, tile % kLoadFan, p.max_groups + p.shared_groups), 1);
    } else {
        lds_barrier();
    }
    // y[t][h0 + r] = shared(t)[r] + sum over the token's k slots of cw * d,
    // where d (of the slot's group, row and token) is its block-column
    // partials summed in column order.  Lane j of a group of JS lanes takes
    // slot j (0 for a skipped slot); the slot terms are summed by a fixed tree
    // over the group.
    const int n_out = p.T * nrows;
    for (int base = 0; base < n_out; base += kGemvThreads / JS) {
        const int it = base + tid / JS, j = tid % JS;
        const bool live = it < n_out;
        const int t = live ? it / nrows : 0, r = live ? it - t * nrows : 0;
        float v = 0.f;
        if (live && j < p.k) {
            const int gs = R.slot_src[t * p.k + j];   // group * NT + token in group
            if (gs >= 0) {
                const int gg = gs / NT, tt = gs - (gs / NT) * NT;
                v = cw * sum_columns(part + ((gg * p.dn_rows + r) * NT + tt) * nbp_r, nb_r);
            }
        }
        v = row_sum_f32(v);
        if (JS == 32) v += __shfl_xor(v, 16);
        if (live && j == 0) {
            float acc = v;
            if (p.shared) {
                const int sg = t / NT, st = t - sg * NT;
                acc = sum_columns(part + sh_off + ((sg * p.dn_rows + r) * NT + st) * nbp_s, nb_s) + v;
            }
            p.y[(size_t)t * p.H + h0 + r] = R.fail ? __uint_as_float(0x7FC00000u) : acc;
        }
    }
}

// The workgroup after the down tiles returns the call's shared state to zero
// for the next call, off every other workgroup's path: once every ready flag
// of every replica is up (so every gate/up counter update has landed) and
// every down workgroup has counted its `a` words as loaded (so every `a` store
// has landed and no one reads `a` again), it clears the counters, the flags,
// the load count and the `a` words of this call.
template <int NT>
__device__ void janitor_role(const DecodeParams& p, RouteLDS& R) {
    const int tid = threadIdx.x;
    if (load_error(p.err) != 0) return;   // an unchecked earlier failure: the state stays as it is
    const int ng = R.n_groups, nsg = p.shared_groups, n_ctr = p.max_groups + p.shared_groups;
    // Every ready flag of every replica, and every replica's prefetch hint at
    // its full count (one per group).
    for (int i = tid; i < p.n_ready * (ng + nsg + 1); i += kGemvThreads) {
        const int r = i / (ng + nsg + 1), gi = i - r * (ng + nsg + 1);
        const bool hint = gi == ng + nsg;
        const int ctr = hint ? n_ctr : (gi < ng ? gi : p.max_groups + (gi - ng));
        const int need = hint ? ng + nsg : 1;
        const int* w = sync_ready(p.sync, r, ctr, n_ctr);
        bounded_wait<2>([&]() __attribute__((always_inline)) { return __hip_atomic_load(w, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) >= need; },
                        p.polls, p.err);
    }
    const int fan = min(kLoadFan, p.tiles_dn);
    if (tid < fan) {
        const int members = (p.tiles_dn - tid + kLoadFan - 1) / kLoadFan;
        const int* w = sync_loaded(p.sync, tid, n_ctr);
        bounded_wait<2>([&]() __attribute__((always_inline)) { return __hip_atomic_load(w, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) >= members; },
                        p.polls, p.err);
    }
    __syncthreads();
    for (int i = tid; i < n_ctr; i += kGemvThreads)
        __hip_atomic_store(sync_group(p.sync, i), 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    for (int i = tid; i < p.n_ready * (n_ctr + 1); i += kGemvThreads)
        __hip_atomic_store(sync_ready(p.sync, i / (n_ctr + 1), i % (n_ctr + 1), n_ctr), 0, __ATOMIC_RELAXED,
                           __HIP_MEMORY_SCOPE_AGENT);
    if (tid < fan) __hip_atomic_store(sync_loaded(p.sync, tid, n_ctr), 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    const int na = p.max_groups * p.FF, nas = p.T * p.FFs;
    for (int i = tid; i < na; i += kGemvThreads) __hip_atomic_store(p.a + i, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    for (int i = tid; i < nas; i += kGemvThreads)
        __hip_atomic_store(p.as + i, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

template <int QT, int NTERM, bool PAIR>
__global__ void __launch_bounds__(kGemvThreads, 3) decode_layer_kernel(DecodeParams p) {
    constexpr int NT = 1;   // one token
    extern __shared__ __align__(16) float lds[];   // 16-byte aligned: float4 reads
    __shared__ RouteLDS R;
    const int tid = threadIdx.x;
    const int wg = blockIdx.x;
    if (NT == 1 && p.x_off >= 0 && wg < p.n_gu && tid >= 64) {
        // One token: while the first wave routes, the others arrange the
        // token's activation slice of every block column in LDS (the routing's
        // closing barrier publishes them).
        constexpr int QK = QTraits<QT>::QK;
        const int nblk = p.H / QK;
        for (int b = tid - 64; b < nblk; b += kGemvThreads - 64) {
            XSlice<QT, NTERM> xsl;
            if constexpr (NTERM == 1)
                load_slice_bf16<QT, 1>(xsl, (const uint16_t*)p.x + b * QK, nullptr, p.z);
            else
                load_slice_f32<QT>(xsl, (const float*)p.x + b * QK, p.z);
            slice_to_lds<QT, NTERM>(xsl, reinterpret_cast<uint32_t*>(lds) + p.x_off + b * SliceWords<QT, NTERM>::N);
        }
    }
    // Only the down workgroups (the combine) and workgroup 0 (w_out) read the
    // weights: the gate/up workgroups skip the softmax, which is on the path to
    // their weight loads.
    const int dn_tile = wg >= p.n_gu && wg - p.n_gu < p.tiles_dn ? wg - p.n_gu : -1;
    route_and_bucket(p, R, wg >= p.n_gu || (wg == 0 && p.w_out));
    if (wg == 0) {
        for (int q = tid; q < p.T * p.k; q += kGemvThreads) {
            if (p.ids_out) p.ids_out[q] = R.id[q];
            if (p.w_out) p.w_out[q] = R.w[q];
        }
    }
    if (R.bad) {
        // Invalid caller-supplied routing: nothing is computed; the down
        // workgroups write NaN rows.
        if (dn_tile >= 0) {
            const int h0 = dn_tile * p.dn_rows, nrows = min(p.dn_rows, p.H - h0);
            for (int i = tid; i < p.T * nrows; i += kGemvThreads)
                p.y[(size_t)(i / nrows) * p.H + h0 + i % nrows] = __uint_as_float(0x7FC00000u);
        }
        return;
    }
    if (wg < p.n_gu) gateup_role<QT, NT, NTERM, PAIR>(p, R, wg, lds);
    if (dn_tile >= 0) down_role<QT, NT>(p, R, dn_tile, lds);
    else if (wg >= p.n_gu) janitor_role<NT>(p, R);
}

// ---------------------------------------------------------------------------------------------
// Host side of the decode path.
// ---------------------------------------------------------------------------------------------
GemvShape gemv_shape(int H, int FF, int FFs, int qtype, float z, int T, int k, int n_cu) {
    GemvShape g{};
    const int qk = codes_per_block(qtype);
    const int NT = 1;   // one token (T == 1)
    g.H = H;
    g.FF = FF;
    g.FFs = FFs;
    g.qtype = qtype;
    g.z = z;
    const int nblk_gu = H / qk;
    // Lanes take one block column each, or two adjacent ones where that puts
    // more lanes to work (the sums are the same bits either way).
    const int P1 = kGemvThreads / nblk_gu;
    const int P2 = nblk_gu % 2 == 0 ? kGemvThreads / (nblk_gu / 2) : 0;
    g.gu_pair = P2 * (nblk_gu / 2) > P1 * nblk_gu ? 1 : 0;
    const int P = g.gu_pair ? P2 : P1;
    const int max_pass = g.gu_pair ? kMaxPassPair : kMaxPass;
    // Passes per gate/up workgroup (tile rows = P * passes).  The busiest CU
    // holds k = ceil(tiles / CUs) tiles, one wave each on every SIMD, and
    // runs k x passes passes of block products; k waves a SIMD hide each
    // other's dependency stalls, so a pass costs less with more of them.
    // Cost k x passes x w(k), with w(1..3) = 57, 45, 42: the cycles per
    // instruction of these products measured with one wave a SIMD (5.7), and
    // a fit to the sweep of pass counts at both decode shapes.  Counts whose
    // gate/up tiles, with the fewest down tiles (the most rows a down tile
    // takes), would not all be resident at once (three a CU) are skipped: a
    // down workgroup dispatched late starts its routing and prefetch late.
    // The larger count wins a tie.  Strata decode: 540 tiles of 2 passes;
    // Gemma, with two block columns a lane: 394 tiles of 4 passes.
    const int cus = n_cu > 0 ? n_cu : 256;
    g.max_groups = T * k;
    const int nb_r = FF / qk, nb_s = FFs / qk;
    const size_t units = (size_t)g.max_groups * nb_r + (size_t)(FFs ? (T + NT - 1) / NT : 0) * nb_s;
    // A down thread prefetches at most rows_per_thread rows of its unit;
    // with few units, S = 256 / units threads share a unit's rows.
    int s_min = (int)(kGemvThreads / units);
    s_min = s_min < 1 ? 1 : s_min;
    int rows_cap = rows_per_thread(qtype) * s_min;
    rows_cap = rows_cap > kMaxRowsDn ? kMaxRowsDn : rows_cap;
    {
        const int sg = FFs ? (T + NT - 1) / NT : 0;
        const long fewest_dn = (H + rows_cap - 1) / rows_cap;
        static const int w[4] = {0, 57, 45, 42};
        g.gu_passes = 0;
        long best = 0;
        for (int pp = max_pass; pp >= 1; --pp) {
            const int tr = P * pp;
            const long tiles = (long)g.max_groups * ((FF + tr - 1) / tr) + (long)sg * (FFs ? (FFs + tr - 1) / tr : 0);
            const long kk = (tiles + cus - 1) / cus;
            if (kk > 3 || tiles + fewest_dn + 1 > 3L * cus) continue;
            const long cost = kk * pp * w[kk];
            if (g.gu_passes == 0 || cost < best) {
                g.gu_passes = pp;
                best = cost;
            }
        }
        if (g.gu_passes == 0) g.gu_passes = max_pass;   // no count keeps them all resident: the fewest tiles
    }
    g.tile_rows_gu = P * g.gu_passes;
    g.tiles_gu = (FF + g.tile_rows_gu - 1) / g.tile_rows_gu;
    g.tiles_gu_s = FFs ? (FFs + g.tile_rows_gu - 1) / g.tile_rows_gu : 0;
    const int per_expert = (T + NT - 1) / NT;
    g.shared_groups = FFs ? per_expert : 0;
    g.n_gu = g.max_groups * g.tiles_gu + g.shared_groups * g.tiles_gu_s;
    // One token: the arranged activation slices follow the gate/up partials
    // (sized for fp32 activations, the larger slice).
    const int ncol_gu = nblk_gu % 2 == 0 ? nblk_gu / 2 : nblk_gu;   // lane pairs add their partials first
    const size_t part_gu = (size_t)2 * g.tile_rows_gu * ((ncol_gu + 3) & ~3) * NT * 4;
    g.x_off = T == 1 ? (int)(part_gu / 4) : -1;
    const int sw = ((qk == 64 ? 64 : 32) + (qk == 64 ? 3 : 1) + 1 + 3) & ~3;
    const size_t lds_gu = part_gu + (T == 1 ? (size_t)nblk_gu * sw * 4 : 0);
    // Down workgroups own tiles of r output rows.  The row count changes no
    // summation order; it sets the time of the busiest CU, which runs
    // ceil(tiles / CUs) tiles of r rows each.  r is the value that makes that
    // product smallest (the larger r on a tie) among those whose partial sums
    // fit in LDS and with which every workgroup of the launch is resident at
    // once (three a CU while LDS allows; a workgroup that waits to be
    // dispatched lengthens the launch by a whole tile time).
    // partials padded to 4 columns per (group, row, token), plus one sum each
    const size_t per_row =
        ((size_t)g.max_groups * ((nb_r + 3) & ~3) + (size_t)g.shared_groups * ((nb_s + 3) & ~3) + g.max_groups +
         g.shared_groups) * NT * 4;
    // One token: the `a` words are staged in LDS ahead of the partials.
    const long words = (long)g.max_groups * FF + FFs;
    g.stage_words = (T == 1 && words <= kStageMaxWords) ? (int)words : 0;
    const size_t stage = g.stage_words ? (size_t)stage_bytes(g.stage_words) : 0;
    int rows = 0;
    long best = 0;
    for (int r = rows_cap; r >= 1; --r) {
        const size_t lds = std::max(per_row * r + stage, lds_gu);
        if (per_row * r + stage > kDecodeLdsBudget) continue;
        const int tiles = (H + r - 1) / r;
        const long per_cu = std::min<long>(3, (long)(160 * 1024) / (long)(lds + kDecodeStaticLds));
        if ((long)g.n_gu + tiles + 1 > per_cu * cus) continue;
        const long cost = (long)((tiles + cus - 1) / cus) * r;
        if (rows == 0 || cost < best) {
            rows = r;
            best = cost;
        }
    }
    if (rows == 0) {   // nothing fits every workgroup at once: the largest tile LDS allows
        rows = rows_cap;
        while (rows > 1 && per_row * rows + stage > kDecodeLdsBudget) --rows;
    }
    g.tile_rows_dn = rows;
    g.tiles_dn = (H + rows - 1) / rows;
    const size_t lds_dn = per_row * rows + stage;
    g.lds_bytes = lds_dn > lds_gu ? lds_dn : lds_gu;
    g.grid = g.n_gu + g.tiles_dn + 1;   // + the workgroup that resets the shared state
    return g;
}

template <int QT, int NTERM, bool PAIR>
static hipError_t launch_decode_t(const GemvShape& g, DecodeParams& p, hipStream_t s) {
    // Allow the dynamic LDS the largest shapes need, once per device.
    static std::mutex mu;
    static std::set<int> done;
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    {
        std::lock_guard<std::mutex> lock(mu);
        if (!done.count(dev)) {
            e = hipFuncSetAttribute((const void*)decode_layer_kernel<QT, NTERM, PAIR>,
                                    hipFuncAttributeMaxDynamicSharedMemorySize, 128 * 1024);
            if (e != hipSuccess) return e;
            done.insert(dev);
        }
    }
    hipLaunchKernelGGL((decode_layer_kernel<QT, NTERM, PAIR>), dim3(g.grid), dim3(kGemvThreads), g.lds_bytes, s, p);
    return hipGetLastError();
}

hipError_t launch_decode_layer(const GemvShape& g, const void* const* table, const void* single, const void* shared,
                               const void* x, int x_dtype, const float* logits, int T, int E, int k, int renorm,
                               int identity, const LayerOpts& o, int* ids_out, float* w_out, const SmallLayout& L,
                               char* ws, float* y, hipStream_t s, StageMarks* marks) {
    DecodeParams p{};
    p.table = table;
    p.single = (const uint8_t*)single;
    p.shared = (const uint8_t*)shared;
    p.x = x;
    p.logits = logits;
    p.T = T;
    p.E = E;
    p.k = k;
    p.renorm = renorm;
    p.identity = identity;
    p.H = g.H;
    p.FF = g.FF;
    p.FFs = g.FFs;
    p.z = g.z;
    p.act = o.act;
    p.down_scale = o.down_scale;
    p.ids_in = o.ids_in;
    p.w_in = o.w_in;
    p.ids_out = ids_out;
    p.w_out = w_out;
    p.a = (uint32_t*)(ws + L.a);
    p.as = (uint32_t*)(ws + L.as);
    p.y = y;
    p.sync = (int*)(ws + L.sync);
    p.err = p.sync + kErrWord;
    p.polls = wait_polls();
    p.gu_passes = g.gu_passes;
    p.tiles_gu = g.tiles_gu;
    p.tiles_gu_s = g.tiles_gu_s;
    p.max_groups = g.max_groups;
    p.shared_groups = g.shared_groups;
    p.n_gu = g.n_gu;
    p.dn_rows = g.tile_rows_dn;
    p.tiles_dn = g.tiles_dn;
    p.n_ready = g.tiles_dn < kReadyReplicas ? g.tiles_dn : kReadyReplicas;
    p.stage_words = g.stage_words;
    p.x_off = g.x_off;
    stage_mark(marks, s);
    hipError_t e;
    const bool bf = x_dtype == 1;
    if (g.qtype == 1)
        e = bf ? launch_decode_t<1, 1, false>(g, p, s) : launch_decode_t<1, 2, false>(g, p, s);
    else if (!g.gu_pair)
        e = bf ? launch_decode_t<2, 1, false>(g, p, s) : launch_decode_t<2, 2, false>(g, p, s);
    else
        e = bf ? launch_decode_t<2, 1, true>(g, p, s) : launch_decode_t<2, 2, true>(g, p, s);
    stage_mark(marks, s);
    return e;
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
