// Verify-window layer (2 <= T <= 8 tokens): one fused kernel per layer.
//
// A speculative verify window scores a few draft tokens at once, and under a
// skewed expert popularity those tokens share experts (Strata, "The plan:
// three destinations per expert": an expert chosen by several tokens of the
// window is read once).  Here the tokens that chose an expert form groups of
// up to two, and each group's weights are read once for its tokens.  (A
// group of every token of the expert would make the work items of hot
// experts several times heavier than the rest, which costs more time than
// the re-reads of hot experts by their later groups.)
//
// Work items, in the order every workgroup derives them from the routing
// (groups of two tokens first):
//   gate/up items  (group, tile of FF rows): the codes of every pass of the
//                  tile are loaded once and held in registers while the
//                  group's tokens go through them one at a time; the SwiGLU
//                  output rows are published as never-zero packed words;
//   down items     (group, chunk of H rows): the group's `a` rows are
//                  arranged into dot-pair slices in LDS once, the down codes
//                  of the chunk are held in registers, and the tokens go
//                  through them one at a time; the result of each (slot, row)
//                  is published as a never-zero fp32 word.
// The shared expert's groups hold the window's tokens two at a time; its down
// items cover a chunk in several sub-ranges of rows.
//
// Workgroup w takes the gate/up items w, w + G, ... and then the down items
// G - 1 - w, 2G - 1 - w, ... (G = the grid; reversed, so that the workgroups
// with the most gate/up items get the fewest down items).  G is at most the
// number of workgroups the GPU holds at once (two per CU where registers and
// LDS allow), so that every workgroup is resident: a down item waits for
// gate/up items of other workgroups, which never wait, so every wait ends.
// (If other work holds part of the GPU, the waits last until it leaves room.)
// Each gate/up tile bumps its group's counter, and the down items of a group
// start once its counter is complete (no wait for other groups).  Each down
// item then bumps its chunk's counter once its d words are issued.  When a
// chunk's count is complete, up to eight workgroups that are done with their
// own items combine it, each a part of its rows: y[t][h] = shared +
// sum_j w[t][j] d, the slots summed in rank order, so the output does not
// depend on timing.  Readers of `a` and d read again any word still 0, so a
// count that runs ahead of the words costs a reload, not a wrong value.
//
// Every piece of shared state is returned to zero by its last user: the last
// down item of a group clears the group's counters and `a` rows; each
// combining part clears the d words it read, and the last part of a chunk its
// counters.
//
// Failures.  A bounded wait that gives up ORs kErrTimeout into the
// workspace's error word, and from then on every value its workgroup
// publishes (d words, output rows) is NaN, so the failure reaches y.  Every
// workgroup reads the error word when its gate/up items are done, before its
// first wait (not earlier: an agent-coherent load in flight holds every
// barrier of its workgroup): if a failure that moe_workspace_check has not
// cleared is there, the workgroup writes NaN rows and does nothing else, so
// no wait runs on stale shared state.
#include <map>
#include <mutex>
#include <utility>

#include "moe_gemv_common.h"

namespace moe {

constexpr int kWinPairs = kSmallT * kMaxK;   // (token, slot) pairs of a window
constexpr int kWinMaxPass = 8;               // passes per item (rows = P * passes)
// Tokens of one expert per group: a hot expert's tokens are split over
// several groups, so that no work item holds many more tokens than others
// (its weights are read once per group).
constexpr int kWinGroup = 2;
constexpr int kWinShared = (kSmallT + kWinGroup - 1) / kWinGroup;   // groups of the shared expert, at most
constexpr int kWinCombineParts = 8;          // workgroups that combine one chunk, at most
constexpr int kWinItemCost = 4;              // a gate/up item's fixed work, in passes (an estimate)

struct WindowParams {
    const void* const* table;
    const uint8_t* single;      // one expert's blob when table == nullptr (moe_expert_ffn)
    const uint8_t* shared;
    const void* x;              // [T][H] bf16 or fp32
    const float* logits;        // [T][E]
    int T, E, k, renorm, identity;
    int H, FF, FFs;
    float z;
    int act;                    // gate activation (kActSilu / kActGeluTanh)
    const float* down_scale;    // [E] per routed expert, or null
    const int* ids_in;          // [T][k] caller-supplied routing, or null
    const float* w_in;          // [T][k]
    int* ids_out;               // [T][k] or null
    float* w_out;               // [T][k] or null
    uint32_t* a;                // [T*k][FF] by sorted pair (expert, token), packed bf16 hi | lo << 16
    uint32_t* as;               // [T][FFs] the shared expert's
    uint32_t* d;                // [8k + 8][H] fp32 bits: slot t*k + j, then 8k + t for the shared expert
    float* y;                   // [T][H]
    int* sync;                  // window sync lines, see win_* below
    int* err;                   // the workspace's error word (sync + kErrWord)
    long polls;                 // bound of every wait
    int dn_passes, chunk_rows, n_chunks;
    int sh_passes, sh_rows, sh_items;
    int n_wg;                   // the grid
    int x_off;                  // gate/up: LDS word offset of the activation slices
    int stage_words;            // down: LDS words reserved for the staged `a` rows
};

// Sync lines (16 ints each): line 1 the error word; per group g (routed
// groups g < 8k, the shared expert's groups from 8k on) its gate/up tile
// count (complete at tiles_gu) and its down item count; then per chunk its
// down item count, then per chunk the count of its combined parts.
__device__ __forceinline__ int* win_gu_count(int* s, int g) { return s + 16 * (2 + 2 * g); }
__device__ __forceinline__ int* win_dn_count(int* s, int g) { return s + 16 * (3 + 2 * g); }
__device__ __forceinline__ int* win_chunk(int* s, int k, int c) { return s + 16 * (2 + 2 * (kSmallT * k + kWinShared) + c); }
__device__ __forceinline__ int* win_combined(int* s, int k, int n_chunks, int c) {
    return s + 16 * (2 + 2 * (kSmallT * k + kWinShared) + n_chunks + c);
}


struct WinLDS {
    int id[kWinPairs];
    float w[kWinPairs];
    float cw[kWinPairs];            // combine weight: w times the expert's down scale; 0 for a skipped slot
    int on[kWinPairs];              // the slot has a group (not skipped)
    alignas(16) int key[kWinPairs + 4];   // expert << 8 | slot, padded with INT_MAX
    int sorted[kWinPairs];          // sorted position -> slot
    int group_first[kWinPairs + 1]; // first sorted position of each group; [n_groups] = T * k
    int gorder[kWinPairs];          // groups in work order: full groups (kWinGroup tokens) first
    int n_groups;
    int gu_passes, tiles_gu, tiles_gu_s;   // this call's gate/up tiling (gu_tiling)
    int flag_reset;
    int fail;               // publish NaN: an earlier failure, or one of this workgroup's waits gave up
    int prior;              // 1: an unchecked failure of an earlier call; -1: not looked at yet
    int bad;                // a caller-supplied id outside [0, E) with a nonzero weight
};

constexpr uint32_t kNaNBits = 0x7FC00000u;   // never 0, so a published NaN reads as written

// Gate/up passes per tile for this call's groups: the count p of passes
// (at most kWinMaxPass) that makes the busiest workgroup's share, rounds of
// items times (p + kWinItemCost), the smallest (the larger p on a tie: fewer
// items).  kWinItemCost prices an item's fixed work (its row sums, SwiGLU,
// stores and count) in passes; without it the smallest tiles would win.
// With 63 groups of the Strata shape on 512 workgroups, 7 passes give 1,008
// items in 2 rounds (22) where 8 give 882 items, also in 2 rounds (24); with
// 65 groups 8 passes stay (2 rounds against 3).  Every workgroup derives the
// same tiling from the same routing.  One wave: lane i < kWinMaxPass prices
// kWinMaxPass - i passes.
__device__ __forceinline__ void gu_tiling(const WindowParams& p, WinLDS& R, int n_groups, int P, int lane) {
    const int n_sg = p.FFs ? (p.T + kWinGroup - 1) / kWinGroup : 0;
    const int gp = kWinMaxPass - min(lane, kWinMaxPass - 1);
    const int rows = P * gp;
    const int t = (p.FF + rows - 1) / rows, ts = p.FFs ? (p.FFs + rows - 1) / rows : 0;
    const int items = n_groups * t + n_sg * ts;
    const uint32_t cost = (uint32_t)min((items + p.n_wg - 1) / p.n_wg * (gp + kWinItemCost), 1 << 25);
    // (cost, lane): the lowest cost, then the most passes
    const uint32_t best = wave_min_u32(lane < kWinMaxPass ? cost * 64u + (uint32_t)lane : 0xFFFFFFFFu);
    if (lane == (int)(best & 63u)) {
        R.gu_passes = gp;
        R.tiles_gu = t;
        R.tiles_gu_s = ts;
    }
}

// Routing of the T tokens (wave w takes tokens w and w + 4), then the groups:
// pairs sorted by (expert, token), each run of one expert cut into groups of
// at most kWinGroup pairs.  With caller-supplied routing (Krasis white paper
// 7.5), zero-weight slots sort after every other pair and get no group, so
// their experts are never read; a nonzero weight on an id outside [0, E)
// flags kErrBadId and fails the call.
// `scratch` is the dynamic LDS, free until the roles start (128 keys per wave).
__device__ __forceinline__ void route_window(const WindowParams& p, WinLDS& R, uint64_t* scratch, int P_gu) {
    const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
    const int k = p.k, n = p.T * k;
    bool bad_any = false;
    // Wave w routes tokens w and w + 4 (T <= 8).
    int rid[2] = {0, 0};
    float rwt[2] = {1.f, 1.f};
    if (!p.ids_in && !p.identity && wv < p.T)
        wave_topk2(p.logits + (size_t)wv * p.E, p.logits + (size_t)(wv + 4) * p.E, wv + 4 < p.T, p.E, k, p.renorm,
                   lane, scratch + 128 * wv, rid, rwt);
    for (int t = wv; t < p.T; t += kGemvThreads / 64) {
        int id = 0;
        float wt = 1.f;
        bool on = true;
        if (p.ids_in) {
            id = lane < k ? p.ids_in[t * k + lane] : 0;
            wt = lane < k ? p.w_in[t * k + lane] : 0.f;
            on = wt != 0.f;
            const bool bad = lane < k && on && (id < 0 || id >= p.E);
            if (bad) flag_error(p.err, kErrBadId);
            bad_any |= __ballot(bad) != 0;
            on = on && !bad;
        } else if (!p.identity) {
            id = t == wv ? rid[0] : rid[1];
            wt = t == wv ? rwt[0] : rwt[1];
        }
        if (lane < k) {
            R.id[t * k + lane] = id;
            R.w[t * k + lane] = wt;
            float cw = wt;
            if (p.down_scale && on) cw = wt * p.down_scale[id];
            if (!on) cw = 0.f;
            R.cw[t * k + lane] = cw;
            R.on[t * k + lane] = on;
            // skipped slots sort after every pair (ids are below 2^10)
            R.key[t * k + lane] = on ? (id << 8 | (t * k + lane)) : (0x7F000000 | (t * k + lane));
        }
    }
    if (tid < 4) R.key[n + tid] = 0x7FFFFFFF;
    if (tid == 0) {
        R.fail = 0;
        R.prior = -1;
        R.bad = 0;
    }
    __syncthreads();
    if (bad_any && lane == 0) R.bad = 1;
    // Keys are distinct (a token selects an expert at most once), so each
    // pair's count of smaller keys is its sorted position.
    if (tid < n) {
        const int mine = R.key[tid];
        int rank = 0;
        for (int j = 0; j < n; j += 4) {
            const int4 q = *reinterpret_cast<const int4*>(&R.key[j]);
            rank += (q.x < mine) + (q.y < mine) + (q.z < mine) + (q.w < mine);
        }
        R.sorted[rank] = tid;
    }
    __syncthreads();
    if (wv == 0) {
        // The pairs with a group: all of them, or those of nonzero weight
        // (sorted first).
        int na = n;
        if (p.ids_in) {
            na = 0;
            for (int r0 = 0; r0 < n; r0 += 64) na += __popcll(__ballot(r0 + lane < n && R.on[r0 + lane]));
        }
        // A group starts at every kWinGroup-th pair of a run of one expert.
        int base = 0, carry = 0;   // carry: the run start in effect at the end of the previous 64 pairs
        for (int r0 = 0; r0 < na; r0 += 64) {
            const int r = r0 + lane;
            const bool run_start = r < na && (r == 0 || R.id[R.sorted[r - 1]] != R.id[R.sorted[r]]);
            const uint64_t m = __ballot(run_start);
            const uint64_t upto = m & (lane == 63 ? ~0ull : ((2ull << lane) - 1));
            const int rs = upto ? r0 + 63 - __clzll(upto) : carry;
            const bool start = r < na && (r - rs) % kWinGroup == 0;
            const uint64_t gm = __ballot(start);
            if (start) R.group_first[base + lanes_below(gm)] = r;
            base += __popcll(gm);
            carry = __builtin_amdgcn_readlane(rs, 63);
        }
        if (lane == 0) {
            R.n_groups = base;
            R.group_first[base] = na;
        }
        __builtin_amdgcn_wave_barrier();
        // Work order: the groups with kWinGroup tokens (the heaviest items)
        // first, each class in group order, so that round-robin items put
        // at most about one heavy item on each workgroup.
        const int ng = base;
        int n_full = 0;
        for (int g0 = 0; g0 < ng; g0 += 64) {
            const int g = g0 + lane;
            n_full += __popcll(__ballot(g < ng && R.group_first[g + 1] - R.group_first[g] == kWinGroup));
        }
        int fb = 0, pb = n_full;
        for (int g0 = 0; g0 < ng; g0 += 64) {
            const int g = g0 + lane;
            const bool full = g < ng && R.group_first[g + 1] - R.group_first[g] == kWinGroup;
            const bool part = g < ng && !full;
            const uint64_t mf = __ballot(full), mp = __ballot(part);
            if (full) R.gorder[fb + lanes_below(mf)] = g;
            if (part) R.gorder[pb + lanes_below(mp)] = g;
            fb += __popcll(mf);
            pb += __popcll(mp);
        }
        gu_tiling(p, R, ng, P_gu, lane);
    }
    __syncthreads();
}

// One gate/up item: group (or the shared expert) and tile.
struct GuItem {
    const uint8_t* blob;
    uint32_t* out;
    int g, first, n_e, rows, f0;
    bool sh;
    bool none;   // no item: its loads read one chunk (the buffers' turn needs loads, not these bytes)
};

__device__ __forceinline__ GuItem gu_item(const WindowParams& p, const WinLDS& R, int item, int n_routed, int Rr) {
    GuItem it;
    it.sh = item >= n_routed;
    int tile;
    if (!it.sh) {
        const int tg = __builtin_amdgcn_readfirstlane(R.tiles_gu);   // uniform: scalar arithmetic
        const int gi = item / tg;
        it.g = R.gorder[gi];
        tile = item - gi * tg;
        it.first = R.group_first[it.g];
        it.n_e = R.group_first[it.g + 1] - it.first;
        it.blob = p.table ? table_blob(p.table, R.id[R.sorted[it.first]]) : p.single;
        it.rows = p.FF;
        it.out = p.a;
    } else {   // shared group sg: tokens kWinGroup * sg ..
        const int ts = __builtin_amdgcn_readfirstlane(R.tiles_gu_s);
        const int i2 = item - n_routed, sg = i2 / ts;
        it.g = kSmallT * p.k + sg;
        tile = i2 - sg * ts;
        it.first = kWinGroup * sg;
        it.n_e = min(kWinGroup, p.T - it.first);
        it.blob = p.shared;
        it.rows = p.FFs;
        it.out = p.as;
    }
    it.f0 = tile * Rr;
    it.none = false;
    return it;
}

// Every pass's codes and scales of the item's tile at once, from clamped rows
// (the last tile's overhang re-reads its last row): all loads in flight
// together, and no branch per pass.
struct GuCodes {
    uint4 cg[kWinMaxPass], cu[kWinMaxPass];
    uint16_t sg[kWinMaxPass], su[kWinMaxPass];
};

__device__ __forceinline__ void gu_load(const GuItem& it, int nblk, int P, int gp, int rp, int b, GuCodes& c) {
    const size_t plane = (size_t)it.rows * nblk;
    const uint8_t* gcode = it.blob;
    const uint8_t* gscale = it.blob + plane * 16;
    const uint8_t* ucode = it.blob + plane * 18;
    const uint8_t* uscale = ucode + plane * 16;
#pragma unroll
    for (int m = 0; m < kWinMaxPass; ++m) {
        const int f = min(it.f0 + min(m, gp - 1) * P + rp, it.rows - 1);
        const size_t blk = it.none ? 0 : (size_t)f * nblk + b;
        if (it.sh) {   // the shared expert: read by every call
            c.cg[m] = ldg_u4(gcode + blk * 16);
            c.cu[m] = ldg_u4(ucode + blk * 16);
        } else {
            c.cg[m] = ldg_u4_nt(gcode + blk * 16);
            c.cu[m] = ldg_u4_nt(ucode + blk * 16);
        }
        c.sg[m] = ldg_u16(gscale + blk * 2);
        c.su[m] = ldg_u16(uscale + blk * 2);
    }
}

// The item's tokens through the held codes, one at a time (its slice in
// registers), two per round of partial sums; then SwiGLU, the published `a`
// rows, and the tile counted.
template <int QT, int NTERM>
__device__ __forceinline__ void gu_compute(const WindowParams& p, const WinLDS& R, const GuItem& it, GuCodes& c,
                                           float* lds, int nblk, int P, int gp, int rp, int b, bool active) {
    constexpr int QK = QTraits<QT>::QK, SW = SliceWords<QT, NTERM>::N;
    const int tid = threadIdx.x;
    const int Rr = P * gp;
    // With an even count of block columns, lanes 2j and 2j + 1 (columns b and
    // b + 1 of one row) add their partials first: ncol columns per (row,
    // token), padded to ncp.
    const bool pairs = (nblk & 1) == 0;
    const int ncol = pairs ? nblk / 2 : nblk;
    const int ncp = (ncol + 3) & ~3;
    const uint32_t* xsl = reinterpret_cast<const uint32_t*>(lds) + p.x_off;
    for (int t0 = 0; t0 < it.n_e; t0 += 2) {
        const int nt = min(2, it.n_e - t0);
#pragma unroll 1
        for (int i = 0; i < nt; ++i) {
            // Opaque to the compiler per token: the codes' shifted copies are
            // then formed at their use, not hoisted out of this loop.
#pragma unroll
            for (int m = 0; m < kWinMaxPass; ++m) {
                pin_u4(c.cg[m]);
                pin_u4(c.cu[m]);
            }
            const int tok = it.sh ? it.first + t0 + i : R.sorted[it.first + t0 + i] / p.k;
            XSlice<QT, NTERM> xs[1];
            if (p.x_off >= 0) {
                slice_from_lds<QT, NTERM>(xs[0], xsl + (tok * nblk + b) * SW);
            } else {   // slices too large for LDS: straight from the activations
                if constexpr (NTERM == 1)
                    load_slice_bf16<QT, 1>(xs[0], (const uint16_t*)p.x + (size_t)tok * p.H + b * QK, nullptr, p.z);
                else
                    load_slice_f32<QT>(xs[0], (const float*)p.x + (size_t)tok * p.H + b * QK, p.z);
            }
            // The partials' addresses are formed here, not hoisted out of the
            // token loop (where holding them would spill registers).
            int pb = (rp * 2 + i) * ncp + (pairs ? (b >> 1) : b);
            asm volatile("" : "+v"(pb));
#pragma unroll
            for (int m = 0; m < kWinMaxPass; ++m) {
                const int f = it.f0 + m * P + rp;
                if (active && m < gp && f < it.rows) {
                    float og[1], ou[1];
                    block_dot<QT, NTERM, 1>(c.cg[m], scale_at_use(c.sg[m]), xs, 1, og);
                    block_dot<QT, NTERM, 1>(c.cu[m], scale_at_use(c.su[m]), xs, 1, ou);
                    if (pairs) {
                        og[0] += dpp_xor1_f32(og[0]);
                        ou[0] += dpp_xor1_f32(ou[0]);
                    }
                    if (!pairs || (b & 1) == 0) {
                        // part[((mat * Rr + rr) * 2 + i) * ncp + col] with rr = m * P + rp
                        float* q = lds + pb + m * P * 2 * ncp;
                        q[0] = og[0];
                        q[Rr * 2 * ncp] = ou[0];
                    }
                }
            }
        }
        lds_barrier();
        for (int i = tid; i < Rr * 2; i += kGemvThreads) {
            const int rr = i >> 1, t = i & 1;
            const int f = it.f0 + rr;
            if (f >= it.rows || t >= nt) continue;
            const float gv = sum_columns4(lds + ((0 * Rr + rr) * 2 + t) * ncp, ncol);
            const float uv = sum_columns4(lds + ((1 * Rr + rr) * 2 + t) * ncp, ncol);
            const float av = act_gate(gv, p.act) * uv;
            const int orow = it.first + t0 + t;   // routed: sorted pair; shared: token
            __hip_atomic_store(it.out + (size_t)orow * it.rows + f, pack_a(av), __ATOMIC_RELAXED,
                               __HIP_MEMORY_SCOPE_AGENT);
        }
        lds_barrier();   // the partials are reused by the next pair
    }
    // Count the tile without waiting, for its stores or for the count: a
    // reader that sees the group complete before a word of `a` has landed
    // reads the word again (it is still 0).
    if (tid == 0) atomic_add_detached(win_gu_count(p.sync, it.g), 1);
}

// Items blockIdx.x, + n_wg, ...: the next item's codes are loaded before
// the current one is computed (two buffers in turn), so that its loads
// overlap the compute.  With no next item, one chunk is read.
template <int QT, int NTERM>
__device__ __forceinline__ void gateup_window(const WindowParams& p, const WinLDS& R, float* lds) {
    constexpr int QK = QTraits<QT>::QK, SW = SliceWords<QT, NTERM>::N;
    const int tid = threadIdx.x;
    const int n_routed = __builtin_amdgcn_readfirstlane(R.n_groups * R.tiles_gu);
    const int n_items =
        n_routed + (p.FFs ? (p.T + kWinGroup - 1) / kWinGroup * __builtin_amdgcn_readfirstlane(R.tiles_gu_s) : 0);
    const int nblk = p.H / QK;
    const int P = kGemvThreads / nblk;
    const bool active = tid < P * nblk;
    const int rp = active ? tid / nblk : 0, b = active ? tid - (tid / nblk) * nblk : 0;
    const int gp = __builtin_amdgcn_readfirstlane(R.gu_passes);
    const int Rr = P * gp;
    int item = blockIdx.x;
    if (item >= n_items) return;
    // Every token's activation slice of every block column, once per
    // workgroup, while the first item's weights are on their way: the words of
    // a thread's first two slices (bf16) are loaded before the weights, so
    // that arranging them waits for them alone.
    const bool pre = NTERM == 1 && p.x_off >= 0;
    const int n_x = p.T * nblk;
    uint32_t xr[2][QK / 2];
    if (pre) {
#pragma unroll
        for (int i = 0; i < 2; ++i) {
            const int sx = min(tid + kGemvThreads * i, n_x - 1);
            const int t = sx / nblk, bb = sx - t * nblk;
            const uint4* src = reinterpret_cast<const uint4*>((const uint16_t*)p.x + (size_t)t * p.H + bb * QK);
#pragma unroll
            for (int v = 0; v < QK / 8; ++v) {
                const uint4 u = ldg_u4(src + v);
                xr[i][4 * v + 0] = u.x;
                xr[i][4 * v + 1] = u.y;
                xr[i][4 * v + 2] = u.z;
                xr[i][4 * v + 3] = u.w;
            }
        }
    }
    GuItem ia = gu_item(p, R, item, n_routed, Rr), ib;
    GuCodes ca, cb;
    gu_load(ia, nblk, P, gp, rp, b, ca);
    if (p.x_off >= 0) {
        uint32_t* xsl = reinterpret_cast<uint32_t*>(lds) + p.x_off;
        if (pre) {
#pragma unroll
            for (int i = 0; i < 2; ++i) {
                const int sx = tid + kGemvThreads * i;
                if (sx < n_x) {
                    XSlice<QT, NTERM> x1;
                    arrange_pairs<QT>(xr[i], x1.pr[0]);
                    finish_slice<QT, NTERM>(x1, p.z);
                    slice_to_lds<QT, NTERM>(x1, xsl + sx * SW);
                }
            }
        }
        for (int s = tid + (pre ? 2 * kGemvThreads : 0); s < n_x; s += kGemvThreads) {
            const int t = s / nblk, bb = s - t * nblk;
            XSlice<QT, NTERM> x1;
            if constexpr (NTERM == 1)
                load_slice_bf16<QT, 1>(x1, (const uint16_t*)p.x + (size_t)t * p.H + bb * QK, nullptr, p.z);
            else
                load_slice_f32<QT>(x1, (const float*)p.x + (size_t)t * p.H + bb * QK, p.z);
            slice_to_lds<QT, NTERM>(x1, xsl + s * SW);
        }
    }
    __syncthreads();
    while (true) {
        int next = item + p.n_wg;
        ib = gu_item(p, R, next < n_items ? next : item, n_routed, Rr);
        ib.none = next >= n_items;
        gu_load(ib, nblk, P, gp, rp, b, cb);
        gu_compute<QT, NTERM>(p, R, ia, ca, lds, nblk, P, gp, rp, b, active);
        if (next >= n_items) break;
        item = next;
        next = item + p.n_wg;
        ia = gu_item(p, R, next < n_items ? next : item, n_routed, Rr);
        ia.none = next >= n_items;
        gu_load(ia, nblk, P, gp, rp, b, ca);
        gu_compute<QT, NTERM>(p, R, ib, cb, lds, nblk, P, gp, rp, b, active);
        if (next >= n_items) break;
        item = next;
    }
}

// Four published fp32 words, read agent-coherently.
typedef uint32_t win_u32x4 __attribute__((ext_vector_type(4)));
__device__ __forceinline__ win_u32x4 load_coherent4(__amdgpu_buffer_rsrc_t rsrc, uint32_t off) {
    return __builtin_amdgcn_raw_buffer_load_b128(rsrc, (int)off, 0, kCpolSc1);
}

__device__ __forceinline__ uint32_t min4(win_u32x4 v) { return min(min(v[0], v[1]), min(v[2], v[3])); }

// Read again, until no word is 0, four words that showed a 0 (written, but
// not yet visible here).
// A wait that gives up leaves NaN in the words (and the error flagged).
__device__ __forceinline__ win_u32x4 reload_published4(const WindowParams& p, __amdgpu_buffer_rsrc_t rsrc,
                                                    uint32_t off) {
    win_u32x4 v = load_coherent4(rsrc, off);
    const bool ok = bounded_wait(
        [&]() __attribute__((always_inline)) {
            if (min4(v) != 0u) return true;
            v = load_coherent4(rsrc, off);
            return false;
        },
        p.polls, p.err);
    if (!ok) v = win_u32x4{kNaNBits, kNaNBits, kNaNBits, kNaNBits};
    return v;
}

__device__ __forceinline__ float4 as_float4(win_u32x4 v) {
    return make_float4(__uint_as_float(v[0]), __uint_as_float(v[1]), __uint_as_float(v[2]), __uint_as_float(v[3]));
}

// Pairwise sum of v[0..N) in natural order: ((v0 + v1) + (v2 + v3)) + ...,
// the association that row_sum_f32 leaves in lane 0 for N = 16 (each of its
// DPP steps adds lanes i and i ^ 1, i ^ 2, then the mirrored halves, and
// every single addition is commutative).
template <int N>
__device__ __forceinline__ float pairwise_sum(const float* v) {
    if constexpr (N == 1) return v[0];
    else return pairwise_sum<N / 2>(v) + pairwise_sum<N / 2>(v + N / 2);
}

// Sum over slots [j0, j0 + 16) of cw[t][j] * d[t * k + j] for 4 consecutive
// rows h.. (0 past k and, with caller-supplied routing, for a skipped slot,
// whose d is never written), pairwise in slot order; all 16 loads in flight
// together, then one check (a word still 0 is read again).
template <bool ROUTED>
__device__ __forceinline__ void slot_sums16(const WindowParams& p, const WinLDS& R, __amdgpu_buffer_rsrc_t rsrc, int t,
                                            int h, int j0, float (&out)[4]) {
    const int k = p.k;
    win_u32x4 raw[16];
    bool on[16];
#pragma unroll
    for (int j = 0; j < 16; ++j) {
        on[j] = j0 + j < k && (!ROUTED || R.on[t * k + j0 + j]);
        const int jj = j0 + j < k ? j0 + j : 0;   // past k: slot 0 again, unused
        raw[j] = load_coherent4(rsrc, 4u * (uint32_t)((t * k + jj) * p.H + h));
        if (ROUTED && !on[j]) raw[j] = win_u32x4{1u, 1u, 1u, 1u};
    }
    uint32_t m = 0xFFFFFFFFu;
#pragma unroll
    for (int j = 0; j < 16; ++j) m = min(m, min4(raw[j]));
    if (m == 0u) {
#pragma unroll
        for (int j = 0; j < 16; ++j)
            if (on[j] && min4(raw[j]) == 0u)
                raw[j] = reload_published4(p, rsrc, 4u * (uint32_t)((t * k + j0 + j) * p.H + h));
    }
#pragma unroll
    for (int e = 0; e < 4; ++e) {
        float v[16];
#pragma unroll
        for (int j = 0; j < 16; ++j) v[j] = on[j] ? R.cw[t * k + j0 + j] * __uint_as_float(raw[j][e]) : 0.f;
        out[e] = pairwise_sum<16>(v);
    }
}

// y rows [h0, h0 + 4 n4) of every token: shared + sum_j w[t][j] d[t * k + j],
// the slot terms added as the one-token kernel adds them (lane j of a group
// of 16 or 32 lanes holds slot j's term, 0 past k, and a DPP tree sums the
// group: pairwise in slot order), so a token's output is the same alone and
// inside a window; the shared term is added last.  Each thread takes 4
// consecutive rows of one token.  The d words read are cleared for the next
// call.
template <bool ROUTED>
__device__ __forceinline__ void combine_rows(const WindowParams& p, const WinLDS& R, int h0, int n4) {
    const int k = p.k;
    const int nq = p.T * n4;
    const bool failed = R.fail;
    const __amdgpu_buffer_rsrc_t rsrc =
        __builtin_amdgcn_make_buffer_rsrc((void*)p.d, 0, (kSmallT * k + kSmallT) * p.H * 4, kRsrcWord3);
    for (int qd = threadIdx.x; qd < nq; qd += kGemvThreads) {
        const int t = qd / n4, h = h0 + 4 * (qd - t * n4);
        float acc[4];
        slot_sums16<ROUTED>(p, R, rsrc, t, h, 0, acc);
        if (k > 16) {
            float hi[4];
            slot_sums16<ROUTED>(p, R, rsrc, t, h, 16, hi);
#pragma unroll
            for (int e = 0; e < 4; ++e) acc[e] = acc[e] + hi[e];
        }
        if (p.FFs) {
            const uint32_t off = 4u * (uint32_t)((kSmallT * k + t) * p.H + h);
            win_u32x4 sv = load_coherent4(rsrc, off);
            if (min4(sv) == 0u) sv = reload_published4(p, rsrc, off);
#pragma unroll
            for (int e = 0; e < 4; ++e) acc[e] = __uint_as_float(sv[e]) + acc[e];
        }
        if (failed) acc[0] = acc[1] = acc[2] = acc[3] = __uint_as_float(kNaNBits);
        *reinterpret_cast<float4*>(p.y + (size_t)t * p.H + h) = make_float4(acc[0], acc[1], acc[2], acc[3]);
        const uint4 zero = make_uint4(0u, 0u, 0u, 0u);
        for (int j = 0; j < k; ++j) *reinterpret_cast<uint4*>(p.d + (size_t)(t * k + j) * p.H + h) = zero;
        if (p.FFs) *reinterpret_cast<uint4*>(p.d + (size_t)(kSmallT * k + t) * p.H + h) = zero;
    }
}

// One down item: group (or the shared expert) and chunk (or sub-range).
struct DnItem {
    const uint8_t* dcode;
    const uint8_t* dscale;
    const uint32_t* a_src;
    int g, ch, h0, nrows, first, n_e, K, group_items;
    bool sh;
    bool none;   // no item: its loads read one chunk
};

template <int QK>
__device__ __forceinline__ DnItem dn_item(const WindowParams& p, const WinLDS& R, int item, int n_routed) {
    DnItem it;
    it.sh = item >= n_routed;
    const uint8_t* blob;
    if (!it.sh) {
        const int gi = item / p.n_chunks;
        it.g = R.gorder[gi];
        it.ch = item - gi * p.n_chunks;
        it.h0 = it.ch * p.chunk_rows;
        it.nrows = min(p.chunk_rows, p.H - it.h0);
        it.first = R.group_first[it.g];
        it.n_e = R.group_first[it.g + 1] - it.first;
        blob = p.table ? table_blob(p.table, R.id[R.sorted[it.first]]) : p.single;
        it.K = p.FF;
        it.a_src = p.a + (size_t)it.first * p.FF;
        it.group_items = p.n_chunks;
    } else {
        const int per_sg = p.n_chunks * p.sh_items;
        const int sg = (item - n_routed) / per_sg;
        const int i2 = item - n_routed - sg * per_sg;
        it.ch = i2 / p.sh_items;
        const int sub = i2 - it.ch * p.sh_items;
        const int c0 = it.ch * p.chunk_rows, c1 = min(c0 + p.chunk_rows, p.H);
        it.h0 = c0 + sub * p.sh_rows;
        it.nrows = min(p.sh_rows, c1 - it.h0);   // <= 0: an empty sub-range, still counted
        it.g = kSmallT * p.k + sg;
        it.first = kWinGroup * sg;
        it.n_e = min(kWinGroup, p.T - it.first);
        blob = p.shared;
        it.K = p.FFs;
        it.a_src = p.as + (size_t)it.first * p.FFs;
        it.group_items = per_sg;
    }
    const int nb = it.K / QK;
    it.dcode = blob + (size_t)2 * it.K * (p.H / QK) * kBlockBytes;   // after gate and up
    it.dscale = it.dcode + (size_t)p.H * nb * 16;
    it.none = false;
    return it;
}

struct DnCodes {
    uint4 c[kWinMaxPass];
    uint16_t sc[kWinMaxPass];
};

// Thread (rp, b) of an item: row rp of each pass of P = 256 / nb rows, block
// column b.
struct DnLane {
    int nb, P, rp, b;
    bool active;
};

__device__ __forceinline__ DnLane dn_lane(int K, int QK) {
    DnLane l;
    l.nb = K / QK;
    l.P = kGemvThreads / l.nb;
    const int tid = threadIdx.x;
    l.active = tid < l.P * l.nb;
    l.rp = l.active ? tid / l.nb : 0;
    l.b = l.active ? tid - l.rp * l.nb : 0;
    return l;
}

// Every pass's down codes at once, from clamped rows (an item of fewer passes
// re-reads its last row): all loads in flight together, no branch per pass.
__device__ __forceinline__ void dn_load(const WindowParams& p, const DnItem& it, const DnLane& l, DnCodes& c) {
    const int rlast = max(it.nrows, 1) - 1;
#pragma unroll
    for (int m = 0; m < kWinMaxPass; ++m) {
        const int r = min(l.rp + m * l.P, rlast);
        const size_t blk = it.none ? 0 : (size_t)(min(it.h0 + r, p.H - 1)) * l.nb + l.b;
        c.c[m] = it.sh ? ldg_u4(it.dcode + blk * 16) : ldg_u4_nt(it.dcode + blk * 16);
        c.sc[m] = ldg_u16(it.dscale + blk * 2);
    }
}

// Thread 0, before the workgroup's first wait: whether the error word holds
// an unchecked failure of an earlier call (R.prior).  The load is issued
// after the item's weight loads, whose arrival the first poll waits for
// anyway, so it costs no time.
__device__ __forceinline__ bool prior_failure(const WindowParams& p, WinLDS& R) {
    if (R.prior < 0) R.prior = load_error(p.err) != 0;
    return R.prior != 0;
}

// Wait for the group's gate/up and take its `a` rows (nothing on an earlier
// failure).
template <int QK>
__device__ __forceinline__ void dn_begin(const WindowParams& p, WinLDS& R, const DnItem& it, float* lds) {
    if (threadIdx.x == 0 && !prior_failure(p, R)) {
        const int need = __builtin_amdgcn_readfirstlane(it.sh ? R.tiles_gu_s : R.tiles_gu);
        const int* cnt = win_gu_count(p.sync, it.g);
        if (!bounded_wait([&]() __attribute__((always_inline)) { return __hip_atomic_load(cnt, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) >= need; },
                          p.polls, p.err))
            R.fail = 1;
    }
    __syncthreads();
    if (R.prior > 0) return;
    if (p.stage_words) {
        // Each slice (token i, block column b) once, arranged into dot pairs
        // of its hi and lo terms in LDS for every thread of column b.
        constexpr int QT = QK == 64 ? 1 : 2, SW = SliceWords<QT, 2>::N;
        const int nb = it.K / QK;
        const __amdgpu_buffer_rsrc_t a_rsrc =
            __builtin_amdgcn_make_buffer_rsrc((void*)it.a_src, 0, it.n_e * it.K * 4, kRsrcWord3);
        for (int sl = threadIdx.x; sl < it.n_e * nb; sl += kGemvThreads) {
            uint32_t w[QK];
            // slice sl = i * nb + b starts at word i * K + b * QK = sl * QK
            long n = 0;
            while (!load_packed_words<QT>(w, a_rsrc, 4u * (uint32_t)(sl * QK)) || p.polls == 0) {
                if (++n > p.polls) {   // a bound of 0 gives up at once
                    flag_error(p.err, kErrTimeout);
                    R.fail = 1;
                    break;
                }
                __builtin_amdgcn_s_sleep(1);
            }
            XSlice<QT, 2> xs;
            slice_from_packed<QT>(xs, w, p.z);
            slice_to_lds<QT, 2>(xs, reinterpret_cast<uint32_t*>(lds) + sl * SW);
        }
    }
    __syncthreads();
}

// Run the item's tokens through the held codes and publish d; count the item,
// and combine the chunk or clear the group's state when this item is the
// last of either.
template <int QT>
__device__ __forceinline__ void dn_finish(const WindowParams& p, WinLDS& R, const DnItem& it, const DnLane& l,
                                          DnCodes& c, float* lds, int& old_dn) {
    constexpr int QK = QTraits<QT>::QK, SW = SliceWords<QT, 2>::N;
    const int tid = threadIdx.x;
    float* part = lds + p.stage_words;
    const __amdgpu_buffer_rsrc_t a_rsrc =
        __builtin_amdgcn_make_buffer_rsrc((void*)it.a_src, 0, it.n_e * it.K * 4, kRsrcWord3);
    // With the rows staged, this item holds its `a`: count it now; else after
    // the compute.
    if (p.stage_words && tid == 0)
        old_dn = __hip_atomic_fetch_add(win_dn_count(p.sync, it.g), 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    const int nbp = (l.nb + 3) & ~3;
    for (int t0 = 0; t0 < it.n_e; t0 += 2) {
        const int nt = min(2, it.n_e - t0);
        // One token at a time (its slice in registers), two per round of
        // partial sums.
#pragma unroll 1
        for (int i = 0; i < nt; ++i) {
#pragma unroll
            for (int m = 0; m < kWinMaxPass; ++m) pin_u4(c.c[m]);
            const int sl = (t0 + i) * l.nb + l.b;
            XSlice<QT, 2> xs[1];
            if (p.stage_words) {
                slice_from_lds<QT, 2>(xs[0], reinterpret_cast<const uint32_t*>(lds) + sl * SW);
            } else {
                // Rows too large for LDS: straight from `a`, again while a word
                // is still 0.
                uint32_t w[QK];
                long n = 0;
                while (!load_packed_words<QT>(w, a_rsrc, 4u * (uint32_t)(sl * QK)) || p.polls == 0) {
                    if (++n > p.polls) {   // a bound of 0 gives up at once
                        flag_error(p.err, kErrTimeout);
                        R.fail = 1;
                        break;
                    }
                    __builtin_amdgcn_s_sleep(1);
                }
                slice_from_packed<QT>(xs[0], w, p.z);
            }
#pragma unroll
            for (int m = 0; m < kWinMaxPass; ++m) {
                const int r = l.rp + m * l.P;
                if (l.active && r < it.nrows) {   // r < nrows <= P * passes
                    float o[1];
                    block_dot<QT, 2, 1>(c.c[m], scale_at_use(c.sc[m]), xs, 1, o);
                    part[(r * 2 + i) * nbp + l.b] = o[0];
                }
            }
        }
        lds_barrier();
        const bool failed = R.fail;
        for (int i = tid; i < it.nrows * 2; i += kGemvThreads) {
            const int r = i >> 1, t = i & 1;
            if (t >= nt) continue;
            const float v = sum_columns(part + (r * 2 + t) * nbp, l.nb);
            const int drow = it.sh ? kSmallT * p.k + it.first + t0 + t : R.sorted[it.first + t0 + t];
            __hip_atomic_store(p.d + (size_t)drow * p.H + it.h0 + r, failed ? kNaNBits : nonzero_bits(v),
                               __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        }
        // The partials are reused by the next pair.  The barrier does not
        // wait for the d stores (nor for the next item's code loads issued
        // before this item): the combine that the count below may start
        // reads a word again while it is still 0.
        lds_barrier();
    }
    // Count the item in its chunk (its d words are issued) and, without
    // staged rows, in its group; the group count is looked at in dn_settle.
    if (tid == 0) {
        if (!p.stage_words)
            old_dn = __hip_atomic_fetch_add(win_dn_count(p.sync, it.g), 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        atomic_add_detached(win_chunk(p.sync, p.k, it.ch), 1);
    }
}

// After an item's group count has returned (thread 0 holds it): clear the
// group's state if the item was the group's last to take its `a` rows.
__device__ __forceinline__ void dn_settle(const WindowParams& p, WinLDS& R, const DnItem& it, int old_dn) {
    const int tid = threadIdx.x;
    if (tid == 0) R.flag_reset = old_dn == it.group_items - 1;
    __syncthreads();
    if (R.flag_reset) {
        // Every item of the group holds its `a` rows: clear them, and the
        // group's counters.
        for (int i = tid; i < it.n_e * it.K; i += kGemvThreads)
            __hip_atomic_store(const_cast<uint32_t*>(it.a_src) + i, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        if (tid == 0) {
            __hip_atomic_store(win_gu_count(p.sync, it.g), 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            __hip_atomic_store(win_dn_count(p.sync, it.g), 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        }
    }
    __syncthreads();   // the flags are written again by the next settle
}

// Items n_wg - 1 - blockIdx.x, + n_wg, ...: the next item's codes are
// loaded once the current one's `a` rows are in LDS (the staging waits for
// every load of the workgroup), before its compute.
template <int QT>
__device__ __forceinline__ void down_window(const WindowParams& p, WinLDS& R, float* lds) {
    constexpr int QK = QTraits<QT>::QK;
    const int n_routed = R.n_groups * p.n_chunks;
    const int n_sg = p.FFs ? (p.T + kWinGroup - 1) / kWinGroup : 0;
    const int n_items = n_routed + n_sg * p.n_chunks * p.sh_items;
    // Down items go to the workgroups in reverse order: those with the most
    // gate/up items (the low indices) get the fewest down items.
    const int first_item = p.n_wg - 1 - (int)blockIdx.x;
    int item = first_item;
    if (item >= n_items) return;
    DnItem ia = dn_item<QK>(p, R, item, n_routed), ib;
    DnLane la = dn_lane(ia.K, QK), lb;
    DnCodes ca, cb;
    dn_load(p, ia, la, ca);
    // Counts of the previous item (thread 0), settled after the next item's
    // `a` rows are in LDS.
    int od_a = 0, od_b = 0;
    while (true) {
        int next = item + p.n_wg;
        dn_begin<QK>(p, R, ia, lds);
        if (R.prior > 0) return;
        if (item != first_item) dn_settle(p, R, ib, od_b);
        ib = dn_item<QK>(p, R, next < n_items ? next : item, n_routed);
        ib.none = next >= n_items;
        lb = dn_lane(ib.K, QK);
        dn_load(p, ib, lb, cb);
        dn_finish<QT>(p, R, ia, la, ca, lds, od_a);
        if (next >= n_items) {
            dn_settle(p, R, ia, od_a);
            break;
        }
        item = next;
        next = item + p.n_wg;
        dn_begin<QK>(p, R, ib, lds);
        if (R.prior > 0) return;
        dn_settle(p, R, ia, od_a);
        ia = dn_item<QK>(p, R, next < n_items ? next : item, n_routed);
        ia.none = next >= n_items;
        la = dn_lane(ia.K, QK);
        dn_load(p, ia, la, ca);
        dn_finish<QT>(p, R, ib, lb, cb, lds, od_b);
        if (next >= n_items) {
            dn_settle(p, R, ib, od_b);
            break;
        }
        item = next;
    }
}

// The combine, once a chunk's down items are all counted, split into parts of
// its rows over several workgroups (each workgroup's loads in flight are
// bounded, so one workgroup per chunk would take several round trips): part
// slots s = w, w + G, ... of n_chunks * hp (hp parts per chunk).  A
// workgroup's own down items are done before it waits, and the items it waits
// for never wait for it.  The last part of a chunk to see it complete clears
// the chunk's counters.
__device__ __forceinline__ void combine_window(const WindowParams& p, WinLDS& R) {
    const int n_sg = p.FFs ? (p.T + kWinGroup - 1) / kWinGroup : 0;
    const int need_chunk = R.n_groups + n_sg * p.sh_items;
    const int hp = max(1, min(kWinCombineParts, p.n_wg / p.n_chunks));
    for (int sl = blockIdx.x; sl < p.n_chunks * hp; sl += p.n_wg) {
        const int c = sl / hp, part = sl - c * hp;
        const int c0 = c * p.chunk_rows, nr4 = (min(c0 + p.chunk_rows, p.H) - c0) / 4;
        const int q0 = part * nr4 / hp, q1 = (part + 1) * nr4 / hp;
        if (threadIdx.x == 0 && !prior_failure(p, R)) {
            const int* cnt = win_chunk(p.sync, p.k, c);
            if (!bounded_wait(
                    [&]() __attribute__((always_inline)) { return __hip_atomic_load(cnt, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) >= need_chunk; },
                    p.polls, p.err))
                R.fail = 1;
        }
        __syncthreads();
        if (R.prior > 0) return;
        // Count this part as one that has seen the chunk complete (no part
        // looks at the chunk's counter after that); the count returns while
        // the rows are combined.
        int old = 0;
        if (threadIdx.x == 0)
            old = __hip_atomic_fetch_add(win_combined(p.sync, p.k, p.n_chunks, c), 1, __ATOMIC_RELAXED,
                                         __HIP_MEMORY_SCOPE_AGENT);
        __syncthreads();
        if (p.ids_in) combine_rows<true>(p, R, c0 + 4 * q0, q1 - q0);
        else combine_rows<false>(p, R, c0 + 4 * q0, q1 - q0);
        if (threadIdx.x == 0) {
            if (old == hp - 1) {
                __hip_atomic_store(win_chunk(p.sync, p.k, c), 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                __hip_atomic_store(win_combined(p.sync, p.k, p.n_chunks, c), 0, __ATOMIC_RELAXED,
                                   __HIP_MEMORY_SCOPE_AGENT);
            }
        }
    }
}

template <int QT, int NTERM>
__global__ void __launch_bounds__(kGemvThreads, 2) window_layer_kernel(WindowParams p) {
    extern __shared__ __align__(16) float lds[];
    __shared__ WinLDS R;
    route_window(p, R, reinterpret_cast<uint64_t*>(lds), kGemvThreads / (p.H / QTraits<QT>::QK));
    if (blockIdx.x == 0) {
        for (int q = threadIdx.x; q < p.T * p.k; q += kGemvThreads) {
            if (p.ids_out) p.ids_out[q] = R.id[q];
            if (p.w_out) p.w_out[q] = R.w[q];
        }
    }
    if (!R.bad) {
        gateup_window<QT, NTERM>(p, R, lds);
        down_window<QT>(p, R, lds);
        if (R.prior <= 0) combine_window(p, R);
        // A workgroup without a down item or combine part looks too, so that
        // on an earlier failure every workgroup writes its share of NaN rows.
        if (threadIdx.x == 0) prior_failure(p, R);
        __syncthreads();
    }
    if (R.bad || R.prior > 0) {
        // Invalid caller-supplied routing, or an unchecked earlier failure
        // (stale shared state: no wait ran on it): every output row is NaN.
        for (int q = blockIdx.x * kGemvThreads + threadIdx.x; q < p.T * p.H; q += p.n_wg * kGemvThreads)
            p.y[q] = __uint_as_float(kNaNBits);
    }
}

// ---------------------------------------------------------------------------------------------
// Host side.
// ---------------------------------------------------------------------------------------------
constexpr size_t kWinLdsMax = 100 * 1024;   // dynamic LDS beyond which slices and `a` are read from memory

WindowShape window_shape(int H, int FF, int FFs, int qtype, int x_dtype, int T, int k) {
    WindowShape g{};
    const int qk = codes_per_block(qtype);
    const int nblk = H / qk, P = kGemvThreads / nblk;
    const int nb_r = FF / qk, P_r = kGemvThreads / nb_r;
    // Activation slice words per block column (SliceWords): dot pairs of one
    // (bf16) or two (fp32) terms, the per-q offsets and z * sum x.
    const int nterm = x_dtype == 1 ? 1 : 2;
    const int sw = (nterm * qk / 2 + (qk == 64 ? 3 : 1) + 1 + 3) & ~3;
    const size_t x_bytes = (size_t)T * nblk * sw * 4;
    // The largest gate/up tiling: it sizes the partials and bounds the items
    // (the kernel picks the pass count of each call from its groups, gu_tiling).
    g.gu_passes = kWinMaxPass;
    const int rows_gu = P * g.gu_passes;
    g.tiles_gu = (FF + rows_gu - 1) / rows_gu;
    g.tiles_gu_s = FFs ? (FFs + rows_gu - 1) / rows_gu : 0;
    const int ncol = nblk % 2 == 0 ? nblk / 2 : nblk;
    const size_t part_gu = (size_t)2 * rows_gu * 2 * ((ncol + 3) & ~3) * 4;
    g.x_off = (int)(part_gu / 4);
    // Every token's slices in LDS unless that would pass the budget; then each
    // token's slice is read from the activations where it is used.
    const bool x_lds = part_gu + x_bytes <= kWinLdsMax;
    if (!x_lds) g.x_off = -1;
    const size_t lds_gu = part_gu + (x_lds ? x_bytes : 0);
    // Down: chunks of 8 passes of the routed experts' rows; the shared
    // expert covers a chunk in sub-ranges of at most 8 passes.
    g.dn_passes = kWinMaxPass;
    g.chunk_rows = P_r * g.dn_passes;
    g.n_chunks = (H + g.chunk_rows - 1) / g.chunk_rows;
    size_t part_dn = (size_t)g.chunk_rows * 2 * ((nb_r + 3) & ~3) * 4;
    if (FFs) {
        const int nb_s = FFs / qk, P_s = kGemvThreads / nb_s;
        const int ps = (g.chunk_rows + P_s - 1) / P_s;
        g.sh_passes = ps > kWinMaxPass ? kWinMaxPass : ps;
        g.sh_rows = P_s * g.sh_passes;
        g.sh_items = (g.chunk_rows + g.sh_rows - 1) / g.sh_rows;
        const size_t pss = (size_t)g.sh_rows * 2 * ((nb_s + 3) & ~3) * 4;
        part_dn = pss > part_dn ? pss : part_dn;
    }
    // One group's `a` rows as arranged slices (hi and lo dot pairs, the
    // per-q offsets and z * sum: SliceWords), unless they would pass the
    // budget; then each thread reads its slices from `a`.
    const int sw2 = (qk + (qk == 64 ? 3 : 1) + 1 + 3) & ~3;
    const long slices = (long)(T < kWinGroup ? T : kWinGroup) * ((FF > FFs ? FF : FFs) / qk);
    g.stage_words = (int)(slices * sw2);
    if ((size_t)g.stage_words * 4 + part_dn > kWinLdsMax) g.stage_words = 0;
    const size_t lds_dn = (size_t)g.stage_words * 4 + part_dn;
    g.lds_bytes = lds_gu > lds_dn ? lds_gu : lds_dn;
    const size_t topk_scratch = (size_t)kGemvThreads / 64 * 128 * 8;   // the routing's, before any of the above
    if (g.lds_bytes < topk_scratch) g.lds_bytes = topk_scratch;
    const int n_sg = FFs ? (T + kWinGroup - 1) / kWinGroup : 0;
    const int max_gu = T * k * g.tiles_gu + n_sg * g.tiles_gu_s;
    const int max_dn = T * k * g.n_chunks + n_sg * g.n_chunks * g.sh_items;
    g.max_items = max_gu > max_dn ? max_gu : max_dn;
    g.grid = 0;   // set at launch from the GPU's capacity
    return g;
}

size_t window_sync_bytes(int k, int n_chunks) {
    return (size_t)64 * (2 + 2 * (kSmallT * k + kWinShared) + 2 * n_chunks);
}

template <int QT, int NTERM>
static hipError_t launch_window_t(const WindowShape& g, const WindowParams& p, hipStream_t s) {
    // (the grid is p.n_wg, see window_grid; window_capacity has allowed the LDS)
    hipLaunchKernelGGL((window_layer_kernel<QT, NTERM>), dim3(p.n_wg), dim3(kGemvThreads), g.lds_bytes, s, p);
    return hipGetLastError();
}

// Workgroups the current GPU holds at once for this instantiation and LDS
// size (the kernel's registers and LDS decide), times its CUs.  Cached per
// (device, LDS size); the cache is shared by every thread of the process.
template <int QT, int NTERM>
static hipError_t window_capacity(size_t lds_bytes, int* out) {
    static std::mutex mu;
    static std::map<std::pair<int, size_t>, int> cache;
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    std::lock_guard<std::mutex> lock(mu);
    auto it = cache.find({dev, lds_bytes});
    if (it == cache.end()) {
        e = hipFuncSetAttribute((const void*)window_layer_kernel<QT, NTERM>, hipFuncAttributeMaxDynamicSharedMemorySize,
                                148 * 1024);
        if (e != hipSuccess) return e;
        int n_cu = 0, per_cu = 0;
        e = hipDeviceGetAttribute(&n_cu, hipDeviceAttributeMultiprocessorCount, dev);
        if (e != hipSuccess) return e;
        e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, (const void*)window_layer_kernel<QT, NTERM>,
                                                         kGemvThreads, lds_bytes);
        if (e != hipSuccess) return e;
        it = cache.emplace(std::make_pair(dev, lds_bytes), per_cu * n_cu).first;
    }
    *out = it->second;
    return hipSuccess;
}

static hipError_t window_grid(const WindowShape& g, int qtype, int x_dtype, int* grid) {
    int cap = 0;
    hipError_t e;
    const bool bf = x_dtype == 1;
    if (qtype == 1)
        e = bf ? window_capacity<1, 1>(g.lds_bytes, &cap) : window_capacity<1, 2>(g.lds_bytes, &cap);
    else
        e = bf ? window_capacity<2, 1>(g.lds_bytes, &cap) : window_capacity<2, 2>(g.lds_bytes, &cap);
    if (e != hipSuccess) return e;
    if (cap < 1) return hipErrorInvalidConfiguration;
    *grid = g.max_items < cap ? g.max_items : cap;
    return hipSuccess;
}

hipError_t launch_window_layer(const WindowShape& g, const void* const* table, const void* single,
                               const void* shared, const void* x, int x_dtype, const float* logits, int T, int E,
                               int k, int renorm, int identity, const LayerOpts& o, int qtype, float z, int H, int FF,
                               int FFs, int* ids_out, float* w_out, const SmallLayout& L, char* ws, float* y,
                               hipStream_t s, StageMarks* marks) {
    WindowParams p{};
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
    p.H = H;
    p.FF = FF;
    p.FFs = FFs;
    p.z = z;
    p.act = o.act;
    p.down_scale = o.down_scale;
    p.ids_in = o.ids_in;
    p.w_in = o.w_in;
    p.ids_out = ids_out;
    p.w_out = w_out;
    p.a = (uint32_t*)(ws + L.a);
    p.as = (uint32_t*)(ws + L.as);
    p.d = (uint32_t*)(ws + L.d);
    p.y = y;
    p.sync = (int*)(ws + L.sync);
    p.err = p.sync + kErrWord;
    p.polls = wait_polls();
    p.dn_passes = g.dn_passes;
    p.chunk_rows = g.chunk_rows;
    p.n_chunks = g.n_chunks;
    p.sh_passes = g.sh_passes;
    p.sh_rows = g.sh_rows;
    p.sh_items = g.sh_items;
    int grid = 0;
    hipError_t e = window_grid(g, qtype, x_dtype, &grid);
    if (e != hipSuccess) return e;
    p.n_wg = grid;
    p.x_off = g.x_off;
    p.stage_words = g.stage_words;
    stage_mark(marks, s);
    const bool bf = x_dtype == 1;
    if (qtype == 1)
        e = bf ? launch_window_t<1, 1>(g, p, s) : launch_window_t<1, 2>(g, p, s);
    else
        e = bf ? launch_window_t<2, 1>(g, p, s) : launch_window_t<2, 2>(g, p, s);
    stage_mark(marks, s);
    return e;
}

}  // namespace moe
