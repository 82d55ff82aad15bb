// tree_attention_verify: one attention layer of the target's verify pass over
// committed KV plus each node's ancestors, bf16 in / fp32 softmax / bf16 out.
//
// What is computed: the decoding-extensions glossary ("Beam Search、约束解码与
// Tree/Self Speculation"), section "Packed tree attention" and the
// packed-vs-branch experiment: every candidate query sees the whole committed
// prefix and its own ancestor chain (self included), never siblings or
// cousins; candidate Q and K are rotated (interleaved-pair RoPE) at their tree
// positions, committed K is stored already rotated; scores are q.k/sqrt(D).
// "02 · Token Tree 与 Tree Attention" §3 (position = context + depth) and the
// tree-attention verification essay's KV section (the tree's K/V are written
// into one tentative region in node order).
//
// How, on gfx950:
//  1. attn_prep_kernel: workgroup 0 builds the work plan on the device (no
//     host round trip); workgroup 1 + p handles nodes 4p .. 4p + 3 of the
//     batch, one per 128-thread part.  A part computes its node's rotation
//     angles in fp64 (reduced modulo 2 pi before sincos), stores cos and sin
//     times scale * log2(e) as fp32 for the main kernel, rotates K in fp64,
//     rounds it once to bf16 and writes it with V into slot ctx + i.
//  2. attn_main_kernel, persistent, 8 waves: a work item is (request, KV
//     head, row tile of 128 or 256 query rows, slot chunk).  Rows are (node,
//     query head of the GQA group) pairs, node-major, so every context K/V
//     byte feeds all rows of its KV head.  A wave owns one or two 16-row
//     blocks and keeps their Q in registers, rotated in fp32 in the item's
//     prologue.  K and V tiles of 32 slots
//     stream through an LDS ring (up to 6 tiles in flight) by direct
//     global->LDS loads; V stays row-major and is read transposed by
//     ds_read_b64_tr_b16.  S^T = K Q^T and O^T += V^T P^T run on
//     v_mfma_f32_16x16x32_bf16, so P^T comes out of the score accumulators
//     already in the B-operand layout.  Online softmax in fp32 (exp2
//     domain).  The tree part of a row tile rides with its last chunk: tree
//     keys 32 at a time, masked by one word of each row's ancestor mask.
//     The plan deals items to workgroups largest estimated cost first, in
//     snake order, so the workgroups finish close together; the row tiles of
//     one slot chunk stay consecutive and land on one XCD (blockIdx ->
//     XCD-major virtual id), where their repeated K/V reads can hit that
//     XCD's L2.
//  3. attn_combine_kernel: log-sum-exp merge of the chunks of row tiles whose
//     context was split; single-chunk tiles are written directly by step 2.

#include <algorithm>
#include <atomic>
#include <type_traits>

#include "ttv_device.h"

namespace {

constexpr int kWaves = 8;               // waves of the largest row tile
constexpr int kRowsPerWave = 32;        // query rows per wave: kMB blocks of 16
constexpr int kMB = kRowsPerWave / 16;
constexpr int kTileM = kWaves * kRowsPerWave;   // largest row tile (8 waves x 32 rows)
constexpr int kTileMin = 128;                       // row tile of small batches (16 rows per wave)
constexpr int kPrepWaves = 8;           // prep workgroups (plan and node rotation)
constexpr int kPrepThreads = kPrepWaves * TTV_WAVE;
constexpr int kPrepNodes = 4;           // tree nodes per prep workgroup (one per 128 threads)
constexpr int kKT = 32;                 // key slots per LDS tile (= one mask word)
constexpr int kTargetItems = 448;       // chunking aims at about this many work items (batched
                                        // serving: 448 about 4 % faster than 640, 1024 or more 15-25 % slower)
constexpr int kChunkMin = 128;          // shortest context chunk (slots)
constexpr int kMaxBatch = 4096;         // plan keeps per-request prefix sums in LDS
constexpr int kNumXcd = 8;
constexpr int kMaxGrid = 1024;          // main-kernel workgroups at most (one per CU)
constexpr int kCostBuckets = 1024;      // plan's bucket sort of item costs (32 per octave)
constexpr int kPreciseCtx = 256;        // requests with a shorter context run every tile precise
constexpr int kCombThreads = 256;       // combine workgroup
constexpr int kCombBatch = 8;           // chunk partials a combine thread loads before using any
constexpr int kClaimLead = 4;           // tiles before an item's end at which the next is claimed
constexpr float kLazyRescale = 8.0f;    // log2 headroom before the running max is moved
constexpr float kNegBig = -1.0e30f;
// Tile classes of the attention loop (see attn_main_kernel).
constexpr int kClassPlain = 0;
constexpr int kClassMasked = 1;
constexpr int kClassPrecise = 2;

// RoPE inverse frequencies base^(-2m/D), m < D/2, computed on the host in
// double and passed by value.
struct RopeTable {
    double inv[64];
};

struct PlanHeader {
    int32_t n_items;
    int32_t n_combine;
    int32_t chunk_len;
    int32_t queue[kNumXcd];  // per-XCD work-queue cursors of the main kernel
    int32_t reserved[53];
};

typedef __bf16 ttv_bf16x2v __attribute__((ext_vector_type(2)));
typedef float ttv_f32x2v __attribute__((ext_vector_type(2)));

// Two fp64 values to packed bf16 (a in the low half), nearest-even: rounded
// to odd in fp32, then the hardware's packed fp32 -> bf16 conversion.
__device__ __forceinline__ uint32_t pack_bf16_f64(double a, double b) {
    const ttv_f32x2v f = {ttv_f64_to_f32_odd(a), ttv_f64_to_f32_odd(b)};
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(f, ttv_bf16x2v));
}

struct Item {
    int32_t b, kvh, tile, s;
    int32_t n, ctx, c0, c1;
    int32_t kmax, pslot, nc, nt;
};

struct Combine {
    int32_t b, kvh, tile, s;
    int32_t n, pslot0, stride, nc;
};

struct Layout {
    int64_t max_groups, max_items, max_partials;
    size_t off_items, off_combine, off_glist, off_gpos, off_rope, off_po, off_pml, total;
};

size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

Layout make_layout(int64_t B, int64_t T, int64_t Hq, int64_t Hkv, int64_t D) {
    Layout L;
    const int64_t G = Hq / Hkv;
    L.max_groups = Hkv * ((T * G + kTileMin - 1) / kTileMin + B);
    L.max_items = kTargetItems + L.max_groups;
    L.max_partials = 2 * kTargetItems;
    size_t off = align256(sizeof(PlanHeader));
    L.off_items = off;  // slots in workgroup order: up to max_items + one row of the grid
    off = align256(off + (size_t)(L.max_items + kMaxGrid) * sizeof(Item));
    L.off_combine = off;
    off = align256(off + (size_t)L.max_groups * sizeof(Combine));
    L.off_glist = off;  // the plan's groups (first item, bucket), at most one per item
    off = align256(off + (size_t)L.max_items * sizeof(int2));
    L.off_gpos = off;   // each group's first position, at its first item's index
    off = align256(off + (size_t)L.max_items * sizeof(int32_t));
    L.off_rope = off;   // per node: (cos, sin) * scale * log2(e) of each rotation pair, fp32
    off = align256(off + (size_t)T * (D / 2) * sizeof(float2));
    L.off_po = off;
    off = align256(off + (size_t)L.max_partials * kTileM * D * 2);
    L.off_pml = off;
    off = align256(off + (size_t)L.max_partials * kTileM * sizeof(float4));
    L.total = off;
    return L;
}

struct CacheView {
    uint16_t* k;
    uint16_t* v;
    const int32_t* table;
    int32_t paged, hkv, cap, max_blocks, num_blocks;
};

// Element offset of (request b, kv head h, slot) in the cache; -1 if unmapped.
__device__ __forceinline__ int64_t cache_row(const CacheView& c, int b, int h, int slot, int D) {
    if (!c.paged) return (((int64_t)b * c.hkv + h) * c.cap + slot) * D;
    const int lb = slot >> 4;
    if (lb >= c.max_blocks) return -1;
    const int blk = c.table[(int64_t)b * c.max_blocks + lb];
    if (blk < 0 || blk >= c.num_blocks) return -1;
    return (((int64_t)blk * c.hkv + h) * TTV_BLOCK_SIZE + (slot & 15)) * D;
}

// Elements of K (or V) in the cache: the bound of the debug build's checks.
__device__ __forceinline__ int64_t cache_elems(const CacheView& c, int B, int D) {
    return c.paged ? (int64_t)c.num_blocks * c.hkv * TTV_BLOCK_SIZE * D : (int64_t)B * c.hkv * c.cap * D;
}

// ---------------------------------------------------------------------------
// 1. Prep: RoPE of Q (into the workspace) and K (into the cache), V copy, and
//    (one extra workgroup) the work plan.
// ---------------------------------------------------------------------------

// Snake placement over `grid` workgroups (per_xcd = grid / 8 per XCD),
// n_items > grid: full rounds, then m = n_items % grid items in a last round
// that fills positions 0 .. m-1 when its index is even and grid-m .. grid-1
// when odd; position v belongs to XCD v / per_xcd.  XCD x's first filled
// position (as an index inside the XCD) in such an odd round:
__host__ __device__ inline int xcd_first_filled(int grid, int m, int x) {
    const int per_xcd = grid / kNumXcd;
    return min(per_xcd, max(0, grid - m - x * per_xcd));
}
// Items of XCD x over all rounds.
__host__ __device__ inline int xcd_items(int grid, int n_items, int x) {
    const int per_xcd = grid / kNumXcd;
    const int r = n_items / grid, m = n_items % grid;
    const int last = (r & 1) ? per_xcd - xcd_first_filled(grid, m, x)
                             : min(per_xcd, max(0, m - x * per_xcd));
    return r * per_xcd + last;
}

// Work stealing for a workgroup whose XCD's list is used up: the queue
// cursors of all XCDs are read, the one with the most items left is claimed
// from, and a lost race (another workgroup took the last item) tries again.
// Returns the slot of the claimed item, or -1 once every list is used up.
// Cursors only grow, so every pass either claims or sees less work left.
__device__ inline int steal_item(int32_t* queue, int grid, int n_items) {
    const int per_xcd = grid / kNumXcd;
    for (int attempt = 0; attempt < 2 * kNumXcd; ++attempt) {
        int cur[kNumXcd];
#pragma unroll
        for (int x = 0; x < kNumXcd; ++x)
            cur[x] = __hip_atomic_load(queue + x, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        int best = -1, best_left = 0;
#pragma unroll
        for (int x = 0; x < kNumXcd; ++x) {
            const int left = xcd_items(grid, n_items, x) - per_xcd - cur[x];
            if (left > best_left) {
                best_left = left;
                best = x;
            }
        }
        if (best < 0) return -1;
        const int i = per_xcd + __hip_atomic_fetch_add(queue + best, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        if (i < xcd_items(grid, n_items, best)) return i * kNumXcd + best;
    }
    return -1;
}

// Inlined on purpose: called out of line, its register count (over 160)
// became the prep kernel's and held every node workgroup to one per CU.
__device__ __attribute__((always_inline)) void build_plan(const int32_t* __restrict__ node_offsets,
                           const int32_t* __restrict__ ctx_lens, int B, int n_max,
                           int64_t total_nodes, int G, int Hkv, int cap_limit, int tile_m,
                           int target_items, int grid, PlanHeader* hdr, Item* items,
                           Combine* combine, int64_t max_items, int64_t max_groups,
                           int64_t max_partials, int2* group_list, int32_t* group_pos,
                           int32_t* err, int32_t* s_off, int32_t* s_ctx,
                           int32_t* s_items, int32_t* s_parts) {  // LDS, B + 1 ints each
    __shared__ unsigned long long s_wsum[kPrepWaves];
    __shared__ int32_t s_wtot[2][kPrepWaves];
    __shared__ int32_t s_bucket[kCostBuckets];  // counts, then placement cursors
    __shared__ int32_t s_ncomb, s_ngroups;
    const int tid = threadIdx.x;
    const int lane = tid & 63, wv = tid >> 6;
    if (tid == 0) s_ncomb = s_ngroups = 0;
    // The offsets and lengths are read once, into LDS.
    for (int j = tid; j <= B; j += kPrepThreads) {
        s_off[j] = node_offsets[j];
        if (j < B) s_ctx[j] = ctx_lens[j];
    }
    __syncthreads();
    // Phase 1: total slot work, W = Hkv * sum over row tiles of (ctx + tree keys).
    unsigned long long my_work = 0;
    for (int b = tid; b < B; b += kPrepThreads) {
        const int s = s_off[b];
        const int n = s_off[b + 1] - s;
        const int ctx = s_ctx[b];
        if (s < 0 || n < 0 || n > n_max || (int64_t)s + n > total_nodes || ctx < 0) continue;
        if (cap_limit >= 0 && (int64_t)ctx + n > cap_limit) continue;
        const int rows = n * G;
        const int nt = (rows + tile_m - 1) / tile_m;
        for (int t = 0; t < nt; ++t) {
            const int last_row = min((t + 1) * tile_m, rows) - 1;
            my_work += (unsigned long long)(ctx + last_row / G + 1);
        }
    }
    my_work *= (unsigned long long)Hkv;
    // workgroup sum: lane shuffles, then one LDS slot per wave
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) {
        const uint32_t lo = __shfl_xor((uint32_t)my_work, off), hi = __shfl_xor((uint32_t)(my_work >> 32), off);
        my_work += ((unsigned long long)hi << 32) | lo;
    }
    if (lane == 0) s_wsum[wv] = my_work;
    __syncthreads();
    unsigned long long W = 0;
#pragma unroll
    for (int w = 0; w < kPrepWaves; ++w) W += s_wsum[w];
    long long cl = (long long)((W + target_items - 1) / target_items);
    cl = ((cl + kKT - 1) / kKT) * kKT;
    if (cl < kChunkMin) cl = kChunkMin;
    if (cl > (1ll << 30)) cl = 1ll << 30;
    const int chunk_len = (int)cl;

    // Phase 2: per-request item and partial counts, exclusive prefix sums
    // (lane scans, then the wave totals; the carry is the same in every thread).
    int carry_items = 0, carry_parts = 0;
    for (int base = 0; base < B; base += kPrepThreads) {
        const int b = base + tid;
        int ni = 0, np = 0;
        if (b < B) {
            const int s = s_off[b];
            const int n = s_off[b + 1] - s;
            const int ctx = s_ctx[b];
            bool ok = !(s < 0 || n < 0 || n > n_max || (int64_t)s + n > total_nodes || ctx < 0);
            if (ok && cap_limit >= 0 && (int64_t)ctx + n > cap_limit) {
                ok = false;
                atomicOr(err + b, TTV_ERR_CAPACITY);
            }
            if (ok && n > 0) {
                const int nt = (n * G + tile_m - 1) / tile_m;
                const int nc = ctx > chunk_len ? (ctx + chunk_len - 1) / chunk_len : 1;
                ni = Hkv * nt * nc;
                np = nc > 1 ? ni : 0;
            }
        }
        int si = ni, sp = np;  // inclusive scans within the wave
#pragma unroll
        for (int off = 1; off < 64; off <<= 1) {
            const int ti = __shfl_up(si, off), tp = __shfl_up(sp, off);
            if (lane >= off) {
                si += ti;
                sp += tp;
            }
        }
        if (lane == 63) {
            s_wtot[0][wv] = si;
            s_wtot[1][wv] = sp;
        }
        __syncthreads();
        int pre_i = carry_items, pre_p = carry_parts;
#pragma unroll
        for (int w = 0; w < kPrepWaves; ++w) {
            const int vi = s_wtot[0][w], vp = s_wtot[1][w];
            if (w < wv) {
                pre_i += vi;
                pre_p += vp;
            }
            carry_items += vi;
            carry_parts += vp;
        }
        if (b < B) {
            s_items[b] = pre_i + si - ni;
            s_parts[b] = pre_p + sp - np;
        }
        __syncthreads();  // s_wtot is rewritten by the next block
    }
    if (tid == 0) {
        s_items[B] = carry_items;
        s_parts[B] = carry_parts;
    }
    __syncthreads();
    int n_items = s_items[B];
    // Both bounds hold by construction of chunk_len (see make_layout).  Should
    // either ever trip, nothing runs and every request is flagged, so no
    // caller reads outputs the call never wrote.
    if (n_items > max_items || s_parts[B] > max_partials) {
        n_items = 0;
        for (int b = tid; b < B; b += kPrepThreads) atomicOr(err + b, TTV_ERR_CAPACITY);
    }

    // Phase 3: item descriptors (request found by binary search on the prefix).
    auto make_item = [&](int x, Item& it) __attribute__((always_inline)) {
        int lo = 0, hi = B - 1;
        while (lo < hi) {  // last b with s_items[b] <= x
            const int mid = (lo + hi + 1) >> 1;
            if (s_items[mid] <= x) lo = mid;
            else hi = mid - 1;
        }
        const int b = lo;
        const int s = s_off[b];
        const int n = s_off[b + 1] - s;
        const int ctx = s_ctx[b];
        const int nt = (n * G + tile_m - 1) / tile_m;
        const int nc = ctx > chunk_len ? (ctx + chunk_len - 1) / chunk_len : 1;
        const int local = x - s_items[b];
        const int t = local % nt;
        const int rest = local / nt;
        const int chunk = rest % nc;
        it.b = b;
        it.kvh = rest / nc;
        it.tile = t;
        it.s = s;
        it.n = n;
        it.ctx = ctx;
        it.c0 = chunk * chunk_len;
        it.c1 = min(ctx, it.c0 + chunk_len);
        const int last_row = min((t + 1) * tile_m, n * G) - 1;
        it.kmax = chunk == nc - 1 ? last_row / G + 1 : 0;
        it.pslot = nc > 1 ? s_parts[b] + local : -1;
        it.nc = nc;
        it.nt = nt;
        return chunk;
    };
    // Estimated cost of an item, in tenths of a microsecond per 32-key tile
    // (measured: about 1.3 us with two 16-row blocks per wave, 0.8 us with
    // one, twice that when precise) plus about 7 us of prologue and
    // epilogue; bucketed on a log scale, 32 buckets per octave.
    auto cost_bucket = [&](const Item& it) __attribute__((always_inline)) {
        const int rows = min(tile_m, it.n * G - it.tile * tile_m);
        const int per_tile = ((rows + 15) / 16 > kWaves ? 13 : 8) * (it.ctx < kPreciseCtx ? 2 : 1);
        const int tiles = (it.c1 - it.c0 + kKT - 1) / kKT + (it.kmax + kKT - 1) / kKT;
        const uint32_t key = 70u + (uint32_t)tiles * (uint32_t)per_tile;
        const int msb = 31 - __builtin_clz(key);
        return 32 * msb + (int)((key >> (msb - 5)) & 31u);  // key >= 70, so msb >= 6
    };
    // Placement: the main kernel's workgroup w runs the items at slots w,
    // grid + w, 2 grid + w, ...; virtual workgroup v is workgroup
    // (v % per_xcd) * 8 + v / per_xcd, so consecutive virtual ids share an
    // XCD (hardware places workgroup w on XCD w % 8).
    // - At most one item per workgroup: item x on virtual workgroup x, over a
    //   multiple of 8 workgroups, so the row tiles of one chunk (consecutive
    //   items, the same K/V) run side by side on one XCD.
    // - More: whole (request, KV head, chunk) groups, largest estimated cost
    //   first, each group's row tiles at consecutive positions, dealt in
    //   snake order -- round r of `grid` positions goes to virtual
    //   workgroups 0 .. grid-1 for even r and grid-1 .. 0 for odd r -- so
    //   each workgroup's total comes out close to the mean and a group's
    //   tiles still run side by side (the order inside a cost bucket is
    //   arbitrary).
    const bool snake = n_items > grid;
    if (snake) {
        for (int k = tid; k < kCostBuckets; k += kPrepThreads) s_bucket[k] = 0;
        __syncthreads();
        // A group (request, KV head, chunk: its nt row tiles are consecutive
        // items) is counted by its first tile, which also lists the group as
        // (first item, bucket + 1024 nt); nt <= 512, bucket < 1024.
        for (int x = tid; x < n_items; x += kPrepThreads) {
            Item it;
            make_item(x, it);
            if (it.tile == 0) {
                const int k = cost_bucket(it);
                atomicAdd(&s_bucket[k], it.nt);
                const int gi = atomicAdd(&s_ngroups, 1);
                if (TTV_DCHECK(gi < max_items, TTV_SITE_PLAN)) group_list[gi] = make_int2(x, k + 1024 * it.nt);
            }
        }
        __syncthreads();
        // cursors: bucket k starts after every item of the buckets above it
        // (thread i owns buckets 1023 - 2i and 1022 - 2i)
        static_assert(kCostBuckets == 2 * kPrepThreads, "two buckets per thread");
        const int k_hi = kCostBuckets - 1 - 2 * tid;
        const int c_hi = s_bucket[k_hi], c_lo = s_bucket[k_hi - 1];
        int sc = c_hi + c_lo;  // inclusive scan within the wave
#pragma unroll
        for (int off = 1; off < 64; off <<= 1) {
            const int tv = __shfl_up(sc, off);
            if (lane >= off) sc += tv;
        }
        if (lane == 63) s_wtot[0][wv] = sc;
        __syncthreads();
        int pre = sc - c_hi - c_lo;
#pragma unroll
        for (int w = 0; w < kPrepWaves; ++w)
            if (w < wv) pre += s_wtot[0][w];
        s_bucket[k_hi] = pre;
        s_bucket[k_hi - 1] = pre + c_hi;
        __syncthreads();
    }
    auto add_combine = [&](const Item& it) __attribute__((always_inline)) {
        const int ci = atomicAdd(&s_ncomb, 1);
        if (ci < max_groups) {
            Combine cb;
            cb.b = it.b;
            cb.kvh = it.kvh;
            cb.tile = it.tile;
            cb.s = it.s;
            cb.n = it.n;
            cb.pslot0 = it.pslot;
            cb.stride = it.nt;
            cb.nc = it.nc;
            combine[ci] = cb;
        }
    };
    if (!snake) {
        const int per_xcd = (n_items + kNumXcd - 1) / kNumXcd;
        for (int x = tid; x < n_items; x += kPrepThreads) {
            Item it;
            const int chunk = make_item(x, it);
            const int64_t slot = (int64_t)(x % per_xcd) * kNumXcd + x / per_xcd;
            if (TTV_DCHECK(slot < max_items && it.pslot < max_partials, TTV_SITE_PLAN)) items[slot] = it;
            if (it.nc > 1 && chunk == 0) add_combine(it);
        }
    } else {
        // Each group takes nt consecutive positions from its bucket's cursor
        // (first position kept at its first item's index in group_pos); then
        // every item places itself at its group's first position plus its
        // row tile.  (A group placing its own tiles in a loop left the
        // threads of groups with many tiles running long serial loops.)
        const int n_groups = s_ngroups;
        for (int g = tid; g < n_groups; g += kPrepThreads) {
            const int2 e = group_list[g];
            if (TTV_DCHECK(e.x >= 0 && e.x < max_items, TTV_SITE_PLAN))
                group_pos[e.x] = atomicAdd(&s_bucket[e.y & 1023], e.y >> 10);
        }
        __syncthreads();
        const int per_xcd = grid / kNumXcd;
        for (int x = tid; x < n_items; x += kPrepThreads) {
            Item it;
            const int chunk = make_item(x, it);
            if (it.nc > 1 && chunk == 0) add_combine(it);
            const int p = group_pos[x - it.tile] + it.tile, r = p / grid, k = p % grid;
            const int v = (r & 1) ? grid - 1 - k : k;
            // XCD xc's items sit at slots i * 8 + xc, i = 0, 1, ... with no
            // gaps: a partial odd round (positions grid-m .. grid-1) starts
            // each XCD's share at its first filled position
            const int xc = v / per_xcd, j = v % per_xcd;
            const int j_lo = (r == n_items / grid && (r & 1)) ? xcd_first_filled(grid, n_items % grid, xc) : 0;
            const int64_t slot = (int64_t)r * grid + (j - j_lo) * kNumXcd + xc;
            if (TTV_DCHECK(slot < max_items && it.pslot < max_partials, TTV_SITE_PLAN)) items[slot] = it;
        }
    }
    __syncthreads();
    if (tid == 0) {
        hdr->n_items = n_items;
        for (int x = 0; x < kNumXcd; ++x) hdr->queue[x] = 0;
        hdr->n_combine = min((int64_t)s_ncomb, max_groups);
        hdr->chunk_len = chunk_len;
        // bounds the debug build's main and combine kernels check against
        hdr->reserved[0] = (int32_t)total_nodes;
        hdr->reserved[1] = (int32_t)max_partials;
    }
}

template <int D>
// At most 64 registers, so eight waves per SIMD (four 512-thread
// workgroups per CU) keep a large batch's node workgroups in one round.
__global__ __launch_bounds__(kPrepThreads, 8) void attn_prep_kernel(
    const int32_t* __restrict__ node_offsets, const int32_t* __restrict__ ctx_lens, int B,
    int n_max, int64_t total_nodes,
    const uint16_t* __restrict__ k_new, const uint16_t* __restrict__ v_new,
    const int32_t* __restrict__ positions, CacheView cache, int Hq, RopeTable rope,
    double q_mult, float2* __restrict__ rope_cs, int tile_m,
    int target_items, int grid, PlanHeader* hdr, Item* items, Combine* combine, int64_t max_items,
    int64_t max_groups, int64_t max_partials, int2* group_list, int32_t* group_pos,
    int32_t* __restrict__ err) {
    const int Hkv = cache.hkv;
    const int G = Hq / Hkv;
    // node_offsets and ctx_lens staged in LDS (B + 1 ints each), then the
    // plan's prefix sums (B + 1 each, plan workgroup only).
    extern __shared__ int32_t s_dyn[];
    int32_t* s_off = s_dyn;
    int32_t* s_ctx = s_dyn + (B + 1);
    // Workgroup 0 builds the plan (dispatched first, so it overlaps the
    // rest); workgroup 1 + p rotates nodes 2p and 2p + 1 of the whole batch.
    if (blockIdx.x == 0) {
        build_plan(node_offsets, ctx_lens, B, n_max, total_nodes, G, Hkv,
                   cache.paged ? -1 : cache.cap, tile_m, target_items, grid, hdr, items, combine,
                   max_items, max_groups, max_partials, group_list, group_pos, err, s_off, s_ctx,
                   s_dyn + 2 * (B + 1),
                   s_dyn + 3 * (B + 1));
        return;
    }
    // Four nodes per workgroup, one per 128-thread part (two waves each), so
    // a large batch runs its nodes in a quarter as many workgroups.
    constexpr int kPart = kPrepThreads / kPrepNodes;
    static_assert(kPart >= 64, "a part computes D/2 <= 64 angles");
    const int part = threadIdx.x / kPart;
    const int tid = threadIdx.x % kPart;
    const int64_t node = kPrepNodes * ((int64_t)blockIdx.x - 1) + part;
    const bool has_node = node < total_nodes;  // uniform over the part's waves
    constexpr int kVec = 8;
    const int kv_vecs = cache.hkv * D / kVec;
    // K's rotation in fp64: with fp32, x0 cos - x1 sin loses absolute
    // accuracy when the two products nearly cancel, which shows up as bf16
    // ulps of the stored K on small results.
    __shared__ double s_cos2[kPrepNodes][D / 2], s_sin2[kPrepNodes][D / 2];
    double* s_cos = s_cos2[part];
    double* s_sin = s_sin2[part];
    // The node's own loads do not depend on which request owns it, so they
    // are issued first; the request is then found in the staged offsets.
    ttv_u32x4 k_first = {0u, 0u, 0u, 0u}, v_first = {0u, 0u, 0u, 0u};
    int pos = 0;
    if (has_node) {
        if (tid < kv_vecs) {
            const int64_t e = node * cache.hkv * D + (int64_t)tid * kVec;
            k_first = *(const ttv_u32x4*)(k_new + e);
            v_first = *(const ttv_u32x4*)(v_new + e);
        }
        pos = positions[node];
    }
    for (int j = threadIdx.x; j <= B; j += kPrepThreads) {
        s_off[j] = node_offsets[j];
        if (j < B) s_ctx[j] = ctx_lens[j];
    }
    if (has_node && tid < D / 2) {
        // the angle is reduced modulo 2*pi before sincos
        const double ang = (double)pos * rope.inv[tid];
        const double two_pi = 6.283185307179586476925;
        const double red = ang - two_pi * rint(ang / two_pi);
        double sn, cs;
        sincos(red, &sn, &cs);
        s_cos[tid] = cs;
        s_sin[tid] = sn;
        // the main kernel rotates Q with these, scaled by scale * log2(e)
        rope_cs[node * (D / 2) + tid] = make_float2((float)(cs * q_mult), (float)(sn * q_mult));
    }
    __syncthreads();
    if (!has_node) return;  // after the workgroup's only barrier
    // owning request: the last b with node_offsets[b] <= node (offsets are
    // non-decreasing; the checks below reject anything else)
    int lo = 0, hi = B - 1;
    while (lo < hi) {
        const int mid = (lo + hi + 1) >> 1;
        if (s_off[mid] <= node) lo = mid;
        else hi = mid - 1;
    }
    // The request is uniform over the part (a wave lies in one part); saying
    // so keeps its values in scalar registers and lets one lane per wave
    // raise a flag.
    const int b = __builtin_amdgcn_readfirstlane(lo);
    const int s = __builtin_amdgcn_readfirstlane(s_off[b]);
    const int n = __builtin_amdgcn_readfirstlane(s_off[b + 1]) - s;
    const int i = (int)(node - s);
    const int ctx = __builtin_amdgcn_readfirstlane(s_ctx[b]);
    const bool ok = s >= 0 && n >= 0 && n <= n_max && (int64_t)s + n <= total_nodes && i >= 0 &&
                    i < n && ctx >= 0 && (cache.paged || (int64_t)ctx + n <= cache.cap);
    if (!ok) return;  // uniform; the plan flags the request
    int64_t dst_first = -1;
    if (tid < kv_vecs) dst_first = cache_row(cache, b, (tid * kVec) / D, ctx + i, D);
    // K (rotated, rounded once from fp64) and V (copied) into slot ctx + i.
    for (int v = tid; v < kv_vecs; v += kPart) {
        const int h = (v * kVec) / D;
        const int d0 = (v * kVec) % D;
        const bool first = v == tid;
        const int64_t dst = first ? dst_first : cache_row(cache, b, h, ctx + i, D);
        if (dst < 0) {  // unmapped slot: one flag per wave, not one per lane
            const uint64_t bad = __ballot(1);
            if ((threadIdx.x & 63) == __builtin_ctzll(bad)) atomicOr(err + b, TTV_ERR_BLOCK_TABLE);
            continue;
        }
        if (!TTV_DCHECK(dst + d0 + kVec <= cache_elems(cache, B, D), TTV_SITE_PREP_CACHE)) continue;
        const int64_t e = node * Hkv * D + (int64_t)v * kVec;
        const ttv_u32x4 kin = first ? k_first : *(const ttv_u32x4*)(k_new + e);
        ttv_u32x4 ko;
#pragma unroll
        for (int w = 0; w < 4; ++w) {
            const double x0 = ttv_bf16_bits_to_f64(kin[w] & 0xFFFFu);
            const double x1 = ttv_bf16_bits_to_f64(kin[w] >> 16);
            const int m = (d0 >> 1) + w;
            const double c = s_cos[m], sn = s_sin[m];
            ko[w] = pack_bf16_f64(x0 * c - x1 * sn, x1 * c + x0 * sn);
        }
        *(ttv_u32x4*)(cache.k + dst + d0) = ko;
        *(ttv_u32x4*)(cache.v + dst + d0) = first ? v_first : *(const ttv_u32x4*)(v_new + e);
    }
}

// ---------------------------------------------------------------------------
// 2. Main kernel.
//
// LDS holds a ring of (K tile, V tile) stages -- 8 for items with a long
// context, 4 for precise items, whose rows' Q low parts take the space of
// the other 4 -- and the tile nodes' mask rows, all filled by direct
// global->LDS loads (global_load_lds: no registers hold data in flight).  A
// tile is 32 key slots in kChunks chunks of K and of V; waves 0..3 (one per
// SIMD) load them, wave w chunks w, w + 4, ..., so a loading wave issues
// 2 kCpw DMA instructions per tile (half as many waves doing the address
// work as with one chunk per wave) and waits on its own vmcnt before a
// barrier publishes the tile.  The DMA is issued through
// inline asm: the compiler then neither counts it nor guards every later LDS
// read with a wait for all loads in flight; the explicit vmcnt ladder and the
// raw barriers order it.
//
// K rows are stored with an XOR swizzle of their 16-byte pieces
// (piece ^ row % P) so the 16 rows an MFMA operand read touches fall in
// distinct banks.  V rows are stored row-major with piece ^ (2 row % P) and
// read with ds_read_b64_tr_b16, which hands each lane four keys of one
// head-dim column: exactly the V^T operand, no transposing store.
// ---------------------------------------------------------------------------

template <int D, int kW, int kRows = kW * kRowsPerWave>
struct MainCfg {
    static constexpr int kTile = kRows;                    // query rows per work item
    static constexpr int kPieces = D / 8;                  // 16-byte pieces per row
    static constexpr int kRowBytes = D * 2;
    static constexpr int kTileBytes = kKT * kRowBytes;     // one K or V tile
    static constexpr int kChunkRows = 1024 / kRowBytes;    // rows per DMA instruction (64 x 16 B)
    static constexpr int kChunks = kKT / kChunkRows;       // DMA instructions per K (or V) tile
    // waves 0 .. kIssueWaves-1 (one per SIMD) load a tile: wave w loads
    // chunks w, w + kIssueWaves, ... (kCpw of them); the other waves none
    static constexpr int kIssueWaves = kChunks < 4 ? kChunks : 4;
    static constexpr int kCpw = kChunks / kIssueWaves;
    static_assert(kChunks % kIssueWaves == 0 && kIssueWaves <= kW, "chunks spread evenly over the issuing waves");
    static_assert(kCpw <= 2, "at most two chunks per wave");
    static constexpr int kOpsPerTile = 2 * kCpw;           // DMA instructions per tile per loading wave
    static constexpr int kStageBytes = 2 * kTileBytes;
    // LDS: 8 stages; precise items use the first 4 and keep their rows' Q
    // low parts in the space of the other 4.
    static constexpr int kStagesShort = 4;
    static constexpr int kStagesLong = 8;
    static constexpr int kQloOffset = kStagesShort * kStageBytes;
    static constexpr int kQloBytes = kTile * kRowBytes;
    static constexpr int kMainBytes = kStagesLong * kStageBytes;
    // per-lane DMA byte offsets of the issuing waves (K and V, kCpw chunks)
    static constexpr int kOffTableBytes = kIssueWaves * TTV_WAVE * kCpw * 8;
    // after the offset table: the next-item slots of the work queue
    static constexpr int kMiscBytes = 256;
    static constexpr int kMaskOffset = kMainBytes + kOffTableBytes + kMiscBytes;
    static_assert(kQloOffset + kQloBytes <= kMainBytes, "Q lo fits in stages 4..7");
};

__device__ __forceinline__ int swz_k(int row, int piece, int P) { return piece ^ (row & (P - 1)); }
__device__ __forceinline__ int swz_v(int row, int piece, int P) { return piece ^ ((2 * row) & (P - 1)); }

template <int N>
__device__ __forceinline__ void wait_vmcnt() {
    // s_waitcnt: vmcnt[3:0] | expcnt(7) << 4 | lgkmcnt(15) << 8 | vmcnt[5:4] << 14
    __builtin_amdgcn_s_waitcnt((N & 15) | (7 << 4) | (15 << 8) | ((N >> 4) << 14));
}

// Wait until at most k tiles' worth (kOps loads each) of this wave's loads
// are outstanding (k in 0..5).
template <int kOps>
__device__ __forceinline__ void wait_vmcnt_tiles(int k) {
    if (k >= 5) wait_vmcnt<5 * kOps>();
    else if (k == 4) wait_vmcnt<4 * kOps>();
    else if (k == 3) wait_vmcnt<3 * kOps>();
    else if (k == 2) wait_vmcnt<2 * kOps>();
    else if (k == 1) wait_vmcnt<kOps>();
    else wait_vmcnt<0>();
}

__device__ __forceinline__ void raw_barrier() {
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
}

typedef short ttv_i16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) ttv_i16x4 lds_i16x4;

// The lane's id from an instruction the compiler may neither move nor reuse.
// The tile loads' per-lane addresses and the epilogue's output indices are
// derived from it where they are used: derived from the ordinary lane index,
// the compiler computed them once, held them across the tile loop and spilled
// them, and each reload's memory wait (which cannot count the loads issued
// through asm) also waited for every tile load in flight.  (Recomputing the
// rows' tree-mask index this way instead made the tile loop slower.)
__device__ __forceinline__ int fresh_lane() {
    int l;
    asm volatile("v_mbcnt_lo_u32_b32 %0, -1, 0\n\tv_mbcnt_hi_u32_b32 %0, -1, %0" : "=v"(l));
    return l;
}

// Byte address of an LDS location, as the ds_* instructions take it.
__device__ __forceinline__ uint32_t lds_offset(const void* p) {
    return (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) char*)p;
}

// 16 (or 4) bytes per lane from global memory into LDS at base + lane * 16 (4).
// lds_base must be wave-uniform.
__device__ __forceinline__ void dma16(uint32_t lds_base, const void* g) {
    const uint32_t base = __builtin_amdgcn_readfirstlane(lds_base);
    asm volatile("s_mov_b32 m0, %0\n\tglobal_load_lds_dwordx4 %1, off" ::"s"(base), "v"(g)
                 : "memory", "m0");
}
// Same, with a wave-uniform base address and a 32-bit per-lane byte offset.
__device__ __forceinline__ void dma16s(uint32_t lds_base, const void* sbase, uint32_t voff) {
    const uint32_t base = __builtin_amdgcn_readfirstlane(lds_base);
    const uint64_t g = (uint64_t)(uintptr_t)sbase;
    // readfirstlane returns int: widen through uint32_t, never by sign extension
    const uint32_t g_lo = (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)g);
    const uint32_t g_hi = (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)(g >> 32));
    const uint64_t gs = ((uint64_t)g_hi << 32) | (uint64_t)g_lo;
    asm volatile("s_mov_b32 m0, %0\n\tglobal_load_lds_dwordx4 %1, %2" ::"s"(base), "v"(voff), "s"(gs)
                 : "memory", "m0");
}
__device__ __forceinline__ void dma4(uint32_t lds_base, const void* g) {
    const uint32_t base = __builtin_amdgcn_readfirstlane(lds_base);
    asm volatile("s_mov_b32 m0, %0\n\tglobal_load_lds_dword %1, off" ::"s"(base), "v"(g)
                 : "memory", "m0");
}

// Round two floats to a bf16 pair (hardware round-to-nearest-even).
__device__ __forceinline__ uint32_t pack_bf16(float a, float b) {
    return __builtin_bit_cast(uint32_t, __builtin_convertvector((ttv_f32x2v){a, b}, ttv_bf16x2v));
}

// x *= a, written back into x's own register: the rare rescale branch then
// leaves the accumulators where the MFMAs keep them (no copies on the path
// that skips it).
__device__ __forceinline__ void scale_in_place(ttv_f32x4& v, float a) { v *= a; }

// max over the four lanes l, l^16, l^32, l^48 (the lane groups sharing a row)
__device__ __forceinline__ float group_max(float t) {
    auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(t), __float_as_uint(t), false, false);
    t = fmaxf(__uint_as_float(a[0]), __uint_as_float(a[1]));
    auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(t), __float_as_uint(t), false, false);
    return fmaxf(__uint_as_float(b[0]), __uint_as_float(b[1]));
}
__device__ __forceinline__ float group_sum(float t) {
    auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(t), __float_as_uint(t), false, false);
    t = __uint_as_float(a[0]) + __uint_as_float(a[1]);
    auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(t), __float_as_uint(t), false, false);
    return __uint_as_float(b[0]) + __uint_as_float(b[1]);
}

template <int D, bool kPaged>
__device__ __forceinline__ const uint16_t* kv_row_ptr(const CacheView& c, const uint16_t* base,
                                                      int b, int h, int slot, int blk) {
    if (!kPaged) return base + (((int64_t)b * c.hkv + h) * c.cap + slot) * D;
    return base + (((int64_t)blk * c.hkv + h) * TTV_BLOCK_SIZE + (slot & 15)) * D;
}

// Physical blocks holding the rows of each chunk wave w loads for a tile
// (slots slot0 .. slot0 + valid - 1): the first and the last of those rows,
// which span at most two blocks.  Wave-uniform scalar reads of the block
// table; the tile loop fetches them one tile ahead of the loads that use them.
struct TileBlocks {
    int32_t first[2], last[2];
};

template <int D, int kW, bool kPaged>
__device__ __forceinline__ TileBlocks tile_blocks(const CacheView& c, const int32_t* __restrict__ table,
                                                  int b, int slot0, int valid, int wave) {
    using MC = MainCfg<D, kW>;
    TileBlocks tb{{0, 0}, {0, 0}};
    if (!kPaged || wave >= MC::kIssueWaves) return tb;
#pragma unroll
    for (int j = 0; j < MC::kCpw; ++j) {
        const int ch = wave + j * MC::kIssueWaves;
        const int r_first = min(ch * MC::kChunkRows, valid - 1);
        const int r_last = min(ch * MC::kChunkRows + MC::kChunkRows - 1, valid - 1);
        const int lb0 = (slot0 + r_first) >> 4;
        const int lb1 = (slot0 + r_last) >> 4;
        tb.first[j] = lb0 < c.max_blocks ? table[(int64_t)b * c.max_blocks + lb0] : -1;
        tb.last[j] = lb1 < c.max_blocks ? table[(int64_t)b * c.max_blocks + lb1] : -1;
    }
    return tb;
}

// Issue the LDS-DMA loads of one tile (slots slot0 .. slot0 + valid - 1; rows
// past valid repeat the last valid slot, so every LDS byte is defined).
// Wave w loads chunks w, w + kW, ... (kChunkRows rows each) of K and of V.
template <int D, int kW, bool kPaged>
__device__ __forceinline__ void issue_tile(const CacheView& c, TileBlocks tb, int b, int kvh, int slot0,
                                           int valid, uint32_t stage, int wave, int32_t* err) {
    using MC = MainCfg<D, kW>;
    constexpr int P = MC::kPieces;
    if (wave >= MC::kIssueWaves) return;
#pragma unroll
    for (int j = 0; j < MC::kCpw; ++j) {
        const int ch = wave + j * MC::kIssueWaves;
        const int r_first = min(ch * MC::kChunkRows, valid - 1);
        const int lane = fresh_lane();
        int bf = tb.first[j], bl = tb.last[j];
        if (kPaged && (bf < 0 || bf >= c.num_blocks || bl < 0 || bl >= c.num_blocks)) {
            if (lane == 0) atomicOr(err + b, TTV_ERR_BLOCK_TABLE);
            bf = bl = 0;  // load a valid block; the request is flagged
        }
        const int row = ch * MC::kChunkRows + lane / P;
        const int phys = lane % P;
        int slot = slot0 + min(row, valid - 1);
        if (!TTV_DCHECK(kPaged || (slot >= 0 && slot < c.cap), TTV_SITE_MAIN_CACHE)) slot = 0;
        const int blk = (!kPaged || (slot >> 4) == ((slot0 + r_first) >> 4)) ? bf : bl;
        const uint16_t* krow = kv_row_ptr<D, kPaged>(c, c.k, b, kvh, slot, blk);
        const uint16_t* vrow = kv_row_ptr<D, kPaged>(c, c.v, b, kvh, slot, blk);
        const uint32_t chunk_off = ch * MC::kChunkRows * MC::kRowBytes;
        dma16(stage + chunk_off, krow + 8 * swz_k(row, phys, P));
        dma16(stage + MC::kTileBytes + chunk_off, vrow + 8 * swz_v(row, phys, P));
    }
}

template <int D, bool kPaged, int kW, int kRows>
__global__ __launch_bounds__(kW * TTV_WAVE) void attn_main_kernel(
    const PlanHeader* __restrict__ hdr, const Item* __restrict__ items,
    const uint16_t* q,  // not __restrict__: keeps its loads ahead of the prologue fence
    const float2* __restrict__ rope_cs, const uint32_t* __restrict__ mask, int mask_words,
    CacheView cache, const int32_t* __restrict__ table, int Hq, uint16_t* __restrict__ out,
    ttv_f16x4* __restrict__ part_o, float4* __restrict__ part_ml, int32_t* __restrict__ queue,
    int32_t* __restrict__ err) {
    using MC = MainCfg<D, kW, kRows>;
    constexpr int kTileR = MC::kTile;
    // 16-row blocks per wave that a full tile fills (1 or 2)
    constexpr int kMBr = (kTileR + 16 * kW - 1) / (16 * kW);
    static_assert(kMBr >= 1 && kMBr <= kMB, "one or two row blocks per wave");
    constexpr int P = MC::kPieces;
    constexpr int KC = D / 32;   // 32-wide k chunks of the head dim
    constexpr int DB = D / 16;   // 16-row blocks of the head dim
    extern __shared__ __attribute__((aligned(16))) char smem[];
    const uint32_t ring = lds_offset(smem);
    const uint32_t qlo_s = ring + MC::kQloOffset;
    const uint32_t mask_base = ring + MC::kMaskOffset;
    const uint32_t* mask_s = (const uint32_t*)(smem + MC::kMaskOffset);
    int32_t* const s_next = (int32_t*)(smem + MC::kMainBytes + MC::kOffTableBytes);
    // This issuing wave's row of the DMA offset table (its own lanes only, so
    // it needs no barrier): chunk j's K and V byte offsets inside a stage.
    uint32_t* const off_row = (uint32_t*)(smem + MC::kMainBytes) + (size_t)(threadIdx.x >> 6) * TTV_WAVE * MC::kCpw * 2;

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    // wave index as a scalar, so branches on it stay uniform (an exec-masked
    // branch would run both sides' s_waitcnt)
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int l16 = lane & 15;
    const int g4 = lane >> 4;
    // This workgroup's items sit at slots blockIdx.x + k * gridDim.x (see
    // the plan), so the first one's load does not wait for n_items.
    const Item first_item = items[blockIdx.x];
    const int n_items = hdr->n_items;
#ifdef TTV_DEBUG
    const int64_t dbg_nodes = hdr->reserved[0], dbg_partials = hdr->reserved[1];
#endif
    const int Hkv = cache.hkv;
    const int G = Hq / Hkv;
    const int grid = gridDim.x, wg = blockIdx.x;
    // More items than workgroups: XCD x = wg % 8 owns the items at slots
    // i * 8 + x, i < xcd_items (the plan's snake order, largest estimated
    // cost first).  Its workgroups take i = wg / 8 first, then claim the
    // next i from the XCD's queue cursor as they finish, so a workgroup that
    // drew short items takes more of them.  The claim for the next item is
    // made kClaimLead tiles before an item ends; its answer lands during those
    // tiles.  Once its XCD's list is used up, an idle workgroup takes items
    // left on the other XCDs (steal_item).
    // Otherwise one item each on as many workgroups as items, a multiple of
    // 8, consecutive items on one XCD: workgroup wg holds the item at slot wg.
    const bool dyn = n_items > grid;
    const int xcd = wg % kNumXcd, per_xcd = grid / kNumXcd;
    bool more;
    int n_xcd = 0;
    if (dyn) {
        n_xcd = xcd_items(grid, n_items, xcd);
        more = true;  // the first round is full
    } else {
        const int active = ((n_items + kNumXcd - 1) / kNumXcd) * kNumXcd;
        const int per = active / kNumXcd, xcd_slot = wg / kNumXcd;
        more = xcd_slot < per && xcd * per + xcd_slot < n_items;
    }

    // Per-lane LDS byte offsets inside a stage / the Q-lo block.
    uint32_t koff[KC];  // K operand: row l16 (+16 kb), piece 4kc + g4
#pragma unroll
    for (int kc = 0; kc < KC; ++kc) koff[kc] = l16 * MC::kRowBytes + 16 * swz_k(l16, 4 * kc + g4, P);
    // V^T operand: ds_read_b64_tr_b16 at row 16h + 4g4 + l16 / 4, head dim
    // 16db + 4 (l16 % 4); the XOR swizzle of row + 16 equals that of row.
    uint32_t voff[DB];
#pragma unroll
    for (int db = 0; db < DB; ++db) {
        const int row = 4 * g4 + (l16 >> 2);
        const int d = 16 * db + 4 * (l16 & 3);
        voff[db] = row * MC::kRowBytes + 16 * swz_v(row, d >> 3, P) + 2 * (d & 7);
    }
    // A operand of all ones: 1^T P^T gives the row sums of P.
    const ttv_bf16x8 kOnes = __builtin_bit_cast(
        ttv_bf16x8, ttv_u32x4{0x3F803F80u, 0x3F803F80u, 0x3F803F80u, 0x3F803F80u});
    if (wave < MC::kIssueWaves) {
#pragma unroll
        for (int j = 0; j < MC::kCpw; ++j) {
            const int f_row = (wave + j * MC::kIssueWaves) * MC::kChunkRows + lane / P;
            const int f_phys = lane % P;
            const int f_rowb = (kPaged ? (f_row & 15) : f_row) * MC::kRowBytes;
            off_row[(2 * j) * TTV_WAVE + lane] = f_rowb + 16 * swz_k(f_row, f_phys, P);
            off_row[(2 * j + 1) * TTV_WAVE + lane] = f_rowb + 16 * swz_v(f_row, f_phys, P);
        }
    }

    for (int k = 0, slot = wg; more; ++k) {
        const Item it = k == 0 ? first_item : items[slot];
        const int rows = it.n * G;
        const int n_ctx_tiles = (it.c1 - it.c0 + kKT - 1) / kKT;
        const int n_tree_tiles = (it.kmax + kKT - 1) / kKT;
        const int n_tiles = n_ctx_tiles + n_tree_tiles;
        // The next item is claimed from this XCD's cursor kClaimLead tiles
        // before the item ends (at its start when it is shorter), so the
        // atomic's latency hides behind the last tiles while a claimed item
        // waits only briefly -- the longer it waits, the fewer items idle
        // workgroups of other XCDs find to take.
        int claim = 0;  // lane 0 of wave 0
        const int tau_claim = n_tiles > kClaimLead ? n_tiles - kClaimLead : -1;
        if (dyn && tid == 0 && tau_claim < 0)
            claim = __hip_atomic_fetch_add(queue + xcd, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        // Three classes of tiles.  Plain: whole context tiles.  Masked: the
        // partial context tile and the tree tiles.  Precise: every tile of a
        // request with a short context, where few keys can dominate a row's
        // softmax; these are masked and run Q and P as bf16 hi + lo pairs
        // (two MFMAs each), with the Q low parts in LDS.  An item is either
        // all precise, or plain tiles [0, n_plain) then masked tiles.
        const bool precise = it.ctx < kPreciseCtx;
        const int n_plain = precise ? 0 : (it.c1 - it.c0) / kKT;
        // Ring depth: precise items share LDS with the Q low parts.
        const int stages = precise ? MC::kStagesShort : MC::kStagesLong;
        const int smask = stages - 1;
        const int ahead = stages - 1;  // tiles issued ahead of the one consumed
        const int node0 = (it.tile * kTileR) / G;
        const int node1 = min(it.n - 1, (it.tile * kTileR + kTileR - 1) / G);
        const int tree_limit = it.ctx + it.kmax;
        auto tile_slot0 = [&](int tau) __attribute__((always_inline)) {
            return tau < n_ctx_tiles ? it.c0 + tau * kKT : it.ctx + (tau - n_ctx_tiles) * kKT;
        };
        auto tile_valid = [&](int tau, int slot0) __attribute__((always_inline)) {
            return min(kKT, (tau < n_ctx_tiles ? it.c1 : tree_limit) - slot0);
        };
        auto blocks_of = [&](int tau) __attribute__((always_inline)) {
            const int slot0 = tile_slot0(tau);
            return tile_blocks<D, kW, kPaged>(cache, table, it.b, slot0, tile_valid(tau, slot0), wave);
        };
        auto issue = [&](int tau, TileBlocks tb) __attribute__((always_inline)) {
            const int slot0 = tile_slot0(tau);
            issue_tile<D, kW, kPaged>(cache, tb, it.b, it.kvh, slot0, tile_valid(tau, slot0),
                                  ring + (tau & smask) * MC::kStageBytes, wave, err);
        };
        TileBlocks next_blocks{{0, 0}, {0, 0}};  // blocks of the next tile to issue
        // Paged, two whole context tiles t0 and t0 + 1 (t0 even): their four
        // blocks are consecutive table entries, one per 16 slots.
        auto whole_pair_blocks = [&](int t0, TileBlocks& x0, TileBlocks& x1) __attribute__((always_inline)) {
            if (wave >= MC::kIssueWaves) return;
            const int32_t* tp = table + (int64_t)it.b * cache.max_blocks + (it.c0 >> 4) + 2 * t0;
            const int32_t e0 = tp[0], e1 = tp[1], e2 = tp[2], e3 = tp[3];
#pragma unroll
            for (int j = 0; j < MC::kCpw; ++j) {
                const bool second = (wave + j * MC::kIssueWaves) * MC::kChunkRows >= 16;
                x0.first[j] = x0.last[j] = second ? e1 : e0;
                x1.first[j] = x1.last[j] = second ? e3 : e2;
            }
        };
        // Fast issue path for whole context tiles (slot0 = c0 + 32 tau, no
        // clamping): an issue is a wave-uniform base plus a per-lane byte
        // offset per chunk this wave loads (from the first row of the chunk's
        // paged block, or from the tile's first slot).  A chunk's rows of such
        // a tile lie in one paged block: slot0 is a multiple of 32 and a chunk
        // is a 16-aligned sub-range of rows.
        // A whole tile's DMA offsets come from the table: read before the
        // wait and barrier that precede the issue (their latency hides behind
        // them), so no offset is live across the tile loop, where the
        // compiler would spill it and the reload's vmcnt wait would also
        // drain the ring (its count cannot see the DMAs, issued through asm).
        auto read_offsets = [&](uint32_t (&o)[2 * MC::kCpw]) __attribute__((always_inline)) {
#pragma unroll
            for (int j = 0; j < 2 * MC::kCpw; ++j) o[j] = off_row[j * TTV_WAVE + lane];
        };
        auto issue_whole = [&](int tau, TileBlocks tb, const uint32_t (&o)[2 * MC::kCpw]) __attribute__((always_inline)) {
            if (wave >= MC::kIssueWaves) return;
            const int slot0 = it.c0 + tau * kKT;
            const uint32_t stage = ring + (tau & smask) * MC::kStageBytes;
#pragma unroll
            for (int j = 0; j < MC::kCpw; ++j) {
                const uint32_t kb = o[2 * j], vb = o[2 * j + 1];
                const int ch = wave + j * MC::kIssueWaves;
                int64_t row0;  // element offset of the tile's (first) row of this KV head
                if (kPaged) {
                    // An unmapped block loads block 0 instead (the prologue
                    // flagged the request); a select, not a branch, so the
                    // base stays scalar math.
                    const int32_t e = tb.first[j];
                    const int blk = __builtin_amdgcn_readfirstlane((uint32_t)e < (uint32_t)cache.num_blocks ? e : 0);
                    row0 = ((int64_t)blk * cache.hkv + it.kvh) * TTV_BLOCK_SIZE * D;
                } else {
                    const bool in = TTV_DCHECK(slot0 >= 0 && slot0 + kKT <= cache.cap, TTV_SITE_MAIN_CACHE);
                    row0 = (((int64_t)it.b * cache.hkv + it.kvh) * cache.cap + (in ? slot0 : 0)) * D;
                }
                const uint32_t chunk_off = ch * MC::kChunkRows * MC::kRowBytes;
                dma16s(stage + chunk_off, cache.k + row0, kb);
                dma16s(stage + MC::kTileBytes + chunk_off, cache.v + row0, vb);
            }
        };

        // ---- prologue: Q and its cos / sin into registers (ordinary loads);
        // the tile nodes' mask rows and tiles 0 and 1 into LDS (DMA); one full
        // wait covers all of them, so the compiler tracks nothing in flight
        // afterwards.  Tiles 2 .. ahead - 1 are issued after that wait and
        // stay in flight into the loop.
        // Row blocks of 16 rows (nblk of them in this tile).  Paired: waves
        // w < ceil(nblk / 2) take blocks 2w and 2w + 1 (NMB = 2; an odd
        // count leaves the last wave one block past the tile, computed and
        // dropped); single: waves w < nblk take block w (NMB = 1).  Pairs run
        // when the tile has more blocks than waves, and for a partly filled
        // 256-row tile over at least 128 key tiles: there, fewer waves with
        // two blocks each (one per SIMD for up to 8 blocks) beat more waves
        // with one (the long Medusa workload's 76-row tiles: about 4 % of
        // the call); over short contexts single blocks were faster.  Every
        // busy wave of an item runs the same count: waves that share a SIMD
        // and run different counts were measured slower than both running two.
        const int nblk = (min(kTileR, rows - it.tile * kTileR) + 15) / 16;
        const int pairs_w = kMBr == 2 && (nblk > kW || (nblk >= 2 && n_tiles >= 128)) ? min(kW, (nblk + 1) / 2) : 0;
        const int nmb = pairs_w ? (wave < pairs_w ? 2 : 0) : (wave < nblk ? 1 : 0);
        int rblk[kMB];
        rblk[0] = nmb == 2 ? 2 * wave : wave;
        rblk[1] = 2 * wave + 1;
        // Q: each lane loads the 8 head-dim entries per 32-wide chunk that
        // its B operand holds (4 rotation pairs) with their cos and sin; they
        // are rotated after the prologue's wait (see below).
        ttv_bf16x8 qreg[kMB][KC];
        ttv_u32x4 qraw[kMB][KC];
        float4 qtab[kMB][KC][2];
        int row_node[kMB];
#pragma unroll
        for (int mb = 0; mb < kMBr; ++mb) {
            const int r = it.tile * kTileR + 16 * rblk[mb] + l16;
            const bool ok = r < rows;
            const int rc = min(r, rows - 1);  // rows past the tile end reuse its last row
            const int node = rc / G, g = rc % G;
            row_node[mb] = ok ? node - node0 : -1;
            const uint16_t* src = q + ((int64_t)(it.s + node) * Hq + it.kvh * G + g) * D;
            const float4* cs = (const float4*)(rope_cs + (int64_t)(it.s + node) * (D / 2));
#pragma unroll
            for (int kc = 0; kc < KC; ++kc) {
                qraw[mb][kc] = *(const ttv_u32x4*)(src + 32 * kc + 8 * g4);
                qtab[mb][kc][0] = cs[(16 * kc + 4 * g4) / 2];
                qtab[mb][kc][1] = cs[(16 * kc + 4 * g4) / 2 + 1];
            }
        }
        if (n_tree_tiles > 0) {
            // the tile nodes' mask rows, copied flat (row stride mask_words)
            const int words = (node1 - node0 + 1) * mask_words;
            const uint32_t* src = mask + (int64_t)(it.s + node0) * mask_words;
            for (int j = wave; j * 64 < words; j += kW)
                dma4(mask_base + j * 256, src + min(j * 64 + lane, words - 1));
        }
        for (int j = 0; j < 2 && j < n_tiles; ++j) issue(j, blocks_of(j));
        if (kPaged) {
            // Every table entry the item's tiles use, checked once here (after
            // the first tiles' loads are out, four loads per thread in flight
            // at a time): the whole-tile loads of the loop only clamp a bad
            // entry.
            const int end_slot = n_tree_tiles > 0 ? tree_limit : it.c1;
            const int e_end = min((end_slot + 15) >> 4, cache.max_blocks);
            const int32_t* trow = table + (int64_t)it.b * cache.max_blocks;
            constexpr int kStride = kW * TTV_WAVE;
            bool bad = false;
            for (int e = (it.c0 >> 4) + tid; e < e_end; e += 4 * kStride) {
                int32_t v[4];
#pragma unroll
                for (int u = 0; u < 4; ++u) v[u] = e + u * kStride < e_end ? trow[e + u * kStride] : 0;
#pragma unroll
                for (int u = 0; u < 4; ++u) bad |= (uint32_t)v[u] >= (uint32_t)cache.num_blocks;
            }
            if (bad) atomicOr(err + it.b, TTV_ERR_BLOCK_TABLE);
        }
        // A full wait and a fenced barrier (not the loop's raw one, so the two
        // cannot be merged).
        __builtin_amdgcn_s_waitcnt(0);
        __syncthreads();
        // Q rotated in fp32 (the table carries scale * log2(e)), now that its
        // loads have landed (rotating at once would put their latency in front
        // of the tile loads); the bf16 result stays in registers.  Precise
        // items also keep the bf16 residual, in LDS swizzled like K, where
        // only this lane reads it.
#pragma unroll
        for (int mb = 0; mb < kMBr; ++mb) {
            const int rl = 16 * rblk[mb] + l16;
#pragma unroll
            for (int kc = 0; kc < KC; ++kc) {
                ttv_u32x4 hi, lo;
#pragma unroll
                for (int w = 0; w < 4; ++w) {
                    const float4 t4 = qtab[mb][kc][w >> 1];
                    const float c = (w & 1) ? t4.z : t4.x, sn = (w & 1) ? t4.w : t4.y;
                    const float x0 = ttv_bf16_lo(qraw[mb][kc][w]), x1 = ttv_bf16_hi(qraw[mb][kc][w]);
                    const float r0 = __builtin_fmaf(x0, c, -x1 * sn);
                    const float r1 = __builtin_fmaf(x1, c, x0 * sn);
                    hi[w] = pack_bf16(r0, r1);
                    lo[w] = pack_bf16(r0 - ttv_bf16_lo(hi[w]), r1 - ttv_bf16_hi(hi[w]));
                }
                qreg[mb][kc] = __builtin_bit_cast(ttv_bf16x8, hi);
                if (precise && mb < nmb)
                    *(ttv_u32x4*)(smem + (qlo_s - ring) + rl * MC::kRowBytes + 16 * swz_k(rl, 4 * kc + g4, P)) = lo;
            }
        }
        // Long-context items (8 stages) issue two tiles per barrier from the
        // loop, so their prologue leaves tiles 6 and 7 to the loop's first
        // barrier; precise items (4 stages) issue one tile per barrier.
        // Measured against one tile per barrier: contiguous 2-4 % faster,
        // paged about 3 % on the long Medusa workload.  A paged pair reads
        // its block numbers right before the wait that precedes its issue:
        // holding them from the previous iteration instead pushed the kernel
        // into spilling and ran it 30-50 % slower.
        const bool pairs = !precise;
        const int pro_end = pairs ? MC::kStagesLong - 2 : ahead;
        for (int j = 2; j < pro_end && j < n_tiles; ++j) issue(j, blocks_of(j));
        if (kPaged && precise && pro_end < n_tiles) next_blocks = blocks_of(pro_end);

        // The item body, compiled for NMB = 2, 1 and 0 row blocks per wave.
        auto body = [&](auto nmb_c) __attribute__((always_inline)) {
            constexpr int NMB = decltype(nmb_c)::value;
            ttv_f32x4 o[DB][kMB], lacc[kMB];
#pragma unroll
            for (int mb = 0; mb < NMB; ++mb) {
#pragma unroll
                for (int db = 0; db < DB; ++db) o[db][mb] = ttv_f32x4{0.f, 0.f, 0.f, 0.f};
                lacc[mb] = ttv_f32x4{0.f, 0.f, 0.f, 0.f};
            }
            float m_run[kMB];
#pragma unroll
            for (int mb = 0; mb < NMB; ++mb) m_run[mb] = kNegBig;

            // S^T[key][row] of tile tau: keys 16kb + 4g4 + r, rows 16mb + l16.
            auto scores = [&](auto cls, int tau, ttv_f32x4 (&S)[2][kMB]) __attribute__((always_inline)) {
                constexpr bool kPrecise = decltype(cls)::value == kClassPrecise;
                const char* kst = smem + (tau & smask) * MC::kStageBytes;
#pragma unroll
                for (int kc = 0; kc < KC; ++kc) {
                    ttv_bf16x8 qlo[kMB];
                    if (kPrecise) {
#pragma unroll
                        for (int mb = 0; mb < NMB; ++mb) {
                            const int rl = 16 * rblk[mb] + l16;
                            qlo[mb] = *(const ttv_bf16x8*)(smem + (qlo_s - ring) + rl * MC::kRowBytes +
                                                           16 * swz_k(rl, 4 * kc + g4, P));
                        }
                    }
#pragma unroll
                    for (int kb = 0; kb < 2; ++kb) {
                        const ttv_bf16x8 a = *(const ttv_bf16x8*)(kst + koff[kc] + kb * 16 * MC::kRowBytes);
#pragma unroll
                        for (int mb = 0; mb < NMB; ++mb) {
                            S[kb][mb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
                                a, qreg[mb][kc], kc == 0 ? ttv_f32x4{0.f, 0.f, 0.f, 0.f} : S[kb][mb], 0, 0, 0);
                            if (kPrecise)
                                S[kb][mb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, qlo[mb], S[kb][mb], 0, 0, 0);
                        }
                    }
                }
            };

            // Keys a row may not see become -inf: slots past the tile's valid
            // count and, on tree tiles, keys that are not the row node's
            // ancestors (or the node itself).  Branch-free.
            auto mask_scores = [&](int tau, ttv_f32x4 (&S)[2][kMB]) __attribute__((always_inline)) {
                const int valid = tile_valid(tau, tile_slot0(tau));
                const bool tree = tau >= n_ctx_tiles;
                const uint32_t vbits = valid >= 32 ? 0xFFFFFFFFu : ((1u << valid) - 1u);
                const int word = tree ? tau - n_ctx_tiles : 0;
#pragma unroll
                for (int mb = 0; mb < NMB; ++mb) {
                    const int nl = row_node[mb];
                    const uint32_t mw = mask_s[max(nl, 0) * mask_words + word];
                    const uint32_t w = (vbits & (tree ? (nl >= 0 ? mw : 0u) : 0xFFFFFFFFu)) >> (4 * g4);
#pragma unroll
                    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
                        for (int r = 0; r < 4; ++r)
                            S[kb][mb][r] = ((w >> (16 * kb + r)) & 1u) ? S[kb][mb][r] : -INFINITY;
                }
            };

            // This lane's part of each row maximum (the other three parts sit in
            // lanes l ^ 16, l ^ 32, l ^ 48).
            auto row_max = [&](const ttv_f32x4 (&S)[2][kMB], float (&tmax)[kMB]) __attribute__((always_inline)) {
#pragma unroll
                for (int mb = 0; mb < NMB; ++mb) {
                    const float t0 = __builtin_fmaxf(__builtin_fmaxf(S[0][mb][0], S[0][mb][1]),
                                                     __builtin_fmaxf(S[0][mb][2], S[0][mb][3]));
                    const float t1 = __builtin_fmaxf(__builtin_fmaxf(S[1][mb][0], S[1][mb][1]),
                                                     __builtin_fmaxf(S[1][mb][2], S[1][mb][3]));
                    tmax[mb] = __builtin_fmaxf(t0, t1);
                }
            };

            // Lazy rescale: the running max moves only when some row of the wave
            // outgrew it by more than 2^kLazyRescale (p stays below that
            // meanwhile); rare after the first tile.  Plain tiles carry shifted
            // scores s - m (the score MFMAs start from -m), the others raw ones.
            auto rescale_if_needed = [&](auto cls, ttv_f32x4 (&S)[2][kMB],
                                         const float (&tmax)[kMB]) __attribute__((always_inline)) {
                constexpr bool kShifted = decltype(cls)::value == kClassPlain;
                bool need = false;
#pragma unroll
                for (int mb = 0; mb < NMB; ++mb) need |= tmax[mb] > (kShifted ? kLazyRescale : m_run[mb] + kLazyRescale);
                if (__builtin_expect(__ballot(need) != 0, 0)) {
#pragma unroll
                    for (int mb = 0; mb < NMB; ++mb) {
                        float alpha;
                        if (kShifted) {
                            const float sh = __builtin_fmaxf(group_max(tmax[mb]), 0.f);
                            m_run[mb] += sh;
                            alpha = __builtin_amdgcn_exp2f(-sh);
#pragma unroll
                            for (int kb = 0; kb < 2; ++kb) S[kb][mb] -= sh;
                        } else {
                            const float m_new = __builtin_fmaxf(m_run[mb], group_max(tmax[mb]));
                            alpha = __builtin_amdgcn_exp2f(m_run[mb] - m_new);
                            m_run[mb] = m_new;
                        }
                        scale_in_place(lacc[mb], alpha);
#pragma unroll
                        for (int db = 0; db < DB; ++db) scale_in_place(o[db][mb], alpha);
                    }
                }
            };

            // p = 2^(s - m) as bf16 (plus, when precise, the bf16 of what the
            // rounding dropped).
            auto exp_pack = [&](auto cls, const ttv_f32x4 (&S)[2][kMB], ttv_bf16x8 (&pb)[kMB],
                                ttv_bf16x8 (&pl)[kMB]) __attribute__((always_inline)) {
                constexpr bool kPrecise = decltype(cls)::value == kClassPrecise;
                constexpr bool kShifted = decltype(cls)::value == kClassPlain;
#pragma unroll
                for (int mb = 0; mb < NMB; ++mb) {
                    float p[8];
#pragma unroll
                    for (int e = 0; e < 8; ++e)
                        p[e] = __builtin_amdgcn_exp2f(kShifted ? S[e >> 2][mb][e & 3] : S[e >> 2][mb][e & 3] - m_run[mb]);
                    uint32_t packed[4];
#pragma unroll
                    for (int e = 0; e < 4; ++e) packed[e] = pack_bf16(p[2 * e], p[2 * e + 1]);
                    pb[mb] = __builtin_bit_cast(ttv_bf16x8, ttv_u32x4{packed[0], packed[1], packed[2], packed[3]});
                    if (kPrecise) {
                        uint32_t lo[4];
#pragma unroll
                        for (int e = 0; e < 4; ++e)
                            lo[e] = pack_bf16(p[2 * e] - ttv_bf16_lo(packed[e]), p[2 * e + 1] - ttv_bf16_hi(packed[e]));
                        pl[mb] = __builtin_bit_cast(ttv_bf16x8, ttv_u32x4{lo[0], lo[1], lo[2], lo[3]});
                    }
                }
            };

            // O^T[d][row] += V^T[d][key] P^T[key][row] and l += 1^T P^T (an MFMA
            // against a ones operand, so l sums the same bf16 P that multiplies
            // V).  MFMA k index 8g4 + j is key 4g4 + j (j < 4) or 16 + 4g4 + j - 4
            // (j >= 4); each half comes from one ds_read_b64_tr_b16 over rows
            // 16h + 4g4 .. +3.
            auto load_vt = [&](int tau, int db) __attribute__((always_inline)) {
                const uint32_t vst = ring + (tau & smask) * MC::kStageBytes + MC::kTileBytes;
                ttv_i16x4 half[2];
#pragma unroll
                for (int h = 0; h < 2; ++h)
                    half[h] = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                        (lds_i16x4*)(uintptr_t)(vst + voff[db] + h * 16 * MC::kRowBytes));
                return __builtin_bit_cast(ttv_bf16x8,
                                          __builtin_shufflevector(half[0], half[1], 0, 1, 2, 3, 4, 5, 6, 7));
            };
            auto pv_half = [&](auto cls, int half, const ttv_bf16x8 (&va)[DB], const ttv_bf16x8 (&pb)[kMB],
                               const ttv_bf16x8 (&pl)[kMB]) __attribute__((always_inline)) {
                constexpr bool kPrecise = decltype(cls)::value == kClassPrecise;
#pragma unroll
                for (int db = half * DB / 2; db < (half + 1) * DB / 2; ++db)
#pragma unroll
                    for (int mb = 0; mb < NMB; ++mb) {
                        o[db][mb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(va[db], pb[mb], o[db][mb], 0, 0, 0);
                        if (kPrecise)
                            o[db][mb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(va[db], pl[mb], o[db][mb], 0, 0, 0);
                    }
                if (half == 1) {
#pragma unroll
                    for (int mb = 0; mb < NMB; ++mb) {
                        lacc[mb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kOnes, pb[mb], lacc[mb], 0, 0, 0);
                        if (kPrecise)
                            lacc[mb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kOnes, pl[mb], lacc[mb], 0, 0, 0);
                    }
                }
            };
            auto pv_mfma = [&](auto cls, const ttv_bf16x8 (&va)[DB], const ttv_bf16x8 (&pb)[kMB],
                               const ttv_bf16x8 (&pl)[kMB]) __attribute__((always_inline)) {
                constexpr bool kPrecise = decltype(cls)::value == kClassPrecise;
#pragma unroll
                for (int db = 0; db < DB; ++db)
#pragma unroll
                    for (int mb = 0; mb < NMB; ++mb) {
                        o[db][mb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(va[db], pb[mb], o[db][mb], 0, 0, 0);
                        if (kPrecise)
                            o[db][mb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(va[db], pl[mb], o[db][mb], 0, 0, 0);
                    }
#pragma unroll
                for (int mb = 0; mb < NMB; ++mb) {
                    lacc[mb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kOnes, pb[mb], lacc[mb], 0, 0, 0);
                    if (kPrecise)
                        lacc[mb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kOnes, pl[mb], lacc[mb], 0, 0, 0);
                }
            };

            // Before the scores of tile tau + 1: this wave's loads of that tile
            // have landed (the later ones up to tile tau + ahead - 1 may stay in
            // flight) and a barrier publishes them; the barrier also retires
            // stage (tau - 1) % stages, which the load of tile tau + ahead then
            // reuses.
            // Long-context classes (8 stages): at even tau, tiles tau + 1 and
            // tau + 2 must have landed (their scores are computed in iterations
            // tau and tau + 1); at most tiles tau + 3 .. tau + 5 stay in flight;
            // the barrier retires tiles tau - 2 and tau - 1, whose stages take
            // tiles tau + 6 and tau + 7.  Odd tau needs neither wait nor barrier.
            auto advance = [&](auto cls, int tau) __attribute__((always_inline)) {
                constexpr bool kPrecise = decltype(cls)::value == kClassPrecise;
                if constexpr (!kPrecise) {
                    if (tau & 1) return;
                    const int t0 = tau + MC::kStagesLong - 2;
                    // paged: the pair's block numbers are read here, right
                    // before the wait, so their latency hides behind it
                    TileBlocks b0 = next_blocks, b1 = next_blocks;
                    if (kPaged) {
                        if (t0 + 1 < n_plain) {
                            whole_pair_blocks(t0, b0, b1);
                        } else {
                            if (t0 < n_tiles) b0 = blocks_of(t0);
                            if (t0 + 1 < n_tiles) b1 = blocks_of(t0 + 1);
                        }
                    }
                    uint32_t offs[2 * MC::kCpw];
                    if (wave < MC::kIssueWaves) {
                        read_offsets(offs);
                        wait_vmcnt_tiles<MC::kOpsPerTile>(min(3, max(0, n_tiles - 3 - tau)));
                    }
                    raw_barrier();
                    if (t0 < n_tiles) {
                        if (t0 < n_plain) issue_whole(t0, b0, offs);
                        else issue(t0, b0);
                    }
                    if (t0 + 1 < n_tiles) {
                        if (t0 + 1 < n_plain) issue_whole(t0 + 1, b1, offs);
                        else issue(t0 + 1, b1);
                    }
                } else {
                    constexpr int kA = (kPrecise ? MC::kStagesShort : MC::kStagesLong) - 1;
                    if (tau + kA < n_tiles) {  // steady state: kA - 2 later tiles stay in flight
                        uint32_t offs[2 * MC::kCpw];
                        if (wave < MC::kIssueWaves) {
                            read_offsets(offs);
                            wait_vmcnt<MC::kOpsPerTile * (kA - 2)>();
                        }
                        raw_barrier();
                        if (tau + kA < n_plain) issue_whole(tau + kA, next_blocks, offs);
                        else issue(tau + kA, next_blocks);
                    } else {
                        if (wave < MC::kIssueWaves)
                            wait_vmcnt_tiles<MC::kOpsPerTile>(min(kA - 2, n_tiles - 2 - tau));
                        raw_barrier();
                    }
                }
            };

            // Software pipeline: iteration tau computes the scores of tile tau + 1
            // while it runs the softmax and P.V of tile tau, so the MFMAs of one
            // overlap the VALU work of the other.
            ttv_f32x4 S[2][kMB], S_next[2][kMB];
            float tmax[kMB];
            ttv_bf16x8 pb[kMB], pl[kMB];
            constexpr std::integral_constant<int, kClassPlain> cPlain{};
            constexpr std::integral_constant<int, kClassMasked> cMasked{};
            constexpr std::integral_constant<int, kClassPrecise> cPrecise{};
            auto first = [&](auto cls) __attribute__((always_inline)) {
                scores(cls, 0, S);
                if (decltype(cls)::value != kClassPlain) mask_scores(0, S);
                row_max(S, tmax);
                if (decltype(cls)::value == kClassPlain) {
                    // whole tile, every key visible: start the running max at the
                    // tile's row max and shift the scores by it
#pragma unroll
                    for (int mb = 0; mb < NMB; ++mb) {
                        m_run[mb] = group_max(tmax[mb]);
#pragma unroll
                        for (int kb = 0; kb < 2; ++kb) S[kb][mb] -= m_run[mb];
                        tmax[mb] -= m_run[mb];
                    }
                }
            };
            // One pipelined iteration: scores of tile tau + 1 (S_nxt), softmax
            // and P.V of tile tau (S_cur).  The work is cut into phases that the
            // scheduler may not mix (sched_barrier): each phase pairs one k-chunk
            // of score MFMAs with a quarter of the exponentials, and the LDS
            // reads of the next phase are issued one phase ahead; the last phase
            // runs the P.V MFMAs next to the mask and row maxima of tile tau + 1.
            auto iteration = [&](auto cur, auto next, int tau, ttv_f32x4 (&S_cur)[2][kMB],
                                 ttv_f32x4 (&S_nxt)[2][kMB]) __attribute__((always_inline)) {
                constexpr bool kCurPrecise = decltype(cur)::value == kClassPrecise;
                constexpr bool kNextPrecise = decltype(next)::value == kClassPrecise;
                constexpr bool kNextMasked = decltype(next)::value != kClassPlain;
                constexpr bool kCurShifted = decltype(cur)::value == kClassPlain;
                if (dyn && wave == 0 && tau == tau_claim) {
                    if (lane == 0)
                        claim = __hip_atomic_fetch_add(queue + xcd, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                }
                rescale_if_needed(cur, S_cur, tmax);
                advance(cur, tau);
                const char* kst = smem + ((tau + 1) & smask) * MC::kStageBytes;
                ttv_bf16x8 ka[KC][2], qlo[KC][kMB], va[DB];
                // plain scores start from -m (shifted), the others from 0
                ttv_f32x4 s_init[kMB];
#pragma unroll
                for (int mb = 0; mb < NMB; ++mb) {
                    const float z = kNextMasked ? 0.f : -m_run[mb];
                    s_init[mb] = ttv_f32x4{z, z, z, z};
                }
                auto load_k = [&](int kc) __attribute__((always_inline)) {
#pragma unroll
                    for (int kb = 0; kb < 2; ++kb)
                        ka[kc][kb] = *(const ttv_bf16x8*)(kst + koff[kc] + kb * 16 * MC::kRowBytes);
                    if (kNextPrecise) {
#pragma unroll
                        for (int mb = 0; mb < NMB; ++mb) {
                            const int rl = 16 * rblk[mb] + l16;
                            qlo[kc][mb] = *(const ttv_bf16x8*)(smem + (qlo_s - ring) + rl * MC::kRowBytes +
                                                               16 * swz_k(rl, 4 * kc + g4, P));
                        }
                    }
                };
                auto qk = [&](int kc) __attribute__((always_inline)) {
#pragma unroll
                    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
                        for (int mb = 0; mb < NMB; ++mb) {
                            S_nxt[kb][mb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
                                ka[kc][kb], qreg[mb][kc], kc == 0 ? s_init[mb] : S_nxt[kb][mb], 0, 0, 0);
                            if (kNextPrecise)
                                S_nxt[kb][mb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ka[kc][kb], qlo[kc][mb],
                                                                                        S_nxt[kb][mb], 0, 0, 0);
                        }
                };
                float p[kMB][8];
                uint32_t packed[kMB][4];
                auto ex = [&](int mb, int half) __attribute__((always_inline)) {
#pragma unroll
                    for (int e = 4 * half; e < 4 * half + 4; ++e)
                        p[mb][e] = __builtin_amdgcn_exp2f(kCurShifted ? S_cur[e >> 2][mb][e & 3]
                                                                      : S_cur[e >> 2][mb][e & 3] - m_run[mb]);
#pragma unroll
                    for (int e = 2 * half; e < 2 * half + 2; ++e)
                        packed[mb][e] = pack_bf16(p[mb][2 * e], p[mb][2 * e + 1]);
                };
                // A phase ends in a scheduling fence; inside it, the scheduler is
                // asked to alternate one MFMA with one VALU instruction and one
                // LDS read, so the wave issues VALU work and operand reads while
                // each MFMA runs (MFMA and VALU co-issue only when interleaved).
                // Measured against one MFMA per two VALU: about 2 % faster on the
                // long Medusa workload, the same elsewhere; three VALU, no
                // pattern, or a raised wave priority in the loop body were slower.
                auto phase = [] {
#pragma unroll
                    for (int i = 0; i < 9; ++i) {
                        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // MFMA
                        __builtin_amdgcn_sched_group_barrier(0x002, 1, 0);  // VALU
                        __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);  // LDS read
                    }
                    __builtin_amdgcn_sched_barrier(0);
                };
                // Phases for D = 128 (KC = 4); with D = 64 the last two carry no
                // score MFMAs.
                static_assert(KC == 2 || KC == 4, "head_dim 64 or 128");
                load_k(0);
                load_k(1);
#pragma unroll
                for (int db = 0; db < DB / 2; ++db) va[db] = load_vt(tau, db);
                phase();
                qk(0);
                if (NMB > 0) ex(0, 0);
                if (KC > 2) load_k(2);
                phase();
                qk(1);
                if (NMB > 0) ex(0, 1);
                if (KC > 2) load_k(3);
                phase();
                if (KC > 2) qk(2);
                if (NMB > 1) ex(1, 0);
                phase();
                if (KC > 2) qk(3);
                if (NMB > 1) ex(1, 1);
#pragma unroll
                for (int mb = 0; mb < NMB; ++mb) {
                    pb[mb] = __builtin_bit_cast(ttv_bf16x8, ttv_u32x4{packed[mb][0], packed[mb][1], packed[mb][2],
                                                                      packed[mb][3]});
                    if (kCurPrecise) {
                        uint32_t lo[4];
#pragma unroll
                        for (int e = 0; e < 4; ++e)
                            lo[e] = pack_bf16(p[mb][2 * e] - ttv_bf16_lo(packed[mb][e]),
                                              p[mb][2 * e + 1] - ttv_bf16_hi(packed[mb][e]));
                        pl[mb] = __builtin_bit_cast(ttv_bf16x8, ttv_u32x4{lo[0], lo[1], lo[2], lo[3]});
                    }
                }
                phase();
                // P.V in two halves; the V^T operands of the second half load
                // while the first half runs.
                pv_half(cur, 0, va, pb, pl);
#pragma unroll
                for (int db = DB / 2; db < DB; ++db) va[db] = load_vt(tau, db);
                phase();
                pv_half(cur, 1, va, pb, pl);
                if (kNextMasked) mask_scores(tau + 1, S_nxt);
                row_max(S_nxt, tmax);
                phase();
                // A paged cache's block numbers for the tile the next iteration
                // loads: read now, so the scalar loads return during its barrier.
                if constexpr (kPaged && kCurPrecise) {
                    const int t = tau + MC::kStagesShort;
                    if (t < n_tiles) next_blocks = blocks_of(t);
                }
            };
            auto copy_scores = [&](ttv_f32x4 (&dst)[2][kMB], const ttv_f32x4 (&src)[2][kMB]) __attribute__((always_inline)) {
#pragma unroll
                for (int kb = 0; kb < 2; ++kb)
#pragma unroll
                    for (int mb = 0; mb < NMB; ++mb) dst[kb][mb] = src[kb][mb];
            };
            auto last = [&](auto cur, int tau) __attribute__((always_inline)) {
                rescale_if_needed(cur, S, tmax);
                exp_pack(cur, S, pb, pl);
                ttv_bf16x8 va[DB];
#pragma unroll
                for (int db = 0; db < DB; ++db) va[db] = load_vt(tau, db);
                pv_mfma(cur, va, pb, pl);
            };
            // Runs tiles [tau, end) of one class; the tile after them (if any) is
            // of class `after`.  Two iterations per trip, so the two score sets
            // swap roles without copies.
            auto run = [&](auto cls, auto after, int& tau, int end) __attribute__((always_inline)) {
                for (; tau + 2 < end; tau += 2) {
                    iteration(cls, cls, tau, S, S_next);
                    iteration(cls, cls, tau + 1, S_next, S);
                }
                if (tau + 1 < end) {
                    iteration(cls, cls, tau, S, S_next);
                    copy_scores(S, S_next);
                    ++tau;
                }
                if (tau < end) {
                    if (tau + 1 < n_tiles) {
                        iteration(cls, after, tau, S, S_next);
                        copy_scores(S, S_next);
                    } else {
                        last(cls, tau);
                    }
                    ++tau;
                }
            };
            int tau = 0;
            if (precise) {
                first(cPrecise);
                run(cPrecise, cPrecise, tau, n_tiles);
            } else {
                if (n_plain > 0) first(cPlain);
                else first(cMasked);
                run(cPlain, cMasked, tau, n_plain);
                run(cMasked, cMasked, tau, n_tiles);
            }

            float l_run[kMB];
#pragma unroll
            for (int mb = 0; mb < NMB; ++mb) l_run[mb] = lacc[mb][0];
            // Lane holds O^T[d = 16db + 4g4 + r][row 16mb + l16]; the lane's
            // indices come from fresh_lane (the output addresses were held
            // across the loop, spilled, and reloaded behind a full wait).
            const int lane_e = fresh_lane();
            const int l16e = lane_e & 15, g4e = lane_e >> 4;
            // 16-byte stores: lanes g4 and g4 ^ 1 (rows of 16 lanes, swapped by
            // v_permlane16_swap) trade halves of their 8-byte pieces of head-dim
            // blocks 2k (X) and 2k + 1 (Y), so an even lane stores X of both
            // (columns 32k + 4g4 .. + 7) and an odd lane Y of both (columns
            // 32k + 16 + 4(g4 - 1) .. + 7): the four lanes of a row cover 64
            // contiguous bytes per store.  Both lanes of a pair hold the same
            // row, so they skip rows together.
            const bool odd = g4e & 1;
            auto pair16 = [&](ttv_u32x2 X, ttv_u32x2 Y) __attribute__((always_inline)) {
                const auto r0 = __builtin_amdgcn_permlane16_swap(X[0], Y[0], false, false);
                const auto r1 = __builtin_amdgcn_permlane16_swap(X[1], Y[1], false, false);
                return odd ? ttv_u32x4{r0[0], r1[0], Y[0], Y[1]} : ttv_u32x4{X[0], X[1], r0[1], r1[1]};
            };
            const int col16 = odd ? 16 + 4 * (g4e - 1) : 4 * g4e;  // + 32k
#pragma unroll
            for (int mb = 0; mb < NMB; ++mb) {
                const int r_local = 16 * rblk[mb] + l16e;
                const int r = it.tile * kTileR + r_local;
                if (r >= rows) continue;
                if (it.pslot < 0) {
                    const int node = r / G, g = r % G;
                    if (!TTV_DCHECK((int64_t)it.s + node < dbg_nodes, TTV_SITE_MAIN_OUT)) continue;
                    uint16_t* dst = out + ((int64_t)(it.s + node) * Hq + it.kvh * G + g) * D;
                    const float inv_l = 1.0f / l_run[mb];
                    auto piece = [&](int db) __attribute__((always_inline)) {
                        ttv_u32x2 w;
                        w[0] = pack_bf16(o[db][mb][0] * inv_l, o[db][mb][1] * inv_l);
                        w[1] = pack_bf16(o[db][mb][2] * inv_l, o[db][mb][3] * inv_l);
                        return w;
                    };
#pragma unroll
                    for (int k = 0; k < DB / 2; ++k)
                        *(ttv_u32x4*)(dst + 32 * k + col16) = pair16(piece(2 * k), piece(2 * k + 1));
                } else {
                    // Partial: o / l scaled by a power of two 2^-e that brings the
                    // row's largest |o / l| into [0.5, 1), as fp16 (11-bit
                    // precision relative to that maximum); (m, l, 2^e) beside it.
                    const float inv_l = 1.0f / l_run[mb];
                    float amax = 0.f;
#pragma unroll
                    for (int db = 0; db < DB; ++db)
#pragma unroll
                        for (int q = 0; q < 4; ++q) amax = __builtin_fmaxf(amax, __builtin_fabsf(o[db][mb][q]));
                    const int e = __builtin_amdgcn_frexp_expf(group_max(amax) * inv_l);
                    const float sc = __builtin_amdgcn_ldexpf(inv_l, -e);
                    if (!TTV_DCHECK(it.pslot < dbg_partials, TTV_SITE_MAIN_OUT)) continue;
                    ttv_f16x4* dst = part_o + (((int64_t)it.pslot * kTileR + r_local) * D) / 4;
                    auto piece = [&](int db) __attribute__((always_inline)) {
                        return __builtin_bit_cast(ttv_u32x2, __builtin_convertvector(o[db][mb] * sc, ttv_f16x4));
                    };
#pragma unroll
                    for (int k = 0; k < DB / 2; ++k)
                        *(ttv_u32x4*)(dst + (32 * k + col16) / 4) = pair16(piece(2 * k), piece(2 * k + 1));
                    if (g4e == 0)
                        part_ml[(int64_t)it.pslot * kTileR + r_local] =
                            make_float4(m_run[mb], l_run[mb], __builtin_amdgcn_ldexpf(1.0f, e), 0.f);
                }
            }
        };
        {
            if constexpr (kMBr == 2) {
                if (nmb == 2) body(std::integral_constant<int, 2>{});
                else if (nmb == 1) body(std::integral_constant<int, 1>{});
                else body(std::integral_constant<int, 0>{});
            } else {
                if (nmb >= 1) body(std::integral_constant<int, 1>{});
                else body(std::integral_constant<int, 0>{});
            }
        }
        // the claimed next item, for every wave after the barrier below (the
        // write has landed before wave 0 reaches it)
        if (dyn && wave == 0) {
            if (lane == 0) s_next[k & 1] = per_xcd + claim;
            __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0)
        }
        // The next item reuses the LDS (ring, Q-lo, mask): a barrier, but no
        // memory fence.  Every LDS read of this item has fed an MFMA or a
        // store by now and every tile load has landed, while the item's
        // output stores may stay in flight into the next item (nothing in
        // this kernel reads them): they retire under its prologue wait
        // instead of delaying this barrier (about 3 us per item).
        raw_barrier();
        if (dyn) {
            const int i = s_next[k & 1];
            if (i < n_xcd) {
                slot = i * kNumXcd + xcd;
            } else {
                // This XCD's list is used up and the workgroup is idle: take
                // an item from the XCD with the most left (the XCDs do not
                // run at the same speed).  Claimed only now, not one item
                // ahead, so a stolen item never waits behind a running one.
                if (tid == 0) s_next[2] = steal_item(queue, grid, n_items);
                __syncthreads();
                slot = s_next[2];
            }
            more = slot >= 0;
        } else {
            more = false;
        }
    }
}

template <int D, int kW, int kRows>
size_t main_lds_bytes(int G, int mask_words) {
    using MC = MainCfg<D, kW, kRows>;
    const int nodes = MC::kTile / G + 2;
    const size_t mask_bytes = (size_t)((nodes * mask_words + 63) / 64) * 256;
    return (size_t)MC::kMaskOffset + mask_bytes;
}

// ---------------------------------------------------------------------------
// 3. Combine: merge the chunk partials of split row tiles.
// ---------------------------------------------------------------------------

template <int D, int kTileR>
__global__ __launch_bounds__(kCombThreads) void attn_combine_kernel(
    const PlanHeader* __restrict__ hdr, const Combine* __restrict__ combine, int Hq, int Hkv,
    const ttv_f16x4* __restrict__ part_o, const float4* __restrict__ part_ml,
    uint16_t* __restrict__ out) {
    constexpr int kLanesPerRow = D / 8;                 // each lane: 8 consecutive d (16 bytes)
    constexpr int kRowsPerPass = kCombThreads / kLanesPerRow;
    constexpr int kRowBlocks = kTileR / kRowsPerPass;
    const int n_work = hdr->n_combine * kRowBlocks;
    const int G = Hq / Hkv;
    const int tid = threadIdx.x;
#ifdef TTV_DEBUG
    const int64_t dbg_nodes = hdr->reserved[0], dbg_partials = hdr->reserved[1];
#endif
    // A workgroup's units are wk = blockIdx.x + i * gridDim.x; the next
    // unit's descriptor is loaded while this one merges.
    Combine cb_next;
    if (blockIdx.x < n_work) cb_next = combine[blockIdx.x / kRowBlocks];
    for (int wk = blockIdx.x; wk < n_work; wk += gridDim.x) {
        const Combine cb = cb_next;
        if (wk + (int)gridDim.x < n_work) cb_next = combine[(wk + gridDim.x) / kRowBlocks];
        const int r_local = (wk % kRowBlocks) * kRowsPerPass + tid / kLanesPerRow;
        const int d = (tid % kLanesPerRow) * 8;
        const int r = cb.tile * kTileR + r_local;
        if (r >= cb.n * G) continue;
        if (!TTV_DCHECK(cb.pslot0 >= 0 && cb.pslot0 + (int64_t)(cb.nc - 1) * cb.stride < dbg_partials &&
                            (int64_t)cb.s + r / G < dbg_nodes,
                        TTV_SITE_COMBINE))
            continue;
        // Chunks in batches of NB: every load of a batch is issued before any
        // is used, so one memory latency covers the batch; the batch maximum
        // then rescales the running sums once.  Past the last chunk the
        // loads repeat it (in bounds, no branch) and count zero; NB = 4 for
        // tiles of at most 4 chunks keeps those repeats few.
        float mmax = kNegBig, lsum = 0.f;
        ttv_f32x4 acc0 = {0.f, 0.f, 0.f, 0.f}, acc1 = {0.f, 0.f, 0.f, 0.f};
        auto merge = [&](auto nb_c) __attribute__((always_inline)) {
            constexpr int NB = decltype(nb_c)::value;
            for (int c0 = 0; c0 < cb.nc; c0 += NB) {
                float4 ml[NB];  // m, l, scale of the fp16 o / l
                ttv_u32x4 ov[NB];
#pragma unroll
                for (int j = 0; j < NB; ++j) {
                    const int c = min(c0 + j, cb.nc - 1);
                    const int64_t ps = cb.pslot0 + (int64_t)c * cb.stride;
                    ml[j] = part_ml[ps * kTileR + r_local];
                    ov[j] = *(const ttv_u32x4*)(part_o + ((ps * kTileR + r_local) * D + d) / 4);
                }
                float m_new = mmax;
#pragma unroll
                for (int j = 0; j < NB; ++j) m_new = fmaxf(m_new, ml[j].x);
                const float a_old = __builtin_amdgcn_exp2f(mmax - m_new);
                lsum *= a_old;
                acc0 *= a_old;
                acc1 *= a_old;
#pragma unroll
                for (int j = 0; j < NB; ++j) {
                    const float e = __builtin_amdgcn_exp2f(ml[j].x - m_new) * ml[j].y;
                    const float a = c0 + j < cb.nc ? e : 0.f;
                    const float w = a * ml[j].z;
                    lsum += a;
                    const ttv_f16x4 h0 = __builtin_bit_cast(ttv_f16x4, ttv_u32x2{ov[j][0], ov[j][1]});
                    const ttv_f16x4 h1 = __builtin_bit_cast(ttv_f16x4, ttv_u32x2{ov[j][2], ov[j][3]});
                    acc0 += __builtin_convertvector(h0, ttv_f32x4) * w;
                    acc1 += __builtin_convertvector(h1, ttv_f32x4) * w;
                }
                mmax = m_new;
            }
        };
        if (cb.nc <= 4) merge(std::integral_constant<int, 4>{});
        else merge(std::integral_constant<int, kCombBatch>{});
        const float inv = 1.0f / lsum;
        const int node = r / G, g = r % G;
        uint16_t* dst = out + ((int64_t)(cb.s + node) * Hq + cb.kvh * G + g) * D + d;
        ttv_u32x4 w4;
        w4[0] = ttv_pack_bf16x2(acc0[0] * inv, acc0[1] * inv);
        w4[1] = ttv_pack_bf16x2(acc0[2] * inv, acc0[3] * inv);
        w4[2] = ttv_pack_bf16x2(acc1[0] * inv, acc1[1] * inv);
        w4[3] = ttv_pack_bf16x2(acc1[2] * inv, acc1[3] * inv);
        *(ttv_u32x4*)dst = w4;
    }
}

// Per-device host state: the CU count and which kernels already had their
// dynamic-LDS limit raised (a function attribute is set per device).
// Atomics, so concurrent calls from several host threads stay well defined.
constexpr int kMaxDevices = 64;
struct DeviceState {
    std::atomic<int> cus{0};
    std::atomic<unsigned> lds_raised{0};
};
DeviceState g_device[kMaxDevices];

DeviceState& device_state() {
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) dev = 0;
    return g_device[dev];
}

int num_cus() {
    DeviceState& st = device_state();
    int cus = st.cus.load(std::memory_order_relaxed);
    if (cus > 0) return cus;
    int dev = 0;
    cus = 0;
    if (hipGetDevice(&dev) != hipSuccess ||
        hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
        cus <= 0)
        cus = 256;
    st.cus.store(cus, std::memory_order_relaxed);
    return cus;
}

// Raises a kernel's dynamic-LDS limit once per device; `bit` names the kernel.
bool raise_lds_limit(const void* kern, unsigned bit, int bytes) {
    DeviceState& st = device_state();
    if (st.lds_raised.load(std::memory_order_acquire) & bit) return true;
    if (hipFuncSetAttribute(kern, hipFuncAttributeMaxDynamicSharedMemorySize, bytes) != hipSuccess)
        return false;
    st.lds_raised.fetch_or(bit, std::memory_order_release);
    return true;
}

bool valid_common(const ttv_batch* bt, const ttv_kv_cache* c, int32_t n_heads) {
    if (!bt || !c) return false;
    if (bt->batch < 0 || bt->batch > kMaxBatch || bt->n_max < 0 ||
        bt->n_max > TTV_MAX_TREE_NODES || bt->total_nodes < 0 ||
        bt->total_nodes > (int64_t)bt->batch * bt->n_max)
        return false;
    if (c->head_dim != 64 && c->head_dim != 128) return false;
    if (c->n_kv_heads < 1 || n_heads < 1 || n_heads % c->n_kv_heads != 0) return false;
    if (n_heads / c->n_kv_heads > 64) return false;
    if (c->layout == TTV_KV_CONTIGUOUS) {
        if (c->capacity < 0) return false;
    } else if (c->layout == TTV_KV_PAGED) {
        if (c->block_size != TTV_BLOCK_SIZE || c->max_blocks < 1 || c->num_blocks < 1) return false;
    } else {
        return false;
    }
    return true;
}

template <int D>
int launch_attention(const ttv_batch* bt, const uint16_t* q, const uint16_t* k_new,
                     const uint16_t* v_new, const uint32_t* mask, int32_t mask_words,
                     const int32_t* positions, const ttv_kv_cache* cache, int32_t n_heads,
                     float rope_base, double scale, uint16_t* out, char* ws, const Layout& L,
                     int32_t* err, hipStream_t stream) {
    CacheView cv;
    cv.k = (uint16_t*)cache->k;
    cv.v = (uint16_t*)cache->v;
    cv.table = cache->block_table;
    cv.paged = cache->layout == TTV_KV_PAGED;
    cv.hkv = cache->n_kv_heads;
    cv.cap = cache->capacity;
    cv.max_blocks = cache->max_blocks;
    cv.num_blocks = cache->num_blocks;
    PlanHeader* hdr = (PlanHeader*)ws;
    Item* items = (Item*)(ws + L.off_items);
    Combine* comb = (Combine*)(ws + L.off_combine);
    float2* rope_cs = (float2*)(ws + L.off_rope);
    ttv_f16x4* po = (ttv_f16x4*)(ws + L.off_po);
    float4* pml = (float4*)(ws + L.off_pml);
    const double q_mult = scale * 1.4426950408889634074;  // scores come out in log2 units
    RopeTable rope;
    for (int m = 0; m < 64; ++m) rope.inv[m] = m < D / 2 ? pow((double)rope_base, -2.0 * m / D) : 0.0;
    // Few row tiles (a small batch): 128-row items, about one item per CU;
    // otherwise 256-row items, a few per CU.
    const int G = n_heads / cache->n_kv_heads;
    const int64_t tiles256 =
        (int64_t)bt->batch * cache->n_kv_heads * (((int64_t)bt->n_max * G + kTileM - 1) / kTileM);
    // 256-row items need the mask rows of up to 256 / G + 2 nodes beside the
    // 128 KB ring; when those do not fit in 160 KB of LDS (one query head per
    // KV head with trees over 992 nodes) the 128-row items run instead.
    constexpr size_t kLdsLimit = 160 * 1024;
    const bool small = tiles256 < num_cus() || main_lds_bytes<D, 8, kTileM>(G, mask_words) > kLdsLimit;
    // Checked before anything is launched, so a rejected call has no effect.
    if (main_lds_bytes<D, 8, kTileMin>(G, mask_words) > kLdsLimit) return TTV_EINVAL;
    const int tile_m = small ? kTileMin : kTileM;
    const int target_items = small ? num_cus() : kTargetItems;
    const int cus = num_cus();
    int64_t grid = (int64_t)cus;  // one workgroup per CU (LDS and registers bound it)
    if (grid > L.max_items) grid = ((L.max_items + kNumXcd - 1) / kNumXcd) * kNumXcd;
    grid = ((grid + kNumXcd - 1) / kNumXcd) * kNumXcd;
    if (grid > kMaxGrid) grid = kMaxGrid;
    dim3 prep_grid((unsigned)(1 + (bt->total_nodes + kPrepNodes - 1) / kPrepNodes));  // plan + nodes
    const size_t prep_lds = (size_t)4 * (bt->batch + 1) * sizeof(int32_t);
    if (!raise_lds_limit((const void*)attn_prep_kernel<D>, D == 128 ? 1u : 2u, 80 * 1024))
        return TTV_EHIP;
    hipLaunchKernelGGL(attn_prep_kernel<D>, prep_grid, dim3(kPrepThreads), prep_lds, stream,
                       bt->node_offsets, bt->ctx_lens, bt->batch, bt->n_max, bt->total_nodes,
                       k_new, v_new, positions, cv, n_heads, rope, q_mult, rope_cs, tile_m,
                       target_items, (int)grid, hdr, items,
                       comb, L.max_items, L.max_groups, L.max_partials, (int2*)(ws + L.off_glist),
                       (int32_t*)(ws + L.off_gpos), err);
    if (hipGetLastError() != hipSuccess) return TTV_EHIP;
    auto run_main = [&](auto rows) -> int {
        constexpr int kW = 8;
        constexpr int kRows = decltype(rows)::value;
        using MC = MainCfg<D, kW, kRows>;
        const size_t lds = main_lds_bytes<D, kW, kRows>(n_heads / cache->n_kv_heads, mask_words);
        auto kern = cv.paged ? attn_main_kernel<D, true, kW, kRows> : attn_main_kernel<D, false, kW, kRows>;
        // one bit per main-kernel variant (head dim, layout, row tile)
        const unsigned bit = 4u << ((D == 128 ? 0 : 4) + (cv.paged ? 0 : 2) + (kRows == kTileM ? 0 : 1));
        if (!raise_lds_limit((const void*)kern, bit, 160 * 1024)) return TTV_EHIP;
        hipLaunchKernelGGL(kern, dim3((unsigned)grid), dim3(kW * TTV_WAVE), lds, stream, hdr, items,
                           q, rope_cs, mask, mask_words, cv, cache->block_table, n_heads, out, po,
                           pml, hdr->queue, err);
        if (hipGetLastError() != hipSuccess) return TTV_EHIP;
        hipLaunchKernelGGL((attn_combine_kernel<D, MC::kTile>), dim3((unsigned)(4 * cus)), dim3(kCombThreads), 0,
                           stream, hdr, comb, n_heads, cache->n_kv_heads, po, pml, out);
        return hipGetLastError() == hipSuccess ? TTV_OK : TTV_EHIP;
    };
    return small ? run_main(std::integral_constant<int, kTileMin>{})
                 : run_main(std::integral_constant<int, kTileM>{});
}

}  // namespace

extern "C" TTV_API size_t tree_attention_workspace_bytes(const ttv_batch* bt,
                                                         const ttv_kv_cache* cache,
                                                         int32_t n_heads) {
    if (!valid_common(bt, cache, n_heads)) return 0;
    return make_layout(bt->batch, bt->total_nodes, n_heads, cache->n_kv_heads, cache->head_dim)
        .total;
}

extern "C" TTV_API int tree_attention_verify(const ttv_batch* bt, const void* q, const void* k_new,
                                             const void* v_new, const uint32_t* mask,
                                             int32_t mask_words, const int32_t* positions,
                                             const ttv_kv_cache* cache, int32_t n_heads,
                                             float rope_base, float softmax_scale, void* out,
                                             void* workspace, size_t workspace_bytes,
                                             int32_t* err, hipStream_t stream) {
    if (!valid_common(bt, cache, n_heads)) return TTV_EINVAL;
    if (!(rope_base > 0.f) || softmax_scale < 0.f) return TTV_EINVAL;
    if (mask_words < (bt->n_max + 31) / 32 || mask_words > TTV_MAX_TREE_NODES / 32) return TTV_EINVAL;
    if (bt->batch == 0) return TTV_OK;
    if (!bt->node_offsets || !bt->ctx_lens || !cache->k || !cache->v || !err || !workspace)
        return TTV_EINVAL;
    if (cache->layout == TTV_KV_PAGED && !cache->block_table) return TTV_EINVAL;
    if (bt->total_nodes > 0 && (!q || !k_new || !v_new || !mask || !positions || !out))
        return TTV_EINVAL;
    if (((uintptr_t)workspace & 255) ||
        (((uintptr_t)q | (uintptr_t)k_new | (uintptr_t)v_new | (uintptr_t)out |
          (uintptr_t)cache->k | (uintptr_t)cache->v) & 15))
        return TTV_EINVAL;
    const Layout L =
        make_layout(bt->batch, bt->total_nodes, n_heads, cache->n_kv_heads, cache->head_dim);
    if (workspace_bytes < L.total) return TTV_ENOSPC;
    const double scale =
        softmax_scale > 0.f ? (double)softmax_scale : 1.0 / sqrt((double)cache->head_dim);
    if (cache->head_dim == 128)
        return launch_attention<128>(bt, (const uint16_t*)q, (const uint16_t*)k_new,
                                     (const uint16_t*)v_new, mask, mask_words, positions, cache,
                                     n_heads, rope_base, scale, (uint16_t*)out, (char*)workspace,
                                     L, err, stream);
    return launch_attention<64>(bt, (const uint16_t*)q, (const uint16_t*)k_new,
                                (const uint16_t*)v_new, mask, mask_words, positions, cache,
                                n_heads, rope_base, scale, (uint16_t*)out, (char*)workspace, L,
                                err, stream);
}

TTV_DEBUG_TU(attention)
