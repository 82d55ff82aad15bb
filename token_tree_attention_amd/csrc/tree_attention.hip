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
//  1. attn_prep_kernel, one workgroup per node: rotates that node's Q (all
//     query heads, pre-multiplied by scale*log2(e), bf16) into the workspace
//     and its K (bf16) plus V into the tentative cache slots ctx + i.  Angles
//     are reduced in fp64 before the fp32 sin/cos.  One extra workgroup
//     builds the work plan on the device (no host round trip).
//  2. attn_main_kernel, persistent: a work item is (request, KV head, row
//     tile of 256 query rows, slot chunk).  Rows are (node, query head of the
//     GQA group) pairs, node-major, so every context K/V byte feeds all rows
//     of its KV head.  Each of 4 waves owns 64 rows and keeps their Q in
//     registers.  K and V tiles of 32 slots are staged in LDS (V transposed)
//     with one tile in flight while the previous one is consumed.  S^T = K Q^T
//     and O^T += V^T P^T run on v_mfma_f32_16x16x32_bf16, so P^T comes out of
//     the score accumulators already in the B-operand layout.  Online softmax
//     in fp32 (exp2 domain).  The tree part of a row tile is the last chunk:
//     tree keys 32 at a time, masked by one word of each row's ancestor mask.
//     Items are laid out so that the row tiles of one slot chunk are
//     consecutive and land on one XCD (blockIdx -> XCD-major virtual id),
//     where their repeated K/V reads hit that XCD's L2.
//  3. attn_combine_kernel: log-sum-exp merge of the chunks of row tiles whose
//     context was split; single-chunk tiles are written directly by step 2.

#include <type_traits>

#include "ttv_device.h"

namespace {

constexpr int kWaves = 4;
constexpr int kRowsPerWave = 64;
constexpr int kTileM = kWaves * kRowsPerWave;
constexpr int kThreads = kWaves * TTV_WAVE;
constexpr int kKT = 32;                 // key slots per LDS tile (= one mask word)
constexpr int kTargetItems = 1024;      // chunking aims at about this many work items
constexpr int kChunkMin = 256;          // shortest context chunk (slots)
constexpr int kMaxBatch = 4096;         // plan keeps per-request prefix sums in LDS
constexpr int kNumXcd = 8;
constexpr int kPreciseCtx = 256;       // requests with a shorter context run every tile precise
constexpr float kNegBig = -1.0e30f;

struct PlanHeader {
    int32_t n_items;
    int32_t n_combine;
    int32_t chunk_len;
    int32_t reserved[61];
};

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
    size_t off_items, off_combine, off_q, off_qlo, off_po, off_pml, total;
};

size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

Layout make_layout(int64_t B, int64_t T, int64_t Hq, int64_t Hkv, int64_t D) {
    Layout L;
    const int64_t G = Hq / Hkv;
    L.max_groups = Hkv * ((T * G + kTileM - 1) / kTileM + B);
    L.max_items = kTargetItems + L.max_groups;
    L.max_partials = 2 * kTargetItems;
    size_t off = align256(sizeof(PlanHeader));
    L.off_items = off;
    off = align256(off + (size_t)L.max_items * sizeof(Item));
    L.off_combine = off;
    off = align256(off + (size_t)L.max_groups * sizeof(Combine));
    L.off_q = off;
    off = align256(off + (size_t)T * Hq * D * 2);
    L.off_qlo = off;
    off = align256(off + (size_t)T * Hq * D * 2);
    L.off_po = off;
    off = align256(off + (size_t)L.max_partials * kTileM * D * 4);
    L.off_pml = off;
    off = align256(off + (size_t)L.max_partials * kTileM * 8);
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

// ---------------------------------------------------------------------------
// 1. Prep: RoPE of Q (into the workspace) and K (into the cache), V copy, and
//    (one extra workgroup) the work plan.
// ---------------------------------------------------------------------------

__device__ void build_plan(const int32_t* __restrict__ node_offsets,
                           const int32_t* __restrict__ ctx_lens, int B, int n_max,
                           int64_t total_nodes, int G, int Hkv, int cap_limit,
                           PlanHeader* hdr, Item* items, Combine* combine, int64_t max_items,
                           int64_t max_groups, int64_t max_partials, int32_t* err) {
    __shared__ int32_t s_items[kMaxBatch + 1];
    __shared__ int32_t s_parts[kMaxBatch + 1];
    __shared__ unsigned long long s_work;
    __shared__ int32_t s_carry_items, s_carry_parts, s_ncomb;
    __shared__ int32_t t_i[kThreads], t_p[kThreads];
    const int tid = threadIdx.x;
    if (tid == 0) {
        s_work = 0;
        s_ncomb = 0;
    }
    __syncthreads();
    // Phase 1: total slot work, W = Hkv * sum over row tiles of (ctx + tree keys).
    unsigned long long my_work = 0;
    for (int b = tid; b < B; b += kThreads) {
        const int s = node_offsets[b];
        const int n = node_offsets[b + 1] - s;
        const int ctx = ctx_lens[b];
        if (s < 0 || n < 0 || n > n_max || (int64_t)s + n > total_nodes || ctx < 0) continue;
        if (cap_limit >= 0 && (int64_t)ctx + n > cap_limit) continue;
        const int rows = n * G;
        const int nt = (rows + kTileM - 1) / kTileM;
        for (int t = 0; t < nt; ++t) {
            const int last_row = min((t + 1) * kTileM, rows) - 1;
            my_work += (unsigned long long)(ctx + last_row / G + 1);
        }
    }
    my_work *= (unsigned long long)Hkv;
    atomicAdd(&s_work, my_work);
    __syncthreads();
    const unsigned long long W = s_work;
    long long cl = (long long)((W + kTargetItems - 1) / kTargetItems);
    cl = ((cl + kKT - 1) / kKT) * kKT;
    if (cl < kChunkMin) cl = kChunkMin;
    if (cl > (1ll << 30)) cl = 1ll << 30;
    const int chunk_len = (int)cl;

    // Phase 2: per-request item and partial counts, exclusive prefix sums.
    if (tid == 0) {
        s_carry_items = 0;
        s_carry_parts = 0;
    }
    __syncthreads();
    for (int base = 0; base < B; base += kThreads) {
        const int b = base + tid;
        int ni = 0, np = 0;
        if (b < B) {
            const int s = node_offsets[b];
            const int n = node_offsets[b + 1] - s;
            const int ctx = ctx_lens[b];
            bool ok = !(s < 0 || n < 0 || n > n_max || (int64_t)s + n > total_nodes || ctx < 0);
            if (ok && cap_limit >= 0 && (int64_t)ctx + n > cap_limit) {
                ok = false;
                atomicOr(err + b, TTV_ERR_CAPACITY);
            }
            if (ok && n > 0) {
                const int nt = (n * G + kTileM - 1) / kTileM;
                const int nc = ctx > chunk_len ? (ctx + chunk_len - 1) / chunk_len : 1;
                ni = Hkv * nt * nc;
                np = nc > 1 ? ni : 0;
            }
        }
        // inclusive scan over the workgroup (Hillis-Steele in LDS)
        t_i[tid] = ni;
        t_p[tid] = np;
        __syncthreads();
        for (int off = 1; off < kThreads; off <<= 1) {
            const int ai = tid >= off ? t_i[tid - off] : 0;
            const int ap = tid >= off ? t_p[tid - off] : 0;
            __syncthreads();
            t_i[tid] += ai;
            t_p[tid] += ap;
            __syncthreads();
        }
        if (b < B) {
            s_items[b] = s_carry_items + t_i[tid] - ni;
            s_parts[b] = s_carry_parts + t_p[tid] - np;
        }
        __syncthreads();
        if (tid == kThreads - 1) {
            s_carry_items += t_i[tid];
            s_carry_parts += t_p[tid];
        }
        __syncthreads();
    }
    if (tid == 0) {
        s_items[B] = s_carry_items;
        s_parts[B] = s_carry_parts;
    }
    __syncthreads();
    int n_items = s_items[B];
    // Both bounds hold by construction of chunk_len (see make_layout); stay safe anyway.
    if (n_items > max_items || s_parts[B] > max_partials) n_items = 0;

    // Phase 3: item descriptors (request found by binary search on the prefix).
    for (int x = tid; x < n_items; x += kThreads) {
        int lo = 0, hi = B - 1;
        while (lo < hi) {  // last b with s_items[b] <= x
            const int mid = (lo + hi + 1) >> 1;
            if (s_items[mid] <= x) lo = mid;
            else hi = mid - 1;
        }
        const int b = lo;
        const int s = node_offsets[b];
        const int n = node_offsets[b + 1] - s;
        const int ctx = ctx_lens[b];
        const int nt = (n * G + kTileM - 1) / kTileM;
        const int nc = ctx > chunk_len ? (ctx + chunk_len - 1) / chunk_len : 1;
        const int local = x - s_items[b];
        const int t = local % nt;
        const int rest = local / nt;
        const int chunk = rest % nc;
        const int kvh = rest / nc;
        Item it;
        it.b = b;
        it.kvh = kvh;
        it.tile = t;
        it.s = s;
        it.n = n;
        it.ctx = ctx;
        it.c0 = chunk * chunk_len;
        it.c1 = min(ctx, it.c0 + chunk_len);
        const int last_row = min((t + 1) * kTileM, n * G) - 1;
        it.kmax = chunk == nc - 1 ? last_row / G + 1 : 0;
        it.pslot = nc > 1 ? s_parts[b] + local : -1;
        it.nc = nc;
        it.nt = nt;
        items[x] = it;
        if (nc > 1 && chunk == 0) {
            const int ci = atomicAdd(&s_ncomb, 1);
            if (ci < max_groups) {
                Combine cb;
                cb.b = b;
                cb.kvh = kvh;
                cb.tile = t;
                cb.s = s;
                cb.n = n;
                cb.pslot0 = it.pslot;
                cb.stride = nt;
                cb.nc = nc;
                combine[ci] = cb;
            }
        }
    }
    __syncthreads();
    if (tid == 0) {
        hdr->n_items = n_items;
        hdr->n_combine = min((int64_t)s_ncomb, max_groups);
        hdr->chunk_len = chunk_len;
    }
}

template <int D>
__global__ __launch_bounds__(kThreads) void attn_prep_kernel(
    const int32_t* __restrict__ node_offsets, const int32_t* __restrict__ ctx_lens, int B,
    int n_max, int64_t total_nodes, const uint16_t* __restrict__ q,
    const uint16_t* __restrict__ k_new, const uint16_t* __restrict__ v_new,
    const int32_t* __restrict__ positions, CacheView cache, int Hq, float rope_base,
    double q_mult, uint16_t* __restrict__ q_hi, uint16_t* __restrict__ q_lo, PlanHeader* hdr,
    Item* items, Combine* combine, int64_t max_items, int64_t max_groups, int64_t max_partials,
    int32_t* __restrict__ err) {
    const int b = blockIdx.y;
    const int Hkv = cache.hkv;
    const int G = Hq / Hkv;
    if (b == B) {
        if (blockIdx.x == 0)
            build_plan(node_offsets, ctx_lens, B, n_max, total_nodes, G, Hkv,
                       cache.paged ? -1 : cache.cap, hdr, items, combine, max_items, max_groups,
                       max_partials, err);
        return;
    }
    const int i = blockIdx.x;
    const int s = node_offsets[b];
    const int n = node_offsets[b + 1] - s;
    const int ctx = ctx_lens[b];
    if (s < 0 || n < 0 || n > n_max || (int64_t)s + n > total_nodes || ctx < 0) return;
    if (i >= n) return;
    if (!cache.paged && (int64_t)ctx + n > cache.cap) return;  // flagged by the plan

    // Rotation in fp64: with fp32, x0 cos - x1 sin loses absolute accuracy
    // when the two products nearly cancel, which shows up as several bf16
    // ulps on small results.  The work is N_b * (Hq + Hkv) * D/2 pairs.
    __shared__ double s_cos[D / 2], s_sin[D / 2];
    const int tid = threadIdx.x;
    const int node = s + i;
    const int pos = positions[node];
    if (tid < D / 2) {
        // inv_freq_m = base^(-2m/D); the angle is reduced modulo 2*pi first.
        const double inv = exp2(-(2.0 * tid / D) * log2((double)rope_base));
        const double ang = (double)pos * inv;
        const double two_pi = 6.283185307179586476925;
        const double red = ang - two_pi * rint(ang / two_pi);
        double sn, cs;
        sincos(red, &sn, &cs);
        s_cos[tid] = cs;
        s_sin[tid] = sn;
    }
    __syncthreads();
    constexpr int kVec = 8;
    // Q: rotated, scaled by softmax_scale*log2(e), stored as bf16 hi + lo parts.
    const int q_vecs = Hq * D / kVec;
    for (int v = tid; v < q_vecs; v += kThreads) {
        const int64_t e = (int64_t)node * Hq * D + (int64_t)v * kVec;
        const ttv_u32x4 in = *(const ttv_u32x4*)(q + e);
        const int d0 = (v * kVec) % D;
        ttv_u32x4 hi4, lo4;
#pragma unroll
        for (int w = 0; w < 4; ++w) {
            const double x0 = ttv_bf16_bits_to_f64(in[w] & 0xFFFFu);
            const double x1 = ttv_bf16_bits_to_f64(in[w] >> 16);
            const int m = (d0 >> 1) + w;
            const double c = s_cos[m], sn = s_sin[m];
            const double r0 = (x0 * c - x1 * sn) * q_mult;
            const double r1 = (x1 * c + x0 * sn) * q_mult;
            const uint32_t h0 = ttv_f64_to_bf16_bits(r0), h1 = ttv_f64_to_bf16_bits(r1);
            hi4[w] = h0 | (h1 << 16);
            lo4[w] = ttv_f64_to_bf16_bits(r0 - ttv_bf16_bits_to_f64(h0)) |
                     (ttv_f64_to_bf16_bits(r1 - ttv_bf16_bits_to_f64(h1)) << 16);
        }
        *(ttv_u32x4*)(q_hi + e) = hi4;
        *(ttv_u32x4*)(q_lo + e) = lo4;
    }
    // K (rotated, rounded once from fp64) and V (copied) into slot ctx + i.
    const int kv_vecs = Hkv * D / kVec;
    for (int v = tid; v < kv_vecs; v += kThreads) {
        const int h = (v * kVec) / D;
        const int d0 = (v * kVec) % D;
        const int64_t dst = cache_row(cache, b, h, ctx + i, D);
        if (dst < 0) {
            atomicOr(err + b, TTV_ERR_BLOCK_TABLE);
            continue;
        }
        const int64_t e = (int64_t)node * Hkv * D + (int64_t)v * kVec;
        const ttv_u32x4 kin = *(const ttv_u32x4*)(k_new + e);
        ttv_u32x4 ko;
#pragma unroll
        for (int w = 0; w < 4; ++w) {
            const double x0 = ttv_bf16_bits_to_f64(kin[w] & 0xFFFFu);
            const double x1 = ttv_bf16_bits_to_f64(kin[w] >> 16);
            const int m = (d0 >> 1) + w;
            const double c = s_cos[m], sn = s_sin[m];
            ko[w] = ttv_f64_to_bf16_bits(x0 * c - x1 * sn) |
                    (ttv_f64_to_bf16_bits(x1 * c + x0 * sn) << 16);
        }
        *(ttv_u32x4*)(cache.k + dst + d0) = ko;
        *(ttv_u32x4*)(cache.v + dst + d0) = *(const ttv_u32x4*)(v_new + e);
    }
}

// ---------------------------------------------------------------------------
// 2. Main kernel.
// ---------------------------------------------------------------------------

template <int D>
struct Smem {
    static constexpr int kKStride = D + 8;        // bf16 elements per K row (pad 16 B)
    static constexpr int kVStride = kKT + 4;      // bf16 elements per transposed V row (8-byte aligned rows)
    static constexpr int kQStride = D + 8;        // bf16 elements per staged Q-lo row
    uint16_t k[2][kKT * kKStride];
    uint16_t vt[2][D * kVStride];
    uint16_t qlo[kTileM * kQStride];              // low parts of the tile's Q (precise tiles)
};

template <int D>
struct TileShape {
    static constexpr int kPieces = D / 8;                       // 16-byte pieces per row
    static constexpr int kKIter = kKT * kPieces / kThreads;     // K pieces per thread
    static constexpr int kVPairs = (kKT / 2) * kPieces;         // (key pair, piece) units
    static constexpr int kVIter = (kVPairs + kThreads - 1) / kThreads;
    static_assert(kKT * kPieces % kThreads == 0, "K tile must split evenly");
};

template <int D>
__device__ __forceinline__ void load_tile(const CacheView& c, int b, int kvh, int slot0,
                                          int valid, ttv_u32x4 (&kreg)[TileShape<D>::kKIter],
                                          ttv_u32x4 (&vreg)[2 * TileShape<D>::kVIter], int tid,
                                          int32_t* err) {
    using TS = TileShape<D>;
#pragma unroll
    for (int u = 0; u < TS::kKIter; ++u) {
        const int p = tid + kThreads * u;
        const int key = p / TS::kPieces, piece = p % TS::kPieces;
        ttv_u32x4 val = {0u, 0u, 0u, 0u};
        if (key < valid) {
            const int64_t r = cache_row(c, b, kvh, slot0 + key, D);
            if (r >= 0) val = *(const ttv_u32x4*)(c.k + r + piece * 8);
            else atomicOr(err + b, TTV_ERR_BLOCK_TABLE);
        }
        kreg[u] = val;
    }
    // V: thread handles keys 2kp and 2kp+1 of one piece, for the transposed store.
#pragma unroll
    for (int u = 0; u < TS::kVIter; ++u) {
        const int p = tid + kThreads * u;
        const int kp = p / TS::kPieces, piece = p % TS::kPieces;
#pragma unroll
        for (int h = 0; h < 2; ++h) {
            const int key = 2 * kp + h;
            ttv_u32x4 val = {0u, 0u, 0u, 0u};
            if (p < TS::kVPairs && key < valid) {
                const int64_t r = cache_row(c, b, kvh, slot0 + key, D);
                if (r >= 0) val = *(const ttv_u32x4*)(c.v + r + piece * 8);
            }
            vreg[2 * u + h] = val;
        }
    }
}

template <int D>
__device__ __forceinline__ void store_tile(Smem<D>& sm, int buf,
                                           const ttv_u32x4 (&kreg)[TileShape<D>::kKIter],
                                           const ttv_u32x4 (&vreg)[2 * TileShape<D>::kVIter],
                                           int tid) {
    using TS = TileShape<D>;
#pragma unroll
    for (int u = 0; u < TS::kKIter; ++u) {
        const int p = tid + kThreads * u;
        const int key = p / TS::kPieces, piece = p % TS::kPieces;
        *(ttv_u32x4*)(&sm.k[buf][key * Smem<D>::kKStride + piece * 8]) = kreg[u];
    }
    uint32_t* base = (uint32_t*)&sm.vt[buf][0];
#pragma unroll
    for (int u = 0; u < TS::kVIter; ++u) {
        const int p = tid + kThreads * u;
        if (p >= TS::kVPairs) continue;
        const int kp = p / TS::kPieces, piece = p % TS::kPieces;
        const ttv_u32x4 a = vreg[2 * u], bb = vreg[2 * u + 1];
#pragma unroll
        for (int w = 0; w < 4; ++w) {
            // rows d = piece*8 + 2w and d + 1; columns (keys) 2kp, 2kp+1
            const uint32_t lo = (a[w] & 0xFFFFu) | (bb[w] << 16);
            const uint32_t hi = (a[w] >> 16) | (bb[w] & 0xFFFF0000u);
            const int d = piece * 8 + 2 * w;
            base[(d * Smem<D>::kVStride + 2 * kp) >> 1] = lo;
            base[((d + 1) * Smem<D>::kVStride + 2 * kp) >> 1] = hi;
        }
    }
}

template <int D>
__global__ __launch_bounds__(kThreads) void attn_main_kernel(
    const PlanHeader* __restrict__ hdr, const Item* __restrict__ items,
    const uint16_t* __restrict__ q_hi, const uint16_t* __restrict__ q_lo,
    const uint32_t* __restrict__ mask, int mask_words, CacheView cache, int Hq,
    uint16_t* __restrict__ out, float* __restrict__ part_o, float2* __restrict__ part_ml,
    int32_t* __restrict__ err) {
    __shared__ Smem<D> sm;
    constexpr int KC = D / 32;   // 32-wide k chunks of the head dim
    constexpr int DB = D / 16;   // 16-row blocks of the head dim
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int l16 = lane & 15;
    const int g4 = lane >> 4;
    const int n_items = hdr->n_items;
    const int Hkv = cache.hkv;
    const int G = Hq / Hkv;
    // XCD-major virtual id: consecutive ids share an XCD (hardware places
    // workgroup x on XCD x % 8).
    const int per_xcd = gridDim.x / kNumXcd;
    const int vid = (blockIdx.x % kNumXcd) * per_xcd + blockIdx.x / kNumXcd;

    for (int x = vid; x < n_items; x += gridDim.x) {
        const Item it = items[x];
        const int rows = it.n * G;
        const int row_base = it.tile * kTileM + wave * kRowsPerWave;
        const int n_ctx_tiles = (it.c1 - it.c0 + kKT - 1) / kKT;
        const int n_tree_tiles = (it.kmax + kKT - 1) / kKT;
        const int n_tiles = n_ctx_tiles + n_tree_tiles;
        // Tiles where few keys can dominate a row's softmax get Q and P as
        // bf16 hi + lo pairs (two MFMAs each): tree tiles, and every tile of a
        // short-context request.
        const bool precise_ctx = it.ctx < kPreciseCtx;
        const bool any_precise = n_tree_tiles > 0 || precise_ctx;

        // Q^T operands: qreg[mb][kc] holds Q[row 16mb + l16][32kc + 8g4 .. +7].
        ttv_bf16x8 qreg[4][KC];
        int row_node[4];
#pragma unroll
        for (int mb = 0; mb < 4; ++mb) {
            const int r = row_base + 16 * mb + l16;
            const bool ok = r < rows;
            const int node = ok ? r / G : 0;
            const int g = ok ? r % G : 0;
            row_node[mb] = ok ? node : -1;
            const uint16_t* src = q_hi + ((int64_t)(it.s + node) * Hq + it.kvh * G + g) * D;
#pragma unroll
            for (int kc = 0; kc < KC; ++kc) {
                ttv_u32x4 v = {0u, 0u, 0u, 0u};
                if (ok) v = *(const ttv_u32x4*)(src + 32 * kc + 8 * g4);
                qreg[mb][kc] = __builtin_bit_cast(ttv_bf16x8, v);
            }
        }
        if (any_precise) {  // stage the tile's Q low parts in LDS
            constexpr int kPieces = D / 8;
            for (int p = tid; p < kTileM * kPieces; p += kThreads) {
                const int rl = p / kPieces, piece = p % kPieces;
                const int r = it.tile * kTileM + rl;
                ttv_u32x4 v = {0u, 0u, 0u, 0u};
                if (r < rows) {
                    const int node = r / G, g = r % G;
                    v = *(const ttv_u32x4*)(q_lo + ((int64_t)(it.s + node) * Hq + it.kvh * G + g) * D +
                                            piece * 8);
                }
                *(ttv_u32x4*)(&sm.qlo[rl * Smem<D>::kQStride + piece * 8]) = v;
            }
        }

        ttv_f32x4 o[DB][4];
#pragma unroll
        for (int db = 0; db < DB; ++db)
#pragma unroll
            for (int mb = 0; mb < 4; ++mb) o[db][mb] = ttv_f32x4{0.f, 0.f, 0.f, 0.f};
        float m_run[4], l_run[4];
#pragma unroll
        for (int mb = 0; mb < 4; ++mb) {
            m_run[mb] = kNegBig;
            l_run[mb] = 0.f;
        }

        ttv_u32x4 kreg[TileShape<D>::kKIter], vreg[2 * TileShape<D>::kVIter];
        auto tile_src = [&](int tau, int& slot0, int& valid) {
            if (tau < n_ctx_tiles) {
                slot0 = it.c0 + tau * kKT;
                valid = min(kKT, it.c1 - slot0);
            } else {
                const int k0 = (tau - n_ctx_tiles) * kKT;
                slot0 = it.ctx + k0;
                valid = min(kKT, it.kmax - k0);
            }
        };

        // One tile: scores, mask, online softmax, P.V.  kPrecise selects the
        // hi + lo variant.
        auto consume = [&](auto precise_tag, int tau, int buf) {
            constexpr bool kPrecise = decltype(precise_tag)::value;
            int slot0, valid;
            tile_src(tau, slot0, valid);
            const bool tree = tau >= n_ctx_tiles;
            // S^T[key][row] for keys 16kb + 4g4 + r, rows 16mb + l16.
            ttv_f32x4 sacc[2][4];
#pragma unroll
            for (int kb = 0; kb < 2; ++kb)
#pragma unroll
                for (int mb = 0; mb < 4; ++mb) sacc[kb][mb] = ttv_f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int kc = 0; kc < KC; ++kc) {
                ttv_bf16x8 qlo[4];
                if (kPrecise) {
#pragma unroll
                    for (int mb = 0; mb < 4; ++mb)
                        qlo[mb] = *(const ttv_bf16x8*)(&sm.qlo[(wave * kRowsPerWave + 16 * mb + l16) *
                                                                  Smem<D>::kQStride + 32 * kc + 8 * g4]);
                }
#pragma unroll
                for (int kb = 0; kb < 2; ++kb) {
                    const ttv_bf16x8 a = *(const ttv_bf16x8*)(
                        &sm.k[buf][(16 * kb + l16) * Smem<D>::kKStride + 32 * kc + 8 * g4]);
#pragma unroll
                    for (int mb = 0; mb < 4; ++mb) {
                        sacc[kb][mb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, qreg[mb][kc],
                                                                               sacc[kb][mb], 0, 0, 0);
                        if (kPrecise)
                            sacc[kb][mb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, qlo[mb],
                                                                                   sacc[kb][mb], 0, 0, 0);
                    }
                }
            }
            // Mask: keys past the valid count, and (tree tiles) non-ancestors.
            uint32_t vis[4];
#pragma unroll
            for (int mb = 0; mb < 4; ++mb) {
                uint32_t w = valid >= 32 ? 0xFFFFFFFFu : ((1u << valid) - 1u);
                if (tree) {
                    const int k0 = (tau - n_ctx_tiles) * kKT;
                    const int node = row_node[mb];
                    w &= node >= 0 ? mask[(int64_t)(it.s + node) * mask_words + (k0 >> 5)] : 0u;
                }
                vis[mb] = w;
            }
            ttv_bf16x8 pb[4], pl[4];
#pragma unroll
            for (int mb = 0; mb < 4; ++mb) {
                float sv[8];
#pragma unroll
                for (int kb = 0; kb < 2; ++kb)
#pragma unroll
                    for (int r = 0; r < 4; ++r) {
                        const int key = 16 * kb + 4 * g4 + r;
                        sv[4 * kb + r] = ((vis[mb] >> key) & 1u) ? sacc[kb][mb][r] : -INFINITY;
                    }
                float tmax = sv[0];
#pragma unroll
                for (int e = 1; e < 8; ++e) tmax = fmaxf(tmax, sv[e]);
                tmax = fmaxf(tmax, __shfl_xor(tmax, 16, TTV_WAVE));
                tmax = fmaxf(tmax, __shfl_xor(tmax, 32, TTV_WAVE));
                const float m_new = fmaxf(m_run[mb], tmax);
                const float alpha = exp2f(m_run[mb] - m_new);
                m_run[mb] = m_new;
                float psum = 0.f;
                uint32_t packed[4], packed_lo[4];
#pragma unroll
                for (int e = 0; e < 8; e += 2) {
                    const float p0 = exp2f(sv[e] - m_new);
                    const float p1 = exp2f(sv[e + 1] - m_new);
                    psum += p0 + p1;
                    packed[e >> 1] = ttv_pack_bf16x2(p0, p1);
                    if (kPrecise)
                        packed_lo[e >> 1] = ttv_pack_bf16x2(p0 - ttv_bf16_lo(packed[e >> 1]),
                                                            p1 - ttv_bf16_hi(packed[e >> 1]));
                }
                l_run[mb] = l_run[mb] * alpha + psum;
                pb[mb] = __builtin_bit_cast(ttv_bf16x8, ttv_u32x4{packed[0], packed[1], packed[2], packed[3]});
                if (kPrecise)
                    pl[mb] = __builtin_bit_cast(ttv_bf16x8,
                                                ttv_u32x4{packed_lo[0], packed_lo[1], packed_lo[2], packed_lo[3]});
#pragma unroll
                for (int db = 0; db < DB; ++db) o[db][mb] *= alpha;
            }
            // O^T[d][row] += V^T[d][key] P^T[key][row]; MFMA k index 8g4 + j maps to
            // key 4g4 + j (j < 4) and 16 + 4g4 + j - 4 (j >= 4).
#pragma unroll
            for (int db = 0; db < DB; ++db) {
                const uint16_t* vrow = &sm.vt[buf][(16 * db + l16) * Smem<D>::kVStride];
                const ttv_u32x2 lo = *(const ttv_u32x2*)(vrow + 4 * g4);
                const ttv_u32x2 hi = *(const ttv_u32x2*)(vrow + 16 + 4 * g4);
                const ttv_bf16x8 a = __builtin_bit_cast(ttv_bf16x8, ttv_u32x4{lo[0], lo[1], hi[0], hi[1]});
#pragma unroll
                for (int mb = 0; mb < 4; ++mb) {
                    o[db][mb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, pb[mb], o[db][mb], 0, 0, 0);
                    if (kPrecise)
                        o[db][mb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, pl[mb], o[db][mb], 0, 0, 0);
                }
            }
        };

        if (n_tiles > 0) {
            int slot0, valid;
            tile_src(0, slot0, valid);
            load_tile<D>(cache, it.b, it.kvh, slot0, valid, kreg, vreg, tid, err);
            store_tile<D>(sm, 0, kreg, vreg, tid);
        }
        __syncthreads();
        for (int tau = 0; tau < n_tiles; ++tau) {
            const int buf = tau & 1;
            if (tau + 1 < n_tiles) {  // next tile in flight while this one is consumed
                int slot0, valid;
                tile_src(tau + 1, slot0, valid);
                load_tile<D>(cache, it.b, it.kvh, slot0, valid, kreg, vreg, tid, err);
            }
            if (precise_ctx || tau >= n_ctx_tiles)
                consume(std::integral_constant<bool, true>{}, tau, buf);
            else
                consume(std::integral_constant<bool, false>{}, tau, buf);
            if (tau + 1 < n_tiles) store_tile<D>(sm, buf ^ 1, kreg, vreg, tid);
            __syncthreads();
        }

        // Row sums across the 4 lane groups holding a row's keys.
#pragma unroll
        for (int mb = 0; mb < 4; ++mb) {
            l_run[mb] += __shfl_xor(l_run[mb], 16, TTV_WAVE);
            l_run[mb] += __shfl_xor(l_run[mb], 32, TTV_WAVE);
        }
        // Lane holds O^T[d = 16db + 4g4 + r][row 16mb + l16].
#pragma unroll
        for (int mb = 0; mb < 4; ++mb) {
            const int r_local = wave * kRowsPerWave + 16 * mb + l16;
            const int r = it.tile * kTileM + r_local;
            if (r >= rows) continue;
            if (it.pslot < 0) {
                const int node = r / G, g = r % G;
                uint16_t* dst = out + ((int64_t)(it.s + node) * Hq + it.kvh * G + g) * D;
                const float inv_l = 1.0f / l_run[mb];
#pragma unroll
                for (int db = 0; db < DB; ++db) {
                    ttv_u32x2 w;
                    w[0] = ttv_pack_bf16x2(o[db][mb][0] * inv_l, o[db][mb][1] * inv_l);
                    w[1] = ttv_pack_bf16x2(o[db][mb][2] * inv_l, o[db][mb][3] * inv_l);
                    *(ttv_u32x2*)(dst + 16 * db + 4 * g4) = w;
                }
            } else {
                float* dst = part_o + ((int64_t)it.pslot * kTileM + r_local) * D;
#pragma unroll
                for (int db = 0; db < DB; ++db) *(ttv_f32x4*)(dst + 16 * db + 4 * g4) = o[db][mb];
                if (g4 == 0)
                    part_ml[(int64_t)it.pslot * kTileM + r_local] = make_float2(m_run[mb], l_run[mb]);
            }
        }
        __syncthreads();  // the next item restages Q-lo and tile 0
    }
}

// ---------------------------------------------------------------------------
// 3. Combine: merge the chunk partials of split row tiles.
// ---------------------------------------------------------------------------

template <int D>
__global__ __launch_bounds__(kThreads) void attn_combine_kernel(
    const PlanHeader* __restrict__ hdr, const Combine* __restrict__ combine, int Hq, int Hkv,
    const float* __restrict__ part_o, const float2* __restrict__ part_ml,
    uint16_t* __restrict__ out) {
    constexpr int kLanesPerRow = D / 4;                 // each lane: 4 consecutive d
    constexpr int kRowsPerPass = kThreads / kLanesPerRow;
    constexpr int kRowBlocks = kTileM / kRowsPerPass;
    const int n_work = hdr->n_combine * kRowBlocks;
    const int G = Hq / Hkv;
    const int tid = threadIdx.x;
    for (int wk = blockIdx.x; wk < n_work; wk += gridDim.x) {
        const Combine cb = combine[wk / kRowBlocks];
        const int r_local = (wk % kRowBlocks) * kRowsPerPass + tid / kLanesPerRow;
        const int d = (tid % kLanesPerRow) * 4;
        const int r = cb.tile * kTileM + r_local;
        if (r >= cb.n * G) continue;
        float mmax = kNegBig;
        for (int c = 0; c < cb.nc; ++c)
            mmax = fmaxf(mmax, part_ml[(int64_t)(cb.pslot0 + c * cb.stride) * kTileM + r_local].x);
        float lsum = 0.f;
        ttv_f32x4 acc = {0.f, 0.f, 0.f, 0.f};
        for (int c = 0; c < cb.nc; ++c) {
            const int64_t ps = cb.pslot0 + (int64_t)c * cb.stride;
            const float2 ml = part_ml[ps * kTileM + r_local];
            const float w = exp2f(ml.x - mmax);
            lsum += w * ml.y;
            const ttv_f32x4 v = *(const ttv_f32x4*)(part_o + (ps * kTileM + r_local) * D + d);
            acc += w * v;
        }
        const float inv = 1.0f / lsum;
        const int node = r / G, g = r % G;
        uint16_t* dst = out + ((int64_t)(cb.s + node) * Hq + cb.kvh * G + g) * D + d;
        ttv_u32x2 w2;
        w2[0] = ttv_pack_bf16x2(acc[0] * inv, acc[1] * inv);
        w2[1] = ttv_pack_bf16x2(acc[2] * inv, acc[3] * inv);
        *(ttv_u32x2*)dst = w2;
    }
}

int g_num_cus = 0;

int num_cus() {
    if (g_num_cus > 0) return g_num_cus;
    int dev = 0, cus = 256;
    if (hipGetDevice(&dev) == hipSuccess)
        hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
    g_num_cus = cus > 0 ? cus : 256;
    return g_num_cus;
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
    uint16_t* q_hi = (uint16_t*)(ws + L.off_q);
    uint16_t* q_lo = (uint16_t*)(ws + L.off_qlo);
    float* po = (float*)(ws + L.off_po);
    float2* pml = (float2*)(ws + L.off_pml);
    const double q_mult = scale * 1.4426950408889634074;  // scores come out in log2 units
    dim3 prep_grid(bt->n_max > 0 ? bt->n_max : 1, bt->batch + 1);
    hipLaunchKernelGGL(attn_prep_kernel<D>, prep_grid, dim3(kThreads), 0, stream,
                       bt->node_offsets, bt->ctx_lens, bt->batch, bt->n_max, bt->total_nodes, q,
                       k_new, v_new, positions, cv, n_heads, rope_base, q_mult, q_hi, q_lo, hdr, items,
                       comb, L.max_items, L.max_groups, L.max_partials, err);
    if (hipGetLastError() != hipSuccess) return TTV_EHIP;
    const int cus = num_cus();
    int64_t grid = (int64_t)cus;  // one 256-row workgroup per CU (LDS and registers bound it)
    if (grid > L.max_items) grid = ((L.max_items + kNumXcd - 1) / kNumXcd) * kNumXcd;
    grid = ((grid + kNumXcd - 1) / kNumXcd) * kNumXcd;
    hipLaunchKernelGGL(attn_main_kernel<D>, dim3((unsigned)grid), dim3(kThreads), 0, stream, hdr,
                       items, q_hi, q_lo, mask, mask_words, cv, n_heads, out, po, pml, err);
    if (hipGetLastError() != hipSuccess) return TTV_EHIP;
    hipLaunchKernelGGL(attn_combine_kernel<D>, dim3((unsigned)(2 * cus)), dim3(kThreads), 0,
                       stream, hdr, comb, n_heads, cache->n_kv_heads, po, pml, out);
    return hipGetLastError() == hipSuccess ? TTV_OK : TTV_EHIP;
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
    if (mask_words < (bt->n_max + 31) / 32) return TTV_EINVAL;
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
