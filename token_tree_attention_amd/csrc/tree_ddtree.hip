// tree_ddtree_build: DDTree's draft tree from the drafter's per-depth logits.
//
// "Accelerating Speculative Decoding with Block Diffusion Draft Trees" notes:
// with a factorised draft the B most probable prefixes form the optimal,
// prefix-closed tree (§4.2); each depth's top-min(B, V) tokens suffice
// (§4.3, Lemma 1); Algorithm 1 (§5) pops prefixes best-first from a heap of
// rank tuples, pushing each popped prefix's next sibling (last rank + 1) and
// first child (rank 1 one depth down), and after B pops holds the top-B
// prefixes in descending score order.
//
// Readings (shared with the input generator of the DDTree workloads): a
// depth's distribution is the softmax of its logits truncated to the top K
// and renormalised over them (log q = z - lse, the sum in lse taken in rank
// order); the top-K order is by logit descending then token id ascending;
// equal scores pop in increasing rank-tuple order, a tuple before its
// extensions; node i is the i-th popped prefix.
//
// Kernel 1, one 1024-thread workgroup per (depth, request): radix select of
// the K-th largest 64-bit key (order key of the logit, then the complement of
// the token id, so keys are distinct and the lowest ids win ties) in 8-bit
// digits, the low word's passes only when ties at the K-th logit must be
// split; a gather of the K keys at or above it; a bitonic sort of them in
// LDS; then log q, the exponentials in parallel and their sum by one thread
// in rank order, as the definition adds it.  Every pass over the vocab keeps
// 32 loads per thread in flight.
// Kernel 2, one wave per request: Algorithm 1's priority queue as a frontier
// array in LDS (at most budget + 1 live entries: a popped entry's slot takes
// its next sibling, its first child takes a new slot), each lane caching the
// best entry among the slots it owns; a pop is a wave-wide maximum of the
// cached scores.  Exact score ties are decided by the rank tuples, compared
// by walking the two entries' parent chains through the popped nodes (the
// rank at the shallowest depth where they differ; a tuple before its
// extensions).  The request's log q table is copied into LDS first when it
// fits, so a pop reads its sibling's log q there instead of from memory.

#include <atomic>

#include "ttv_device.h"

namespace {

constexpr int kTopkThreads = 1024;
constexpr int kTopkWaves = kTopkThreads / TTV_WAVE;
constexpr int kBatch = 32;         // loads in flight per thread in a vocab pass
constexpr int kMaxK = 1024;
constexpr int kMaxDepths = 20;     // depths a request may have
constexpr int kHeapLanes = TTV_WAVE;
constexpr int kMaxSlots = kMaxK + kHeapLanes;  // live frontier entries: at most budget + 1

__device__ __forceinline__ float key_to_float(uint32_t k) {
    const uint32_t bits = (k & 0x80000000u) ? (k & 0x7FFFFFFFu) : ~k;
    return __uint_as_float(bits);
}

// f(v, key) for every v < vocab, key = (order key of z[v]) << 32 | ~v; each
// thread loads kBatch values before using any.
template <typename F>
__device__ __forceinline__ void for_each_key(const float* __restrict__ row, int64_t vocab, F&& f) {
    const int tid = threadIdx.x;
    for (int64_t base = 0; base < vocab; base += (int64_t)kBatch * kTopkThreads) {
        float x[kBatch];
#pragma unroll
        for (int j = 0; j < kBatch; ++j) {
            const int64_t v = base + (int64_t)j * kTopkThreads + tid;
            x[j] = v < vocab ? row[v] : 0.f;
        }
#pragma unroll
        for (int j = 0; j < kBatch; ++j) {
            const int64_t v = base + (int64_t)j * kTopkThreads + tid;
            if (v < vocab)
                f(((uint64_t)ttv_order_key(__float_as_uint(x[j])) << 32) | (uint64_t)(0xFFFFFFFFu - (uint32_t)v));
        }
    }
}

// The same over a row whose length is a multiple of 4 and whose start is
// 16-byte aligned: four consecutive entries per 16-byte load, kVBatch loads
// in flight per thread.
constexpr int kVBatch = 8;
template <typename F>
__device__ __forceinline__ void for_each_key4(const float* __restrict__ row, int64_t vocab, F&& f) {
    const int tid = threadIdx.x;
    const int64_t n4 = vocab / 4;
    for (int64_t base = 0; base < n4; base += (int64_t)kVBatch * kTopkThreads) {
        float4 x[kVBatch];
#pragma unroll
        for (int j = 0; j < kVBatch; ++j) {
            const int64_t c = base + (int64_t)j * kTopkThreads + tid;
            x[j] = c < n4 ? *(const float4*)(row + 4 * c) : make_float4(0.f, 0.f, 0.f, 0.f);
        }
#pragma unroll
        for (int j = 0; j < kVBatch; ++j) {
            const int64_t c = base + (int64_t)j * kTopkThreads + tid;
            if (c < n4) {
                const float e[4] = {x[j].x, x[j].y, x[j].z, x[j].w};
#pragma unroll
                for (int k = 0; k < 4; ++k) {
                    const uint32_t v = (uint32_t)(4 * c + k);
                    f(((uint64_t)ttv_order_key(__float_as_uint(e[k])) << 32) | (uint64_t)(0xFFFFFFFFu - v));
                }
            }
        }
    }
}

constexpr int kHistBits = 12;              // first pass: the keys' top 12 bits
constexpr int kHistBins = 1 << kHistBits;
constexpr int kCandCap = 4096;             // candidates the fast path keeps in LDS

__global__ __launch_bounds__(kTopkThreads) void ddtree_topk_kernel(
    const float* __restrict__ z, int32_t depths, int64_t vocab, int32_t K,
    int32_t* __restrict__ tok_out, double* __restrict__ logq_out) {
    __shared__ uint32_t s_hist[kHistBins];
    __shared__ uint32_t s_sel[2];  // digit, count above it
    __shared__ uint32_t s_count;
    __shared__ uint32_t s_wsum[kTopkWaves];
    __shared__ uint64_t s_cand[kMaxK];
    __shared__ uint64_t s_pool[kCandCap];
    __shared__ double s_exp[kMaxK];
    __shared__ double s_lse;
    const int d = blockIdx.x;
    const int r = blockIdx.y;
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const float* row = z + ((int64_t)r * depths + d) * vocab;
    const bool vec = (vocab % 4) == 0 && ((uintptr_t)row % 16) == 0;
    auto each_key = [&](auto&& f) {
        if (vec) for_each_key4(row, vocab, f);
        else for_each_key(row, vocab, f);
    };
    // wave-aggregated slot claim in a buffer (order irrelevant: sorted later)
    auto claim = [&](bool keep) -> uint32_t {
        const uint64_t m = __ballot(keep);
        if (m == 0) return 0xFFFFFFFFu;
        uint32_t base = 0;
        const int leader = __builtin_ctzll(m);
        if (lane == leader) base = atomicAdd(&s_count, (uint32_t)__builtin_popcountll(m));
        base = __shfl(base, leader);
        return keep ? base + (uint32_t)__builtin_popcountll(m & ((1ull << lane) - 1ull)) : 0xFFFFFFFFu;
    };

    // ---- fast path: one histogram pass over the keys' top 12 bits, the bin
    // holding the K-th largest key, then every key at or above that bin
    // gathered into LDS (when they fit), where the exact selection runs.
    for (int i = tid; i < kHistBins; i += kTopkThreads) s_hist[i] = 0;
    if (tid == 0) s_count = 0;
    __syncthreads();
    each_key([&](uint64_t key) { atomicAdd(&s_hist[(uint32_t)(key >> (64 - kHistBits))], 1u); });
    __syncthreads();
    // suffix sums from the top bin: thread t owns bins 4095 - 4t .. 4092 - 4t
    uint32_t own = 0;
#pragma unroll
    for (int q = 0; q < 4; ++q) own += s_hist[kHistBins - 1 - 4 * tid - q];
    uint32_t inc = own;  // inclusive scan over threads (top bins first)
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
        const uint32_t t = __shfl_up(inc, off);
        if (lane >= off) inc += t;
    }
    if (lane == 63) s_wsum[tid >> 6] = inc;
    __syncthreads();
    uint32_t before = 0;  // keys in the bins above this thread's
    for (int w = 0; w < (tid >> 6); ++w) before += s_wsum[w];
    before += inc - own;
    if (before < (uint32_t)K && before + own >= (uint32_t)K) {
        uint32_t acc = before;
        int bin = kHistBins - 1 - 4 * tid;
        for (int q = 0; q < 4; ++q, --bin) {
            acc += s_hist[bin];
            if (acc >= (uint32_t)K) break;
        }
        s_sel[0] = (uint32_t)bin;  // the K-th largest key's bin
        s_sel[1] = acc;            // keys at or above it
    }
    __syncthreads();
    const uint32_t tbin = s_sel[0];
    const uint32_t n_pool = s_sel[1];
    const bool fast = n_pool <= (uint32_t)kCandCap;
    __syncthreads();  // s_sel is rewritten by the selection below
    uint64_t prefix = 0, pmask = 0;
    uint32_t k_rem = (uint32_t)K;
    if (fast) {
        auto take = [&](uint64_t key) {
            const uint32_t pos = claim((uint32_t)(key >> (64 - kHistBits)) >= tbin);
            if (pos != 0xFFFFFFFFu && TTV_DCHECK(pos < (uint32_t)kCandCap, TTV_SITE_DDTREE)) s_pool[pos] = key;
        };
        if (vec) {
            // most chunks of four hold no candidate: one ballot per chunk
            // skips them, the claims run only where some lane has one
            const uint32_t tkey = tbin << (32 - kHistBits);  // lowest order key in bin tbin
            const int64_t n4 = vocab / 4;
            for (int64_t base = 0; base < n4; base += (int64_t)kVBatch * kTopkThreads) {
                float4 x[kVBatch];
#pragma unroll
                for (int j = 0; j < kVBatch; ++j) {
                    const int64_t c = base + (int64_t)j * kTopkThreads + tid;
                    x[j] = c < n4 ? *(const float4*)(row + 4 * c) : make_float4(-INFINITY, -INFINITY, -INFINITY, -INFINITY);
                }
#pragma unroll
                for (int j = 0; j < kVBatch; ++j) {
                    const int64_t c = base + (int64_t)j * kTopkThreads + tid;
                    const float e[4] = {x[j].x, x[j].y, x[j].z, x[j].w};
                    bool any = false;
#pragma unroll
                    for (int k = 0; k < 4; ++k) any |= ttv_order_key(__float_as_uint(e[k])) >= tkey;
                    if (__ballot(any && c < n4) == 0) continue;  // uniform
#pragma unroll
                    for (int k = 0; k < 4; ++k) {
                        const uint32_t v = (uint32_t)(4 * c + k);
                        const uint64_t key = ((uint64_t)ttv_order_key(__float_as_uint(e[k])) << 32) | (uint64_t)(0xFFFFFFFFu - v);
                        const uint32_t pos = claim(c < n4 && (uint32_t)(key >> (64 - kHistBits)) >= tbin);
                        if (pos != 0xFFFFFFFFu && TTV_DCHECK(pos < (uint32_t)kCandCap, TTV_SITE_DDTREE)) s_pool[pos] = key;
                    }
                }
            }
        } else {
            each_key(take);
        }
        __syncthreads();
    }
    // ---- radix select of the K-th largest key, 8-bit digits, over the
    // gathered pool (fast path) or the row.  High word first; the low word
    // (the token id) only splits ties at the K-th logit, so its passes run
    // only when the keys equal to the selected high word outnumber the slots
    // left for them.
    for (int shift = 56; shift >= 0; shift -= 8) {
        for (int i = tid; i < 256; i += kTopkThreads) s_hist[i] = 0;
        __syncthreads();
        auto count = [&](uint64_t key) {
            if ((key & pmask) == prefix) atomicAdd(&s_hist[(uint32_t)(key >> shift) & 255u], 1u);
        };
        if (fast) {
            for (uint32_t i = tid; i < n_pool; i += kTopkThreads) count(s_pool[i]);
        } else {
            each_key(count);
        }
        __syncthreads();
        if (tid < TTV_WAVE) {
            // The digit holding the k_rem-th largest key and the count above
            // it: wave 0, lane l owning digits 255 - 4l .. 252 - 4l, a scan
            // over the lanes from the top digits down.
            uint32_t own = 0;
#pragma unroll
            for (int q = 0; q < 4; ++q) own += s_hist[255 - 4 * lane - q];
            uint32_t inc = own;
#pragma unroll
            for (int off = 1; off < TTV_WAVE; off <<= 1) {
                const uint32_t t = __shfl_up(inc, off);
                if (lane >= off) inc += t;
            }
            const uint32_t before = inc - own;
            // the lane where the count reaches k_rem (the last lane takes digit
            // 0 whatever remains, as a scan down to digit 1 would)
            if ((before < k_rem && inc >= k_rem) || (lane == TTV_WAVE - 1 && inc < k_rem)) {
                uint32_t above = before;
                int dig = 255 - 4 * lane;
                for (int q = 0; q < 3; ++q, --dig) {
                    if (above + s_hist[dig] >= k_rem) break;
                    above += s_hist[dig];
                }
                s_sel[0] = (uint32_t)dig;
                s_sel[1] = above;
                // after the high word: stop when every element at this prefix is kept
                s_count = (shift == 32 && above + s_hist[dig] == k_rem) ? 1u : 0u;
            }
        }
        __syncthreads();
        prefix |= (uint64_t)s_sel[0] << shift;
        pmask |= (uint64_t)255 << shift;
        k_rem -= s_sel[1];
        const bool done = s_count != 0;
        __syncthreads();  // s_sel, s_count and s_hist are rewritten next
        if (done) break;
    }
    // Keys kept: those above `prefix` on the bits of pmask, and those equal to
    // it there (exactly k_rem of them, all of them when the passes stopped early).
    if (tid == 0) s_count = 0;
    for (int i = tid; i < kMaxK; i += kTopkThreads) s_cand[i] = 0ull;
    __syncthreads();
    auto keep_key = [&](uint64_t key) {
        const uint32_t pos = claim((key & pmask) >= prefix);
        if (pos != 0xFFFFFFFFu && TTV_DCHECK(pos < (uint32_t)kMaxK, TTV_SITE_DDTREE)) s_cand[pos] = key;
    };
    if (fast) {
        // every lane of a wave takes part in claim's ballot
        for (uint32_t i0 = 0; i0 < n_pool; i0 += kTopkThreads) {
            const uint32_t i = i0 + tid;
            const uint32_t pos = claim(i < n_pool && (s_pool[i < n_pool ? i : 0] & pmask) >= prefix);
            if (pos != 0xFFFFFFFFu && TTV_DCHECK(pos < (uint32_t)kMaxK, TTV_SITE_DDTREE)) s_cand[pos] = s_pool[i];
        }
    } else {
        each_key(keep_key);
    }
    __syncthreads();

    // ---- bitonic sort, descending: one key per thread; partners closer than
    // 64 are in the same wave (shuffles), farther ones go through LDS
    static_assert(kMaxK == kTopkThreads, "one key per thread");
    uint64_t key = s_cand[tid];
    for (int k = 2; k <= kMaxK; k <<= 1) {
        for (int j = k >> 1; j > 0; j >>= 1) {
            uint64_t other;
            if (j >= TTV_WAVE) {
                __syncthreads();  // every thread has read the previous exchange
                s_cand[tid] = key;
                __syncthreads();
                other = s_cand[tid ^ j];
            } else {
                const uint32_t lo = __shfl_xor((uint32_t)key, j, TTV_WAVE);
                const uint32_t hi = __shfl_xor((uint32_t)(key >> 32), j, TTV_WAVE);
                other = ((uint64_t)hi << 32) | lo;
            }
            const bool desc = (tid & k) == 0;
            const bool lower = (tid & j) == 0;
            const uint64_t mx = key > other ? key : other;
            const uint64_t mn = key > other ? other : key;
            key = (desc == lower) ? mx : mn;
        }
    }
    __syncthreads();
    s_cand[tid] = key;
    __syncthreads();

    // ---- log q over the kept K: exp(z_r - z_1) in parallel, the sum in rank order
    const double m = (double)key_to_float((uint32_t)(s_cand[0] >> 32));
    for (int i = tid; i < K; i += kTopkThreads)
        s_exp[i] = exp((double)key_to_float((uint32_t)(s_cand[i] >> 32)) - m);
    __syncthreads();
    if (tid == 0) {
        // in rank order; the reads of a block of 16 are issued together
        double s = 0.0;
        int i = 0;
        for (; i + 16 <= K; i += 16) {
            double v[16];
#pragma unroll
            for (int q = 0; q < 16; ++q) v[q] = s_exp[i + q];
#pragma unroll
            for (int q = 0; q < 16; ++q) s += v[q];
        }
        for (; i < K; ++i) s += s_exp[i];
        s_lse = m + log(s);
    }
    __syncthreads();
    const int64_t obase = ((int64_t)r * depths + d) * K;
    for (int i = tid; i < K; i += kTopkThreads) {
        const uint64_t key = s_cand[i];
        tok_out[obase + i] = (int32_t)(0xFFFFFFFFu - (uint32_t)key);
        logq_out[obase + i] = (double)key_to_float((uint32_t)(key >> 32)) - s_lse;
    }
}

// Wave-wide maximum of a double, in every lane: DPP steps inside each row of
// 16 lanes, then the cross-row swaps (as 32-bit halves, moved together).
template <int kCtrl>
__device__ __forceinline__ double dpp_f64(double v) {
    const uint64_t u = (uint64_t)__double_as_longlong(v);
    const uint32_t lo = (uint32_t)__builtin_amdgcn_mov_dpp((int)(uint32_t)u, kCtrl, 0xF, 0xF, false);
    const uint32_t hi = (uint32_t)__builtin_amdgcn_mov_dpp((int)(uint32_t)(u >> 32), kCtrl, 0xF, 0xF, false);
    return __longlong_as_double((long long)(((uint64_t)hi << 32) | lo));
}

__device__ __forceinline__ double wave_max_f64(double v) {
    v = fmax(v, dpp_f64<0xB1>(v));   // quad_perm [1,0,3,2]
    v = fmax(v, dpp_f64<0x4E>(v));   // quad_perm [2,3,0,1]
    v = fmax(v, dpp_f64<0x141>(v));  // row_half_mirror
    v = fmax(v, dpp_f64<0x140>(v));  // row_mirror
    const uint64_t u = (uint64_t)__double_as_longlong(v);
    auto lo = __builtin_amdgcn_permlane16_swap((uint32_t)u, (uint32_t)u, false, false);
    auto hi = __builtin_amdgcn_permlane16_swap((uint32_t)(u >> 32), (uint32_t)(u >> 32), false, false);
    v = fmax(__longlong_as_double((long long)(((uint64_t)hi[0] << 32) | lo[0])),
             __longlong_as_double((long long)(((uint64_t)hi[1] << 32) | lo[1])));
    const uint64_t w = (uint64_t)__double_as_longlong(v);
    auto lo2 = __builtin_amdgcn_permlane32_swap((uint32_t)w, (uint32_t)w, false, false);
    auto hi2 = __builtin_amdgcn_permlane32_swap((uint32_t)(w >> 32), (uint32_t)(w >> 32), false, false);
    return fmax(__longlong_as_double((long long)(((uint64_t)hi2[0] << 32) | lo2[0])),
                __longlong_as_double((long long)(((uint64_t)hi2[1] << 32) | lo2[1])));
}

// 16 bytes per lane from global memory into LDS at lds_base + lane * 16
// (lds_base wave-uniform), through the direct global-to-LDS path.
__device__ __forceinline__ void dma16(uint32_t lds_base, const void* g) {
    const uint32_t base = __builtin_amdgcn_readfirstlane(lds_base);
    asm volatile("s_mov_b32 m0, %0\n\tglobal_load_lds_dwordx4 %1, off" ::"s"(base), "v"(g) : "memory", "m0");
}

__global__ __launch_bounds__(kHeapLanes) void ddtree_heap_kernel(
    const int32_t* __restrict__ toks, const double* __restrict__ logq, int32_t depths, int32_t K,
    int32_t budget, int32_t lq_in_lds, int32_t* __restrict__ parents, int32_t* __restrict__ tokens,
    int32_t* __restrict__ n_nodes) {
    constexpr int kPerLane = kMaxSlots / kHeapLanes;
    static_assert(kPerLane * kHeapLanes == kMaxSlots, "whole slots per lane");
    // Frontier entries; slot i is read by lane i % 64.  Scores are finite
    // (log q = z - lse with finite z), so -inf marks an empty slot.
    __shared__ double e_score[kMaxSlots];
    __shared__ double e_lq[kMaxSlots];  // log q of the entry's own (last) rank
    __shared__ int16_t e_par[kMaxSlots];
    __shared__ int16_t e_rank[kMaxSlots];
    __shared__ int8_t e_depth[kMaxSlots];
    // popped nodes, written out after the loop
    __shared__ int16_t n_par[kMaxK];
    __shared__ int16_t n_rank[kMaxK];
    __shared__ int8_t n_depth[kMaxK];
    __shared__ double s_first[kMaxDepths];  // log q of rank 1 at each depth
    extern __shared__ __attribute__((aligned(16))) double s_lq[];  // [depths, K] when lq_in_lds
    const int r = blockIdx.x;
    const int lane = threadIdx.x;
    const int32_t* tk = toks + (int64_t)r * depths * K;
    const double* lq = logq + (int64_t)r * depths * K;
    if (lq_in_lds) {
        // 1 KB per DMA instruction; the last one's lanes past the table load
        // its final 16 bytes again, into LDS the launch rounded up for them
        const int64_t bytes = (int64_t)depths * K * 8;
        const uint32_t base = (uint32_t)(uintptr_t)(__attribute__((address_space(3))) double*)s_lq;
        for (int64_t off = 0; off < bytes; off += 1024) {
            const int64_t src = min(off + 16 * lane, bytes - 16);
            dma16(base + (uint32_t)off, (const char*)lq + src);
        }
        __builtin_amdgcn_s_waitcnt(0);
    }
    for (int i = lane; i < depths; i += kHeapLanes) s_first[i] = lq[(int64_t)i * K];
    if (lane == 0) {
        e_score[0] = lq[0];
        e_lq[0] = lq[0];
        e_par[0] = -1;
        e_rank[0] = 0;
        e_depth[0] = 0;
    }
    __syncthreads();
    // Rank-tuple order of frontier entries a and b: walk the deeper one up to
    // the other's depth, then both up together to their common ancestor; the
    // shallowest depth where the ranks differ decides, and equal common parts
    // put the shorter tuple first.
    auto tuple_less = [&](int a, int b) -> bool {
        int da = e_depth[a], db = e_depth[b];
        const int la = da, lb = db;
        int ra = e_rank[a], pa = e_par[a];
        int rb = e_rank[b], pb = e_par[b];
        for (; da > db; --da) {
            ra = n_rank[pa];
            pa = n_par[pa];
        }
        for (; db > da; --db) {
            rb = n_rank[pb];
            pb = n_par[pb];
        }
        int res = 0;
        for (;;) {
            if (ra != rb) res = ra < rb ? -1 : 1;
            if (pa == pb) break;  // the same node (or both at depth 0): the rest is equal
            ra = n_rank[pa];
            pa = n_par[pa];
            rb = n_rank[pb];
            pb = n_par[pb];
        }
        return res != 0 ? res < 0 : la < lb;
    };
    // Each lane caches the best entry among its slots (score, slot; -inf and
    // -1 when it has none).  Per pop: a wave maximum of the cached scores
    // picks the entry; the popped slot takes the next sibling and the owner
    // of that slot rescans its slots with one slot per lane; the lane that
    // owns the child's new slot compares it with its cached best.
    double my = lane == 0 ? e_score[0] : -INFINITY;
    int best = lane == 0 ? 0 : -1;
    int n_slots = 1;
    int n = 0;
    for (; n < budget; ++n) {
        const double top = wave_max_f64(my);
        if (top == -INFINITY) break;  // the frontier is empty
        uint64_t cand = __ballot(my == top);
        int wslot = __builtin_amdgcn_readlane(best, __builtin_ctzll(cand));
        cand &= cand - 1;
        while (cand) {  // exact score ties across lanes: the lowest rank tuple
            const int cs = __builtin_amdgcn_readlane(best, __builtin_ctzll(cand));
            cand &= cand - 1;
            if (tuple_less(cs, wslot)) wslot = cs;
        }
        const double s = e_score[wslot];
        const double lq_cur = e_lq[wslot];
        const int par = __builtin_amdgcn_readfirstlane(e_par[wslot]);
        const int d = __builtin_amdgcn_readfirstlane(e_depth[wslot]);
        const int rk = __builtin_amdgcn_readfirstlane(e_rank[wslot]);
        const bool sib = rk + 1 < K;
        const bool child = d + 1 < depths;
        // the sibling's log q: from the LDS copy, else a scalar load
        const double lq_next = !sib ? 0.0 : lq_in_lds ? s_lq[d * K + rk + 1] : lq[(int64_t)d * K + rk + 1];
        __syncthreads();  // every lane has read the popped entry
        const int cslot = n_slots;
        if (lane == 0) {
            n_par[n] = (int16_t)par;
            n_depth[n] = (int8_t)d;
            n_rank[n] = (int16_t)rk;
            // the next sibling takes the popped slot: score - log q^(rk) + log q^(rk + 1), in that order
            if (sib) {
                e_score[wslot] = s - lq_cur + lq_next;
                e_lq[wslot] = lq_next;
                e_rank[wslot] = (int16_t)(rk + 1);
            } else {
                e_score[wslot] = -INFINITY;
            }
            // the first child, one depth down, in a new slot
            if (child && TTV_DCHECK(cslot < kMaxSlots && n < kMaxK, TTV_SITE_DDTREE)) {
                e_score[cslot] = s + s_first[d + 1];
                e_lq[cslot] = s_first[d + 1];
                e_par[cslot] = (int16_t)n;
                e_rank[cslot] = 0;
                e_depth[cslot] = (int8_t)(d + 1);
            }
        }
        if (child) ++n_slots;
        __syncthreads();  // the new entries are visible to every lane
        // the popped slot's owner: best of its slots, lane k reading its k-th
        const int owner = wslot & (kHeapLanes - 1);
        const int mine = owner + kHeapLanes * lane;
        const double v = (lane < kPerLane && mine < n_slots) ? e_score[mine] : -INFINITY;
        const double vmax = wave_max_f64(v);
        int nb = -1;
        if (vmax != -INFINITY) {
            uint64_t c2 = __ballot(v == vmax);
            nb = owner + kHeapLanes * __builtin_ctzll(c2);
            c2 &= c2 - 1;
            while (c2) {
                const int cs = owner + kHeapLanes * __builtin_ctzll(c2);
                c2 &= c2 - 1;
                if (tuple_less(cs, nb)) nb = cs;
            }
        }
        if (lane == owner) {
            my = vmax;
            best = nb;
        }
        // the child's slot, when another lane owns it
        if (child && lane == (cslot & (kHeapLanes - 1)) && lane != owner) {
            const double cv = e_score[cslot];
            if (best < 0 || cv > my || (cv == my && tuple_less(cslot, best))) {
                my = cv;
                best = cslot;
            }
        }
    }
    if (lane == 0) n_nodes[r] = n;
    for (int i = lane; i < budget; i += kHeapLanes) {
        const bool live = i < n;
        parents[(int64_t)r * budget + i] = live ? (int32_t)n_par[i] : -1;
        tokens[(int64_t)r * budget + i] = live ? tk[(int64_t)n_depth[i] * K + n_rank[i]] : -1;
    }
}

// Dynamic LDS the heap kernel may take beside its static arrays (about 28 KB).
constexpr size_t kHeapLdsDynamic = 128 * 1024 + 4 * 1024;

// Raises the heap kernel's dynamic-LDS limit once per device.
bool raise_heap_lds() {
    constexpr int kMaxDev = 64;
    static std::atomic<bool> done[kMaxDev];
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDev) dev = 0;
    if (done[dev].load(std::memory_order_acquire)) return true;
    if (hipFuncSetAttribute((const void*)ddtree_heap_kernel, hipFuncAttributeMaxDynamicSharedMemorySize,
                            (int)kHeapLdsDynamic) != hipSuccess)
        return false;
    done[dev].store(true, std::memory_order_release);
    return true;
}

}  // namespace

extern "C" TTV_API size_t tree_ddtree_workspace_bytes(int32_t requests, int32_t depths, int64_t vocab,
                                                      int32_t budget) {
    if (requests < 0 || depths < 1 || depths > kMaxDepths || vocab < 1 || vocab >= (1ll << 31) ||
        budget < 1 || budget > kMaxK)
        return 0;
    const int64_t K = vocab < budget ? vocab : budget;
    const size_t bytes = (size_t)requests * depths * K * (sizeof(int32_t) + sizeof(double)) + 256;
    return bytes;
}

extern "C" TTV_API int tree_ddtree_build(int32_t requests, int32_t depths, int64_t vocab, int32_t budget,
                                         const float* draft_logits, int32_t* parents, int32_t* tokens,
                                         int32_t* n_nodes, void* workspace, size_t workspace_bytes,
                                         hipStream_t stream) {
    const size_t need = tree_ddtree_workspace_bytes(requests, depths, vocab, budget);
    if (need == 0 || requests > 65535) return TTV_EINVAL;
    if (requests == 0) return TTV_OK;
    if (!draft_logits || !parents || !tokens || !n_nodes || !workspace) return TTV_EINVAL;
    if (((uintptr_t)workspace & 255) || ((uintptr_t)draft_logits & 3)) return TTV_EINVAL;
    if (workspace_bytes < need) return TTV_ENOSPC;
    const int32_t K = (int32_t)(vocab < budget ? vocab : budget);
    double* logq = (double*)workspace;
    int32_t* toks = (int32_t*)((char*)workspace + (size_t)requests * depths * K * sizeof(double));
    hipLaunchKernelGGL(ddtree_topk_kernel, dim3((unsigned)depths, (unsigned)requests), dim3(kTopkThreads), 0,
                       stream, draft_logits, depths, vocab, K, toks, logq);
    if (hipGetLastError() != hipSuccess) return TTV_EHIP;
    // the log q table in LDS when it fits beside the frontier (and starts
    // 16-byte aligned in every request's slice, for the copy)
    const size_t lq_bytes = ((size_t)depths * K * sizeof(double) + 1023) / 1024 * 1024;
    const bool lq_in_lds = ((int64_t)depths * K) % 2 == 0 && lq_bytes <= kHeapLdsDynamic;
    if (lq_in_lds && !raise_heap_lds()) return TTV_EHIP;
    hipLaunchKernelGGL(ddtree_heap_kernel, dim3((unsigned)requests), dim3(64), lq_in_lds ? lq_bytes : 0, stream,
                       toks, logq, depths, K, budget, (int32_t)lq_in_lds, parents, tokens, n_nodes);
    return hipGetLastError() == hipSuccess ? TTV_OK : TTV_EHIP;
}

TTV_DEBUG_TU(ddtree)
