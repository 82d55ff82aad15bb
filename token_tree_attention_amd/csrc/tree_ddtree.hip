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
// the K-th largest order key over the vocab (four 8-bit histogram passes),
// a gather of the elements above it plus the lowest-index ties at it, a
// bitonic sort of the K candidates in LDS, then log q (the sum by one thread
// in rank order, as the definition adds it).
// Kernel 2, one workgroup per request: the heap of Algorithm 1 in LDS, run by
// one lane; an entry holds its score, its rank tuple packed for comparison
// (11 bits per depth, rank + 1, 5 depths per 64-bit word, depth 0 in the
// most significant field, so a shorter tuple compares below its
// extensions), its parent node, depth and last rank.

#include "ttv_device.h"

namespace {

constexpr int kTopkThreads = 1024;
constexpr int kMaxK = 1024;
constexpr int kMaxDepths = 20;     // 4 key words x 5 fields
constexpr int kKeyWords = 4;
constexpr int kMaxHeap = kMaxK + 2;

__device__ __forceinline__ float key_to_float(uint32_t k) {
    const uint32_t bits = (k & 0x80000000u) ? (k & 0x7FFFFFFFu) : ~k;
    return __uint_as_float(bits);
}

__global__ __launch_bounds__(kTopkThreads) void ddtree_topk_kernel(
    const float* __restrict__ z, int32_t depths, int64_t vocab, int32_t K,
    int32_t* __restrict__ tok_out, double* __restrict__ logq_out) {
    __shared__ uint32_t s_hist[256];
    __shared__ uint32_t s_sel[2];  // digit, count above it
    __shared__ uint64_t s_cand[kMaxK];
    __shared__ uint32_t s_wsum[2][kTopkThreads / TTV_WAVE];
    __shared__ double s_lse;
    const int d = blockIdx.x;
    const int r = blockIdx.y;
    const int tid = threadIdx.x;
    const float* row = z + ((int64_t)r * depths + d) * vocab;

    // ---- radix select: the K-th largest order key -------------------------
    uint32_t prefix = 0, pmask = 0;
    uint32_t k_rem = (uint32_t)K;
    for (int shift = 24; shift >= 0; shift -= 8) {
        for (int i = tid; i < 256; i += kTopkThreads) s_hist[i] = 0;
        __syncthreads();
        for (int64_t v = tid; v < vocab; v += kTopkThreads) {
            const uint32_t u = ttv_order_key(__float_as_uint(row[v]));
            if ((u & pmask) == prefix) atomicAdd(&s_hist[(u >> shift) & 255u], 1u);
        }
        __syncthreads();
        if (tid == 0) {
            uint32_t above = 0;
            int dig = 255;
            for (; dig > 0; --dig) {
                if (above + s_hist[dig] >= k_rem) break;
                above += s_hist[dig];
            }
            s_sel[0] = (uint32_t)dig;
            s_sel[1] = above;
        }
        __syncthreads();
        prefix |= s_sel[0] << shift;
        pmask |= 255u << shift;
        k_rem -= s_sel[1];
        __syncthreads();  // s_sel and s_hist are rewritten by the next pass
    }
    const uint32_t vk = prefix;       // the K-th largest key
    const uint32_t ties = k_rem;      // elements equal to vk that are kept (lowest indices)
    const uint32_t n_gt = (uint32_t)K - ties;

    // ---- gather: contiguous index segments, block scans of the counts -----
    const int64_t seg = (vocab + kTopkThreads - 1) / kTopkThreads;
    const int64_t v0 = (int64_t)tid * seg, v1 = min(vocab, v0 + seg);
    uint32_t c_gt = 0, c_eq = 0;
    for (int64_t v = v0; v < v1; ++v) {
        const uint32_t u = ttv_order_key(__float_as_uint(row[v]));
        c_gt += u > vk;
        c_eq += u == vk;
    }
    const int lane = tid & 63, wv = tid >> 6;
    uint32_t sg = c_gt, se = c_eq;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
        const uint32_t tg = __shfl_up(sg, off), te = __shfl_up(se, off);
        if (lane >= off) {
            sg += tg;
            se += te;
        }
    }
    if (lane == 63) {
        s_wsum[0][wv] = sg;
        s_wsum[1][wv] = se;
    }
    for (int i = tid; i < kMaxK; i += kTopkThreads) s_cand[i] = 0ull;
    __syncthreads();
    uint32_t pg = sg - c_gt, pe = se - c_eq;
    for (int w = 0; w < wv; ++w) {
        pg += s_wsum[0][w];
        pe += s_wsum[1][w];
    }
    for (int64_t v = v0; v < v1; ++v) {
        const uint32_t u = ttv_order_key(__float_as_uint(row[v]));
        const uint64_t key = ((uint64_t)u << 32) | (uint64_t)(0xFFFFFFFFu - (uint32_t)v);
        if (u > vk) s_cand[pg++] = key;
        else if (u == vk) {
            if (pe < ties) s_cand[n_gt + pe] = key;
            ++pe;
        }
    }
    __syncthreads();

    // ---- bitonic sort, descending ------------------------------------------
    for (int k = 2; k <= kMaxK; k <<= 1) {
        for (int j = k >> 1; j > 0; j >>= 1) {
            for (int i = tid; i < kMaxK; i += kTopkThreads) {
                const int p = i ^ j;
                if (p > i) {
                    const uint64_t a = s_cand[i], b = s_cand[p];
                    const bool desc = (i & k) == 0;
                    if (desc ? (a < b) : (a > b)) {
                        s_cand[i] = b;
                        s_cand[p] = a;
                    }
                }
            }
            __syncthreads();
        }
    }

    // ---- log q over the kept K, the sum in rank order ------------------------
    if (tid == 0) {
        const double m = (double)key_to_float((uint32_t)(s_cand[0] >> 32));
        double s = 0.0;
        for (int i = 0; i < K; ++i) s += exp((double)key_to_float((uint32_t)(s_cand[i] >> 32)) - m);
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

struct HeapKey {
    uint64_t w[kKeyWords];
};

__device__ __forceinline__ bool key_less(const HeapKey& a, const HeapKey& b) {
#pragma unroll
    for (int i = 0; i < kKeyWords; ++i)
        if (a.w[i] != b.w[i]) return a.w[i] < b.w[i];
    return false;
}

__device__ __forceinline__ void key_set(HeapKey& k, int depth, int rank) {
    const int w = depth / 5, sh = 11 * (4 - depth % 5);
    k.w[w] = (k.w[w] & ~((uint64_t)2047 << sh)) | ((uint64_t)(rank + 1) << sh);
}

__global__ __launch_bounds__(64) void ddtree_heap_kernel(
    const int32_t* __restrict__ toks, const double* __restrict__ logq, int32_t depths, int32_t K,
    int32_t budget, int32_t* __restrict__ parents, int32_t* __restrict__ tokens,
    int32_t* __restrict__ n_nodes) {
    __shared__ double h_score[kMaxHeap];
    __shared__ HeapKey h_key[kMaxHeap];
    __shared__ int16_t h_par[kMaxHeap];
    __shared__ int16_t h_rank[kMaxHeap];
    __shared__ int8_t h_depth[kMaxHeap];
    const int r = blockIdx.x;
    if (threadIdx.x != 0) return;
    const int32_t* tk = toks + (int64_t)r * depths * K;
    const double* lq = logq + (int64_t)r * depths * K;
    // entry a pops before entry b
    auto before = [&](int a, int b) {
        if (h_score[a] != h_score[b]) return h_score[a] > h_score[b];
        return key_less(h_key[a], h_key[b]);
    };
    auto swap_entries = [&](int a, int b) {
        const double ts = h_score[a]; h_score[a] = h_score[b]; h_score[b] = ts;
        const HeapKey tk2 = h_key[a]; h_key[a] = h_key[b]; h_key[b] = tk2;
        const int16_t tp = h_par[a]; h_par[a] = h_par[b]; h_par[b] = tp;
        const int16_t tr = h_rank[a]; h_rank[a] = h_rank[b]; h_rank[b] = tr;
        const int8_t td = h_depth[a]; h_depth[a] = h_depth[b]; h_depth[b] = td;
    };
    int size = 0;
    auto push = [&](double score, const HeapKey& key, int par, int depth, int rank) {
        int i = size++;
        h_score[i] = score;
        h_key[i] = key;
        h_par[i] = (int16_t)par;
        h_depth[i] = (int8_t)depth;
        h_rank[i] = (int16_t)rank;
        while (i > 0) {
            const int p = (i - 1) >> 1;
            if (!before(i, p)) break;
            swap_entries(i, p);
            i = p;
        }
    };
    HeapKey k0 = {{0ull, 0ull, 0ull, 0ull}};
    key_set(k0, 0, 0);
    push(lq[0], k0, -1, 0, 0);
    int n = 0;
    while (size > 0 && n < budget) {
        // pop the top
        const double s = h_score[0];
        const HeapKey key = h_key[0];
        const int par = h_par[0], d = h_depth[0], rk = h_rank[0];
        --size;
        if (size > 0) {
            h_score[0] = h_score[size];
            h_key[0] = h_key[size];
            h_par[0] = h_par[size];
            h_depth[0] = h_depth[size];
            h_rank[0] = h_rank[size];
            int i = 0;
            for (;;) {
                const int a = 2 * i + 1, b = a + 1;
                if (a >= size) break;
                const int c = (b < size && before(b, a)) ? b : a;
                if (!before(c, i)) break;
                swap_entries(i, c);
                i = c;
            }
        }
        const int node = n++;
        parents[(int64_t)r * budget + node] = par;
        tokens[(int64_t)r * budget + node] = tk[(int64_t)d * K + rk];
        // the next sibling: score - log q^(rk) + log q^(rk + 1), in that order
        if (rk + 1 < K) {
            HeapKey ks = key;
            key_set(ks, d, rk + 1);
            push(s - lq[(int64_t)d * K + rk] + lq[(int64_t)d * K + rk + 1], ks, par, d, rk + 1);
        }
        // the first child, one depth down
        if (d + 1 < depths) {
            HeapKey kc = key;
            key_set(kc, d + 1, 0);
            push(s + lq[(int64_t)(d + 1) * K], kc, node, d + 1, 0);
        }
    }
    n_nodes[r] = n;
    for (int i = n; i < budget; ++i) {
        parents[(int64_t)r * budget + i] = -1;
        tokens[(int64_t)r * budget + i] = -1;
    }
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
    hipLaunchKernelGGL(ddtree_heap_kernel, dim3((unsigned)requests), dim3(64), 0, stream, toks, logq, depths, K,
                       budget, parents, tokens, n_nodes);
    return hipGetLastError() == hipSuccess ? TTV_OK : TTV_EHIP;
}
