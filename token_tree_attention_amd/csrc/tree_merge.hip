// tree_merge_sequences: SpecInfer's bottom-up tree, the distinct prefixes of a
// request's independent draft sequences.
//
// "02 · Token Tree 与 Tree Attention" §3: SpecInfer merges independent drafts
// along their common prefixes into one token tree; the decoding-extensions
// glossary's packed node table shows branches [4,5,6], [4,7,8], [9,0,1]
// becoming 8 unique nodes: tokens [4,9,5,7,0,6,8,1], parents
// [-1,-1,0,0,1,2,3,4].  Readings: a sequence ends at its first negative
// entry; nodes are numbered level by level, and within a level in the order
// the sequences (by index) first reach them.
//
// One workgroup per request, one thread per sequence (its tokens loaded eight
// depths at a time), one pass per depth: a
// sequence's (parent node, token) pair at that depth starts a node when no
// lower-indexed sequence has the same pair; the starting sequences are
// numbered by a block scan; the others take the node of the lowest-indexed
// sequence with their pair.

#include "ttv_device.h"

namespace {

constexpr int kMergeThreads = 1024;  // sequences per request at most

__global__ __launch_bounds__(kMergeThreads) void merge_sequences_kernel(
    int32_t n_seqs, int32_t seq_len, const int32_t* __restrict__ seqs, int32_t max_nodes,
    int32_t* __restrict__ parents, int32_t* __restrict__ tokens, int32_t* __restrict__ n_nodes,
    int32_t* __restrict__ err) {
    __shared__ __attribute__((aligned(16))) uint64_t s_key[kMergeThreads];  // each sequence's pair at this depth
    __shared__ int32_t s_node[kMergeThreads];  // its node at this depth (-1: none)
    __shared__ int32_t s_wsum[kMergeThreads / TTV_WAVE];
    __shared__ int32_t s_any;
    const int r = blockIdx.x;
    const int m = threadIdx.x;
    const int lane = m & 63, wv = m >> 6;
    const int32_t* seq = seqs + ((int64_t)r * n_seqs + (m < n_seqs ? m : 0)) * seq_len;
    int prev = -1;        // this sequence's node one level up (-1 at depth 0)
    bool alive = m < n_seqs;
    int base = 0;         // nodes numbered so far
    bool overflow = false;
    constexpr int kAhead = 8;  // tokens of this sequence loaded together (one latency per 8 depths)
    int ahead[kAhead];
    for (int d = 0; d < seq_len; ++d) {
        if (d % kAhead == 0) {
#pragma unroll
            for (int k = 0; k < kAhead; ++k) ahead[k] = alive && d + k < seq_len ? seq[d + k] : -1;
        }
        int t = -1;
        if (alive) {
#pragma unroll
            for (int k = 0; k < kAhead; ++k)
                if (k == d % kAhead) t = ahead[k];
            if (t < 0) alive = false;
        }
        // (parent, token) as one 64-bit key; an ended sequence matches nothing
        const uint64_t key = alive ? ((uint64_t)(uint32_t)(prev + 2) << 32) | (uint32_t)t : ~0ull - (uint64_t)m;
        s_key[m] = key;
        if (m == 0) s_any = 0;
        __syncthreads();
        if (alive) atomicOr(&s_any, 1);
        // the lowest-indexed sequence with the same pair: every lower key is
        // compared (two per 16-byte read, no early exit, so the reads pipeline)
        int first = m;
        if (alive) {
            for (int k = 0; k < m; k += 2) {
                const ulonglong2 kk = *(const ulonglong2*)(s_key + k);
                if (kk.x == key) first = min(first, k);
                if (k + 1 < m && kk.y == key) first = min(first, k + 1);
            }
        }
        const int starts = alive && first == m;
        // block exclusive scan of the starts, in sequence order
        int inc = starts;
#pragma unroll
        for (int off = 1; off < 64; off <<= 1) {
            const int v = __shfl_up(inc, off);
            if (lane >= off) inc += v;
        }
        if (lane == 63) s_wsum[wv] = inc;
        __syncthreads();
        if (!s_any) break;  // uniform: every sequence has ended
        int pre = inc - starts, total = 0;
        for (int w = 0; w < kMergeThreads / TTV_WAVE; ++w) {
            if (w < wv) pre += s_wsum[w];
            total += s_wsum[w];
        }
        if (base + total > max_nodes) {
            overflow = true;
            break;  // uniform
        }
        const int node = starts ? base + pre : -1;
        s_node[m] = node;
        if (starts && TTV_DCHECK(node >= 0 && node < max_nodes, TTV_SITE_MERGE)) {
            parents[(int64_t)r * max_nodes + node] = prev;
            tokens[(int64_t)r * max_nodes + node] = t;
        }
        __syncthreads();
        prev = alive ? (starts ? node : s_node[first]) : -1;
        base += total;
        __syncthreads();  // s_key / s_node / s_wsum are rewritten by the next depth
    }
    if (m == 0) {
        n_nodes[r] = overflow ? 0 : base;
        if (overflow) atomicOr(err + r, TTV_ERR_TOO_MANY_NODES);
    }
    if (!overflow)
        for (int i = base + m; i < max_nodes; i += kMergeThreads) {
            parents[(int64_t)r * max_nodes + i] = -1;
            tokens[(int64_t)r * max_nodes + i] = -1;
        }
}

}  // namespace

extern "C" TTV_API int tree_merge_sequences(int32_t requests, int32_t n_seqs, int32_t seq_len,
                                            const int32_t* seqs, int32_t max_nodes, int32_t* parents,
                                            int32_t* tokens, int32_t* n_nodes, int32_t* err,
                                            hipStream_t stream) {
    if (requests < 0 || requests > 65535 || n_seqs < 1 || n_seqs > kMergeThreads || seq_len < 1 ||
        seq_len > TTV_MAX_TREE_NODES || max_nodes < 1 || max_nodes > TTV_MAX_TREE_NODES)
        return TTV_EINVAL;
    if (requests == 0) return TTV_OK;
    if (!seqs || !parents || !tokens || !n_nodes || !err) return TTV_EINVAL;
    hipLaunchKernelGGL(merge_sequences_kernel, dim3((unsigned)requests), dim3(kMergeThreads), 0, stream, n_seqs,
                       seq_len, seqs, max_nodes, parents, tokens, n_nodes, err);
    return hipGetLastError() == hipSuccess ? TTV_OK : TTV_EHIP;
}

// ---------------------------------------------------------------------------
// tree_eagle_grow: EAGLE's layer-by-layer tree and its global rerank.
//
// "02 · Token Tree 与 Tree Attention" §3: EAGLE grows the tree layer by layer,
// each step expanding the current layer's top-k nodes by top-k children
// ("layer x topk"); §5: the dynamic tree scores a node by its prefix survival
// probability (the product of the draft confidences on its path) and keeps
// the N_tree most promising nodes overall.  Readings: score = parent's score
// times the node's confidence (float64, in that order); a layer's expanded
// nodes are its k best by (score descending, creation index ascending), in
// that order, and the j-th of them gets the drafter's j-th row of k
// children; the kept nodes are the budget best of all created nodes in the
// same order (a parent precedes its children there, so the set is
// prefix-closed), renumbered in creation order.
//
// One workgroup per request; an order position is a rank count (how many
// nodes come before this one), which keeps ties exact.
namespace {

constexpr int kGrowThreads = 1024;
constexpr int kGrowMaxK = 16;
constexpr int kGrowMaxLayers = 16;
constexpr int kGrowMaxNodes = kGrowMaxK + (kGrowMaxLayers - 1) * kGrowMaxK * kGrowMaxK;  // 3856

__global__ __launch_bounds__(kGrowThreads) void eagle_grow_kernel(
    int32_t k, int32_t layers, const int32_t* __restrict__ root_tokens, const float* __restrict__ root_conf,
    const int32_t* __restrict__ child_tokens, const float* __restrict__ child_conf, int32_t budget,
    int32_t* __restrict__ parents, int32_t* __restrict__ tokens, int32_t* __restrict__ n_nodes) {
    __shared__ double s_score[kGrowMaxNodes];
    __shared__ int16_t s_par[kGrowMaxNodes];
    __shared__ int32_t s_tok[kGrowMaxNodes];
    __shared__ int16_t s_new[kGrowMaxNodes];
    __shared__ int16_t s_exp[kGrowMaxK];
    __shared__ int32_t s_wsum[kGrowThreads / TTV_WAVE];
    const int r = blockIdx.x;
    const int tid = threadIdx.x;
    const int kk = k * k;
    // before(a, b): node a comes first in (score descending, index ascending)
    auto before = [&](int a, int b) { return s_score[a] > s_score[b] || (s_score[a] == s_score[b] && a < b); };
    if (tid < k) {
        s_score[tid] = (double)root_conf[(int64_t)r * k + tid];
        s_par[tid] = -1;
        s_tok[tid] = root_tokens[(int64_t)r * k + tid];
    }
    __syncthreads();
    int p0 = 0, p1 = k;  // the previous layer's nodes
    for (int l = 1; l < layers; ++l) {
        // the previous layer's k best, by rank
        for (int x = p0 + tid; x < p1; x += kGrowThreads) {
            int rank = 0;
            for (int y = p0; y < p1; ++y) rank += before(y, x);
            if (rank < k) s_exp[rank] = (int16_t)x;
        }
        __syncthreads();
        const int base = p1;
        const int64_t lrow = ((int64_t)r * (layers - 1) + (l - 1)) * kk;
        for (int t = tid; t < kk; t += kGrowThreads) {
            const int parent = s_exp[t / k];
            s_par[base + t] = (int16_t)parent;
            s_tok[base + t] = child_tokens[lrow + t];
            s_score[base + t] = s_score[parent] * (double)child_conf[lrow + t];
        }
        __syncthreads();
        p0 = base;
        p1 = base + kk;
    }
    const int total = p1;
    const int keep_n = total < budget ? total : budget;
    // kept flags, then creation-order numbering by a block scan
    int kept_local[(kGrowMaxNodes + kGrowThreads - 1) / kGrowThreads];
    int count = 0;
    const int per = (total + kGrowThreads - 1) / kGrowThreads;
    const int x0 = tid * per;
    for (int q = 0; q < per; ++q) {
        const int x = x0 + q;
        int kept = 0;
        if (x < total) {
            int rank = 0;
            for (int y = 0; y < total; ++y) rank += before(y, x);
            kept = rank < keep_n;
        }
        kept_local[q] = kept;
        count += kept;
    }
    const int lane = tid & 63, wv = tid >> 6;
    int inc = count;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
        const int v = __shfl_up(inc, off);
        if (lane >= off) inc += v;
    }
    if (lane == 63) s_wsum[wv] = inc;
    __syncthreads();
    int pre = inc - count;
    for (int w = 0; w < wv; ++w) pre += s_wsum[w];
    for (int q = 0; q < per; ++q) {
        const int x = x0 + q;
        if (x < total) s_new[x] = kept_local[q] ? (int16_t)pre : (int16_t)-1;
        pre += kept_local[q];
    }
    __syncthreads();
    for (int x = tid; x < total; x += kGrowThreads) {
        const int nx = s_new[x];
        if (nx >= 0 && TTV_DCHECK(nx < budget && (s_par[x] < 0 || s_new[s_par[x]] >= 0), TTV_SITE_MERGE)) {
            parents[(int64_t)r * budget + nx] = s_par[x] < 0 ? -1 : s_new[s_par[x]];
            tokens[(int64_t)r * budget + nx] = s_tok[x];
        }
    }
    for (int i = keep_n + tid; i < budget; i += kGrowThreads) {
        parents[(int64_t)r * budget + i] = -1;
        tokens[(int64_t)r * budget + i] = -1;
    }
    if (tid == 0) n_nodes[r] = keep_n;
}

}  // namespace

extern "C" TTV_API int tree_eagle_grow(int32_t requests, int32_t k, int32_t layers, const int32_t* root_tokens,
                                       const float* root_conf, const int32_t* child_tokens,
                                       const float* child_conf, int32_t budget, int32_t* parents,
                                       int32_t* tokens, int32_t* n_nodes, hipStream_t stream) {
    if (requests < 0 || requests > 65535 || k < 1 || k > kGrowMaxK || layers < 1 || layers > kGrowMaxLayers ||
        budget < 1 || budget > TTV_MAX_TREE_NODES)
        return TTV_EINVAL;
    if (requests == 0) return TTV_OK;
    if (!root_tokens || !root_conf || !parents || !tokens || !n_nodes) return TTV_EINVAL;
    if (layers > 1 && (!child_tokens || !child_conf)) return TTV_EINVAL;
    hipLaunchKernelGGL(eagle_grow_kernel, dim3((unsigned)requests), dim3(kGrowThreads), 0, stream, k, layers,
                       root_tokens, root_conf, child_tokens, child_conf, budget, parents, tokens, n_nodes);
    return hipGetLastError() == hipSuccess ? TTV_OK : TTV_EHIP;
}

TTV_DEBUG_TU(merge)
