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
// One workgroup per request, one thread per sequence, one pass per depth: a
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
    __shared__ int32_t s_par[kMergeThreads];   // the pair of each sequence at this depth
    __shared__ int32_t s_tok[kMergeThreads];
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
    for (int d = 0; d < seq_len; ++d) {
        int t = -1;
        if (alive) {
            t = seq[d];
            if (t < 0) alive = false;
        }
        s_par[m] = alive ? prev : -2;
        s_tok[m] = t;
        if (m == 0) s_any = 0;
        __syncthreads();
        if (alive) atomicOr(&s_any, 1);
        // the lowest-indexed sequence with the same pair
        int first = m;
        if (alive)
            for (int k = 0; k < m; ++k)
                if (s_par[k] == prev && s_tok[k] == t) {
                    first = k;
                    break;
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
        if (starts) {
            parents[(int64_t)r * max_nodes + node] = prev;
            tokens[(int64_t)r * max_nodes + node] = t;
        }
        __syncthreads();
        prev = alive ? (starts ? node : s_node[first]) : -1;
        base += total;
        __syncthreads();  // s_par / s_tok / s_node / s_wsum are rewritten by the next depth
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
