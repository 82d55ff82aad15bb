// tree_build: parent list -> bit-packed ancestor mask, depth, positions and
// retrieve indices, one workgroup per request.
//
// What is computed follows the decoding-extensions glossary ("Beam Search、
// 约束解码与 Tree/Self Speculation", section "Packed tree attention": a node sees
// the committed prefix and its own ancestor chain, self included; siblings
// share a position) and "02 · Token Tree 与 Tree Attention" §3 (position =
// context length + depth; bit-packed QLEN-only mask; retrieve_index /
// next_token / next_sibling for walking the tree after verify).
//
// How: every node is one thread.  Depth and the ancestor bit-sets come from
// pointer jumping in LDS (ceil(log2(depth+1)) synchronous rounds instead of a
// walk per node), the bit-sets in passes of 8 words (256 nodes) so LDS stays
// at 32 KB for any tree up to 1024 nodes.  First child and next sibling come
// from sorting (parent, index) keys with a bitonic network: wave shuffles for
// partner distances below 64, LDS for the rest; after the sort, children of
// one parent are adjacent and in index order.

#include "ttv_device.h"

namespace {

constexpr int kMaskPassWords = 8;

__global__ __launch_bounds__(1024) void tree_build_kernel(
    const int32_t* __restrict__ node_offsets, const int32_t* __restrict__ ctx_lens,
    int32_t n_max, int64_t total_nodes, const int32_t* __restrict__ parents,
    uint32_t* __restrict__ mask, int32_t mask_words, int32_t* __restrict__ depth_out,
    int32_t* __restrict__ pos_out, int32_t* __restrict__ ridx_out,
    int32_t* __restrict__ next_token_out, int32_t* __restrict__ next_sibling_out,
    int32_t* __restrict__ err) {
    __shared__ int32_t s_anc[1024];
    __shared__ int32_t s_dist[1024];
    __shared__ uint32_t s_key[1024];
    __shared__ int32_t s_first[1024];
    __shared__ uint32_t s_rows[1024 * kMaskPassWords];
    __shared__ int32_t s_bad;

    const int b = blockIdx.x;
    const int tid = threadIdx.x;
    const int nthr = blockDim.x;  // power of two, >= 64 and >= n_max

    // Request 0 starts at node 0 (node_offsets[0] = 0): its parents load
    // before the offsets arrive and are used only if the offset read is 0.
    const bool spec = b == 0 && tid < n_max && tid < total_nodes;
    const int par_spec = spec ? parents[tid] : -1;
    const int s = node_offsets[b];
    const int e = node_offsets[b + 1];
    const int ctx = ctx_lens[b];
    const int n = e - s;
    int flags = 0;
    if (s < 0 || n < 0 || (int64_t)e > total_nodes || n > n_max) flags |= TTV_ERR_TOO_MANY_NODES;
    if (ctx < 0) flags |= TTV_ERR_BAD_LENGTH;
    if (flags) {  // uniform over the workgroup
        if (tid == 0) err[b] = flags;
        return;
    }
    if (tid == 0) s_bad = 0;
    __syncthreads();

    int par = -1;
    if (tid < n) {
        par = (b == 0 && s == 0) ? par_spec : parents[s + tid];
        if (par < -1 || par >= tid) {
            atomicOr(&s_bad, 1);
            par = -1;  // keep every later index in range
        }
    }

    // ---- depth: distance to the top of the tree by pointer jumping --------
    int anc = par;
    int dist = par >= 0 ? 1 : 0;
    s_anc[tid] = anc;
    s_dist[tid] = dist;
    __syncthreads();
    while (__syncthreads_or(anc >= 0)) {
        int nanc = anc, ndist = dist;
        if (anc >= 0) {
            ndist = dist + s_dist[anc];
            nanc = s_anc[anc];
        }
        __syncthreads();
        anc = nanc;
        dist = ndist;
        s_anc[tid] = anc;
        s_dist[tid] = dist;
        __syncthreads();
    }
    const int depth = dist;

    // ---- ancestor bit-sets by pointer jumping, 8 words per pass ------------
    const int used_words = (n + 31) >> 5;
    for (int w0 = 0; w0 < used_words; w0 += kMaskPassWords) {
        uint32_t row[kMaskPassWords];
#pragma unroll
        for (int c = 0; c < kMaskPassWords; ++c) {
            const int w = w0 + c;
            row[c] = (tid < n && (tid >> 5) == w) ? (1u << (tid & 31)) : 0u;
        }
        int jump = par;
#pragma unroll
        for (int c = 0; c < kMaskPassWords; ++c) s_rows[tid * kMaskPassWords + c] = row[c];
        s_anc[tid] = jump;
        __syncthreads();
        while (__syncthreads_or(jump >= 0)) {
            uint32_t add[kMaskPassWords];
            int njump = jump;
#pragma unroll
            for (int c = 0; c < kMaskPassWords; ++c) add[c] = 0u;
            if (jump >= 0) {
#pragma unroll
                for (int c = 0; c < kMaskPassWords; ++c) add[c] = s_rows[jump * kMaskPassWords + c];
                njump = s_anc[jump];
            }
            __syncthreads();
#pragma unroll
            for (int c = 0; c < kMaskPassWords; ++c) {
                row[c] |= add[c];
                s_rows[tid * kMaskPassWords + c] = row[c];
            }
            jump = njump;
            s_anc[tid] = jump;
            __syncthreads();
        }
        if (tid < n) {
            uint32_t* out_row = mask + (int64_t)(s + tid) * mask_words;
#pragma unroll
            for (int c = 0; c < kMaskPassWords; ++c)
                if (w0 + c < mask_words) out_row[w0 + c] = row[c];
        }
        __syncthreads();
    }
    if (tid < n && TTV_DCHECK((int64_t)s + tid < total_nodes, TTV_SITE_BUILD_NODE)) {
        uint32_t* out_row = mask + (int64_t)(s + tid) * mask_words;
        const int first_zero = ((used_words + kMaskPassWords - 1) / kMaskPassWords) * kMaskPassWords;
        for (int w = first_zero; w < mask_words; ++w) out_row[w] = 0u;
    }

    // ---- first child / next sibling: sort (parent + 1, index) keys ---------
    uint32_t key = tid < n ? ((uint32_t)(par + 1) << 10) | (uint32_t)tid : 0xFFFFFFFFu;
    for (int k = 2; k <= nthr; k <<= 1) {
        for (int j = k >> 1; j > 0; j >>= 1) {
            uint32_t other;
            if (j >= TTV_WAVE) {
                s_key[tid] = key;
                __syncthreads();
                other = s_key[tid ^ j];
                __syncthreads();
            } else {
                other = __shfl_xor(key, j, TTV_WAVE);
            }
            const bool ascending = (tid & k) == 0;
            const bool lower = (tid & j) == 0;
            const uint32_t lo = key < other ? key : other;
            const uint32_t hi = key < other ? other : key;
            key = (ascending == lower) ? lo : hi;
        }
    }
    s_key[tid] = key;
    s_first[tid] = -1;
    __syncthreads();
    int sibling_of = -1, sibling_val = -1;
    if (key != 0xFFFFFFFFu) {
        const int node = (int)(key & 1023u);
        const uint32_t group = key >> 10;
        const uint32_t nxt = tid + 1 < nthr ? s_key[tid + 1] : 0xFFFFFFFFu;
        sibling_of = node;
        sibling_val = (nxt != 0xFFFFFFFFu && (nxt >> 10) == group) ? (int)(nxt & 1023u) : -1;
        const bool group_start = tid == 0 || (s_key[tid - 1] >> 10) != group;
        if (group_start && group > 0) s_first[group - 1] = node;
    }
    __syncthreads();
    if (sibling_of >= 0 && TTV_DCHECK(sibling_of < n && (int64_t)s + sibling_of < total_nodes, TTV_SITE_BUILD_NODE))
        next_sibling_out[s + sibling_of] = sibling_val;
    if (tid < n && TTV_DCHECK((int64_t)s + tid < total_nodes, TTV_SITE_BUILD_NODE)) {
        depth_out[s + tid] = depth;
        pos_out[s + tid] = ctx + depth;
        ridx_out[s + tid] = s + b + 1 + tid;
        next_token_out[s + tid] = s_first[tid];
    }
    if (tid == 0) err[b] = s_bad ? TTV_ERR_BAD_PARENT : 0;
}

}  // namespace

extern "C" TTV_API int tree_build(const ttv_batch* bt, const int32_t* parents, uint32_t* mask,
                                  int32_t mask_words, int32_t* depth, int32_t* positions,
                                  int32_t* retrieve_index, int32_t* retrieve_next_token,
                                  int32_t* retrieve_next_sibling, int32_t* err,
                                  hipStream_t stream) {
    if (!bt || bt->batch < 0 || bt->n_max < 0 || bt->n_max > TTV_MAX_TREE_NODES ||
        bt->total_nodes < 0)
        return TTV_EINVAL;
    if (bt->batch == 0) return TTV_OK;
    if (!bt->node_offsets || !bt->ctx_lens || !err) return TTV_EINVAL;
    if (mask_words < (bt->n_max + 31) / 32 || mask_words > 1 << 20) return TTV_EINVAL;
    if (bt->total_nodes > 0 &&
        (!parents || !mask || !depth || !positions || !retrieve_index || !retrieve_next_token ||
         !retrieve_next_sibling))
        return TTV_EINVAL;
    if (bt->total_nodes > (int64_t)bt->batch * bt->n_max) return TTV_EINVAL;
    int threads = TTV_WAVE;
    while (threads < bt->n_max) threads <<= 1;
    hipLaunchKernelGGL(tree_build_kernel, dim3(bt->batch), dim3(threads), 0, stream,
                       bt->node_offsets, bt->ctx_lens, bt->n_max, bt->total_nodes, parents, mask,
                       mask_words, depth, positions, retrieve_index, retrieve_next_token,
                       retrieve_next_sibling, err);
    return hipGetLastError() == hipSuccess ? TTV_OK : TTV_EHIP;
}

TTV_DEBUG_TU(build)
