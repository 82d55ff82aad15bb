// tree_kv_commit: move the accepted path's K/V into place and release the
// rest of the tentative region.
//
// Follows the decoding-extensions glossary ("Tree/Self Speculation": cache
// [10,11] with accepted [4,7] becomes [10,11,4,7]; every other tentative node
// is rolled back and released), the tree-attention verification essay (the
// tree's KV sits in one region in node order; after verification the accepted
// path is kept and the rest becomes recyclable, which with a paged cache means
// releasing pages) and "02 · Token Tree 与 Tree Attention" §4 (the chosen
// path's KV becomes the next round's prompt).
//
// One workgroup per request, so a request's block table is read for the
// moves and edited for the release by the same workgroup.  In-place safety:
// the node at depth d has local index i_d >= d (its d ancestors come first),
// so destination slot ctx+d never equals a later source ctx+i_d' (d' > d),
// only possibly an earlier one.  The moves run in rounds over increasing
// (depth, 16-byte piece) ranges, any number of KV heads and head dims; each
// round loads all its pieces before a barrier and stores after it, and later
// rounds only read bytes no earlier round writes.

#include "ttv_device.h"

namespace {

constexpr int kCommitThreads = 256;
constexpr int kPiecesPerThread = 8;  // 16-byte pieces held per thread per round

__global__ __launch_bounds__(kCommitThreads) void kv_commit_kernel(
    const int32_t* __restrict__ node_offsets, const int32_t* __restrict__ ctx_lens,
    int32_t n_max, int64_t total_nodes, uint16_t* __restrict__ kc, uint16_t* __restrict__ vc,
    int32_t layout, int32_t n_kv_heads, int32_t head_dim, int32_t capacity,
    int32_t* __restrict__ block_table, int32_t max_blocks, int32_t block_size,
    int32_t num_blocks, const int32_t* __restrict__ accept_len,
    const int32_t* __restrict__ accepted_nodes, int32_t max_accept, int32_t* __restrict__ new_lens,
    int32_t* __restrict__ released_blocks, int32_t* __restrict__ num_released,
    int32_t* __restrict__ err) {
    __shared__ int32_t s_path[TTV_MAX_TREE_NODES];
    // paged: the table entries of the tentative region, read once
    __shared__ int32_t s_blk[TTV_MAX_TREE_NODES / TTV_BLOCK_SIZE + 2];
    __shared__ int32_t s_flags;

    const int b = blockIdx.x;
    const int tid = threadIdx.x;
    // The path's first entries load with the request's lengths, not after them.
    const int path_first = tid < max_accept ? accepted_nodes[(int64_t)b * max_accept + tid] : 0;
    const int s = node_offsets[b];
    const int n = node_offsets[b + 1] - s;
    const int ctx = ctx_lens[b];
    const int a = accept_len[b];
    const bool paged = layout == TTV_KV_PAGED;
    if (tid == 0) s_flags = 0;
    __syncthreads();

    int flags = 0;
    if (s < 0 || n < 0 || n > n_max || (int64_t)s + n > total_nodes) flags |= TTV_ERR_TOO_MANY_NODES;
    if (ctx < 0) flags |= TTV_ERR_BAD_LENGTH;
    if (!flags && (a < 0 || a > n || a > max_accept)) flags |= TTV_ERR_ACCEPT;
    if (!flags) {
        const int64_t end = (int64_t)ctx + n;
        if (!paged) {
            if (end > capacity) flags |= TTV_ERR_CAPACITY;
        } else {
            const int64_t nblk = (end + block_size - 1) / block_size;
            if (nblk > max_blocks) flags |= TTV_ERR_CAPACITY;
        }
    }
    const int prior = err[b];
    if (flags || prior) {  // uniform: leave the request untouched
        if (tid == 0) {
            new_lens[b] = ctx;
            if (paged && num_released) num_released[b] = 0;
            if (flags) atomicOr(err + b, flags);
        }
        return;
    }
    // Validate the path (strictly increasing local ids in range) and, for a
    // paged cache, every table entry the request's tentative region uses.
    for (int d = tid; d < a; d += kCommitThreads) {
        const int i = d == tid ? path_first : accepted_nodes[(int64_t)b * max_accept + d];
        s_path[d] = i;
        if (i < d || i >= n) atomicOr(&s_flags, TTV_ERR_ACCEPT);
    }
    if (paged) {
        const int first = ctx / block_size;
        const int last = (ctx + n + block_size - 1) / block_size;
        for (int j = first + tid; j < last; j += kCommitThreads) {
            const int blk = block_table[(int64_t)b * max_blocks + j];
            s_blk[j - first] = blk;
            if (blk < 0 || blk >= num_blocks) atomicOr(&s_flags, TTV_ERR_BLOCK_TABLE);
        }
    }
    __syncthreads();
    for (int d = tid + 1; d < a; d += kCommitThreads)
        if (s_path[d] <= s_path[d - 1]) atomicOr(&s_flags, TTV_ERR_ACCEPT);
    __syncthreads();
    if (s_flags) {
        if (tid == 0) {
            new_lens[b] = ctx;
            if (paged && num_released) num_released[b] = 0;
            atomicOr(err + b, s_flags);
        }
        return;
    }

    // Moves: a unit is (depth d, KV head h, K or V): head_dim bf16 = head_dim/8
    // pieces.  The a * pieces_per_depth pieces are taken in increasing
    // (depth, piece) order, kCommitThreads * kPiecesPerThread per round; a
    // round loads all its pieces, then a barrier, then stores them.  A round
    // never stores over a piece a later round still reads: a later round
    // reads sources ctx + i_d' with d' at least the depths stored so far, and
    // i_d' >= d' > every destination depth d stored before it (or the same
    // depth, whose source differs from its destination unless i_d = d, which
    // is not moved).
    const int pieces_per_row = head_dim / 8;
    const int units_per_depth = n_kv_heads * 2;
    const int64_t pieces_per_depth = (int64_t)units_per_depth * pieces_per_row;
    constexpr int kRound = kCommitThreads * kPiecesPerThread;
    const int64_t row_stride = head_dim;  // elements
    auto slot_offset = [&](int slot, int h) -> int64_t {
        if (!paged) return (((int64_t)b * n_kv_heads + h) * capacity + slot) * row_stride;
        // every slot moved lies in the tentative region [ctx, ctx + n)
        const int blk = s_blk[slot / block_size - ctx / block_size];
        return (((int64_t)blk * n_kv_heads + h) * block_size + slot % block_size) * row_stride;
    };
    const int64_t total = (int64_t)a * pieces_per_depth;
    for (int64_t p0 = 0; p0 < total; p0 += kRound) {
        ttv_u32x4 held[kPiecesPerThread];
        int64_t dst_off[kPiecesPerThread];
        uint16_t* dst_base[kPiecesPerThread];
#pragma unroll
        for (int k = 0; k < kPiecesPerThread; ++k) {
            dst_base[k] = nullptr;
            const int64_t p = p0 + tid + k * kCommitThreads;
            if (p < total) {
                const int d = (int)(p / pieces_per_depth);
                const int r = (int)(p % pieces_per_depth);
                const int unit = r / pieces_per_row;
                const int piece = r % pieces_per_row;
                const int h = unit >> 1;
                const int i = s_path[d];
                // debug build: both rows inside the cache (the request's own
                // region when contiguous, a pool block when paged)
                const int64_t elems = paged ? (int64_t)num_blocks * n_kv_heads * block_size * row_stride
                                            : (int64_t)gridDim.x * n_kv_heads * capacity * row_stride;
                if (i != d && TTV_DCHECK(slot_offset(ctx + i, h) >= 0 && slot_offset(ctx + i, h) + 8 * pieces_per_row <= elems &&
                                             slot_offset(ctx + d, h) >= 0 && slot_offset(ctx + d, h) + 8 * pieces_per_row <= elems,
                                         TTV_SITE_COMMIT)) {
                    uint16_t* base = (unit & 1) ? vc : kc;
                    const int64_t src = slot_offset(ctx + i, h) + piece * 8;
                    held[k] = *(const ttv_u32x4*)(base + src);
                    dst_base[k] = base;
                    dst_off[k] = slot_offset(ctx + d, h) + piece * 8;
                }
            }
        }
        __syncthreads();
#pragma unroll
        for (int k = 0; k < kPiecesPerThread; ++k)
            if (dst_base[k]) *(ttv_u32x4*)(dst_base[k] + dst_off[k]) = held[k];
        __syncthreads();
    }

    const int new_len = ctx + a;
    if (tid == 0) new_lens[b] = new_len;
    if (paged) {
        const int first = (new_len + block_size - 1) / block_size;
        const int last = (ctx + n + block_size - 1) / block_size;
        for (int j = first + tid; j < last; j += kCommitThreads) {
            if (!TTV_DCHECK(j < max_blocks && j - first < max_blocks, TTV_SITE_COMMIT)) continue;
            if (released_blocks)  // the staged entry (first >= ctx / block_size)
                released_blocks[(int64_t)b * max_blocks + (j - first)] = s_blk[j - ctx / block_size];
            block_table[(int64_t)b * max_blocks + j] = -1;
        }
        if (released_blocks)
            for (int k = (last > first ? last - first : 0) + tid; k < max_blocks; k += kCommitThreads)
                released_blocks[(int64_t)b * max_blocks + k] = -1;
        if (tid == 0 && num_released) num_released[b] = last > first ? last - first : 0;
    }
}

}  // namespace

extern "C" TTV_API int tree_kv_commit(const ttv_batch* bt, const ttv_kv_cache* cache,
                                      const int32_t* accept_len, const int32_t* accepted_nodes,
                                      int32_t max_accept, int32_t* new_lens,
                                      int32_t* released_blocks, int32_t* num_released,
                                      int32_t* err, hipStream_t stream) {
    if (!bt || !cache || bt->batch < 0 || bt->n_max < 0 || bt->n_max > TTV_MAX_TREE_NODES ||
        bt->total_nodes < 0 || bt->total_nodes > (int64_t)bt->batch * bt->n_max)
        return TTV_EINVAL;
    if (max_accept < 1 || max_accept > TTV_MAX_TREE_NODES) return TTV_EINVAL;
    if (cache->head_dim != 64 && cache->head_dim != 128) return TTV_EINVAL;
    if (cache->n_kv_heads < 1) return TTV_EINVAL;
    if (cache->layout == TTV_KV_CONTIGUOUS) {
        if (cache->capacity < 0) return TTV_EINVAL;
    } else if (cache->layout == TTV_KV_PAGED) {
        if (cache->block_size != TTV_BLOCK_SIZE || cache->max_blocks < 1 || cache->num_blocks < 1 ||
            !cache->block_table)
            return TTV_EINVAL;
        if (!released_blocks || !num_released) return TTV_EINVAL;
    } else {
        return TTV_EINVAL;
    }
    if (bt->batch == 0) return TTV_OK;
    if (!bt->node_offsets || !bt->ctx_lens || !cache->k || !cache->v || !accept_len ||
        !accepted_nodes || !new_lens || !err)
        return TTV_EINVAL;
    if ((((uintptr_t)cache->k) | ((uintptr_t)cache->v)) & 15) return TTV_EINVAL;
    hipLaunchKernelGGL(kv_commit_kernel, dim3(bt->batch), dim3(kCommitThreads), 0, stream,
                       bt->node_offsets, bt->ctx_lens, bt->n_max, bt->total_nodes,
                       (uint16_t*)cache->k, (uint16_t*)cache->v, cache->layout, cache->n_kv_heads,
                       cache->head_dim, cache->capacity, cache->block_table, cache->max_blocks,
                       cache->block_size, cache->num_blocks, accept_len, accepted_nodes,
                       max_accept, new_lens, released_blocks, num_released, err);
    return hipGetLastError() == hipSuccess ? TTV_OK : TTV_EHIP;
}

TTV_DEBUG_TU(commit)
