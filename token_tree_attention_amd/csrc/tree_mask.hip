// Dense mask modes for interop: tree_expand_mask and tree_pack_mask.
//
// "02 · Token Tree 与 Tree Attention" §3 lists three forms of the tree mask
// that build_tree_kernel_efficient can emit: FULL_MASK, QLEN_ONLY and the
// bit-packed QLEN-only form this library's attention reads.  The glossary's
// packed-vs-branch experiment uses the full form: tree_mask [N, prefix + N],
// the committed prefix always visible, then the ancestor-only tree part.
//
// tree_expand_mask turns the bit-packed rows (tree_build's output) into one
// byte per column, either QLEN_ONLY ([T, row_stride], byte j = bit j) or
// FULL ([T, row_stride], bytes 0 .. ctx-1 = 1, byte ctx + j = bit j);
// bytes past the row's columns are 0.  Grid: (column blocks of 4096 bytes,
// local row, request); each thread writes 16 bytes.
//
// tree_pack_mask goes the other way for a caller that holds a dense mask in
// either mode: bit j of node i's packed row = its dense byte j (QLEN_ONLY) or
// ctx + j (FULL).  A request is refused (TTV_ERR_BAD_MASK) when some row is
// not a mask the attention can run: a FULL row hiding a context column, a
// nonzero byte at or past the next node's column (a later node, or past the
// tree), or the node's own column zero.  One workgroup per (row, request).

#include "ttv_device.h"

namespace {

constexpr int kExpandThreads = 256;
constexpr int kExpandBytes = 16;  // per thread
constexpr int kPackThreads = 256;

__global__ __launch_bounds__(kExpandThreads) void expand_mask_kernel(
    const int32_t* __restrict__ node_offsets, const int32_t* __restrict__ ctx_lens, int32_t n_max,
    int64_t total_nodes, const uint32_t* __restrict__ mask, int32_t mask_words, int32_t mode,
    uint8_t* __restrict__ dense, int64_t row_stride, int32_t* __restrict__ err) {
    const int b = blockIdx.z;
    const int i = blockIdx.y;
    const int s = node_offsets[b];
    const int n = node_offsets[b + 1] - s;
    const int ctx = ctx_lens[b];
    if (s < 0 || n < 0 || n > n_max || (int64_t)s + n > total_nodes || ctx < 0) {
        if (i == 0 && blockIdx.x == 0 && threadIdx.x == 0) atomicOr(err + b, TTV_ERR_TOO_MANY_NODES);
        return;
    }
    if (i >= n) return;
    const int64_t base = mode == TTV_MASK_FULL ? ctx : 0;
    if (base + n > row_stride) {
        if (i == 0 && blockIdx.x == 0 && threadIdx.x == 0) atomicOr(err + b, TTV_ERR_CAPACITY);
        return;
    }
    const uint32_t* mrow = mask + (int64_t)(s + i) * mask_words;
    uint8_t* drow = dense + (int64_t)(s + i) * row_stride;
    const int64_t c0 = ((int64_t)blockIdx.x * kExpandThreads + threadIdx.x) * kExpandBytes;
    if (c0 >= row_stride) return;
    auto byte_at = [&](int64_t c) -> uint32_t {
        if (c < base) return 1u;
        const int64_t j = c - base;
        if (j >= n) return 0u;
        return (mrow[j >> 5] >> (j & 31)) & 1u;
    };
    const bool vec = (row_stride % kExpandBytes) == 0 && (((uintptr_t)dense) % kExpandBytes) == 0;
    if (vec) {
        ttv_u32x4 w;
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            uint32_t v = 0;
#pragma unroll
            for (int k = 0; k < 4; ++k) v |= byte_at(c0 + 4 * q + k) << (8 * k);
            w[q] = v;
        }
        *(ttv_u32x4*)(drow + c0) = w;
    } else {
        for (int k = 0; k < kExpandBytes && c0 + k < row_stride; ++k) drow[c0 + k] = (uint8_t)byte_at(c0 + k);
    }
}

__global__ __launch_bounds__(kPackThreads) void pack_mask_kernel(
    const int32_t* __restrict__ node_offsets, const int32_t* __restrict__ ctx_lens, int32_t n_max,
    int64_t total_nodes, const uint8_t* __restrict__ dense, int64_t row_stride, int32_t mode,
    uint32_t* __restrict__ mask, int32_t mask_words, int32_t* __restrict__ err) {
    __shared__ int s_bad;
    const int b = blockIdx.z;
    const int i = blockIdx.y;
    const int tid = threadIdx.x;
    const int s = node_offsets[b];
    const int n = node_offsets[b + 1] - s;
    const int ctx = ctx_lens[b];
    if (s < 0 || n < 0 || n > n_max || (int64_t)s + n > total_nodes || ctx < 0) {
        if (i == 0 && tid == 0) atomicOr(err + b, TTV_ERR_TOO_MANY_NODES);
        return;
    }
    if (i >= n) return;
    const int64_t base = mode == TTV_MASK_FULL ? ctx : 0;
    if (base + n > row_stride) {
        if (i == 0 && tid == 0) atomicOr(err + b, TTV_ERR_CAPACITY);
        return;
    }
    __shared__ uint32_t s_words[TTV_MAX_TREE_NODES / 32];
    if (tid == 0) s_bad = 0;
    for (int w = tid; w < mask_words; w += kPackThreads) s_words[w] = 0u;
    __syncthreads();
    const uint8_t* drow = dense + (int64_t)(s + i) * row_stride;
    bool bad = false;
    // Rules per column c: context columns (c < base) all visible; the tree
    // columns up to the node's own (base .. base + i) give the packed bits,
    // the node's own set; nothing at or past column base + i + 1.
    auto column = [&](int64_t c, uint32_t byte, uint32_t& lo, uint32_t& hi, int w0) __attribute__((always_inline)) {
        if (c < base) {
            bad |= byte == 0;
        } else if (c > base + i) {
            bad |= byte != 0;
        } else {
            const int j = (int)(c - base);
            if (j == i) bad |= byte == 0;
            if (byte) {
                if ((j >> 5) == w0) lo |= 1u << (j & 31);
                else hi |= 1u << (j & 31);
            }
        }
    };
    const bool vec = (row_stride % 16) == 0 && ((uintptr_t)dense % 16) == 0;
    if (vec) {
        // 16 columns per load; they touch at most two packed words
        for (int64_t p = tid; p < row_stride / 16; p += kPackThreads) {
            const ttv_u32x4 v = *(const ttv_u32x4*)(drow + 16 * p);
            const int64_t c0 = 16 * p;
            const int w0 = c0 >= base ? (int)((c0 - base) >> 5) : 0;
            uint32_t lo = 0u, hi = 0u;
#pragma unroll
            for (int q = 0; q < 16; ++q) column(c0 + q, (v[q >> 2] >> (8 * (q & 3))) & 0xFFu, lo, hi, w0);
            if (lo && TTV_DCHECK(w0 < mask_words, TTV_SITE_MASK)) atomicOr(&s_words[w0], lo);
            if (hi && TTV_DCHECK(w0 + 1 < mask_words, TTV_SITE_MASK)) atomicOr(&s_words[w0 + 1], hi);
        }
    } else {
        for (int64_t c = tid; c < row_stride; c += kPackThreads) {
            uint32_t lo = 0u, hi = 0u;
            const int w0 = c >= base ? (int)((c - base) >> 5) : 0;
            column(c, drow[c], lo, hi, w0);
            if (lo && TTV_DCHECK(w0 < mask_words, TTV_SITE_MASK)) atomicOr(&s_words[w0], lo);
        }
    }
    if (bad) atomicOr(&s_bad, 1);
    __syncthreads();
    uint32_t* mrow = mask + (int64_t)(s + i) * mask_words;
    for (int w = tid; w < mask_words && TTV_DCHECK((int64_t)s + i < total_nodes, TTV_SITE_MASK); w += kPackThreads)
        mrow[w] = s_words[w];
    __syncthreads();
    if (tid == 0 && s_bad) atomicOr(err + b, TTV_ERR_BAD_MASK);
}

bool valid_batch(const ttv_batch* bt) {
    return bt && bt->batch >= 0 && bt->batch <= 65535 && bt->n_max >= 0 &&
           bt->n_max <= TTV_MAX_TREE_NODES && bt->total_nodes >= 0 &&
           bt->total_nodes <= (int64_t)bt->batch * bt->n_max;
}

}  // namespace

extern "C" TTV_API int tree_expand_mask(const ttv_batch* bt, const uint32_t* mask, int32_t mask_words,
                                        int32_t mode, uint8_t* dense, int64_t row_stride, int32_t* err,
                                        hipStream_t stream) {
    if (!valid_batch(bt)) return TTV_EINVAL;
    if (mode != TTV_MASK_QLEN_ONLY && mode != TTV_MASK_FULL) return TTV_EINVAL;
    if (mask_words < (bt->n_max + 31) / 32 || mask_words > TTV_MAX_TREE_NODES / 32) return TTV_EINVAL;
    if (row_stride < bt->n_max || row_stride > ((int64_t)1 << 31)) return TTV_EINVAL;
    if (bt->batch == 0 || bt->n_max == 0) return TTV_OK;
    if (!bt->node_offsets || !bt->ctx_lens || !err) return TTV_EINVAL;
    if (bt->total_nodes > 0 && (!mask || !dense)) return TTV_EINVAL;
    const int64_t per_block = (int64_t)kExpandThreads * kExpandBytes;
    const int64_t xblocks = (row_stride + per_block - 1) / per_block;
    hipLaunchKernelGGL(expand_mask_kernel, dim3((unsigned)xblocks, (unsigned)bt->n_max, (unsigned)bt->batch),
                       dim3(kExpandThreads), 0, stream, bt->node_offsets, bt->ctx_lens, bt->n_max,
                       bt->total_nodes, mask, mask_words, mode, dense, row_stride, err);
    return hipGetLastError() == hipSuccess ? TTV_OK : TTV_EHIP;
}

extern "C" TTV_API int tree_pack_mask(const ttv_batch* bt, const uint8_t* dense, int64_t row_stride,
                                      int32_t mode, uint32_t* mask, int32_t mask_words, int32_t* err,
                                      hipStream_t stream) {
    if (!valid_batch(bt)) return TTV_EINVAL;
    if (mode != TTV_MASK_QLEN_ONLY && mode != TTV_MASK_FULL) return TTV_EINVAL;
    if (mask_words < (bt->n_max + 31) / 32 || mask_words > TTV_MAX_TREE_NODES / 32) return TTV_EINVAL;
    if (row_stride < bt->n_max || row_stride > ((int64_t)1 << 31)) return TTV_EINVAL;
    if (bt->batch == 0 || bt->n_max == 0) return TTV_OK;
    if (!bt->node_offsets || !bt->ctx_lens || !err) return TTV_EINVAL;
    if (bt->total_nodes > 0 && (!mask || !dense)) return TTV_EINVAL;
    hipLaunchKernelGGL(pack_mask_kernel, dim3(1, (unsigned)bt->n_max, (unsigned)bt->batch), dim3(kPackThreads),
                       0, stream, bt->node_offsets, bt->ctx_lens, bt->n_max, bt->total_nodes, dense, row_stride,
                       mode, mask, mask_words, err);
    return hipGetLastError() == hipSuccess ? TTV_OK : TTV_EHIP;
}

TTV_DEBUG_TU(mask)
