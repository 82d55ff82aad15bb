// tree_greedy_accept: vocab argmax of every logits row, then the greedy walk.
//
// The walk follows the decoding-extensions glossary (verify_tree experiment:
// keep the candidates that extend the accepted prefix with the target's next
// token, stop at the first depth without a match), "02 · Token Tree 与 Tree
// Attention" §4 (from the root, accept the child equal to the target's greedy
// choice, continue from it; with no matching child the choice is the
// correction / bonus token) and the DDTree notes §7.2 (all node logits come
// from the one verify pass, so the walk needs no further target pass).
//
// Kernel 1 streams the logits: each workgroup scans one vocab chunk of one
// row with 16-byte loads, keeps a (value, lowest index) pair per thread, and
// reduces to one 64-bit key (order-preserving value bits, then the
// complemented index, so a plain max picks the lowest index on ties).
// Kernel 2 runs one workgroup per request: it reduces the chunk keys of the
// request's rows, stages tokens and retrieve links in LDS, rebuilds each
// node's parent from the links (pointer jumping) and walks with all threads
// searching a depth's children at once.

#include <atomic>

#include "ttv_device.h"

// Argmax-key scratch of tree_greedy_accept_noalloc: one 64-bit key per
// (logits row, vocab chunk), 4 MiB per device, held until the process ends.
// Host code never uses this name as an address: it takes the device address
// with hipGetSymbolAddress once per device (scratch_of_current_device).
constexpr size_t kNoAllocScratchBytes = (size_t)4 << 20;
static __device__ __align__(256) uint64_t scratch[kNoAllocScratchBytes / sizeof(uint64_t)];

namespace {

constexpr int kArgmaxThreads = 256;
constexpr int64_t kChunkQuantum = 2048;    // elements; keeps 16-byte alignment for fp32 and bf16
constexpr int64_t kTargetWorkgroups = 8192;
constexpr int kWalkThreads = 256;
constexpr int kSerialWalkMax = 256;  // trees up to this many nodes walk on one thread

struct ChunkPlan {
    int64_t chunk_len;
    int64_t n_chunks;
};

ChunkPlan plan_chunks(int64_t rows, int64_t vocab) {
    ChunkPlan p;
    int64_t want = rows > 0 ? (kTargetWorkgroups + rows - 1) / rows : 1;
    if (want < 1) want = 1;
    int64_t len = (vocab + want - 1) / want;
    len = ((len + kChunkQuantum - 1) / kChunkQuantum) * kChunkQuantum;
    if (len < 2 * kChunkQuantum) len = 2 * kChunkQuantum;
    p.chunk_len = len;
    p.n_chunks = (vocab + len - 1) / len;
    return p;
}

// One row's value at index idx: the logit itself (greedy), or, with noise,
// fl32(fl32(x * inv_t) + g): the temperature-scaled logit plus that element's
// Gumbel noise, each operation rounded once (no fused multiply-add), so the
// sampled choice is the argmax of exactly these float32 values.
template <bool kNoise>
__device__ __forceinline__ float choice_value(float x, float g, float inv_t) {
    if (!kNoise) return x;
    return __fadd_rn(__fmul_rn(x, inv_t), g);
}

template <bool kBf16, bool kNoise>
__global__ __launch_bounds__(kArgmaxThreads) void row_argmax_partial_kernel(
    const void* __restrict__ logits, const float* __restrict__ noise, float inv_t, int64_t vocab,
    int64_t chunk_len, int64_t n_chunks, uint64_t* __restrict__ partial) {
    __shared__ uint64_t s_red[kArgmaxThreads / TTV_WAVE];
    const int64_t row = blockIdx.x / n_chunks;
    const int64_t chunk = blockIdx.x % n_chunks;
    const int64_t e0 = chunk * chunk_len;
    const int64_t e1 = e0 + chunk_len < vocab ? e0 + chunk_len : vocab;
    const int tid = threadIdx.x;
    constexpr int kEpv = kBf16 ? 8 : 4;  // elements per 16-byte vector
    const size_t esize = kBf16 ? 2 : 4;
    const char* row_base = (const char*)logits + (size_t)row * (size_t)vocab * esize;
    const float* noise_row = kNoise ? noise + (size_t)row * (size_t)vocab : nullptr;

    // Start from the thread's first element so an all -inf range still names
    // its lowest index; threads with no element report key 0 (below any value).
    float best = -INFINITY;
    const bool vec_ok = ((vocab * (int64_t)esize) % 16 == 0) && (((uintptr_t)logits & 15) == 0) &&
                        (!kNoise || (vocab % 4 == 0 && ((uintptr_t)noise & 15) == 0));
    uint32_t best_i = 0xFFFFFFFFu;
    {
        const int64_t first = e0 + (int64_t)tid * (vec_ok ? kEpv : 1);
        if (first < e1) best_i = (uint32_t)first;
    }
    if (vec_ok) {
        const ttv_u32x4* vbase = (const ttv_u32x4*)row_base;
        const ttv_u32x4* nbase = (const ttv_u32x4*)noise_row;
        constexpr int kNv = kNoise ? kEpv / 4 : 0;  // 16-byte noise vectors per logits vector
        const int64_t stride = (int64_t)kArgmaxThreads * kEpv;
        for (int64_t base = e0 + (int64_t)tid * kEpv; base < e1; base += 4 * stride) {
            ttv_u32x4 v[4];
            ttv_u32x4 nz[4][kNv > 0 ? kNv : 1];
#pragma unroll
            for (int u = 0; u < 4; ++u) {
                const int64_t idx = base + u * stride;
                if (idx < e1) {
                    v[u] = __builtin_nontemporal_load(vbase + idx / kEpv);
#pragma unroll
                    for (int k = 0; k < kNv; ++k) nz[u][k] = __builtin_nontemporal_load(nbase + idx / 4 + k);
                }
            }
#pragma unroll
            for (int u = 0; u < 4; ++u) {
                const int64_t idx = base + u * stride;
                if (idx < e1) {
#pragma unroll
                    for (int w = 0; w < 4; ++w) {
                        if (kBf16) {
                            const float g0 = kNoise ? __uint_as_float(nz[u][w / 2][2 * (w % 2)]) : 0.f;
                            const float g1 = kNoise ? __uint_as_float(nz[u][w / 2][2 * (w % 2) + 1]) : 0.f;
                            const float f0 = choice_value<kNoise>(ttv_bf16_lo(v[u][w]), g0, inv_t);
                            const float f1 = choice_value<kNoise>(ttv_bf16_hi(v[u][w]), g1, inv_t);
                            if (f0 > best) { best = f0; best_i = (uint32_t)(idx + 2 * w); }
                            if (f1 > best) { best = f1; best_i = (uint32_t)(idx + 2 * w + 1); }
                        } else {
                            const float g = kNoise ? __uint_as_float(nz[u][0][w]) : 0.f;
                            const float f = choice_value<kNoise>(__uint_as_float(v[u][w]), g, inv_t);
                            if (f > best) { best = f; best_i = (uint32_t)(idx + w); }
                        }
                    }
                }
            }
        }
    } else {
        for (int64_t idx = e0 + tid; idx < e1; idx += kArgmaxThreads) {
            float f;
            if (kBf16) f = __uint_as_float((uint32_t)((const uint16_t*)row_base)[idx] << 16);
            else f = ((const float*)row_base)[idx];
            f = choice_value<kNoise>(f, kNoise ? noise_row[idx] : 0.f, inv_t);
            if (f > best) { best = f; best_i = (uint32_t)idx; }
        }
    }
    TTV_DCHECK(best_i == 0xFFFFFFFFu || (best_i >= (uint64_t)e0 && best_i < (uint64_t)e1), TTV_SITE_ACCEPT_KEY);
    uint64_t key = best_i == 0xFFFFFFFFu ? 0ull : ttv_argmax_key(__float_as_uint(best), best_i);
    key = ttv_wave_max_u64(key);
    if ((tid & (TTV_WAVE - 1)) == 0) s_red[tid / TTV_WAVE] = key;
    __syncthreads();
    if (tid == 0) {
        uint64_t k = s_red[0];
#pragma unroll
        for (int w = 1; w < kArgmaxThreads / TTV_WAVE; ++w) k = s_red[w] > k ? s_red[w] : k;
        partial[row * n_chunks + chunk] = k;
    }
}

__global__ __launch_bounds__(kWalkThreads) void greedy_walk_kernel(
    const int32_t* __restrict__ node_offsets, int32_t n_max, int64_t total_nodes, const uint64_t* __restrict__ partial,
    int64_t n_chunks, const int32_t* __restrict__ tokens, const int32_t* __restrict__ next_token,
    const int32_t* __restrict__ next_sibling, int32_t max_accept, int32_t* __restrict__ accept_len,
    int32_t* __restrict__ accepted_nodes, int32_t* __restrict__ out_tokens,
    int32_t* __restrict__ row_argmax, int32_t* __restrict__ err) {
    __shared__ unsigned long long s_key[TTV_MAX_TREE_NODES + 1];
    __shared__ int32_t s_tok[TTV_MAX_TREE_NODES];
    __shared__ int32_t s_first[TTV_MAX_TREE_NODES];
    __shared__ int32_t s_next[TTV_MAX_TREE_NODES];
    __shared__ int32_t s_path[TTV_MAX_TREE_NODES + 1];
    __shared__ int32_t s_par[TTV_MAX_TREE_NODES];   // parent rebuilt from the links
    __shared__ int32_t s_prev[TTV_MAX_TREE_NODES];  // previous sibling, then jumps
    __shared__ int32_t s_wmin[kWalkThreads / TTV_WAVE];
    __shared__ int32_t s_walk[3];  // serial walk's result: accepted, bonus, flags

    const int b = blockIdx.x;
    const int tid = threadIdx.x;
    // Stages the argmax key of rows [s + b, s + b + n] (the maximum of each
    // row's chunk keys) and the nodes' tokens and retrieve links in LDS.
    auto stage = [&](int s, int n) {
        const int64_t nc = n_chunks;
        const uint64_t* pk = partial + ((int64_t)s + b) * nc;
        // This thread's node links load first; then each row's chunk keys,
        // up to NB of them in flight before any is compared (past the last
        // chunk the loads repeat it, which leaves the maximum unchanged).
        int tok = 0, fc = -1, nx = -1;
        if (tid < n) {
            tok = tokens[s + tid];
            fc = next_token[s + tid];
            nx = next_sibling[s + tid];
        }
        auto reduce_rows = [&](auto nb_c) {
            constexpr int NB = decltype(nb_c)::value;
            for (int r = tid; r <= n; r += kWalkThreads) {
                const uint64_t* row = pk + (int64_t)r * nc;
                uint64_t best = 0ull;
                for (int64_t c0 = 0; c0 < nc; c0 += NB) {
                    uint64_t k[NB];
#pragma unroll
                    for (int u = 0; u < NB; ++u) k[u] = row[min(c0 + u, nc - 1)];
#pragma unroll
                    for (int u = 0; u < NB; ++u) best = k[u] > best ? k[u] : best;
                }
                s_key[r] = best;
            }
        };
        if (nc <= 4) reduce_rows(std::integral_constant<int, 4>{});
        else if (nc <= 8) reduce_rows(std::integral_constant<int, 8>{});
        else reduce_rows(std::integral_constant<int, 32>{});
        if (tid < n) {
            s_tok[tid] = tok;
            s_first[tid] = fc;
            s_next[tid] = nx;
        }
        for (int i = tid + kWalkThreads; i < n; i += kWalkThreads) {
            s_tok[i] = tokens[s + i];
            s_first[i] = next_token[s + i];
            s_next[i] = next_sibling[s + i];
        }
        __syncthreads();
    };
    // Request 0 starts at node 0 (node_offsets[0] = 0): stage up to n_max
    // nodes before the offsets arrive, and redo it only if they disagree.
    const bool spec = b == 0;
    const int n_spec = (int)min((int64_t)n_max, total_nodes);
    if (spec) stage(0, n_spec);
    const int s = node_offsets[b];
    const int n = node_offsets[b + 1] - s;
    if (s < 0 || n < 0 || n > n_max || (int64_t)s + n > total_nodes) {  // uniform
        if (tid == 0) {
            accept_len[b] = 0;
            atomicOr(err + b, TTV_ERR_TOO_MANY_NODES);
        }
        return;
    }
    if (!spec || s != 0) stage(s, n);
    const int64_t row0 = (int64_t)s + b;
    if (row_argmax && TTV_DCHECK(row0 + n < total_nodes + gridDim.x, TTV_SITE_WALK))
        for (int r = tid; r <= n; r += kWalkThreads) row_argmax[row0 + r] = (int32_t)ttv_key_index(s_key[r]);
    int a = 0, flags = 0;
    int target = (int)ttv_key_index(s_key[0]);
    if (n <= kSerialWalkMax) {
        // Small trees: thread 0 follows the links (a depth's sibling list is
        // short; the parallel walk's barriers would cost more).
        if (tid == 0) {
            int j = n > 0 ? 0 : -1;  // node 0 is the root's first child (parent[0] == -1)
            while (j >= 0) {
                // scan the sibling list starting at j for the target token
                while (j >= 0 && s_tok[j] != target) {
                    const int nx = s_next[j];
                    j = (nx > j && nx < n) ? nx : -1;
                }
                if (j < 0) break;
                if (a == max_accept) {
                    flags |= TTV_ERR_ACCEPT;
                    break;
                }
                s_path[a++] = j;
                target = (int)ttv_key_index(s_key[1 + j]);
                const int fc = s_first[j];
                j = (fc > j && fc < n) ? fc : -1;
            }
            s_walk[0] = a;
            s_walk[1] = target;
            s_walk[2] = flags;
        }
        __syncthreads();
        a = s_walk[0];
        target = s_walk[1];
        flags = s_walk[2];
    } else {
        // Parents from the links (forward links only, as the walk follows them):
        // a first child's parent is the node naming it; a later sibling's is its
        // previous sibling's, resolved by pointer jumping over the backward
        // previous-sibling links (about log2 of the longest sibling list rounds).
        // Node 0 is the root's first child (parent -1).  kUnknown marks a node
        // no link reaches; such a node is never matched.
        constexpr int kUnknown = -2;
        for (int i = tid; i < n; i += kWalkThreads) {
            s_par[i] = i == 0 ? -1 : kUnknown;
            s_prev[i] = -1;
        }
        __syncthreads();
        for (int i = tid; i < n; i += kWalkThreads) {
            const int fc = s_first[i], nx = s_next[i];
            if (fc > i && fc < n) s_par[fc] = i;
            if (nx > i && nx < n) s_prev[nx] = i;
        }
        __syncthreads();
        for (;;) {
            bool open = false;
            int par_new[(TTV_MAX_TREE_NODES + kWalkThreads - 1) / kWalkThreads];
            int prev_new[(TTV_MAX_TREE_NODES + kWalkThreads - 1) / kWalkThreads];
#pragma unroll
            for (int u = 0; u * kWalkThreads < TTV_MAX_TREE_NODES; ++u) {
                const int i = tid + u * kWalkThreads;
                par_new[u] = kUnknown;
                prev_new[u] = -1;
                if (i < n) {
                    par_new[u] = s_par[i];
                    prev_new[u] = s_prev[i];
                    if (par_new[u] == kUnknown && prev_new[u] >= 0) {
                        const int pp = s_par[prev_new[u]];
                        if (pp != kUnknown) par_new[u] = pp;
                        else prev_new[u] = s_prev[prev_new[u]];
                        open = open || (par_new[u] == kUnknown && prev_new[u] >= 0);
                    }
                }
            }
            __syncthreads();  // every read of this round before any write
#pragma unroll
            for (int u = 0; u * kWalkThreads < TTV_MAX_TREE_NODES; ++u) {
                const int i = tid + u * kWalkThreads;
                if (i < n) {
                    s_par[i] = par_new[u];
                    s_prev[i] = prev_new[u];
                }
            }
            if (!__syncthreads_or(open)) break;
        }
        // The walk: from the root, the lowest-index child of the current node
        // whose token is the current choice, found by all threads at once.
        constexpr int kNone = 0x7FFFFFFF;
        int cur = -1;
        for (;;) {
            int best = kNone;
            for (int i = tid; i < n; i += kWalkThreads)
                if (s_par[i] == cur && s_tok[i] == target) {
                    best = i;  // i increases, so the first hit is this thread's lowest
                    break;
                }
#pragma unroll
            for (int off = 32; off >= 1; off >>= 1) best = min(best, __shfl_xor(best, off));
            if ((tid & (TTV_WAVE - 1)) == 0) s_wmin[tid / TTV_WAVE] = best;
            __syncthreads();
            int j = kNone;
#pragma unroll
            for (int w = 0; w < kWalkThreads / TTV_WAVE; ++w) j = min(j, s_wmin[w]);
            __syncthreads();  // s_wmin is rewritten by the next depth
            if (j == kNone) break;
            if (a == max_accept) {
                flags |= TTV_ERR_ACCEPT;
                break;
            }
            if (tid == 0) s_path[a] = j;
            ++a;
            target = (int)ttv_key_index(s_key[1 + j]);
            cur = j;
        }
    }
    // a, target (the bonus) and flags are the same in every thread
    if (tid == 0) {
        accept_len[b] = a;
        if (flags) atomicOr(err + b, flags);
    }
    __syncthreads();  // s_path, written by thread 0
    for (int k = tid; k < max_accept; k += kWalkThreads)
        accepted_nodes[(int64_t)b * max_accept + k] =
            k < a && TTV_DCHECK(s_path[k] >= 0 && s_path[k] < n, TTV_SITE_WALK) ? s_path[k] : -1;
    for (int k = tid; k <= max_accept; k += kWalkThreads)
        out_tokens[(int64_t)b * (max_accept + 1) + k] =
            k < a ? s_tok[s_path[k]] : (k == a ? target : -1);
}

// The scratch array's device address on each device, taken once per device
// with that device current (the array's name is only a host-side stand-in).
constexpr int kMaxDevices = 64;
std::atomic<uint64_t*> g_scratch[kMaxDevices];

int scratch_of_current_device(uint64_t** out) {
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess) return TTV_EHIP;
    if (dev < 0 || dev >= kMaxDevices) return TTV_EINVAL;
    uint64_t* p = g_scratch[dev].load(std::memory_order_acquire);
    if (!p) {
        void* addr = nullptr;
        if (hipGetSymbolAddress(&addr, HIP_SYMBOL(scratch)) != hipSuccess || !addr) return TTV_EHIP;
        p = (uint64_t*)addr;
        g_scratch[dev].store(p, std::memory_order_release);
    }
    *out = p;
    return TTV_OK;
}

int check_accept_args(const ttv_batch* bt, int32_t logits_dtype, int64_t vocab, int32_t max_accept) {
    if (!bt || bt->batch < 0 || bt->n_max < 0 || bt->n_max > TTV_MAX_TREE_NODES ||
        bt->total_nodes < 0 || bt->total_nodes > (int64_t)bt->batch * bt->n_max)
        return TTV_EINVAL;
    if (logits_dtype != TTV_DTYPE_FP32 && logits_dtype != TTV_DTYPE_BF16) return TTV_EINVAL;
    if (vocab <= 0 || vocab >= (1ll << 31) || max_accept < 1 || max_accept > TTV_MAX_TREE_NODES)
        return TTV_EINVAL;
    return TTV_OK;
}

int check_accept_pointers(const ttv_batch* bt, const void* logits, const int32_t* tokens,
                          const int32_t* retrieve_next_token, const int32_t* retrieve_next_sibling,
                          const int32_t* accept_len, const int32_t* accepted_nodes,
                          const int32_t* out_tokens, const int32_t* err) {
    if (!bt->node_offsets || !logits || !accept_len || !accepted_nodes || !out_tokens || !err)
        return TTV_EINVAL;
    if (bt->total_nodes > 0 && (!tokens || !retrieve_next_token || !retrieve_next_sibling))
        return TTV_EINVAL;
    return TTV_OK;
}

// The two launches of an accept call, with the argmax keys in `partial`:
// greedy when noise is null, else the temperature-sampled choice.
int launch_accept(const ttv_batch* bt, const void* logits, int32_t logits_dtype, int64_t vocab,
                  const float* noise, float inv_t, const int32_t* tokens,
                  const int32_t* retrieve_next_token, const int32_t* retrieve_next_sibling,
                  int32_t max_accept, int32_t* accept_len, int32_t* accepted_nodes,
                  int32_t* out_tokens, int32_t* row_argmax, uint64_t* partial, int32_t* err,
                  hipStream_t stream) {
    const int64_t rows = bt->total_nodes + bt->batch;
    const ChunkPlan p = plan_chunks(rows, vocab);
    const int64_t grid = rows * p.n_chunks;
    if (grid > 0x7FFFFFFF) return TTV_EINVAL;
    auto argmax = [&](auto kern) {
        hipLaunchKernelGGL(kern, dim3((unsigned)grid), dim3(kArgmaxThreads), 0, stream, logits, noise,
                           inv_t, vocab, p.chunk_len, p.n_chunks, partial);
    };
    const bool bf16 = logits_dtype == TTV_DTYPE_BF16;
    if (noise) {
        if (bf16) argmax(row_argmax_partial_kernel<true, true>);
        else argmax(row_argmax_partial_kernel<false, true>);
    } else {
        if (bf16) argmax(row_argmax_partial_kernel<true, false>);
        else argmax(row_argmax_partial_kernel<false, false>);
    }
    if (hipGetLastError() != hipSuccess) return TTV_EHIP;
    hipLaunchKernelGGL(greedy_walk_kernel, dim3(bt->batch), dim3(kWalkThreads), 0, stream,
                       bt->node_offsets, bt->n_max, bt->total_nodes, partial, p.n_chunks, tokens,
                       retrieve_next_token, retrieve_next_sibling, max_accept, accept_len,
                       accepted_nodes, out_tokens, row_argmax, err);
    return hipGetLastError() == hipSuccess ? TTV_OK : TTV_EHIP;
}

}  // namespace

extern "C" TTV_API size_t tree_greedy_accept_workspace_bytes(const ttv_batch* bt, int64_t vocab) {
    if (!bt || bt->batch < 0 || bt->total_nodes < 0 || vocab <= 0 || vocab >= (1ll << 31))
        return 0;
    const int64_t rows = bt->total_nodes + bt->batch;
    const ChunkPlan p = plan_chunks(rows, vocab);
    const size_t bytes = (size_t)rows * (size_t)p.n_chunks * sizeof(uint64_t);
    return bytes > 0 ? bytes : 256;
}

extern "C" TTV_API int tree_greedy_accept(
    const ttv_batch* bt, const void* logits, int32_t logits_dtype, int64_t vocab,
    const int32_t* tokens, const int32_t* retrieve_next_token,
    const int32_t* retrieve_next_sibling, int32_t max_accept, int32_t* accept_len,
    int32_t* accepted_nodes, int32_t* out_tokens, int32_t* row_argmax, void* workspace,
    size_t workspace_bytes, int32_t* err, hipStream_t stream) {
    int st = check_accept_args(bt, logits_dtype, vocab, max_accept);
    if (st != TTV_OK) return st;
    if (bt->batch == 0) return TTV_OK;
    st = check_accept_pointers(bt, logits, tokens, retrieve_next_token, retrieve_next_sibling,
                               accept_len, accepted_nodes, out_tokens, err);
    if (st != TTV_OK) return st;
    if (!workspace) return TTV_EINVAL;
    const size_t need = tree_greedy_accept_workspace_bytes(bt, vocab);
    if (workspace_bytes < need) return TTV_ENOSPC;
    return launch_accept(bt, logits, logits_dtype, vocab, nullptr, 1.0f, tokens,
                         retrieve_next_token, retrieve_next_sibling, max_accept, accept_len,
                         accepted_nodes, out_tokens, row_argmax, (uint64_t*)workspace, err, stream);
}

extern "C" TTV_API int tree_greedy_accept_noalloc(
    const ttv_batch* bt, const void* logits, int32_t logits_dtype, int64_t vocab,
    const int32_t* tokens, const int32_t* retrieve_next_token,
    const int32_t* retrieve_next_sibling, int32_t max_accept, int32_t* accept_len,
    int32_t* accepted_nodes, int32_t* out_tokens, int32_t* row_argmax, int32_t* err,
    hipStream_t stream) {
    int st = check_accept_args(bt, logits_dtype, vocab, max_accept);
    if (st != TTV_OK) return st;
    // The keys must fit the static scratch: checked before any device call.
    if (tree_greedy_accept_workspace_bytes(bt, vocab) > kNoAllocScratchBytes) return TTV_ENOSPC;
    if (bt->batch == 0) return TTV_OK;
    st = check_accept_pointers(bt, logits, tokens, retrieve_next_token, retrieve_next_sibling,
                               accept_len, accepted_nodes, out_tokens, err);
    if (st != TTV_OK) return st;
    uint64_t* keys = nullptr;
    st = scratch_of_current_device(&keys);
    if (st != TTV_OK) return st;
    // Every key slot the walk reads is written by this call's argmax launch,
    // so the scratch needs no clearing.
    return launch_accept(bt, logits, logits_dtype, vocab, nullptr, 1.0f, tokens,
                         retrieve_next_token, retrieve_next_sibling, max_accept, accept_len,
                         accepted_nodes, out_tokens, row_argmax, keys, err, stream);
}

extern "C" TTV_API int tree_sample_accept(
    const ttv_batch* bt, const void* logits, int32_t logits_dtype, int64_t vocab,
    float temperature, const float* gumbel, const int32_t* tokens,
    const int32_t* retrieve_next_token, const int32_t* retrieve_next_sibling, int32_t max_accept,
    int32_t* accept_len, int32_t* accepted_nodes, int32_t* out_tokens, int32_t* row_choice,
    void* workspace, size_t workspace_bytes, int32_t* err, hipStream_t stream) {
    int st = check_accept_args(bt, logits_dtype, vocab, max_accept);
    if (st != TTV_OK) return st;
    if (!(temperature > 0.f) || !(temperature < INFINITY)) return TTV_EINVAL;
    const float inv_t = 1.0f / temperature;  // fl32(1 / T): the float32 scale of every logit
    if (!(inv_t < INFINITY)) return TTV_EINVAL;
    if (bt->batch == 0) return TTV_OK;
    st = check_accept_pointers(bt, logits, tokens, retrieve_next_token, retrieve_next_sibling,
                               accept_len, accepted_nodes, out_tokens, err);
    if (st != TTV_OK) return st;
    if (!gumbel || !workspace) return TTV_EINVAL;
    if (tree_greedy_accept_workspace_bytes(bt, vocab) > workspace_bytes) return TTV_ENOSPC;
    return launch_accept(bt, logits, logits_dtype, vocab, gumbel, inv_t, tokens,
                         retrieve_next_token, retrieve_next_sibling, max_accept, accept_len,
                         accepted_nodes, out_tokens, row_choice, (uint64_t*)workspace, err, stream);
}

TTV_DEBUG_TU(accept)
