// tree_stochastic_accept: the stochastic per-edge acceptance walk.
//
// "02 · Token Tree 与 Tree Attention" §4: one target pass gives every node a
// distribution p; from the root each child of the current node is accepted
// or rejected by the min(1, p/q) rule (speculative sampling's: a draft token
// x proposed from q is kept with probability min(1, p(x)/q(x)), and after a
// rejection the target side continues from the residual norm(max(0, p - q)));
// an accepted child becomes the current node; when every child is rejected a
// correction token is sampled at the current node and the walk ends; at a
// leaf the bonus token is sampled from the leaf's p.
//
// Choices made where the page is open: siblings are tried in increasing
// index order, each rejection replacing the target side by the residual; p
// of a row is softmax(logits / T) in float64; node j's accept test is
// u_j * q(x_j) < r(x_j) in float64 (u_j the caller's uniform draw for node j,
// q the draft distribution the children of the current node came from, r the
// current target side); the correction / bonus is the Gumbel-max sample
// argmax_v (log r_v + g_v) over r_v > 0 with the caller's noise g of that row.
//
// For a vocab that is not a multiple of 8, one 1024-thread workgroup per
// request walks the tree; each step that needs the whole distribution (a
// visited row's softmax, a residual, the final sample) is a pass of the
// workgroup over the vocab with fp64 block reductions, each thread loading
// four entries before using any.  Otherwise a group of up to 16 workgroups
// per request walks it, each over a slice of the vocab (below).  The
// current target side is kept as r_v = buf[v] / den: the row's exp values and
// their sum right after a visit, the unnormalised residual and its sum after
// a rejection (buf in the caller's workspace, fp64 [B, vocab]).  The accept
// test forms r_x by that division; the passes over the whole vocab multiply
// by 1 / den instead (within an ulp of the quotient: a float64 division per
// entry cost about as much as the rest of the pass).

#include <algorithm>
#include <atomic>

#include "ttv_device.h"

namespace {

constexpr int kThreads = 1024;
constexpr int kWaves = kThreads / TTV_WAVE;
constexpr int kBatch = 4;  // loads in flight per thread in a vocab pass

__device__ __forceinline__ double shfl_xor_f64(double v, int off) {
    const uint64_t u = __double_as_longlong(v);
    const uint32_t lo = __shfl_xor((uint32_t)u, off, TTV_WAVE);
    const uint32_t hi = __shfl_xor((uint32_t)(u >> 32), off, TTV_WAVE);
    return __longlong_as_double((long long)(((uint64_t)hi << 32) | lo));
}

template <bool kMax, int kNW = kWaves>
__device__ double block_reduce(double v, double* s_red) {
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) {
        const double o = shfl_xor_f64(v, off);
        v = kMax ? fmax(v, o) : v + o;
    }
    const int tid = threadIdx.x;
    __syncthreads();  // s_red may still be read by the previous reduction
    if ((tid & (TTV_WAVE - 1)) == 0) s_red[tid / TTV_WAVE] = v;
    __syncthreads();
    double r = s_red[0];
    for (int w = 1; w < kNW; ++w) r = kMax ? fmax(r, s_red[w]) : r + s_red[w];
    return r;
}

// (score, index) maximum, lowest index on equal scores.
template <int kNW = kWaves>
__device__ int block_argmax(double v, int idx, double* s_val, int* s_idx, double* best = nullptr) {
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) {
        const double ov = shfl_xor_f64(v, off);
        const int oi = __shfl_xor(idx, off, TTV_WAVE);
        if (ov > v || (ov == v && oi < idx)) {
            v = ov;
            idx = oi;
        }
    }
    const int tid = threadIdx.x;
    __syncthreads();
    if ((tid & (TTV_WAVE - 1)) == 0) {
        s_val[tid / TTV_WAVE] = v;
        s_idx[tid / TTV_WAVE] = idx;
    }
    __syncthreads();
    double bv = s_val[0];
    int bi = s_idx[0];
    for (int w = 1; w < kNW; ++w)
        if (s_val[w] > bv || (s_val[w] == bv && s_idx[w] < bi)) {
            bv = s_val[w];
            bi = s_idx[w];
        }
    if (best) *best = bv;
    return bi;
}

template <bool kBf16>
__device__ __forceinline__ double logit_at(const void* logits, int64_t row, int64_t vocab, int64_t v) {
    if (kBf16) return (double)__uint_as_float((uint32_t)((const uint16_t*)logits)[row * vocab + v] << 16);
    return (double)((const float*)logits)[row * vocab + v];
}

// f(v, j) for the entries v = base + j * kThreads + tid, j < kBatch, of every
// batch; load(v, j) runs for all of a batch's entries first, so their loads
// are in flight together.  v increases along each thread's calls.
template <typename Load, typename Use>
__device__ __forceinline__ void vocab_pass(int64_t vocab, Load&& load, Use&& use) {
    const int tid = threadIdx.x;
    for (int64_t base = 0; base < vocab; base += (int64_t)kBatch * kThreads) {
#pragma unroll
        for (int j = 0; j < kBatch; ++j) {
            const int64_t v = base + (int64_t)j * kThreads + tid;
            if (v < vocab) load(v, j);
        }
#pragma unroll
        for (int j = 0; j < kBatch; ++j) {
            const int64_t v = base + (int64_t)j * kThreads + tid;
            if (v < vocab) use(v, j);
        }
    }
}

template <bool kBf16>
__global__ __launch_bounds__(kThreads) void stochastic_walk_kernel(
    const int32_t* __restrict__ node_offsets, int32_t n_max, int64_t total_nodes,
    const void* __restrict__ logits, int64_t vocab, double temperature,
    const float* __restrict__ draft_probs, const float* __restrict__ uniforms,
    const float* __restrict__ gumbel, const int32_t* __restrict__ tokens,
    const int32_t* __restrict__ next_token, const int32_t* __restrict__ next_sibling,
    int32_t max_accept, int32_t* __restrict__ accept_len, int32_t* __restrict__ accepted_nodes,
    int32_t* __restrict__ out_tokens, double* __restrict__ work, int32_t* __restrict__ err) {
    __shared__ int32_t s_path[TTV_MAX_TREE_NODES + 1];
    __shared__ double s_red[kWaves];
    __shared__ int32_t s_ired[kWaves];

    const int b = blockIdx.x;
    const int tid = threadIdx.x;
    const int s = node_offsets[b];
    const int n = node_offsets[b + 1] - s;
    if (s < 0 || n < 0 || n > n_max || (int64_t)s + n > total_nodes) {  // uniform
        if (tid == 0) {
            accept_len[b] = 0;
            atomicOr(err + b, TTV_ERR_TOO_MANY_NODES);
        }
        return;
    }
    double* buf = work + (int64_t)b * vocab;
    const int64_t row0 = (int64_t)s + b;  // the request's root row
    // (x - max) / T as one multiply by 1 / T (the same value when T is a
    // power of two; otherwise within an ulp): an fp64 division per entry
    // cost about as much as the exponential
    const double inv_t = 1.0 / temperature;

    // Visit a row: buf = exp((x - max) / T), den = their sum.
    double xb[kBatch], bb[kBatch];
    float fb[kBatch];
    auto visit = [&](int64_t row) -> double {
        double m = -INFINITY;
        vocab_pass(vocab, [&](int64_t v, int j) { xb[j] = logit_at<kBf16>(logits, row, vocab, v); },
                   [&](int64_t, int j) { m = fmax(m, xb[j]); });
        m = block_reduce<true>(m, s_red);
        double sum = 0.0;
        vocab_pass(vocab, [&](int64_t v, int j) { xb[j] = logit_at<kBf16>(logits, row, vocab, v); },
                   [&](int64_t v, int j) {
                       const double e = exp((xb[j] - m) * inv_t);
                       buf[v] = e;
                       sum += e;
                   });
        __syncthreads();  // buf written before any thread reads another's entry
        return block_reduce<false>(sum, s_red);
    };

    int a = 0, flags = 0, final_token = -1;
    int cur = -1;
    int64_t row = row0;
    double den = visit(row);
    for (;;) {
        // children of the current node, lowest index first
        int j = cur < 0 ? (n > 0 ? 0 : -1) : next_token[s + cur];
        if (j >= 0 && (j <= cur || j >= n)) j = -1;
        const float* q = draft_probs + row * vocab;
        int accepted = -1;
        while (j >= 0) {
            const int x = tokens[s + j];
            const double r_x = (x >= 0 && x < vocab) ? buf[x] / den : 0.0;
            const double qx = (x >= 0 && x < vocab) ? (double)q[x] : 0.0;
            const bool take = (double)uniforms[s + j] * qx < r_x;
            __syncthreads();  // every thread has read buf[x] before the residual rewrites it
            if (take) {
                accepted = j;
                break;
            }
            // rejected: the target side becomes norm(max(0, r - q)); left as it
            // was when nothing remains above q (r == q up to rounding)
            double z = 0.0;
            auto load_bq = [&](int64_t v, int jj) {
                bb[jj] = buf[v];
                fb[jj] = q[v];
            };
            const double inv_den = 1.0 / den;
            vocab_pass(vocab, load_bq, [&](int64_t, int jj) { z += fmax(bb[jj] * inv_den - (double)fb[jj], 0.0); });
            z = block_reduce<false>(z, s_red);
            if (z > 0.0) {
                vocab_pass(vocab, load_bq,
                           [&](int64_t v, int jj) { buf[v] = fmax(bb[jj] * inv_den - (double)fb[jj], 0.0); });
                den = z;
                __syncthreads();
            }
            const int nx = next_sibling[s + j];
            j = (nx > j && nx < n) ? nx : -1;
        }
        if (accepted < 0) {
            // correction / bonus: Gumbel-max sample of the current side
            const float* g = gumbel + row * vocab;
            const double inv_den = 1.0 / den;
            double best = -INFINITY;
            int best_i = 0x7FFFFFFF;
            vocab_pass(vocab,
                       [&](int64_t v, int jj) {
                           bb[jj] = buf[v];
                           fb[jj] = g[v];
                       },
                       [&](int64_t v, int jj) {
                           const double r = bb[jj] * inv_den;
                           if (r > 0.0) {
                               const double sc = log(r) + (double)fb[jj];
                               if (sc > best) {  // v increases per thread: the first maximum is the lowest index
                                   best = sc;
                                   best_i = (int)v;
                               }
                           }
                       });
            final_token = block_argmax(best, best_i, s_red, s_ired);
            if (final_token == 0x7FFFFFFF) final_token = -1;
            break;
        }
        if (a == max_accept) {
            flags |= TTV_ERR_ACCEPT;
            break;
        }
        if (tid == 0) s_path[a] = accepted;
        ++a;
        cur = accepted;
        row = row0 + 1 + (TTV_DCHECK(accepted >= 0 && accepted < n, TTV_SITE_STOCHASTIC) ? accepted : 0);
        __syncthreads();  // every thread has read buf before the next visit rewrites it
        den = visit(row);
    }
    if (tid == 0) {
        accept_len[b] = a;
        if (flags) atomicOr(err + b, flags);
    }
    __syncthreads();  // s_path, written by thread 0
    for (int k = tid; k < max_accept; k += kThreads)
        accepted_nodes[(int64_t)b * max_accept + k] = k < a ? s_path[k] : -1;
    for (int k = tid; k <= max_accept; k += kThreads)
        out_tokens[(int64_t)b * (max_accept + 1) + k] =
            k < a ? tokens[s + s_path[k]] : (k == a ? final_token : -1);
}

// The same walk for a vocab that is a multiple of 8: each thread takes
// chunks of 8 consecutive entries (one 16-byte load of bf16 logits, two of
// fp32, four of fp64), so far more bytes are in flight per thread than with
// one entry per load; a rejection writes the residual into the request's
// second buffer in the same pass that sums it (the first buffer keeps the
// current side when nothing remains above q).  Entries are visited in
// increasing order per thread, as above.  When the device holds them all at
// once, a request is walked by a group of up to 16 such workgroups, each over
// its own slice of the vocab (below): the walk is a chain of dependent
// full-vocab passes, and one workgroup per request left seven in eight CUs
// idle on a batch of 32.
constexpr int kVec = 8;
constexpr int kVThreads = 512;  // 128 registers per thread (two workgroups per CU): a chunk in flight
constexpr int kVWaves = kVThreads / TTV_WAVE;

__device__ __forceinline__ void load8_logits(const void* logits, bool bf16, int64_t off, float (&x)[kVec]) {
    if (bf16) {
        const ttv_u32x4 w = *(const ttv_u32x4*)((const uint16_t*)logits + off);
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            x[2 * k] = __uint_as_float(w[k] << 16);
            x[2 * k + 1] = __uint_as_float(w[k] & 0xFFFF0000u);
        }
    } else {
        const float4 a = *(const float4*)((const float*)logits + off);
        const float4 c = *(const float4*)((const float*)logits + off + 4);
        x[0] = a.x; x[1] = a.y; x[2] = a.z; x[3] = a.w;
        x[4] = c.x; x[5] = c.y; x[6] = c.z; x[7] = c.w;
    }
}
__device__ __forceinline__ void load8_f32(const float* p, float (&x)[kVec]) {
    const float4 a = *(const float4*)p, c = *(const float4*)(p + 4);
    x[0] = a.x; x[1] = a.y; x[2] = a.z; x[3] = a.w;
    x[4] = c.x; x[5] = c.y; x[6] = c.z; x[7] = c.w;
}
__device__ __forceinline__ void load8_f64(const double* p, double (&x)[kVec]) {
#pragma unroll
    for (int k = 0; k < 4; ++k) {
        const double2 v = *(const double2*)(p + 2 * k);
        x[2 * k] = v.x;
        x[2 * k + 1] = v.y;
    }
}
__device__ __forceinline__ void store8_f64(double* p, const double (&x)[kVec]) {
#pragma unroll
    for (int k = 0; k < 4; ++k) *(double2*)(p + 2 * k) = make_double2(x[2 * k], x[2 * k + 1]);
}

// Chunks c = base + j * kVThreads + tid, j < NB, of every batch of the slice
// [c_lo, c_hi): load(c, j) for the whole batch, then use(c, j).
template <int NB, typename Load, typename Use>
__device__ __forceinline__ void chunk_pass(int64_t c_lo, int64_t c_hi, Load&& load, Use&& use) {
    const int tid = threadIdx.x;
    for (int64_t base = c_lo; base < c_hi; base += (int64_t)NB * kVThreads) {
#pragma unroll
        for (int j = 0; j < NB; ++j) {
            const int64_t c = base + (int64_t)j * kVThreads + tid;
            if (c < c_hi) load(c, j);
        }
#pragma unroll
        for (int j = 0; j < NB; ++j) {
            const int64_t c = base + (int64_t)j * kVThreads + tid;
            if (c < c_hi) use(c, j);
        }
    }
}

// A request may be walked by a group of P workgroups, each over its own slice
// of the vocab's chunks.  Every reduction is then taken over the workgroup
// and exchanged: each member publishes its result and waits for the others',
// and all combine the P results in member order, so the whole group holds the
// same value and takes the same decisions.  A result travels as 32-bit words,
// each in a 64-bit atomic word beside the number of the exchange (from 1), so
// a word read with the expected number is that exchange's word: no fence is
// needed, and no member ever reads another's entries of the request's
// buffers (the accept test recomputes its entry, below).  Exchange e uses
// word set e mod 2: a member writes exchange e + 2 only after every member
// has written e + 1, i.e. has finished reading e.  The workspace holds one
// record per request after the two buffers, zeroed before each walk.
constexpr int kMaxGroup = 16;
constexpr int kXWords = 4;  // 32-bit words per member per exchange
constexpr int64_t kGroupRecord = 1024;
struct GroupRecord {
    uint64_t w[2][kMaxGroup][kXWords];  // (exchange number << 32) | word
};
static_assert(sizeof(GroupRecord) <= kGroupRecord, "group record");
// A wait for the rest of the group gives up after this many ticks of the
// 100 MHz real-time clock (about 0.3 s): it then flags TTV_ERR_SYNC and
// waits no more, so every workgroup still ends.
constexpr long long kSpinTicks = 1ll << 25;

__global__ void group_clear_kernel(unsigned char* __restrict__ groups, int32_t n) {
    const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    constexpr int kPer = kGroupRecord / 8;
    if (i < (int64_t)n * kPer) ((uint64_t*)groups)[i] = 0;
}

__device__ __forceinline__ uint32_t lo32(double v) { return (uint32_t)__double_as_longlong(v); }
__device__ __forceinline__ uint32_t hi32(double v) { return (uint32_t)((uint64_t)__double_as_longlong(v) >> 32); }
__device__ __forceinline__ double f64_of(uint32_t lo, uint32_t hi) {
    return __longlong_as_double((long long)(((uint64_t)hi << 32) | lo));
}

// Exchange number e: member p publishes words w0..w3 (the first n_words of
// them; uniform over the workgroup) and waits until every member's are in;
// member k's word i is then s_x[k * kXWords + i] for every thread.  Wave 0's
// lanes poll one word each.  Returns true once a wait has timed out (late
// stays true and later calls do not wait).
__device__ __forceinline__ bool group_exchange(GroupRecord* rec, int group, int p, int e, int n_words,
                                               uint32_t w0, uint32_t w1, uint32_t w2, uint32_t w3, bool late,
                                               uint32_t* s_x, int* s_flag) {
    const int tid = threadIdx.x;
    uint64_t(*const set)[kXWords] = rec->w[e & 1];
    if (tid < n_words) {
        const uint32_t w = tid == 0 ? w0 : tid == 1 ? w1 : tid == 2 ? w2 : w3;
        __hip_atomic_store(&set[p][tid], ((uint64_t)(uint32_t)e << 32) | w, __ATOMIC_RELAXED,
                           __HIP_MEMORY_SCOPE_AGENT);
    }
    if (tid < TTV_WAVE) {
        const int k = tid / n_words, i = tid % n_words;
        const bool mine = k < group;
        uint64_t v = 0;
        bool ok = !mine;
        int f = late;
        const long long t0 = wall_clock64();
        for (;;) {
            if (!ok) {
                v = __hip_atomic_load(&set[k][i], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                ok = (uint32_t)(v >> 32) == (uint32_t)e;
            }
            if (__all(ok)) break;
            if (f || wall_clock64() - t0 > kSpinTicks) {
                f = 1;
                break;
            }
            __builtin_amdgcn_s_sleep(1);
        }
        if (mine) s_x[k * kXWords + i] = (uint32_t)v;
        if (tid == 0) *s_flag = f;
    }
    __syncthreads();
    return *s_flag != 0;
}

// One step of a residual at one entry: max(0, r - q) with r = side * f, one
// fused rounding for the product and difference; the pass over a slice and
// the accept test's recomputation both use it, so they agree bit for bit.
__device__ __forceinline__ double residual_entry(double side, double f, double q) {
    return fmax(__builtin_fma(side, f, -q), 0.0);
}

template <bool kBf16>
// Four waves per SIMD: two workgroups per CU, so twice the members per request.
__global__ __launch_bounds__(kVThreads, 4) void stochastic_walk_vec_kernel(
    const int32_t* __restrict__ node_offsets, int32_t n_max, int64_t total_nodes,
    const void* __restrict__ logits, int64_t vocab, double temperature,
    const float* __restrict__ draft_probs, const float* __restrict__ uniforms,
    const float* __restrict__ gumbel, const int32_t* __restrict__ tokens,
    const int32_t* __restrict__ next_token, const int32_t* __restrict__ next_sibling,
    int32_t max_accept, int32_t* __restrict__ accept_len, int32_t* __restrict__ accepted_nodes,
    int32_t* __restrict__ out_tokens, double* __restrict__ work, int32_t* __restrict__ err,
    int32_t batch, int32_t group, unsigned char* __restrict__ groups) {
    __shared__ int32_t s_path[TTV_MAX_TREE_NODES + 1];
    __shared__ double s_red[kVWaves];
    __shared__ int32_t s_ired[kVWaves];
    __shared__ int s_flag;
    __shared__ double s_scale[kMaxGroup];  // per member: exp((its maximum - the row's) / T)
    __shared__ double s_mloc[kMaxGroup];   // per member: the maximum its exponentials subtract
    __shared__ uint32_t s_x[kMaxGroup * kXWords];  // the last exchange's words
    // the residuals applied at the current node, for the accept test's
    // recomputation: 1 / den before each, and its flags (1: the side was
    // scaled, 2: the residual replaced the side)
    __shared__ double s_hinv[TTV_MAX_TREE_NODES];
    __shared__ uint8_t s_hflag[TTV_MAX_TREE_NODES];

    // Workgroup w serves request b as member p of its group.  With groups,
    // the members of request b are w = (b / 8) * 8P + 8p + b % 8: all on the
    // XCD that w % 8 names, the grid padded to a multiple of 8 requests.
    int b = blockIdx.x, p = 0;
    if (group > 1) {
        const int w8 = blockIdx.x / 8;
        p = w8 % group;
        b = (w8 / group) * 8 + blockIdx.x % 8;
        if (b >= batch) return;  // padding: uniform over the workgroup
    }
    const int tid = threadIdx.x;
    const int s = node_offsets[b];
    const int n = node_offsets[b + 1] - s;
    if (s < 0 || n < 0 || n > n_max || (int64_t)s + n > total_nodes) {  // uniform over the group
        if (tid == 0 && p == 0) {
            accept_len[b] = 0;
            atomicOr(err + b, TTV_ERR_TOO_MANY_NODES);
        }
        return;
    }
    // the current side and the residual being formed, swapped on a rejection
    double* cur_buf = work + (int64_t)(2 * b) * vocab;
    double* alt_buf = cur_buf + vocab;
    const int64_t n_chunks = vocab / kVec;
    const int64_t c_lo = n_chunks * p / group, c_hi = n_chunks * (p + 1) / group;  // this member's slice
    const int64_t row0 = (int64_t)s + b;  // the request's root row
    const double inv_t = 1.0 / temperature;  // see stochastic_walk_kernel

    GroupRecord* const grec = group > 1 ? (GroupRecord*)(groups + b * kGroupRecord) : nullptr;
    int epoch = 0;
    bool late = false;
    // Sum over the request: the workgroup's, then the group's in member order.
    auto reduce_sum = [&](double v) -> double {
        double r = block_reduce<false, kVWaves>(v, s_red);
        if (group == 1) return r;
        late = group_exchange(grec, group, p, ++epoch, 2, lo32(r), hi32(r), 0, 0, late, s_x, &s_flag);
        r = f64_of(s_x[0], s_x[1]);
        for (int k = 1; k < group; ++k) r += f64_of(s_x[k * kXWords], s_x[k * kXWords + 1]);
        return r;
    };

    // Visit a row.  Each member takes the maximum m_p of its slice and stores
    // cur = exp((x - m_p) / T), summing them; one group-wide reduction then
    // gives the row's maximum M and den = sum over p (in member order) of
    // sum_p * exp((m_p - M) / T), so the side is cur[v] * s_scale[member of
    // v] / den: exp((x - M) / T) / den formed as a product of two
    // exponentials (within a few ulps).  One workgroup has m_p = M and the
    // scale exactly 1.
    bool scaled = false;  // the side carries the members' scales (after a visit)
    int n_hist = 0;       // residuals applied at the current node
    if (tid < kMaxGroup) s_scale[tid] = 1.0;
    auto visit = [&](int64_t row) -> double {
        constexpr int NB = 1;
        float xs[NB][kVec];
        float mf = -INFINITY;  // the logits are floats, so their maximum is exact
        chunk_pass<NB>(c_lo, c_hi, [&](int64_t c, int j) { load8_logits(logits, kBf16, row * vocab + c * kVec, xs[j]); },
                       [&](int64_t, int j) {
#pragma unroll
                           for (int k = 0; k < kVec; ++k) mf = fmaxf(mf, xs[j][k]);
                       });
        const double m_p = block_reduce<true, kVWaves>((double)mf, s_red);
        // a slice of -inf logits contributes nothing (rather than inf - inf)
        const double m = m_p == -INFINITY ? 0.0 : m_p;
        double sum = 0.0;
        chunk_pass<NB>(c_lo, c_hi, [&](int64_t c, int j) { load8_logits(logits, kBf16, row * vocab + c * kVec, xs[j]); },
                       [&](int64_t c, int j) {
                           double e[kVec];
#pragma unroll
                           for (int k = 0; k < kVec; ++k) {
                               e[k] = exp(((double)xs[j][k] - m) * inv_t);
                               sum += e[k];
                           }
                           store8_f64(cur_buf + c * kVec, e);
                       });
        const double s_p = block_reduce<false, kVWaves>(sum, s_red);
        scaled = true;
        n_hist = 0;
        if (group == 1) {
            if (tid == 0) s_mloc[0] = m;
            __syncthreads();  // s_mloc
            return s_p;
        }
        late = group_exchange(grec, group, p, ++epoch, 4, lo32(m_p), hi32(m_p), lo32(s_p), hi32(s_p), late, s_x,
                              &s_flag);
        double M = -INFINITY;
        for (int k = 0; k < group; ++k) M = fmax(M, f64_of(s_x[k * kXWords], s_x[k * kXWords + 1]));
        if (tid < group) {
            const double mk = f64_of(s_x[tid * kXWords], s_x[tid * kXWords + 1]);
            s_mloc[tid] = mk == -INFINITY ? 0.0 : mk;
            s_scale[tid] = mk == -INFINITY ? 0.0 : exp((mk - M) * inv_t);
        }
        __syncthreads();  // s_mloc, s_scale
        double den = 0.0;
        for (int k = 0; k < group; ++k) den += f64_of(s_x[k * kXWords + 2], s_x[k * kXWords + 3]) * s_scale[k];
        return den;
    };

    int a = 0, flags = 0, final_token = -1;
    int cur = -1;
    int64_t row = row0;
    double den = visit(row);
    for (;;) {
        int j = cur < 0 ? (n > 0 ? 0 : -1) : next_token[s + cur];
        if (j >= 0 && (j <= cur || j >= n)) j = -1;
        const float* q = draft_probs + row * vocab;
        int accepted = -1;
        while (j >= 0) {
            const int x = tokens[s + j];
            double r_x = 0.0;
            if (x >= 0 && x < vocab) {
                int px = 0;  // the member whose slice holds x
                while (px + 1 < group && n_chunks * (px + 1) / group <= x / kVec) ++px;
                // entry x of the side, formed as member px formed it: the
                // visit's exponential, then each residual applied since
                double side = exp((logit_at<kBf16>(logits, row, vocab, x) - s_mloc[px]) * inv_t);
                const double qx = (double)q[x];
                for (int i = 0; i < min(n_hist, TTV_MAX_TREE_NODES); ++i) {
                    const int fl = s_hflag[i];
                    const double t = residual_entry(side, ((fl & 1) ? s_scale[px] : 1.0) * s_hinv[i], qx);
                    if (fl & 2) side = t;
                }
                r_x = (scaled ? side * s_scale[px] : side) / den;
            }
            const double qx = (x >= 0 && x < vocab) ? (double)q[x] : 0.0;
            const bool take = (double)uniforms[s + j] * qx < r_x;
            if (take) {
                accepted = j;
                break;
            }
            // rejected: the residual max(0, r - q) into the other buffer, summed
            // in the same pass; it becomes the current side when the sum is
            // positive (otherwise r == q up to rounding and r stays)
            constexpr int NB = 1;
            double bb[NB][kVec];
            float fq[NB][kVec];
            double z = 0.0;
            const double inv_d = 1.0 / den;
            const double inv_den = (scaled ? s_scale[p] : 1.0) * inv_d;
            chunk_pass<NB>(c_lo, c_hi,
                           [&](int64_t c, int jj) {
                               load8_f64(cur_buf + c * kVec, bb[jj]);
                               load8_f32(q + c * kVec, fq[jj]);
                           },
                           [&](int64_t c, int jj) {
                               double t[kVec];
#pragma unroll
                               for (int k = 0; k < kVec; ++k) {
                                   t[k] = residual_entry(bb[jj][k], inv_den, (double)fq[jj][k]);
                                   z += t[k];
                               }
                               store8_f64(alt_buf + c * kVec, t);
                           });
            z = reduce_sum(z);
            if (tid == 0 && n_hist < TTV_MAX_TREE_NODES) {
                s_hinv[n_hist] = inv_d;
                s_hflag[n_hist] = (scaled ? 1 : 0) | (z > 0.0 ? 2 : 0);
            }
            ++n_hist;
            __syncthreads();  // s_hinv, s_hflag
            if (z > 0.0) {
                double* const t = cur_buf;
                cur_buf = alt_buf;
                alt_buf = t;
                den = z;
                scaled = false;
            }
            const int nx = next_sibling[s + j];
            j = (nx > j && nx < n) ? nx : -1;
        }
        if (accepted < 0) {
            // correction / bonus: Gumbel-max sample of the current side
            const float* g = gumbel + row * vocab;
            constexpr int NB = 1;
            double bb[NB][kVec];
            float fg[NB][kVec];
            const double inv_den = (scaled ? s_scale[p] : 1.0) * (1.0 / den);
            double best = -INFINITY;
            int best_i = 0x7FFFFFFF;
            chunk_pass<NB>(c_lo, c_hi,
                           [&](int64_t c, int jj) {
                               load8_f64(cur_buf + c * kVec, bb[jj]);
                               load8_f32(g + c * kVec, fg[jj]);
                           },
                           [&](int64_t c, int jj) {
#pragma unroll
                               for (int k = 0; k < kVec; ++k) {
                                   const double r = bb[jj][k] * inv_den;
                                   if (r > 0.0) {
                                       const double sc = log(r) + (double)fg[jj][k];
                                       if (sc > best) {  // entries increase per thread: the first maximum is the lowest index
                                           best = sc;
                                           best_i = (int)(c * kVec + k);
                                       }
                                   }
                               }
                           });
            double bv;
            final_token = block_argmax<kVWaves>(best, best_i, s_red, s_ired, &bv);
            if (group > 1) {
                late = group_exchange(grec, group, p, ++epoch, 3, lo32(bv), hi32(bv), (uint32_t)final_token, 0, late,
                                      s_x, &s_flag);
                bv = f64_of(s_x[0], s_x[1]);
                final_token = (int)s_x[2];
                for (int k = 1; k < group; ++k) {  // slices ascend with k: ties keep the lower index
                    const double o = f64_of(s_x[k * kXWords], s_x[k * kXWords + 1]);
                    const int oi = (int)s_x[k * kXWords + 2];
                    if (o > bv || (o == bv && oi < final_token)) {
                        bv = o;
                        final_token = oi;
                    }
                }
            }
            if (final_token == 0x7FFFFFFF) final_token = -1;
            break;
        }
        if (a == max_accept) {
            flags |= TTV_ERR_ACCEPT;
            break;
        }
        if (tid == 0) s_path[a] = accepted;
        ++a;
        cur = accepted;
        row = row0 + 1 + (TTV_DCHECK(accepted >= 0 && accepted < n, TTV_SITE_STOCHASTIC) ? accepted : 0);
        __syncthreads();  // s_path, and the walk's reads of LDS before the next visit
        den = visit(row);
    }
    if (late) flags |= TTV_ERR_SYNC;
    if (tid == 0 && (p == 0 || late)) {
        if (p == 0) accept_len[b] = a;
        if (flags) atomicOr(err + b, flags);
    }
    if (p != 0) return;  // uniform over the workgroup: one member writes the walk
    __syncthreads();  // s_path, written by thread 0
    for (int k = tid; k < max_accept; k += kVThreads)
        accepted_nodes[(int64_t)b * max_accept + k] = k < a ? s_path[k] : -1;
    for (int k = tid; k <= max_accept; k += kVThreads)
        out_tokens[(int64_t)b * (max_accept + 1) + k] =
            k < a ? tokens[s + s_path[k]] : (k == a ? final_token : -1);
}

}  // namespace

namespace {

// Two fp64 buffers of the vocab per request (the chunked path swaps them),
// then, 256-byte aligned, one group record per request.
size_t buffers_bytes(int64_t batch, int64_t vocab) {
    return (2 * (size_t)batch * (size_t)vocab * sizeof(double) + 255) & ~(size_t)255;
}

// Workgroups of the grouped walk that the device holds at once, per device
// and logits type (0 until asked).
constexpr int kMaxDevices = 64;
std::atomic<int> g_resident[kMaxDevices][2];

template <bool kBf16>
int resident_walkers() {
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return 0;
    std::atomic<int>& slot = g_resident[dev][kBf16 ? 1 : 0];
    int r = slot.load(std::memory_order_relaxed);
    if (r > 0) return r;
    int per_cu = 0, cus = 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, stochastic_walk_vec_kernel<kBf16>, kVThreads, 0) !=
            hipSuccess ||
        hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
        return 0;
    r = per_cu * cus;
    if (r > 0) slot.store(r, std::memory_order_relaxed);
    return r;
}

// Members per request: as many as the device holds for the padded batch at
// once, up to kMaxGroup, with at least half a chunk per thread each.
template <bool kBf16>
int walk_group(int64_t batch, int64_t n_chunks) {
    const int64_t padded = (batch + 7) / 8 * 8;
    int64_t g = std::min<int64_t>(kMaxGroup, resident_walkers<kBf16>() / padded);
    g = std::min<int64_t>(g, n_chunks / (kVThreads / 2));
    return g > 1 ? (int)g : 1;
}

template <bool kBf16>
void launch_vec(const ttv_batch* bt, const void* logits, int64_t vocab, float temperature,
                const float* draft_probs, const float* uniforms, const float* gumbel, const int32_t* tokens,
                const int32_t* next_token, const int32_t* next_sibling, int32_t max_accept,
                int32_t* accept_len, int32_t* accepted_nodes, int32_t* out_tokens, void* workspace,
                int32_t* err, hipStream_t stream) {
    const int group = walk_group<kBf16>(bt->batch, vocab / kVec);
    unsigned char* groups = (unsigned char*)workspace + buffers_bytes(bt->batch, vocab);
    int64_t grid = bt->batch;
    if (group > 1) {
        // every word of every request's record: a stale exchange number would pass for a fresh one
        const int64_t words = (int64_t)bt->batch * (kGroupRecord / 8);
        hipLaunchKernelGGL(group_clear_kernel, dim3((unsigned)((words + 255) / 256)), dim3(256), 0, stream, groups,
                           bt->batch);
        grid = (bt->batch + 7) / 8 * 8 * group;
    }
    hipLaunchKernelGGL(stochastic_walk_vec_kernel<kBf16>, dim3((unsigned)grid), dim3(kVThreads), 0, stream,
                       bt->node_offsets, bt->n_max, bt->total_nodes, logits, vocab, (double)temperature,
                       draft_probs, uniforms, gumbel, tokens, next_token, next_sibling, max_accept, accept_len,
                       accepted_nodes, out_tokens, (double*)workspace, err, bt->batch, group, groups);
}

}  // namespace

extern "C" TTV_API size_t tree_stochastic_accept_workspace_bytes(const ttv_batch* bt, int64_t vocab) {
    if (!bt || bt->batch < 0 || vocab <= 0 || vocab >= (1ll << 31)) return 0;
    const size_t bytes = buffers_bytes(bt->batch, vocab) + (size_t)bt->batch * kGroupRecord;
    return bytes > 0 ? bytes : 256;
}

extern "C" TTV_API int tree_stochastic_accept(
    const ttv_batch* bt, const void* logits, int32_t logits_dtype, int64_t vocab, float temperature,
    const float* draft_probs, const float* uniforms, const float* gumbel, const int32_t* tokens,
    const int32_t* retrieve_next_token, const int32_t* retrieve_next_sibling, int32_t max_accept,
    int32_t* accept_len, int32_t* accepted_nodes, int32_t* out_tokens, void* workspace,
    size_t workspace_bytes, int32_t* err, hipStream_t stream) {
    if (!bt || bt->batch < 0 || bt->n_max < 0 || bt->n_max > TTV_MAX_TREE_NODES ||
        bt->total_nodes < 0 || bt->total_nodes > (int64_t)bt->batch * bt->n_max)
        return TTV_EINVAL;
    if (logits_dtype != TTV_DTYPE_FP32 && logits_dtype != TTV_DTYPE_BF16) return TTV_EINVAL;
    if (vocab <= 0 || vocab >= (1ll << 31) || max_accept < 1 || max_accept > TTV_MAX_TREE_NODES)
        return TTV_EINVAL;
    if (!(temperature > 0.f) || !(temperature < INFINITY)) return TTV_EINVAL;
    if (bt->batch == 0) return TTV_OK;
    if (!bt->node_offsets || !logits || !draft_probs || !gumbel || !accept_len || !accepted_nodes ||
        !out_tokens || !err || !workspace)
        return TTV_EINVAL;
    if (bt->total_nodes > 0 && (!tokens || !uniforms || !retrieve_next_token || !retrieve_next_sibling))
        return TTV_EINVAL;
    if (workspace_bytes < tree_stochastic_accept_workspace_bytes(bt, vocab)) return TTV_ENOSPC;
    auto launch = [&](auto kern, int threads) {
        hipLaunchKernelGGL(kern, dim3(bt->batch), dim3(threads), 0, stream, bt->node_offsets,
                           bt->n_max, bt->total_nodes, logits, vocab, (double)temperature,
                           draft_probs, uniforms, gumbel, tokens, retrieve_next_token,
                           retrieve_next_sibling, max_accept, accept_len, accepted_nodes,
                           out_tokens, (double*)workspace, err);
    };
    if (vocab % kVec == 0) {
        auto vec = logits_dtype == TTV_DTYPE_BF16 ? launch_vec<true> : launch_vec<false>;
        vec(bt, logits, vocab, temperature, draft_probs, uniforms, gumbel, tokens, retrieve_next_token,
            retrieve_next_sibling, max_accept, accept_len, accepted_nodes, out_tokens, workspace, err, stream);
    } else {
        if (logits_dtype == TTV_DTYPE_BF16) launch(stochastic_walk_kernel<true>, kThreads);
        else launch(stochastic_walk_kernel<false>, kThreads);
    }
    return hipGetLastError() == hipSuccess ? TTV_OK : TTV_EHIP;
}

TTV_DEBUG_TU(stochastic)
