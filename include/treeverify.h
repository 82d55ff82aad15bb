/*
 * treeverify.h -- C ABI of the MI355X (gfx950) token-tree verification path.
 *
 * One verification round of tree speculative decoding, as four calls:
 *
 *   tree_build             parent list -> ancestor mask, depths, positions,
 *                          retrieve / next-token / next-sibling indices
 *   tree_attention_verify  one attention layer over committed KV + ancestors
 *   tree_greedy_accept     vocab argmax per node + greedy walk from the root
 *   tree_kv_commit         move accepted K/V into place, release the rest
 *
 * and two further acceptance rules over the same tree metadata:
 *
 *   tree_sample_accept     the walk with temperature-sampled choices
 *   tree_stochastic_accept the stochastic min(1, p/q) per-edge walk
 *
 * the dense mask forms for interop (tree_expand_mask, tree_pack_mask), and
 * the draft-tree construction that feeds tree_build: DDTree's best-first
 * top-B tree (tree_ddtree_build), SpecInfer's prefix merge
 * (tree_merge_sequences) and EAGLE's layer-by-layer growth with a global
 * rerank (tree_eagle_grow).
 *
 * Pages that define the operations (cited by title and section):
 *   [GLOSSARY] "Beam Search、约束解码与 Tree/Self Speculation"
 *              (llm-glossary.tokens-kit.com, decoding extensions): sections
 *              "Tree/Self Speculation", "Packed tree attention", the
 *              packed-vs-branch experiment and the verify_tree experiment.
 *   [ESSAY]    "投机解码的树状注意力验证" (wiblog.cn): custom attention mask;
 *              KV cache and batching constraints.
 *   [ATLAS]    "02 · Token Tree 与 Tree Attention" (llm-infra-atlas): §2 token
 *              tree, §3 mask rules and build_tree_kernel_efficient I/O, §4
 *              verify flow and KV release.
 *   [DDTREE]   "Accelerating Speculative Decoding with Block Diffusion Draft
 *              Trees" notes: §6 worked example, §7 tree attention and walk.
 *   [DECODING] "解码：采样、束搜索和推测性解码": "Gumbel Max技巧".
 *
 * Conventions shared by every call
 * --------------------------------
 * - Every pointer inside a call is a DEVICE pointer unless stated otherwise;
 *   the ttv_batch / ttv_kv_cache structs themselves live in host memory and
 *   are read during the call only.
 * - Requests: B requests; request b owns nodes node_offsets[b] ..
 *   node_offsets[b+1]-1 of every per-node array (T = node_offsets[B] nodes in
 *   all).  Node indices inside a request are local (0 .. N_b-1).
 * - Trees are packed in topological order: parent[i] is -1 (the node hangs off
 *   the committed context) or a local index < i ([GLOSSARY] "Packed tree
 *   attention"; [ESSAY] mask section: level order or depth-first order).
 * - Logits rows: request b owns rows node_offsets[b] + b ... (N_b + 1 rows);
 *   its row 0 is the target's prediction at the last committed token (the
 *   walk's root) and row 1 + i the prediction after node i.
 * - bf16 is the upper half of an IEEE float32 (uint16 storage).
 * - Ownership: the caller allocates every buffer, including workspaces.  The
 *   library allocates nothing, frees nothing and keeps no pointer once the
 *   call returns.  The only state it keeps between calls is per device and
 *   read-only after the first call there: the compute-unit count and which
 *   kernels already have their shared-memory limit raised.  Calls are
 *   asynchronous on the given stream, reentrant and thread-safe.
 * - Host-level errors: the return value is TTV_OK, or TTV_EINVAL (a null
 *   pointer, a size out of range, an unsupported head_dim / head ratio /
 *   dtype / layout; nothing is launched), TTV_ENOSPC (workspace too small;
 *   nothing launched) or TTV_EHIP (a launch failed).
 * - Device-level errors: err[B] (int32, device).  tree_build WRITES err[b];
 *   the later calls OR bits into it.  A flagged request's outputs are
 *   undefined; the other requests are unaffected.  The caller reads err
 *   after its single synchronisation.
 */
#ifndef TREEVERIFY_H
#define TREEVERIFY_H

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

#define TTV_API __attribute__((visibility("default")))

/* Host return codes. */
#define TTV_OK      0
#define TTV_EINVAL -1
#define TTV_EHIP   -2
#define TTV_ENOSPC -3

/* Device error bits in err[b]. */
#define TTV_ERR_BAD_PARENT      1   /* a parent outside [-1, i-1] */
#define TTV_ERR_TOO_MANY_NODES  2   /* N_b > n_max, or node_offsets not non-decreasing */
#define TTV_ERR_CAPACITY        4   /* ctx_b + N_b beyond the cache (capacity / mapped blocks) */
#define TTV_ERR_BLOCK_TABLE     8   /* a needed block-table entry is -1 or >= num_blocks */
#define TTV_ERR_ACCEPT          16  /* the walk would exceed max_accept, or commit got a bad path */
#define TTV_ERR_BAD_LENGTH      32  /* ctx_lens[b] < 0 */
#define TTV_ERR_BAD_MASK        64  /* tree_pack_mask: a dense row the attention cannot run */
#define TTV_ERR_SYNC            128 /* tree_stochastic_accept: a request's workgroups did not
                                       all run at once (another stream held the device); its
                                       outputs are undefined */

/* Limits. */
#define TTV_MAX_TREE_NODES 1024     /* N_b <= 1024, so mask rows need <= 32 words */
#define TTV_BLOCK_SIZE     16       /* paged cache block size (tokens) */

/* Logits dtypes. */
#define TTV_DTYPE_FP32 0
#define TTV_DTYPE_BF16 1

/* Dense mask modes (tree_expand_mask / tree_pack_mask). */
#define TTV_MASK_QLEN_ONLY 0        /* one byte per tree column */
#define TTV_MASK_FULL      1        /* one byte per column of context + tree */

/* KV cache layouts. */
#define TTV_KV_CONTIGUOUS 0         /* k, v: bf16 [B, n_kv_heads, capacity, head_dim] */
#define TTV_KV_PAGED      1         /* k, v: bf16 [num_blocks, n_kv_heads, block_size, head_dim] */

typedef struct ttv_batch {
    int32_t batch;                  /* B >= 0 */
    int32_t n_max;                  /* host bound on N_b, 0 .. TTV_MAX_TREE_NODES */
    int64_t total_nodes;            /* T = node_offsets[B] (host copy) */
    const int32_t* node_offsets;    /* device int32 [B+1], node_offsets[0] = 0, non-decreasing */
    const int32_t* ctx_lens;        /* device int32 [B], committed tokens per request */
} ttv_batch;

typedef struct ttv_kv_cache {
    void* k;                        /* device bf16, layout below */
    void* v;                        /* device bf16, same layout as k */
    int32_t layout;                 /* TTV_KV_CONTIGUOUS or TTV_KV_PAGED */
    int32_t n_kv_heads;             /* Hkv >= 1 */
    int32_t head_dim;               /* D: 64 or 128 */
    int32_t capacity;               /* contiguous: slots per request (>= max ctx_b + N_b) */
    int32_t* block_table;           /* paged: device int32 [B, max_blocks]; logical block j of
                                       request b is physical block block_table[b*max_blocks + j];
                                       -1 = unmapped.  tree_kv_commit writes -1 into released
                                       entries. */
    int32_t max_blocks;             /* paged: columns of block_table */
    int32_t block_size;             /* paged: must be TTV_BLOCK_SIZE */
    int32_t num_blocks;             /* paged: physical blocks in the pool */
} ttv_kv_cache;

/*
 * Debug builds.  libtreeverify_debug.so is this library compiled with
 * TTV_DEBUG defined: its kernels check the bounds of their data-dependent
 * memory accesses.  A failed check counts, records the first failing site,
 * and skips (or redirects to a valid address) the access it guards; no
 * kernel traps.  The sites:
 */
#define TTV_SITE_BUILD_NODE     1   /* tree_build: an output row past total_nodes */
#define TTV_SITE_PREP_NODE      2   /* attention prep: a node row past total_nodes */
#define TTV_SITE_PREP_CACHE     3   /* attention prep: a tentative K/V row outside the cache */
#define TTV_SITE_PLAN           4   /* attention plan: an item, partial or combine slot past its region */
#define TTV_SITE_MAIN_CACHE     5   /* attention main: a K/V tile row outside the cache */
#define TTV_SITE_MAIN_OUT       6   /* attention main: an output or partial row past its buffer */
#define TTV_SITE_COMBINE        7   /* attention combine: a partial slot or output row past its buffer */
#define TTV_SITE_ACCEPT_KEY     8   /* argmax: a row or chunk key past the workspace */
#define TTV_SITE_WALK           9   /* greedy / sampled walk: a node or row index out of range */
#define TTV_SITE_COMMIT         10  /* commit: a source or destination row outside the cache */
#define TTV_SITE_STOCHASTIC     11  /* stochastic walk: a token or row out of range */
#define TTV_SITE_DDTREE         12  /* DDTree build: a frontier slot, node or candidate out of range */
#define TTV_SITE_MASK           13  /* dense masks: a row or column out of range */
#define TTV_SITE_MERGE          14  /* SpecInfer merge / EAGLE growth: a node past its row */

/*
 * ttv_debug_report -- the debug build's failed-check count (summed over the
 * library's kernels) and the first failing site (0 if none), for the current
 * device; reset != 0 clears them.  Synchronous: call it after synchronising
 * the streams the checked calls ran on.  A release build returns TTV_EINVAL
 * and reports 0 / 0.
 */
TTV_API int ttv_debug_report(uint32_t* violations, int32_t* first_site, int32_t reset);

/* Library version (major*10000 + minor*100 + patch). */
TTV_API int32_t ttv_version(void);

/* Short description of a TTV_* return code (static string). */
TTV_API const char* ttv_status_string(int32_t status);

/*
 * tree_build -- flatten each request's draft tree ([GLOSSARY] "Packed tree
 * attention" node table; [ATLAS] §3 build_tree_kernel_efficient outputs).
 *
 * in : parents      int32 [T]   local parent of every node (-1 = off the context)
 * out: mask         uint32 [T, mask_words]; bit (j % 32) of word (j / 32) of
 *                   node i's row is set iff local node j is i or an ancestor
 *                   of i (ancestor-only visibility, self included).  The
 *                   committed context is always visible and not stored
 *                   (QLEN-only form).  Unused bits are 0.
 *                   mask_words >= ceil(n_max / 32).
 *      depth        int32 [T]   0 for a node hanging off the context
 *      positions    int32 [T]   ctx_b + depth: siblings share a position, the
 *                               packed index is never the position
 *                               ([ATLAS] §3: depths [0,1,1,2], prompt 7 ->
 *                               [7,8,8,9])
 *      retrieve_index        int32 [T]  global logits row of node i:
 *                                       node_offsets[b] + b + 1 + i
 *      retrieve_next_token   int32 [T]  first child of node i (smallest local j
 *                                       with parent j == i), else -1
 *      retrieve_next_sibling int32 [T]  next child of i's parent after i, else -1
 *      err          int32 [B]   written: TTV_ERR_BAD_PARENT, _TOO_MANY_NODES,
 *                               _BAD_LENGTH
 */
TTV_API int tree_build(const ttv_batch* bt, const int32_t* parents,
                       uint32_t* mask, int32_t mask_words,
                       int32_t* depth, int32_t* positions, int32_t* retrieve_index,
                       int32_t* retrieve_next_token, int32_t* retrieve_next_sibling,
                       int32_t* err, hipStream_t stream);

/*
 * Workspace bytes tree_attention_verify needs for this batch and cache (host
 * call, no device access).  Depends only on the host fields of bt and cache
 * and on n_heads.  Returns 0 for invalid arguments.
 */
TTV_API size_t tree_attention_workspace_bytes(const ttv_batch* bt, const ttv_kv_cache* cache,
                                              int32_t n_heads);

/*
 * tree_attention_verify -- one attention layer of the target's verify pass
 * ([GLOSSARY] "Packed tree attention" and the packed-vs-branch experiment;
 * [ATLAS] §3; [DDTREE] §7.1).
 *
 * For request b, node i, query head h (KV head h / (n_heads / n_kv_heads)):
 *   q' = RoPE(q[i,h], positions[i]), k'_j = RoPE(k_new[j], positions[j]),
 *   interleaved pairs (x_2m, x_2m+1), inv_freq_m = rope_base^(-2m/D),
 *   (x0 cos - x1 sin, x1 cos + x0 sin);
 *   keys = committed K[0 .. ctx_b-1] (already rotated in the cache) followed
 *   by k'_j for every j with mask bit j of row i set; values likewise (V is
 *   not rotated);  out[i,h] = softmax(q'.keys * scale) . values, with the
 *   softmax max and sum in fp32.
 * Side effect: k'_j (bf16) and v_new[j] are written into slots ctx_b + j of
 * the cache (the tentative region, [ESSAY] KV cache section).
 *
 * in : q       bf16 [T, n_heads, D];  k_new, v_new  bf16 [T, n_kv_heads, D]
 *      mask, mask_words, positions  as produced by tree_build
 *      cache   ctx_b + N_b <= capacity (contiguous) or every logical block
 *              < ceil((ctx_b + N_b) / 16) mapped (paged); else err bit 4 / 8
 *      rope_base > 0; softmax_scale 0 means 1/sqrt(D)
 * out: out     bf16 [T, n_heads, D]
 *      workspace  device, >= tree_attention_workspace_bytes(), 256-byte aligned
 *      err     OR-ed: TTV_ERR_CAPACITY, TTV_ERR_BLOCK_TABLE, _TOO_MANY_NODES.
 *              Should the device-side work plan ever exceed the workspace's
 *              bounds, nothing is computed and every request gets
 *              TTV_ERR_CAPACITY.
 * Supported: D in {64, 128}; n_heads % n_kv_heads == 0 with at most 64 query
 * heads per KV head; n_max <= 1024 for every head ratio; mask_words in
 * [ceil(n_max / 32), 32]; B <= 4096.  Anything else returns TTV_EINVAL
 * before any launch, so a rejected call has no device-side effect.
 */
TTV_API int tree_attention_verify(const ttv_batch* bt, const void* q, const void* k_new,
                                  const void* v_new, const uint32_t* mask, int32_t mask_words,
                                  const int32_t* positions, const ttv_kv_cache* cache,
                                  int32_t n_heads, float rope_base, float softmax_scale,
                                  void* out, void* workspace, size_t workspace_bytes,
                                  int32_t* err, hipStream_t stream);

/* Workspace bytes tree_greedy_accept needs (host call).  0 for invalid arguments. */
TTV_API size_t tree_greedy_accept_workspace_bytes(const ttv_batch* bt, int64_t vocab);

/*
 * tree_greedy_accept -- greedy verification walk ([GLOSSARY] verify_tree
 * experiment; [ATLAS] §4; [DDTREE] §7.2).
 *
 * For each request: choice[r] = argmax_v logits[row r, v] (ties to the lowest
 * v; -0.0 equals +0.0; inputs must be finite), for its N_b + 1 rows.  Then,
 * from the root (row 0), take the lowest-index child whose token equals the
 * current choice (children of the root are the nodes with parent -1, reached
 * from node 0 through retrieve_next_sibling; children of node j from
 * retrieve_next_token[j]); repeat with that child's row; stop when no child
 * matches.  The last choice is the bonus / correction token.
 *
 * in : logits   fp32 or bf16 [T + B, vocab] (row-major, row stride = vocab)
 *      tokens   int32 [T];  retrieve_next_token, retrieve_next_sibling from tree_build
 *      max_accept >= 1: capacity of accepted_nodes rows
 * out: accept_len     int32 [B]                  a_b accepted nodes
 *      accepted_nodes int32 [B, max_accept]      local node ids at depths 0..a_b-1
 *                                                (entries >= a_b set to -1)
 *      out_tokens     int32 [B, max_accept + 1]  accepted tokens then the bonus
 *                                                (entries > a_b set to -1)
 *      row_argmax     int32 [T + B] or NULL      choice of every logits row
 *      workspace      device, >= tree_greedy_accept_workspace_bytes()
 *      err            OR-ed: TTV_ERR_ACCEPT if a further match exists at max_accept
 */
TTV_API int tree_greedy_accept(const ttv_batch* bt, const void* logits, int32_t logits_dtype,
                               int64_t vocab, const int32_t* tokens,
                               const int32_t* retrieve_next_token,
                               const int32_t* retrieve_next_sibling, int32_t max_accept,
                               int32_t* accept_len, int32_t* accepted_nodes, int32_t* out_tokens,
                               int32_t* row_argmax, void* workspace, size_t workspace_bytes,
                               int32_t* err, hipStream_t stream);

/*
 * tree_expand_mask -- the bit-packed mask rows in one of the two dense forms
 * ([ATLAS] §3: build_tree_kernel_efficient emits FULL_MASK, QLEN_ONLY or the
 * bit-packed form; [GLOSSARY] packed-vs-branch experiment: tree_mask
 * [N, prefix + N] with the prefix always visible), for callers whose
 * attention takes a dense mask.
 *
 * in : mask, mask_words     bit-packed rows as tree_build writes them
 *      mode                 TTV_MASK_QLEN_ONLY: byte j of node i's row = bit j;
 *                           TTV_MASK_FULL: bytes 0 .. ctx_b - 1 = 1, byte
 *                           ctx_b + j = bit j
 *      row_stride           bytes per dense row, >= n_max (QLEN_ONLY) and
 *                           >= ctx_b + N_b for every request (FULL)
 * out: dense  uint8 [T, row_stride]; bytes past the row's columns are 0
 *      err    OR-ed: TTV_ERR_CAPACITY (FULL row longer than row_stride; the
 *             request's rows are not written), _TOO_MANY_NODES
 */
TTV_API int tree_expand_mask(const ttv_batch* bt, const uint32_t* mask, int32_t mask_words,
                             int32_t mode, uint8_t* dense, int64_t row_stride, int32_t* err,
                             hipStream_t stream);

/*
 * tree_pack_mask -- a caller's dense mask (either mode, nonzero byte =
 * visible) packed into the bit-packed rows tree_attention_verify reads.
 * A request is refused with TTV_ERR_BAD_MASK (its packed rows undefined)
 * when a row is not a tree mask the attention can run: a FULL row with a
 * context column zero, a nonzero byte in the column of a later node or past
 * the tree, or the node's own column zero.
 *
 * in : dense uint8 [T, row_stride]; mode; row_stride as in tree_expand_mask
 * out: mask uint32 [T, mask_words], mask_words in [ceil(n_max / 32), 32]
 *      err  OR-ed: TTV_ERR_BAD_MASK, _CAPACITY, _TOO_MANY_NODES
 */
TTV_API int tree_pack_mask(const ttv_batch* bt, const uint8_t* dense, int64_t row_stride,
                           int32_t mode, uint32_t* mask, int32_t mask_words, int32_t* err,
                           hipStream_t stream);

/* Workspace bytes tree_ddtree_build needs (host call); 0 for invalid sizes. */
TTV_API size_t tree_ddtree_workspace_bytes(int32_t requests, int32_t depths, int64_t vocab,
                                           int32_t budget);

/*
 * tree_ddtree_build -- DDTree's draft tree, the step before tree_build
 * ([DDTREE] §4.2: the top-B prefixes of a factorised draft are the optimal,
 * prefix-closed tree; §4.3 Lemma 1: each depth's top-min(B, V) tokens
 * suffice; §5 Algorithm 1: a best-first heap over rank tuples, popping a
 * prefix and pushing its next sibling and its first child).
 *
 * Per request and depth d: the top K = min(budget, vocab) tokens by logit
 * (descending, then token id ascending), log q = z - lse over those K (lse =
 * z_1 + log(sum_r exp(z_r - z_1)), summed in rank order, float64).  Then
 * Algorithm 1 with float64 scores (a sibling's score = parent entry's score -
 * log q(rank) + log q(rank + 1), a child's = score + log q(rank 1 of the next
 * depth)); equal scores pop in increasing rank-tuple order, a tuple before
 * its extensions.  Node i is the i-th popped prefix.
 *
 * in : draft_logits  float32 [requests, depths, vocab] (finite)
 *      depths in [1, 20]; budget in [1, 1024]; requests <= 65535
 * out: parents int32 [requests, budget]   -1 at depth 1, else an earlier node
 *      tokens  int32 [requests, budget]
 *      n_nodes int32 [requests]           min(budget, number of prefixes);
 *                                         entries past it are -1
 *      workspace  device, 256-byte aligned, >= tree_ddtree_workspace_bytes()
 * The parents / tokens rows feed tree_build directly (topological order).
 */
TTV_API int tree_ddtree_build(int32_t requests, int32_t depths, int64_t vocab, int32_t budget,
                              const float* draft_logits, int32_t* parents, int32_t* tokens,
                              int32_t* n_nodes, void* workspace, size_t workspace_bytes,
                              hipStream_t stream);

/*
 * tree_merge_sequences -- SpecInfer's tree: the distinct prefixes of each
 * request's independent draft sequences ([ATLAS] §3: SpecInfer merges
 * independent drafts along common prefixes, bottom-up; [GLOSSARY] packed
 * node table: branches [4,5,6], [4,7,8], [9,0,1] become 8 unique nodes,
 * tokens [4,9,5,7,0,6,8,1], parents [-1,-1,0,0,1,2,3,4]).
 *
 * A sequence ends at its first negative entry.  Nodes are numbered level by
 * level (depth 0 first), within a level in the order the sequences, by
 * index, first reach them, so the output is topological (it feeds
 * tree_build).
 *
 * in : seqs int32 [requests, n_seqs, seq_len]; n_seqs <= 1024;
 *      seq_len <= 1024; max_nodes <= 1024 (row length of the outputs)
 * out: parents, tokens int32 [requests, max_nodes] (-1 past n_nodes)
 *      n_nodes int32 [requests]
 *      err     int32 [requests] OR-ed: TTV_ERR_TOO_MANY_NODES when the
 *              distinct prefixes exceed max_nodes (n_nodes = 0, rows undefined)
 */
TTV_API int tree_merge_sequences(int32_t requests, int32_t n_seqs, int32_t seq_len,
                                 const int32_t* seqs, int32_t max_nodes, int32_t* parents,
                                 int32_t* tokens, int32_t* n_nodes, int32_t* err,
                                 hipStream_t stream);

/*
 * tree_eagle_grow -- EAGLE's dynamic tree ([ATLAS] §3: grown layer by layer,
 * each step expanding the current layer's top-k nodes by top-k children;
 * §5: a node scores its prefix survival probability, the product of the
 * draft confidences on its path, and the N_tree most promising nodes are
 * kept).
 *
 * Per request: layer 0 is the k candidates (root_tokens, root_conf); for
 * each further layer l the k best nodes of layer l - 1, by (score
 * descending, creation index ascending), are expanded, the j-th of them by
 * the drafter's row j of k children (child_tokens / child_conf [l - 1][j]);
 * a child's score is its parent's times its confidence (float64).  The
 * budget best of all created nodes in the same order (prefix-closed: a
 * parent precedes its children) are kept and numbered in creation order
 * (topological: the rows feed tree_build).
 *
 * in : root_tokens int32 [requests, k], root_conf float32 [requests, k]
 *      child_tokens int32 / child_conf float32 [requests, layers - 1, k, k]
 *      k in [1, 16]; layers in [1, 16]; budget in [1, 1024]
 * out: parents, tokens int32 [requests, budget] (-1 past n_nodes);
 *      n_nodes int32 [requests] = min(budget, k + (layers - 1) k^2)
 */
TTV_API int tree_eagle_grow(int32_t requests, int32_t k, int32_t layers, const int32_t* root_tokens,
                            const float* root_conf, const int32_t* child_tokens,
                            const float* child_conf, int32_t budget, int32_t* parents,
                            int32_t* tokens, int32_t* n_nodes, hipStream_t stream);

/*
 * tree_sample_accept -- the verifier walk with temperature sampling instead of
 * greedy choices ([DDTREE] §7.2: each step picks a token by the target's own
 * decoding rule, greedy or temperature sampling, and follows the drafted
 * child carrying it; §7.3: the result is distributed as plain autoregressive
 * sampling from the target, so the walk is lossless; [DECODING] "Gumbel Max
 * 技巧": a sample of softmax(h) is argmax_i (h_i + g_i) with precomputed
 * Gumbel noise g).
 *
 * For every logits row: choice = argmax_v fl32(fl32(x_v * fl32(1 / T)) + g_v),
 * float32 throughout with one rounding per operation (no fused multiply-add),
 * lowest v on ties, -0.0 equal to +0.0; then exactly tree_greedy_accept's walk
 * with these choices.  Same outputs and device error bits as
 * tree_greedy_accept; row_choice (nullable) gets every row's choice.
 *
 * in : temperature  finite, > 0 (1 / T must be finite in float32)
 *      gumbel       float32 [T + B, vocab], row-major like the logits: the
 *                   caller's Gumbel(0, 1) draws, one per logit
 *      workspace    >= tree_greedy_accept_workspace_bytes(bt, vocab)
 */
TTV_API int tree_sample_accept(const ttv_batch* bt, const void* logits, int32_t logits_dtype,
                               int64_t vocab, float temperature, const float* gumbel,
                               const int32_t* tokens, const int32_t* retrieve_next_token,
                               const int32_t* retrieve_next_sibling, int32_t max_accept,
                               int32_t* accept_len, int32_t* accepted_nodes, int32_t* out_tokens,
                               int32_t* row_choice, void* workspace, size_t workspace_bytes,
                               int32_t* err, hipStream_t stream);

/* Workspace bytes tree_stochastic_accept needs (host call): fp64 [B, 2, vocab],
 * then 1024 bytes per request for the reductions across the workgroups that
 * share a request (padded to 256 bytes between the two). */
TTV_API size_t tree_stochastic_accept_workspace_bytes(const ttv_batch* bt, int64_t vocab);

/*
 * tree_stochastic_accept -- the stochastic per-edge walk ([ATLAS] §4: from the
 * root, each child of the current node is accepted or rejected by the
 * min(1, p/q) rule; an accepted child becomes the current node; when every
 * child is rejected a correction token is sampled at the current node; at a
 * leaf the bonus token is sampled from the leaf's p).
 *
 * Per request, in float64: p_r = softmax(x_r / T) for a visited logits row
 * r; the target side starts as p_r; the current node's children are tried in
 * increasing index order: child j (token t) is accepted iff
 * u_j * q_r(t) < side(t); a rejection replaces the side by
 * max(0, side - q_r) / sum(max(0, side - q_r)) (kept as it was if that sum
 * is 0).  When no child is accepted the last token is
 * argmax_v (log side_v + g_r,v) over side_v > 0 (lowest v on ties): the
 * correction, or the bonus at a leaf.
 *
 * in : logits        fp32 or bf16 [T + B, vocab], rows as in tree_greedy_accept
 *      temperature   finite, > 0
 *      draft_probs   float32 [T + B, vocab]: row r is the draft distribution
 *                    the children of row r's node were proposed from
 *      uniforms      float32 [T]: node j's uniform draw in [0, 1)
 *      gumbel        float32 [T + B, vocab]: Gumbel(0, 1) noise per logit
 *      tokens, retrieve_next_token, retrieve_next_sibling, max_accept as in
 *      tree_greedy_accept
 * out: accept_len, accepted_nodes, out_tokens as in tree_greedy_accept (the
 *      last token is the correction / bonus; -1 for a flagged request)
 *      workspace     >= tree_stochastic_accept_workspace_bytes(bt, vocab)
 *      err           OR-ed: TTV_ERR_ACCEPT if an acceptance would exceed
 *                    max_accept; TTV_ERR_TOO_MANY_NODES for bad offsets;
 *                    TTV_ERR_SYNC if the workgroups that share a request
 *                    (vocab a multiple of 8: up to 16 per request, as many as
 *                    the device holds at once) waited over ~0.3 s for one
 *                    another, which work on another stream can cause
 */
TTV_API int tree_stochastic_accept(const ttv_batch* bt, const void* logits, int32_t logits_dtype,
                                   int64_t vocab, float temperature, const float* draft_probs,
                                   const float* uniforms, const float* gumbel,
                                   const int32_t* tokens, const int32_t* retrieve_next_token,
                                   const int32_t* retrieve_next_sibling, int32_t max_accept,
                                   int32_t* accept_len, int32_t* accepted_nodes,
                                   int32_t* out_tokens, void* workspace, size_t workspace_bytes,
                                   int32_t* err, hipStream_t stream);

/*
 * tree_greedy_accept_noalloc -- tree_greedy_accept for callers that cannot
 * allocate device memory (code under HIP graph capture, tight serving loops,
 * harnesses that forbid hipMalloc).  Same arguments, results and device error
 * bits as tree_greedy_accept, without the workspace: the argmax keys go to a
 * static 4 MiB scratch array the library holds on each device it runs on
 * until the process ends.  The call allocates and frees nothing.
 *
 * Limit: tree_greedy_accept_workspace_bytes(bt, vocab) <= 4 MiB, else
 * TTV_ENOSPC before any device call (every workload of up to 14144 logits
 * rows of 32000 or 4100 rows of 151936 needs well under 1 MiB).
 * Concurrency: every call on one GPU shares that GPU's scratch, so calls that
 * overlap on one GPU (different streams or host threads without ordering)
 * race and give undefined results; calls ordered on one stream are safe.
 * Nothing in the scratch needs clearing between calls: each call writes
 * every key its walk reads.
 */
TTV_API int tree_greedy_accept_noalloc(const ttv_batch* bt, const void* logits,
                                       int32_t logits_dtype, int64_t vocab,
                                       const int32_t* tokens,
                                       const int32_t* retrieve_next_token,
                                       const int32_t* retrieve_next_sibling,
                                       int32_t max_accept, int32_t* accept_len,
                                       int32_t* accepted_nodes, int32_t* out_tokens,
                                       int32_t* row_argmax, int32_t* err, hipStream_t stream);

/*
 * tree_kv_commit -- commit the accepted path and roll back the rest
 * ([GLOSSARY] "Tree/Self Speculation": cache [10,11] + accepted [4,7] ->
 * [10,11,4,7]; [ESSAY] KV cache section; [ATLAS] §4 after acceptance).
 *
 * For each request: the accepted node at depth d (local id i_d) moves from
 * slot ctx_b + i_d to slot ctx_b + d, K and V, every KV head, bit-exact,
 * reading the values the slots held before the call (in-place safe).  The
 * bonus token has no KV yet and is not committed.  new_lens[b] = ctx_b + a_b.
 * Contiguous: slots >= new_len become free (contents undefined).
 * Paged: logical blocks j in [ceil(new_len/16), ceil((ctx_b + N_b)/16)) are
 * released: their physical ids go to released_blocks[b*max_blocks + k] in
 * logical order, num_released[b] is set, and block_table entries become -1.
 *
 * Any n_kv_heads >= 1 and head_dim in {64, 128}: a request's moves run in
 * rounds of 2048 sixteen-byte pieces until every piece has moved.
 *
 * in : accept_len [B], accepted_nodes [B, max_accept] from tree_greedy_accept
 * out: new_lens int32 [B]; released_blocks int32 [B, max_blocks] and
 *      num_released int32 [B] (paged only; may be NULL for contiguous)
 *      err  OR-ed: TTV_ERR_ACCEPT (accept_len outside [0, min(N_b, max_accept)],
 *           or the ids not strictly increasing, an id i_d below its depth d,
 *           or an id >= N_b), _CAPACITY, _BLOCK_TABLE.  The ids are not
 *           checked against the tree's parent links (tree_greedy_accept
 *           produces a root-down path).  A flagged request is left untouched.
 */
TTV_API int tree_kv_commit(const ttv_batch* bt, const ttv_kv_cache* cache,
                           const int32_t* accept_len, const int32_t* accepted_nodes,
                           int32_t max_accept, int32_t* new_lens, int32_t* released_blocks,
                           int32_t* num_released, int32_t* err, hipStream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* TREEVERIFY_H */
