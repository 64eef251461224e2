/*
 * spec_verify.h -- C ABI of libspecverify.so: the target model's verification
 * step of speculative decoding on one AMD Instinct MI355X (gfx950).
 *
 * Three calls make one verify step:
 *   spec_verify_attn  attention of every request's verify tokens (a chain of
 *                     gamma_i+1 tokens or a draft tree of up to 64 nodes) over
 *                     its paged bf16 KV cache, with grouped-query heads;
 *   spec_accept       greedy acceptance: the target's argmax over the whole
 *                     vocabulary at every verify position, then the longest
 *                     matching prefix (chain) or deepest accepted root path (tree);
 *   kv_compact        moves the accepted path's K/V into consecutive slots of
 *                     the request's cache, in place, for every layer.
 * Further calls, each described where it is declared: spec_accept_compact
 * (acceptance and compaction in one launch), the chunked-verification calls
 * (spec_chunk_start, spec_verify_attn_chunk_plan/_run, spec_accept_chunk),
 * stochastic acceptance (spec_accept_stochastic for chains,
 * spec_accept_stochastic_tree for draft trees), the verify-budget scheduler
 * (spec_verify_budget, host memory), and spec_verify_attn_noalloc.
 *
 * Sources (page titles; sections as the pages name them):
 *   SwiftSpec (ASPLOS 2026), "Fused Latency-Optimized Kernels": padding-free
 *     attention that verifies all gamma+1 draft tokens at once, and a fused
 *     "return verification result + KV update" operation whose result is a
 *     short message to the drafter.
 *   SwiftSpec, "Tree-Aware KV Cache Management": each tree node owns its KV
 *     prefix (its root path); only the accepted path's KV is kept.
 *   DSpark, glossary "Speculative Decoding": the longest matching prefix of
 *     the draft is accepted.
 *   FASER, "Per-Request Length Adaptation": gamma differs per request.
 *   SSD, engine optimisations paragraph: PagedAttention (block tables).
 *
 * Common conventions
 *   - Every pointer is a DEVICE pointer unless stated otherwise.  bf16 data is
 *     passed as void* holding 16-bit bf16 bit patterns.  `stream` is a
 *     hipStream_t (NULL = the default stream).
 *   - Calls are stream-ordered and asynchronous; outputs are valid once the
 *     stream has reached the call.  The library keeps no state between calls,
 *     allocates no memory and retains no pointer; callers own every buffer.
 *     Two calls that share a workspace must not overlap in time.
 *   - Request i owns verify rows [cu_q[i], cu_q[i+1]) of every [T, ...] array
 *     (padding-free packing), 0 <= q_i = cu_q[i+1]-cu_q[i] <= 64.  Row 0 of a
 *     request is the root (the last committed token); a chain's row j is the
 *     j-th draft token; a tree's rows are its nodes with tree_parent[o+0] = -1
 *     and 0 <= tree_parent[o+j] < j (local indices).
 *   - The K and V caches of one layer are [num_pages][num_kv_heads][page_size]
 *     [head_dim] bf16 (token-major pages, PagedAttention's layout).  The calls
 *     named *_vt take the V cache with every (page, head) block stored
 *     transposed instead, [num_pages][num_kv_heads][head_dim][page_size], so
 *     that the keys of one column d are contiguous: the attention's P.V
 *     product reads V by columns, and with this layout each of its operand
 *     loads is one 16-byte read with no repacking (the K cache layout is the
 *     same for both).  Request i's logical slot p is physical page
 *     block_tables[i*max_blocks_per_seq + p/page_size], slot p % page_size:
 *     K row, and V row (V column for *_vt), p % page_size of that page.
 *     The committed context occupies slots [0, L_i) (L_i = context_lens[i]) and
 *     the verify tokens' K/V, written by the caller's QKV projection, occupy
 *     slots [L_i, L_i+q_i) in row order.
 *   - Query head h reads KV head h / (num_q_heads/num_kv_heads).
 *
 * Errors
 *   Host-checkable argument errors return a nonzero sv_status before anything
 *   is enqueued.  A failed HIP launch returns SV_ERR_HIP and sv_last_error()
 *   describes it (thread-local).  Content errors that only the device can see
 *   (bad cu_q, q_i > 64, a page id outside [0, num_pages), more pages than
 *   max_blocks_per_seq, a bad parent array) never cause an out-of-bounds
 *   access: the affected request's outputs are unspecified and a bit is set
 *   in the workspace's device status word, read with the *_device_status
 *   calls.
 */
#ifndef SPEC_VERIFY_H
#define SPEC_VERIFY_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum sv_status {
    SV_OK = 0,
    SV_ERR_NULL = 1,        /* a required pointer is NULL */
    SV_ERR_SHAPE = 2,       /* a size argument is out of range or inconsistent */
    SV_ERR_UNSUPPORTED = 3, /* head_dim, page_size or head grouping not supported */
    SV_ERR_WORKSPACE = 4,   /* workspace_bytes below the *_workspace_size value */
    SV_ERR_ALIAS = 5,       /* an output overlaps an input it must not overlap */
    SV_ERR_HIP = 6          /* a HIP call failed; see sv_last_error() */
} sv_status;

#define SV_MAX_VERIFY_TOKENS 64 /* per request: gamma_i+1 or tree nodes (one 64-bit ancestor word) */
#define SV_PAGE_SIZE 16         /* tokens per KV page */

/* Device status bits (see *_device_status). */
#define SV_DEV_BAD_CU_Q 0x1u        /* cu_q not non-decreasing from 0 to total_q */
#define SV_DEV_BAD_CONTEXT 0x2u     /* context_lens[i] < 0 */
#define SV_DEV_TOO_MANY_TOKENS 0x4u /* q_i > 64 */
#define SV_DEV_BAD_PARENT 0x8u      /* tree_parent violates root=-1, 0<=parent[j]<j */
#define SV_DEV_BAD_PAGE 0x10u       /* a needed block-table entry is outside [0, num_pages) */
#define SV_DEV_TOO_MANY_PAGES 0x20u /* ceil((L_i+q_i)/page_size) > max_blocks_per_seq */
#define SV_DEV_SYNC_TIMEOUT 0x40u   /* spec_accept_compact: a bounded wait between work items ran out */
#define SV_DEV_BAD_TOKEN 0x80u      /* spec_accept_stochastic: a draft token outside [0, vocab) */

/* ------------------------------------------------------------------------- */
/* Verify attention                                                           */
/* ------------------------------------------------------------------------- */

/* Workspace bytes spec_verify_attn needs for these sizes (host function). */
size_t spec_verify_attn_workspace_size(int batch, int total_q, int num_q_heads, int num_kv_heads,
                                       int head_dim);

/*
 * out[t, h, :] = softmax_p(scale * q[t,h,:] . K[p,g,:] + M[t,p]) . V[p,g,:]
 * where for row t = cu_q[i]+j, key p of request i is visible (M = 0) iff
 * p < L_i, or p = L_i + k with k = j or k an ancestor of j (chain: k <= j);
 * otherwise M = -inf.  Keys are the L_i+q_i slots of the request's cache.
 *
 *   q            bf16 [total_q, num_q_heads, head_dim]
 *   k_cache      bf16 [num_pages, num_kv_heads, page_size, head_dim] (one layer)
 *   v_cache      bf16 [num_pages, num_kv_heads, page_size, head_dim] (one layer);
 *                spec_verify_attn_vt: [num_pages, num_kv_heads, head_dim, page_size]
 *   block_tables int32 [batch, max_blocks_per_seq]
 *   context_lens int32 [batch]  L_i (verify tokens excluded)
 *   cu_q         int32 [batch+1] prefix sums of q_i
 *   tree_parent  int32 [total_q] local parents, or NULL for chains
 *   out          bf16 [total_q, num_q_heads, head_dim]; must not overlap q/k/v
 *   softmax_scale  > 0, or 0 for 1/sqrt(head_dim); negative or non-finite
 *                  values return SV_ERR_SHAPE
 *   workspace    device buffer of at least spec_verify_attn_workspace_size()
 *                bytes (contents need no initialisation; overwritten)
 * Supported: head_dim 64 or 128, page_size 16, num_q_heads % num_kv_heads == 0
 * with at most 64 query heads per KV head.
 */
int spec_verify_attn(const void *q, const void *k_cache, const void *v_cache,
                     const int32_t *block_tables, int max_blocks_per_seq,
                     const int32_t *context_lens, const int32_t *cu_q, const int32_t *tree_parent,
                     void *out, int batch, int total_q, int num_q_heads, int num_kv_heads,
                     int head_dim, int page_size, int num_pages, float softmax_scale,
                     void *workspace, size_t workspace_bytes, void *stream);

/* spec_verify_attn with the V cache's pages stored transposed (see above). */
int spec_verify_attn_vt(const void *q, const void *k_cache, const void *v_cache,
                        const int32_t *block_tables, int max_blocks_per_seq,
                        const int32_t *context_lens, const int32_t *cu_q, const int32_t *tree_parent,
                        void *out, int batch, int total_q, int num_q_heads, int num_kv_heads,
                        int head_dim, int page_size, int num_pages, float softmax_scale,
                        void *workspace, size_t workspace_bytes, void *stream);

/*
 * The two halves of spec_verify_attn, for callers that verify many layers
 * with the same batch: the work decomposition (the "plan") depends only on
 * context_lens, cu_q, the head counts and the page-count limits, so one
 * spec_verify_attn_plan per verify step serves every layer's
 * spec_verify_attn_run.  spec_verify_attn == plan + run.
 *
 * spec_verify_attn_plan writes the plan into `workspace` (same size as for
 * spec_verify_attn); max_blocks_per_seq and num_pages bound the requests'
 * pages.  spec_verify_attn_run must be given the same batch metadata and
 * sizes as the plan it uses (stream-ordered after it) and must not overlap
 * another run or plan on the same workspace.  A run with metadata that
 * differs from its plan still reads only valid memory, but its outputs are
 * unspecified.  spec_verify_attn_run_vt takes transposed V pages; one plan
 * serves both layouts.
 */
int spec_verify_attn_plan(const int32_t *context_lens, const int32_t *cu_q, int max_blocks_per_seq,
                          int batch, int total_q, int num_q_heads, int num_kv_heads, int head_dim,
                          int num_pages, void *workspace, size_t workspace_bytes, void *stream);

int spec_verify_attn_run(const void *q, const void *k_cache, const void *v_cache,
                         const int32_t *block_tables, int max_blocks_per_seq,
                         const int32_t *context_lens, const int32_t *cu_q,
                         const int32_t *tree_parent, void *out, int batch, int total_q,
                         int num_q_heads, int num_kv_heads, int head_dim, int page_size,
                         int num_pages, float softmax_scale, void *workspace,
                         size_t workspace_bytes, void *stream);

int spec_verify_attn_run_vt(const void *q, const void *k_cache, const void *v_cache,
                            const int32_t *block_tables, int max_blocks_per_seq,
                            const int32_t *context_lens, const int32_t *cu_q,
                            const int32_t *tree_parent, void *out, int batch, int total_q,
                            int num_q_heads, int num_kv_heads, int head_dim, int page_size,
                            int num_pages, float softmax_scale, void *workspace,
                            size_t workspace_bytes, void *stream);

/* Waits for `stream`, then stores the device status bits of the last
 * spec_verify_attn (plan and runs) that used `workspace` into *flags (host
 * pointer). */
int spec_verify_attn_device_status(const void *workspace, uint32_t *flags, void *stream);

/*
 * Diagnostic: the attention kernel's phase timeline.  Only the trace build of
 * the library (libspecverify_trace.so, compiled with SV_PHASE_TRACE) records
 * one; in it, every wave of every workgroup range stores up to 2048 64-bit
 * words (shader-clock time << 8 | phase code) into a static device array of
 * the library, overwriting it on each attention launch.  Waits for the
 * device, then copies min(bytes, *total_bytes) of that array into host_dst
 * (host pointer; may be NULL with bytes = 0) and, if clear != 0, zeroes it.
 * *total_bytes (may be NULL) receives the array's size.  Layout and codes:
 * word (w * 4 + wave) * 2048 + i is event i of that wave of range w (w < 512); codes are
 * 1 range header read, 2 first unit ready, 3 round start, 4 next loads
 * issued, 5 round data in, 6 block computed, 7 unit written, 8 next unit
 * entered, 9 range done.  Errors: SV_ERR_UNSUPPORTED in the production build,
 * SV_ERR_HIP.
 */
int spec_verify_attn_phase_trace(void *host_dst, size_t bytes, int clear, size_t *total_bytes);

/*
 * For callers that cannot allocate device memory (code under stream or graph
 * capture, tight serving loops, harnesses that forbid allocation):
 * spec_verify_attn with no workspace argument.  The arguments and the result
 * are those of spec_verify_attn (token-major V pages); the workspace is a
 * static device array inside the library of SV_NOALLOC_SCRATCH_BYTES, which
 * each GPU the library runs on holds from the first call on it until the
 * process ends.  The call allocates nothing (no hipMalloc, no allocating
 * library routine).  Its first call on a device looks the array's device
 * address up once (hipGetSymbolAddress, with that device current).
 *
 *   device_status  DEVICE pointer to one uint32, or NULL: receives the call's
 *                  device status bits (as spec_verify_attn_device_status
 *                  would report them), stream-ordered.
 * Errors: those of spec_verify_attn, and SV_ERR_WORKSPACE (before anything is
 * enqueued) when these sizes need more workspace than the array holds
 * (spec_verify_attn_workspace_size() > SV_NOALLOC_SCRATCH_BYTES).
 * Every call on one GPU uses the same array: calls on one GPU must not
 * overlap in time (two streams, two host threads), or they race.  Nothing in
 * the array needs to start at any value: each call writes all it reads.
 */
#define SV_NOALLOC_SCRATCH_BYTES ((size_t)40 << 20)

int spec_verify_attn_noalloc(const void *q, const void *k_cache, const void *v_cache,
                             const int32_t *block_tables, int max_blocks_per_seq,
                             const int32_t *context_lens, const int32_t *cu_q,
                             const int32_t *tree_parent, void *out, int batch, int total_q,
                             int num_q_heads, int num_kv_heads, int head_dim, int page_size,
                             int num_pages, float softmax_scale, uint32_t *device_status,
                             void *stream);

/* ------------------------------------------------------------------------- */
/* Greedy acceptance                                                          */
/* ------------------------------------------------------------------------- */

/* Workspace bytes spec_accept needs (host function). */
size_t spec_accept_workspace_size(int batch, int total_q, int vocab);

/*
 * target_argmax[t] = lowest index of the maximum of logits[t, 0:vocab]
 *   (IEEE comparison, so -0 equals +0; logits must be finite).
 * Chain: n_i = largest k <= q_i-1 with draft_tokens[o+j] == target_argmax[o+j-1]
 *   for every 1 <= j <= k.
 * Tree: node j is accepted iff draft_tokens[o+a] == target_argmax[o+parent[a]]
 *   for every non-root node a on its root path; the accepted node of greatest
 *   depth (lowest index on ties) is chosen and n_i is its depth.
 * Outputs: accept_len[i] = n_i + 1 (bonus token counted; 0 when q_i = 0);
 *   accepted_path[o+k] = k-th node of the accepted root path for k <= n_i, -1 after;
 *   out_tokens[o+k] = target_argmax[o + accepted_path[o+k]] for k <= n_i, -1 after.
 *
 *   logits       fp32 [total_q, vocab]; row o+j is the target's prediction after row j
 *   draft_tokens int32 [total_q]; the entry at each root is ignored
 *   cu_q, tree_parent as for spec_verify_attn
 *   target_argmax int32 [total_q] out;  accept_len int32 [batch] out;
 *   accepted_path int32 [total_q] out;  out_tokens int32 [total_q] out
 */
int spec_accept(const float *logits, int vocab, const int32_t *draft_tokens, const int32_t *cu_q,
                const int32_t *tree_parent, int batch, int total_q, int32_t *target_argmax,
                int32_t *accept_len, int32_t *accepted_path, int32_t *out_tokens, void *workspace,
                size_t workspace_bytes, void *stream);

/* Waits for `stream`, then stores the device status bits of the last
 * spec_accept that used `workspace` into *flags (host pointer). */
int spec_accept_device_status(const void *workspace, uint32_t *flags, void *stream);

/* ------------------------------------------------------------------------- */
/* KV compaction                                                              */
/* ------------------------------------------------------------------------- */

/*
 * For every layer l < num_layers (cache base + l*layer_stride_elems elements),
 * request i, KV head g and k = 0..accept_len[i]-1: logical slot
 * L_i + accepted_path[o+k] is copied into logical slot L_i + k, all sources
 * being read before any destination is written.  Chains (path[k] = k) move
 * nothing.  new_context_lens[i] = L_i + accept_len[i].
 * Slots past the new length are left unchanged; the caller's page allocator
 * releases pages beyond ceil(new_len/page_size).  NOT idempotent: run once per
 * verify step.
 *
 *   k_cache, v_cache  bf16 caches in the layouts above (kv_compact_vt:
 *                     V pages transposed), modified in place
 *   context_lens      int32 [batch] L_i before the step (not modified)
 *   cu_q         int32 [batch+1] as for spec_verify_attn (total_q = cu_q[batch])
 *   accepted_path, accept_len  as produced by spec_accept
 *   new_context_lens  int32 [batch] out; must not alias context_lens.  A
 *                     request whose path or pages break the contract is left
 *                     untouched and gets new_context_lens[i] = -1.
 */
int kv_compact(void *k_cache, void *v_cache, int64_t layer_stride_elems, int num_layers,
               const int32_t *block_tables, int max_blocks_per_seq, const int32_t *context_lens,
               const int32_t *cu_q, const int32_t *accepted_path, const int32_t *accept_len,
               int32_t *new_context_lens, int batch, int total_q, int num_kv_heads, int head_dim,
               int page_size, int num_pages, void *stream);

int kv_compact_vt(void *k_cache, void *v_cache, int64_t layer_stride_elems, int num_layers,
                  const int32_t *block_tables, int max_blocks_per_seq, const int32_t *context_lens,
                  const int32_t *cu_q, const int32_t *accepted_path, const int32_t *accept_len,
                  int32_t *new_context_lens, int batch, int total_q, int num_kv_heads, int head_dim,
                  int page_size, int num_pages, void *stream);

/* ------------------------------------------------------------------------- */
/* Lossless stochastic acceptance (chains and trees)                         */
/* ------------------------------------------------------------------------- */
/*
 * DSpark, glossary "Speculative Decoding": the verification rule keeps the
 * target's distribution.  The rule is speculative sampling (rejection
 * sampling): for request i with verify rows o..o+gamma (row o = root),
 *   p_j = softmax(logits[o+j-1] / temperature), q_j = draft_probs[o+j];
 *   draft j is accepted iff u[o+j] * q_j(x_j) < p_j(x_j), x_j = draft_tokens[o+j];
 *   the walk stops at the first rejection; n = accepted drafts;
 *   y = the smallest v whose cumulative weight exceeds w[i] * (total weight),
 *   the weights being max(0, p_{n+1} - q_{n+1}) after a rejection (p_{n+1}
 *   if those have no mass) and p_{gamma+1} when every draft was accepted.
 * Outputs: accept_len[i] = n + 1; accepted_path[o+k] = k for k <= n, -1 after;
 * out_tokens[o+k] = x_{k+1} for k < n, out_tokens[o+n] = y, -1 after.  The
 * random numbers are inputs (uniform in [0, 1)), so a call is deterministic.
 * Arithmetic is fp32 (exp2 of logit*log2(e)/T): an acceptance or a draw whose
 * margin is within fp32 rounding may differ from an fp64 evaluation.
 *
 *   logits, draft_probs  fp32 [total_q, vocab] (draft_probs row o, the root, unused;
 *                        each draft row sums to 1)
 *   draft_tokens int32 [total_q]; uniform_accept fp32 [total_q]; uniform_sample fp32 [batch]
 *   temperature  > 0;  chains (trees: spec_accept_stochastic_tree below)
 *   workspace    at least spec_accept_stochastic_workspace_size() bytes (no initialisation)
 * Device status (spec_accept_stochastic_device_status): SV_DEV_BAD_CU_Q,
 * SV_DEV_BAD_TOKEN.
 */
size_t spec_accept_stochastic_workspace_size(int batch, int total_q, int vocab);

int spec_accept_stochastic(const float *logits, const float *draft_probs, int vocab,
                           float temperature, const int32_t *draft_tokens,
                           const float *uniform_accept, const float *uniform_sample,
                           const int32_t *cu_q, int batch, int total_q, int32_t *accept_len,
                           int32_t *accepted_path, int32_t *out_tokens, void *workspace,
                           size_t workspace_bytes, void *stream);

/*
 * Draft trees.  SwiftSpec ("Tree-aware KV cache management") verifies a tree of
 * draft tokens per request; DSpark's glossary asks the rule to keep the target's
 * distribution, and the pages give no rule for trees.  This call takes multi-draft
 * rejection sampling: with tree_parent as for spec_accept (parent[o] = -1,
 * 0 <= parent[o+k] < k), the walk starts at the root c = 0 with p' = p_c =
 * softmax(logits[o+c] / temperature); the children k of c are tested in index
 * order, child k accepted iff u[o+k] * q_k(x_k) < p'(x_k) (q_k = draft_probs[o+k],
 * the distribution x_k was drawn from); an accepted child becomes c (p' restarts
 * from its row); a rejection replaces p' by max(0, p' - q_k) normalised when that
 * has mass (else p' stays); when no child of c is accepted, y is drawn with w[i]
 * by inverse CDF from the last residual with mass (unnormalised), or from p_c.
 * Outputs: accept_len[i] = n + 1 (n accepted drafts); accepted_path[o+t] = node
 * index of the t-th path node (0 = root) for t <= n, -1 after; out_tokens[o+t] =
 * draft token of path node t+1 for t < n, y at t = n, -1 after.  A tree with one
 * child per node gives spec_accept_stochastic's results.  Each rejection costs one
 * pass over the vocabulary (its residual's mass), inside one workgroup per request.
 * Arguments, workspace (spec_accept_stochastic_workspace_size) and precision as for
 * spec_accept_stochastic; tree_parent int32 [total_q].  Device status: also
 * SV_DEV_BAD_PARENT (that request: accept_len 0, its path and tokens -1).
 */
int spec_accept_stochastic_tree(const float *logits, const float *draft_probs, int vocab,
                                float temperature, const int32_t *draft_tokens, const int32_t *tree_parent,
                                const float *uniform_accept, const float *uniform_sample,
                                const int32_t *cu_q, int batch, int total_q, int32_t *accept_len,
                                int32_t *accepted_path, int32_t *out_tokens, void *workspace,
                                size_t workspace_bytes, void *stream);

int spec_accept_stochastic_device_status(const void *workspace, uint32_t *flags, void *stream);

/* ------------------------------------------------------------------------- */
/* Fused acceptance + compaction                                              */
/* ------------------------------------------------------------------------- */
/*
 * SwiftSpec, "Fused Latency-Optimized Kernels": the verification result and
 * the KV update come out of one kernel.  spec_accept_compact = spec_accept
 * followed by kv_compact, in ONE launch: the argmax slices, each request's
 * walk and (for draft trees) the K/V moves are work items that workgroups
 * take in that order from a counter in the workspace; a walk starts once
 * its rows' slices are done and a move group once its request's walk is.
 * Outputs are those of spec_accept and kv_compact with the same arguments.
 *
 *   arguments    as for spec_accept (logits .. out_tokens) and kv_compact
 *                (k_cache .. num_pages); accepted_path and accept_len are
 *                both outputs here and inputs of the moves.
 *   workspace    at least spec_accept_compact_workspace_size() bytes, and
 *                ZERO-FILLED before its first use (allocate it with zeros).
 *                Every call ends by zeroing all it wrote there (apart from
 *                the status word), so one workspace, sized for the largest
 *                shape, serves calls of any (batch, total_q, vocab) in turn.
 *                Two calls on one workspace must not overlap in time.
 * Device status (spec_accept_device_status on this workspace): the bits of
 * spec_accept, plus SV_DEV_SYNC_TIMEOUT if a wait between work items gave up
 * (outputs of the affected requests are then unspecified).  A call whose
 * workspace was not zero at its start reports SV_DEV_SYNC_TIMEOUT and, if
 * its counters cannot be brought back to zero, leaves them: zero-fill the
 * workspace again before the next call.
 */
size_t spec_accept_compact_workspace_size(int batch, int total_q, int vocab);

int spec_accept_compact(const float *logits, int vocab, const int32_t *draft_tokens,
                        const int32_t *cu_q, const int32_t *tree_parent, int batch, int total_q,
                        int32_t *target_argmax, int32_t *accept_len, int32_t *accepted_path,
                        int32_t *out_tokens, void *k_cache, void *v_cache,
                        int64_t layer_stride_elems, int num_layers, const int32_t *block_tables,
                        int max_blocks_per_seq, const int32_t *context_lens,
                        int32_t *new_context_lens, int num_kv_heads, int head_dim, int page_size,
                        int num_pages, void *workspace, size_t workspace_bytes, void *stream);

/* spec_accept_compact over caches whose V pages are stored transposed. */
int spec_accept_compact_vt(const float *logits, int vocab, const int32_t *draft_tokens,
                           const int32_t *cu_q, const int32_t *tree_parent, int batch, int total_q,
                           int32_t *target_argmax, int32_t *accept_len, int32_t *accepted_path,
                           int32_t *out_tokens, void *k_cache, void *v_cache,
                           int64_t layer_stride_elems, int num_layers, const int32_t *block_tables,
                           int max_blocks_per_seq, const int32_t *context_lens,
                           int32_t *new_context_lens, int num_kv_heads, int head_dim, int page_size,
                           int num_pages, void *workspace, size_t workspace_bytes, void *stream);

/* ------------------------------------------------------------------------- */
/* Chunked verification with early pruning                                    */
/* ------------------------------------------------------------------------- */
/*
 * FASER, "Early Token Pruning": verification runs over chunks of each
 * request's verify tokens, and at every chunk boundary the tokens behind an
 * already rejected prefix are dropped, so no work is spent on them.  A verify
 * step becomes a loop that runs on the device from start to end:
 *
 *   spec_chunk_start(cu_q, ...)                -> chunk_begin, cu_chunk
 *   repeat ceil(max_i q_i / chunk_size) times (the host knows the draft lengths):
 *     (every layer) spec_verify_attn_chunk_plan / _run over the chunk's rows
 *     spec_accept_chunk(logits, ...)           -> next_begin, next_cu
 *     swap (chunk_begin, cu_chunk) with (next_begin, next_cu)
 *
 * and ends with the same accept_len / accepted_path / out_tokens as
 * spec_accept over all verify tokens (the tokens dropped are never accepted).
 * Request i's rows in a chunk are its verify tokens
 * [chunk_begin[i], chunk_begin[i] + c_i), c_i = cu_chunk[i+1] - cu_chunk[i]
 * (c_i = 0: not in this chunk).  No host call needs a chunk's row count: the
 * kernels read cu_chunk[batch] on the device, so no call waits for the
 * device and the whole loop can be captured in one graph; once every
 * request has ended, cu_chunk[batch] = 0 and the remaining calls do
 * nothing.  All arrays keep the packing of all verify tokens (total_q of
 * them): cu_q, tree_parent, draft_tokens, target_argmax, accepted_path,
 * out_tokens, and also q, out and logits, whose row cu_q[i] + j is verify
 * token j of request i; a chunk reads and writes its own rows in place.  The
 * verify tokens' K/V are in the cache from the start, as for
 * spec_verify_attn.
 */

/* First chunk: chunk_begin[i] = 0 and cu_chunk = prefix sums of
 * min(chunk_size, q_i).  chunk_begin int32 [batch], cu_chunk int32 [batch+1]
 * (outputs, must not overlap each other or cu_q). */
int spec_chunk_start(const int32_t *cu_q, int batch, int total_q, int chunk_size,
                     int32_t *chunk_begin, int32_t *cu_chunk, void *stream);

/*
 * Verify attention of one chunk's rows: verify token j = chunk_begin[i]+r of
 * request i (row cu_q[i] + j of q and out) attends, as in spec_verify_attn,
 * to slots p < L_i and p = L_i + k for k = j or k an ancestor of j (chain:
 * k <= j); rows of other tokens are neither read nor written.  The workspace
 * is sized with spec_verify_attn_workspace_size for total_q rows; the
 * plan/run contract is that of spec_verify_attn_plan and spec_verify_attn_run.
 * Device status: SV_DEV_BAD_CU_Q also covers a chunk that does not lie inside
 * its request, or cu_chunk[batch] > total_q.
 *
 *   q, out       bf16 [total_q, num_q_heads, head_dim], one row per verify token
 *   cu_q         int32 [batch+1] packing of all verify tokens, total_q of them
 *   chunk_begin  int32 [batch];  cu_chunk int32 [batch+1]
 *   tree_parent  int32 [total_q] or NULL for chains
 *   other arguments as for spec_verify_attn
 */
int spec_verify_attn_chunk_plan(const int32_t *context_lens, const int32_t *cu_q, int total_q,
                                const int32_t *chunk_begin, const int32_t *cu_chunk, int max_blocks_per_seq,
                                int batch, int num_q_heads, int num_kv_heads, int head_dim, int num_pages,
                                void *workspace, size_t workspace_bytes, void *stream);

int spec_verify_attn_chunk_run(const void *q, const void *k_cache, const void *v_cache,
                               const int32_t *block_tables, int max_blocks_per_seq,
                               const int32_t *context_lens, const int32_t *cu_q, int total_q,
                               const int32_t *chunk_begin, const int32_t *cu_chunk, const int32_t *tree_parent,
                               void *out, int batch, int num_q_heads, int num_kv_heads, int head_dim,
                               int page_size, int num_pages, float softmax_scale, void *workspace,
                               size_t workspace_bytes, void *stream);

int spec_verify_attn_chunk_run_vt(const void *q, const void *k_cache, const void *v_cache,
                                  const int32_t *block_tables, int max_blocks_per_seq,
                                  const int32_t *context_lens, const int32_t *cu_q, int total_q,
                                  const int32_t *chunk_begin, const int32_t *cu_chunk, const int32_t *tree_parent,
                                  void *out, int batch, int num_q_heads, int num_kv_heads, int head_dim,
                                  int page_size, int num_pages, float softmax_scale, void *workspace,
                                  size_t workspace_bytes, void *stream);

/* Workspace bytes spec_accept_chunk needs for any chunk of a step with
 * total_q verify tokens (host function). */
size_t spec_accept_chunk_workspace_size(int batch, int total_q, int vocab);

/*
 * Acceptance after one chunk.  target_argmax[o + j] (o = cu_q[i]) is computed
 * for the chunk's tokens from logits row o + j; the entries of earlier tokens
 * must hold what earlier chunks of the same step wrote.  With
 * e = chunk_begin[i] + c_i, the edge into node j (chain: parent j-1) is
 * decided once its parent is < e; a node is alive while no decided edge on
 * its root path mismatches.  If some node in [e, q_i) is alive, the request
 * continues: next_begin[i] = e and it gets min(chunk_size, q_i - e) rows in
 * the next chunk.  Otherwise it ends here: accept_len[i],
 * accepted_path[o..o+q_i) and out_tokens[o..o+q_i) are written exactly as
 * spec_accept would write them, and it gets 0 rows next.  Requests with
 * c_i = 0 are left unchanged.  next_cu int32 [batch+1] = prefix sums of the
 * next chunk's rows (next_cu[batch] = 0 once every request has ended).
 * next_begin / next_cu must not overlap chunk_begin / cu_chunk.  chunk_size
 * is the one given to spec_chunk_start (it bounds a chunk's rows).
 *
 *   logits       fp32 [total_q, vocab], one row per verify token (only the
 *                chunk's rows are read)
 *   draft_tokens int32 [total_q]; cu_q, tree_parent as for spec_accept
 *   workspace    at least spec_accept_chunk_workspace_size(batch, total_q, vocab) bytes
 * Device status (spec_accept_device_status): as spec_accept, plus
 * SV_DEV_BAD_CU_Q for a chunk that does not lie inside its request.
 */
int spec_accept_chunk(const float *logits, int vocab, const int32_t *draft_tokens,
                      const int32_t *cu_q, const int32_t *tree_parent, const int32_t *chunk_begin,
                      const int32_t *cu_chunk, int batch, int total_q, int chunk_size,
                      int32_t *target_argmax, int32_t *accept_len, int32_t *accepted_path,
                      int32_t *out_tokens, int32_t *next_begin, int32_t *next_cu, void *workspace,
                      size_t workspace_bytes, void *stream);

/* ------------------------------------------------------------------------- */
/* Verify-budget scheduling (host)                                            */
/* ------------------------------------------------------------------------- */
/*
 * DSpark, "Hardware-aware prefix scheduler": choose how many draft positions
 * of each request to verify so that the expected tokens emitted per second,
 * Theta = tau * SPS(B), is largest.  Request i has gamma_i = cu_draft[i+1] -
 * cu_draft[i] draft positions with conditional survival probabilities
 * c = cond_survival[cu_draft[i] .. cu_draft[i+1]) (chance that draft k is
 * accepted once drafts 1..k-1 were); S_k = c_1 * ... * c_k.  All (request,
 * position) candidates are sorted by S, largest first (equal S: earlier
 * position, then lower request), and admitted one at a time on top of the
 * batch's root rows; for B = batch + admitted rows, tau = batch (one bonus
 * token per request) + the admitted S values, and SPS(B) is the engine's
 * verify steps per second at B rows, linearly interpolated in the table
 * (sps_rows strictly increasing, > 0; sps_value >= 0) and clamped at its
 * ends.  The first batch with the largest Theta is returned:
 * verify_len[i] = drafts of request i to verify (a prefix), *batch_rows = B,
 * *theta = Theta.  All pointers are HOST pointers; nothing runs on the GPU.
 * Errors: SV_ERR_NULL, SV_ERR_SHAPE (gamma_i outside [0, 63], cu_draft[0]
 * != 0, a survival value outside [0, 1] or NaN, a bad SPS table).
 */
int spec_verify_budget(const float *cond_survival, const int32_t *cu_draft, int batch,
                       const float *sps_rows, const float *sps_value, int n_sps,
                       int32_t *verify_len, int32_t *batch_rows, double *theta);

/* ------------------------------------------------------------------------- */
/* HBM read-ceiling probe (measurement aid, not part of the verify step)      */
/* ------------------------------------------------------------------------- */

#define SV_PROBE_SINK_WORDS 131072 /* uint32 words spec_hbm_read_probe may write to sink */

/* Streams the listed K and V cache blocks with the verify-attention kernel's
 * load pattern (16-byte nontemporal loads, 1 KB per instruction, one pair of
 * blocks in flight per wave while the previous pair is consumed) and does
 * nothing else with them, so the attention's KV-stream rate can be compared
 * with what a pure read kernel reaches on the same pages of the same device.
 * chunks[c] (DEVICE, int32 [n_chunks]) names one (page, KV head) block:
 * chunk_bytes at byte offset chunks[c] * chunk_bytes of k_cache and of
 * v_cache (DEVICE) - for the cache layouts above, page * Hkv + h
 * with chunk_bytes = 16 * D * 2 (2048 or 4096).  buffer_chunks is the number
 * of blocks each cache holds; an index outside [0, buffer_chunks) reads
 * block 0 instead.  Each lane writes the XOR of the 32-bit words it read to
 * one word of sink (DEVICE, uint32 [sink_words >= SV_PROBE_SINK_WORDS]; 256
 * words per workgroup, two workgroups per compute unit up to 512, the rest
 * untouched),
 * which keeps the loads: over a zeroed sink, the XOR of all its words is the
 * XOR of every word of the listed blocks of both caches.
 * Asynchronous on `stream`; n_chunks = 0 does nothing.  Errors: SV_ERR_NULL,
 * SV_ERR_SHAPE (n_chunks < 0, buffer_chunks <= 0, sink too small),
 * SV_ERR_UNSUPPORTED (chunk_bytes not 2048 or 4096), SV_ERR_HIP. */
int spec_hbm_read_probe(const void *k_cache, const void *v_cache, const int32_t *chunks, int64_t n_chunks,
                        int chunk_bytes, int64_t buffer_chunks, uint32_t *sink, int64_t sink_words,
                        void *stream);

/* ------------------------------------------------------------------------- */
/* Diagnostics (host)                                                         */
/* ------------------------------------------------------------------------- */

/* Static description of a status code. */
const char *sv_status_string(int status);

/* Thread-local detail of the most recent failing call on this thread ("" if none). */
const char *sv_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* SPEC_VERIFY_H */
