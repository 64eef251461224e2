/*
 * oracle.c -- plain, slow CPU reference for the speculative-decoding
 * verification step.  TEST INFRASTRUCTURE ONLY: it is called by the tests,
 * by the smoke check and by the benchmark's CPU-baseline leg, never by the
 * product path.  It shares no code with the HIP library.
 *
 * Every floating-point step is done in double precision (fp64).  bf16 inputs
 * are widened exactly.  Nothing is blocked, fused or reordered beyond what
 * the definitions below state.
 *
 * Sources (page titles; sections named as on the pages):
 *  - SwiftSpec (ASPLOS 2026), "Fused Latency-Optimized Kernels": the target
 *    verifies all gamma+1 draft tokens at once with a padding-free attention
 *    kernel, and returns the verification result together with a KV update.
 *  - SwiftSpec, "Tree-Aware KV Cache Management": every draft-tree node has
 *    its own KV prefix (its root path); after verification only the accepted
 *    path's KV is kept and rejected paths are released.
 *  - DSpark, glossary entry "Speculative Decoding": the target checks the
 *    drafted prefixes in parallel and accepts the longest matching prefix.
 *  - FASER, "Per-Request Length Adaptation": each request in a batch carries
 *    its own draft length gamma_i.
 *  - FASER, "Early Token Pruning": verification over chunks of the verify
 *    tokens drops, at each chunk boundary, the tokens behind a rejected prefix.
 *  - SSD, section on integrating recent inference optimisations: the engine
 *    uses PagedAttention, i.e. a paged KV cache addressed through per-request
 *    block tables.
 *
 * Conventions (the pages leave these open; the plainest reading is taken):
 *  - Request i has q_i verify tokens packed at rows [cu_q[i], cu_q[i+1]).
 *    Token 0 is the root (last committed token); a chain has parent(j)=j-1,
 *    a tree gives parent[] with parent[0]=-1 and parent[j]<j.
 *  - The verify tokens' K/V already sit in logical slots [L_i, L_i+q_i) of
 *    the request's paged cache, in token order.  Logical slot p lives in
 *    physical page block_tables[i][p / page_size], slot p % page_size.
 *  - Cache layout: [num_pages][num_kv_heads][page_size][head_dim] (bf16).
 *  - Query head h reads KV head h / (Hq/Hkv).
 *  - Logits row cu_q[i]+j is the target's prediction after token j.
 *  - Greedy acceptance; accept_len counts the bonus token.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

#define ORACLE_OK 0
#define ORACLE_BAD_ARG 1
#define ORACLE_BAD_CONTENT 2
#define ORACLE_NO_MEMORY 3

static double bf16_to_double(uint16_t bits) {
    uint32_t u = (uint32_t)bits << 16;
    float f;
    memcpy(&f, &u, sizeof f);
    return (double)f;
}

/* parent of verify token j of a request (chain when tree_parent is NULL) */
static int parent_of(const int32_t *tree_parent, int o, int j) {
    if (tree_parent == NULL) return j - 1;
    return tree_parent[o + j];
}

/* Validates one request's parent array: root -1, every other parent earlier. */
static int check_parents(const int32_t *tree_parent, int o, int q) {
    if (tree_parent == NULL) return 1;
    if (q > 0 && tree_parent[o] != -1) return 0;
    for (int j = 1; j < q; ++j) {
        int p = tree_parent[o + j];
        if (p < 0 || p >= j) return 0;
    }
    return 1;
}

/* 1 iff token k is token j itself or one of j's ancestors (walks parents). */
static int is_ancestor_or_self(const int32_t *tree_parent, int o, int k, int j) {
    int a = j;
    while (a >= 0) {
        if (a == k) return 1;
        a = parent_of(tree_parent, o, a);
    }
    return 0;
}

/* Physical element offset of logical slot p of request i, KV head g. */
static long long slot_offset(const int32_t *block_tables, int max_blocks, int i, int p, int g,
                             int num_kv_heads, int page_size, int head_dim) {
    int page = block_tables[(long long)i * max_blocks + p / page_size];
    return (((long long)page * num_kv_heads + g) * page_size + (p % page_size)) * (long long)head_dim;
}

/*
 * Host threads the oracle's verify attention uses (OpenMP over independent
 * (request, KV head) pairs; 0 = the OpenMP default).  Every output element
 * is computed by one thread with the same operations in the same order
 * whatever the thread count, so the result does not depend on it.
 */
int oracle_set_threads(int n) {
#ifdef _OPENMP
    if (n > 0) omp_set_num_threads(n);
    return omp_get_max_threads();
#else
    (void)n;
    return 1;
#endif
}

/* Rows of one (request i, KV head g): every verify token j and every query
 * head h of g's group, as defined above oracle_verify_attn. */
static int verify_attn_group(const uint16_t *q, const uint16_t *k_cache, const uint16_t *v_cache,
                             const int32_t *block_tables, int max_blocks, const int32_t *context_lens,
                             const int32_t *cu_q, const int32_t *tree_parent, int num_q_heads,
                             int num_kv_heads, int head_dim, int page_size, double scale, int i,
                             int g, double *out) {
    const int G = num_q_heads / num_kv_heads;
    const int L = context_lens[i];
    const int o = cu_q[i];
    const int qn = cu_q[i + 1] - cu_q[i];
    const int nk = L + qn;
    /* explicit mask matrix M[j][p] */
    double *mask = (double *)malloc(sizeof(double) * (size_t)qn * (size_t)nk);
    double *s = (double *)malloc(sizeof(double) * (size_t)nk);
    if (!mask || !s) { free(mask); free(s); return ORACLE_NO_MEMORY; }
    for (int j = 0; j < qn; ++j)
        for (int p = 0; p < nk; ++p) {
            int vis = (p < L) || is_ancestor_or_self(tree_parent, o, p - L, j);
            mask[(size_t)j * nk + p] = vis ? 0.0 : -INFINITY;
        }
    for (int j = 0; j < qn; ++j) {
        for (int h = 0; h < num_q_heads; ++h) {
            if (h / G != g) continue;
            const uint16_t *qrow = q + ((long long)(o + j) * num_q_heads + h) * head_dim;
            /* scores */
            for (int p = 0; p < nk; ++p) {
                const uint16_t *krow = k_cache + slot_offset(block_tables, max_blocks, i, p, g,
                                                             num_kv_heads, page_size, head_dim);
                double dot = 0.0;
                for (int d = 0; d < head_dim; ++d)
                    dot += bf16_to_double(qrow[d]) * bf16_to_double(krow[d]);
                s[p] = scale * dot + mask[(size_t)j * nk + p];
            }
            /* two-pass softmax */
            double m = -INFINITY;
            for (int p = 0; p < nk; ++p)
                if (s[p] > m) m = s[p];
            double z = 0.0;
            for (int p = 0; p < nk; ++p) {
                s[p] = exp(s[p] - m); /* masked: exp(-inf) = 0 */
                z += s[p];
            }
            double *orow = out + ((long long)(o + j) * num_q_heads + h) * head_dim;
            for (int d = 0; d < head_dim; ++d) orow[d] = 0.0;
            for (int p = 0; p < nk; ++p) {
                const double w = s[p] / z;
                const uint16_t *vrow = v_cache + slot_offset(block_tables, max_blocks, i, p, g,
                                                             num_kv_heads, page_size, head_dim);
                for (int d = 0; d < head_dim; ++d) orow[d] += w * bf16_to_double(vrow[d]);
            }
        }
    }
    free(mask);
    free(s);
    return ORACLE_OK;
}

/*
 * Verify attention (one layer), fp64, explicit mask matrix.
 * For request i in [req_begin, req_end), token j, query head h:
 *   visible(p) = p < L_i                                  (committed prefix)
 *             or (p = L_i + k, k ancestor-or-self of j)   (verify tokens)
 *   M[j][p]    = 0 if visible else -inf
 *   s_p        = scale * sum_d q[j,h,d] * K[p,g,d] + M[j][p]
 *   out[j,h,:] = sum_p softmax(s)_p * V[p,g,:]
 * out is [T, Hq, D] fp64; rows of requests outside the range are untouched.
 * The inputs of every request are checked first; then the independent
 * (request, KV head) pairs are computed, in parallel over host threads.
 */
int oracle_verify_attn(const uint16_t *q, const uint16_t *k_cache, const uint16_t *v_cache,
                       const int32_t *block_tables, int max_blocks, const int32_t *context_lens,
                       const int32_t *cu_q, const int32_t *tree_parent, int batch, int num_q_heads,
                       int num_kv_heads, int head_dim, int page_size, int num_pages, double scale,
                       int req_begin, int req_end, double *out) {
    if (num_kv_heads <= 0 || num_q_heads % num_kv_heads != 0 || head_dim <= 0 || page_size <= 0)
        return ORACLE_BAD_ARG;
    if (req_begin < 0 || req_end > batch || req_begin > req_end) return ORACLE_BAD_ARG;
    for (int i = req_begin; i < req_end; ++i) {
        const int L = context_lens[i];
        const int o = cu_q[i];
        const int qn = cu_q[i + 1] - cu_q[i];
        const int nk = L + qn;
        if (L < 0 || qn < 0) return ORACLE_BAD_CONTENT;
        if (qn == 0) continue;
        if (!check_parents(tree_parent, o, qn)) return ORACLE_BAD_CONTENT;
        if ((nk + page_size - 1) / page_size > max_blocks) return ORACLE_BAD_CONTENT;
        for (int p = 0; p < (nk + page_size - 1) / page_size; ++p) {
            int pg = block_tables[(long long)i * max_blocks + p];
            if (pg < 0 || pg >= num_pages) return ORACLE_BAD_CONTENT;
        }
    }
    const long long n_tasks = (long long)(req_end - req_begin) * num_kv_heads;
    int rc = ORACLE_OK;
#pragma omp parallel for schedule(dynamic, 1)
    for (long long t = 0; t < n_tasks; ++t) {
        const int i = req_begin + (int)(t / num_kv_heads);
        const int g = (int)(t % num_kv_heads);
        if (cu_q[i + 1] - cu_q[i] == 0) continue;
        int r = verify_attn_group(q, k_cache, v_cache, block_tables, max_blocks, context_lens, cu_q,
                                  tree_parent, num_q_heads, num_kv_heads, head_dim, page_size, scale,
                                  i, g, out);
        if (r != ORACLE_OK) {
#pragma omp atomic write
            rc = r;
        }
    }
    return rc;
}

/*
 * One-token decode reference: a single query (request i, query head h)
 * standing at logical position pos attends to every cached key in [0, pos]
 * with no mask at all.  Used to check that verifying a chain equals decoding
 * its tokens one by one.  out is [head_dim] fp64.
 */
int oracle_decode_attn(const uint16_t *q_row, const uint16_t *k_cache, const uint16_t *v_cache,
                       const int32_t *block_tables, int max_blocks, int i, int h, int pos,
                       int num_q_heads, int num_kv_heads, int head_dim, int page_size,
                       double scale, double *out) {
    if (num_kv_heads <= 0 || num_q_heads % num_kv_heads != 0 || pos < 0) return ORACLE_BAD_ARG;
    const int g = h / (num_q_heads / num_kv_heads);
    const int nk = pos + 1;
    double *s = (double *)malloc(sizeof(double) * (size_t)nk);
    if (!s) return ORACLE_NO_MEMORY;
    double m = -INFINITY;
    for (int p = 0; p < nk; ++p) {
        const uint16_t *krow = k_cache + slot_offset(block_tables, max_blocks, i, p, g, num_kv_heads,
                                                     page_size, head_dim);
        double dot = 0.0;
        for (int d = 0; d < head_dim; ++d) dot += bf16_to_double(q_row[d]) * bf16_to_double(krow[d]);
        s[p] = scale * dot;
        if (s[p] > m) m = s[p];
    }
    double z = 0.0;
    for (int p = 0; p < nk; ++p) { s[p] = exp(s[p] - m); z += s[p]; }
    for (int d = 0; d < head_dim; ++d) out[d] = 0.0;
    for (int p = 0; p < nk; ++p) {
        const uint16_t *vrow = v_cache + slot_offset(block_tables, max_blocks, i, p, g, num_kv_heads,
                                                     page_size, head_dim);
        for (int d = 0; d < head_dim; ++d) out[d] += (s[p] / z) * bf16_to_double(vrow[d]);
    }
    free(s);
    return ORACLE_OK;
}

/*
 * Greedy target token of every logits row: the naive left-to-right scan,
 * so the lowest index wins ties and IEEE comparison makes -0 equal +0.
 */
int oracle_argmax(const float *logits, long long rows, long long vocab, int32_t *out) {
    if (vocab <= 0 || rows < 0) return ORACLE_BAD_ARG;
    for (long long r = 0; r < rows; ++r) {
        const float *x = logits + r * vocab;
        long long best = 0;
        for (long long v = 1; v < vocab; ++v)
            if (x[v] > x[best]) best = v;
        out[r] = (int32_t)best;
    }
    return ORACLE_OK;
}

/*
 * Greedy acceptance (longest matching prefix; for trees, the deepest accepted
 * root path).  target[] is the argmax of each logits row.
 *   chain: n = largest k <= q_i-1 with draft[o+j] == target[o+j-1] for all 1<=j<=k
 *   tree:  acc[0] = 1; acc[j] = acc[parent[j]] && draft[o+j] == target[o+parent[j]];
 *          depth[j] = depth[parent[j]] + 1; best = accepted node of greatest depth,
 *          lowest index among equals; path = root..best; n = depth[best]
 * Outputs: accept_len[i] = n+1 (bonus token counted);
 *          accepted_path[o+k] = path[k] for k <= n, -1 beyond;
 *          out_tokens[o+k]    = target[o+path[k]] for k <= n, -1 beyond.
 * A request with q_i = 0 gets accept_len 0.
 */
int oracle_accept(const int32_t *draft, const int32_t *target, const int32_t *cu_q,
                  const int32_t *tree_parent, int batch, int32_t *accept_len,
                  int32_t *accepted_path, int32_t *out_tokens) {
    for (int i = 0; i < batch; ++i) {
        const int o = cu_q[i];
        const int qn = cu_q[i + 1] - cu_q[i];
        if (qn < 0) return ORACLE_BAD_CONTENT;
        for (int k = 0; k < qn; ++k) { accepted_path[o + k] = -1; out_tokens[o + k] = -1; }
        if (qn == 0) { accept_len[i] = 0; continue; }
        if (!check_parents(tree_parent, o, qn)) return ORACLE_BAD_CONTENT;
        int n = 0;
        int *path = (int *)malloc(sizeof(int) * (size_t)qn);
        if (!path) return ORACLE_NO_MEMORY;
        if (tree_parent == NULL) {
            while (n < qn - 1 && draft[o + n + 1] == target[o + n]) ++n;
            for (int k = 0; k <= n; ++k) path[k] = k;
        } else {
            int *acc = (int *)malloc(sizeof(int) * (size_t)qn);
            int *depth = (int *)malloc(sizeof(int) * (size_t)qn);
            if (!acc || !depth) { free(acc); free(depth); free(path); return ORACLE_NO_MEMORY; }
            acc[0] = 1;
            depth[0] = 0;
            for (int j = 1; j < qn; ++j) {
                const int p = tree_parent[o + j];
                acc[j] = acc[p] && draft[o + j] == target[o + p];
                depth[j] = depth[p] + 1;
            }
            int best = 0;
            for (int j = 1; j < qn; ++j)
                if (acc[j] && depth[j] > depth[best]) best = j;
            n = depth[best];
            for (int a = best, k = n; a >= 0; a = tree_parent[o + a], --k) path[k] = a;
            free(acc);
            free(depth);
        }
        accept_len[i] = n + 1;
        for (int k = 0; k <= n; ++k) {
            accepted_path[o + k] = path[k];
            out_tokens[o + k] = target[o + path[k]];
        }
        free(path);
    }
    return ORACLE_OK;
}

/*
 * One step of chunked verification with early pruning (FASER, "Early Token
 * Pruning": verification runs over chunks of the verify tokens, and at each
 * chunk boundary the tokens behind an already rejected prefix are dropped).
 * Request i verified tokens [0, e) so far, e = chunk_begin[i] + chunk_len[i];
 * target[] is read for those tokens only.  For a token j >= 1 with parent p,
 * the edge p -> j is decided when p < e and then matches iff
 * draft[o+j] == target[o+p].  Token j is alive iff no decided edge on its
 * root path fails to match.
 *   - chunk_len[i] == 0: the request is not in this chunk; nothing changes
 *     (next_len = 0, next_begin = chunk_begin).
 *   - e < q_i and some token in [e, q_i) is alive: the request goes on,
 *     next_begin = e, next_len = min(chunk_size, q_i - e).
 *   - otherwise it ends: the result of oracle_accept computed with the
 *     tokens < e only (a token >= e counts as not accepted), next_len = 0,
 *     next_begin = e.
 */
int oracle_accept_chunk_step(const int32_t *draft, const int32_t *target, const int32_t *cu_q,
                             const int32_t *tree_parent, const int32_t *chunk_begin,
                             const int32_t *chunk_len, int batch, int chunk_size,
                             int32_t *accept_len, int32_t *accepted_path, int32_t *out_tokens,
                             int32_t *next_begin, int32_t *next_len) {
    if (chunk_size <= 0) return ORACLE_BAD_ARG;
    for (int i = 0; i < batch; ++i) {
        const int o = cu_q[i];
        const int qn = cu_q[i + 1] - cu_q[i];
        const int s = chunk_begin[i], c = chunk_len[i];
        if (qn < 0 || s < 0 || c < 0 || s + c > qn) return ORACLE_BAD_CONTENT;
        if (c == 0) { next_begin[i] = s; next_len[i] = 0; continue; }
        if (!check_parents(tree_parent, o, qn)) return ORACLE_BAD_CONTENT;
        const int e = s + c;
        /* alive tokens: walk every token's root path over the decided edges */
        int go_on = 0;
        for (int j = e; j < qn && !go_on; ++j) {
            int alive = 1;
            for (int a = j; a > 0; a = parent_of(tree_parent, o, a)) {
                const int p = parent_of(tree_parent, o, a);
                if (p < e && draft[o + a] != target[o + p]) { alive = 0; break; }
            }
            go_on = alive;
        }
        if (go_on) {
            next_begin[i] = e;
            next_len[i] = qn - e < chunk_size ? qn - e : chunk_size;
            continue;
        }
        /* the request ends: greedy acceptance over the tokens < e */
        for (int k = 0; k < qn; ++k) { accepted_path[o + k] = -1; out_tokens[o + k] = -1; }
        int *acc = (int *)malloc(sizeof(int) * (size_t)qn);
        int *depth = (int *)malloc(sizeof(int) * (size_t)qn);
        int *path = (int *)malloc(sizeof(int) * (size_t)qn);
        if (!acc || !depth || !path) { free(acc); free(depth); free(path); return ORACLE_NO_MEMORY; }
        acc[0] = 1;
        depth[0] = 0;
        for (int j = 1; j < qn; ++j) {
            const int p = parent_of(tree_parent, o, j);
            acc[j] = j < e && acc[p] && draft[o + j] == target[o + p];
            depth[j] = depth[p] + 1;
        }
        int best = 0;
        for (int j = 1; j < qn; ++j)
            if (acc[j] && depth[j] > depth[best]) { best = j; }
        const int n = depth[best];
        for (int a = best, k = n; a >= 0; a = parent_of(tree_parent, o, a), --k) path[k] = a;
        accept_len[i] = n + 1;
        for (int k = 0; k <= n; ++k) {
            accepted_path[o + k] = path[k];
            out_tokens[o + k] = target[o + accepted_path[o + k]];
        }
        next_begin[i] = e;
        next_len[i] = 0;
        free(acc);
        free(depth);
        free(path);
    }
    return ORACLE_OK;
}

/*
 * Copy-based KV compaction.  For every layer, the whole pool is first
 * snapshotted; then for each request i, KV head g and k = 0..accept_len_i-1
 * the snapshot's logical slot L_i + path[k] is written into logical slot
 * L_i + k.  Every other slot keeps its value.  new_context_lens[i] =
 * L_i + accept_len_i.  Rejected slots beyond the new length are left as they
 * are (the caller releases pages past the new length).
 */
int oracle_compact(uint16_t *k_cache, uint16_t *v_cache, long long layer_stride_elems, int num_layers,
                   const int32_t *block_tables, int max_blocks, const int32_t *context_lens,
                   const int32_t *cu_q, const int32_t *accepted_path, const int32_t *accept_len,
                   int32_t *new_context_lens, int batch, int num_kv_heads, int head_dim,
                   int page_size, int num_pages) {
    const long long pool = (long long)num_pages * num_kv_heads * page_size * head_dim;
    for (int i = 0; i < batch; ++i) {
        const int qn = cu_q[i + 1] - cu_q[i];
        const int n1 = accept_len[i];
        if (n1 < 0 || n1 > qn) return ORACLE_BAD_CONTENT;
        for (int k = 0; k < n1; ++k) {
            int pk = accepted_path[cu_q[i] + k];
            if (pk < k || pk >= qn || (k == 0 && pk != 0) ||
                (k > 0 && pk <= accepted_path[cu_q[i] + k - 1]))
                return ORACLE_BAD_CONTENT;
        }
        int nk = context_lens[i] + qn;
        if ((nk + page_size - 1) / page_size > max_blocks) return ORACLE_BAD_CONTENT;
    }
    uint16_t *snap = (uint16_t *)malloc(sizeof(uint16_t) * (size_t)pool);
    if (!snap) return ORACLE_NO_MEMORY;
    for (int layer = 0; layer < num_layers; ++layer) {
        for (int which = 0; which < 2; ++which) {
            uint16_t *cache = (which == 0 ? k_cache : v_cache) + (long long)layer * layer_stride_elems;
            memcpy(snap, cache, sizeof(uint16_t) * (size_t)pool);
            for (int i = 0; i < batch; ++i) {
                const int L = context_lens[i];
                for (int g = 0; g < num_kv_heads; ++g)
                    for (int k = 0; k < accept_len[i]; ++k) {
                        const int src = L + accepted_path[cu_q[i] + k];
                        const int dst = L + k;
                        long long so = slot_offset(block_tables, max_blocks, i, src, g, num_kv_heads,
                                                   page_size, head_dim);
                        long long d0 = slot_offset(block_tables, max_blocks, i, dst, g, num_kv_heads,
                                                   page_size, head_dim);
                        memcpy(cache + d0, snap + so, sizeof(uint16_t) * (size_t)head_dim);
                    }
            }
        }
    }
    free(snap);
    for (int i = 0; i < batch; ++i) new_context_lens[i] = context_lens[i] + accept_len[i];
    return ORACLE_OK;
}
