// C ABI of libspecverify: host-side argument validation, workspace layout and
// kernel launches.  Argument errors are detected here, before any HIP call.
#include <math.h>
#include <stdarg.h>
#include <stdio.h>
#include <string.h>

#include <algorithm>
#include <atomic>
#include <mutex>

#include "sv_internal.h"
#include "read_probe.h"

namespace {

thread_local char g_last_error[512] = "";

int fail(int status, const char *fmt, ...) __attribute__((format(printf, 2, 3)));
int fail(int status, const char *fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_last_error, sizeof g_last_error, fmt, ap);
  va_end(ap);
  return status;
}

int ok() {
  g_last_error[0] = '\0';
  return SV_OK;
}

int check_launch(const char *what) {
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return fail(SV_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
  return ok();
}

bool overlaps(const void *a, size_t an, const void *b, size_t bn) {
  const char *x = static_cast<const char *>(a), *y = static_cast<const char *>(b);
  return x < y + bn && y < x + an;
}

int read_status(const void *workspace, size_t offset, uint32_t *flags, void *stream) {
  if (!workspace || !flags) return fail(SV_ERR_NULL, "workspace and flags must be non-NULL");
  hipStream_t s = static_cast<hipStream_t>(stream);
  uint32_t v = 0;
  hipError_t e = hipMemcpyAsync(&v, static_cast<const char *>(workspace) + offset, sizeof v,
                                hipMemcpyDeviceToHost, s);
  if (e == hipSuccess) e = hipStreamSynchronize(s);
  if (e != hipSuccess) return fail(SV_ERR_HIP, "device status read: %s", hipGetErrorString(e));
  *flags = v;
  return ok();
}

int accept_args(const float *logits, int vocab, const int32_t *draft_tokens, const int32_t *cu_q,
                const int32_t *tree_parent, int batch, int total_q, int32_t *target_argmax,
                int32_t *accept_len, int32_t *accepted_path, int32_t *out_tokens, void *workspace,
                size_t workspace_bytes, bool fused, sv::AcceptArgs *out, bool *empty) {
  *empty = false;
  if (batch < 0 || total_q < 0)
    return fail(SV_ERR_SHAPE, "batch (%d) and total_q (%d) must be >= 0", batch, total_q);
  if (vocab <= 0) return fail(SV_ERR_SHAPE, "vocab %d must be > 0", vocab);
  if (total_q > (long long)batch * sv::kMaxTokens)
    return fail(SV_ERR_SHAPE, "total_q %d exceeds batch*64", total_q);
  if (batch == 0) {
    *empty = true;
    return ok();
  }
  if (!cu_q || !accept_len || !workspace)
    return fail(SV_ERR_NULL, "acceptance: a required pointer is NULL");
  if (total_q > 0 && (!logits || !draft_tokens || !target_argmax || !accepted_path || !out_tokens))
    return fail(SV_ERR_NULL, "acceptance: a required pointer is NULL");
  const sv::AcceptLayout lay = fused ? sv::fused_layout(batch, total_q, vocab)
                                     : sv::accept_layout(batch, total_q, vocab);
  if (workspace_bytes < lay.total)
    return fail(SV_ERR_WORKSPACE, "workspace %zu bytes < required %zu", workspace_bytes, lay.total);
  const size_t tb = (size_t)total_q * 4;
  if (overlaps(target_argmax, tb, accepted_path, tb) || overlaps(target_argmax, tb, out_tokens, tb) ||
      overlaps(accepted_path, tb, out_tokens, tb) ||
      overlaps(accept_len, (size_t)batch * 4, target_argmax, tb) ||
      overlaps(accept_len, (size_t)batch * 4, accepted_path, tb) ||
      overlaps(accept_len, (size_t)batch * 4, out_tokens, tb))
    return fail(SV_ERR_ALIAS, "spec_accept outputs overlap");
  sv::AcceptArgs a;
  memset(&a, 0, sizeof a);
  a.logits = logits;
  a.draft = draft_tokens;
  a.cu_q = cu_q;
  a.tree_parent = tree_parent;
  a.target_argmax = target_argmax;
  a.accept_len = accept_len;
  a.accepted_path = accepted_path;
  a.out_tokens = out_tokens;
  a.ws = static_cast<char *>(workspace);
  a.lay = lay;
  a.batch = batch;
  a.total_q = total_q;
  a.vocab = vocab;
  a.rows = total_q;
  *out = a;
  return ok();
}

int compact_args(void *k_cache, void *v_cache, int64_t layer_stride_elems, int num_layers,
                 const int32_t *block_tables, int max_blocks_per_seq, const int32_t *context_lens,
                 const int32_t *cu_q, const int32_t *accepted_path, const int32_t *accept_len,
                 int32_t *new_context_lens, int batch, int total_q, int num_kv_heads, int head_dim,
                 int page_size, int num_pages, sv::CompactArgs *out, bool *empty) {
  *empty = false;
  if (batch < 0 || total_q < 0 || num_layers < 0)
    return fail(SV_ERR_SHAPE, "batch, total_q and num_layers must be >= 0");
  if (head_dim != 64 && head_dim != 128)
    return fail(SV_ERR_UNSUPPORTED, "head_dim %d (supported: 64, 128)", head_dim);
  if (page_size != sv::kPage)
    return fail(SV_ERR_UNSUPPORTED, "page_size %d (supported: 16)", page_size);
  if (num_kv_heads <= 0) return fail(SV_ERR_SHAPE, "num_kv_heads must be > 0");
  if (batch == 0) {
    *empty = true;
    return ok();
  }
  if (!block_tables || !context_lens || !cu_q || !accept_len || !new_context_lens)
    return fail(SV_ERR_NULL, "kv_compact: a required pointer is NULL");
  if (num_layers > 0 && (!k_cache || !v_cache))
    return fail(SV_ERR_NULL, "kv_compact: cache pointers are NULL");
  if (total_q > 0 && !accepted_path) return fail(SV_ERR_NULL, "kv_compact: accepted_path is NULL");
  if (max_blocks_per_seq <= 0 || num_pages <= 0)
    return fail(SV_ERR_SHAPE, "max_blocks_per_seq and num_pages must be > 0");
  const long long pool = (long long)num_pages * num_kv_heads * page_size * head_dim;
  if (num_layers > 1 && layer_stride_elems < pool)
    return fail(SV_ERR_SHAPE, "layer_stride_elems %lld smaller than one pool (%lld)",
                (long long)layer_stride_elems, pool);
  if (new_context_lens == context_lens ||
      overlaps(new_context_lens, (size_t)batch * 4, context_lens, (size_t)batch * 4))
    return fail(SV_ERR_ALIAS, "new_context_lens must not alias context_lens");
  sv::CompactArgs a;
  a.k_cache = static_cast<uint16_t *>(k_cache);
  a.v_cache = static_cast<uint16_t *>(v_cache);
  a.layer_stride = layer_stride_elems;
  a.num_layers = num_layers;
  a.block_tables = block_tables;
  a.max_blocks = max_blocks_per_seq;
  a.context_lens = context_lens;
  a.cu_q = cu_q;
  a.accepted_path = accepted_path;
  a.accept_len = accept_len;
  a.new_context_lens = new_context_lens;
  a.batch = batch;
  a.total_q = total_q;
  a.num_kv_heads = num_kv_heads;
  a.head_dim = head_dim;
  a.num_pages = num_pages;
  *out = a;
  return ok();
}

}  // namespace

extern "C" {

const char *sv_status_string(int status) {
  switch (status) {
    case SV_OK: return "ok";
    case SV_ERR_NULL: return "a required pointer is NULL";
    case SV_ERR_SHAPE: return "a size argument is out of range or inconsistent";
    case SV_ERR_UNSUPPORTED: return "unsupported head_dim, page_size or head grouping";
    case SV_ERR_WORKSPACE: return "workspace too small";
    case SV_ERR_ALIAS: return "an output overlaps an input";
    case SV_ERR_HIP: return "a HIP call failed";
    default: return "unknown status";
  }
}

const char *sv_last_error(void) { return g_last_error; }

size_t spec_verify_attn_workspace_size(int batch, int total_q, int num_q_heads, int num_kv_heads,
                                       int head_dim) {
  if (batch < 0 || total_q < 0 || num_kv_heads <= 0 || num_q_heads <= 0 ||
      num_q_heads % num_kv_heads != 0 || head_dim <= 0)
    return 0;
  return sv::attn_layout(batch, total_q, num_q_heads, num_kv_heads, head_dim).total;
}

}  // extern "C"

namespace {

// Shared argument checks of the verify-attention calls; on success fills the
// kernel argument block (metadata only; data pointers are set by the caller).
int attn_common(const int32_t *block_tables, int max_blocks_per_seq, const int32_t *context_lens,
                const int32_t *cu_q, int batch, int total_q, int num_q_heads, int num_kv_heads,
                int head_dim, int page_size, int num_pages, void *workspace,
                size_t workspace_bytes, bool need_tables, sv::AttnArgs *a, bool *empty) {
  *empty = false;
  if (batch < 0 || total_q < 0)
    return fail(SV_ERR_SHAPE, "batch (%d) and total_q (%d) must be >= 0", batch, total_q);
  if (num_q_heads <= 0 || num_kv_heads <= 0 || num_q_heads % num_kv_heads != 0)
    return fail(SV_ERR_SHAPE, "num_q_heads (%d) must be a positive multiple of num_kv_heads (%d)",
                num_q_heads, num_kv_heads);
  if (num_q_heads / num_kv_heads > 64)
    return fail(SV_ERR_UNSUPPORTED, "more than 64 query heads per KV head");
  if (head_dim != 64 && head_dim != 128)
    return fail(SV_ERR_UNSUPPORTED, "head_dim %d (supported: 64, 128)", head_dim);
  if (page_size != sv::kPage)
    return fail(SV_ERR_UNSUPPORTED, "page_size %d (supported: 16)", page_size);
  if (total_q > (long long)batch * sv::kMaxTokens)
    return fail(SV_ERR_SHAPE, "total_q %d exceeds batch*64", total_q);
  if (batch == 0 || total_q == 0) {
    *empty = true;
    return ok();
  }
  if (!context_lens || !cu_q || !workspace || (need_tables && !block_tables))
    return fail(SV_ERR_NULL, "spec_verify_attn: a required pointer is NULL");
  if (max_blocks_per_seq <= 0 || num_pages <= 0)
    return fail(SV_ERR_SHAPE, "max_blocks_per_seq (%d) and num_pages (%d) must be > 0",
                max_blocks_per_seq, num_pages);
  const sv::AttnLayout lay = sv::attn_layout(batch, total_q, num_q_heads, num_kv_heads, head_dim);
  if (workspace_bytes < lay.total)
    return fail(SV_ERR_WORKSPACE, "workspace %zu bytes < required %zu", workspace_bytes, lay.total);
  memset(a, 0, sizeof *a);
  a->block_tables = block_tables;
  a->context_lens = context_lens;
  a->cu_q = cu_q;
  a->ws = static_cast<char *>(workspace);
  a->lay = lay;
  a->batch = batch;
  a->total_q = total_q;
  a->num_q_heads = num_q_heads;
  a->num_kv_heads = num_kv_heads;
  a->group = num_q_heads / num_kv_heads;
  a->max_blocks = max_blocks_per_seq;
  a->num_pages = num_pages;
  a->cu_full = cu_q;
  a->total_full = total_q;
  return ok();
}

// Chunked rows: cu_rows packs the rows, cu_full and total_full all verify
// tokens; chunk_begin gives each request's first token among the rows.
int attn_chunk(const int32_t *cu_full, int total_full, const int32_t *chunk_begin, int batch,
               sv::AttnArgs *a) {
  if (!cu_full || !chunk_begin) return fail(SV_ERR_NULL, "chunked verify: cu_q or chunk_begin is NULL");
  if (total_full < 0 || total_full > (long long)batch * sv::kMaxTokens)
    return fail(SV_ERR_SHAPE, "total_q %d must be in [0, batch*64]", total_full);
  a->chunk_begin = chunk_begin;
  a->cu_full = cu_full;
  a->total_full = total_full;
  return ok();
}

// One persistent attention workgroup per compute unit of the current device
// (queried after every argument check, right before launching).
int set_grid(sv::AttnArgs *a) {
  int dev = 0, cus = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e == hipSuccess) e = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
  if (e != hipSuccess) return fail(SV_ERR_HIP, "device query: %s", hipGetErrorString(e));
  a->grid = cus < 1 ? 1 : (cus > sv::kMaxGrid ? sv::kMaxGrid : cus);
  return ok();
}

int attn_data(const void *q, const void *k_cache, const void *v_cache, const int32_t *tree_parent,
              void *out, int head_dim, int page_size, float softmax_scale, bool v_transposed,
              sv::AttnArgs *a) {
  if (!q || !k_cache || !v_cache || !out)
    return fail(SV_ERR_NULL, "spec_verify_attn: a required pointer is NULL");
  if (!(softmax_scale >= 0.0f && isfinite(softmax_scale)))
    return fail(SV_ERR_SHAPE, "softmax_scale must be finite and >= 0 (0 selects 1/sqrt(head_dim))");
  const size_t qo_bytes = (size_t)a->total_q * a->num_q_heads * head_dim * 2;
  const size_t kv_bytes = (size_t)a->num_pages * a->num_kv_heads * page_size * head_dim * 2;
  if (overlaps(out, qo_bytes, q, qo_bytes) || overlaps(out, qo_bytes, k_cache, kv_bytes) ||
      overlaps(out, qo_bytes, v_cache, kv_bytes) || overlaps(out, qo_bytes, a->ws, a->lay.total))
    return fail(SV_ERR_ALIAS, "out overlaps q, the caches or the workspace");
  a->q = static_cast<const uint16_t *>(q);
  a->k_cache = static_cast<const uint16_t *>(k_cache);
  a->v_cache = static_cast<const uint16_t *>(v_cache);
  a->tree_parent = tree_parent;
  a->out = static_cast<uint16_t *>(out);
  const float scale = softmax_scale == 0.0f ? 1.0f / sqrtf((float)head_dim) : softmax_scale;
  a->scale_log2 = scale * 1.4426950408889634f;
  a->v_transposed = v_transposed;
  return ok();
}

int attn_run(const void *q, const void *k_cache, const void *v_cache, const int32_t *block_tables,
             int max_blocks_per_seq, const int32_t *context_lens, const int32_t *cu_q,
             const int32_t *tree_parent, void *out, int batch, int total_q, int num_q_heads,
             int num_kv_heads, int head_dim, int page_size, int num_pages, float softmax_scale,
             void *workspace, size_t workspace_bytes, void *stream, bool with_plan, bool v_transposed,
             const char *what) {
  sv::AttnArgs a;
  bool empty;
  int rc = attn_common(block_tables, max_blocks_per_seq, context_lens, cu_q, batch, total_q,
                       num_q_heads, num_kv_heads, head_dim, page_size, num_pages, workspace,
                       workspace_bytes, true, &a, &empty);
  if (rc != SV_OK || empty) return rc;
  rc = attn_data(q, k_cache, v_cache, tree_parent, out, head_dim, page_size, softmax_scale, v_transposed, &a);
  if (rc != SV_OK) return rc;
  if ((rc = set_grid(&a)) != SV_OK) return rc;
  if (with_plan) sv::launch_verify_attn_plan(a, static_cast<hipStream_t>(stream));
  sv::launch_verify_attn_run(a, head_dim, static_cast<hipStream_t>(stream));
  return check_launch(what);
}

// A chunk's rows are read and written in place in q and out, which hold one
// row per verify token (total_q); their count, cu_chunk[batch], is read on
// the device, with total_q as its bound.
int attn_chunk_run(const void *q, const void *k_cache, const void *v_cache, const int32_t *block_tables,
                   int max_blocks_per_seq, const int32_t *context_lens, const int32_t *cu_q, int total_q,
                   const int32_t *chunk_begin, const int32_t *cu_chunk, const int32_t *tree_parent, void *out,
                   int batch, int num_q_heads, int num_kv_heads, int head_dim, int page_size, int num_pages,
                   float softmax_scale, void *workspace, size_t workspace_bytes, void *stream, bool v_transposed,
                   const char *what) {
  sv::AttnArgs a;
  bool empty;
  int rc = attn_common(block_tables, max_blocks_per_seq, context_lens, cu_chunk, batch, total_q,
                       num_q_heads, num_kv_heads, head_dim, page_size, num_pages, workspace,
                       workspace_bytes, true, &a, &empty);
  if (rc != SV_OK || empty) return rc;
  if ((rc = attn_chunk(cu_q, total_q, chunk_begin, batch, &a)) != SV_OK) return rc;
  rc = attn_data(q, k_cache, v_cache, tree_parent, out, head_dim, page_size, softmax_scale, v_transposed, &a);
  if (rc != SV_OK) return rc;
  if ((rc = set_grid(&a)) != SV_OK) return rc;
  sv::launch_verify_attn_run(a, head_dim, static_cast<hipStream_t>(stream));
  return check_launch(what);
}

}  // namespace

extern "C" {

int spec_verify_attn_plan(const int32_t *context_lens, const int32_t *cu_q, int max_blocks_per_seq,
                          int batch, int total_q, int num_q_heads, int num_kv_heads, int head_dim,
                          int num_pages, void *workspace, size_t workspace_bytes, void *stream) {
  sv::AttnArgs a;
  bool empty;
  int rc = attn_common(nullptr, max_blocks_per_seq, context_lens, cu_q, batch, total_q, num_q_heads,
                       num_kv_heads, head_dim, sv::kPage, num_pages, workspace, workspace_bytes,
                       false, &a, &empty);
  if (rc != SV_OK || empty) return rc;
  if ((rc = set_grid(&a)) != SV_OK) return rc;
  sv::launch_verify_attn_plan(a, static_cast<hipStream_t>(stream));
  return check_launch("spec_verify_attn_plan");
}

int spec_verify_attn_run(const void *q, const void *k_cache, const void *v_cache,
                         const int32_t *block_tables, int max_blocks_per_seq,
                         const int32_t *context_lens, const int32_t *cu_q,
                         const int32_t *tree_parent, void *out, int batch, int total_q,
                         int num_q_heads, int num_kv_heads, int head_dim, int page_size,
                         int num_pages, float softmax_scale, void *workspace,
                         size_t workspace_bytes, void *stream) {
  return attn_run(q, k_cache, v_cache, block_tables, max_blocks_per_seq, context_lens, cu_q, tree_parent, out,
                  batch, total_q, num_q_heads, num_kv_heads, head_dim, page_size, num_pages, softmax_scale,
                  workspace, workspace_bytes, stream, false, false, "spec_verify_attn_run");
}

int spec_verify_attn_run_vt(const void *q, const void *k_cache, const void *v_cache,
                            const int32_t *block_tables, int max_blocks_per_seq,
                            const int32_t *context_lens, const int32_t *cu_q,
                            const int32_t *tree_parent, void *out, int batch, int total_q,
                            int num_q_heads, int num_kv_heads, int head_dim, int page_size,
                            int num_pages, float softmax_scale, void *workspace,
                            size_t workspace_bytes, void *stream) {
  return attn_run(q, k_cache, v_cache, block_tables, max_blocks_per_seq, context_lens, cu_q, tree_parent, out,
                  batch, total_q, num_q_heads, num_kv_heads, head_dim, page_size, num_pages, softmax_scale,
                  workspace, workspace_bytes, stream, false, true, "spec_verify_attn_run_vt");
}

int spec_verify_attn(const void *q, const void *k_cache, const void *v_cache,
                     const int32_t *block_tables, int max_blocks_per_seq,
                     const int32_t *context_lens, const int32_t *cu_q, const int32_t *tree_parent,
                     void *out, int batch, int total_q, int num_q_heads, int num_kv_heads,
                     int head_dim, int page_size, int num_pages, float softmax_scale,
                     void *workspace, size_t workspace_bytes, void *stream) {
  return attn_run(q, k_cache, v_cache, block_tables, max_blocks_per_seq, context_lens, cu_q, tree_parent, out,
                  batch, total_q, num_q_heads, num_kv_heads, head_dim, page_size, num_pages, softmax_scale,
                  workspace, workspace_bytes, stream, true, false, "spec_verify_attn");
}

int spec_verify_attn_vt(const void *q, const void *k_cache, const void *v_cache,
                        const int32_t *block_tables, int max_blocks_per_seq,
                        const int32_t *context_lens, const int32_t *cu_q, const int32_t *tree_parent,
                        void *out, int batch, int total_q, int num_q_heads, int num_kv_heads,
                        int head_dim, int page_size, int num_pages, float softmax_scale,
                        void *workspace, size_t workspace_bytes, void *stream) {
  return attn_run(q, k_cache, v_cache, block_tables, max_blocks_per_seq, context_lens, cu_q, tree_parent, out,
                  batch, total_q, num_q_heads, num_kv_heads, head_dim, page_size, num_pages, softmax_scale,
                  workspace, workspace_bytes, stream, true, true, "spec_verify_attn_vt");
}

int spec_verify_attn_chunk_plan(const int32_t *context_lens, const int32_t *cu_q, int total_q,
                                const int32_t *chunk_begin, const int32_t *cu_chunk, int max_blocks_per_seq,
                                int batch, int num_q_heads, int num_kv_heads, int head_dim, int num_pages,
                                void *workspace, size_t workspace_bytes, void *stream) {
  sv::AttnArgs a;
  bool empty;
  int rc = attn_common(nullptr, max_blocks_per_seq, context_lens, cu_chunk, batch, total_q,
                       num_q_heads, num_kv_heads, head_dim, sv::kPage, num_pages, workspace,
                       workspace_bytes, false, &a, &empty);
  if (rc != SV_OK || empty) return rc;
  if ((rc = attn_chunk(cu_q, total_q, chunk_begin, batch, &a)) != SV_OK) return rc;
  if ((rc = set_grid(&a)) != SV_OK) return rc;
  sv::launch_verify_attn_plan(a, static_cast<hipStream_t>(stream));
  return check_launch("spec_verify_attn_chunk_plan");
}

int spec_verify_attn_chunk_run(const void *q, const void *k_cache, const void *v_cache,
                               const int32_t *block_tables, int max_blocks_per_seq,
                               const int32_t *context_lens, const int32_t *cu_q, int total_q,
                               const int32_t *chunk_begin, const int32_t *cu_chunk, const int32_t *tree_parent,
                               void *out, int batch, int num_q_heads, int num_kv_heads, int head_dim,
                               int page_size, int num_pages, float softmax_scale, void *workspace,
                               size_t workspace_bytes, void *stream) {
  return attn_chunk_run(q, k_cache, v_cache, block_tables, max_blocks_per_seq, context_lens, cu_q, total_q,
                        chunk_begin, cu_chunk, tree_parent, out, batch, num_q_heads, num_kv_heads, head_dim,
                        page_size, num_pages, softmax_scale, workspace, workspace_bytes, stream, false,
                        "spec_verify_attn_chunk_run");
}

int spec_verify_attn_chunk_run_vt(const void *q, const void *k_cache, const void *v_cache,
                                  const int32_t *block_tables, int max_blocks_per_seq,
                                  const int32_t *context_lens, const int32_t *cu_q, int total_q,
                                  const int32_t *chunk_begin, const int32_t *cu_chunk, const int32_t *tree_parent,
                                  void *out, int batch, int num_q_heads, int num_kv_heads, int head_dim,
                                  int page_size, int num_pages, float softmax_scale, void *workspace,
                                  size_t workspace_bytes, void *stream) {
  return attn_chunk_run(q, k_cache, v_cache, block_tables, max_blocks_per_seq, context_lens, cu_q, total_q,
                        chunk_begin, cu_chunk, tree_parent, out, batch, num_q_heads, num_kv_heads, head_dim,
                        page_size, num_pages, softmax_scale, workspace, workspace_bytes, stream, true,
                        "spec_verify_attn_chunk_run_vt");
}

int spec_hbm_read_probe(const void *k_cache, const void *v_cache, const int32_t *chunks, int64_t n_chunks,
                        int chunk_bytes, int64_t buffer_chunks, uint32_t *sink, int64_t sink_words,
                        void *stream) {
  if (n_chunks < 0 || buffer_chunks <= 0)
    return fail(SV_ERR_SHAPE, "n_chunks (%lld) must be >= 0 and buffer_chunks (%lld) > 0",
                (long long)n_chunks, (long long)buffer_chunks);
  if (chunk_bytes != 2048 && chunk_bytes != 4096)
    return fail(SV_ERR_UNSUPPORTED, "chunk_bytes %d (supported: 2048, 4096)", chunk_bytes);
  if (sink_words < SV_PROBE_SINK_WORDS)
    return fail(SV_ERR_SHAPE, "sink holds %lld words < %d", (long long)sink_words, SV_PROBE_SINK_WORDS);
  if (n_chunks == 0) return ok();
  if (!k_cache || !v_cache || !chunks || !sink) return fail(SV_ERR_NULL, "spec_hbm_read_probe: a pointer is NULL");
  sv::AttnArgs a;
  int rc = set_grid(&a);
  if (rc != SV_OK) return rc;
  static_assert(sv::kMaxGrid * 256 <= SV_PROBE_SINK_WORDS, "probe sink");
  const int grid = a.grid * sv::kProbeWgPerCu > sv::kMaxGrid ? sv::kMaxGrid : a.grid * sv::kProbeWgPerCu;
  sv::launch_hbm_read_probe(k_cache, v_cache, chunks, n_chunks, chunk_bytes, buffer_chunks, sink, grid,
                            static_cast<hipStream_t>(stream));
  return check_launch("spec_hbm_read_probe");
}

int spec_verify_attn_device_status(const void *workspace, uint32_t *flags, void *stream) {
  return read_status(workspace, 0, flags, stream);
}

int spec_verify_attn_phase_trace(void *host_dst, size_t bytes, int clear, size_t *total_bytes) {
  size_t total = 0;
  const hipError_t e = sv::verify_attn_phase_trace(host_dst, bytes, clear != 0, &total);
  if (total_bytes) *total_bytes = total;
  if (e == hipErrorNotSupported) return fail(SV_ERR_UNSUPPORTED, "not a phase-trace build");
  if (e != hipSuccess) return fail(SV_ERR_HIP, "phase trace: %s", hipGetErrorString(e));
  return ok();
}

size_t spec_accept_workspace_size(int batch, int total_q, int vocab) {
  if (batch < 0 || total_q < 0 || vocab <= 0) return 0;
  return sv::accept_layout(batch, total_q, vocab).total;
}

int spec_accept(const float *logits, int vocab, const int32_t *draft_tokens, const int32_t *cu_q,
                const int32_t *tree_parent, int batch, int total_q, int32_t *target_argmax,
                int32_t *accept_len, int32_t *accepted_path, int32_t *out_tokens, void *workspace,
                size_t workspace_bytes, void *stream) {
  sv::AcceptArgs a;
  bool empty;
  int rc = accept_args(logits, vocab, draft_tokens, cu_q, tree_parent, batch, total_q, target_argmax,
                       accept_len, accepted_path, out_tokens, workspace, workspace_bytes, false, &a, &empty);
  if (rc != SV_OK || empty) return rc;
  sv::launch_accept(a, static_cast<hipStream_t>(stream));
  return check_launch("spec_accept");
}

size_t spec_accept_chunk_workspace_size(int batch, int total_q, int vocab) {
  if (batch < 0 || total_q < 0 || vocab <= 0) return 0;
  size_t m = sv::chunk_layout(batch, 0, vocab).total;
  for (int rows = 1; rows <= total_q; ++rows) {
    const size_t t = sv::chunk_layout(batch, rows, vocab).total;
    if (t > m) m = t;
  }
  return m;
}

int spec_chunk_start(const int32_t *cu_q, int batch, int total_q, int chunk_size,
                     int32_t *chunk_begin, int32_t *cu_chunk, void *stream) {
  if (batch < 0 || total_q < 0 || total_q > (long long)batch * sv::kMaxTokens)
    return fail(SV_ERR_SHAPE, "batch (%d) and total_q (%d) out of range", batch, total_q);
  if (chunk_size <= 0) return fail(SV_ERR_SHAPE, "chunk_size %d must be > 0", chunk_size);
  if (!cu_q || !cu_chunk || (batch > 0 && !chunk_begin))
    return fail(SV_ERR_NULL, "spec_chunk_start: a required pointer is NULL");
  if (overlaps(chunk_begin, (size_t)batch * 4, cu_chunk, (size_t)(batch + 1) * 4) ||
      overlaps(cu_chunk, (size_t)(batch + 1) * 4, cu_q, (size_t)(batch + 1) * 4))
    return fail(SV_ERR_ALIAS, "spec_chunk_start outputs overlap");
  sv::AcceptArgs a;
  memset(&a, 0, sizeof a);
  a.cu_q = cu_q;
  a.batch = batch;
  a.total_q = total_q;
  a.chunk_size = chunk_size;
  a.next_begin = chunk_begin;
  a.next_cu = cu_chunk;
  sv::launch_chunk_start(a, static_cast<hipStream_t>(stream));
  return check_launch("spec_chunk_start");
}

int spec_accept_chunk(const float *logits, int vocab, const int32_t *draft_tokens,
                      const int32_t *cu_q, const int32_t *tree_parent, const int32_t *chunk_begin,
                      const int32_t *cu_chunk, int batch, int total_q, int chunk_size,
                      int32_t *target_argmax, int32_t *accept_len, int32_t *accepted_path,
                      int32_t *out_tokens, int32_t *next_begin, int32_t *next_cu, void *workspace,
                      size_t workspace_bytes, void *stream) {
  if (batch < 0 || total_q < 0)
    return fail(SV_ERR_SHAPE, "batch (%d) and total_q (%d) must be >= 0", batch, total_q);
  if (vocab <= 0) return fail(SV_ERR_SHAPE, "vocab %d must be > 0", vocab);
  if (chunk_size <= 0) return fail(SV_ERR_SHAPE, "chunk_size %d must be > 0", chunk_size);
  if (total_q > (long long)batch * sv::kMaxTokens)
    return fail(SV_ERR_SHAPE, "total_q %d exceeds batch*64", total_q);
  if (batch == 0) return ok();
  if (!cu_q || !chunk_begin || !cu_chunk || !accept_len || !next_begin || !next_cu || !workspace)
    return fail(SV_ERR_NULL, "spec_accept_chunk: a required pointer is NULL");
  if (total_q > 0 && (!draft_tokens || !target_argmax || !accepted_path || !out_tokens))
    return fail(SV_ERR_NULL, "spec_accept_chunk: a required pointer is NULL");
  if (total_q > 0 && !logits) return fail(SV_ERR_NULL, "spec_accept_chunk: logits is NULL");
  // the most rows a chunk can have; the chunk's own count, cu_chunk[batch], is read on the device
  const int rows = (int)std::min<long long>(total_q, (long long)batch * std::min(chunk_size, sv::kMaxTokens));
  const sv::AcceptLayout lay = sv::chunk_layout(batch, rows, vocab);
  if (workspace_bytes < lay.total)
    return fail(SV_ERR_WORKSPACE, "workspace %zu bytes < required %zu", workspace_bytes, lay.total);
  const size_t tb = (size_t)total_q * 4, bb = (size_t)batch * 4, cb = (size_t)(batch + 1) * 4;
  if (overlaps(target_argmax, tb, accepted_path, tb) || overlaps(target_argmax, tb, out_tokens, tb) ||
      overlaps(accepted_path, tb, out_tokens, tb) || overlaps(accept_len, bb, target_argmax, tb) ||
      overlaps(accept_len, bb, accepted_path, tb) || overlaps(accept_len, bb, out_tokens, tb) ||
      overlaps(next_begin, bb, chunk_begin, bb) || overlaps(next_begin, bb, cu_chunk, cb) ||
      overlaps(next_cu, cb, chunk_begin, bb) || overlaps(next_cu, cb, cu_chunk, cb) ||
      overlaps(next_begin, bb, next_cu, cb))
    return fail(SV_ERR_ALIAS, "spec_accept_chunk outputs overlap each other or the chunk inputs");
  sv::AcceptArgs a;
  memset(&a, 0, sizeof a);
  a.logits = logits;
  a.draft = draft_tokens;
  a.cu_q = cu_q;
  a.tree_parent = tree_parent;
  a.target_argmax = target_argmax;
  a.accept_len = accept_len;
  a.accepted_path = accepted_path;
  a.out_tokens = out_tokens;
  a.ws = static_cast<char *>(workspace);
  a.lay = lay;
  a.batch = batch;
  a.total_q = total_q;
  a.vocab = vocab;
  a.rows = rows;
  a.cu_rows = cu_chunk;
  a.chunk_begin = chunk_begin;
  a.chunk_size = chunk_size;
  a.next_begin = next_begin;
  a.next_cu = next_cu;
  sv::launch_accept_chunk(a, static_cast<hipStream_t>(stream));
  return check_launch("spec_accept_chunk");
}

int spec_accept_device_status(const void *workspace, uint32_t *flags, void *stream) {
  return read_status(workspace, 0, flags, stream);
}

}  // extern "C"

namespace {

int compact_call(void *k_cache, void *v_cache, int64_t layer_stride_elems, int num_layers,
                 const int32_t *block_tables, int max_blocks_per_seq, const int32_t *context_lens,
                 const int32_t *cu_q, const int32_t *accepted_path, const int32_t *accept_len,
                 int32_t *new_context_lens, int batch, int total_q, int num_kv_heads, int head_dim,
                 int page_size, int num_pages, void *stream, bool v_transposed, const char *what) {
  sv::CompactArgs a;
  bool empty;
  int rc = compact_args(k_cache, v_cache, layer_stride_elems, num_layers, block_tables, max_blocks_per_seq,
                        context_lens, cu_q, accepted_path, accept_len, new_context_lens, batch, total_q,
                        num_kv_heads, head_dim, page_size, num_pages, &a, &empty);
  if (rc != SV_OK || empty) return rc;
  a.v_transposed = v_transposed;
  sv::launch_kv_compact(a, static_cast<hipStream_t>(stream));
  return check_launch(what);
}

}  // namespace

extern "C" {

int kv_compact(void *k_cache, void *v_cache, int64_t layer_stride_elems, int num_layers,
               const int32_t *block_tables, int max_blocks_per_seq, const int32_t *context_lens,
               const int32_t *cu_q, const int32_t *accepted_path, const int32_t *accept_len,
               int32_t *new_context_lens, int batch, int total_q, int num_kv_heads, int head_dim,
               int page_size, int num_pages, void *stream) {
  return compact_call(k_cache, v_cache, layer_stride_elems, num_layers, block_tables, max_blocks_per_seq,
                      context_lens, cu_q, accepted_path, accept_len, new_context_lens, batch, total_q,
                      num_kv_heads, head_dim, page_size, num_pages, stream, false, "kv_compact");
}

int kv_compact_vt(void *k_cache, void *v_cache, int64_t layer_stride_elems, int num_layers,
                  const int32_t *block_tables, int max_blocks_per_seq, const int32_t *context_lens,
                  const int32_t *cu_q, const int32_t *accepted_path, const int32_t *accept_len,
                  int32_t *new_context_lens, int batch, int total_q, int num_kv_heads, int head_dim,
                  int page_size, int num_pages, void *stream) {
  return compact_call(k_cache, v_cache, layer_stride_elems, num_layers, block_tables, max_blocks_per_seq,
                      context_lens, cu_q, accepted_path, accept_len, new_context_lens, batch, total_q,
                      num_kv_heads, head_dim, page_size, num_pages, stream, true, "kv_compact_vt");
}

size_t spec_accept_stochastic_workspace_size(int batch, int total_q, int vocab) {
  if (batch < 0 || total_q < 0 || vocab <= 0) return 0;
  return sv::stoch_layout(batch, total_q, vocab).total;
}

}  // extern "C"

namespace {

int stochastic_call(const float *logits, const float *draft_probs, int vocab, float temperature,
                    const int32_t *draft_tokens, const int32_t *tree_parent, const float *uniform_accept,
                    const float *uniform_sample, const int32_t *cu_q, int batch, int total_q, int32_t *accept_len,
                    int32_t *accepted_path, int32_t *out_tokens, void *workspace, size_t workspace_bytes,
                    void *stream, const char *name) {
  if (batch < 0 || total_q < 0 || total_q > (long long)batch * sv::kMaxTokens)
    return fail(SV_ERR_SHAPE, "%s: batch (%d) and total_q (%d) out of range", name, batch, total_q);
  if (vocab <= 0) return fail(SV_ERR_SHAPE, "%s: vocab %d must be > 0", name, vocab);
  if (!(temperature > 0.0f) || !isfinite(temperature))
    return fail(SV_ERR_SHAPE, "%s: temperature must be finite and > 0", name);
  if (batch == 0) return ok();
  if (!cu_q || !accept_len || !uniform_sample || !workspace)
    return fail(SV_ERR_NULL, "%s: a required pointer is NULL", name);
  if (total_q > 0 && (!logits || !draft_probs || !draft_tokens || !uniform_accept || !accepted_path ||
                      !out_tokens))
    return fail(SV_ERR_NULL, "%s: a required pointer is NULL", name);
  const sv::StochLayout lay = sv::stoch_layout(batch, total_q, vocab);
  if (workspace_bytes < lay.total)
    return fail(SV_ERR_WORKSPACE, "%s: workspace %zu bytes < required %zu", name, workspace_bytes, lay.total);
  const size_t tb = (size_t)total_q * 4, bb = (size_t)batch * 4;
  if (overlaps(accepted_path, tb, out_tokens, tb) || overlaps(accept_len, bb, accepted_path, tb) ||
      overlaps(accept_len, bb, out_tokens, tb))
    return fail(SV_ERR_ALIAS, "%s outputs overlap", name);
  sv::StochArgs a;
  memset(&a, 0, sizeof a);
  a.logits = logits;
  a.draft_probs = draft_probs;
  a.draft = draft_tokens;
  a.parent = tree_parent;
  a.u = uniform_accept;
  a.w = uniform_sample;
  a.cu_q = cu_q;
  a.accept_len = accept_len;
  a.accepted_path = accepted_path;
  a.out_tokens = out_tokens;
  a.ws = static_cast<char *>(workspace);
  a.lay = lay;
  a.batch = batch;
  a.total_q = total_q;
  a.vocab = vocab;
  a.c = 1.4426950408889634f / temperature;
  sv::launch_stochastic(a, static_cast<hipStream_t>(stream));
  return check_launch(name);
}

}  // namespace

extern "C" {

int spec_accept_stochastic(const float *logits, const float *draft_probs, int vocab,
                           float temperature, const int32_t *draft_tokens,
                           const float *uniform_accept, const float *uniform_sample,
                           const int32_t *cu_q, int batch, int total_q, int32_t *accept_len,
                           int32_t *accepted_path, int32_t *out_tokens, void *workspace,
                           size_t workspace_bytes, void *stream) {
  return stochastic_call(logits, draft_probs, vocab, temperature, draft_tokens, nullptr, uniform_accept,
                         uniform_sample, cu_q, batch, total_q, accept_len, accepted_path, out_tokens, workspace,
                         workspace_bytes, stream, "spec_accept_stochastic");
}

int spec_accept_stochastic_tree(const float *logits, const float *draft_probs, int vocab,
                                float temperature, const int32_t *draft_tokens, const int32_t *tree_parent,
                                const float *uniform_accept, const float *uniform_sample,
                                const int32_t *cu_q, int batch, int total_q, int32_t *accept_len,
                                int32_t *accepted_path, int32_t *out_tokens, void *workspace,
                                size_t workspace_bytes, void *stream) {
  if (batch > 0 && total_q > 0 && !tree_parent)
    return fail(SV_ERR_NULL, "spec_accept_stochastic_tree: tree_parent is NULL");
  return stochastic_call(logits, draft_probs, vocab, temperature, draft_tokens, tree_parent, uniform_accept,
                         uniform_sample, cu_q, batch, total_q, accept_len, accepted_path, out_tokens, workspace,
                         workspace_bytes, stream, "spec_accept_stochastic_tree");
}

int spec_accept_stochastic_device_status(const void *workspace, uint32_t *flags, void *stream) {
  return read_status(workspace, 0, flags, stream);
}

size_t spec_accept_compact_workspace_size(int batch, int total_q, int vocab) {
  if (batch < 0 || total_q < 0 || vocab <= 0) return 0;
  return sv::fused_layout(batch, total_q, vocab).total;
}

}  // extern "C"

namespace {

int accept_compact_call(const float *logits, int vocab, const int32_t *draft_tokens, const int32_t *cu_q,
                        const int32_t *tree_parent, int batch, int total_q, int32_t *target_argmax,
                        int32_t *accept_len, int32_t *accepted_path, int32_t *out_tokens, void *k_cache,
                        void *v_cache, int64_t layer_stride_elems, int num_layers, const int32_t *block_tables,
                        int max_blocks_per_seq, const int32_t *context_lens, int32_t *new_context_lens,
                        int num_kv_heads, int head_dim, int page_size, int num_pages, void *workspace,
                        size_t workspace_bytes, void *stream, bool v_transposed, const char *what) {
  sv::AcceptArgs a;
  sv::CompactArgs c;
  bool empty_a, empty_c;
  int rc = accept_args(logits, vocab, draft_tokens, cu_q, tree_parent, batch, total_q, target_argmax,
                       accept_len, accepted_path, out_tokens, workspace, workspace_bytes, true, &a, &empty_a);
  if (rc != SV_OK) return rc;
  rc = compact_args(k_cache, v_cache, layer_stride_elems, num_layers, block_tables, max_blocks_per_seq,
                    context_lens, cu_q, accepted_path, accept_len, new_context_lens, batch, total_q,
                    num_kv_heads, head_dim, page_size, num_pages, &c, &empty_c);
  if (rc != SV_OK || empty_a || empty_c) return rc;
  const size_t tb = (size_t)total_q * 4, bb = (size_t)batch * 4;
  if (overlaps(new_context_lens, bb, accept_len, bb) || overlaps(new_context_lens, bb, target_argmax, tb) ||
      overlaps(new_context_lens, bb, accepted_path, tb) || overlaps(new_context_lens, bb, out_tokens, tb))
    return fail(SV_ERR_ALIAS, "spec_accept_compact outputs overlap");
  c.v_transposed = v_transposed;
  sv::launch_accept_compact(a, c, static_cast<hipStream_t>(stream));
  return check_launch(what);
}

}  // namespace

extern "C" {

int spec_accept_compact(const float *logits, int vocab, const int32_t *draft_tokens,
                        const int32_t *cu_q, const int32_t *tree_parent, int batch, int total_q,
                        int32_t *target_argmax, int32_t *accept_len, int32_t *accepted_path,
                        int32_t *out_tokens, void *k_cache, void *v_cache,
                        int64_t layer_stride_elems, int num_layers, const int32_t *block_tables,
                        int max_blocks_per_seq, const int32_t *context_lens,
                        int32_t *new_context_lens, int num_kv_heads, int head_dim, int page_size,
                        int num_pages, void *workspace, size_t workspace_bytes, void *stream) {
  return accept_compact_call(logits, vocab, draft_tokens, cu_q, tree_parent, batch, total_q, target_argmax,
                             accept_len, accepted_path, out_tokens, k_cache, v_cache, layer_stride_elems,
                             num_layers, block_tables, max_blocks_per_seq, context_lens, new_context_lens,
                             num_kv_heads, head_dim, page_size, num_pages, workspace, workspace_bytes, stream,
                             false, "spec_accept_compact");
}

int spec_accept_compact_vt(const float *logits, int vocab, const int32_t *draft_tokens,
                           const int32_t *cu_q, const int32_t *tree_parent, int batch, int total_q,
                           int32_t *target_argmax, int32_t *accept_len, int32_t *accepted_path,
                           int32_t *out_tokens, void *k_cache, void *v_cache,
                           int64_t layer_stride_elems, int num_layers, const int32_t *block_tables,
                           int max_blocks_per_seq, const int32_t *context_lens,
                           int32_t *new_context_lens, int num_kv_heads, int head_dim, int page_size,
                           int num_pages, void *workspace, size_t workspace_bytes, void *stream) {
  return accept_compact_call(logits, vocab, draft_tokens, cu_q, tree_parent, batch, total_q, target_argmax,
                             accept_len, accepted_path, out_tokens, k_cache, v_cache, layer_stride_elems,
                             num_layers, block_tables, max_blocks_per_seq, context_lens, new_context_lens,
                             num_kv_heads, head_dim, page_size, num_pages, workspace, workspace_bytes, stream,
                             true, "spec_accept_compact_vt");
}

}  // extern "C"

// ---------------------------------------------------------------------------
// spec_verify_attn with no caller workspace and no allocation: for callers
// that cannot allocate device memory (code under stream capture, tight
// serving loops, harnesses that forbid it).  The attention workspace lives in
// `scratch`, a file-scope device array that every GPU the library runs on
// holds for the life of the process.  In host code `scratch` names a host
// stand-in, not device memory: its device address is taken once per device
// with hipGetSymbolAddress and only that address is handed to kernels.
// ---------------------------------------------------------------------------
namespace {

constexpr size_t kScratchBytes = SV_NOALLOC_SCRATCH_BYTES;

__device__ __align__(256) unsigned char scratch[kScratchBytes];

constexpr int kMaxDevices = 64;
std::atomic<void *> g_scratch_ptr[kMaxDevices];
std::mutex g_scratch_mu;

// device address of `scratch` on the current device (looked up on the first
// call on that device, with that device current)
int scratch_on_current_device(void **ptr) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return fail(SV_ERR_HIP, "hipGetDevice: %s", hipGetErrorString(e));
  if (dev < 0 || dev >= kMaxDevices) return fail(SV_ERR_UNSUPPORTED, "device index %d >= %d", dev, kMaxDevices);
  void *p = g_scratch_ptr[dev].load(std::memory_order_acquire);
  if (p == nullptr) {
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    p = g_scratch_ptr[dev].load(std::memory_order_relaxed);
    if (p == nullptr) {
      e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
      if (e != hipSuccess || p == nullptr)
        return fail(SV_ERR_HIP, "hipGetSymbolAddress(scratch): %s", hipGetErrorString(e));
      g_scratch_ptr[dev].store(p, std::memory_order_release);
    }
  }
  *ptr = p;
  return SV_OK;
}

}  // namespace

extern "C" {

int spec_verify_attn_noalloc(const void *q, const void *k_cache, const void *v_cache,
                             const int32_t *block_tables, int max_blocks_per_seq,
                             const int32_t *context_lens, const int32_t *cu_q,
                             const int32_t *tree_parent, void *out, int batch, int total_q,
                             int num_q_heads, int num_kv_heads, int head_dim, int page_size,
                             int num_pages, float softmax_scale, uint32_t *device_status,
                             void *stream) {
  const size_t need = spec_verify_attn_workspace_size(batch, total_q, num_q_heads, num_kv_heads, head_dim);
  if (need > kScratchBytes)
    return fail(SV_ERR_WORKSPACE,
                "spec_verify_attn_noalloc: these sizes need %zu bytes of workspace, more than the %zu bytes "
                "of its static scratch; use spec_verify_attn with a caller workspace",
                need, kScratchBytes);
  // every host-checkable argument error first, before any HIP call
  sv::AttnArgs a;
  bool empty;
  int rc = attn_common(block_tables, max_blocks_per_seq, context_lens, cu_q, batch, total_q, num_q_heads,
                       num_kv_heads, head_dim, page_size, num_pages, reinterpret_cast<void *>(uintptr_t(256)),
                       kScratchBytes, true, &a, &empty);
  if (rc != SV_OK || empty) return rc;
  rc = attn_data(q, k_cache, v_cache, tree_parent, out, head_dim, page_size, softmax_scale, false, &a);
  if (rc != SV_OK) return rc;
  void *ws = nullptr;
  if ((rc = scratch_on_current_device(&ws)) != SV_OK) return rc;
  rc = attn_run(q, k_cache, v_cache, block_tables, max_blocks_per_seq, context_lens, cu_q, tree_parent, out,
                batch, total_q, num_q_heads, num_kv_heads, head_dim, page_size, num_pages, softmax_scale, ws,
                kScratchBytes, stream, true, false, "spec_verify_attn_noalloc");
  if (rc != SV_OK || device_status == nullptr) return rc;
  // the status word is the first word of the workspace (written by the plan and run)
  const hipError_t e = hipMemcpyAsync(device_status, ws, sizeof(uint32_t), hipMemcpyDeviceToDevice,
                                      static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return fail(SV_ERR_HIP, "spec_verify_attn_noalloc status copy: %s", hipGetErrorString(e));
  return ok();
}

}  // extern "C"

