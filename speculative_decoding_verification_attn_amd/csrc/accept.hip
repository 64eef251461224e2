// Greedy acceptance of drafted tokens on gfx950.
//
// What is computed (DSpark, glossary "Speculative Decoding": the longest
// matching prefix of the draft is accepted; SwiftSpec, "Tree-Aware KV Cache
// Management" and "Fused Latency-Optimized Kernels": for a draft tree the
// accepted root path is kept and the result goes back as a short message):
//   t[r]      = lowest index of the maximum of logits row r (full vocabulary)
//   accepted  = chain: longest prefix with draft[j] == t[j-1];
//               tree: deepest node whose every root-path edge matches
//               (draft[a] == t[parent[a]]), lowest index among equals.
//
// Two launches:
//   argmax_partial_kernel  grid (splits, rows): each workgroup streams one slice
//                          of one logits row with 16-byte loads and reduces
//                          (value, index) pairs with wave shuffles;
//   accept_kernel          one workgroup per request: reduces the slice
//                          partials of its rows, then one wave walks the
//                          request (<= 64 tokens, one lane per token) with a
//                          ballot of edge matches against ancestor masks.
#include <limits.h>

#include "sv_device.h"
#include "sv_internal.h"

namespace sv {

namespace {

struct Best {
  float v;
  int i;  // -1 = empty
};

// larger value wins; equal values: lower index wins (IEEE ==, so -0 == +0)
__device__ inline Best better(Best a, Best b) {
  if (b.i < 0) return a;
  if (a.i < 0) return b;
  if (b.v > a.v || (b.v == a.v && b.i < a.i)) return b;
  return a;
}

__device__ inline Best wave_best(Best x) {
#pragma unroll
  for (int d = 32; d >= 1; d >>= 1) {
    Best y;
    y.v = __shfl_xor(x.v, d);
    y.i = __shfl_xor(x.i, d);
    x = better(x, y);
  }
  return x;
}

__global__ __launch_bounds__(kArgmaxThreads) void argmax_partial_kernel(AcceptArgs a) {
  __shared__ float s_v[kArgmaxThreads / 64];
  __shared__ int s_i[kArgmaxThreads / 64];
  const int split = blockIdx.x;
  const int row = blockIdx.y;
  const int splits = a.lay.splits;
  const int V = a.vocab;
  if (split == 0 && row == 0 && threadIdx.x == 0)
    reinterpret_cast<int32_t *>(a.ws + a.lay.hdr)[0] = 0;
  if (row >= a.rows) return;  // the grid has one row even when there are none
  // slice bounds, multiples of 4 so 16-byte loads stay aligned when V % 4 == 0
  int per = (V + splits - 1) / splits;
  per = (per + 3) & ~3;
  const int lo = min(V, split * per);
  const int hi = min(V, lo + per);
  const float *x = a.logits + (size_t)row * V;
  Best b{-INFINITY, -1};
  if ((V & 3) == 0) {
    // each thread walks its float4s in increasing index order; strict '>'
    // keeps the lowest index among equal values within the thread.  Every
    // load instruction covers 1 KB of the row contiguously and no byte is
    // read twice, so the loads are nontemporal (streamed, not kept).
    const int nv = (hi - lo) >> 2;
    const float4v *x4 = reinterpret_cast<const float4v *>(x + lo);
    constexpr int U = 4;
    int k = threadIdx.x;
    for (; k + (U - 1) * kArgmaxThreads < nv; k += U * kArgmaxThreads) {
      float4v v[U];
#pragma unroll
      for (int u = 0; u < U; ++u) v[u] = __builtin_nontemporal_load(x4 + k + u * kArgmaxThreads);
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const int base = lo + 4 * (k + u * kArgmaxThreads);
        if (b.i < 0 || v[u].x > b.v) { b.v = v[u].x; b.i = base; }
        if (v[u].y > b.v) { b.v = v[u].y; b.i = base + 1; }
        if (v[u].z > b.v) { b.v = v[u].z; b.i = base + 2; }
        if (v[u].w > b.v) { b.v = v[u].w; b.i = base + 3; }
      }
    }
    for (; k < nv; k += kArgmaxThreads) {
      const float4v v = __builtin_nontemporal_load(x4 + k);
      const int base = lo + 4 * k;
      if (b.i < 0 || v.x > b.v) { b.v = v.x; b.i = base; }
      if (v.y > b.v) { b.v = v.y; b.i = base + 1; }
      if (v.z > b.v) { b.v = v.z; b.i = base + 2; }
      if (v.w > b.v) { b.v = v.w; b.i = base + 3; }
    }
  } else {
    for (int k = lo + threadIdx.x; k < hi; k += kArgmaxThreads) {
      const float v = x[k];
      if (b.i < 0 || v > b.v) { b.v = v; b.i = k; }
    }
  }
  b = wave_best(b);
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  if (lane == 0) {
    s_v[wave] = b.v;
    s_i[wave] = b.i;
  }
  __syncthreads();
  if (threadIdx.x == 0) {
    Best r{s_v[0], s_i[0]};
#pragma unroll
    for (int w = 1; w < kArgmaxThreads / 64; ++w) r = better(r, Best{s_v[w], s_i[w]});
    float2 *part = reinterpret_cast<float2 *>(a.ws + a.lay.part);
    part[(size_t)row * splits + split] = make_float2(r.v, __int_as_float(r.i));
  }
}

__global__ __launch_bounds__(256) void accept_kernel(AcceptArgs a) {
  __shared__ float s_pv[kMaxTokens * kArgmaxMaxSplits];
  __shared__ int s_pi[kMaxTokens * kArgmaxMaxSplits];
  __shared__ int s_t[kMaxTokens];
  const int i = blockIdx.x;
  const int tid = threadIdx.x;
  const int splits = a.lay.splits;
  unsigned *status = reinterpret_cast<unsigned *>(a.ws + a.lay.hdr);
  const int o = a.cu_q[i];
  const int c1 = a.cu_q[i + 1];
  const int q = c1 - o;
  if (o < 0 || c1 < o || c1 > a.total_q || q > kMaxTokens) {
    if (tid == 0) {
      atomicOr(status, q > kMaxTokens && o >= 0 && c1 <= a.total_q ? SV_DEV_TOO_MANY_TOKENS
                                                                   : SV_DEV_BAD_CU_Q);
      a.accept_len[i] = 0;
    }
    return;
  }
  if (i == 0 && tid == 0 && (a.cu_q[0] != 0 || a.cu_q[a.batch] != a.total_q))
    atomicOr(status, SV_DEV_BAD_CU_Q);
  if (q == 0) {
    if (tid == 0) a.accept_len[i] = 0;
    return;
  }
  // 1. gather the slice partials of this request's rows
  const float2 *part = reinterpret_cast<const float2 *>(a.ws + a.lay.part);
  const int np = q * splits;
  for (int k = tid; k < np; k += 256) {
    const float2 p = part[(size_t)o * splits + k];
    s_pv[k] = p.x;
    s_pi[k] = __float_as_int(p.y);
  }
  __syncthreads();
  // 2. one thread per row finishes the argmax (splits in index order)
  if (tid < q) {
    Best b{s_pv[tid * splits], s_pi[tid * splits]};
    for (int s = 1; s < splits; ++s) b = better(b, Best{s_pv[tid * splits + s], s_pi[tid * splits + s]});
    s_t[tid] = b.i;
    a.target_argmax[o + tid] = b.i;
  }
  __syncthreads();
  if (tid >= 64) return;
  // 3. the walk: lane j is verify token j
  const int j = tid;
  bool parents_ok;
  const uint64_t anc = ancestor_mask(a.tree_parent, o, q, j, &parents_ok);
  if (!parents_ok && j == 0) atomicOr(status, SV_DEV_BAD_PARENT);
  int par = -1;
  if (j < q && j > 0) par = a.tree_parent ? a.tree_parent[o + j] : j - 1;
  if (par < 0 || par >= j) par = -1;
  const bool match = j < q && par >= 0 && a.draft[o + j] == s_t[par];
  const uint64_t matched = __ballot(match) | 1ull;
  const bool accepted = j < q && (anc & ~matched) == 0ull;
  const int depth = __popcll(anc) - 1;
  // key: deeper first, then lower index
  int key = accepted ? ((depth << 6) | (63 - j)) : -1;
#pragma unroll
  for (int d = 32; d >= 1; d >>= 1) key = max(key, __shfl_xor(key, d));
  const int best = 63 - (key & 63);
  const int n = key >> 6;
  const uint64_t path_mask = __shfl(anc, best);
  if (j < q) {
    if ((path_mask >> j) & 1ull) {
      const int rank = __popcll(path_mask & ((1ull << j) - 1ull));
      a.accepted_path[o + rank] = j;
      a.out_tokens[o + rank] = s_t[j];
    }
    if (j > n) {
      a.accepted_path[o + j] = -1;
      a.out_tokens[o + j] = -1;
    }
  }
  if (j == 0) a.accept_len[i] = n + 1;
}

// --------------------------------------------------------------------------
// Chunked acceptance with early pruning (FASER, "Early Token Pruning": the
// verification is split into chunks of verify tokens, and at every chunk
// boundary the tokens behind an already rejected prefix are dropped).
//
// One workgroup per request.  The argmaxes of the chunk's rows complete the
// target tokens of verify tokens [0, e), e = chunk_begin + rows.  An edge
// (parent p -> node j) is decided once p < e.  A node is still alive if no
// decided edge on its root path mismatches; the request goes on with its
// next chunk [e, e + chunk_size) while some node >= e is alive, and otherwise
// ends here with the same result as unchunked acceptance: every node >= e is
// dead (so not accepted) and every edge into the nodes < e is decided.
// --------------------------------------------------------------------------
__global__ __launch_bounds__(256) void accept_chunk_kernel(AcceptArgs a) {
  __shared__ float s_pv[kMaxTokens * kArgmaxMaxSplits];
  __shared__ int s_pi[kMaxTokens * kArgmaxMaxSplits];
  __shared__ int s_t[kMaxTokens];
  const int i = blockIdx.x;
  const int tid = threadIdx.x;
  const int splits = a.lay.splits;
  unsigned *status = reinterpret_cast<unsigned *>(a.ws + a.lay.hdr);
  int32_t *next_len = reinterpret_cast<int32_t *>(a.ws + a.lay.next_len);
  const int o = a.cu_q[i], c1 = a.cu_q[i + 1], q = c1 - o;
  const int r0 = a.cu_rows[i], r1 = a.cu_rows[i + 1], c = r1 - r0;
  const int s0 = a.chunk_begin[i];
  const bool bad_full = o < 0 || c1 < o || c1 > a.total_q;
  if (bad_full || q > kMaxTokens || r0 < 0 || r1 < r0 || r1 > a.rows || s0 < 0 || s0 + c > q) {
    if (tid == 0) {
      atomicOr(status, !bad_full && q > kMaxTokens ? SV_DEV_TOO_MANY_TOKENS : SV_DEV_BAD_CU_Q);
      next_len[i] = 0;
      a.next_begin[i] = 0;
    }
    return;
  }
  if (i == 0 && tid == 0 &&
      (a.cu_q[0] != 0 || a.cu_q[a.batch] != a.total_q || a.cu_rows[0] != 0 || a.cu_rows[a.batch] != a.rows))
    atomicOr(status, SV_DEV_BAD_CU_Q);
  if (c == 0) {  // not in this chunk: finished earlier (or q == 0)
    if (tid == 0) {
      next_len[i] = 0;
      a.next_begin[i] = s0;
      if (q == 0) a.accept_len[i] = 0;
    }
    return;
  }
  // 1. the chunk rows' argmaxes; earlier tokens' come from earlier chunks
  const float2 *part = reinterpret_cast<const float2 *>(a.ws + a.lay.part);
  const int np = c * splits;
  for (int k = tid; k < np; k += 256) {
    const float2 p = part[(size_t)r0 * splits + k];
    s_pv[k] = p.x;
    s_pi[k] = __float_as_int(p.y);
  }
  for (int j = tid; j < s0; j += 256) s_t[j] = a.target_argmax[o + j];
  __syncthreads();
  if (tid < c) {
    Best b{s_pv[tid * splits], s_pi[tid * splits]};
    for (int sp = 1; sp < splits; ++sp) b = better(b, Best{s_pv[tid * splits + sp], s_pi[tid * splits + sp]});
    s_t[s0 + tid] = b.i;
    a.target_argmax[o + s0 + tid] = b.i;
  }
  __syncthreads();
  if (tid >= 64) return;
  // 2. decided edges, alive nodes
  const int j = tid;
  const int e = s0 + c;
  bool parents_ok;
  const uint64_t anc = ancestor_mask(a.tree_parent, o, q, j, &parents_ok);
  if (!parents_ok && j == 0) atomicOr(status, SV_DEV_BAD_PARENT);
  int par = -1;
  if (j < q && j > 0) par = a.tree_parent ? a.tree_parent[o + j] : j - 1;
  if (par < 0 || par >= j) par = -1;
  const bool mismatch = j < q && par >= 0 && par < e && a.draft[o + j] != s_t[par];
  const uint64_t bad = __ballot(mismatch);
  const bool path_ok = j < q && (anc & bad) == 0ull;
  const bool go_on = e < q && __ballot(path_ok && j >= e) != 0ull;
  if (go_on) {
    if (j == 0) {
      next_len[i] = min(a.chunk_size, q - e);
      a.next_begin[i] = e;
    }
    return;
  }
  // 3. the request ends: deepest accepted node among [0, e)
  const bool accepted = j < e && path_ok;
  const int depth = __popcll(anc) - 1;
  int key = accepted ? ((depth << 6) | (63 - j)) : -1;
#pragma unroll
  for (int d = 32; d >= 1; d >>= 1) key = max(key, __shfl_xor(key, d));
  const int best = 63 - (key & 63);
  const int n = key >> 6;
  const uint64_t path_mask = __shfl(anc, best);
  if (j < q) {
    if ((path_mask >> j) & 1ull) {
      const int rank = __popcll(path_mask & ((1ull << j) - 1ull));
      a.accepted_path[o + rank] = j;
      a.out_tokens[o + rank] = s_t[j];
    }
    if (j > n) {
      a.accepted_path[o + j] = -1;
      a.out_tokens[o + j] = -1;
    }
  }
  if (j == 0) {
    a.accept_len[i] = n + 1;
    next_len[i] = 0;
    a.next_begin[i] = e;
  }
}

// Packing of the next chunk: next_cu = exclusive prefix sums of the rows per
// request (one workgroup).  start: the first chunk of a step, rows
// min(chunk_size, q_i) from token 0.
__global__ __launch_bounds__(kPlanThreads) void chunk_scan_kernel(AcceptArgs a, bool start) {
  __shared__ int s_scan[16];
  const int32_t *next_len = reinterpret_cast<const int32_t *>(a.ws + a.lay.next_len);
  int carry = 0;
  for (int base = 0; base < a.batch; base += kPlanThreads) {
    const int i = base + threadIdx.x;
    int len = 0;
    if (i < a.batch) {
      if (start) {
        const int q = a.cu_q[i + 1] - a.cu_q[i];
        len = max(0, min(a.chunk_size, min(q, kMaxTokens)));
        a.next_begin[i] = 0;
      } else {
        len = next_len[i];
      }
    }
    int total;
    const int ex = block_excl_scan_1024<int>(len, s_scan, &total);
    if (i < a.batch) a.next_cu[i] = carry + ex;
    carry += total;
  }
  if (threadIdx.x == 0) a.next_cu[a.batch] = carry;
}

}  // namespace

void launch_accept(const AcceptArgs &a, hipStream_t stream) {
  dim3 grid(a.lay.splits, a.rows > 0 ? a.rows : 1);
  argmax_partial_kernel<<<grid, kArgmaxThreads, 0, stream>>>(a);
  accept_kernel<<<a.batch, 256, 0, stream>>>(a);
}

void launch_accept_chunk(const AcceptArgs &a, hipStream_t stream) {
  dim3 grid(a.lay.splits, a.rows > 0 ? a.rows : 1);
  argmax_partial_kernel<<<grid, kArgmaxThreads, 0, stream>>>(a);
  accept_chunk_kernel<<<a.batch, 256, 0, stream>>>(a);
  chunk_scan_kernel<<<1, kPlanThreads, 0, stream>>>(a, false);
}

void launch_chunk_start(const AcceptArgs &a, hipStream_t stream) {
  chunk_scan_kernel<<<1, kPlanThreads, 0, stream>>>(a, true);
}

}  // namespace sv
