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

#include "compact_device.h"
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

// (value, lowest index) of the maximum of logits row `row` over slice `split`
// of `splits`; the workgroup (kArgmaxThreads) cooperates, the result is valid
// in thread 0.
__device__ inline Best argmax_slice(const float *logits, int V, int row, int split, int splits) {
  __shared__ float s_v[kArgmaxThreads / 64];
  __shared__ int s_i[kArgmaxThreads / 64];
  // slice bounds, multiples of 4 so 16-byte loads stay aligned when V % 4 == 0
  int per = (V + splits - 1) / splits;
  per = (per + 3) & ~3;
  const int lo = min(V, split * per);
  const int hi = min(V, lo + per);
  const float *x = logits + (size_t)row * V;
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
  Best r{s_v[0], s_i[0]};
#pragma unroll
  for (int w = 1; w < kArgmaxThreads / 64; ++w) r = better(r, Best{s_v[w], s_i[w]});
  return r;
}

__global__ __launch_bounds__(kArgmaxThreads) void argmax_partial_kernel(AcceptArgs a) {
  const int split = blockIdx.x;
  const int row = blockIdx.y;
  const int splits = a.lay.splits;
  if (split == 0 && row == 0 && threadIdx.x == 0)
    reinterpret_cast<int32_t *>(a.ws + a.lay.hdr)[0] = 0;
  if (row >= a.rows) return;  // the grid has one row even when there are none
  int lrow = row;
  if (a.chunk_begin) {  // a chunk's rows, as many as cu_rows says, each a verify token's logits row
    if (row >= a.cu_rows[a.batch]) return;
    lrow = reinterpret_cast<const int32_t *>(a.ws + a.lay.row_map)[row];
    if (lrow < 0 || lrow >= a.total_q) return;  // a malformed chunk: flagged by accept_chunk_kernel
  }
  const Best r = argmax_slice(a.logits, a.vocab, lrow, split, splits);
  if (threadIdx.x == 0) {
    float2 *part = reinterpret_cast<float2 *>(a.ws + a.lay.part);
    part[(size_t)row * splits + split] = make_float2(r.v, __int_as_float(r.i));
  }
}

// Acceptance of request i (rows o..o+q-1, 1 <= q <= 64) from the slice
// partials in the workspace: finishes the row argmaxes, then one wave walks
// the request.  Called by a whole 256-thread workgroup.
template <bool kCoherent = false>
__device__ inline void accept_request(const AcceptArgs &a, int i, int o, int q) {
  __shared__ int s_t[kMaxTokens];
  const int tid = threadIdx.x;
  const int splits = a.lay.splits;
  unsigned *status = reinterpret_cast<unsigned *>(a.ws + a.lay.hdr);
  // 1-2. one thread per row reduces the row's slice partials (splits in index order)
  const float2 *part = reinterpret_cast<const float2 *>(a.ws + a.lay.part);
  if (tid < q) {
    const float2 *pr = part + (size_t)(o + tid) * splits;
    Best b{-INFINITY, -1};
    for (int s0 = 0; s0 < splits; s0 += 8) {
      float2 p[8];  // eight independent loads in flight, then reduced in index order
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        const float2 *src = pr + min(s0 + u, splits - 1);
        if constexpr (kCoherent) {  // written by other workgroups of the same launch
          const uint64_t bits = __hip_atomic_load(reinterpret_cast<const uint64_t *>(src), __ATOMIC_RELAXED,
                                                  __HIP_MEMORY_SCOPE_AGENT);
          p[u] = __builtin_bit_cast(float2, bits);
        } else {
          p[u] = *src;
        }
      }
#pragma unroll
      for (int u = 0; u < 8; ++u)
        if (s0 + u < splits) b = better(b, Best{p[u].x, __float_as_int(p[u].y)});
    }
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

__global__ __launch_bounds__(256) void accept_kernel(AcceptArgs a) {
  const int i = blockIdx.x;
  const int tid = threadIdx.x;
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
  accept_request(a, i, o, q);
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
      (a.cu_q[0] != 0 || a.cu_q[a.batch] != a.total_q || a.cu_rows[0] != 0 || a.cu_rows[a.batch] > a.rows))
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

// The verify token (logits row) of each of a chunk's rows, cu_q[i] +
// chunk_begin[i] + r for row cu_rows[i] + r (one workgroup); rows of a
// malformed chunk get -1 (accept_chunk_kernel reports it).
__global__ __launch_bounds__(kPlanThreads) void chunk_rows_kernel(AcceptArgs a) {
  int32_t *map = reinterpret_cast<int32_t *>(a.ws + a.lay.row_map);
  for (int i = threadIdx.x; i < a.batch; i += kPlanThreads) {
    const int r0 = a.cu_rows[i], r1 = a.cu_rows[i + 1];
    const int o = a.cu_q[i], q = a.cu_q[i + 1] - o, s0 = a.chunk_begin[i];
    if (r0 < 0 || r1 < r0 || r1 > a.rows) continue;
    const bool ok = o >= 0 && q >= 0 && o + q <= a.total_q && s0 >= 0 && s0 + (r1 - r0) <= q;
    for (int r = r0; r < r1; ++r) map[r] = ok ? o + s0 + (r - r0) : -1;
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

// --------------------------------------------------------------------------
// Acceptance and compaction in one launch (SwiftSpec, "Fused Latency-
// Optimized Kernels": the verification result and the KV update come out of
// one kernel).
//
// The work items, in order: the argmax slices (row, split), which never wait;
// the walk of each request, which waits until the slices of its rows are
// done; then, for draft trees, the compaction groups (request, every
// groups-th (layer, head) pair), each waiting until its request's walk is
// done.  The slices are workgroups 0 .. n_slices-1; every later workgroup
// takes its item from a ticket counter, so an item only waits for items that
// come before it and were taken by workgroups already running (the slices
// have lower workgroup indices, which the dispatcher starts first).  Every
// wait is bounded: one that runs out sets SV_DEV_SYNC_TIMEOUT and makes the
// remaining waits give up, so the launch always ends.  The last waiting item
// to finish waits until every slice has finished too and then zeroes all
// that the call wrote to the workspace (counters, slice partials, move
// lists): the counters of the next call lie at offsets that depend on its
// shape, so the workspace must be all zero, not only where this call keeps
// its counters.
// --------------------------------------------------------------------------
constexpr int kSpinLimit = 1 << 21;
constexpr int kFusedCompactItems = 128;

// Data passed between workgroups of the launch (slice partials, move lists,
// flags) is written and read only with agent-scope atomic loads and stores,
// which reach the coherent level directly; a producer waits until its data
// stores are complete before it raises a flag.  No acquire or release
// fence is needed, so no waiting workgroup invalidates or writes back the
// L2 of its XCD while the slices stream.
__device__ inline void store_coherent(int32_t *p, int v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ inline int load_coherent(const int32_t *p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
// this thread's stores have completed before anything it issues next
__device__ inline void stores_complete() {
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
  __builtin_amdgcn_s_waitcnt(0);
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
}

// thread-level bounded wait until *p >= need.  The first wait that runs out
// raises *abort, and every later wait of the launch gives up at once, so a
// broken launch still ends quickly.
__device__ inline bool wait_at_least(int32_t *p, int need, int32_t *abort) {
  for (int it = 0; it < kSpinLimit; ++it) {
    if (load_coherent(p) >= need) return true;
    if (load_coherent(abort) != 0) return false;
    __builtin_amdgcn_s_sleep(32);  // about 2048 cycles between polls
  }
  store_coherent(abort, 1);
  return false;
}

// eight workgroups per CU for the streaming slices (the compaction items
// then keep part of their move buffer in scratch)
// wave-level bounded wait (called by all 64 lanes of one wave): lane r
// waits until arrive[r] >= need for r < n; true once all are there
__device__ inline bool wave_wait_all(const int32_t *arrive, int n, int need, int32_t *abort) {
  const int lane = threadIdx.x & 63;
  bool ready = lane >= n;
  for (int it = 0; it < kSpinLimit; ++it) {
    if (!ready) ready = load_coherent(arrive + lane) >= need;
    if (__all(ready)) return true;
    if (load_coherent(abort) != 0) return false;
    __builtin_amdgcn_s_sleep(32);
  }
  store_coherent(abort, 1);
  return false;
}

template <int D, bool VT>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(8))) void accept_compact_kernel(AcceptArgs a, CompactArgs c, int n_slices,
                                                             int groups, int n_total) {
  __shared__ int s_item, s_flag, s_nmove;
  __shared__ int s_src[kMaxTokens], s_dst[kMaxTokens];
  int32_t *hdr = reinterpret_cast<int32_t *>(a.ws + a.lay.hdr);
  unsigned *status = reinterpret_cast<unsigned *>(hdr);
  int32_t *arrive = reinterpret_cast<int32_t *>(a.ws + a.lay.arrive);
  int32_t *done = reinterpret_cast<int32_t *>(a.ws + a.lay.done);
  int32_t *moves = reinterpret_cast<int32_t *>(a.ws + a.lay.moves);
  const int tid = threadIdx.x;
  const int splits = a.lay.splits;
  int32_t *abort = &hdr[5];
  // The slices (which never wait) are workgroups 0 .. n_slices-1; the other
  // workgroups take the items that wait from a ticket counter, in order.
  int t = blockIdx.x;
  if (t >= n_slices) {
    if (tid == 0) s_item = n_slices + __hip_atomic_fetch_add(&hdr[2], 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    __syncthreads();
    t = s_item;
    if (t < n_slices || t >= n_total) {  // counters not cleared (workspace not zero-filled)
      if (tid == 0) {
        __hip_atomic_store(abort, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        // the bit must land after item 0 has cleared the status word; item 0
        // is a slice, which never waits, so this wait ends
        for (int it = 0; it < kSpinLimit && load_coherent(&hdr[4]) == 0; ++it) __builtin_amdgcn_s_sleep(32);
        atomicOr(status, SV_DEV_SYNC_TIMEOUT);
      }
      t = n_total;  // no item
    }
  }
  if (t == 0 && tid == 0) {  // the first item clears the status word for this call
    store_coherent(&hdr[0], 0);
    stores_complete();
    store_coherent(&hdr[4], 1);
  }
  if (t < n_slices) {
    // 1. one argmax slice
    const int row = t / splits, split = t - (t / splits) * splits;
    const Best r = argmax_slice(a.logits, a.vocab, row, split, splits);
    if (tid == 0) {
      uint64_t *part = reinterpret_cast<uint64_t *>(a.ws + a.lay.part);
      __hip_atomic_store(part + (size_t)row * splits + split,
                         __builtin_bit_cast(uint64_t, make_float2(r.v, __int_as_float(r.i))), __ATOMIC_RELAXED,
                         __HIP_MEMORY_SCOPE_AGENT);
      stores_complete();
      __hip_atomic_fetch_add(&arrive[row], 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
  } else if (t < n_slices + a.batch) {
    // 2. the walk of request i, then its move list
    const int i = t - n_slices;
    const int o = a.cu_q[i], c1 = a.cu_q[i + 1], q = c1 - o;
    const bool valid = o >= 0 && c1 >= o && c1 <= a.total_q && q <= kMaxTokens;
    if (tid < 64) {  // one wave: the status word is cleared and every row's slices are done
      bool ok = true;
      if (tid == 0) ok = wait_at_least(&hdr[4], 1, abort);
      ok = __shfl(ok, 0);
      if (ok && valid) ok = wave_wait_all(arrive + o, q, splits, abort);
      if (tid == 0) s_flag = ok;
    }
    __syncthreads();
    if (tid == 0) {
      const bool ok = s_flag;
      if (!ok) atomicOr(status, SV_DEV_SYNC_TIMEOUT);
      if (!valid)
        atomicOr(status, q > kMaxTokens && o >= 0 && c1 <= a.total_q ? SV_DEV_TOO_MANY_TOKENS : SV_DEV_BAD_CU_Q);
      if (i == 0 && (a.cu_q[0] != 0 || a.cu_q[a.batch] != a.total_q)) atomicOr(status, SV_DEV_BAD_CU_Q);
      s_flag = ok && valid;
    }
    __syncthreads();
    const bool go = s_flag;
    if (go && q > 0) accept_request<true>(a, i, o, q);
    __syncthreads();
    if (tid == 0) {
      if (!go || q == 0) a.accept_len[i] = 0;
      __threadfence_block();
      const int32_t *bt = c.block_tables + (size_t)i * c.max_blocks;
      const int L = c.context_lens[i];
      int *mv = moves + (size_t)i * kFusedMoveWords;
      const int nmove = go ? compact_moves(a.accepted_path + o, a.accept_len[i], q, L, bt, c.max_blocks,
                                           c.num_pages, s_src, s_dst)
                           : -1;
      store_coherent(&mv[0], nmove);
      for (int m = 0; m < nmove; ++m) {
        store_coherent(&mv[1 + m], s_src[m]);
        store_coherent(&mv[1 + (kMaxTokens - 1) + m], s_dst[m]);
      }
      c.new_context_lens[i] = nmove >= 0 ? L + a.accept_len[i] : -1;
      stores_complete();
      store_coherent(&done[i], 1);
    }
  } else if (t < n_total) {
    // 3. one compaction group of request i (trees only)
    const int ci = t - n_slices - a.batch;
    const int i = ci / groups, g = ci - (ci / groups) * groups;
    if (tid < 64) {  // one wave: wait for the walk, then lane m fetches move m
      bool ok = true;
      if (tid == 0) ok = wait_at_least(&done[i], 1, abort);
      ok = __shfl(ok, 0);
      if (!ok && tid == 0) atomicOr(status, SV_DEV_SYNC_TIMEOUT);
      const int *mv = moves + (size_t)i * kFusedMoveWords;
      const int n = ok ? load_coherent(&mv[0]) : 0;
      if (tid < n) {
        s_src[tid] = load_coherent(&mv[1 + tid]);
        s_dst[tid] = load_coherent(&mv[1 + (kMaxTokens - 1) + tid]);
      }
      if (tid == 0) s_nmove = n > 0 ? n : 0;
    }
    __syncthreads();
    if (s_nmove > 0)
      compact_pairs<D, VT>(c.k_cache, c.v_cache, c.layer_stride, c.num_layers, c.num_kv_heads,
                       c.block_tables + (size_t)i * c.max_blocks, s_src, s_dst, s_nmove, g, groups);
  }
  // The last waiting item to finish zeroes what the call wrote.  Only the
  // waiting items count themselves out (one atomic each); the slices are
  // waited for here through their per-row arrival counts, which in a valid
  // call are already complete (every row's walk waited for them) and
  // otherwise (bad cu_q, a wait that gave up) soon are: slices never wait.
  if (blockIdx.x < n_slices) return;
  __syncthreads();
  if (tid == 0)
    s_flag = __hip_atomic_fetch_add(&hdr[3], 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) ==
             n_total - n_slices - 1;
  __syncthreads();
  if (!s_flag) return;
  bool slices_done = true;
  for (int r = tid; r < a.total_q && slices_done; r += 256) {
    int it = 0;
    while (it < kSpinLimit && load_coherent(arrive + r) < splits) {
      __builtin_amdgcn_s_sleep(32);
      ++it;
    }
    slices_done = it < kSpinLimit;
  }
  if (!__syncthreads_and(slices_done)) {
    // a slice never arrived: the counters were not zero at the start of the
    // call; leave them for the caller to zero-fill again
    if (tid == 0) atomicOr(status, SV_DEV_SYNC_TIMEOUT);
    return;
  }
  uint64_t *part = reinterpret_cast<uint64_t *>(a.ws + a.lay.part);
  for (size_t e = tid; e < (size_t)a.total_q * splits; e += 256) part[e] = 0;
  for (int r = tid; r < a.total_q; r += 256) arrive[r] = 0;
  for (int i = tid; i < a.batch; i += 256) {
    done[i] = 0;
    int *mv = moves + (size_t)i * kFusedMoveWords;
    const int nmove = max(0, min(load_coherent(&mv[0]), kMaxTokens - 1));
    for (int m = 0; m < nmove; ++m) {
      mv[1 + m] = 0;
      mv[1 + (kMaxTokens - 1) + m] = 0;
    }
    mv[0] = 0;
  }
  if (tid == 0) {
    hdr[2] = 0;
    hdr[3] = 0;
    hdr[4] = 0;
    hdr[5] = 0;
  }
}

}  // namespace

void launch_accept(const AcceptArgs &a, hipStream_t stream) {
  dim3 grid(a.lay.splits, a.rows > 0 ? a.rows : 1);
  argmax_partial_kernel<<<grid, kArgmaxThreads, 0, stream>>>(a);
  accept_kernel<<<a.batch, 256, 0, stream>>>(a);
}

void launch_accept_chunk(const AcceptArgs &a, hipStream_t stream) {
  chunk_rows_kernel<<<1, kPlanThreads, 0, stream>>>(a);
  dim3 grid(a.lay.splits, a.rows > 0 ? a.rows : 1);
  argmax_partial_kernel<<<grid, kArgmaxThreads, 0, stream>>>(a);
  accept_chunk_kernel<<<a.batch, 256, 0, stream>>>(a);
  chunk_scan_kernel<<<1, kPlanThreads, 0, stream>>>(a, false);
}

void launch_chunk_start(const AcceptArgs &a, hipStream_t stream) {
  chunk_scan_kernel<<<1, kPlanThreads, 0, stream>>>(a, true);
}

}  // namespace sv

namespace sv {

void launch_accept_compact(const AcceptArgs &a, const CompactArgs &c, hipStream_t stream) {
  const int n_slices = a.total_q * a.lay.splits;
  const int pairs = c.num_layers * c.num_kv_heads;
  int groups = 0;
  if (a.tree_parent != nullptr && pairs > 0) {
    // fewer, longer compaction items than kv_compact's grid: each item takes a
    // ticket and counts itself out with an atomic on one address
    groups = kFusedCompactItems / (a.batch > 0 ? a.batch : 1);
    if (groups > pairs) groups = pairs;
    if (groups < 1) groups = 1;
  }
  const int n_total = n_slices + a.batch + a.batch * groups;
  if (c.head_dim == 128) {
    if (c.v_transposed)
      accept_compact_kernel<128, true><<<n_total, 256, 0, stream>>>(a, c, n_slices, groups, n_total);
    else
      accept_compact_kernel<128, false><<<n_total, 256, 0, stream>>>(a, c, n_slices, groups, n_total);
  } else {
    if (c.v_transposed)
      accept_compact_kernel<64, true><<<n_total, 256, 0, stream>>>(a, c, n_slices, groups, n_total);
    else
      accept_compact_kernel<64, false><<<n_total, 256, 0, stream>>>(a, c, n_slices, groups, n_total);
  }
}

}  // namespace sv
