// In-place compaction of the accepted path's K/V on gfx950.
//
// What is computed (SwiftSpec, "Tree-Aware KV Cache Management": after
// verification only the accepted path's KV is kept and rejected branches are
// dropped; "Fused Latency-Optimized Kernels": the KV update accompanies the
// verification result): for every layer, request i, KV head g and
// k = 0..accept_len_i-1, logical slot L_i + path[k] moves to slot L_i + k.
//
// Launch: grid (batch, layer x head groups), 256 threads.  A workgroup first
// checks the request's path (path[0] = 0, strictly increasing, inside the
// request) and its pages, builds the list of slots that really move
// (path[k] != k; chains have none and exit at once), then for each of its
// (layer, head) pairs reads every source row into registers with 16-byte
// loads, waits at a barrier, and only then writes the destinations.  Reading
// all sources before any write is what makes the in-place move safe: a
// destination slot can be the source of another move.
#include "compact_device.h"

namespace sv {

namespace {

template <int D, bool VT>
__global__ __launch_bounds__(256) void kv_compact_kernel(CompactArgs a) {
  __shared__ int s_dst[kMaxTokens];
  __shared__ int s_src[kMaxTokens];
  __shared__ int s_nmove;
  const int i = blockIdx.x;
  const int tid = threadIdx.x;
  const int o = a.cu_q[i];
  const int c1 = a.cu_q[i + 1];
  const int qn = c1 - o;
  const int L = a.context_lens[i];
  const int n1 = a.accept_len[i];
  const int32_t *bt = a.block_tables + (size_t)i * a.max_blocks;

  if (tid == 0) {
    const bool ok = o >= 0 && c1 >= o && c1 <= a.total_q;
    const int nmove = ok ? compact_moves(a.accepted_path + o, n1, qn, L, bt, a.max_blocks, a.num_pages,
                                         s_src, s_dst)
                         : -1;
    s_nmove = nmove > 0 ? nmove : 0;
    if (blockIdx.y == 0) a.new_context_lens[i] = nmove >= 0 ? L + n1 : -1;
  }
  __syncthreads();
  const int nmove = s_nmove;
  if (nmove == 0) return;
  compact_pairs<D, VT>(a.k_cache, a.v_cache, a.layer_stride, a.num_layers, a.num_kv_heads, bt, s_src, s_dst,
                   nmove, blockIdx.y, gridDim.y);
}

}  // namespace

void launch_kv_compact(const CompactArgs &a, hipStream_t stream) {
  const int pairs = a.num_layers * a.num_kv_heads;
  int gy = 4096 / (a.batch > 0 ? a.batch : 1);
  if (gy > pairs) gy = pairs;
  if (gy > 65535) gy = 65535;
  if (gy < 1) gy = 1;
  dim3 grid(a.batch, gy);
  if (a.head_dim == 128) {
    if (a.v_transposed)
      kv_compact_kernel<128, true><<<grid, 256, 0, stream>>>(a);
    else
      kv_compact_kernel<128, false><<<grid, 256, 0, stream>>>(a);
  } else {
    if (a.v_transposed)
      kv_compact_kernel<64, true><<<grid, 256, 0, stream>>>(a);
    else
      kv_compact_kernel<64, false><<<grid, 256, 0, stream>>>(a);
  }
}

}  // namespace sv
