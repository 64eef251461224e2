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
#include "sv_device.h"
#include "sv_internal.h"

namespace sv {

namespace {

template <int D>
__global__ __launch_bounds__(256) void kv_compact_kernel(CompactArgs a) {
  constexpr int CPR = D / 8;                               // 16-byte chunks per row
  constexpr int MAXU = ((kMaxTokens - 1) * CPR * 2 + 255) / 256;  // units per thread
  __shared__ int s_dst[kMaxTokens];
  __shared__ int s_src[kMaxTokens];
  __shared__ int s_nmove;
  __shared__ int s_ok;
  const int i = blockIdx.x;
  const int tid = threadIdx.x;
  const int o = a.cu_q[i];
  const int c1 = a.cu_q[i + 1];
  const int qn = c1 - o;
  const int L = a.context_lens[i];
  const int n1 = a.accept_len[i];
  const int32_t *bt = a.block_tables + (size_t)i * a.max_blocks;

  if (tid == 0) {
    bool ok = o >= 0 && c1 >= o && c1 <= a.total_q && qn <= kMaxTokens && L >= 0 && n1 >= 0 &&
              n1 <= qn;
    if (ok && ((long long)L + qn + kPage - 1) / kPage > a.max_blocks) ok = false;
    int prev = -1, nmove = 0;
    for (int k = 0; ok && k < n1; ++k) {
      const int pk = a.accepted_path[o + k];
      if (pk < k || pk >= qn || pk <= prev || (k == 0 && pk != 0)) {
        ok = false;
        break;
      }
      prev = pk;
      if (pk != k) {
        s_dst[nmove] = L + k;
        s_src[nmove] = L + pk;
        ++nmove;
      }
    }
    // every page a move touches must be a real page
    for (int m = 0; ok && m < nmove; ++m) {
      const int pd = bt[s_dst[m] / kPage], ps = bt[s_src[m] / kPage];
      if (pd < 0 || pd >= a.num_pages || ps < 0 || ps >= a.num_pages) ok = false;
    }
    s_ok = ok;
    s_nmove = ok ? nmove : 0;
    if (blockIdx.y == 0) a.new_context_lens[i] = ok ? L + n1 : -1;
  }
  __syncthreads();
  const int nmove = s_nmove;
  if (nmove == 0) return;

  const size_t page_stride = (size_t)a.num_kv_heads * kPage * D;
  const int units = nmove * CPR * 2;  // (move, chunk, K|V)
  const int pairs = a.num_layers * a.num_kv_heads;
  for (int p = blockIdx.y; p < pairs; p += gridDim.y) {
    const int layer = p / a.num_kv_heads;
    const int g = p - layer * a.num_kv_heads;
    uint16_t *kc = a.k_cache + (size_t)layer * a.layer_stride;
    uint16_t *vc = a.v_cache + (size_t)layer * a.layer_stride;
    uint4 buf[MAXU];
#pragma unroll
    for (int u = 0; u < MAXU; ++u) {
      const int idx = tid + u * 256;
      if (idx < units) {
        const int which = idx / (nmove * CPR);
        const int rem = idx - which * nmove * CPR;
        const int mv = rem / CPR, ch = rem - mv * CPR;
        const int s = s_src[mv];
        const uint16_t *base = (which ? vc : kc) + (size_t)bt[s / kPage] * page_stride +
                               (size_t)g * kPage * D + (size_t)(s % kPage) * D + ch * 8;
        buf[u] = *reinterpret_cast<const uint4 *>(base);
      }
    }
    __builtin_amdgcn_s_waitcnt(0);  // this thread's source loads have returned
    __syncthreads();                // ... and so have every other thread's
#pragma unroll
    for (int u = 0; u < MAXU; ++u) {
      const int idx = tid + u * 256;
      if (idx < units) {
        const int which = idx / (nmove * CPR);
        const int rem = idx - which * nmove * CPR;
        const int mv = rem / CPR, ch = rem - mv * CPR;
        const int d = s_dst[mv];
        uint16_t *base = (which ? vc : kc) + (size_t)bt[d / kPage] * page_stride +
                         (size_t)g * kPage * D + (size_t)(d % kPage) * D + ch * 8;
        *reinterpret_cast<uint4 *>(base) = buf[u];
      }
    }
  }
}

}  // namespace

void launch_kv_compact(const CompactArgs &a, hipStream_t stream) {
  const int pairs = a.num_layers * a.num_kv_heads;
  int gy = 4096 / (a.batch > 0 ? a.batch : 1);
  if (gy > pairs) gy = pairs;
  if (gy > 65535) gy = 65535;
  if (gy < 1) gy = 1;
  dim3 grid(a.batch, gy);
  if (a.head_dim == 128)
    kv_compact_kernel<128><<<grid, 256, 0, stream>>>(a);
  else
    kv_compact_kernel<64><<<grid, 256, 0, stream>>>(a);
}

}  // namespace sv
