// Device helpers of the in-place K/V compaction, shared by kv_compact and the
// fused acceptance + compaction launch.
//
// What is computed (SwiftSpec, "Tree-Aware KV Cache Management": after
// verification only the accepted path's KV is kept; "Fused Latency-Optimized
// Kernels": the KV update accompanies the verification result): for every
// layer, KV head g and k = 0..accept_len-1, logical slot L + path[k] moves to
// slot L + k.  Reading every source before writing any destination makes the
// move safe in place (a destination can be another move's source).
#pragma once

#include "sv_device.h"
#include "sv_internal.h"

namespace sv {

// One thread checks a request's accepted path (path[0] = 0, strictly
// increasing, inside the request, pages valid) and lists the slots that move
// (path[k] != k).  Returns the number of moves, or -1 if the path or a page
// breaks the contract.
__device__ inline int compact_moves(const int32_t *path, int n1, int qn, int L, const int32_t *bt,
                                    int max_blocks, int num_pages, int *src, int *dst) {
  if (L < 0 || n1 < 0 || n1 > qn || qn > kMaxTokens) return -1;
  if (((long long)L + qn + kPage - 1) / kPage > max_blocks) return -1;
  int prev = -1, nmove = 0;
  for (int k = 0; k < n1; ++k) {
    const int pk = path[k];
    if (pk < k || pk >= qn || pk <= prev || (k == 0 && pk != 0)) return -1;
    prev = pk;
    if (pk != k) {
      dst[nmove] = L + k;
      src[nmove] = L + pk;
      ++nmove;
    }
  }
  for (int m = 0; m < nmove; ++m) {
    const int pd = bt[dst[m] / kPage], ps = bt[src[m] / kPage];
    if (pd < 0 || pd >= num_pages || ps < 0 || ps >= num_pages) return -1;
  }
  return nmove;
}

// The workgroup (256 threads) moves the listed slots (src/dst in shared
// memory) for (layer, head) pairs p = p0, p0 + pstep, ... < num_layers * Hkv:
// every source is read into registers, all loads have returned in every
// thread (barrier), and only then are destinations written.  A K slot is a
// row of D contiguous values (16-byte chunks).  A V slot is a row too when
// V pages are token-major (VT false); when they are stored transposed
// ([D][16 tokens], VT true) it is a column: D values 32 bytes apart, moved
// one 2-byte element at a time.
template <int D, bool VT>
__device__ inline void compact_pairs(uint16_t *k_cache, uint16_t *v_cache, int64_t layer_stride,
                                     int num_layers, int num_kv_heads, const int32_t *bt,
                                     const int *src, const int *dst, int nmove, int p0, int pstep) {
  constexpr int CPR = D / 8;                                       // 16-byte chunks of a row
  constexpr int MAXK = ((kMaxTokens - 1) * CPR + 255) / 256;       // row chunks per thread
  constexpr int MAXV = VT ? ((kMaxTokens - 1) * D + 255) / 256 : 1;  // V column elements per thread
  const int tid = threadIdx.x;
  const size_t page_stride = (size_t)num_kv_heads * kPage * D;
  const int kunits = nmove * CPR, vunits = VT ? nmove * D : 0;
  const int pairs = num_layers * num_kv_heads;
  for (int p = p0; p < pairs; p += pstep) {
    const int layer = p / num_kv_heads;
    const int g = p - layer * num_kv_heads;
    uint16_t *kc = k_cache + (size_t)layer * layer_stride + (size_t)g * kPage * D;
    uint16_t *vc = v_cache + (size_t)layer * layer_stride + (size_t)g * kPage * D;
    auto krow = [&](int slot) { return kc + (size_t)bt[slot / kPage] * page_stride + (size_t)(slot % kPage) * D; };
    auto vcol = [&](int slot) { return vc + (size_t)bt[slot / kPage] * page_stride + (slot % kPage); };
    auto vrow = [&](int slot) { return vc + (size_t)bt[slot / kPage] * page_stride + (size_t)(slot % kPage) * D; };
    uint4 kb[MAXK], vr[VT ? 1 : MAXK];
    uint16_t vb[MAXV];
#pragma unroll
    for (int u = 0; u < MAXK; ++u) {
      const int idx = tid + u * 256;
      if (idx < kunits) {
        const int mv = idx / CPR, ch = idx - mv * CPR;
        kb[u] = *reinterpret_cast<const uint4 *>(krow(src[mv]) + ch * 8);
        if constexpr (!VT) vr[u] = *reinterpret_cast<const uint4 *>(vrow(src[mv]) + ch * 8);
      }
    }
#pragma unroll
    for (int u = 0; u < MAXV; ++u) {
      const int idx = tid + u * 256;
      if (idx < vunits) {
        const int mv = idx / D, d = idx - mv * D;
        vb[u] = vcol(src[mv])[(size_t)d * kPage];
      }
    }
    __builtin_amdgcn_s_waitcnt(0);  // this thread's source loads have returned
    __syncthreads();                // ... and so have every other thread's
#pragma unroll
    for (int u = 0; u < MAXK; ++u) {
      const int idx = tid + u * 256;
      if (idx < kunits) {
        const int mv = idx / CPR, ch = idx - mv * CPR;
        *reinterpret_cast<uint4 *>(krow(dst[mv]) + ch * 8) = kb[u];
        if constexpr (!VT) *reinterpret_cast<uint4 *>(vrow(dst[mv]) + ch * 8) = vr[u];
      }
    }
#pragma unroll
    for (int u = 0; u < MAXV; ++u) {
      const int idx = tid + u * 256;
      if (idx < vunits) {
        const int mv = idx / D, d = idx - mv * D;
        vcol(dst[mv])[(size_t)d * kPage] = vb[u];
      }
    }
    __syncthreads();  // the next pair's reads come after this pair's writes
  }
}

}  // namespace sv
