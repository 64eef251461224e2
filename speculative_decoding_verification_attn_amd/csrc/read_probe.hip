// HBM read-ceiling probe: streams a list of K and V cache blocks with the
// load pattern of the attention kernel and nothing else, so that the
// attention's KV-stream rate can be set against what a pure read kernel
// reaches on the same pages of the same device (the published 8 TB/s is an
// interface rate that no access pattern reaches).
//
// Each listed chunk is one (page, KV head) block of the K cache and the same
// block of the V cache (chunk_bytes each).  The list is cut into contiguous
// slices, one per wave (two workgroups of four waves per compute unit); a
// wave loads two chunks of K and V (16-byte
// nontemporal loads, 1 KB per instruction) while it folds the previous two
// into a running XOR, so one pair is in flight while another is consumed,
// as in the attention kernel.  The XORs go to sink[] so no load can be
// removed; together they are the XOR of every word of the listed blocks.
#include "read_probe.h"

namespace sv {

namespace {

constexpr int kProbeWaves = 4;

typedef unsigned u32x4v __attribute__((ext_vector_type(4)));

template <int PER>  // 1 KB instructions per chunk
struct ProbeBuf {
  u32x4v k[2][PER], v[2][PER];
};

template <int PER>
__device__ inline void probe_load(ProbeBuf<PER> &b, const uint8_t *k, const uint8_t *v, const int32_t *chunks,
                                  int64_t c, int64_t c_last, int64_t buffer_chunks, int lane) {
#pragma unroll
  for (int x = 0; x < 2; ++x) {
    const int64_t cc = min(c + x, c_last);  // past the slice: its last chunk again
    int64_t idx = chunks[cc];
    if (idx < 0 || idx >= buffer_chunks) idx = 0;
    const size_t base = (size_t)idx * (PER * 1024) + (size_t)lane * 16;
#pragma unroll
    for (int j = 0; j < PER; ++j) {
      b.k[x][j] = __builtin_nontemporal_load(reinterpret_cast<const u32x4v *>(k + base + j * 1024));
      b.v[x][j] = __builtin_nontemporal_load(reinterpret_cast<const u32x4v *>(v + base + j * 1024));
    }
  }
}

// XOR of the pair's words; the second chunk only if it lies in the slice
// (past it the load re-read the slice's last chunk), so the XOR of all sink
// words is the XOR of every word of the listed blocks
template <int PER>
__device__ inline uint32_t probe_fold(const ProbeBuf<PER> &b, bool second) {
  uint32_t x = 0;
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < PER; ++j) {
      const u32x4v a = b.k[i][j] ^ b.v[i][j];
      const uint32_t y = a.x ^ a.y ^ a.z ^ a.w;
      x ^= (i == 0 || second) ? y : 0u;
    }
  return x;
}

template <int PER>
__global__ __launch_bounds__(64 * kProbeWaves) void hbm_read_probe_kernel(const uint8_t *k, const uint8_t *v,
                                                                        const int32_t *chunks, int64_t n,
                                                                        int64_t buffer_chunks, uint32_t *sink) {
  const int lane = threadIdx.x & 63;
  const int64_t gw = (int64_t)blockIdx.x * kProbeWaves + (threadIdx.x >> 6);
  const int64_t nw = (int64_t)gridDim.x * kProbeWaves;
  const int64_t c0 = n * gw / nw, c1 = n * (gw + 1) / nw;
  uint32_t x = 0;
  if (c0 < c1) {
    ProbeBuf<PER> A, B;
    probe_load<PER>(A, k, v, chunks, c0, c1 - 1, buffer_chunks, lane);
    for (int64_t c = c0;;) {
      probe_load<PER>(B, k, v, chunks, c + 2, c1 - 1, buffer_chunks, lane);
      x ^= probe_fold<PER>(A, c + 1 < c1);
      c += 2;
      if (c >= c1) break;
      probe_load<PER>(A, k, v, chunks, c + 2, c1 - 1, buffer_chunks, lane);
      x ^= probe_fold<PER>(B, c + 1 < c1);
      c += 2;
      if (c >= c1) break;
    }
  }
  sink[gw * 64 + lane] = x;
}

}  // namespace

void launch_hbm_read_probe(const void *k, const void *v, const int32_t *chunks, int64_t n, int chunk_bytes,
                           int64_t buffer_chunks, uint32_t *sink, int grid, hipStream_t stream) {
  const uint8_t *kb = static_cast<const uint8_t *>(k), *vb = static_cast<const uint8_t *>(v);
  if (chunk_bytes == 4096)
    hbm_read_probe_kernel<4><<<grid, 64 * kProbeWaves, 0, stream>>>(kb, vb, chunks, n, buffer_chunks, sink);
  else
    hbm_read_probe_kernel<2><<<grid, 64 * kProbeWaves, 0, stream>>>(kb, vb, chunks, n, buffer_chunks, sink);
}

}  // namespace sv
