// Verify attention over a paged bf16 KV cache with grouped-query heads,
// padding-free ragged chains and ancestor-masked draft trees, on gfx950.
//
// What is computed (SwiftSpec, "Fused Latency-Optimized Kernels" and
// "Tree-Aware KV Cache Management"; FASER, "Per-Request Length Adaptation";
// SSD's PagedAttention): every verify row of request i attends to the i-th
// request's committed context [0, L_i) and to those verify tokens that lie on
// its own root path, all read through the request's block table.
//
// Three launches:
//   attn_plan_kernel     one workgroup: validates per-request metadata, splits
//                        the (request, query-row tile, KV head) work into key
//                        chunks of equal size, writes the work-item table;
//   verify_attn_kernel   one workgroup per work item; four waves stream
//                        disjoint 32-key blocks of the chunk straight from HBM
//                        into MFMA operand registers (no LDS staging), keep an
//                        fp32 online softmax per query row, and merge through
//                        LDS at the end;
//   attn_combine_kernel  log-sum-exp merge of the chunks of split rows.
//
// MFMA formulation (v_mfma_f32_32x32x16_bf16, A 32xK, B Kx32, C 32x32):
//   S^T[key][row] = K[key][:] . Q^T[:][row]     A = K rows (one key per lane,
//                                               8 contiguous d per lane),
//                                               B = Q^T (loaded once)
//   O^T[d][row]  += V^T[d][key] . P^T[key][row] A = V^T (each lane holds 4
//                                               contiguous d of 8 keys, so a
//                                               V row is one 256-byte read by
//                                               32 lanes), B = P^T straight
//                                               from the S^T accumulator.
// Both accumulators keep a query row per lane, so the softmax statistics of a
// row live in one lane pair (lanes n and n+32) and never need a transpose.
#include "sv_device.h"
#include "sv_internal.h"

namespace sv {

namespace {

struct SegInfo {  // mirrors the int4 written by the plan kernel
  int req, rowgroup, nchunk, slot;
};

// --------------------------------------------------------------------------
// plan
// --------------------------------------------------------------------------
__global__ __launch_bounds__(kPlanThreads) void attn_plan_kernel(AttnArgs a) {
  __shared__ int s_scan[16];
  __shared__ long long s_red[16];
  int32_t *hdr = reinterpret_cast<int32_t *>(a.ws + a.lay.hdr);
  int4 *req = reinterpret_cast<int4 *>(a.ws + a.lay.req_meta);
  int4 *segs = reinterpret_cast<int4 *>(a.ws + a.lay.segs);
  int2 *items = reinterpret_cast<int2 *>(a.ws + a.lay.items);
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int B = a.batch, G = a.group, Hkv = a.num_kv_heads;
  unsigned flags = 0;
  if (tid == 0) {
    hdr[0] = 0;
    if (a.cu_q[0] != 0 || a.cu_q[B] != a.total_q) flags |= SV_DEV_BAD_CU_Q;
  }
  __syncthreads();

  // pass 1: per request rowgroups and keys; segment bases; total work
  long long work = 0;
  int seg_carry = 0;
  for (int base = 0; base < B; base += kPlanThreads) {
    const int i = base + tid;
    int rg = 0, keys = 0;
    if (i < B) {
      const int c0 = a.cu_q[i], c1 = a.cu_q[i + 1];
      const int L = a.context_lens[i];
      const int q = c1 - c0;
      bool ok = true;
      if (c0 < 0 || c1 < c0 || c1 > a.total_q) { flags |= SV_DEV_BAD_CU_Q; ok = false; }
      if (ok && q > kMaxTokens) { flags |= SV_DEV_TOO_MANY_TOKENS; ok = false; }
      if (L < 0) { flags |= SV_DEV_BAD_CONTEXT; ok = false; }
      if (ok) {
        const long long need = ((long long)L + q + kPage - 1) / kPage;
        if (need > a.max_blocks) { flags |= SV_DEV_TOO_MANY_PAGES; ok = false; }
      }
      if (ok && q > 0) {
        rg = (G * q + kTileRows - 1) / kTileRows;
        keys = L + q;
        work += (long long)rg * keys;
      }
      req[i] = make_int4(0, 0, rg, keys);  // keys parked in .w until pass 2
    }
    int tile_total;
    const int excl = block_excl_scan_1024(rg, s_scan, &tile_total);
    if (i < B) req[i].x = seg_carry + excl;
    seg_carry += tile_total;
  }
  const long long total_work = block_sum_1024(work, s_red) * Hkv;
  long long C = (total_work + kTargetItems - 1) / kTargetItems;
  C = ((C + kMinChunkKeys - 1) / kMinChunkKeys) * kMinChunkKeys;
  if (C < kMinChunkKeys) C = kMinChunkKeys;
  const int chunk = (int)C;

  // pass 2: chunks per request and item bases
  int item_carry = 0;
  for (int base = 0; base < B; base += kPlanThreads) {
    const int i = base + tid;
    int n_items = 0;
    int4 r = make_int4(0, 0, 0, 0);
    if (i < B) {
      r = req[i];
      const int nchunk = r.z > 0 ? (r.w + chunk - 1) / chunk : 0;
      r.w = nchunk;
      n_items = r.z * Hkv * nchunk;
    }
    int tile_total;
    const int excl = block_excl_scan_1024(n_items, s_scan, &tile_total);
    if (i < B) {
      r.y = item_carry + excl;
      req[i] = r;
    }
    item_carry += tile_total;
  }
  __syncthreads();

  // Requests whose cu_q ranges overlap (an inconsistent cu_q) could push the
  // counts past the workspace bounds; then nothing is scheduled at all.
  const bool fits = seg_carry <= a.lay.seg_bound && item_carry <= a.lay.item_bound;
  if (!fits) flags |= SV_DEV_BAD_CU_Q;

  // pass 3: one wave per request writes its segments and work items
  for (int i = wave; fits && i < B; i += kPlanThreads / 64) {
    const int4 r = req[i];
    const int per_seg = Hkv * r.w;
    for (int s = lane; s < r.z; s += 64)
      segs[r.x + s] = make_int4(i, s, r.w, r.y + s * per_seg);
    const int n = r.z * per_seg;
    for (int t = lane; t < n; t += 64) {
      const int s = t / per_seg, rem = t - s * per_seg;
      const int h = rem / r.w, c = rem - h * r.w;
      items[r.y + t] = make_int2(r.x + s, (h << 16) | c);
    }
  }
  // status word: OR of all threads' bits
  if (flags) atomicOr(reinterpret_cast<unsigned *>(hdr), flags);
  if (tid == 0) {
    hdr[1] = fits ? item_carry : 0;
    hdr[2] = chunk;
    hdr[3] = fits ? seg_carry : 0;
  }
}

// --------------------------------------------------------------------------
// attention
// --------------------------------------------------------------------------
template <int D>
__global__ __launch_bounds__(64 * kAttnWaves) __attribute__((amdgpu_waves_per_eu(2, 2))) void verify_attn_kernel(AttnArgs a) {
  constexpr int KK = D / 16;   // k-steps of the S^T product (16 d each)
  constexpr int DPL = D / 32;  // contiguous d per lane of a V row; O^T tiles
  static_assert(D == 64 || D == 128, "head_dim");
  __shared__ float sm_o[kAttnWaves][DPL][16][64];
  __shared__ float sm_m[kAttnWaves][32];
  __shared__ float sm_l[kAttnWaves][32];

  const int32_t *hdr = reinterpret_cast<const int32_t *>(a.ws + a.lay.hdr);
  const int n_items = hdr[1];
  const int item = blockIdx.x;
  if (item >= n_items) return;
  const int chunk = hdr[2];
  const int2 it = reinterpret_cast<const int2 *>(a.ws + a.lay.items)[item];
  const int4 sg4 = reinterpret_cast<const int4 *>(a.ws + a.lay.segs)[it.x];
  const SegInfo sg{sg4.x, sg4.y, sg4.z, sg4.w};
  const int h = it.y >> 16, c_idx = it.y & 0xffff;

  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int n = lane & 31, hh = lane >> 5;
  const int i = sg.req;
  const int o = a.cu_q[i];
  const int qn = a.cu_q[i + 1] - o;
  const int L = a.context_lens[i];
  const int nk = L + qn;
  const int G = a.group;

  // this lane's query row (token-major: row R = token * G + head-in-group)
  const int R = sg.rowgroup * kTileRows + n;
  const bool row_ok = R < G * qn;
  const int tok = row_ok ? R / G : 0;
  const int gq = R - (R / G) * G;
  bool parents_ok;
  const uint64_t anc_all = ancestor_mask(a.tree_parent, o, qn, lane, &parents_ok);
  // the shuffle must run on every lane: a source lane whose own row is past
  // the end would be inactive and read back as zero
  const uint64_t anc_tok = __shfl(anc_all, tok);
  const uint64_t anc = row_ok ? anc_tok : 0ull;
  if (!parents_ok && threadIdx.x == 0 && c_idx == 0 && h == 0 && sg.rowgroup == 0)
    atomicOr(reinterpret_cast<unsigned *>(a.ws + a.lay.hdr), SV_DEV_BAD_PARENT);

  // Q^T operand: row n, d = 16*kk + 8*hh .. +7
  bf16x8 qop[KK];
  {
    const uint16_t *qrow =
        a.q + ((size_t)(o + tok) * a.num_q_heads + (size_t)h * G + gq) * D + 8 * hh;
#pragma unroll
    for (int kk = 0; kk < KK; ++kk) {
      if (row_ok)
        qop[kk] = *reinterpret_cast<const bf16x8 *>(qrow + 16 * kk);
      else
        qop[kk] = bf16x8{};
    }
  }

  const int kbeg = c_idx * chunk;
  const int kend = min(nk, kbeg + chunk);
  const int bbeg = kbeg / kBlockKeys;
  const int bend = (kend + kBlockKeys - 1) / kBlockKeys;
  const int32_t *bt = a.block_tables + (size_t)i * a.max_blocks;
  const int npages = (nk + kPage - 1) / kPage;
  const size_t head_off = (size_t)h * kPage * D;
  const size_t page_stride = (size_t)a.num_kv_heads * kPage * D;

  float m = -INFINITY, l = 0.f;
  floatx16 acc[DPL];
#pragma unroll
  for (int c = 0; c < DPL; ++c) acc[c] = floatx16{};
  bool bad_page = false;

  for (int b = bbeg + wave; b < bend; b += kAttnWaves) {
    const int key0 = b * kBlockKeys;
    const int lp = key0 / kPage;
    // pages past the request's last page are not read; a needed page id
    // outside [0, num_pages) is reported and read as zeros
    int pg0 = lp < npages ? bt[lp] : -1;
    int pg1 = lp + 1 < npages ? bt[lp + 1] : -1;
    if (lp < npages && (pg0 < 0 || pg0 >= a.num_pages)) { bad_page = true; pg0 = -1; }
    if (lp + 1 < npages && (pg1 < 0 || pg1 >= a.num_pages)) { bad_page = true; pg1 = -1; }

    // K: lane holds key key0+n, d = 16*kk + 8*hh .. +7
    bf16x8 kop[KK];
    {
      const int pg = n < 16 ? pg0 : pg1;
      const bool ok = key0 + n < nk && pg >= 0;
      const uint16_t *krow = a.k_cache + (size_t)(ok ? pg : 0) * page_stride + head_off +
                             (size_t)(n & 15) * D + 8 * hh;
#pragma unroll
      for (int kk = 0; kk < KK; ++kk)
        kop[kk] = ok ? *reinterpret_cast<const bf16x8 *>(krow + 16 * kk) : bf16x8{};
    }
    // V: for key group m2 (keys 16*m2..), slot 8t+4hh+e, lane holds d = DPL*n .. +DPL-1
    uint32_t vraw[2][2][4][DPL / 2];
#pragma unroll
    for (int m2 = 0; m2 < 2; ++m2) {
      const int pg = m2 ? pg1 : pg0;
#pragma unroll
      for (int t = 0; t < 2; ++t)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int slot = 8 * t + 4 * hh + e;
          const bool ok = key0 + 16 * m2 + slot < nk && pg >= 0;
          const uint16_t *vrow = a.v_cache + (size_t)(ok ? pg : 0) * page_stride + head_off +
                                 (size_t)slot * D + DPL * n;
          if constexpr (DPL == 4) {
            uint2 v = ok ? *reinterpret_cast<const uint2 *>(vrow) : make_uint2(0, 0);
            vraw[m2][t][e][0] = v.x;
            vraw[m2][t][e][1] = v.y;
          } else {
            vraw[m2][t][e][0] = ok ? *reinterpret_cast<const uint32_t *>(vrow) : 0u;
          }
        }
    }

    // S^T = K . Q^T ; acc reg r <-> key key0 + 8*(r/4) + 4*hh + r%4, row n
    floatx16 s = floatx16{};
#pragma unroll
    for (int kk = 0; kk < KK; ++kk)
      s = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kop[kk], qop[kk], s, 0, 0, 0);

    float sv[16];
    const bool need_mask = key0 + kBlockKeys > L;
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      float x = s[r] * a.scale_log2;
      if (need_mask) {
        const int key = key0 + 8 * (r >> 2) + 4 * hh + (r & 3);
        const bool vis = key < L || (key < nk && ((anc >> (unsigned)(key - L)) & 1ull));
        x = vis ? x : -INFINITY;
      }
      sv[r] = x;
    }
    float mb = sv[0];
#pragma unroll
    for (int r = 1; r < 16; ++r) mb = fmaxf(mb, sv[r]);
    mb = fmaxf(mb, __shfl_xor(mb, 32));
    const float mnew = fmaxf(m, mb);
    const float mref = mnew == -INFINITY ? 0.f : mnew;
    const float alpha = fast_exp2(m - mref);
    float psum = 0.f;
    uint32_t pw[8];
#pragma unroll
    for (int r = 0; r < 16; r += 2) {
      const float p0 = fast_exp2(sv[r] - mref);
      const float p1 = fast_exp2(sv[r + 1] - mref);
      psum += p0 + p1;
      pw[r >> 1] = pack_bf16x2(p0, p1);
    }
    l = l * alpha + psum;
    m = mnew;
#pragma unroll
    for (int c = 0; c < DPL; ++c) acc[c] *= alpha;

    // O^T += V^T . P^T over the two 16-key groups
#pragma unroll
    for (int m2 = 0; m2 < 2; ++m2) {
      bf16x8 pop;
      {
        uint32_t w4[4] = {pw[4 * m2], pw[4 * m2 + 1], pw[4 * m2 + 2], pw[4 * m2 + 3]};
        pop = __builtin_bit_cast(bf16x8, w4);
      }
#pragma unroll
      for (int c = 0; c < DPL; ++c) {
        // k-slot s = 4t+e <-> key 16*m2 + 8t + 4hh + e; element c of the lane's d-run
        uint32_t w4[4];
#pragma unroll
        for (int pr = 0; pr < 4; ++pr) {
          const int s0 = 2 * pr, s1 = 2 * pr + 1;
          const uint32_t x0 = vraw[m2][s0 >> 2][s0 & 3][c >> 1];
          const uint32_t x1 = vraw[m2][s1 >> 2][s1 & 3][c >> 1];
          w4[pr] = (c & 1) ? ((x0 >> 16) | (x1 & 0xffff0000u)) : ((x0 & 0xffffu) | (x1 << 16));
        }
        const bf16x8 vop = __builtin_bit_cast(bf16x8, w4);
        acc[c] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vop, pop, acc[c], 0, 0, 0);
      }
    }
  }
  if (bad_page) atomicOr(reinterpret_cast<unsigned *>(a.ws + a.lay.hdr), SV_DEV_BAD_PAGE);

  // both lane halves summed different keys of the same row
  l += __shfl_xor(l, 32);

  // ---- merge the waves ----------------------------------------------------
  if (hh == 0) {
    sm_m[wave][n] = m;
    sm_l[wave][n] = l;
  }
#pragma unroll
  for (int c = 0; c < DPL; ++c)
#pragma unroll
    for (int r = 0; r < 16; ++r) sm_o[wave][c][r][lane] = acc[c][r];
  __syncthreads();

  float M = -INFINITY;
#pragma unroll
  for (int w = 0; w < kAttnWaves; ++w) M = fmaxf(M, sm_m[w][n]);
  const float Mref = M == -INFINITY ? 0.f : M;
  float f[kAttnWaves];
  float Lsum = 0.f;
#pragma unroll
  for (int w = 0; w < kAttnWaves; ++w) {
    f[w] = fast_exp2(sm_m[w][n] - Mref);
    Lsum += f[w] * sm_l[w][n];
  }
  // this wave finalises registers r = 4*wave .. 4*wave+3, i.e. output
  // d = DPL*(8*wave + 4*hh) + (0 .. 4*DPL-1), contiguous
  float ov[4 * DPL];
#pragma unroll
  for (int rr = 0; rr < 4; ++rr)
#pragma unroll
    for (int c = 0; c < DPL; ++c) {
      float v = 0.f;
#pragma unroll
      for (int w = 0; w < kAttnWaves; ++w) v += f[w] * sm_o[w][c][4 * wave + rr][lane];
      ov[DPL * rr + c] = v;
    }
  if (!row_ok) return;
  const float inv = Lsum > 0.f ? 1.0f / Lsum : 0.f;
  const int d0 = DPL * (8 * wave + 4 * hh);
  if (sg.nchunk == 1) {
    uint16_t *orow = a.out + ((size_t)(o + tok) * a.num_q_heads + (size_t)h * G + gq) * D + d0;
    uint32_t pk[2 * DPL];
#pragma unroll
    for (int t = 0; t < 2 * DPL; ++t) pk[t] = pack_bf16x2(ov[2 * t] * inv, ov[2 * t + 1] * inv);
#pragma unroll
    for (int t = 0; t < DPL / 2; ++t)
      reinterpret_cast<uint4 *>(orow)[t] = make_uint4(pk[4 * t], pk[4 * t + 1], pk[4 * t + 2], pk[4 * t + 3]);
  } else {
    const int slot = sg.slot + h * sg.nchunk + c_idx;
    float *po = reinterpret_cast<float *>(a.ws + a.lay.part_o) + ((size_t)slot * kTileRows + n) * D + d0;
#pragma unroll
    for (int t = 0; t < DPL; ++t)
      reinterpret_cast<float4 *>(po)[t] =
          make_float4(ov[4 * t] * inv, ov[4 * t + 1] * inv, ov[4 * t + 2] * inv, ov[4 * t + 3] * inv);
    if (wave == 0 && hh == 0) {
      float *pl = reinterpret_cast<float *>(a.ws + a.lay.part_lse);
      pl[(size_t)slot * kTileRows + n] = Lsum > 0.f ? Mref + fast_log2(Lsum) : -INFINITY;
    }
  }
}

// --------------------------------------------------------------------------
// combine chunks of split rows
// --------------------------------------------------------------------------
template <int D>
__global__ __launch_bounds__(256) void attn_combine_kernel(AttnArgs a) {
  constexpr int DT = D / 8;  // d per thread
  const int32_t *hdr = reinterpret_cast<const int32_t *>(a.ws + a.lay.hdr);
  const int s_idx = blockIdx.x / a.num_kv_heads;
  const int h = blockIdx.x - s_idx * a.num_kv_heads;
  if (s_idx >= hdr[3]) return;
  const int4 sg4 = reinterpret_cast<const int4 *>(a.ws + a.lay.segs)[s_idx];
  const SegInfo sg{sg4.x, sg4.y, sg4.z, sg4.w};
  if (sg.nchunk <= 1) return;
  const int n = threadIdx.x >> 3, part = threadIdx.x & 7;
  const int o = a.cu_q[sg.req];
  const int qn = a.cu_q[sg.req + 1] - o;
  const int G = a.group;
  const int R = sg.rowgroup * kTileRows + n;
  if (R >= G * qn) return;
  const int tok = R / G, gq = R - tok * G;
  const int slot0 = sg.slot + h * sg.nchunk;
  const float *pl = reinterpret_cast<const float *>(a.ws + a.lay.part_lse);
  const float *po = reinterpret_cast<const float *>(a.ws + a.lay.part_o);
  float M = -INFINITY;
  for (int c = 0; c < sg.nchunk; ++c) M = fmaxf(M, pl[(size_t)(slot0 + c) * kTileRows + n]);
  const float Mref = M == -INFINITY ? 0.f : M;
  float accv[DT];
#pragma unroll
  for (int t = 0; t < DT; ++t) accv[t] = 0.f;
  float den = 0.f;
  for (int c = 0; c < sg.nchunk; ++c) {
    const float w = fast_exp2(pl[(size_t)(slot0 + c) * kTileRows + n] - Mref);
    den += w;
    const float4 *src = reinterpret_cast<const float4 *>(po + ((size_t)(slot0 + c) * kTileRows + n) * D + part * DT);
#pragma unroll
    for (int t = 0; t < DT / 4; ++t) {
      const float4 v = src[t];
      accv[4 * t] += w * v.x;
      accv[4 * t + 1] += w * v.y;
      accv[4 * t + 2] += w * v.z;
      accv[4 * t + 3] += w * v.w;
    }
  }
  const float inv = den > 0.f ? 1.0f / den : 0.f;
  uint16_t *orow = a.out + ((size_t)(o + tok) * a.num_q_heads + (size_t)h * G + gq) * D + part * DT;
#pragma unroll
  for (int t = 0; t < DT / 8; ++t)
    reinterpret_cast<uint4 *>(orow)[t] =
        make_uint4(pack_bf16x2(accv[8 * t] * inv, accv[8 * t + 1] * inv),
                   pack_bf16x2(accv[8 * t + 2] * inv, accv[8 * t + 3] * inv),
                   pack_bf16x2(accv[8 * t + 4] * inv, accv[8 * t + 5] * inv),
                   pack_bf16x2(accv[8 * t + 6] * inv, accv[8 * t + 7] * inv));
}

}  // namespace

void launch_verify_attn(const AttnArgs &a, int head_dim, hipStream_t stream) {
  attn_plan_kernel<<<1, kPlanThreads, 0, stream>>>(a);
  const int groups_attn = a.lay.item_bound;
  const int groups_comb = a.lay.seg_bound * a.num_kv_heads;
  if (head_dim == 128) {
    verify_attn_kernel<128><<<groups_attn, 64 * kAttnWaves, 0, stream>>>(a);
    attn_combine_kernel<128><<<groups_comb, 256, 0, stream>>>(a);
  } else {
    verify_attn_kernel<64><<<groups_attn, 64 * kAttnWaves, 0, stream>>>(a);
    attn_combine_kernel<64><<<groups_comb, 256, 0, stream>>>(a);
  }
}

}  // namespace sv
