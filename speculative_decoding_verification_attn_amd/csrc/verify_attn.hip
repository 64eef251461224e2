// Verify attention over a paged bf16 KV cache with grouped-query heads,
// padding-free ragged chains and ancestor-masked draft trees, on gfx950.
//
// What is computed (SwiftSpec, "Fused Latency-Optimized Kernels" and
// "Tree-Aware KV Cache Management"; FASER, "Per-Request Length Adaptation";
// SSD's PagedAttention): every verify row of request i attends to the
// request's committed context [0, L_i) and to those verify tokens that lie on
// its own root path, all read through the request's block table.
//
// Work decomposition.  A unit is one (request, KV head, group of up to two
// 32-row query tiles); the rows of a tile are (token, query head) pairs of that
// KV head's group, token-major, so every K/V block a unit reads serves all its
// rows (GQA sharing) in both tiles.  Every unit's keys form ceil((L+q)/32)
// blocks of 32 keys; all units' blocks, in (request, head, tile group) order,
// make one global sequence that is cut into contiguous ranges of equal cost
// (blocks plus a fixed charge per unit start), one per persistent workgroup
// (one per CU).  Only the first and last unit of a range can be cut, so at most
// two partial results per workgroup need merging.
//
// Three launches:
//   attn_plan_kernel     one workgroup, once per step: validates per-request
//                        metadata and writes the unit table, each workgroup's
//                        range and first unit, and the merge records;
//   verify_attn_kernel   the persistent workgroups, once per layer; four waves
//                        (one per SIMD) stream disjoint 32-key blocks straight
//                        from HBM into MFMA operand registers, one block in
//                        flight beside the one computed, with an fp32 online
//                        softmax per query row, then merge through LDS;
//   attn_merge_kernel    log-sum-exp merge of the partials of cut units.
//
// Two V page layouts: token-major ([16 tokens][D] per (page, head), like K)
// and transposed ([D][16 tokens]); the kernel is instantiated for each.  The
// formulation below is the transposed one; with token-major pages a lane
// loads DPL contiguous d of 8 V rows and packs the V^T operand from them, and
// K rows are loaded in plain lane order (see KVBlock and key_of_lane).
//
// MFMA formulation (v_mfma_f32_32x32x16_bf16, A 32xK, B Kx32, C 32x32):
//   S^T[key][row] = K[key][:] . Q^T[:][row]     A = K rows (one key per lane,
//                                               8 contiguous d per lane),
//                                               B = Q^T (staged once in LDS)
//   O^T[d][row]  += V^T[d][key] . P^T[key][row] A = V^T (the V page is stored
//                                               transposed, [D][16 tokens], so
//                                               a lane's 8 keys at one d are
//                                               one 16-byte load and 32 lanes
//                                               read 1 KB contiguous), B = P^T
//                                               straight from the S^T
//                                               accumulator (K rows are loaded
//                                               in the lane order that makes
//                                               each lane's 8 P values 8
//                                               consecutive keys).
// Both accumulators keep a query row per lane, so the softmax statistics of a
// row live in one lane pair (lanes n and n+32) and never need a transpose.
#include <type_traits>
#include "sv_device.h"
#include "sv_internal.h"

namespace sv {

namespace {

// index of the workgroup whose range [start[w], start[w+1]) holds block x:
// the last w < p with start[w] <= x (a workgroup with an empty range shares
// its start with the next one and is never returned)
__device__ inline int wg_of_block(const int32_t *start, int p, int x) {
  int lo = 0, hi = p - 1;
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (start[mid] <= x) lo = mid; else hi = mid - 1;
  }
  return lo;
}

// --------------------------------------------------------------------------
// plan
// --------------------------------------------------------------------------
// Per-request bases live in LDS (or, for very large batches, in the
// workspace): unit base, block base, row tiles, blocks per unit.
__global__ __launch_bounds__(kPlanThreads) void attn_plan_kernel(AttnArgs a) {
  __shared__ int s_scan[16];
  __shared__ long long s_red[16];
  __shared__ int s_req[4][kPlanLdsRequests];
  int32_t *hdr = reinterpret_cast<int32_t *>(a.ws + a.lay.hdr);
  UnitRec *units = reinterpret_cast<UnitRec *>(a.ws + a.lay.units);
  int32_t *wg_start = reinterpret_cast<int32_t *>(a.ws + a.lay.wg_start);
  int32_t *wg_first = reinterpret_cast<int32_t *>(a.ws + a.lay.wg_first);
  UnitRec *wg_rec = reinterpret_cast<UnitRec *>(a.ws + a.lay.wg_rec);
  UnitRec *merge_rec = reinterpret_cast<UnitRec *>(a.ws + a.lay.merge_rec);
  const int tid = threadIdx.x;
  const int B = a.batch, G = a.group, Hkv = a.num_kv_heads;
  const bool in_lds = B <= kPlanLdsRequests;
  int32_t *gmeta = reinterpret_cast<int32_t *>(a.ws + a.lay.req_meta);
  int *ubase = in_lds ? s_req[0] : gmeta;
  int *bbase = in_lds ? s_req[1] : gmeta + B;
  int *rgs = in_lds ? s_req[2] : gmeta + 2 * B;
  int *nblks = in_lds ? s_req[3] : gmeta + 3 * B;
  unsigned flags = 0;
  if (tid == 0) {
    hdr[0] = 0;
    // a chunk's row count is read here (total_q bounds it)
    if (a.cu_q[0] != 0 || (a.chunk_begin ? a.cu_q[B] > a.total_q : a.cu_q[B] != a.total_q)) flags |= SV_DEV_BAD_CU_Q;
  }

  // pass 1: per request row tiles and blocks; unit and block bases
  int unit_carry = 0;
  long long blk_carry = 0;
  for (int base = 0; base < B; base += kPlanThreads) {
    const int i = base + tid;
    int rg = 0, nblk = 0;
    long long n_blocks = 0;
    if (i < B) {
      const int c0 = a.cu_q[i], c1 = a.cu_q[i + 1];
      const int L = a.context_lens[i];
      const int q = c1 - c0;
      bool ok = true;
      if (c0 < 0 || c1 < c0 || c1 > a.total_q) { flags |= SV_DEV_BAD_CU_Q; ok = false; }
      // chunked rows: tokens [s, s+q) of the request's q_full verify tokens
      int s0 = 0;
      if (a.chunk_begin) {
        s0 = a.chunk_begin[i];
        const int f0 = a.cu_full[i], f1 = a.cu_full[i + 1];
        if (f0 < 0 || f1 < f0 || f1 > a.total_full || s0 < 0 || (ok && s0 + q > f1 - f0)) {
          flags |= SV_DEV_BAD_CU_Q;
          ok = false;
        }
      }
      if (ok && s0 + q > kMaxTokens) { flags |= SV_DEV_TOO_MANY_TOKENS; ok = false; }
      if (L < 0) { flags |= SV_DEV_BAD_CONTEXT; ok = false; }
      if (ok && ((long long)L + s0 + q + kPage - 1) / kPage > a.max_blocks) {
        flags |= SV_DEV_TOO_MANY_PAGES;
        ok = false;
      }
      if (ok && q > 0) {
        rg = (G * q + kTileRows * kUnitTiles - 1) / (kTileRows * kUnitTiles);
        nblk = (L + s0 + q + kBlockKeys - 1) / kBlockKeys;
        n_blocks = (long long)rg * Hkv * nblk;
      }
    }
    int tile_units;
    const int u_excl = block_excl_scan_1024<int>(rg * Hkv, s_scan, &tile_units);
    long long tile_blocks;
    const long long b_excl = block_excl_scan_1024<long long>(n_blocks, s_red, &tile_blocks);
    if (i < B) {
      ubase[i] = unit_carry + u_excl;
      // bases beyond 2^31-1 make the plan fail below, so clamping is harmless
      bbase[i] = (int)min(blk_carry + b_excl, 0x7fffffffLL);
      rgs[i] = rg;
      nblks[i] = nblk;
    }
    unit_carry += tile_units;
    blk_carry += tile_blocks;
  }
  const bool fits = unit_carry <= a.lay.unit_bound && blk_carry <= 0x7fffffffLL;
  if (!fits) flags |= SV_DEV_BAD_CU_Q;
  const long long nb = fits ? blk_carry : 0;
  int P = (int)min((long long)a.grid, (nb + kMinBlocksPerWG - 1) / kMinBlocksPerWG);
  if (P < 1) P = 1;
  __syncthreads();

  if (fits) {
    // pass 2: each request's unit records
    for (int i = tid; i < B; i += kPlanThreads) {
      const int rg = rgs[i], nblk = nblks[i], u0 = ubase[i], b0 = bbase[i];
      if (rg == 0) continue;
      const int qn = a.cu_q[i + 1] - a.cu_q[i], L = a.context_lens[i];
      const int s0 = a.chunk_begin ? a.chunk_begin[i] : 0, ot = a.chunk_begin ? a.cu_full[i] : a.cu_q[i];
      const int o = ot + s0;  // q and out rows: one per verify token (a chunk's rows in place)
      for (int k = 0; k < rg * Hkv; ++k) {
        const int h = k / rg, r = k - h * rg;
        units[u0 + k] = UnitRec{make_int4(i, h, r, b0 + k * nblk), make_int4(o, qn, L, nblk),
                                make_int4(s0, ot, 0, 0)};
      }
    }
    // pass 3: range boundaries.  Block x costs 1 and the start of every unit
    // after the first costs kUnitStartCost more, so the cost before block x
    // is F(x) = x + kUnitStartCost * (index of x's unit).  Workgroup w starts
    // at the first block with F >= w * F_total / P: the request by binary
    // search over F at its first block, the unit and block by division.
    const long long kc = kUnitStartCost;
    const long long ftot = nb + kc * (unit_carry > 0 ? unit_carry - 1 : 0);
    for (int w = tid; w <= P && nb > 0; w += kPlanThreads) {
      if (w == P) {
        wg_start[w] = (int)nb;
        continue;
      }
      const long long c = (long long)w * ftot / P;
      int lo = 0, hi = B - 1;
      while (lo < hi) {
        const int mid = (lo + hi + 1) >> 1;
        if (bbase[mid] + kc * ubase[mid] <= c) lo = mid; else hi = mid - 1;
      }
      // requests without units share their bases with the next request, so
      // the last request at or before c has units unless c precedes them all
      long long x = 0;
      if (rgs[lo] > 0) {
        const long long span = nblks[lo] + kc;  // cost of one unit with its start
        const long long off = c - (bbase[lo] + kc * ubase[lo]);
        const long long k = min(off / span, (long long)rgs[lo] * Hkv - 1);
        const long long r = off - k * span;  // >= 0
        x = bbase[lo] + k * nblks[lo] + min(r, (long long)nblks[lo]);
      }
      wg_start[w] = (int)min(x, nb);
    }
    __syncthreads();
    // pass 4: per workgroup w, the unit holding its first block (the request
    // whose block span holds it, by binary search) with a copy of its record,
    // and the cut unit this workgroup merges afterwards: the unit whose first
    // block lies in range w0 = w-1 and which continues into range w.  (A range
    // is empty only when its cost share falls inside one unit-start charge;
    // it then starts at a unit start and has no record.)
    for (int w = tid; w < P && nb > 0; w += kPlanThreads) {
      const int st = min(wg_start[w], (int)nb - 1);
      int lo = 0, hi = B - 1;
      while (lo < hi) {
        const int mid = (lo + hi + 1) >> 1;
        if (bbase[mid] <= st) lo = mid; else hi = mid - 1;
      }
      const int nblk = nblks[lo], rg = rgs[lo];
      const int k = (st - bbase[lo]) / nblk;
      const int u = ubase[lo] + k;
      const int h = k / rg, r = k - h * rg;
      const int ub = bbase[lo] + k * nblk;
      const int qn = a.cu_q[lo + 1] - a.cu_q[lo], L = a.context_lens[lo];
      const int s0 = a.chunk_begin ? a.chunk_begin[lo] : 0, ot = a.chunk_begin ? a.cu_full[lo] : a.cu_q[lo];
      const int o = ot + s0;
      wg_first[w] = u;
      wg_rec[w] = UnitRec{make_int4(lo, h, r, ub), make_int4(o, qn, L, nblk), make_int4(s0, ot, 0, 0)};
      const int w0 = wg_of_block(wg_start, P, ub);
      if (w >= 1 && w0 == w - 1) {
        const int w1 = wg_of_block(wg_start, P, ub + nblk - 1);
        const int side0 = wg_start[w0] == ub ? 0 : 1;
        merge_rec[w] = UnitRec{make_int4(u, w0, w1, side0), make_int4(o, qn, h, r), make_int4(0, 0, 0, 0)};
      } else {
        merge_rec[w] = UnitRec{make_int4(-1, 0, 0, 0), make_int4(0, 0, 0, 0), make_int4(0, 0, 0, 0)};
      }
    }
  }
  if (flags) atomicOr(reinterpret_cast<unsigned *>(hdr), flags);
  if (tid == 0) {
    hdr[1] = nb > 0 ? P : 0;
    hdr[2] = (int)nb;
    hdr[3] = fits ? unit_carry : 0;
  }
}

// Registers of one 32-key block in flight: K rows as MFMA A operands (lane n
// holds key key_of_lane<VT>(n)) and the lane's V values.
//   VT (V pages stored transposed, [D][16 tokens]): vt[m2][c] holds, for
//     d-row n + 32c of the block's page m2, the 8 consecutive keys 8hh..8hh+7,
//     which is the V^T operand as it stands;
//   token-major V pages ([16 tokens][D]): v[m2][t][e] holds the lane's DPL
//     contiguous d (DPL*n ..) of key 16*m2 + 8t + 4hh + e (a V row is read by
//     32 lanes, DPL*2 bytes each), and the V^T operand of column c is packed
//     from element c of the 8 keys.
template <int D, bool VT>
struct KVBlock;
template <int D>
struct KVBlock<D, true> {
  bf16x8 k[D / 16];
  bf16x8 vt[2][D / 32];
};
template <int D>
struct KVBlock<D, false> {
  bf16x8 k[D / 16];
  uint32_t v[2][2][4][D / 64];
};

// Key (0..31 within a 32-key block) whose K row lane n of the S^T product
// loads.  Transposed V: n with bits 2 and 3 swapped; the S^T accumulator then
// holds in register r of lane half hh the score of key 16*(r/8) + 8*hh + r%8,
// so the eight P values a lane packs for one P.V product are 8 consecutive
// keys, the run a transposed V page row stores contiguously.  Token-major V:
// lane n loads key n, and register r of lane half hh holds key
// 8*(r/4) + 4*hh + r%4, the keys whose V rows the lane loaded.
template <bool VT>
__device__ inline int key_of_lane(int n) {
  if constexpr (VT) return (n & ~12) | ((n & 4) << 1) | ((n & 8) >> 1);
  else return n;
}

// key of S^T accumulator register r of lane half hh, relative to the block
template <bool VT>
__device__ inline int key_of_reg(int r, int hh) {
  if constexpr (VT) return 16 * (r >> 3) + 8 * hh + (r & 7);
  else return 8 * (r >> 2) + 4 * hh + (r & 3);
}

typedef const __attribute__((address_space(4))) int32_t *const_i32_ptr;

// Physical pages of the two logical pages of block b, read with scalar loads
// (the block index is wave-uniform).  Pages past the request's last page, and
// ids outside [0, num_pages), are replaced by a valid page (the request's
// first page if its id is valid, else page 0) so every load below stays in
// bounds; *bad records the latter.
__device__ inline int2 block_pages(const_i32_ptr bt, int b, int npages, int num_pages, bool *bad) {
  const int lp = 2 * b;
  const int i0 = min(lp, npages - 1), i1 = min(lp + 1, npages - 1);
  // the three entries are read together: one round trip
  int p0 = bt[i0], p1 = bt[i1];
  int safe = bt[0];
  if (safe < 0 || safe >= num_pages) safe = 0;
  const bool bad0 = p0 < 0 || p0 >= num_pages, bad1 = p1 < 0 || p1 >= num_pages;
  *bad = *bad || (lp < npages && bad0) || (lp + 1 < npages && bad1);
  if (lp >= npages || bad0) p0 = safe;
  if (lp + 1 >= npages || bad1) p1 = safe;
  return make_int2(p0, p1);
}

// K and V take different cache policies.  A V load instruction consumes
// whole lines: 16 B of 32 consecutive d-rows of one transposed page (1 KB
// contiguous), or two whole token-major V rows (DPL*2 B per lane), so it is
// issued nontemporal: streamed through the caches without being kept.  A K
// load instruction covers only 32 B of each of 32 rows (one key per lane, as
// the MFMA A operand needs), and the rest of each line is read by the next
// three instructions, so K uses ordinary loads that keep the line for them.
template <int D, bool VT>
__device__ inline void load_block(KVBlock<D, VT> &buf, const uint16_t *kh, const uint16_t *vh,
                                  int2 pg, int n, int hh, size_t page_stride) {
  constexpr int KK = D / 16, DPL = D / 32;
  const int kn = key_of_lane<VT>(n);
  const uint16_t *krow = kh + (size_t)(kn < 16 ? pg.x : pg.y) * page_stride + (size_t)(kn & 15) * D + 8 * hh;
#pragma unroll
  for (int kk = 0; kk < KK; ++kk) buf.k[kk] = *reinterpret_cast<const bf16x8 *>(krow + 16 * kk);
  typedef unsigned u32x4v __attribute__((ext_vector_type(4)));
  typedef unsigned u32x2v __attribute__((ext_vector_type(2)));
#pragma unroll
  for (int m2 = 0; m2 < 2; ++m2) {
    if constexpr (VT) {
      const uint16_t *vpage = vh + (size_t)(m2 ? pg.y : pg.x) * page_stride + 8 * hh;
#pragma unroll
      for (int c = 0; c < DPL; ++c) {
        const u32x4v x =
            __builtin_nontemporal_load(reinterpret_cast<const u32x4v *>(vpage + (size_t)(n + 32 * c) * kPage));
        buf.vt[m2][c] = __builtin_bit_cast(bf16x8, x);
      }
    } else {
      const uint16_t *vpage = vh + (size_t)(m2 ? pg.y : pg.x) * page_stride + DPL * n;
#pragma unroll
      for (int t = 0; t < 2; ++t)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const uint16_t *vrow = vpage + (size_t)(8 * t + 4 * hh + e) * D;
          if constexpr (DPL == 4) {
            const u32x2v x = __builtin_nontemporal_load(reinterpret_cast<const u32x2v *>(vrow));
            buf.v[m2][t][e][0] = x.x;
            buf.v[m2][t][e][1] = x.y;
          } else {
            buf.v[m2][t][e][0] = __builtin_nontemporal_load(reinterpret_cast<const uint32_t *>(vrow));
          }
        }
    }
  }
}

// One 32-key block for each of the unit's nt query tiles: S^T = K.Q_t^T,
// mask, online softmax, O_t^T += V^T.P_t^T.  The block's K and V registers
// serve every tile, so K/V is read once per unit whatever its row count.
constexpr float kRescaleSlack = 8.0f;  // log2 units

template <int D, bool VT>
__device__ inline void compute_block(KVBlock<D, VT> &buf, const bf16x8 (&qop)[kUnitTiles][D / 16], int nt, int key0,
                                     int L, int nk, const uint64_t (&anc)[kUnitTiles], int hh, float scale_log2,
                                     float (&m)[kUnitTiles], float (&l)[kUnitTiles],
                                     floatx16 (&acc)[kUnitTiles][D / 32]) {
  constexpr int KK = D / 16, DPL = D / 32;
  if (key0 + kBlockKeys > nk) {
    // keys past the request: their V is stale memory (maybe non-finite)
#pragma unroll
    for (int m2 = 0; m2 < 2; ++m2) {
      if constexpr (VT) {
        // element j of vt[m2][c] is key key0 + 16*m2 + 8*hh + j
        uint32_t keep[4];
#pragma unroll
        for (int pr = 0; pr < 4; ++pr) {
          const int k0 = key0 + 16 * m2 + 8 * hh + 2 * pr;
          keep[pr] = (k0 < nk ? 0x0000FFFFu : 0u) | (k0 + 1 < nk ? 0xFFFF0000u : 0u);
        }
#pragma unroll
        for (int c = 0; c < DPL; ++c) {
          typedef unsigned u32x4v __attribute__((ext_vector_type(4)));
          u32x4v x = __builtin_bit_cast(u32x4v, buf.vt[m2][c]);
          x.x &= keep[0];
          x.y &= keep[1];
          x.z &= keep[2];
          x.w &= keep[3];
          buf.vt[m2][c] = __builtin_bit_cast(bf16x8, x);
        }
      } else {
#pragma unroll
        for (int t = 0; t < 2; ++t)
#pragma unroll
          for (int e = 0; e < 4; ++e)
#pragma unroll
            for (int w = 0; w < D / 64; ++w)
              buf.v[m2][t][e][w] = key0 + 16 * m2 + 8 * t + 4 * hh + e < nk ? buf.v[m2][t][e][w] : 0u;
      }
    }
  }
  const bool need_mask = key0 + kBlockKeys > L;
#pragma unroll
  for (int tt = 0; tt < kUnitTiles; ++tt) {
    if (tt >= nt) break;  // wave-uniform
    floatx16 s = floatx16{};
#pragma unroll
    for (int kk = 0; kk < KK; ++kk)
      s = __builtin_amdgcn_mfma_f32_32x32x16_bf16(buf.k[kk], qop[tt][kk], s, 0, 0, 0);

    // keys of acc reg r: key0 + key_of_reg(r, hh).  Scores stay unscaled
    // here; the (positive) scale is folded into the exponent below, and the
    // running max m is kept in the scaled log2 domain.
    if (need_mask) {
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int key = key0 + key_of_reg<VT>(r, hh);
        const bool vis = key < L || (key < nk && ((anc[tt] >> (unsigned)(key - L)) & 1ull));
        s[r] = vis ? s[r] : -INFINITY;
      }
    }
    float mb = s[0];
#pragma unroll
    for (int r = 1; r < 16; ++r) mb = fmaxf(mb, s[r]);
    mb = max_across_halves(mb);
    // Lazy rescaling: the reference max m only moves (and the accumulators
    // are rescaled) once some row's block max exceeds it by more than
    // kRescaleSlack; until then p <= 2^kRescaleSlack, exact in fp32 sums
    // and bf16 P.  m is also taken on the first visible key (m = -inf).
    const float mcand = fmaxf(m[tt], mb * scale_log2);
    if (__builtin_amdgcn_ballot_w64(mcand > m[tt] + kRescaleSlack) != 0ull) {
      const float alpha = fast_exp2(m[tt] - (mcand == -INFINITY ? 0.f : mcand));
      l[tt] *= alpha;
#pragma unroll
      for (int c = 0; c < DPL; ++c) acc[tt][c] *= alpha;
      m[tt] = mcand;
    }
    const float mref = m[tt] == -INFINITY ? 0.f : m[tt];
    float psum = 0.f;
    uint32_t pw[8];
#pragma unroll
    for (int r = 0; r < 16; r += 2) {
      const float p0 = fast_exp2(__builtin_fmaf(s[r], scale_log2, -mref));
      const float p1 = fast_exp2(__builtin_fmaf(s[r + 1], scale_log2, -mref));
      psum += p0 + p1;
      pw[r >> 1] = pack_bf16x2(p0, p1);
    }
    l[tt] += psum;
#pragma unroll
    for (int m2 = 0; m2 < 2; ++m2) {
      uint32_t w4p[4] = {pw[4 * m2], pw[4 * m2 + 1], pw[4 * m2 + 2], pw[4 * m2 + 3]};
      const bf16x8 pop = __builtin_bit_cast(bf16x8, w4p);
      if constexpr (VT) {
        // k-slot 8hh + j <-> key 16*m2 + 8hh + j in both operands
#pragma unroll
        for (int c = 0; c < DPL; ++c)
          acc[tt][c] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(buf.vt[m2][c], pop, acc[tt][c], 0, 0, 0);
      } else {
        // k-slot 8hh + 4t + e <-> key 16*m2 + 8t + 4hh + e in both operands;
        // the V^T operand of column c is element c of the lane's d-run
#pragma unroll
        for (int c = 0; c < DPL; ++c) {
          uint32_t w4[4];
#pragma unroll
          for (int pr = 0; pr < 4; ++pr) {
            const int s0 = 2 * pr, s1 = 2 * pr + 1;
            const uint32_t x0 = buf.v[m2][s0 >> 2][s0 & 3][c >> 1];
            const uint32_t x1 = buf.v[m2][s1 >> 2][s1 & 3][c >> 1];
            w4[pr] = (c & 1) ? pack_hi16(x0, x1) : pack_lo16(x0, x1);
          }
          const bf16x8 vop = __builtin_bit_cast(bf16x8, w4);
          acc[tt][c] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vop, pop, acc[tt][c], 0, 0, 0);
        }
      }
    }
  }
}

// --------------------------------------------------------------------------
// merge the partials of units cut by workgroup range boundaries.  A cut unit
// u spans ranges w0 < w1; it is merged by the workgroups of merge slot
// w0 + 1 (the first range that starts inside it), so each cut unit is merged
// exactly once.  Each merge slot has kTileRows / kMergeRows workgroups of
// kMergeRows waves; a wave merges row n of each of the unit's tiles in turn.
// First the lanes read the pieces' log-sum-exps side by side (64 pieces per
// load) for the common maximum and the normaliser; then the weighted rows are
// summed with every lane holding D/64 consecutive columns, so a row's
// partials are read as 64-lane contiguous runs, eight pieces' loads in flight
// at a time (none of them waits on the sum so far).
// --------------------------------------------------------------------------
constexpr int kMergeRows = 4;

template <int D>
__global__ __launch_bounds__(64 * kMergeRows) void attn_merge_kernel(AttnArgs a) {
  constexpr int DPT = D / 64;
  const int32_t *hdr = reinterpret_cast<const int32_t *>(a.ws + kWsHdr);
  constexpr int kChunks = kTileRows / kMergeRows;
  const int wm = blockIdx.x / kChunks;
  const UnitRec mr = reinterpret_cast<const UnitRec *>(a.ws + kWsMergeRec)[wm];
  if (wm >= hdr[1] || mr.a.x < 0) return;  // no cut unit to merge here
  const int w0 = mr.a.y, w1 = mr.a.z, side0 = mr.a.w;
  const int o = mr.b.x, qn = mr.b.y, h = mr.b.z, rowgroup = mr.b.w;
  const int n = (blockIdx.x - wm * kChunks) * kMergeRows + (threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  const int G = a.group;
  const float *pl = reinterpret_cast<const float *>(a.ws + kWsPartLse);
  const float *po = reinterpret_cast<const float *>(a.ws + kWsPartO);
  // range w0 holds the unit's first block (its first or second partial
  // slot); every later range starts inside the unit (first slot).  No range
  // between w0 and w1 is empty: distinct cost targets inside one unit map to
  // distinct blocks, so an empty range can only begin at a unit start.
  const int np = w1 - w0 + 1;
  auto slot_of = [&](int k, int tt) {
    const int w = w0 + k;
    return (2 * (size_t)w + (k == 0 ? side0 : 0)) * kUnitTiles + tt;
  };
  // rows of pieces k0 + j0 .. k0 + j0 + 7 of tile tt (past the last piece:
  // the last one again, weighted 0 by the caller)
  auto load8 = [&](int tt, int k0, int j0, int kn, float (&x)[8][DPT]) {
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const size_t row = (slot_of(k0 + min(j0 + u, kn - 1), tt) * kTileRows + n) * D;
      if constexpr (DPT == 2) {
        const float2 xv = reinterpret_cast<const float2 *>(po + row)[lane];
        x[u][0] = xv.x;
        x[u][1] = xv.y;
      } else {
        x[u][0] = po[row + lane];
      }
    }
  };
  // The first loads of every tile go out together: each piece's
  // log-sum-exp (lane k holds piece k) and the first eight pieces' rows, so
  // a unit cut into a few pieces costs one memory round trip for all of its
  // tiles rather than one per tile.
  bool valid[kUnitTiles];
  float ls0[kUnitTiles];
  float x0[kUnitTiles][8][DPT];
#pragma unroll
  for (int tt = 0; tt < kUnitTiles; ++tt) {
    valid[tt] = (rowgroup * kUnitTiles + tt) * kTileRows + n < G * qn;
    if (valid[tt]) {
      ls0[tt] = lane < np ? pl[slot_of(lane, tt) * kTileRows + n] : -INFINITY;
      load8(tt, 0, 0, min(64, np), x0[tt]);
    }
  }
#pragma unroll
  for (int tt = 0; tt < kUnitTiles; ++tt) {
    if (!valid[tt]) break;  // rows of a unit are a prefix of its tiles
    const int R = (rowgroup * kUnitTiles + tt) * kTileRows + n;
    const int tok = R / G, gq = R - tok * G;
    float acc[DPT];
#pragma unroll
    for (int t = 0; t < DPT; ++t) acc[t] = 0.f;
    auto add8 = [&](int j0, int kn, float wl, const float (&x)[8][DPT]) {
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        const int j = min(j0 + u, kn - 1);
        const float wt = j0 + u < kn ? __uint_as_float(__builtin_amdgcn_readlane(__float_as_uint(wl), j)) : 0.f;
#pragma unroll
        for (int t = 0; t < DPT; ++t) acc[t] += wt * x[u][t];
      }
    };
    // the common maximum over the pieces' log-sum-exps, 64 pieces per load
    float M = wave_max(ls0[tt]);
    for (int k0 = 64; k0 < np; k0 += 64)
      M = fmaxf(M, wave_max(k0 + lane < np ? pl[slot_of(k0 + lane, tt) * kTileRows + n] : -INFINITY));
    const float Mref = M == -INFINITY ? 0.f : M;
    float den = 0.f;
    for (int k0 = 0; k0 < np; k0 += 64) {
      const float ls = k0 == 0 ? ls0[tt] : (k0 + lane < np ? pl[slot_of(k0 + lane, tt) * kTileRows + n] : -INFINITY);
      const float wl = ls == -INFINITY ? 0.f : fast_exp2(ls - Mref);  // piece k0+lane's weight
      den += wave_sum(wl);
      const int kn = min(64, np - k0);
      for (int j0 = 0; j0 < kn; j0 += 8) {
        if (k0 == 0 && j0 == 0) {
          add8(0, kn, wl, x0[tt]);
        } else {
          float x[8][DPT];
          load8(tt, k0, j0, kn, x);
          add8(j0, kn, wl, x);
        }
      }
    }
    const float inv = den > 0.f ? 1.0f / den : 0.f;
    uint16_t *orow = a.out + ((size_t)(o + tok) * a.num_q_heads + (size_t)h * G + gq) * D;
    if constexpr (DPT == 2)
      reinterpret_cast<uint32_t *>(orow)[lane] = pack_bf16x2(acc[0] * inv, acc[1] * inv);
    else
      orow[lane] = (uint16_t)bf16_bits(acc[0] * inv);
  }
}

// --------------------------------------------------------------------------
// attention (persistent workgroups)
// --------------------------------------------------------------------------
// A unit piece of one workgroup's block range, placed on the workgroup's
// sequence of rounds (in round r of a piece, wave w takes global block
// ps + 4r + w).  Everything here is wave-uniform.
// Unit records are written by the plan launch and only read here, so they are
// read through the scalar cache: a vector load would be counted by vmcnt,
// and waiting for it (its value is needed at once) would also wait for every
// K/V load issued before it.
struct const_unit_ptr {
  const_i32_ptr p;  // UnitRec[]: 12 int32 each
  __device__ UnitRec operator[](int u) const {
    const const_i32_ptr q = p + 12 * (size_t)u;
    UnitRec r;
    r.a = make_int4(q[0], q[1], q[2], q[3]);
    r.b = make_int4(q[4], q[5], q[6], q[7]);
    r.c = make_int4(q[8], q[9], q[10], q[11]);
    return r;
  }
};

struct Walk {
  int u, i, h, rg, ub, o, qn, L, nblk;
  int s, ot;   // first verify token of the rows; the request's first parent entry
  int ps, pe;  // global blocks [ps, pe) of the unit processed by this workgroup
  int g0, nr;  // its rounds [g0, g0 + nr)
  bool has_next;
  UnitRec next;  // record of unit u+1 (fetched after entry, needed at the next advance)
};

__device__ inline void walk_enter(Walk &W, int u, const UnitRec &r, int start, int end, int g0,
                                  const_unit_ptr units, int n_units) {
  W.u = u;
  W.i = r.a.x; W.h = r.a.y; W.rg = r.a.z; W.ub = r.a.w;
  W.o = r.b.x; W.qn = r.b.y; W.L = r.b.z; W.nblk = r.b.w;
  W.s = r.c.x; W.ot = r.c.y;
  W.ps = max(W.ub, start);
  W.pe = min(W.ub + W.nblk, end);
  W.g0 = g0;
  W.nr = (W.pe - W.ps + kAttnWaves - 1) / kAttnWaves;
  W.has_next = W.pe < end && u + 1 < n_units;
}

// Moves the walk forward until round g lies in its piece; false if g is past
// the workgroup's last piece (the walk then stays on the last piece).  Each
// unit entered fetches the record of the unit after it.
__device__ inline bool walk_to(Walk &W, int g, int start, int end, const_unit_ptr units,
                               int n_units) {
  while (g >= W.g0 + W.nr) {
    if (!W.has_next) return false;
    const UnitRec r = W.next;
    walk_enter(W, W.u + 1, r, start, end, W.g0 + W.nr, units, n_units);
    if (W.has_next) W.next = units[W.u + 1];
  }
  return true;
}

// Q^T operand chunks this wave stages for tile tt of a unit: kk = wave*KQ ..
// +KQ-1, for every lane's query row (lane n, half hh).
template <int D>
__device__ inline void load_q_chunks(const AttnArgs &a, const Walk &W, int tt, int wave, int n, int hh,
                                     bf16x8 (&qc)[D / 64]) {
  constexpr int KQ = D / 64;
  const int G = a.group;
  const int R = (W.rg * kUnitTiles + tt) * kTileRows + n;
  const bool row_ok = R < G * W.qn;
  const int tok = row_ok ? R / G : 0;
  const int gq = R - (R / G) * G;
  const uint16_t *qrow =
      a.q + ((size_t)(W.o + tok) * a.num_q_heads + (size_t)W.h * G + gq) * D + 8 * hh;
#pragma unroll
  for (int j = 0; j < KQ; ++j)
    qc[j] = row_ok ? *reinterpret_cast<const bf16x8 *>(qrow + 16 * (wave * KQ + j)) : bf16x8{};
}

// --------------------------------------------------------------------------
// Phase timeline, compiled in diagnostic builds only (SV_PHASE_TRACE; the
// library is then libspecverify_trace.so).  Lane 0 of every wave of range w
// stores up to kPhaseEvents words (time << 8 | code) at
// g_phase_trace[(w * kAttnWaves + wave) * kPhaseEvents + i], time read with
// s_memtime (shader clock, counted per XCD, so only differences within one
// wave are meaningful).  Codes:
//   1 range header read      2 first unit's Q operands in registers
//   3 round start            4 next round's K/V loads issued
//   5 this round's K/V in    6 block computed (or skipped)
//   7 unit merged and written  8 next unit entered      9 range done
// To tell the wait for data from the arithmetic, a trace build waits for the
// whole of a round's K/V before its block (the production build waits load by
// load), and requests the page ids of round g+2 after the block, since every
// timestamp read would otherwise wait for them; both shift the schedule
// slightly.
#ifdef SV_PHASE_TRACE
constexpr int kPhaseEvents = 2048;
__device__ uint64_t g_phase_trace[(size_t)kMaxGrid * kAttnWaves * kPhaseEvents];
#define SV_MARK(code)                                                                              \
  do {                                                                                             \
    const uint64_t sv_t = __builtin_amdgcn_s_memtime();                                            \
    if (lane == 0 && sv_ev < kPhaseEvents)                                                         \
      g_phase_trace[((size_t)wg * kAttnWaves + wave) * kPhaseEvents + sv_ev] = (sv_t << 8) | (code); \
    ++sv_ev;                                                                                       \
  } while (0)
#else
#define SV_MARK(code) ((void)0)
#endif

// s_waitcnt operand for vmcnt(n) with the other counters unconstrained
constexpr int waitcnt_vm(int n) { return (n & 15) | ((n >> 4) << 14) | (7 << 4) | (15 << 8); }

template <int D, bool VT>
__global__ __launch_bounds__(64 * kAttnWaves) __attribute__((amdgpu_waves_per_eu(1, 1))) void verify_attn_kernel(AttnArgs a) {
  constexpr int DPL = D / 32;  // contiguous d per lane of a V row; O^T tiles
  constexpr int KK = D / 16;   // k-steps of the S^T product (16 d each)
  constexpr int KQ = D / 64;   // Q chunks staged per wave
  static_assert(D == 64 || D == 128, "head_dim");
  // O^T accumulators of the waves, four registers per 16-byte entry:
  // [wave][tile column c][register group j][lane] holds registers 4j..4j+3
  __shared__ float4v sm_o[kAttnWaves][DPL][4][64];
  __shared__ float sm_m[kAttnWaves][32];
  __shared__ float sm_l[kAttnWaves][32];
  __shared__ bf16x8 sm_q[kUnitTiles][KK][64];  // Q^T operands, [tile][kk][lane], shared by the waves

  // header words 1..3 are not written by this launch (word 0 only, by atomics)
  const const_i32_ptr hdr = (const_i32_ptr)(uintptr_t)(a.ws + kWsHdr);
  const int P = hdr[1];
  // consecutive ranges on the same XCD (workgroups are dealt round-robin to
  // the 8 XCDs), so units that share K/V (tile groups of one head) meet in
  // one L2
  const int bx = blockIdx.x;
  const int wg = (a.grid % 8 == 0) ? (bx % 8) * (a.grid / 8) + bx / 8 : bx;
  const const_i32_ptr wg_start = (const_i32_ptr)(uintptr_t)(a.ws + kWsWgStart);
  const const_unit_ptr units{(const_i32_ptr)(uintptr_t)(a.ws + ws_units_offset(D))};
  // Everything the range needs first is read in one round trip, before the
  // range count is checked: the per-workgroup arrays have kMaxGrid (+1)
  // entries and wg < grid <= kMaxGrid, so these reads stay in bounds.
  const int n_units = hdr[3];
  const int start0 = wg_start[wg];
  const int end0 = wg_start[wg + 1];
  const int first0 = ((const_i32_ptr)(uintptr_t)(a.ws + kWsWgFirst))[wg];
  const UnitRec rec0 = const_unit_ptr{(const_i32_ptr)(uintptr_t)(a.ws + kWsWgRec)}[wg];
  // one test of all of them (a consistent plan gives every range that holds
  // blocks a first unit of a request i >= 0 with at least one block, whose
  // rows start at a verify token s >= 0)
  if ((wg >= P) | (first0 < 0) | (first0 >= n_units) | (start0 >= end0) | (rec0.a.x < 0) | (rec0.b.w < 1) |
      (rec0.c.x < 0))
    return;

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int n = lane & 31, hh = lane >> 5;
#ifdef SV_PHASE_TRACE
  int sv_ev = 0;
#endif
  SV_MARK(1);
  const int G = a.group;
  const size_t page_stride = (size_t)a.num_kv_heads * kPage * D;
  bool bad_page = false;

  // The workgroup's block range w, [start, end), whose first unit and its
  // record are given.  (Written as a function: the compiler then keeps far
  // fewer scalars live through the round loop, and spills fewer of them to
  // vector-register lanes.)
  auto run_range = [&](const int w, const int start, const int end, const int first_unit, const UnitRec &rec0) {

    // Two walks over the same pieces: the consumer at the round being
    // computed, the producer two rounds ahead (it fetches page ids for round
    // g+2 and issues the K/V loads of round g+1 into the buffer freed by round
    // g-1), so K/V streaming runs on across unit boundaries.
    Walk Wc, Wp;
    walk_enter(Wc, first_unit, rec0, start, end, 0, units, n_units);
    Wp = Wc;

    // per-unit consumer context, one entry per query tile of the unit
    int nt = 1;  // tiles of the consumer's unit
    uint64_t anc[kUnitTiles];
    int nk = 0;
    float m[kUnitTiles], l[kUnitTiles];
    floatx16 acc[kUnitTiles][DPL];
    bf16x8 qpf[kUnitTiles][KQ];  // this wave's Q chunks of every tile of unit qpf_u, read ahead
    int par_pf = -1;             // and the lane's parent entry of that unit
    int qpf_u = -1;

    // enter the consumer's unit: ancestor masks of the lane's rows and Q in LDS
    // A unit's parent entries and Q chunks are read ahead: the range's first
    // unit's at kernel entry, so those round trips overlap the page-id reads,
    // a later unit's in the second round of the unit before it, ahead of that
    // round's K/V loads.  Loads retire in order, so a value read at entry
    // itself would make the wave wait for the next round's K/V loads too (a
    // whole memory round trip per unit); only a unit of one round reads them
    // at entry.
    auto enter_unit = [&]() {
      if (qpf_u != Wc.u) {
        // a unit of one round: read now, and waited for here, so that the
        // path below (and its registers) is the same as after a prefetch
        par_pf = tree_parent_of(a.tree_parent, Wc.ot, Wc.s + Wc.qn, lane);
#pragma unroll
        for (int tt = 0; tt < kUnitTiles; ++tt) load_q_chunks<D>(a, Wc, tt, wave, n, hh, qpf[tt]);
        __builtin_amdgcn_s_waitcnt(waitcnt_vm(0));
      }
      // masks of the verify tokens [0, s+q) (keys L .. L+s+q-1); row r of the
      // unit's tiles is token s + r / G
      bool parents_ok;
      const int par = par_pf;
      const uint64_t anc_all = ancestor_mask_of(a.tree_parent != nullptr, par, Wc.s + Wc.qn, lane, &parents_ok);
      if (!parents_ok && threadIdx.x == 0 && Wc.ps == Wc.ub && Wc.h == 0 && Wc.rg == 0)
        atomicOr(reinterpret_cast<unsigned *>(a.ws + kWsHdr), SV_DEV_BAD_PARENT);
      nt = min(kUnitTiles, (G * Wc.qn + kTileRows - 1) / kTileRows - Wc.rg * kUnitTiles);
#pragma unroll
      for (int tt = 0; tt < kUnitTiles; ++tt) {
        const int R = (Wc.rg * kUnitTiles + tt) * kTileRows + n;
        const bool row_ok = R < G * Wc.qn;
        const int tok = row_ok ? R / G : 0;
        // the shuffle must run on every lane: a source lane whose own row is
        // past the end would be inactive and read back as zero
        const uint64_t anc_tok = __shfl(anc_all, Wc.s + tok);
        anc[tt] = row_ok ? anc_tok : 0ull;
        m[tt] = -INFINITY;
        l[tt] = 0.f;
#pragma unroll
        for (int c = 0; c < DPL; ++c) acc[tt][c] = floatx16{};
      }
      nk = Wc.L + Wc.s + Wc.qn;
#pragma unroll
      for (int tt = 0; tt < kUnitTiles; ++tt) {
        if (tt >= nt) break;
#pragma unroll
        for (int j = 0; j < KQ; ++j) sm_q[tt][wave * KQ + j][lane] = qpf[tt][j];
      }
      qpf_u = -1;
    };

    // The unit's Q^T operands stay in registers while it runs: read from LDS
    // once per unit instead of once per block, the hot loop has no LDS reads
    // to wait for before its MFMAs.
    bf16x8 qop[kUnitTiles][KK];
    auto load_qop = [&]() {
#pragma unroll
      for (int tt = 0; tt < kUnitTiles; ++tt) {
        if (tt >= nt) break;
#pragma unroll
        for (int kk = 0; kk < KK; ++kk) qop[tt][kk] = sm_q[tt][kk][lane];
      }
    };

    // producer: page ids and head of the round it will load next
    int2 pg_next = make_int2(0, 0);
    int h_next = Wp.h;
    auto fetch_pages = [&](int g) {
      walk_to(Wp, g, start, end, units, n_units);
      const int lbk = (Wp.ps - Wp.ub) + kAttnWaves * min(g - Wp.g0, Wp.nr - 1) + wave;
      const int lmax = Wp.pe - Wp.ub - 1;  // a wave without a block re-reads the piece's last one
      const const_i32_ptr bt = (const_i32_ptr)(uintptr_t)(a.block_tables + (size_t)Wp.i * a.max_blocks);
      const int npages = (Wp.L + Wp.s + Wp.qn + kPage - 1) / kPage;
      pg_next = block_pages(bt, min(lbk, lmax), npages, a.num_pages, &bad_page);
      h_next = Wp.h;
    };
    auto produce = [&](KVBlock<D, VT> &buf) {
      load_block<D, VT>(buf, a.k_cache + (size_t)h_next * kPage * D, a.v_cache + (size_t)h_next * kPage * D,
                    pg_next, n, hh, page_stride);
    };

    // finish the consumer's unit: per tile, merge the waves through LDS and
    // write the output or a partial
    auto finish_unit = [&]() {
      const bool whole = Wc.ps == Wc.ub && Wc.pe == Wc.ub + Wc.nblk;
      const int side = Wc.u == first_unit ? 0 : 1;
#pragma unroll
      for (int tt = 0; tt < kUnitTiles; ++tt) {
        if (tt >= nt) break;
        if (tt > 0) __syncthreads();  // every wave has read the previous tile's sm_o
        const float lt = l[tt] + __shfl_xor(l[tt], 32);  // both lane halves summed different keys of a row
        if (hh == 0) {
          sm_m[wave][n] = m[tt];
          sm_l[wave][n] = lt;
        }
#pragma unroll
        for (int c = 0; c < DPL; ++c)
#pragma unroll
          for (int j = 0; j < 4; ++j)
            sm_o[wave][c][j][lane] = float4v{acc[tt][c][4 * j], acc[tt][c][4 * j + 1], acc[tt][c][4 * j + 2],
                                             acc[tt][c][4 * j + 3]};
        __syncthreads();
        float M = -INFINITY;
#pragma unroll
        for (int ww = 0; ww < kAttnWaves; ++ww) M = fmaxf(M, sm_m[ww][n]);
        const float Mref = M == -INFINITY ? 0.f : M;
        float f[kAttnWaves];
        float Lsum = 0.f;
#pragma unroll
        for (int ww = 0; ww < kAttnWaves; ++ww) {
          f[ww] = fast_exp2(sm_m[ww][n] - Mref);
          Lsum += f[ww] * sm_l[ww][n];
        }
        // this wave finalises registers r = 4*wave .. 4*wave+3 of every tile c,
        // O^T rows i = 8*wave + 4*hh + rr: with transposed V pages output
        // d = 32*c + i (ov[4c + rr], four contiguous per c); with token-major
        // pages d = DPL*i + c (ov[DPL*rr + c], 4*DPL contiguous)
        float ov[4 * DPL];
#pragma unroll
        for (int i = 0; i < 4 * DPL; ++i) ov[i] = 0.f;
#pragma unroll
        for (int c = 0; c < DPL; ++c)
#pragma unroll
          for (int ww = 0; ww < kAttnWaves; ++ww) {
            const float4v x = sm_o[ww][c][wave][lane];
#pragma unroll
            for (int rr = 0; rr < 4; ++rr) ov[VT ? 4 * c + rr : DPL * rr + c] += f[ww] * x[rr];
          }
        const float inv = Lsum > 0.f ? 1.0f / Lsum : 0.f;
        const int d0 = VT ? 8 * wave + 4 * hh : DPL * (8 * wave + 4 * hh);
        const int R = (Wc.rg * kUnitTiles + tt) * kTileRows + n;
        if (R < G * Wc.qn) {
          const int tok = R / G, gq = R - tok * G;
          if (whole) {
            uint16_t *orow = a.out + ((size_t)(Wc.o + tok) * a.num_q_heads + (size_t)Wc.h * G + gq) * D + d0;
            if constexpr (VT) {
#pragma unroll
              for (int c = 0; c < DPL; ++c)
                *reinterpret_cast<uint2 *>(orow + 32 * c) =
                    make_uint2(pack_bf16x2(ov[4 * c] * inv, ov[4 * c + 1] * inv),
                               pack_bf16x2(ov[4 * c + 2] * inv, ov[4 * c + 3] * inv));
            } else {
#pragma unroll
              for (int j = 0; j < 4 * DPL; j += 8)
                *reinterpret_cast<uint4 *>(orow + j) =
                    make_uint4(pack_bf16x2(ov[j] * inv, ov[j + 1] * inv), pack_bf16x2(ov[j + 2] * inv, ov[j + 3] * inv),
                               pack_bf16x2(ov[j + 4] * inv, ov[j + 5] * inv), pack_bf16x2(ov[j + 6] * inv, ov[j + 7] * inv));
            }
          } else {
            const size_t slot = (2 * (size_t)w + side) * kUnitTiles + tt;
            float *po = reinterpret_cast<float *>(a.ws + kWsPartO) + (slot * kTileRows + n) * D + d0;
            if constexpr (VT) {
#pragma unroll
              for (int c = 0; c < DPL; ++c)
                *reinterpret_cast<float4 *>(po + 32 * c) =
                    make_float4(ov[4 * c] * inv, ov[4 * c + 1] * inv, ov[4 * c + 2] * inv, ov[4 * c + 3] * inv);
            } else {
#pragma unroll
              for (int j = 0; j < 4 * DPL; j += 4)
                *reinterpret_cast<float4 *>(po + j) =
                    make_float4(ov[j] * inv, ov[j + 1] * inv, ov[j + 2] * inv, ov[j + 3] * inv);
            }
            if (wave == 0 && hh == 0) {
              float *pl = reinterpret_cast<float *>(a.ws + kWsPartLse);
              pl[slot * kTileRows + n] = Lsum > 0.f ? Mref + fast_log2(Lsum) : -INFINITY;
            }
          }
        }
      }
    };

    // one round g: issue the loads of round g+1 into `into` (freed by round
    // g-1), compute round g from `cur`; true once the last unit is finished
    auto round = [&](int g, KVBlock<D, VT> &cur, KVBlock<D, VT> &into) -> bool {
      SV_MARK(3);
      // read ahead the next unit's parent entries and Q chunks once this unit
      // is under way, before this round's K/V loads (see enter_unit)
      if (Wc.has_next && qpf_u != Wc.u + 1 && g == Wc.g0 + 1) {
        Walk Wn;
        walk_enter(Wn, Wc.u + 1, Wc.next, start, end, 0, units, 0);
        par_pf = tree_parent_of(a.tree_parent, Wn.ot, Wn.s + Wn.qn, lane);
#pragma unroll
        for (int tt = 0; tt < kUnitTiles; ++tt) load_q_chunks<D>(a, Wn, tt, wave, n, hh, qpf[tt]);
        qpf_u = Wc.u + 1;
      }
      produce(into);
#ifndef SV_PHASE_TRACE
      fetch_pages(g + 2);
#endif
      const int gb = Wc.ps + kAttnWaves * (g - Wc.g0) + wave;  // this wave's global block
      SV_MARK(4);
#ifdef SV_PHASE_TRACE
      // this round's K/V (the loads before the next round's); a Q prefetch
      // issued this round makes it wait for two of the next round's loads too
      __builtin_amdgcn_s_waitcnt(waitcnt_vm(KK + (VT ? D / 16 : 16)));
#endif
      SV_MARK(5);
      if (gb < Wc.pe)
        compute_block<D, VT>(cur, qop, nt, (gb - Wc.ub) * kBlockKeys, Wc.L, nk, anc, hh,
                         a.scale_log2, m, l, acc);
      SV_MARK(6);
#ifdef SV_PHASE_TRACE
      fetch_pages(g + 2);
#endif
      if (g + 1 == Wc.g0 + Wc.nr) {
        finish_unit();
        SV_MARK(7);
        if (!Wc.has_next) return true;
        walk_to(Wc, g + 1, start, end, units, n_units);
        enter_unit();
        __syncthreads();  // the next unit's Q is in LDS; sm_o may be reused
        load_qop();
        SV_MARK(8);
      }
      return false;
    };

    // The first unit's parent entries and Q chunks (tiles with no rows load
    // nothing) go out first, then the page ids are requested and the first
    // K/V loads issued; the Q operands are staged through LDS after that, so
    // the memory round trips overlap.
    KVBlock<D, VT> A, Bb;
    par_pf = tree_parent_of(a.tree_parent, Wc.ot, Wc.s + Wc.qn, lane);
#pragma unroll
    for (int tt = 0; tt < kUnitTiles; ++tt) load_q_chunks<D>(a, Wc, tt, wave, n, hh, qpf[tt]);
    qpf_u = Wc.u;
    fetch_pages(0);
    produce(A);
    if (Wc.has_next) {  // the first unit's successor, read once the first K/V loads are out
      Wc.next = units[Wc.u + 1];
      Wp.next = Wc.next;
    }
    fetch_pages(1);
    enter_unit();
    __syncthreads();
    load_qop();
    SV_MARK(2);
    for (int g = 0;; g += 2) {
      if (round(g, A, Bb)) break;
      if (round(g + 1, Bb, A)) break;
    }
  };

  run_range(wg, start0, end0, first0, rec0);
  SV_MARK(9);
  if (bad_page) atomicOr(reinterpret_cast<unsigned *>(a.ws + kWsHdr), SV_DEV_BAD_PAGE);
}

}  // namespace

hipError_t verify_attn_phase_trace(void *host_dst, size_t bytes, bool clear, size_t *total) {
#ifdef SV_PHASE_TRACE
  *total = sizeof(g_phase_trace);
  hipError_t e = hipDeviceSynchronize();
  if (e == hipSuccess && host_dst != nullptr && bytes > 0)
    e = hipMemcpyFromSymbol(host_dst, HIP_SYMBOL(g_phase_trace), bytes < *total ? bytes : *total, 0,
                            hipMemcpyDeviceToHost);
  if (e == hipSuccess && clear) {
    void *p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(g_phase_trace));
    if (e == hipSuccess) e = hipMemset(p, 0, *total);
    if (e == hipSuccess) e = hipDeviceSynchronize();
  }
  return e;
#else
  (void)host_dst;
  (void)bytes;
  (void)clear;
  *total = 0;
  return hipErrorNotSupported;
#endif
}

void launch_verify_attn_plan(const AttnArgs &a, hipStream_t stream) {
  attn_plan_kernel<<<1, kPlanThreads, 0, stream>>>(a);
}

void launch_verify_attn_run(const AttnArgs &a, int head_dim, hipStream_t stream) {
  const dim3 grid(a.grid), block(64 * kAttnWaves);
  if (head_dim == 128) {
    if (a.v_transposed)
      verify_attn_kernel<128, true><<<grid, block, 0, stream>>>(a);
    else
      verify_attn_kernel<128, false><<<grid, block, 0, stream>>>(a);
    attn_merge_kernel<128><<<a.grid * (kTileRows / kMergeRows), 64 * kMergeRows, 0, stream>>>(a);
  } else {
    if (a.v_transposed)
      verify_attn_kernel<64, true><<<grid, block, 0, stream>>>(a);
    else
      verify_attn_kernel<64, false><<<grid, block, 0, stream>>>(a);
    attn_merge_kernel<64><<<a.grid * (kTileRows / kMergeRows), 64 * kMergeRows, 0, stream>>>(a);
  }
}

}  // namespace sv
