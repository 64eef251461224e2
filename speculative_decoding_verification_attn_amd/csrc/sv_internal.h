// Internal declarations shared by the HIP translation units of libspecverify.
// gfx950 (CDNA4) only: wave64, MFMA bf16 32x32x16, hardware bf16 conversion.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "spec_verify.h"

namespace sv {

constexpr int kPage = 16;          // tokens per KV page
constexpr int kMaxTokens = 64;     // verify tokens per request (one u64 ancestor word)
constexpr int kBlockKeys = 32;     // keys per MFMA block (two pages)
constexpr int kTileRows = 32;      // query rows per MFMA tile
constexpr int kUnitTiles = 2;      // query tiles of one (request, KV head) sharing each K/V block
constexpr int kAttnWaves = 4;      // waves per attention workgroup (they split the keys)
constexpr int kMaxGrid = 512;      // persistent attention workgroups (one per CU, capped)
constexpr int kMinBlocksPerWG = 8; // at least two 32-key blocks per wave: fewer, longer ranges for small problems
// Range sizing charges each unit start (after the first) this many blocks:
// finishing a unit (merging it across the waves, writing it out) and entering
// the next one stalls a workgroup's stream for two to three rounds of four
// blocks (measured per-workgroup time grows by 4.4-7 us per unit entered, a
// round takes about 2.7 us); a sweep of 4, 8, 12 and 16 put 12 at or near the
// best on every workload measured.
constexpr int kUnitStartCost = 12;
constexpr int kPlanThreads = 1024;
constexpr int kPlanLdsRequests = 4096;  // per-request plan data kept in LDS up to this batch

// ---------------------------------------------------------------------------
// Verify-attention workspace layout (byte offsets, all 256-byte aligned).
//
// A "unit" is one (request, KV head, group of up to kUnitTiles 32-row query
// tiles) triple; its keys are the request's ceil((L+q)/32) blocks of 32 keys,
// and every block a unit loads serves all of its tiles.  All units' blocks form one
// global block sequence, cut into contiguous ranges of equal cost (blocks plus
// a fixed charge per unit start), one per persistent workgroup.  A unit wholly inside one range is written straight
// to the output; a unit cut by range boundaries leaves one partial per
// workgroup that touched it (at most two per workgroup, each with one partial
// per tile), merged afterwards.
// ---------------------------------------------------------------------------
// A unit record: {request, kv head, tile group, first global block},
// {first row o, rows q, context L, blocks per unit} and {first verify token s
// of the rows, the request's first entry in the tree parent array, -, -}.
// Row r of the unit's request is verify token s + r, in row o + r of q and
// out (o = the request's first verify token's row + s: a chunk's rows are
// read and written in place); its keys are the L + s + q slots
// [0, L + s + q).  s = 0 except for chunked verification.
struct UnitRec {
  int4 a;
  int4 b;
  int4 c;
};

struct AttnLayout {
  size_t hdr;        // int32[8]: 0 status bits, 1 active workgroups P, 2 total blocks, 3 units
  size_t wg_start;   // int32[kMaxGrid + 1]: first global block of each workgroup's range
  size_t wg_first;   // int32[kMaxGrid]: first unit of each workgroup's range
  size_t wg_rec;     // UnitRec[kMaxGrid]: a copy of that first unit's record
  size_t merge_rec;  // UnitRec[kMaxGrid]: {cut unit merged here or -1, w0, w1, side of w0}, {o, q, head, tile}
  size_t part_lse;   // float[2*kMaxGrid][kUnitTiles][32] log2-sum-exp of partial rows
  size_t part_o;     // float[2*kMaxGrid][kUnitTiles][32][D] normalised partial outputs
  size_t units;      // UnitRec[unit_bound]
  size_t req_meta;   // int32[4][B]: unit base, block base, row tiles, blocks per unit (large batches)
  size_t total;
  int unit_bound;
};

__host__ __device__ constexpr size_t align256(size_t x) { return (x + 255) & ~size_t(255); }

// Every array up to part_o has a fixed size, so its offset is a constant
// (units follows part_o, whose size depends on head_dim only): the attention
// kernels address them from the workspace base alone, with no per-array
// kernel argument held in registers.
constexpr size_t kWsHdr = 0;
constexpr size_t kWsWgStart = align256(kWsHdr + 8 * sizeof(int32_t));
constexpr size_t kWsWgFirst = align256(kWsWgStart + size_t(kMaxGrid + 1) * sizeof(int32_t));
constexpr size_t kWsWgRec = align256(kWsWgFirst + size_t(kMaxGrid) * sizeof(int32_t));
constexpr size_t kWsMergeRec = align256(kWsWgRec + size_t(kMaxGrid) * sizeof(UnitRec));
constexpr size_t kWsPartLse = align256(kWsMergeRec + size_t(kMaxGrid) * sizeof(UnitRec));
constexpr size_t kWsPartO = align256(kWsPartLse + size_t(2 * kMaxGrid) * kUnitTiles * kTileRows * sizeof(float));
__host__ __device__ constexpr size_t ws_units_offset(int head_dim) {
  return align256(kWsPartO + size_t(2 * kMaxGrid) * kUnitTiles * kTileRows * head_dim * sizeof(float));
}

__host__ __device__ inline AttnLayout attn_layout(int batch, int total_q, int num_q_heads,
                                                  int num_kv_heads, int head_dim) {
  AttnLayout l;
  const int G = num_q_heads / num_kv_heads;
  // units per KV head: sum_i ceil(G*q_i/(32*kUnitTiles)) <= row tiles
  // sum_i ceil(G*q_i/32) <= B + ceil(G*T/32)
  const long long tiles = (long long)batch + ((long long)G * total_q + kTileRows - 1) / kTileRows;
  l.unit_bound = (int)(tiles * num_kv_heads);
  l.hdr = kWsHdr;
  l.wg_start = kWsWgStart;
  l.wg_first = kWsWgFirst;
  l.wg_rec = kWsWgRec;
  l.merge_rec = kWsMergeRec;
  l.part_lse = kWsPartLse;
  l.part_o = kWsPartO;
  size_t off = ws_units_offset(head_dim);
  l.units = off;      off = align256(off + size_t(l.unit_bound) * sizeof(UnitRec));
  l.req_meta = off;   off = align256(off + size_t(batch) * 16);
  l.total = off;
  return l;
}

struct AttnArgs {
  const uint16_t *q;
  const uint16_t *k_cache;
  const uint16_t *v_cache;
  const int32_t *block_tables;
  const int32_t *context_lens;
  const int32_t *cu_q;         // packing of the rows (the chunk's rows when chunked)
  const int32_t *tree_parent;  // parents of all verify tokens, packed by cu_full
  const int32_t *chunk_begin;  // first verify token of each request's rows, or nullptr
  const int32_t *cu_full;      // packing of all verify tokens (== cu_q unless chunked)
  uint16_t *out;
  char *ws;
  AttnLayout lay;
  int batch, total_q, num_q_heads, num_kv_heads, group, max_blocks, num_pages;
  int total_full;    // entries of tree_parent (== total_q unless chunked)
  int grid;          // persistent attention workgroups launched (<= kMaxGrid)
  float scale_log2;  // softmax scale * log2(e)
  bool v_transposed; // V pages [D][16 tokens] (else token-major [16 tokens][D], like K)
};

void launch_verify_attn_plan(const AttnArgs &a, hipStream_t stream);
void launch_verify_attn_run(const AttnArgs &a, int head_dim, hipStream_t stream);
// Phase timeline of the attention kernel (diagnostic builds only): copies up
// to `bytes` of it to host memory and/or clears it.  Returns hipErrorNotSupported
// in the production build.
hipError_t verify_attn_phase_trace(void *host_dst, size_t bytes, bool clear, size_t *total);

// ---------------------------------------------------------------------------
// Acceptance
// ---------------------------------------------------------------------------
constexpr int kArgmaxThreads = 256;
constexpr int kArgmaxTargetGroups = 2048;
constexpr int kArgmaxMinSlice = 4096;
constexpr int kArgmaxMaxSplits = 64;

struct AcceptLayout {
  size_t hdr;       // int32[8]: 0 status bits; fused launch: 2 ticket, 3 finished, 4 status cleared, 5 abort
  size_t part;      // {float value, int index}[rows][splits]
  size_t next_len;  // int32[batch]: rows of each request in the next chunk (chunked acceptance)
  size_t row_map;   // int32[rows]: chunked acceptance, the verify token (logits row) of each chunk row
  // fused acceptance + compaction only (0 otherwise)
  size_t arrive;    // int32[rows]: slices of each row done
  size_t done;      // int32[batch]: request walked, moves listed
  size_t moves;     // int32[batch][kFusedMoveWords]: move count (-1: bad path), then src, dst lists
  size_t total;
  int splits;
};
constexpr int kFusedMoveWords = 2 * kMaxTokens;

__host__ __device__ inline int argmax_splits(int total_q, int vocab) {
  int s = (kArgmaxTargetGroups + (total_q > 0 ? total_q : 1) - 1) / (total_q > 0 ? total_q : 1);
  int by_size = (vocab + kArgmaxMinSlice - 1) / kArgmaxMinSlice;
  if (s > by_size) s = by_size;
  if (s > kArgmaxMaxSplits) s = kArgmaxMaxSplits;
  if (s < 1) s = 1;
  return s;
}

// rows = logits rows (all verify tokens, or one chunk's rows)
__host__ __device__ inline AcceptLayout accept_layout(int batch, int rows, int vocab) {
  AcceptLayout l;
  l.splits = argmax_splits(rows, vocab);
  size_t off = 0;
  l.hdr = off;       off = align256(off + 8 * sizeof(int32_t));
  l.part = off;      off = align256(off + size_t(rows) * l.splits * 8);
  l.next_len = off;  off = align256(off + size_t(batch) * sizeof(int32_t));
  l.arrive = l.done = l.moves = l.row_map = 0;
  l.total = off;
  return l;
}

// chunked acceptance: rows = the most rows a chunk can have
__host__ __device__ inline AcceptLayout chunk_layout(int batch, int rows, int vocab) {
  AcceptLayout l = accept_layout(batch, rows, vocab);
  size_t off = l.total;
  l.row_map = off;  off = align256(off + size_t(rows) * sizeof(int32_t));
  l.total = off;
  return l;
}

__host__ __device__ inline AcceptLayout fused_layout(int batch, int rows, int vocab) {
  AcceptLayout l = accept_layout(batch, rows, vocab);
  size_t off = l.total;
  l.arrive = off;  off = align256(off + size_t(rows) * sizeof(int32_t));
  l.done = off;    off = align256(off + size_t(batch) * sizeof(int32_t));
  l.moves = off;   off = align256(off + size_t(batch) * kFusedMoveWords * sizeof(int32_t));
  l.total = off;
  return l;
}

struct AcceptArgs {
  const float *logits;          // [rows, vocab]; chunked: [total_q, vocab], one row per verify token
  const int32_t *draft;
  const int32_t *cu_q;
  const int32_t *tree_parent;
  int32_t *target_argmax;
  int32_t *accept_len;
  int32_t *accepted_path;
  int32_t *out_tokens;
  char *ws;
  AcceptLayout lay;
  int batch, total_q, vocab;
  int rows;                     // logits rows (== total_q); chunked: the most rows a chunk can have
  // chunked acceptance (FASER early pruning): the chunk's rows are packed by
  // cu_rows (cu_rows[batch] of them, read on the device); request i's rows
  // are its verify tokens [chunk_begin[i], chunk_begin[i] + rows_i), whose
  // logits rows are cu_q[i] + chunk_begin[i] + r
  const int32_t *cu_rows;
  const int32_t *chunk_begin;
  int chunk_size;
  int32_t *next_begin;          // [batch] out
  int32_t *next_cu;             // [batch+1] out
};

void launch_accept(const AcceptArgs &a, hipStream_t stream);

void launch_accept_chunk(const AcceptArgs &a, hipStream_t stream);
// first chunk: next_begin = 0, rows min(chunk_size, q_i), packed in next_cu
void launch_chunk_start(const AcceptArgs &a, hipStream_t stream);

// ---------------------------------------------------------------------------
// Stochastic acceptance (speculative sampling)
// ---------------------------------------------------------------------------
struct StochJob {
  int tr;    // target row whose distribution the next token is drawn from (-1: none)
  int nrej;  // rejections whose residual the draw takes (0: the target row's p itself)
  int out;   // out_tokens entry of the drawn token
  int pad;
  float m, s;  // the target row's softmax stats (log2 domain)
  float w;     // the request's uniform for the draw
  float pad2;
};

// One rejection in force at the node the draw is made at: the rejected draft's
// row and the mass of the residual it left (the normaliser of that residual,
// unused for the last one, whose unnormalised residual is the draw's weights).
struct StochRej {
  int row;
  float mass;
};

struct StochLayout {
  size_t hdr;    // int32[8]: 0 status bits
  size_t stats;  // float2 [total_q][splits]: (max, sum) of each slice of each logits row
  size_t jobs;   // StochJob [batch]
  size_t mass;   // float [batch][nsub]: weight of each 2048-entry sub-slice of the draw
  size_t rej;    // StochRej [batch][kMaxTokens]: the rejections of each request's draw
  size_t total;
  int splits;
  int nsub;
};

__host__ __device__ inline StochLayout stoch_layout(int batch, int total_q, int vocab) {
  StochLayout l;
  l.splits = argmax_splits(total_q, vocab);
  size_t off = 0;
  l.hdr = off;    off = align256(off + 8 * sizeof(int32_t));
  l.stats = off;  off = align256(off + size_t(total_q) * l.splits * 8);
  l.jobs = off;   off = align256(off + size_t(batch) * sizeof(StochJob));
  l.nsub = (vocab + 2047) / 2048;
  l.mass = off;   off = align256(off + size_t(batch) * l.nsub * sizeof(float));
  l.rej = off;    off = align256(off + size_t(batch) * kMaxTokens * sizeof(StochRej));
  l.total = off;
  return l;
}

struct StochArgs {
  const float *logits;       // [total_q, vocab]
  const float *draft_probs;  // [total_q, vocab]
  const int32_t *draft;
  const int32_t *parent;     // [total_q] per-request tree parents, or null for chains
  const float *u;            // [total_q]
  const float *w;            // [batch]
  const int32_t *cu_q;
  int32_t *accept_len;
  int32_t *accepted_path;
  int32_t *out_tokens;
  char *ws;
  StochLayout lay;
  int batch, total_q, vocab;
  float c;                   // log2(e) / temperature
};

void launch_stochastic(const StochArgs &a, hipStream_t stream);

// ---------------------------------------------------------------------------
// KV compaction
// ---------------------------------------------------------------------------
struct CompactArgs {
  uint16_t *k_cache;
  uint16_t *v_cache;
  int64_t layer_stride;
  int num_layers;
  const int32_t *block_tables;
  int max_blocks;
  const int32_t *context_lens;
  const int32_t *cu_q;
  const int32_t *accepted_path;
  const int32_t *accept_len;
  int32_t *new_context_lens;
  int batch, total_q, num_kv_heads, head_dim, num_pages;
  bool v_transposed;  // V pages [D][16 tokens] (else token-major, like K)
};

void launch_kv_compact(const CompactArgs &a, hipStream_t stream);

// acceptance and compaction in one launch (a.lay from fused_layout)
void launch_accept_compact(const AcceptArgs &a, const CompactArgs &c, hipStream_t stream);

}  // namespace sv
