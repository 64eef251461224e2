// Lossless stochastic acceptance of drafted chains (speculative sampling) on
// gfx950.
//
// What is computed: DSpark's glossary ("Speculative Decoding") requires the
// verification rule to keep the target's distribution; the rule used is the
// standard speculative-sampling rejection rule.  For request i (verify tokens
// 0..gamma at rows o..o+gamma, token 0 = root):
//   p_j = softmax(logits[o+j-1] / temperature)   target distribution of position j
//   q_j = draft_probs[o+j]                        drafter's distribution of draft x_j
//   draft j is accepted iff u[o+j] * q_j(x_j) < p_j(x_j); the walk stops at the
//   first rejection; n = accepted drafts;
//   the next token y is drawn with w[i] by inverse CDF from max(0, p - q) at
//   position n+1 (a rejection), or from p_{gamma+1} (all accepted); a residual
//   without mass falls back to p_{n+1}.
// Draft trees (SwiftSpec, "Tree-aware KV cache management"; the pages give no
// rule for them): the siblings of the current node are tested in index order,
// each against the target distribution left over by the siblings rejected before
// it (max(0, p' - q) normalised, kept only when it has mass); an accepted child
// becomes the current node with its own row's p; when no child is accepted the
// draw takes the last residual with mass, or p.  A chain is the case of one
// child per node and gives the same results.
//
// Four launches, all but the walk streaming over the vocabulary:
//   softmax_stats_kernel  grid (splits, rows): per slice of a logits row the
//                         running (max, sum of 2^(x - max)) of x = logit*log2(e)/T;
//   stochastic_walk_kernel  one wave per request: merges the slices' stats,
//                         tests every draft, writes the accepted prefix and the
//                         sampling job (target row, rejections in force, w);
//   stochastic_tree_walk_kernel  (trees, in its place) one workgroup per request:
//                         walks the tree, summing each rejection's residual mass
//                         over the vocabulary with all its threads;
//   sample_mass_kernel    grid (sub-slices of 2048 entries, batch): mass of the
//                         draw's weights per sub-slice;
//   sample_pick_kernel    one workgroup per request: finds the sub-slice holding
//                         w * total, then the entry (thread sums of 8 entries,
//                         their prefix, then the thread's own 8).
#include "sv_device.h"
#include "sv_internal.h"

namespace sv {

namespace {

constexpr int kPickThreads = 256;

struct Stat {
  float m;  // max of x (log2 domain)
  float s;  // sum of 2^(x - m)
};

__device__ inline Stat merge(Stat a, Stat b) {
  const float M = fmaxf(a.m, b.m);
  if (M == -INFINITY) return Stat{-INFINITY, 0.f};
  return Stat{M, a.s * fast_exp2(a.m - M) + b.s * fast_exp2(b.m - M)};
}

__device__ inline Stat wave_merge(Stat x) {
#pragma unroll
  for (int d = 32; d >= 1; d >>= 1) {
    Stat y{__shfl_xor(x.m, d), __shfl_xor(x.s, d)};
    x = merge(x, y);
  }
  return x;
}

__device__ inline void slice_bounds(int V, int splits, int split, int *lo, int *hi) {
  int per = (V + splits - 1) / splits;
  per = (per + 3) & ~3;
  *lo = min(V, split * per);
  *hi = min(V, *lo + per);
}

__global__ __launch_bounds__(256) void softmax_stats_kernel(StochArgs a) {
  __shared__ float s_m[4], s_s[4];
  const int split = blockIdx.x, row = blockIdx.y;
  if (split == 0 && row == 0 && threadIdx.x == 0) reinterpret_cast<int32_t *>(a.ws + a.lay.hdr)[0] = 0;
  if (row >= a.total_q) return;
  int lo, hi;
  slice_bounds(a.vocab, a.lay.splits, split, &lo, &hi);
  const float *x = a.logits + (size_t)row * a.vocab;
  Stat st{-INFINITY, 0.f};
  auto add = [&](float l) {
    const float y = l * a.c;
    if (y > st.m) {
      st.s = st.s * fast_exp2(st.m - y) + 1.f;
      st.m = y;
    } else if (y > -INFINITY) {
      st.s += fast_exp2(y - st.m);
    }
  };
  if ((a.vocab & 3) == 0) {
    // 16-byte nontemporal loads, four in flight per thread (the row is read once)
    const int nv = (hi - lo) >> 2;
    const float4v *x4 = reinterpret_cast<const float4v *>(x + lo);
    int k = threadIdx.x;
    for (; k + 3 * 256 < nv; k += 4 * 256) {
      float4v v[4];
#pragma unroll
      for (int u = 0; u < 4; ++u) v[u] = __builtin_nontemporal_load(x4 + k + u * 256);
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        add(v[u].x);
        add(v[u].y);
        add(v[u].z);
        add(v[u].w);
      }
    }
    for (; k < nv; k += 256) {
      const float4v v = __builtin_nontemporal_load(x4 + k);
      add(v.x);
      add(v.y);
      add(v.z);
      add(v.w);
    }
  } else {
    for (int k = lo + threadIdx.x; k < hi; k += 256) add(__builtin_nontemporal_load(x + k));
  }
  st = wave_merge(st);
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  if (lane == 0) {
    s_m[wave] = st.m;
    s_s[wave] = st.s;
  }
  __syncthreads();
  if (threadIdx.x == 0) {
    Stat r{s_m[0], s_s[0]};
    for (int w = 1; w < 4; ++w) r = merge(r, Stat{s_m[w], s_s[w]});
    reinterpret_cast<float2 *>(a.ws + a.lay.stats)[(size_t)row * a.lay.splits + split] = make_float2(r.m, r.s);
  }
}

// one wave per request
__global__ __launch_bounds__(64) void stochastic_walk_kernel(StochArgs a) {
  const int i = blockIdx.x;
  const int j = threadIdx.x;
  unsigned *status = reinterpret_cast<unsigned *>(a.ws + a.lay.hdr);
  StochJob *jobs = reinterpret_cast<StochJob *>(a.ws + a.lay.jobs);
  const int o = a.cu_q[i], c1 = a.cu_q[i + 1], q = c1 - o;
  if (o < 0 || c1 < o || c1 > a.total_q || q > kMaxTokens) {
    if (j == 0) {
      atomicOr(status, SV_DEV_BAD_CU_Q);
      a.accept_len[i] = 0;
      jobs[i].tr = -1;
    }
    return;
  }
  if (i == 0 && j == 0 && (a.cu_q[0] != 0 || a.cu_q[a.batch] != a.total_q)) atomicOr(status, SV_DEV_BAD_CU_Q);
  if (q == 0) {
    if (j == 0) {
      a.accept_len[i] = 0;
      jobs[i].tr = -1;
    }
    return;
  }
  // stats of row o+j
  Stat st{-INFINITY, 0.f};
  if (j < q) {
    const float2 *ps = reinterpret_cast<const float2 *>(a.ws + a.lay.stats) + (size_t)(o + j) * a.lay.splits;
    for (int k = 0; k < a.lay.splits; ++k) {
      const float2 v = ps[k];
      st = merge(st, Stat{v.x, v.y});
    }
  }
  // draft j (j >= 1) against row j-1
  const Stat prev{__shfl(st.m, max(j - 1, 0)), __shfl(st.s, max(j - 1, 0))};
  bool reject = false;
  if (j >= 1 && j < q) {
    const int x = a.draft[o + j];
    if (x < 0 || x >= a.vocab) {
      atomicOr(status, SV_DEV_BAD_TOKEN);
      reject = true;
    } else {
      const float px = fast_exp2(a.logits[(size_t)(o + j - 1) * a.vocab + x] * a.c - prev.m) / prev.s;
      const float qx = a.draft_probs[(size_t)(o + j) * a.vocab + x];
      reject = !(a.u[o + j] * qx < px);
    }
  }
  const uint64_t rej = __ballot(reject);
  const int n = rej ? __builtin_ctzll(rej) - 1 : q - 1;
  const Stat sn{__shfl(st.m, n), __shfl(st.s, n)};
  if (j < q) {
    a.accepted_path[o + j] = j <= n ? j : -1;
    if (j < n) a.out_tokens[o + j] = a.draft[o + j + 1];
    if (j > n) a.out_tokens[o + j] = -1;
  }
  if (j == 0) {
    a.accept_len[i] = n + 1;
    StochJob jb;
    jb.tr = o + n;
    jb.nrej = n < q - 1 ? 1 : 0;
    if (jb.nrej) reinterpret_cast<StochRej *>(a.ws + a.lay.rej)[(size_t)i * kMaxTokens] = StochRej{o + n + 1, 0.f};
    jb.m = sn.m;
    jb.s = sn.s;
    jb.w = a.w[i];
    jb.out = o + n;
    jobs[i] = jb;
  }
}

// p'(v) at a node whose logits row is lrow (softmax stats m, s) after the
// first cnt rejections of rl: p(v), then each rejection's residual
// max(0, p' - q) divided by its mass
__device__ inline float resid_norm(const StochArgs &a, const float *lrow, float m, float s, const StochRej *rl,
                                   int cnt, int v) {
  float val = fast_exp2(lrow[v] * a.c - m) / s;
  for (int t = 0; t < cnt; ++t) val = fmaxf(0.f, val - a.draft_probs[(size_t)rl[t].row * a.vocab + v]) / rl[t].mass;
  return val;
}

// the draw's weight of entry v: p(v) without rejections, else the last
// rejection's residual, unnormalised
__device__ inline float draw_weight(const StochArgs &a, const StochJob &jb, const StochRej *rl, int nrej, int v) {
  const float *lrow = a.logits + (size_t)jb.tr * a.vocab;
  if (nrej == 0) return fast_exp2(lrow[v] * a.c - jb.m) / jb.s;
  const float pv = resid_norm(a, lrow, jb.m, jb.s, rl, nrej - 1, v);
  return fmaxf(0.f, pv - a.draft_probs[(size_t)rl[nrej - 1].row * a.vocab + v]);
}

__device__ inline const StochRej *rej_list(const StochArgs &a, int i) {
  return reinterpret_cast<const StochRej *>(a.ws + a.lay.rej) + (size_t)i * kMaxTokens;
}

// the draw's weights are summed per sub-slice of kSub entries: thread t of
// the workgroup sums entries base + 8t .. base + 8t + 7, in index order
constexpr int kSub = 2048;
constexpr int kPerThread = kSub / 256;

__device__ inline float thread_weights(const StochArgs &a, const StochJob &jb, const StochRej *rl, int nrej,
                                       int base, float (&wv)[kPerThread]) {
  const int v0 = base + kPerThread * (int)threadIdx.x;
  float val[kPerThread];
  if (v0 + kPerThread <= a.vocab && (a.vocab & 3) == 0) {
    // two 16-byte loads per row (v0 is a multiple of 8 and rows start 16-byte aligned)
    const float4v *lp = reinterpret_cast<const float4v *>(a.logits + (size_t)jb.tr * a.vocab + v0);
    float l[kPerThread];
#pragma unroll
    for (int h = 0; h < kPerThread / 4; ++h) {
      const float4v x = lp[h];
      l[4 * h] = x.x; l[4 * h + 1] = x.y; l[4 * h + 2] = x.z; l[4 * h + 3] = x.w;
    }
#pragma unroll
    for (int e = 0; e < kPerThread; ++e) val[e] = fast_exp2(l[e] * a.c - jb.m) / jb.s;
    for (int t = 0; t < nrej; ++t) {
      const float4v *dp = reinterpret_cast<const float4v *>(a.draft_probs + (size_t)rl[t].row * a.vocab + v0);
      float d[kPerThread];
#pragma unroll
      for (int h = 0; h < kPerThread / 4; ++h) {
        const float4v x = dp[h];
        d[4 * h] = x.x; d[4 * h + 1] = x.y; d[4 * h + 2] = x.z; d[4 * h + 3] = x.w;
      }
      if (t + 1 < nrej) {
        const float M = rl[t].mass;
#pragma unroll
        for (int e = 0; e < kPerThread; ++e) val[e] = fmaxf(0.f, val[e] - d[e]) / M;
      } else {
#pragma unroll
        for (int e = 0; e < kPerThread; ++e) val[e] = fmaxf(0.f, val[e] - d[e]);
      }
    }
  } else {
#pragma unroll
    for (int e = 0; e < kPerThread; ++e) val[e] = draw_weight(a, jb, rl, nrej, min(v0 + e, a.vocab - 1));
  }
  float own = 0.f;
#pragma unroll
  for (int e = 0; e < kPerThread; ++e) {
    wv[e] = v0 + e < a.vocab ? val[e] : 0.f;
    own += wv[e];
  }
  return own;
}

__device__ inline float block_sum_256(float x, float *scratch) {
#pragma unroll
  for (int d = 32; d >= 1; d >>= 1) x += __shfl_xor(x, d);
  if ((threadIdx.x & 63) == 0) scratch[threadIdx.x >> 6] = x;
  __syncthreads();
  const float r = (scratch[0] + scratch[1]) + (scratch[2] + scratch[3]);
  __syncthreads();
  return r;
}

// one workgroup per request of a tree: the children of a node all have larger
// indices than the node, so one scan over the verify tokens in index order
// meets every test of the walk in the rule's order.  A rejection's residual mass
// is a pass over the vocabulary whose entries each walk the rejection list with
// dependent loads, so the pass runs 16 waves, each thread taking kTreeIlp groups
// of entries at a time (four consecutive entries per group with 16-byte loads).
constexpr int kTreeThreads = 1024;
constexpr int kTreeIlp = 4;

__device__ inline float block_sum_tree(float x, float *scratch) {
#pragma unroll
  for (int d = 32; d >= 1; d >>= 1) x += __shfl_xor(x, d);
  if ((threadIdx.x & 63) == 0) scratch[threadIdx.x >> 6] = x;
  __syncthreads();
  float r = 0.f;
#pragma unroll
  for (int w = 0; w < kTreeThreads / 64; ++w) r += scratch[w];
  __syncthreads();
  return r;
}

__global__ __launch_bounds__(kTreeThreads) void stochastic_tree_walk_kernel(StochArgs a) {
  __shared__ float s_m[kMaxTokens], s_s[kMaxTokens];
  __shared__ int s_par[kMaxTokens], s_path[kMaxTokens];
  __shared__ StochRej s_rej[kMaxTokens];
  __shared__ float s_red[kTreeThreads / 64];
  __shared__ int s_dec;
  __shared__ int s_x[kMaxTokens];         // the request's draft tokens
  __shared__ float s_u[kMaxTokens];       // and acceptance uniforms
  __shared__ float s_val[kMaxTokens + 2];  // a test's operands, loaded side by side
  const int i = blockIdx.x, tid = threadIdx.x;
  unsigned *status = reinterpret_cast<unsigned *>(a.ws + a.lay.hdr);
  StochJob *jobs = reinterpret_cast<StochJob *>(a.ws + a.lay.jobs);
  const int o = a.cu_q[i], c1 = a.cu_q[i + 1], q = c1 - o;
  if (o < 0 || c1 < o || c1 > a.total_q || q > kMaxTokens) {
    if (tid == 0) {
      atomicOr(status, SV_DEV_BAD_CU_Q);
      a.accept_len[i] = 0;
      jobs[i].tr = -1;
    }
    return;
  }
  if (i == 0 && tid == 0 && (a.cu_q[0] != 0 || a.cu_q[a.batch] != a.total_q)) atomicOr(status, SV_DEV_BAD_CU_Q);
  if (q == 0) {
    if (tid == 0) {
      a.accept_len[i] = 0;
      jobs[i].tr = -1;
    }
    return;
  }
  int bad = 0;
  if (tid < q) {
    const int pk = a.parent[o + tid];
    bad = tid == 0 ? pk != -1 : (pk < 0 || pk >= tid);
    s_par[tid] = pk;
    Stat st{-INFINITY, 0.f};
    const float2 *ps = reinterpret_cast<const float2 *>(a.ws + a.lay.stats) + (size_t)(o + tid) * a.lay.splits;
    for (int k = 0; k < a.lay.splits; ++k) {
      const float2 v = ps[k];
      st = merge(st, Stat{v.x, v.y});
    }
    s_m[tid] = st.m;
    s_s[tid] = st.s;
    s_x[tid] = a.draft[o + tid];
    s_u[tid] = a.u[o + tid];
  }
  if (tid == 0) s_path[0] = 0;
  if (__syncthreads_or(bad)) {
    if (tid == 0) {
      atomicOr(status, SV_DEV_BAD_PARENT);
      a.accept_len[i] = 0;
      jobs[i].tr = -1;
    }
    if (tid < q) {
      a.accepted_path[o + tid] = -1;
      a.out_tokens[o + tid] = -1;
    }
    return;
  }
  int c = 0, n = 0, cnt = 0;  // current node, accepted drafts, rejections in force at c
  const float *lrow = a.logits + (size_t)o * a.vocab;
  for (int k = 1; k < q; ++k) {
    if (s_par[k] != c) continue;
    // the test's operands in one round trip: the logit of x at c, q_k(x), and
    // q(x) of every rejection in force; then thread 0 evaluates p'(x) from them
    // in resid_norm's order
    const int x = s_x[k];
    const bool x_ok = x >= 0 && x < a.vocab;
    if (x_ok && tid < cnt + 2) {
      const size_t row = tid == 0 ? (size_t)(o + c) : tid == 1 ? (size_t)(o + k) : (size_t)s_rej[tid - 2].row;
      s_val[tid] = (tid == 0 ? a.logits : a.draft_probs)[row * a.vocab + x];
    }
    __syncthreads();
    if (tid == 0) {
      int acc = 0;
      if (!x_ok) {
        atomicOr(status, SV_DEV_BAD_TOKEN);
      } else {
        float px = fast_exp2(s_val[0] * a.c - s_m[c]) / s_s[c];
        for (int t = 0; t < cnt; ++t) px = fmaxf(0.f, px - s_val[2 + t]) / s_rej[t].mass;
        acc = s_u[k] * s_val[1] < px;
      }
      s_dec = acc;
    }
    __syncthreads();
    const int acc = s_dec;
    __syncthreads();
    if (acc) {
      c = k;
      ++n;
      if (tid == 0) s_path[n] = k;
      cnt = 0;
      lrow = a.logits + (size_t)(o + k) * a.vocab;
      continue;
    }
    // rejected: the mass of max(0, p' - q_k), kept as the next residual if positive
    const float *qrow = a.draft_probs + (size_t)(o + k) * a.vocab;
    const float mc = s_m[c], sc = s_s[c];
    float part = 0.f;
    if ((a.vocab & 3) == 0) {
      // 16-byte loads (rows start 16-byte aligned): each thread takes four
      // consecutive entries from each of kTreeIlp groups per iteration
      const int nv4 = a.vocab >> 2;
      const float4v *l4 = reinterpret_cast<const float4v *>(lrow);
      const float4v *q4 = reinterpret_cast<const float4v *>(qrow);
      for (int b0 = tid; b0 < nv4; b0 += kTreeIlp * kTreeThreads) {
        float val[kTreeIlp][4];
#pragma unroll
        for (int g = 0; g < kTreeIlp; ++g) {
          const float4v x = l4[min(b0 + g * kTreeThreads, nv4 - 1)];
          val[g][0] = fast_exp2(x.x * a.c - mc) / sc;
          val[g][1] = fast_exp2(x.y * a.c - mc) / sc;
          val[g][2] = fast_exp2(x.z * a.c - mc) / sc;
          val[g][3] = fast_exp2(x.w * a.c - mc) / sc;
        }
        for (int t = 0; t < cnt; ++t) {
          const float4v *qt = reinterpret_cast<const float4v *>(a.draft_probs + (size_t)s_rej[t].row * a.vocab);
          const float M = s_rej[t].mass;
#pragma unroll
          for (int g = 0; g < kTreeIlp; ++g) {
            const float4v d = qt[min(b0 + g * kTreeThreads, nv4 - 1)];
            val[g][0] = fmaxf(0.f, val[g][0] - d.x) / M;
            val[g][1] = fmaxf(0.f, val[g][1] - d.y) / M;
            val[g][2] = fmaxf(0.f, val[g][2] - d.z) / M;
            val[g][3] = fmaxf(0.f, val[g][3] - d.w) / M;
          }
        }
#pragma unroll
        for (int g = 0; g < kTreeIlp; ++g) {
          if (b0 + g * kTreeThreads < nv4) {
            const float4v d = q4[b0 + g * kTreeThreads];
            part += fmaxf(0.f, val[g][0] - d.x);
            part += fmaxf(0.f, val[g][1] - d.y);
            part += fmaxf(0.f, val[g][2] - d.z);
            part += fmaxf(0.f, val[g][3] - d.w);
          }
        }
      }
    } else {
      for (int v0 = tid; v0 < a.vocab; v0 += kTreeIlp * kTreeThreads) {
        float val[kTreeIlp];
#pragma unroll
        for (int e = 0; e < kTreeIlp; ++e) {
          const int v = min(v0 + e * kTreeThreads, a.vocab - 1);
          val[e] = fast_exp2(lrow[v] * a.c - mc) / sc;
        }
        for (int t = 0; t < cnt; ++t) {
          const float *qt = a.draft_probs + (size_t)s_rej[t].row * a.vocab;
          const float M = s_rej[t].mass;
#pragma unroll
          for (int e = 0; e < kTreeIlp; ++e) {
            const int v = min(v0 + e * kTreeThreads, a.vocab - 1);
            val[e] = fmaxf(0.f, val[e] - qt[v]) / M;
          }
        }
#pragma unroll
        for (int e = 0; e < kTreeIlp; ++e) {
          const int v = v0 + e * kTreeThreads;
          if (v < a.vocab) part += fmaxf(0.f, val[e] - qrow[v]);
        }
      }
    }
    const float M = block_sum_tree(part, s_red);
    if (M > 0.f) {
      if (tid == 0) s_rej[cnt] = StochRej{o + k, M};
      ++cnt;
      __syncthreads();
    }
  }
  __syncthreads();
  StochRej *rej = reinterpret_cast<StochRej *>(a.ws + a.lay.rej) + (size_t)i * kMaxTokens;
  if (tid < cnt) rej[tid] = s_rej[tid];
  if (tid < q) {
    a.accepted_path[o + tid] = tid <= n ? s_path[tid] : -1;
    if (tid < n) a.out_tokens[o + tid] = a.draft[o + s_path[tid + 1]];
    if (tid > n) a.out_tokens[o + tid] = -1;
  }
  if (tid == 0) {
    a.accept_len[i] = n + 1;
    StochJob jb;
    jb.tr = o + c;
    jb.nrej = cnt;
    jb.m = s_m[c];
    jb.s = s_s[c];
    jb.w = a.w[i];
    jb.out = o + n;
    jobs[i] = jb;
  }
}

__global__ __launch_bounds__(256) void sample_mass_kernel(StochArgs a) {
  __shared__ float s_r[4];
  const int sb = blockIdx.x, i = blockIdx.y;
  const StochJob jb = reinterpret_cast<const StochJob *>(a.ws + a.lay.jobs)[i];
  if (jb.tr < 0) return;
  float wv[kPerThread];
  const float own = thread_weights(a, jb, rej_list(a, i), jb.nrej, sb * kSub, wv);
  const float tot = block_sum_256(own, s_r);
  if (threadIdx.x == 0) reinterpret_cast<float *>(a.ws + a.lay.mass)[(size_t)i * a.lay.nsub + sb] = tot;
}

__global__ __launch_bounds__(kPickThreads) void sample_pick_kernel(StochArgs a) {
  __shared__ float s_seg[kPickThreads];
  __shared__ float s_r[4];
  __shared__ int s_k, s_pick, s_residual;
  __shared__ float s_target;
  const int i = blockIdx.x;
  const int tid = threadIdx.x;
  const StochJob jb = reinterpret_cast<const StochJob *>(a.ws + a.lay.jobs)[i];
  if (jb.tr < 0) return;
  const int nsub = a.lay.nsub;
  float *mass = reinterpret_cast<float *>(a.ws + a.lay.mass) + (size_t)i * nsub;
  if (tid == 0) {
    float tot = 0.f;
    for (int k = 0; k < nsub; ++k) tot += mass[k];
    s_residual = jb.nrej > 0 && tot > 0.f;
  }
  __syncthreads();
  const StochRej *rl = rej_list(a, i);
  const int nrej = s_residual ? jb.nrej : 0;
  if (jb.nrej > 0 && nrej == 0) {
    // a residual without mass: draw from p instead (rare; a tree's recorded
    // residuals all have mass); this workgroup recomputes the sub-slice masses of p
    for (int k = 0; k < nsub; ++k) {
      float wv[kPerThread];
      const float tot = block_sum_256(thread_weights(a, jb, rl, 0, k * kSub, wv), s_r);
      if (tid == 0) mass[k] = tot;
    }
    __syncthreads();
  }
  // the sub-slice holding w * total: first k whose running mass exceeds it
  if (tid == 0) {
    float tot = 0.f;
    for (int k = 0; k < nsub; ++k) tot += mass[k];
    const float target = jb.w * tot;
    float run = 0.f;
    int kk = -1, last = 0;
    for (int k = 0; k < nsub; ++k) {
      if (mass[k] > 0.f) last = k;
      if (kk < 0 && run + mass[k] > target) kk = k;
      if (kk < 0) run += mass[k];
    }
    if (kk < 0) {  // rounding: the last sub-slice with mass
      kk = last;
      run = 0.f;
      for (int k = 0; k < kk; ++k) run += mass[k];
    }
    s_k = kk;
    s_target = target - run;
    s_pick = -1;
  }
  __syncthreads();
  const int base = s_k * kSub;
  float wv[kPerThread];
  s_seg[tid] = thread_weights(a, jb, rl, nrej, base, wv);
  __syncthreads();
  if (tid == 0) {  // exclusive prefix of the thread sums, in index order
    float run = 0.f;
    for (int u = 0; u < kPickThreads; ++u) {
      const float x = s_seg[u];
      s_seg[u] = run;
      run += x;
    }
  }
  __syncthreads();
  const float t = s_target;
  const float before = s_seg[tid];
  const float after = tid + 1 < kPickThreads ? s_seg[tid + 1] : INFINITY;
  if (before <= t && t < after) {
    float run = before;
    int pick = -1, lastpos = -1;
#pragma unroll
    for (int e = 0; e < kPerThread; ++e) {
      if (pick < 0 && wv[e] > 0.f) {
        lastpos = base + kPerThread * tid + e;
        run += wv[e];
        if (run > t) pick = lastpos;
      }
    }
    if (pick < 0) pick = lastpos;
    if (pick >= 0) atomicMax(&s_pick, pick);
  }
  __syncthreads();
  if (tid == 0) {
    int y = s_pick;
    if (y < 0) {  // rounding left the target past the sub-slice: its last entry with weight
      for (int v = min(a.vocab, base + kSub) - 1; v >= base; --v)
        if (draw_weight(a, jb, rl, nrej, v) > 0.f) {
          y = v;
          break;
        }
    }
    a.out_tokens[jb.out] = y < 0 ? base : y;
  }
}

}  // namespace

void launch_stochastic(const StochArgs &a, hipStream_t stream) {
  const int rows = a.total_q > 0 ? a.total_q : 1;
  softmax_stats_kernel<<<dim3(a.lay.splits, rows), 256, 0, stream>>>(a);
  if (a.parent)
    stochastic_tree_walk_kernel<<<a.batch, kTreeThreads, 0, stream>>>(a);
  else
    stochastic_walk_kernel<<<a.batch, 64, 0, stream>>>(a);
  sample_mass_kernel<<<dim3(a.lay.nsub, a.batch), 256, 0, stream>>>(a);
  sample_pick_kernel<<<a.batch, kPickThreads, 0, stream>>>(a);
}

}  // namespace sv
