// Device helpers shared by the kernels (wave64 shuffles, bf16 packing,
// ancestor masks of draft trees).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace sv {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float floatx16 __attribute__((ext_vector_type(16)));

__device__ inline float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }
__device__ inline float fast_log2(float x) { return __builtin_amdgcn_logf(x); }

// bf16 bits of x (round to nearest even; gfx950 converts in hardware)
__device__ inline uint32_t bf16_bits(float x) {
  __bf16 b = (__bf16)x;
  return (uint32_t)__builtin_bit_cast(uint16_t, b);
}

typedef float float2v __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2v __attribute__((ext_vector_type(2)));
typedef unsigned u32x2v __attribute__((ext_vector_type(2)));
typedef float float4v __attribute__((ext_vector_type(4)));

// max(x[lane], x[lane ^ 32]) on every lane.  The permlane32 swap exchanges
// the upper half of its first operand with the lower half of its second, so
// with x in both each lane ends up holding x of itself and of its partner in
// the other half: a VALU op, where a shuffle would go through LDS.
__device__ inline float max_across_halves(float x) {
  const unsigned b = __float_as_uint(x);
  const auto r = __builtin_amdgcn_permlane32_swap(b, b, false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}

// Maximum and sum over the 64 lanes of a wave, returned wave-uniform.  DPP
// moves combine within each row of 16 lanes (quad swaps, then the row's
// half-mirror and mirror, after which every lane of a row holds the row's
// result), and the four rows are combined from their lanes 0, 16, 32, 48:
// no LDS round trip, and the same order on every call.
template <int Ctrl>
__device__ inline float dpp_mov(float v) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), Ctrl, 0xF, 0xF, false));
}

template <typename Op>
__device__ inline float wave_reduce(float x, Op op) {
  x = op(x, dpp_mov<0xB1>(x));   // quad_perm [1,0,3,2]
  x = op(x, dpp_mov<0x4E>(x));   // quad_perm [2,3,0,1]
  x = op(x, dpp_mov<0x141>(x));  // row_half_mirror
  x = op(x, dpp_mov<0x140>(x));  // row_mirror
  auto lane_of = [&](int l) { return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(x), l)); };
  return op(op(lane_of(0), lane_of(16)), op(lane_of(32), lane_of(48)));
}

__device__ inline float wave_max(float x) {
  return wave_reduce(x, [](float u, float v) { return fmaxf(u, v); });
}

__device__ inline float wave_sum(float x) {
  return wave_reduce(x, [](float u, float v) { return u + v; });
}

// {lo, hi} rounded to bf16 (nearest even) in one packed conversion
__device__ inline uint32_t pack_bf16x2(float lo, float hi) {
  const bf16x2v b = __builtin_convertvector((float2v){lo, hi}, bf16x2v);
  return __builtin_bit_cast(uint32_t, b);
}

// low halves of x0 and x1 as {x0.lo, x1.lo} (lo16 of the result from x0)
__device__ inline uint32_t pack_lo16(uint32_t x0, uint32_t x1) {
  return __builtin_amdgcn_perm(x1, x0, 0x05040100u);
}

// high halves of x0 and x1 as {x0.hi, x1.hi}
__device__ inline uint32_t pack_hi16(uint32_t x0, uint32_t x1) {
  return __builtin_amdgcn_perm(x1, x0, 0x07060302u);
}

// Ancestor-or-self bitmask of token `lane` of a request with q tokens whose
// rows start at o: bit k is set iff token k lies on the token's root path
// (SwiftSpec, "Tree-Aware KV Cache Management": a node's KV prefix is its root
// path).  Chains (tree_parent == nullptr) have parent j-1.  Must be called by
// the whole wave; lanes >= q return 0.  *ok is false if the parent array
// breaks root = -1, 0 <= parent[j] < j.  Pointer jumping: after round r a
// lane knows its ancestors closer than 2^r, so 6 rounds cover depth <= 63.
//
// The one memory read, the lane's parent entry, is a function of its own so
// that a caller can issue it early and pass the value to ancestor_mask_of.
__device__ inline int tree_parent_of(const int32_t *tree_parent, int o, int q, int lane) {
  return (tree_parent != nullptr && lane < q) ? tree_parent[o + lane] : -1;
}

__device__ inline uint64_t ancestor_mask_of(bool is_tree, int par, int q, int lane, bool *ok) {
  if (!is_tree) {
    *ok = true;
    if (lane >= q) return 0ull;
    return lane == 63 ? ~0ull : ((2ull << lane) - 1ull);
  }
  if (lane >= q) par = -1;
  bool good = lane >= q || (lane == 0 ? par == -1 : (par >= 0 && par < lane));
  if (!good) par = -1;
  *ok = __all(good);
  uint64_t anc = lane < q ? (1ull << lane) : 0ull;
  int jump = par;
#pragma unroll
  for (int r = 0; r < 6; ++r) {
    const int src = jump < 0 ? lane : jump;
    const uint64_t a2 = __shfl(anc, src);
    const int j2 = __shfl(jump, src);
    if (jump >= 0) {
      anc |= a2;
      jump = j2;
    }
  }
  return anc;
}

__device__ inline uint64_t ancestor_mask(const int32_t *tree_parent, int o, int q, int lane, bool *ok) {
  return ancestor_mask_of(tree_parent != nullptr, tree_parent_of(tree_parent, o, q, lane), q, lane, ok);
}

// Exclusive prefix sum over a 1024-thread block; *total receives the sum.
// `scratch` must hold at least 16 values of shared memory.
template <typename T>
__device__ inline T block_excl_scan_1024(T v, T *scratch, T *total) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  T x = v;
#pragma unroll
  for (int d = 1; d < 64; d <<= 1) {
    T y = __shfl_up(x, d);
    if (lane >= d) x += y;
  }
  if (lane == 63) scratch[wave] = x;
  __syncthreads();
  if (wave == 0) {
    T w = lane < 16 ? scratch[lane] : T(0);
#pragma unroll
    for (int d = 1; d < 16; d <<= 1) {
      T y = __shfl_up(w, d);
      if (lane >= d) w += y;
    }
    if (lane < 16) scratch[lane] = w;  // inclusive wave totals
  }
  __syncthreads();
  const T before = wave > 0 ? scratch[wave - 1] : T(0);
  *total = scratch[15];
  __syncthreads();
  return before + x - v;
}

__device__ inline long long block_sum_1024(long long v, long long *scratch) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
#pragma unroll
  for (int d = 32; d >= 1; d >>= 1) v += __shfl_xor(v, d);
  if (lane == 0) scratch[wave] = v;
  __syncthreads();
  long long s = 0;
  for (int w = 0; w < 16; ++w) s += scratch[w];
  __syncthreads();
  return s;
}

}  // namespace sv
