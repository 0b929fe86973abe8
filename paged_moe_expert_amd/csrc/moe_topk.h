// Top-k selection and block scan used by the routing kernels and by the
// gate/up stream that routes tiny batches itself. Not on the pages: the
// selection follows the plain reading stated in the oracle (top-k on raw
// logits, ties to the lower expert index, -0 = +0; softmax over the kept
// logits).
#pragma once

#include "moe_common.h"

namespace rimuru {

// Total order on (logit, expert): larger logit first, then lower index;
// -0 and +0 compare equal. Logits are finite (precondition).
__device__ __forceinline__ uint64_t rank_key(float v, uint32_t e) {
  if (v == 0.0f) v = 0.0f;
  uint32_t u = __float_as_uint(v);
  uint32_t s = (u & 0x80000000u) ? ~u : (u | 0x80000000u);
  return (static_cast<uint64_t>(s) << 32) | (0xffffffffu - e);
}

__device__ __forceinline__ float key_logit(uint64_t key) {
  uint32_t s = static_cast<uint32_t>(key >> 32);
  uint32_t u = (s & 0x80000000u) ? (s & 0x7fffffffu) : ~s;
  return __uint_as_float(u);
}

// One max step with a DPP-permuted copy of v (lanes whose row is masked off
// keep their own value, which the max leaves unchanged).
template <int CTRL, int ROW_MASK>
__device__ __forceinline__ uint64_t dpp_max_step(uint64_t v) {
  const int lo = static_cast<int>(static_cast<uint32_t>(v)), hi = static_cast<int>(static_cast<uint32_t>(v >> 32));
  const uint32_t plo = static_cast<uint32_t>(__builtin_amdgcn_update_dpp(lo, lo, CTRL, ROW_MASK, 0xF, false));
  const uint32_t phi = static_cast<uint32_t>(__builtin_amdgcn_update_dpp(hi, hi, CTRL, ROW_MASK, 0xF, false));
  const uint64_t o = (static_cast<uint64_t>(phi) << 32) | plo;
  return o > v ? o : v;
}

// Max over the wavefront's 64 lanes, returned to every lane. DPP moves stay
// in the VALU (no LDS round trips): pairs, quads, 8 and 16 lanes by quad
// permutes and row mirrors, then row 0 -> 1 and 2 -> 3 by the lane-15
// broadcast and rows 0-1 -> 2-3 by the lane-31 broadcast; lane 63 then holds
// the maximum.
__device__ __forceinline__ uint64_t wave_max_u64(uint64_t v) {
  v = dpp_max_step<0xB1, 0xF>(v);       // quad_perm [1,0,3,2]
  v = dpp_max_step<0x4E, 0xF>(v);       // quad_perm [2,3,0,1]
  v = dpp_max_step<0x141, 0xF>(v);      // row_half_mirror
  v = dpp_max_step<0x140, 0xF>(v);      // row_mirror
  v = dpp_max_step<0x142, 0xA>(v);      // row_bcast:15 into rows 1 and 3
  v = dpp_max_step<0x143, 0xC>(v);      // row_bcast:31 into rows 2 and 3
  const uint32_t lo = __builtin_amdgcn_readlane(static_cast<int>(static_cast<uint32_t>(v)), 63);
  const uint32_t hi = __builtin_amdgcn_readlane(static_cast<int>(static_cast<uint32_t>(v >> 32)), 63);
  return (static_cast<uint64_t>(hi) << 32) | lo;
}


// Top-k of one token's logits by one wavefront. Lane r < k ends with the
// r-th expert (rank order) in *e_out and its logit in *l_out; every lane gets
// the weight denominator's terms in rank order via the returned softmax value.
template <int EPL>
__device__ __forceinline__ void load_logits(const float* row, int E, int lane, float (&v)[EPL]) {
#pragma unroll
  for (int i = 0; i < EPL; ++i) {
    const int e = lane + 64 * i;
    v[i] = (e < E) ? row[e] : 0.0f;
  }
}

template <int EPL>
__device__ __forceinline__ void select_topk_vals(const float (&v)[EPL], int E, int k, int lane,
                                                 uint32_t* e_out, float* w_out) {
  uint64_t key[EPL];
#pragma unroll
  for (int i = 0; i < EPL; ++i) {
    int e = lane + 64 * i;
    key[i] = (e < E) ? rank_key(v[i], static_cast<uint32_t>(e)) : 0ull;
  }
  uint32_t my_e = 0;
  float my_l = 0.0f;
  for (int r = 0; r < k; ++r) {
    uint64_t best = key[0];
#pragma unroll
    for (int i = 1; i < EPL; ++i) best = key[i] > best ? key[i] : best;
    best = wave_max_u64(best);
    uint32_t e = 0xffffffffu - static_cast<uint32_t>(best);
#pragma unroll
    for (int i = 0; i < EPL; ++i)
      if (static_cast<uint32_t>(lane + 64 * i) == e) key[i] = 0ull;
    if (lane == r) {
      my_e = e;
      my_l = key_logit(best);
    }
  }
  // softmax over the kept logits = renormalised full softmax; the sum runs
  // over the kept experts in rank order
  const float m = __shfl(my_l, 0, 64);
  const float ex = (lane < k) ? expf(my_l - m) : 0.0f;
  float s = 0.0f;
  for (int j = 0; j < k; ++j) s += __shfl(ex, j, 64);
  *e_out = my_e;
  *w_out = ex / s;
}

// Exclusive prefix of v over the NT threads of the block; *total gets the sum.
template <int NT = 256>
__device__ __forceinline__ int block_excl_scan(int v, int* total, int* sh) {
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  int incl = v;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    int o = __shfl_up(incl, off, 64);
    if (lane >= off) incl += o;
  }
  if (lane == 63) sh[wv] = incl;
  __syncthreads();
  int before = 0, all = 0;
#pragma unroll
  for (int i = 0; i < NT / 64; ++i) {
    before += (i < wv) ? sh[i] : 0;
    all += sh[i];
  }
  __syncthreads();
  *total = all;
  return before + incl - v;
}

// Tiny batches whose gate/up stream does the routing itself (one wavefront
// a token, one thread an expert): limits of that path.
constexpr int kRoutedMaxT = 4;                  // tokens
constexpr int kRoutedMaxTK = 32;                // routed slots
constexpr int kRoutedMaxE = 256;                // experts
constexpr int kRoutedMaxSorted = 16 * kRoutedMaxTK;  // padded rows: every slot its own 16-row tile at most

// Where the routed stream reads the logits and writes the routing results
// (the same buffers the routing kernels fill).
struct TinyRoute {
  const float* logits;
  int T, k;
  int32_t* topk_ids;
  float* topk_w;
  int32_t* sorted_ids;
  int32_t* expert_off;
  int32_t* tile_expert;
};

// Whether a layer of this shape takes the routed stream for gate/up.
bool streamed_routed_fits(int dtype_bytes, int T, int k, int E, int K, uint64_t tiles_max);

// Gate/up of a tiny batch with its routing (bf16, 16-row tiles; returns
// hipErrorNotSupported for shapes the path does not cover).
template <typename T>
hipError_t launch_streamed_routed(const GemmArgs& g, uint64_t tiles_max, const TinyRoute& rt, hipStream_t st);

}  // namespace rimuru
