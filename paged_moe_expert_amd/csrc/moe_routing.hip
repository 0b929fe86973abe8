// Routing stages of the fused MoE layer and the combine, plus the page-wise
// weight store. Not on the pages: gating, sort and combine follow the plain
// readings stated in the oracle (softmax over the kept top-k logits, stable
// expert grouping padded to the tile height, rank-ordered fp32 sum).
//
//   gating   one wavefront per token: top-k on raw logits, then softmax over
//            the kept logits (the renormalised softmax weights)
//   count    one workgroup per expert: routed slots per expert
//   sort     one workgroup per expert: stable list of slots t*k+j, padded to
//            the tile height, tile -> expert map
//   combine  y[t] = sum_j y_slot[t*k+j], j in rank order
#include <type_traits>

#include "moe_common.h"
#include "moe_topk.h"

namespace rimuru {

// ---------------------------------------------------------------- stage 1: gating

__device__ __forceinline__ float wave_sum_f32(float v) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) v += __shfl_xor(v, off, 64);
  return v;
}

template <int EPL>
__device__ __forceinline__ void select_topk(const float* row, int E, int k, int lane,
                                            uint32_t* e_out, float* w_out) {
  float v[EPL];
  load_logits<EPL>(row, E, lane, v);
  select_topk_vals<EPL>(v, E, k, lane, e_out, w_out);
}

template <int EPL>
__global__ __launch_bounds__(256) void k_gating(const float* __restrict__ logits, int T, int E,
                                                int k, int32_t* __restrict__ ids,
                                                float* __restrict__ w) {
  const int lane = threadIdx.x & 63;
  const int t = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (t >= T) return;
  uint32_t e;
  float wt;
  select_topk<EPL>(logits + static_cast<int64_t>(t) * E, E, k, lane, &e, &wt);
  if (lane < k) {
    ids[static_cast<int64_t>(t) * k + lane] = static_cast<int32_t>(e);
    w[static_cast<int64_t>(t) * k + lane] = wt;
  }
}

// Router projection as its own small GEMM: logits[t, e] = x[t] . w_gate[e]
// (w_gate [E, H] row-major, a Linear layer's weight layout), fp32
// accumulation with 16x16 MFMA tiles; both operands are K-contiguous rows,
// loaded straight into registers. A workgroup computes 16 tokens x 16*NT
// experts with its K range split over 8 wavefronts, summed in fixed
// wavefront order in LDS. Each wavefront loads LA K steps of both operands
// before multiplying, so a block costs about one memory round trip per LA
// steps. Few tokens (decode) take NT = 1 so that w_gate's reads spread over
// as many CUs as possible (one workgroup per token block streaming all of
// w_gate was measured about twice as slow); many tokens take wider expert
// tiles so that x is re-read fewer times.
constexpr int kRouterGW = 8;   // wavefronts per workgroup (K split)
#ifndef RIMURU_ROUTER_WIDE_MINWG
#define RIMURU_ROUTER_WIDE_MINWG 256
#endif
constexpr int kRouterWideMinWG = RIMURU_ROUTER_WIDE_MINWG;
#ifndef RIMURU_ROUTER_MINWG
#define RIMURU_ROUTER_MINWG 1024
#endif

template <typename T, int NT, int LA>
__global__ __launch_bounds__(kRouterGW * 64) void k_router_logits(const T* __restrict__ x,
                                                                  const T* __restrict__ w_gate, int T_, int E,
                                                                  int H, int nsplit, float* __restrict__ logits) {
  typedef Elt<T> X;
  constexpr int VEC = X::VEC, SEG8 = X::SEG8;
  __shared__ float part[kRouterGW][16][16 * NT];
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  const int t0 = blockIdx.x * 16, e0 = blockIdx.y * 16 * NT;
  const int fi = lane & 15, fq = lane >> 4;
  if (wv < nsplit) {
    const int kw = H / nsplit;   // multiple of 32 (chosen by the launcher)
    const int ks = wv;           // K slice of this wavefront
    const T* xa = x + static_cast<int64_t>(min(t0 + fi, T_ - 1)) * H + ks * kw + fq * 8;
    const T* wr[NT];
#pragma unroll
    for (int n = 0; n < NT; ++n)
      wr[n] = w_gate + static_cast<int64_t>(min(e0 + n * 16 + fi, E - 1)) * H + ks * kw + fq * 8;
    f32x4 acc[NT];
#pragma unroll
    for (int n = 0; n < NT; ++n) acc[n] = f32x4{0.f, 0.f, 0.f, 0.f};
    for (int kb = 0; kb < kw; kb += 32 * LA) {
      // Steps past kw re-read the last step with x zeroed: their products are
      // exact zeros, which leave the fp32 sums unchanged. No branch here, so
      // every load of the batch is issued before the first MFMA waits.
      u32x4 a[LA][SEG8], b[LA][NT][SEG8];
#pragma unroll
      for (int j = 0; j < LA; ++j) {
        const int k0 = min(kb + 32 * j, kw - 32);
#pragma unroll
        for (int u = 0; u < SEG8; ++u) a[j][u] = *reinterpret_cast<const u32x4*>(xa + k0 + u * VEC);
#pragma unroll
        for (int n = 0; n < NT; ++n)
#pragma unroll
          for (int u = 0; u < SEG8; ++u) b[j][n][u] = *reinterpret_cast<const u32x4*>(wr[n] + k0 + u * VEC);
      }
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int j = 0; j < LA; ++j) {
        const uint32_t keep = (kb + 32 * j < kw) ? 0xFFFFFFFFu : 0u;
#pragma unroll
        for (int u = 0; u < SEG8; ++u)
#pragma unroll
          for (int c = 0; c < 4; ++c) a[j][u][c] &= keep;
#pragma unroll
        for (int n = 0; n < NT; ++n) acc[n] = X::mma8(a[j], b[j][n], acc[n]);
      }
    }
    // acc[n][r] holds token 4*(lane/16) + r, expert 16n + lane%16
#pragma unroll
    for (int n = 0; n < NT; ++n)
#pragma unroll
      for (int r = 0; r < 4; ++r) part[ks][4 * fq + r][n * 16 + fi] = acc[n][r];
  }
  __syncthreads();
  for (int i = threadIdx.x; i < 16 * 16 * NT; i += kRouterGW * 64) {
    const int tl = i / (16 * NT), el = i % (16 * NT);
    float v = part[0][tl][el];
    for (int sw = 1; sw < nsplit; ++sw) v += part[sw][tl][el];
    const int t = t0 + tl, e = e0 + el;
    if (t < T_ && e < E) logits[static_cast<int64_t>(t) * E + e] = v;
  }
}

template <typename T, int NT, int LA>
void launch_router_nt(const RouterArgs& r, int n_tok, int E, int nsplit, hipStream_t st) {
  const dim3 grid((n_tok + 15) / 16, (E + 16 * NT - 1) / (16 * NT));
  hipLaunchKernelGGL((k_router_logits<T, NT, LA>), grid, dim3(kRouterGW * 64), 0, st,
                     static_cast<const T*>(r.x), static_cast<const T*>(r.w_gate), n_tok, E, r.H, nsplit,
                     r.logits_out);
}

// Many tokens (bf16): a workgroup computes 32 tokens x 32*NE experts over
// the whole hidden dimension, so x is read from HBM once per expert tile and
// w_gate (a few hundred KB) from L2. Both operands are K-contiguous rows,
// copied to LDS asynchronously in stages of 64 K (one 128-byte piece of each
// of the 32 + 32*NE rows), kRouterStages stages in a ring. Within a row
// piece the eight 16-byte octets are stored XOR-swizzled by the row (octet o
// of row r at slot o ^ r%8), so a MFMA operand read (32 rows, one octet
// each) spreads over all LDS banks. A 32x32x16 MFMA sums over the 16 K
// values of octets 2s and 2s+1 in both operands alike. Wavefront w
// multiplies expert block w % NE; with NE < 4 the K steps of a stage are
// split over the 4/NE wavefronts of a block, whose partial sums are added in
// LDS in fixed order.
//
// Measured on the 8192-token, 128-expert router (H = 2048): 16.6-18 us
// against 45 us for the register-operand kernel. Four to eight stages, a
// split of the copies between x-copying and w_gate-copying wavefronts (so
// that the HBM reads of x could run further ahead than the L2 reads of
// w_gate), 64-token workgroups (half the w_gate reads, half the
// workgroups) and staggered K start points were all measured no faster or
// slower: the copies into each CU, 640 KB a workgroup, set the pace.
constexpr int kRouterStages = 6;

// wait until at most n (<= N) groups of C copies are in flight
template <int C, int N>
__device__ __forceinline__ void wait_stages(int n) {
  if constexpr (N == 0) {
    wait_vmem<0>();
  } else {
    if (n >= N) wait_vmem<N * C>();
    else wait_stages<C, N - 1>(n);
  }
}

template <int NE>
__global__ __launch_bounds__(256) void k_router_wide(const uint16_t* __restrict__ x,
                                                     const uint16_t* __restrict__ w_gate, int T_, int E, int H,
                                                     float* __restrict__ logits) {
  constexpr int KS = 4 / NE;                 // wavefronts per expert block (K split)
  constexpr int ROWS = 32 + 32 * NE;         // rows of a stage: 32 of x, then the experts
  constexpr int CPW = ROWS / 8 / 4;          // 1 KB copies per wavefront per stage
  constexpr int STAGE = ROWS * 128;
  constexpr int NS = kRouterStages;
  static_assert(NE == 1 || NE == 2 || NE == 4, "expert blocks");
  static_assert(NS >= 3 && NS * STAGE <= 160 * 1024, "stage ring");
  __shared__ __attribute__((aligned(1024))) uint8_t smem[NS * STAGE];
  typedef __attribute__((address_space(3))) uint8_t lds_u8;
  const uint32_t smem_lds = __builtin_amdgcn_readfirstlane(
      static_cast<uint32_t>(reinterpret_cast<uintptr_t>((lds_u8*)smem)));
  const int lane = threadIdx.x & 63;
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int t0 = blockIdx.x * 32, e0 = blockIdx.y * 32 * NE;
  const int nk = H / 64;

  // copy c of a stage fills rows 8c .. 8c+7 (x rows first, then w_gate
  // rows); lane l fetches octet (l%8) ^ (l/8) of row 8c + l/8, which lands
  // at slot l%8 of that row. Rows past T or E re-read the last one.
  const uint8_t* src[CPW];
#pragma unroll
  for (int d = 0; d < CPW; ++d) {
    const int c = w * CPW + d;
    const int r = 8 * c + (lane >> 3);
    const int oct = (lane & 7) ^ (lane >> 3);
    const uint16_t* row = r < 32 ? x + static_cast<int64_t>(min(t0 + r, T_ - 1)) * H
                                 : w_gate + static_cast<int64_t>(min(e0 + r - 32, E - 1)) * H;
    src[d] = reinterpret_cast<const uint8_t*>(row) + 16 * oct;
  }
  auto issue = [&](int s) {
    const uint32_t dst = smem_lds + (s % NS) * STAGE;
#pragma unroll
    for (int d = 0; d < CPW; ++d) copy_to_lds16(src[d] + s * 128, dst + (w * CPW + d) * 1024);
  };

  const int blk = w % NE, q = w / NE;        // expert block, K split index
  const int r = lane & 31;
  uint32_t aoff[4 / KS], boff[4 / KS];
#pragma unroll
  for (int i = 0; i < 4 / KS; ++i) {
    const int ks = q + KS * i;                 // K step of the stage
    const int slot = (2 * ks + (lane >> 5)) ^ (r & 7);
    aoff[i] = r * 128 + slot * 16;
    boff[i] = (32 + 32 * blk + r) * 128 + slot * 16;
  }
  // Software pipeline: the operands of stage s+1 are read from LDS while
  // the MFMAs of stage s run (issued after them, into the other register
  // set); even and odd K steps go to two accumulators so consecutive MFMAs
  // do not wait on each other.
  constexpr int KPS = 4 / KS;                  // K steps per wavefront per stage
  u32x4 fa[2][KPS], fb[2][KPS];
  auto read = [&](int s, auto J) {
    constexpr int j = decltype(J)::value;
    const uint8_t* base = smem + (s % NS) * STAGE;
#pragma unroll
    for (int i = 0; i < KPS; ++i) {
      fa[j][i] = *reinterpret_cast<const u32x4*>(base + aoff[i]);
      fb[j][i] = *reinterpret_cast<const u32x4*>(base + boff[i]);
    }
  };
  f32x16 acc[2];
#pragma unroll
  for (int i = 0; i < 16; ++i) acc[0][i] = acc[1][i] = 0.0f;
  auto step = [&](int s, auto J) {
    constexpr int j = decltype(J)::value;
    // stage s+1 has landed once at most the copies of the stages after it
    // (at most NS - 3) are in flight
    if (s + 1 < nk) wait_stages<CPW, NS - 3>(min(NS - 3, nk - 2 - s));
    barrier_only();                            // every wavefront has read stage s-1's slot
    if (s + NS - 1 < nk) issue(s + NS - 1);
#pragma unroll
    for (int i = 0; i < KPS; ++i)
      acc[i & 1] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, fa[j][i]),
                                                           __builtin_bit_cast(bf16x8, fb[j][i]), acc[i & 1], 0, 0, 0);
    if (s + 1 < nk) read(s + 1, std::integral_constant<int, j ^ 1>());
  };

  for (int s = 0; s < NS - 1 && s < nk; ++s) issue(s);
  wait_stages<CPW, NS - 2>(min(NS - 2, nk - 1));   // stage 0
  barrier_only();
  read(0, std::integral_constant<int, 0>());
  for (int s = 0; s < nk; s += 2) {
    step(s, std::integral_constant<int, 0>());
    if (s + 1 < nk) step(s + 1, std::integral_constant<int, 1>());
  }
  acc[0] += acc[1];
  if constexpr (KS > 1) {
    __syncthreads();                           // the ring is free: partial sums go there
    float* part = reinterpret_cast<float*>(smem);
    if (q > 0) {
#pragma unroll
      for (int i = 0; i < 16; ++i) part[((q - 1) * NE + blk) * 1024 + i * 64 + lane] = acc[0][i];
    }
    __syncthreads();
    if (q > 0) return;
#pragma unroll
    for (int j = 1; j < KS; ++j)
#pragma unroll
      for (int i = 0; i < 16; ++i) acc[0][i] += part[((j - 1) * NE + blk) * 1024 + i * 64 + lane];
  }
  // acc[0][i] holds token 8(i/4) + 4(lane/32) + i%4, expert 32*blk + lane%32
  const int e = e0 + 32 * blk + r;
  if (e >= E) return;
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    const int t = t0 + 8 * (i >> 2) + 4 * (lane >> 5) + (i & 3);
    if (t < T_) logits[static_cast<int64_t>(t) * E + e] = acc[0][i];
  }
}

// bf16 with a workgroup per CU of 32-token blocks: the LDS-staged kernel.
// Otherwise the register-operand kernel with the widest expert tile that
// still gives RIMURU_ROUTER_MINWG workgroups (LA keeps about 16 tile loads in
// flight per lane); for bf16 (H a multiple of 64 in the layer) that is one
// 16-expert block per workgroup.
template <typename T>
void launch_router(const RouterArgs& r, int n_tok, int E, hipStream_t st) {
  if constexpr (std::is_same<T, uint16_t>::value) {
    // many tokens: whole-row stages through LDS, the widest expert tile that
    // still gives a workgroup per CU
    const int64_t tb = (n_tok + 31) / 32;
    if (r.H % 64 == 0 && tb * ((E + 31) / 32) >= kRouterWideMinWG) {
      const uint16_t* xr = static_cast<const uint16_t*>(r.x);
      const uint16_t* wr = static_cast<const uint16_t*>(r.w_gate);
      if (tb * ((E + 127) / 128) >= kRouterWideMinWG)
        hipLaunchKernelGGL(k_router_wide<4>, dim3(tb, (E + 127) / 128), dim3(256), 0, st, xr, wr, n_tok, E, r.H,
                           r.logits_out);
      else if (tb * ((E + 63) / 64) >= kRouterWideMinWG)
        hipLaunchKernelGGL(k_router_wide<2>, dim3(tb, (E + 63) / 64), dim3(256), 0, st, xr, wr, n_tok, E, r.H,
                           r.logits_out);
      else
        hipLaunchKernelGGL(k_router_wide<1>, dim3(tb, (E + 31) / 32), dim3(256), 0, st, xr, wr, n_tok, E, r.H,
                           r.logits_out);
      return;
    }
  }
  int nsplit = 1;
  for (int n = kRouterGW; n > 1; n /= 2)
    if (r.H % (32 * n) == 0) { nsplit = n; break; }
  const int64_t tb = (n_tok + 15) / 16, et = (E + 15) / 16;
  auto blocks = [&](int nt) { return tb * ((et + nt - 1) / nt); };
  if (blocks(8) >= RIMURU_ROUTER_MINWG) launch_router_nt<T, 8, 2>(r, n_tok, E, nsplit, st);
  else if (blocks(4) >= RIMURU_ROUTER_MINWG) launch_router_nt<T, 4, 4>(r, n_tok, E, nsplit, st);
  else if (blocks(2) >= RIMURU_ROUTER_MINWG) launch_router_nt<T, 2, 8>(r, n_tok, E, nsplit, st);
  else launch_router_nt<T, 1, 8>(r, n_tok, E, nsplit, st);
}

// ---------------------------------------------------------------- stage 2: count

// The slot list is cut into gridDim.y consecutive ranges of a multiple of 4
// slots; workgroup (e, s) counts expert e's slots in range s into
// counts[e * S + s] (several workgroups per expert when there are few
// experts, so that every CU scans). ids is 16-byte aligned (validated); 8
// independent 16-byte loads per thread are in flight per round.
__device__ __forceinline__ void slot_range(int TK, int s, int S, int* lo, int* hi) {
  const int per = ((TK + S - 1) / S + 3) & ~3;
  *lo = min(s * per, TK);
  *hi = min(*lo + per, TK);
}

template <int NT>
__global__ __launch_bounds__(NT) void k_count(const int32_t* __restrict__ ids, int TK,
                                              int32_t* __restrict__ counts) {
  __shared__ int part[NT / 64];
  const int e = blockIdx.x, s = blockIdx.y, S = gridDim.y;
  int lo, hi;
  slot_range(TK, s, S, &lo, &hi);
  const int n4 = (hi - lo) >> 2;
  const u32x4* v = reinterpret_cast<const u32x4*>(ids + lo);
  const uint32_t ue = static_cast<uint32_t>(e);
  int c = 0;
  for (int base = 0; base < n4; base += NT * 8) {
    u32x4 r[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const int i = base + u * NT + threadIdx.x;
      r[u] = (i < n4) ? v[i] : u32x4{~0u, ~0u, ~0u, ~0u};
    }
#pragma unroll
    for (int u = 0; u < 8; ++u)
      c += (r[u][0] == ue) + (r[u][1] == ue) + (r[u][2] == ue) + (r[u][3] == ue);
  }
  for (int f = lo + n4 * 4 + threadIdx.x; f < hi; f += NT) c += (ids[f] == e);
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) c += __shfl_xor(c, off, 64);
  if ((threadIdx.x & 63) == 0) part[threadIdx.x >> 6] = c;
  __syncthreads();
  if (threadIdx.x == 0) {
    int sum = 0;
#pragma unroll
    for (int i = 0; i < NT / 64; ++i) sum += part[i];
    counts[e * S + s] = sum;
  }
}

// ---------------------------------------------------------------- stage 3: sort + align


constexpr int kSortChunk = 64;  // consecutive slots per thread per round (16 x 16-byte loads)

// counts == nullptr: the workgroup builds the per-expert histogram itself in
// LDS (small batches: this saves the separate count launch).
constexpr int kSortSelfCountMax = 4096;   // routed slots

// Workgroup (e, s) places expert e's slots of range s (the ranges of
// k_count, gridDim.y of them): after the slots of the earlier ranges, so the
// segment stays in ascending slot order. The last range's workgroup pads the
// segment and writes its tiles' expert, the first the segment's start.
template <int NT>
__global__ __launch_bounds__(NT) void k_sort_align(const int32_t* __restrict__ ids, int TK, int E,
                                                   int BM, const int32_t* __restrict__ counts,
                                                   int32_t* __restrict__ sorted_ids,
                                                   int32_t* __restrict__ expert_off,
                                                   int32_t* __restrict__ tile_expert) {
  __shared__ int sh[NT / 64];
  __shared__ int hist[kMaxE];
  const int e = blockIdx.x, s = blockIdx.y, S = gridDim.y;
  const int tid = threadIdx.x;
  const uint32_t ue = static_cast<uint32_t>(e);
  int cs = S;                                     // counts of expert e2: cnt_of(e2) sums its S ranges
  if (counts == nullptr) {
    for (int i = tid; i < E; i += NT) hist[i] = 0;
    __syncthreads();
    for (int f = tid; f < TK; f += NT) atomicAdd(&hist[ids[f]], 1);
    __syncthreads();
    counts = hist;
    cs = 1;
  }
  auto cnt_of = [&](int e2) {
    int c = 0;
    for (int j = 0; j < cs; ++j) c += counts[e2 * cs + j];
    return c;
  };
  // start of this expert's padded segment, and the padded total
  int before = 0, total = 0;
  for (int e2 = tid; e2 < E; e2 += NT) {
    int pc = (cnt_of(e2) + BM - 1) / BM * BM;
    total += pc;
    before += (e2 < e) ? pc : 0;
  }
  int sum_before, sum_total;
  block_excl_scan<NT>(before, &sum_before, sh);   // block sums of the per-thread partials
  block_excl_scan<NT>(total, &sum_total, sh);
  const int seg = sum_before;
  const int cnt = cnt_of(e);
  int earlier = 0;                                // this expert's slots in the ranges before s
  for (int j = 0; j < s; ++j) earlier += counts[e * cs + j];
  if (tid == 0 && s == 0) {
    expert_off[e] = seg;
    if (e == 0) expert_off[E] = sum_total;
  }
  int lo = 0, hi = TK;
  if (cs > 1) slot_range(TK, s, S, &lo, &hi);
  const bool vec = (TK & 3) == 0;
  int running = 0;
  for (int base = lo; base < hi; base += NT * kSortChunk) {
    const int f0 = base + tid * kSortChunk;
    uint64_t mask = 0;
    if (vec) {
      u32x4 r[kSortChunk / 4];
#pragma unroll
      for (int u = 0; u < kSortChunk / 4; ++u)
        r[u] = (f0 + 4 * u < hi) ? *reinterpret_cast<const u32x4*>(ids + f0 + 4 * u)
                                 : u32x4{~0u, ~0u, ~0u, ~0u};
#pragma unroll
      for (int u = 0; u < kSortChunk / 4; ++u)
#pragma unroll
        for (int c = 0; c < 4; ++c) mask |= static_cast<uint64_t>(r[u][c] == ue) << (4 * u + c);
    } else {
      for (int i = 0; i < kSortChunk; ++i) {
        const int f = f0 + i;
        if (f < hi && ids[f] == e) mask |= 1ull << i;
      }
    }
    int chunk_total;
    int pos = seg + earlier + running + block_excl_scan<NT>(__popcll(mask), &chunk_total, sh);
    while (mask) {
      const int i = __ffsll(static_cast<long long>(mask)) - 1;
      sorted_ids[pos++] = f0 + i;
      mask &= mask - 1;
    }
    running += chunk_total;
  }
  if (s == S - 1) {
    const int padded = (cnt + BM - 1) / BM * BM;
    for (int i = cnt + tid; i < padded; i += NT) sorted_ids[seg + i] = TK;
    for (int i = tid; i < padded / BM; i += NT) tile_expert[seg / BM + i] = e;
  }
}

// ---------------------------------------------------------------- stages 1-3 for small batches

// One workgroup routes a small batch end to end (one launch instead of the
// gating and sort launches): its 16 wavefronts take the tokens in turn for the
// top-k (the same selection as k_gating), then the segments are laid out as
// k_sort_align lays them out (slots in ascending order, sentinel T*k, tile ->
// expert map): thread e pads expert e's segment, thread f places slot f.
constexpr int kTinyThreads = 1024;
// Up to 16 tokens (one per wavefront). Measured on the 128-expert decode
// layer, cache-cold: 1 and 4 tokens 3 us faster per layer than the gating +
// sort pair, 16 tokens even; at 64 tokens (4 per wavefront, selected one
// after another) the routing stage took 26.5 us against about 14 us.
constexpr int kTinyMaxT = 16;       // tokens
constexpr int kTinyMaxTK = 512;     // routed slots

template <int EPL>
__global__ __launch_bounds__(kTinyThreads) void k_route_tiny(const float* __restrict__ logits, int T, int E, int k,
                                                             int BM, int32_t* __restrict__ topk_ids,
                                                             float* __restrict__ topk_w,
                                                             int32_t* __restrict__ sorted_ids,
                                                             int32_t* __restrict__ expert_off,
                                                             int32_t* __restrict__ tile_expert) {
  __shared__ __attribute__((aligned(16))) int32_t ids[kTinyMaxTK];
  __shared__ int hist[kMaxE];
  __shared__ int sh[kTinyThreads / 64];
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const int TK = T * k;
  for (int e = tid; e < E; e += kTinyThreads) hist[e] = 0;
  // every logits row of the wavefront is loaded before the first selection
  constexpr int kWaves = kTinyThreads / 64;
  constexpr int TPW = kTinyMaxT / kWaves;           // tokens per wavefront
  float v[TPW][EPL];
#pragma unroll
  for (int i = 0; i < TPW; ++i)
    if (wv + kWaves * i < T) load_logits<EPL>(logits + static_cast<int64_t>(wv + kWaves * i) * E, E, lane, v[i]);
#pragma unroll
  for (int i = 0; i < TPW; ++i) {
    const int t = wv + kWaves * i;
    if (t >= T) break;
    uint32_t e;
    float wt;
    select_topk_vals<EPL>(v[i], E, k, lane, &e, &wt);
    if (lane < k) {
      ids[t * k + lane] = static_cast<int32_t>(e);
      topk_ids[t * k + lane] = static_cast<int32_t>(e);
      topk_w[t * k + lane] = wt;
    }
  }
  __syncthreads();
  if (tid < TK) atomicAdd(&hist[ids[tid]], 1);
  __syncthreads();
  const int e = tid;
  const int cnt = e < E ? hist[e] : 0;
  const int padded = (cnt + BM - 1) / BM * BM;
  int total;
  const int seg = block_excl_scan<kTinyThreads>(padded, &total, sh);
  if (e < E) {
    hist[e] = seg;                                  // segment starts (counts are no longer needed)
    expert_off[e] = seg;
    if (e == 0) expert_off[E] = total;
    for (int i = cnt; i < padded; ++i) sorted_ids[seg + i] = TK;
    for (int i = 0; i < padded / BM; ++i) tile_expert[seg / BM + i] = e;
  }
  __syncthreads();
  // slot f goes to its expert's segment at its rank among the expert's
  // earlier slots (ascending slot order, as the stable sort gives)
  if (tid < TK) {
    const int my = ids[tid];
    int rank = 0;
    const int4* q4 = reinterpret_cast<const int4*>(ids);
    for (int q = 0; q < (tid >> 2); ++q) {
      const int4 v = q4[q];
      rank += (v.x == my) + (v.y == my) + (v.z == my) + (v.w == my);
    }
    for (int f = tid & ~3; f < tid; ++f) rank += ids[f] == my;
    sorted_ids[hist[my] + rank] = tid;
  }
}

// ---------------------------------------------------------------- stage 6: combine

// KMAX >= k: all k slot rows are loaded before the first is added (rows past
// k reload row k-1 and are not added), so a thread waits for one memory
// round trip instead of k; the sum still runs j = 0 .. k-1 in order.
// Each slot row is read once: the loads are non-temporal (8192-token
// prefill: 53 -> 48 us).
template <typename T, int KMAX>
__global__ __launch_bounds__(256) void k_combine(const T* __restrict__ yslot, int k, int H,
                                                 T* __restrict__ y) {
  typedef Elt<T> X;
  constexpr int VEC = X::VEC;
  const int t = blockIdx.x;
  const int h0 = (blockIdx.y * 256 + threadIdx.x) * VEC;
  if (h0 >= H) return;
  float acc[VEC];
#pragma unroll
  for (int c = 0; c < VEC; ++c) acc[c] = 0.0f;
  u32x4 rows[KMAX];
#pragma unroll
  for (int j = 0; j < KMAX; ++j)
    rows[j] = __builtin_nontemporal_load(
        reinterpret_cast<const u32x4*>(yslot + (static_cast<int64_t>(t) * k + min(j, k - 1)) * H + h0));
#pragma unroll
  for (int j = 0; j < KMAX; ++j) {
    if (j < k) {
#pragma unroll
      for (int c = 0; c < VEC; ++c) acc[c] += X::to_f32(X::get(rows[j], c));
    }
  }
  u32x4 o;
  if constexpr (X::ES == 2) {
#pragma unroll
    for (int c = 0; c < 4; ++c) o[c] = X::from_f32(acc[2 * c]) | (X::from_f32(acc[2 * c + 1]) << 16);
  } else {
#pragma unroll
    for (int c = 0; c < 4; ++c) o[c] = X::from_f32(acc[c]);
  }
  *reinterpret_cast<u32x4*>(y + static_cast<int64_t>(t) * H + h0) = o;
}

// ---------------------------------------------------------------- weight loading

// A page-table entry naming a page outside the pool (negative, or ending past
// pool_bytes) is skipped: its bytes are not stored and nothing outside the
// pool is ever written.
__global__ __launch_bounds__(256) void k_store_pages(uint8_t* __restrict__ pool, uint64_t pool_pages,
                                                     const int32_t* __restrict__ pt, int P,
                                                     PageDiv pd, const uint8_t* __restrict__ src,
                                                     uint64_t proj_bytes, uint64_t n_segs) {
  for (uint64_t s = blockIdx.x * 256ull + threadIdx.x; s < n_segs; s += gridDim.x * 256ull) {
    uint64_t byte = s * 16;
    uint64_t proj = byte / proj_bytes;
    uint32_t off = static_cast<uint32_t>(byte - proj * proj_bytes);
    uint32_t q = page_index(off, pd);
    const int32_t pg = pt[proj * P + q];
    if (pg < 0 || static_cast<uint64_t>(pg) >= pool_pages) continue;
    uint8_t* dst = pool + static_cast<uint64_t>(pg) * pd.page + (off - q * pd.page);
    *reinterpret_cast<u32x4*>(dst) = *reinterpret_cast<const u32x4*>(src + byte);
  }
}

// ---------------------------------------------------------------- calibration read

// One pass over buf: each thread loads 16-byte pieces gtid, gtid + stride,
// ... eight at a time (independent non-temporal loads in flight; measured the
// fastest of plain/non-temporal loads, 4/8/16 in flight and grids of 1024 to
// 16384 workgroups), XOR-folds them, and stores only when the fold equals a
// fixed pattern, so no load can be dropped and (almost) nothing is written.
constexpr int kReadUnroll = 8;
constexpr int kReadGrid = 16384;

__global__ __launch_bounds__(256) void k_stream_read(const u32x4* __restrict__ buf, uint64_t n16,
                                                     uint32_t* __restrict__ sink) {
  const uint64_t stride = static_cast<uint64_t>(gridDim.x) * 256;
  uint64_t i = static_cast<uint64_t>(blockIdx.x) * 256 + threadIdx.x;
  uint32_t acc = 0;
  for (; i + (kReadUnroll - 1) * stride < n16; i += kReadUnroll * stride) {
    u32x4 v[kReadUnroll];
#pragma unroll
    for (int u = 0; u < kReadUnroll; ++u) v[u] = __builtin_nontemporal_load(buf + i + u * stride);
#pragma unroll
    for (int u = 0; u < kReadUnroll; ++u) acc ^= v[u][0] ^ v[u][1] ^ v[u][2] ^ v[u][3];
  }
  for (; i < n16; i += stride) {
    const u32x4 a = buf[i];
    acc ^= a[0] ^ a[1] ^ a[2] ^ a[3];
  }
  if (acc == 0x5A5A5A5Au) *sink = acc;
}

hipError_t launch_stream_read(const void* buf, uint64_t bytes, uint32_t* sink, hipStream_t st) {
  const uint64_t n16 = bytes / 16;
  if (n16 == 0) return hipSuccess;
  hipLaunchKernelGGL(k_stream_read, dim3(kReadGrid), dim3(256), 0, st, static_cast<const u32x4*>(buf), n16, sink);
  return hipGetLastError();
}

// ---------------------------------------------------------------- launchers

PageDiv make_div(uint32_t page) {
  uint32_t l = 0;
  while ((1ull << l) < page) ++l;
  unsigned __int128 num = (static_cast<unsigned __int128>(1) << 32) * ((1ull << l) - page);
  uint64_t m = static_cast<uint64_t>(num / page) + 1 + (1ull << 32);
  return PageDiv{m, 32 + l, page};
}

hipError_t launch_routing(const float* logits, const RouterArgs* router, int T, int E, int k, int bm,
                          int32_t* topk_ids, float* topk_w, int32_t* counts, int32_t* sorted_ids,
                          int32_t* expert_off, int32_t* tile_expert, hipEvent_t* ev, hipStream_t st) {
  hipError_t err;
  auto mark = [&](int i) -> hipError_t { return ev ? hipEventRecord(ev[i], st) : hipSuccess; };
  const int TK = T * k;
  const int epl = (E + 63) / 64;
  if (router != nullptr) {   // logits = x . w_gate^T first, into router->logits_out
    if (router->bf16) launch_router<uint16_t>(*router, T, E, st);
    else launch_router<float>(*router, T, E, st);
    if ((err = hipGetLastError()) != hipSuccess) return err;
    logits = router->logits_out;
  }
  if (T <= kTinyMaxT && TK <= kTinyMaxTK && E <= kTinyThreads) {
    // a small batch: routing in one workgroup, one launch
    if (epl <= 1) hipLaunchKernelGGL(k_route_tiny<1>, dim3(1), dim3(kTinyThreads), 0, st, logits, T, E, k, bm, topk_ids,
                                     topk_w, sorted_ids, expert_off, tile_expert);
    else if (epl <= 2) hipLaunchKernelGGL(k_route_tiny<2>, dim3(1), dim3(kTinyThreads), 0, st, logits, T, E, k, bm,
                                          topk_ids, topk_w, sorted_ids, expert_off, tile_expert);
    else if (epl <= 4) hipLaunchKernelGGL(k_route_tiny<4>, dim3(1), dim3(kTinyThreads), 0, st, logits, T, E, k, bm,
                                          topk_ids, topk_w, sorted_ids, expert_off, tile_expert);
    else hipLaunchKernelGGL(k_route_tiny<8>, dim3(1), dim3(kTinyThreads), 0, st, logits, T, E, k, bm, topk_ids,
                            topk_w, sorted_ids, expert_off, tile_expert);
    if ((err = hipGetLastError()) != hipSuccess) return err;
    if ((err = mark(1)) != hipSuccess) return err;
    return mark(2);
  }
  const dim3 grid((T + 3) / 4);
  if (epl <= 1) hipLaunchKernelGGL(k_gating<1>, grid, dim3(256), 0, st, logits, T, E, k, topk_ids, topk_w);
  else if (epl <= 2) hipLaunchKernelGGL(k_gating<2>, grid, dim3(256), 0, st, logits, T, E, k, topk_ids, topk_w);
  else if (epl <= 4) hipLaunchKernelGGL(k_gating<4>, grid, dim3(256), 0, st, logits, T, E, k, topk_ids, topk_w);
  else hipLaunchKernelGGL(k_gating<8>, grid, dim3(256), 0, st, logits, T, E, k, topk_ids, topk_w);
  if ((err = hipGetLastError()) != hipSuccess) return err;
  if ((err = mark(1)) != hipSuccess) return err;
  const bool self_count = TK <= kSortSelfCountMax;
  if (self_count) {
    if ((err = mark(2)) != hipSuccess) return err;
    hipLaunchKernelGGL(k_sort_align<256>, dim3(E), dim3(256), 0, st, topk_ids, TK, E, bm, nullptr, sorted_ids,
                       expert_off, tile_expert);
    return hipGetLastError();
  }
  // many slots: the slot list is cut into S ranges (up to kCountSplits) so
  // that a 256-thread workgroup's sort covers its range in one round, and
  // E * S small workgroups scan in parallel
  int S = 1;
  while (S < kCountSplits && static_cast<int64_t>(S) * 256 * kSortChunk < TK) S *= 2;
  hipLaunchKernelGGL(k_count<256>, dim3(E, S), dim3(256), 0, st, topk_ids, TK, counts);
  if ((err = hipGetLastError()) != hipSuccess) return err;
  if ((err = mark(2)) != hipSuccess) return err;
  hipLaunchKernelGGL(k_sort_align<256>, dim3(E, S), dim3(256), 0, st, topk_ids, TK, E, bm, counts, sorted_ids,
                     expert_off, tile_expert);
  return hipGetLastError();
}

template <typename T>
hipError_t launch_combine(const T* yslot, int T_, int k, int H, T* y, hipStream_t st) {
  constexpr int VEC = Elt<T>::VEC;
  const dim3 grid(T_, (H + 256 * VEC - 1) / (256 * VEC));
  if (k <= 2) hipLaunchKernelGGL((k_combine<T, 2>), grid, dim3(256), 0, st, yslot, k, H, y);
  else if (k <= 8) hipLaunchKernelGGL((k_combine<T, 8>), grid, dim3(256), 0, st, yslot, k, H, y);
  else hipLaunchKernelGGL((k_combine<T, kMaxK>), grid, dim3(256), 0, st, yslot, k, H, y);
  return hipGetLastError();
}
template hipError_t launch_combine<uint16_t>(const uint16_t*, int, int, int, uint16_t*, hipStream_t);
template hipError_t launch_combine<float>(const float*, int, int, int, float*, hipStream_t);

hipError_t launch_store_pages(uint8_t* pool, uint64_t pool_bytes, const int32_t* pt, int P, uint32_t page_bytes,
                              const uint8_t* src, uint64_t proj_bytes, uint64_t n_segs, hipStream_t st) {
  uint64_t blocks = (n_segs + 255) / 256;
  if (blocks > 65536) blocks = 65536;
  hipLaunchKernelGGL(k_store_pages, dim3(static_cast<uint32_t>(blocks)), dim3(256), 0, st, pool,
                     pool_bytes / page_bytes, pt, P, make_div(page_bytes), src, proj_bytes, n_segs);
  return hipGetLastError();
}

}  // namespace rimuru
