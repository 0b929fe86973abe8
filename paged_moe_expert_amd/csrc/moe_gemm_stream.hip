// Stages 4 and 5 of the fused MoE layer for few routed rows per expert
// (decode): the grouped GEMM is a stream of expert weights read page by page
// through the expert view's page table (Rimuru paper summary, abstract and
// Figure 11, "Discrete FusedMoE"; Table 1 for the projections).
#include <algorithm>

#include "moe_common.h"
#include "moe_topk.h"

namespace rimuru {

// ---------------------------------------------------------------- stages 4, 5 for few rows: weight streaming

// Few routed rows per expert: the GEMM is a weight stream. A workgroup owns
// one 16-row tile and BN columns; its ksplit wavefronts each own a
// contiguous K range and stream their weight rows with DEPTH steps of loads
// in flight. Each step a wavefront transposes its own 32 x BN weight slice
// through a private LDS buffer (LDS operations of one wavefront complete in
// issue order, so no barrier is needed) and runs the MFMAs; the A operand is
// loaded straight into registers. The ksplit partial sums are added in fixed
// wavefront order at the end, so results are deterministic.
constexpr int kStreamMaxWaves = 4;
constexpr int kStreamK = 32;      // K rows per wavefront step
// column-tile width and steps in flight of the gate/up and down streams
// (compile-time overridable for tuning sweeps), and workgroups per CU
#ifndef RIMURU_STREAM_UP
#define RIMURU_STREAM_UP 128, 2
#endif
#ifndef RIMURU_STREAM_DN
#define RIMURU_STREAM_DN 256, 2
#endif
#ifndef RIMURU_STREAM_WG_PER_CU
#define RIMURU_STREAM_WG_PER_CU 2
#endif
#ifndef RIMURU_STREAM_WAVES
#define RIMURU_STREAM_WAVES 4, 4
#endif
struct StreamWaves { int up, dn; };
constexpr StreamWaves kStreamWaves{RIMURU_STREAM_WAVES};
constexpr int kStreamUpWaves = kStreamWaves.up, kStreamDnWaves = kStreamWaves.dn;
#ifndef RIMURU_STREAM_NARROW
#define RIMURU_STREAM_NARROW 160, 32, 64
#endif
// Few experts touched: narrow the column tile (down to the given widths) while
// fewer than min_groups workgroups would stream. Measured cache-cold on the
// 2048x768 bf16 experts: one token (8 experts) streams gate/up 1.9x faster with
// 32-column tiles, while at 28 experts 168 workgroups of 128 columns beat 336
// of 64 (wider rows per page keep HBM bursts long), hence the low threshold.
struct StreamNarrow { int64_t min_groups; int up_bn, dn_bn; };
constexpr StreamNarrow kStreamNarrow{RIMURU_STREAM_NARROW};
// Average routed rows per expert up to which the weight loads are
// non-temporal. Measured on the 128-expert decode layer: 64 tokens (4 rows an
// expert) 280.6k -> 321.6k tokens/s; 16 tokens 152 -> 138 us cache-cold;
// 256 tokens (16 rows, many experts two row tiles) 1.5% slower cache-cold.
constexpr int kStreamNtRows = 8;
// load policy above kStreamNtRows rows per expert: 2 = per expert, 0 = plain
#ifndef RIMURU_STREAM_NT_MIXED
#define RIMURU_STREAM_NT_MIXED 2
#endif
struct StreamShape { int bn, depth; };
constexpr StreamShape kStreamUp{RIMURU_STREAM_UP}, kStreamDn{RIMURU_STREAM_DN};
// the same for 32-row tiles (two 16-row blocks of accumulators)
#ifndef RIMURU_STREAM32_UP
#define RIMURU_STREAM32_UP 128, 2
#endif
#ifndef RIMURU_STREAM32_DN
#define RIMURU_STREAM32_DN 128, 3
#endif
constexpr StreamShape kStream32Up{RIMURU_STREAM32_UP}, kStream32Dn{RIMURU_STREAM32_DN};
constexpr int kStreamUpBN = kStreamUp.bn, kStreamUpDepth = kStreamUp.depth;
constexpr int kStreamDnBN = kStreamDn.bn, kStreamDnDepth = kStreamDn.depth;

// LDS of one streaming wavefront (its weight slice, then its partial sums)
template <typename T, int BN, bool GATED>
constexpr int stream_wave_lds() {
  return (GATED ? 2 : 1) * kStreamK * (BN + Elt<T>::B_PAD);
}

// NSTEPS > 0: the wavefront's step count is known at compile time and the K
// loop unrolls into straight-line code (a loop back-edge makes the compiler
// wait for every load in flight at the loop head). NSTEPS == 0: runtime loop.
// ONE_PAGE: each projection lies in a single page (P == 1), so a weight
// segment's address is that page's address plus its offset; otherwise every
// segment looks its page up.
// NT: weight loads are non-temporal (streamed past the caches). A streaming
// read of HBM measured 6.9 TB/s with non-temporal loads against 6.2 TB/s
// with plain ones; taken when each expert's weights are read by one row tile
// (few routed rows per expert), where nothing re-reads them in the launch.
// One workgroup's tile (row tile mt of 16*MR rows, column tile nt of expert
// e): MR blocks of 16 rows share every weight fragment. lds holds
// kStreamMaxWaves wavefront slices of stream_wave_lds elements; pt_lds the
// expert's page-table rows (NB * P) when not ONE_PAGE.
template <typename T, int BN, int DEPTH, bool GATED, int NSTEPS, bool ONE_PAGE, bool NT, int MR>
__device__ __forceinline__ void stream_tile(const GemmArgs& a, int ksplit, int mt, int nt, int e, T* lds,
                                            int32_t* pt_lds) {
  typedef Elt<T> X;
  constexpr int NB = GATED ? 2 : 1;
  constexpr int VEC = X::VEC;
  constexpr int CG = BN / VEC;                 // 16-byte column groups per weight row
  constexpr int RG = 64 / CG;                  // row groups per wavefront
  constexpr int RPL = kStreamK / RG;           // consecutive weight rows per lane
  constexpr int TN = BN / 16;
  constexpr int BNP = BN + X::B_PAD;           // row pitch of the wave's weight slice
  constexpr int SEG8 = X::SEG8;
  constexpr int WL = stream_wave_lds<T, BN, GATED>();
  static_assert(CG * RG == 64 && RPL * RG == kStreamK, "stream tile shape");
  static_assert(NB * 16 * BN * 4 <= WL * X::ES, "reduction must fit the wave buffer");   // one row block at a time
  const int r0 = mt * 16 * MR;
  const int n0 = nt * BN;

  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  const int fi = lane & 15, fq = lane >> 4;
  const int kw = a.K / ksplit;
  const int nsteps = kw / kStreamK;
  const int kbase = wv * kw;

  // A operand: row fi of each 16-row block, K values fq*8 .. fq*8+7 of each
  // step. Padding rows read a valid row and are zeroed by a select, so the
  // main loop has no branch around a load (a branch there makes the compiler
  // wait for every load in flight at the join).
  const T* arow[MR];
  bool a_ok[MR];
#pragma unroll
  for (int m = 0; m < MR; ++m) {
    const int r = r0 + 16 * m + fi;
    a_ok[m] = true;
    if (a.kdiv > 0) {
      const int slot = a.sorted_ids[r];
      a_ok[m] = slot < a.TK;
      arow[m] = reinterpret_cast<const T*>(a.A) + static_cast<int64_t>(a_ok[m] ? slot / a.kdiv : 0) * a.lda;
    } else {
      arow[m] = reinterpret_cast<const T*>(a.A) + static_cast<int64_t>(r) * a.lda;
    }
  }
  const int cg = lane % CG, rg = lane / CG;
  // Page lookups read LDS: a global load here would make every weight load
  // wait for all older ones (vector-memory loads retire in order).
  const int32_t* pt_row[NB];
  const uint8_t* page0[NB];                    // ONE_PAGE: the projection's page
  if constexpr (ONE_PAGE) {
#pragma unroll
    for (int b = 0; b < NB; ++b)
      page0[b] = a.pool + static_cast<uint64_t>(static_cast<uint32_t>(a.pt[e * 3 + (GATED ? b : 2)])) * a.pd.page;
  } else {
    for (int i = threadIdx.x; i < NB * a.P; i += blockDim.x) {
      const int b = i / a.P, q = i - b * a.P;
      pt_lds[i] = a.pt[static_cast<int64_t>(e * 3 + (GATED ? b : 2)) * a.P + q];
    }
    __syncthreads();
#pragma unroll
    for (int b = 0; b < NB; ++b) pt_row[b] = pt_lds + b * a.P;
  }
  const uint32_t col_bytes = static_cast<uint32_t>(n0 + cg * VEC) * X::ES;
  const uint32_t row_bytes = static_cast<uint32_t>(a.N) * X::ES;

  u32x4 breg[DEPTH][NB][RPL];
  u32x4 areg[DEPTH][MR][SEG8];
  f32x4 acc[MR][NB][TN];
#pragma unroll
  for (int m = 0; m < MR; ++m)
#pragma unroll
    for (int b = 0; b < NB; ++b)
#pragma unroll
      for (int j = 0; j < TN; ++j) acc[m][b][j] = f32x4{0.f, 0.f, 0.f, 0.f};

  T* wbuf = lds + wv * WL;

  // Loads of step st (clamped to the last step: the surplus loads at the end
  // repeat addresses already in cache and their data is never used).
  auto issue = [&](u32x4 (&br)[NB][RPL], u32x4 (&ar)[MR][SEG8], int st) {
    st = min(st, nsteps - 1);
    const int k0 = kbase + st * kStreamK;
#pragma unroll
    for (int m = 0; m < MR; ++m)
#pragma unroll
      for (int u = 0; u < SEG8; ++u) ar[m][u] = *reinterpret_cast<const u32x4*>(arow[m] + k0 + fq * 8 + u * VEC);
#pragma unroll
    for (int b = 0; b < NB; ++b) {
#pragma unroll
      for (int j = 0; j < RPL; ++j) {
        const uint32_t f = static_cast<uint32_t>(k0 + rg * RPL + j) * row_bytes + col_bytes;
        const uint8_t* p;
        if constexpr (ONE_PAGE) {
          p = page0[b] + f;
        } else {
          const uint32_t q = page_index(f, a.pd);
          p = a.pool + static_cast<uint64_t>(pt_row[b][q]) * a.pd.page + (f - q * a.pd.page);
        }
        if constexpr (NT)
          br[b][j] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
        else
          br[b][j] = *reinterpret_cast<const u32x4*>(p);
      }
    }
  };

  // Multiply step data into the accumulators; live == false (a step past the
  // end) multiplies by a zero A operand, which adds exact zeros.
  auto consume = [&](const u32x4 (&br)[NB][RPL], const u32x4 (&ar)[MR][SEG8], bool live) {
    // the wave's weight slice, row-major as it sits in the pool
#pragma unroll
    for (int b = 0; b < NB; ++b)
#pragma unroll
      for (int j = 0; j < RPL; ++j)
        *reinterpret_cast<u32x4*>(wbuf + b * kStreamK * BNP + (rg * RPL + j) * BNP + cg * VEC) = br[b][j];
    u32x4 af[MR][SEG8];
#pragma unroll
    for (int m = 0; m < MR; ++m) {
      const bool use = live && a_ok[m];
#pragma unroll
      for (int u = 0; u < SEG8; ++u) af[m][u] = use ? ar[m][u] : u32x4{0u, 0u, 0u, 0u};
    }
#pragma unroll
    for (int b = 0; b < NB; ++b) {
#pragma unroll
      for (int j = 0; j < TN; ++j) {
        u32x4 bf[SEG8];
        X::bfrag16(wbuf + b * kStreamK * BNP, BNP, 0, j * 16, lane, bf);
#pragma unroll
        for (int m = 0; m < MR; ++m) acc[m][b][j] = X::mma8(af[m], bf, acc[m][b][j]);
      }
    }
  };

  if constexpr (NSTEPS > 0) {
    // Straight-line pipeline: DEPTH - 1 steps in flight ahead of the one consumed.
#pragma unroll
    for (int d = 0; d < DEPTH - 1; ++d)
      if (d < NSTEPS) issue(breg[d], areg[d], d);
#pragma unroll
    for (int st = 0; st < NSTEPS; ++st) {
      if (st + DEPTH - 1 < NSTEPS)
        issue(breg[(st + DEPTH - 1) % DEPTH], areg[(st + DEPTH - 1) % DEPTH], st + DEPTH - 1);
      consume(breg[st % DEPTH], areg[st % DEPTH], true);
    }
  } else {
    // Branch-free loop: DEPTH - 1 steps in flight ahead of the one consumed.
#pragma unroll
    for (int d = 0; d < DEPTH - 1; ++d) issue(breg[d], areg[d], d);
    for (int s0 = 0; s0 < nsteps; s0 += DEPTH) {
#pragma unroll
      for (int d = 0; d < DEPTH; ++d) {
        issue(breg[(d + DEPTH - 1) % DEPTH], areg[(d + DEPTH - 1) % DEPTH], s0 + d + DEPTH - 1);
        consume(breg[d], areg[d], s0 + d < nsteps);
      }
    }
  }

  // ---- reduce the ksplit partial sums in wavefront order, then the
  // epilogue, one 16-row block at a time through the wavefronts' buffers
  float* red = reinterpret_cast<float*>(wbuf);           // [NB][16][BN] of this wavefront
  constexpr int PER = 4;                                  // outputs per thread per pass
  T* C = reinterpret_cast<T*>(a.C);
#pragma unroll
  for (int m = 0; m < MR; ++m) {
    __syncthreads();                                      // buffers free: last step done, block m-1 read
#pragma unroll
    for (int b = 0; b < NB; ++b)
#pragma unroll
      for (int j = 0; j < TN; ++j)
#pragma unroll
        for (int r = 0; r < 4; ++r) red[(b * 16 + 4 * fq + r) * BN + j * 16 + fi] = acc[m][b][j][r];
    __syncthreads();
    for (int o = threadIdx.x * PER; o < 16 * BN; o += blockDim.x * PER) {
      const int lrow = o / BN, col = o % BN;
      const int row = r0 + 16 * m + lrow;
      float v[NB][PER];
#pragma unroll
      for (int b = 0; b < NB; ++b)
#pragma unroll
        for (int c = 0; c < PER; ++c) v[b][c] = 0.0f;
      for (int w = 0; w < ksplit; ++w) {
        const float* rw = reinterpret_cast<const float*>(lds + w * WL);
#pragma unroll
        for (int b = 0; b < NB; ++b)
#pragma unroll
          for (int c = 0; c < PER; ++c) v[b][c] += rw[(b * 16 + lrow) * BN + col + c];
      }
      if constexpr (GATED) {
        T* dst = C + static_cast<int64_t>(row) * a.ldc + n0 + col;
#pragma unroll
        for (int c = 0; c < PER; ++c) X::put(dst + c, silu(v[0][c]) * v[1][c]);
      } else {
        const int slot = a.sorted_ids[row];
        if (slot < a.TK) {
          const float wt = a.topk_w[slot];
          T* dst = C + static_cast<int64_t>(slot) * a.ldc + n0 + col;
#pragma unroll
          for (int c = 0; c < PER; ++c) X::put(dst + c, wt * v[0][c]);
        }
      }
    }
  }
}

// NT_MODE 0: plain weight loads, 1: non-temporal, 2: per expert --
// non-temporal when the expert's rows are one tile (nothing else in the
// launch reads its weights), plain when several row tiles share them.
template <typename T, int BN, int DEPTH, bool GATED, int NSTEPS, bool ONE_PAGE, int NT_MODE, int MR>
__global__ __launch_bounds__(kStreamMaxWaves * 64, RIMURU_STREAM_WG_PER_CU) void k_paged_gemm_stream(GemmArgs a, int ksplit) {
  __shared__ __attribute__((aligned(16))) T lds[kStreamMaxWaves * stream_wave_lds<T, BN, GATED>()];
  extern __shared__ int32_t pt_lds[];          // this expert's page-table rows (NB * P)

  const int nN = a.N / BN;
  const int n_tiles = a.expert_off[a.E] / (16 * MR);
  const int L = n_tiles * nN;
  const int chunk = (L + 7) >> 3;
  const int xcd = blockIdx.x & 7, idx = blockIdx.x >> 3;
  if (idx >= chunk) return;
  const int logical = xcd * chunk + idx;
  if (logical >= L) return;
  const int mt = logical / nN;
  const int nt = logical - mt * nN;
  const int e = a.tile_expert[mt];
  if constexpr (NT_MODE == 2) {
    if (a.expert_off[e + 1] - a.expert_off[e] == 16 * MR)
      stream_tile<T, BN, DEPTH, GATED, NSTEPS, ONE_PAGE, true, MR>(a, ksplit, mt, nt, e, lds, pt_lds);
    else
      stream_tile<T, BN, DEPTH, GATED, NSTEPS, ONE_PAGE, false, MR>(a, ksplit, mt, nt, e, lds, pt_lds);
  } else {
    stream_tile<T, BN, DEPTH, GATED, NSTEPS, ONE_PAGE, NT_MODE == 1, MR>(a, ksplit, mt, nt, e, lds, pt_lds);
  }
}

// Gate/up stream of a tiny batch (at most kRoutedMaxT tokens) with the
// routing done in the same launch: every workgroup selects the top-k of each
// token and builds the per-expert lists in its own LDS (the same lists in
// every workgroup, as the separate routing kernels would write them), then
// takes its tile from that copy; workgroup 0 also writes the lists and the
// top-k out for the down GEMM, the combine and the caller. This removes the
// routing launch, the largest fixed cost of a one-token layer.
template <typename T, int BN, int DEPTH, int NSTEPS, bool ONE_PAGE>
__global__ __launch_bounds__(kStreamMaxWaves * 64, RIMURU_STREAM_WG_PER_CU) void k_paged_gemm_stream_routed(
    GemmArgs a, int ksplit, TinyRoute rt) {
  __shared__ __attribute__((aligned(16))) T lds[kStreamMaxWaves * stream_wave_lds<T, BN, true>()];
  extern __shared__ int32_t pt_lds[];
  __shared__ int32_t s_ids[kRoutedMaxTK];
  __shared__ float s_w[kRoutedMaxTK];
  __shared__ int32_t s_off[kRoutedMaxE + 1];
  __shared__ int32_t s_sorted[kRoutedMaxSorted];
  __shared__ int32_t s_tile[kRoutedMaxSorted / 16];
  __shared__ int s_scan[kStreamMaxWaves];
  __shared__ int32_t s_pt[3 * kRoutedMaxE];
  constexpr int EPL = kRoutedMaxE / 64;
  constexpr int PTJ = 3 * kRoutedMaxE / (kStreamMaxWaves * 64);
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const int E = a.E, k = rt.k, TK = a.TK;

  // one page a projection: every expert's page-table row (3 entries) is read
  // together with the logits and kept in LDS, so no workgroup waits on a
  // global read for its weights' page after the selection
  int32_t ptv[PTJ];
  if constexpr (ONE_PAGE) {
#pragma unroll
    for (int j = 0; j < PTJ; ++j) {
      const int i = tid + j * kStreamMaxWaves * 64;
      ptv[j] = i < 3 * E ? a.pt[i] : 0;
    }
  }
  // top-k of token wv (one wavefront a token)
  if (wv < rt.T) {
    float v[EPL];
    load_logits<EPL>(rt.logits + static_cast<int64_t>(wv) * E, E, lane, v);
    uint32_t e;
    float wt;
    select_topk_vals<EPL>(v, E, k, lane, &e, &wt);
    if (lane < k) {
      s_ids[wv * k + lane] = static_cast<int32_t>(e);
      s_w[wv * k + lane] = wt;
    }
  }
  if constexpr (ONE_PAGE) {
#pragma unroll
    for (int j = 0; j < PTJ; ++j) {
      const int i = tid + j * kStreamMaxWaves * 64;
      if (i < 3 * E) s_pt[i] = ptv[j];
    }
  }
  __syncthreads();
  // per-expert segments padded to 16 rows (one expert a thread), their
  // starts by a block scan, then every slot at its rank among its expert's
  // earlier slots (ascending slot order, the stable grouping)
  const int cnt_e = [&] {
    int c = 0;
    if (tid < E)
      for (int f = 0; f < TK; ++f) c += s_ids[f] == tid;
    return c;
  }();
  const int padded = (cnt_e + 15) / 16 * 16;
  int total;
  const int seg = block_excl_scan<kStreamMaxWaves * 64>(padded, &total, s_scan);
  if (tid < E) {
    s_off[tid] = seg;
    for (int i = cnt_e; i < padded; ++i) s_sorted[seg + i] = TK;
    for (int i = 0; i < padded / 16; ++i) s_tile[seg / 16 + i] = tid;
  }
  if (tid == 0) s_off[E] = total;
  __syncthreads();
  if (tid < TK) {
    const int my = s_ids[tid];
    int rank = 0;
    for (int f = 0; f < tid; ++f) rank += s_ids[f] == my;
    s_sorted[s_off[my] + rank] = tid;
  }
  __syncthreads();
  if (blockIdx.x == 0) {
    if (tid < TK) {
      rt.topk_ids[tid] = s_ids[tid];
      rt.topk_w[tid] = s_w[tid];
    }
    for (int i = tid; i < total; i += blockDim.x) rt.sorted_ids[i] = s_sorted[i];
    for (int i = tid; i <= E; i += blockDim.x) rt.expert_off[i] = s_off[i];
    for (int i = tid; i < total / 16; i += blockDim.x) rt.tile_expert[i] = s_tile[i];
  }

  // this workgroup's tile, as the stream kernel maps them
  const int nN = a.N / BN;
  const int L = (total / 16) * nN;
  const int chunk = (L + 7) >> 3;
  const int xcd = blockIdx.x & 7, idx = blockIdx.x >> 3;
  if (idx >= chunk) return;
  const int logical = xcd * chunk + idx;
  if (logical >= L) return;
  const int mt = logical / nN;
  const int nt = logical - mt * nN;
  GemmArgs g = a;
  g.sorted_ids = s_sorted;
  g.expert_off = s_off;
  g.tile_expert = s_tile;
  if constexpr (ONE_PAGE) g.pt = s_pt;
  stream_tile<T, BN, DEPTH, true, NSTEPS, ONE_PAGE, true, 1>(g, ksplit, mt, nt, s_tile[mt], lds, pt_lds);
}

// ---------------------------------------------------------------- launchers

namespace {

template <typename T, int BN, int DEPTH, bool GATED, bool ONE_PAGE, int NT, int MR>
void launch_stream_steps(int steps, dim3 gd, dim3 bd, size_t lds, hipStream_t st, const GemmArgs& g, int ksplit) {
  switch (steps) {
#define RIMURU_STREAM_CASE(n) \
    case n: hipLaunchKernelGGL((k_paged_gemm_stream<T, BN, DEPTH, GATED, n, ONE_PAGE, NT, MR>), gd, bd, lds, st, g, ksplit); break;
    RIMURU_STREAM_CASE(2)
    RIMURU_STREAM_CASE(3)
    RIMURU_STREAM_CASE(4)
    RIMURU_STREAM_CASE(6)
    RIMURU_STREAM_CASE(8)
    RIMURU_STREAM_CASE(12)
    RIMURU_STREAM_CASE(16)
#undef RIMURU_STREAM_CASE
    // other step counts: runtime loop, one step less in flight (register budget)
    default: hipLaunchKernelGGL((k_paged_gemm_stream<T, BN, 2, GATED, 0, ONE_PAGE, NT, MR>), gd, bd, lds, st, g, ksplit);
  }
}

template <typename T, int BN, int DEPTH, bool GATED, int MR = 1>
hipError_t launch_stream(const GemmArgs& g, uint64_t tiles_max, hipStream_t st) {
  const int ksteps = g.K / kStreamK;
  const int max_split = GATED ? kStreamUpWaves : kStreamDnWaves;
  const int ksplit = (ksteps % 4 == 0 && max_split >= 4) ? 4 : (ksteps % 2 == 0 && max_split >= 2) ? 2 : 1;
  if (g.N % BN != 0 || g.K % kStreamK != 0) return hipErrorInvalidValue;
  uint64_t blocks = tiles_max * static_cast<uint64_t>(g.N / BN);
  uint64_t grid = (blocks + 7) / 8 * 8;
  if (grid == 0) return hipSuccess;
  const dim3 gd(static_cast<uint32_t>(grid)), bd(ksplit * 64);
  // at most kStreamNtRows routed rows per expert on average: most experts
  // are one row tile, read once, so the weights stream past the caches;
  // above that the choice is made per expert (non-temporal for experts whose
  // rows are one tile, plain loads where several row tiles share weights)
  const bool all_nt = static_cast<int64_t>(g.TK) <= static_cast<int64_t>(kStreamNtRows) * g.E;
  const size_t pt_bytes = g.P == 1 ? 0 : static_cast<size_t>(GATED ? 2 : 1) * g.P * sizeof(int32_t);
  if (g.P == 1) {
    if (all_nt) launch_stream_steps<T, BN, DEPTH, GATED, true, 1, MR>(ksteps / ksplit, gd, bd, 0, st, g, ksplit);
    else launch_stream_steps<T, BN, DEPTH, GATED, true, RIMURU_STREAM_NT_MIXED, MR>(ksteps / ksplit, gd, bd, 0, st, g, ksplit);
  } else {
    if (all_nt) launch_stream_steps<T, BN, DEPTH, GATED, false, 1, MR>(ksteps / ksplit, gd, bd, pt_bytes, st, g, ksplit);
    else launch_stream_steps<T, BN, DEPTH, GATED, false, RIMURU_STREAM_NT_MIXED, MR>(ksteps / ksplit, gd, bd, pt_bytes, st, g, ksplit);
  }
  return hipGetLastError();
}

template <typename T, int BN, int DEPTH>
hipError_t launch_routed(const GemmArgs& g, uint64_t tiles_max, const TinyRoute& rt, hipStream_t st) {
  const uint64_t blocks = tiles_max * static_cast<uint64_t>(g.N / BN);
  const uint64_t grid = (blocks + 7) / 8 * 8;
  const dim3 gd(static_cast<uint32_t>(grid)), bd(kStreamMaxWaves * 64);
  const size_t pt_bytes = g.P == 1 ? 0 : static_cast<size_t>(2) * g.P * sizeof(int32_t);
  const int ksplit = kStreamMaxWaves;
  const bool unrolled = g.K / kStreamK / ksplit == 16;
  if (g.P == 1) {
    if (unrolled) hipLaunchKernelGGL((k_paged_gemm_stream_routed<T, BN, DEPTH, 16, true>), gd, bd, 0, st, g, ksplit, rt);
    else hipLaunchKernelGGL((k_paged_gemm_stream_routed<T, BN, 2, 0, true>), gd, bd, 0, st, g, ksplit, rt);
  } else {
    if (unrolled) hipLaunchKernelGGL((k_paged_gemm_stream_routed<T, BN, DEPTH, 16, false>), gd, bd, pt_bytes, st, g, ksplit, rt);
    else hipLaunchKernelGGL((k_paged_gemm_stream_routed<T, BN, 2, 0, false>), gd, bd, pt_bytes, st, g, ksplit, rt);
  }
  return hipGetLastError();
}

}  // namespace

// The routed stream needs all four wavefronts for the routing (a token each,
// one thread an expert), so it takes shapes whose K splits four ways; the
// column tile is chosen as for the 16-row stream. Every slot's weight loads
// are non-temporal (a tiny batch reads each expert's weights once).
bool streamed_routed_fits(int dtype_bytes, int T, int k, int E, int K, uint64_t tiles_max) {
  // at most 4 tokens: an expert gets at most 4 rows, one 16-row tile, so
  // the padded lists hold at most 16 rows a touched expert (<= 512)
  const int TK = T * k;
  return dtype_bytes == 2 && T >= 1 && T <= kRoutedMaxT && TK <= kRoutedMaxTK && E <= kRoutedMaxE &&
         K % (kStreamK * kStreamMaxWaves) == 0 && kStreamUpWaves >= kStreamMaxWaves &&
         tiles_max >= static_cast<uint64_t>(std::min(TK, E));
}

template <typename T>
hipError_t launch_streamed_routed(const GemmArgs& g, uint64_t tiles_max, const TinyRoute& rt, hipStream_t st) {
  if constexpr (sizeof(T) != 2) {
    return hipErrorNotSupported;
  } else {
    if (g.TK != rt.T * rt.k || !streamed_routed_fits(2, rt.T, rt.k, g.E, g.K, tiles_max)) return hipErrorNotSupported;
    const int64_t touched = std::min<int64_t>(g.E, g.TK);
    auto enough = [&](int bn, int floor_bn) {
      return g.N % bn == 0 && (bn <= floor_bn || touched * (g.N / bn) >= kStreamNarrow.min_groups);
    };
    if (enough(kStreamUpBN, kStreamNarrow.up_bn)) return launch_routed<T, kStreamUpBN, kStreamUpDepth>(g, tiles_max, rt, st);
    if (enough(64, kStreamNarrow.up_bn)) return launch_routed<T, 64, 3>(g, tiles_max, rt, st);
    if (g.N % 32 == 0) return launch_routed<T, 32, 3>(g, tiles_max, rt, st);
    return hipErrorNotSupported;
  }
}

template hipError_t launch_streamed_routed<uint16_t>(const GemmArgs&, uint64_t, const TinyRoute&, hipStream_t);
template hipError_t launch_streamed_routed<float>(const GemmArgs&, uint64_t, const TinyRoute&, hipStream_t);

template <typename T, bool GATED>
hipError_t launch_streamed(int bm, const GemmArgs& g, uint64_t tiles_max, hipStream_t st) {
  if (bm == 32) {
    // 32-row tiles (bf16): two 16-row blocks share every weight fragment, so
    // an expert with up to 32 routed rows reads its weights once; narrower
    // column tiles keep the accumulators of both blocks within the register
    // budget of two workgroups per CU
    if constexpr (sizeof(T) == 4) {
      return hipErrorInvalidValue;
    } else if constexpr (GATED) {
      // projections over several pages: the per-segment page lookups need
      // registers the 128-column tile's accumulators leave no room for (it
      // spills), so those take 64 columns
      if (g.P == 1 && g.N % kStream32Up.bn == 0)
        return launch_stream<T, kStream32Up.bn, kStream32Up.depth, true, 2>(g, tiles_max, st);
      return launch_stream<T, 64, 3, true, 2>(g, tiles_max, st);
    } else {
      if (g.N % kStream32Dn.bn == 0) return launch_stream<T, kStream32Dn.bn, kStream32Dn.depth, false, 2>(g, tiles_max, st);
      return launch_stream<T, 64, 3, false, 2>(g, tiles_max, st);
    }
  }
  if (bm != 16) return hipErrorInvalidValue;
  if constexpr (sizeof(T) == 4) {
    return launch_stream<T, 64, 3, GATED>(g, tiles_max, st);
  } else {
    // Widest column tile that still yields enough workgroups to keep every
    // CU streaming when only a few experts are touched.
    const int64_t touched = std::min<int64_t>(g.E, g.TK);
    auto enough = [&](int bn, int floor_bn) {
      return g.N % bn == 0 && (bn <= floor_bn || touched * (g.N / bn) >= kStreamNarrow.min_groups);
    };
    if constexpr (GATED) {
      if (enough(kStreamUpBN, kStreamNarrow.up_bn)) return launch_stream<T, kStreamUpBN, kStreamUpDepth, true>(g, tiles_max, st);
      if (enough(64, kStreamNarrow.up_bn)) return launch_stream<T, 64, 3, true>(g, tiles_max, st);
      return launch_stream<T, 32, 3, true>(g, tiles_max, st);
    } else {
      // projections over several pages with more than 8 steps a wavefront,
      // or a step count the K loop is not unrolled for (the K split as
      // launch_stream takes it): the page lookups need registers the
      // 256-column tile leaves no room for (it spills), the 128-column one
      // does not
      const int ksteps = g.K / kStreamK;
      const int ksplit = (ksteps % 4 == 0 && kStreamDnWaves >= 4) ? 4 : (ksteps % 2 == 0 && kStreamDnWaves >= 2) ? 2 : 1;
      const int wsteps = ksteps / ksplit;
      const bool unrolled = wsteps == 2 || wsteps == 3 || wsteps == 4 || wsteps == 6 || wsteps == 8;
      const bool long_k = g.P > 1 && !unrolled;
      if (!long_k && enough(kStreamDnBN, kStreamNarrow.dn_bn))
        return launch_stream<T, kStreamDnBN, kStreamDnDepth, false>(g, tiles_max, st);
      if (enough(128, kStreamNarrow.dn_bn)) return launch_stream<T, 128, 3, false>(g, tiles_max, st);
      return launch_stream<T, 64, 3, false>(g, tiles_max, st);
    }
  }
}

template hipError_t launch_streamed<uint16_t, true>(int, const GemmArgs&, uint64_t, hipStream_t);
template hipError_t launch_streamed<uint16_t, false>(int, const GemmArgs&, uint64_t, hipStream_t);
template hipError_t launch_streamed<float, true>(int, const GemmArgs&, uint64_t, hipStream_t);
template hipError_t launch_streamed<float, false>(int, const GemmArgs&, uint64_t, hipStream_t);

}  // namespace rimuru
