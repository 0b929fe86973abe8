// Stages 4 and 5 of the fused MoE layer for many routed rows per expert
// (prefill): a grouped GEMM over the sorted rows whose weight tiles are read
// page by page through the expert view's page table (Rimuru paper summary,
// abstract and Figure 11, "Discrete FusedMoE"; Table 1 for the projections).
//   gemm-up    h = SiLU(x w1) * (x w3)
//   gemm-down  y_slot[t*k+j] = w[t,j] * (h w2)
#include "moe_common.h"

namespace rimuru {

// One workgroup computes a BM x BN tile of C (two tiles, w1 and w3, when
// GATED). WM x WN wavefronts each own a (BM/WM) x (BN/WN) block of 32x32
// MFMA tiles. K advances BK at a time through a double-buffered LDS stage:
// A rows are stored K-contiguous; weight rows are stored as they sit in the
// pool (N-contiguous, row pitch padded against bank conflicts) and the MFMA
// B operand is gathered by LDS transpose reads. PT_LDS stages the expert's
// page-table rows in LDS (dynamic shared memory) so a page lookup never waits
// on a global load.
template <typename T, int BM, int BN, int BK, int WM, int WN, int GM, bool GATED, bool PT_LDS, int NBUF>
__global__ __launch_bounds__(WM* WN * 64) void k_paged_gemm(GemmArgs a) {
  typedef Elt<T> X;
  constexpr int NT = WM * WN * 64;
  constexpr int VEC = X::VEC;
  constexpr int NB = GATED ? 2 : 1;
  constexpr int BKP = BK + VEC;                  // A row pitch: 16 bytes of padding
  constexpr int BNP = BN + X::B_PAD;             // B row pitch
  constexpr int WTM = BM / WM, WTN = BN / WN;
  constexpr int TM = WTM / 32, TN = WTN / 32;
  constexpr int KI = X::KI32;
  constexpr int FE = KI / 2;                     // operand values per lane per MFMA
  constexpr int A_SEGS = BM * BK / VEC;
  constexpr int A_LOADS = (A_SEGS + NT - 1) / NT;
  constexpr int RK = BK * BN / (VEC * NT);       // weight rows per thread per matrix
  constexpr int CG = BN / VEC;                   // 16-byte column groups per weight row
  static_assert(RK >= 1 && RK * VEC * NT == BK * BN, "weight tile must split evenly");
  static_assert(BK % RK == 0 && WTM % 32 == 0 && WTN % 32 == 0 && BK % KI == 0, "tile shape");

  // NBUF == 2: double-buffered stages, one barrier per step. NBUF == 1: one
  // buffer (half the LDS, so larger stages fit); the next stage waits in
  // registers during the MFMAs and is written between two barriers.
  static_assert(NBUF == 1 || NBUF == 2, "one or two LDS stages");
  __shared__ __attribute__((aligned(16))) T As[NBUF][BM * BKP];
  __shared__ __attribute__((aligned(16))) T Bs[NBUF][NB][BK * BNP];
  extern __shared__ int32_t pt_lds[];

  // ---- tile assignment: each XCD (dispatch round-robins over 8) takes one
  // contiguous chunk of the live tiles, walked GM row-tiles at a time.
  const int nN = a.N / BN;
  const int n_tiles = a.expert_off[a.E] / BM;
  const int L = n_tiles * nN;
  const int chunk = (L + 7) >> 3;
  const int xcd = blockIdx.x & 7, idx = blockIdx.x >> 3;
  if (idx >= chunk) return;
  const int logical = xcd * chunk + idx;
  if (logical >= L) return;
  const int gsz = GM * nN;
  const int g = logical / gsz;
  const int rr = logical - g * gsz;
  const int m_first = g * GM;
  const int gm = min(GM, n_tiles - m_first);
  const int mt = m_first + rr % gm;
  const int nt = rr / gm;
  const int e = a.tile_expert[mt];
  const int r0 = mt * BM;
  const int n0 = nt * BN;

  const int tid = threadIdx.x;
  const int lane = tid & 63, wv = tid >> 6;
  const int wm = wv / WN, wn = wv % WN;

  // ---- page-table rows of this expert
  const int32_t* pt_row[NB];
  if constexpr (PT_LDS) {
    for (int i = tid; i < NB * a.P; i += NT) {
      const int b = i / a.P, q = i - b * a.P;
      pt_lds[i] = a.pt[static_cast<int64_t>(e * 3 + (GATED ? b : 2)) * a.P + q];
    }
#pragma unroll
    for (int b = 0; b < NB; ++b) pt_row[b] = pt_lds + b * a.P;
  } else {
#pragma unroll
    for (int b = 0; b < NB; ++b) pt_row[b] = a.pt + static_cast<int64_t>(e * 3 + (GATED ? b : 2)) * a.P;
  }

  // ---- A row sources for this tile (padding rows read row 0 and are zeroed)
  const T* a_src[A_LOADS];
  bool a_ok[A_LOADS];
  int a_row[A_LOADS], a_kv[A_LOADS];
#pragma unroll
  for (int i = 0; i < A_LOADS; ++i) {
    const int sidx = tid + i * NT;
    a_row[i] = sidx / (BK / VEC);
    a_kv[i] = sidx % (BK / VEC);
    a_ok[i] = sidx < A_SEGS;
    int64_t src_row = 0;
    if (a_ok[i]) {
      const int r = r0 + a_row[i];
      if (a.kdiv > 0) {
        const int slot = a.sorted_ids[r];
        a_ok[i] = slot < a.TK;
        src_row = a_ok[i] ? slot / a.kdiv : 0;
      } else {
        src_row = r;
      }
    }
    a_src[i] = reinterpret_cast<const T*>(a.A) + src_row * a.lda + a_kv[i] * VEC;
  }
  const int cb = tid % CG, rb = tid / CG;
  const uint32_t col_bytes = static_cast<uint32_t>(n0 + cb * VEC) * X::ES;
  const uint32_t row_bytes = static_cast<uint32_t>(a.N) * X::ES;

  u32x4 a_reg[A_LOADS];
  u32x4 b_reg[NB][RK];

  auto load_stage = [&](int kt) {
#pragma unroll
    for (int i = 0; i < A_LOADS; ++i) a_reg[i] = *reinterpret_cast<const u32x4*>(a_src[i] + kt * BK);
#pragma unroll
    for (int b = 0; b < NB; ++b) {
#pragma unroll
      for (int j = 0; j < RK; ++j) {
        const uint32_t f = static_cast<uint32_t>(kt * BK + rb * RK + j) * row_bytes + col_bytes;
        const uint32_t q = page_index(f, a.pd);
        const uint8_t* p = a.pool + static_cast<uint64_t>(pt_row[b][q]) * a.pd.page + (f - q * a.pd.page);
        b_reg[b][j] = *reinterpret_cast<const u32x4*>(p);
      }
    }
  };

  auto store_stage = [&](int buf) {
#pragma unroll
    for (int i = 0; i < A_LOADS; ++i) {
      if (tid + i * NT < A_SEGS) {
        const u32x4 v = a_ok[i] ? a_reg[i] : u32x4{0u, 0u, 0u, 0u};
        *reinterpret_cast<u32x4*>(&As[buf][a_row[i] * BKP + a_kv[i] * VEC]) = v;
      }
    }
    // weight rows as they are: 16-byte segments, row pitch BNP
#pragma unroll
    for (int b = 0; b < NB; ++b)
#pragma unroll
      for (int j = 0; j < RK; ++j)
        *reinterpret_cast<u32x4*>(&Bs[buf][b][(rb * RK + j) * BNP + cb * VEC]) = b_reg[b][j];
  };

  f32x16 acc[NB][TM][TN];
#pragma unroll
  for (int b = 0; b < NB; ++b)
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
      for (int j = 0; j < TN; ++j)
#pragma unroll
        for (int r = 0; r < 16; ++r) acc[b][i][j][r] = 0.0f;

  const int nk = a.K / BK;
  const int fi = lane & 31, fq = lane >> 5;  // operand row/column and K half of this lane

  if constexpr (PT_LDS) __syncthreads();
  load_stage(0);
  store_stage(0);
  __syncthreads();
  for (int kt = 0; kt < nk; ++kt) {
    const int buf = (NBUF == 2) ? (kt & 1) : 0;
    if (kt + 1 < nk) load_stage(kt + 1);
#pragma unroll
    for (int kk = 0; kk < BK / KI; ++kk) {
      typename X::Frag af[TM], bfr[NB][TN];
#pragma unroll
      for (int i = 0; i < TM; ++i)
        af[i] = X::frag(&As[buf][(wm * WTM + i * 32 + fi) * BKP + kk * KI + fq * FE]);
#pragma unroll
      for (int b = 0; b < NB; ++b)
#pragma unroll
        for (int j = 0; j < TN; ++j)
          bfr[b][j] = X::bfrag32(Bs[buf][b], BNP, kk * KI, wn * WTN + j * 32, lane);
#pragma unroll
      for (int b = 0; b < NB; ++b)
#pragma unroll
        for (int i = 0; i < TM; ++i)
#pragma unroll
          for (int j = 0; j < TN; ++j) acc[b][i][j] = X::mma32(af[i], bfr[b][j], acc[b][i][j]);
    }
    if constexpr (NBUF == 2) {
      if (kt + 1 < nk) store_stage(buf ^ 1);
      __syncthreads();
    } else if (kt + 1 < nk) {
      __syncthreads();
      store_stage(0);
      __syncthreads();
    }
  }

  // ---- epilogue: acc[r] of a 32x32 tile is row 8*(r/4) + 4*(lane/32) + r%4, column lane%32
  T* C = reinterpret_cast<T*>(a.C);
#pragma unroll
  for (int i = 0; i < TM; ++i) {
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int row = r0 + wm * WTM + i * 32 + 8 * (r >> 2) + 4 * fq + (r & 3);
      if constexpr (GATED) {
#pragma unroll
        for (int j = 0; j < TN; ++j) {
          const int col = n0 + wn * WTN + j * 32 + fi;
          X::put(&C[static_cast<int64_t>(row) * a.ldc + col], silu(acc[0][i][j][r]) * acc[1][i][j][r]);
        }
      } else {
        const int slot = a.sorted_ids[row];
        if (slot < a.TK) {
          const float wt = a.topk_w[slot];
#pragma unroll
          for (int j = 0; j < TN; ++j) {
            const int col = n0 + wn * WTN + j * 32 + fi;
            X::put(&C[static_cast<int64_t>(slot) * a.ldc + col], wt * acc[0][i][j][r]);
          }
        }
      }
    }
  }
}

// ---------------------------------------------------------------- launchers

namespace {

constexpr int kTilePtMax = 4096;  // page-table entries a tiled workgroup stages in LDS

// bf16 tile shapes of the tiled plans (compile-time overridable for tuning
// sweeps): column tile, K step, wavefront grid, LDS stages. UP is the gated
// gate/up GEMM, DN the down GEMM; T128 the 128-row plan, T64 the 64-row one.
#ifndef RIMURU_T128_UP
#define RIMURU_T128_UP 128, 64, 2, 4, 1
#endif
#ifndef RIMURU_T128_DN
#define RIMURU_T128_DN 256, 64, 2, 4, 1
#endif
#ifndef RIMURU_T64_UP
#define RIMURU_T64_UP 128, 64, 2, 4, 1
#endif
#ifndef RIMURU_T64_DN
#define RIMURU_T64_DN 256, 64, 2, 2, 1
#endif
struct TileShape { int bn, bk, wm, wn, nbuf; };
constexpr TileShape kT128Up{RIMURU_T128_UP}, kT128Dn{RIMURU_T128_DN};
constexpr TileShape kT64Up{RIMURU_T64_UP}, kT64Dn{RIMURU_T64_DN};

template <typename T, int BM, int BN, int BK, int WM, int WN, int GM, bool GATED, int NBUF = 2>
hipError_t launch_gemm(const GemmArgs& g, uint64_t tiles_max, hipStream_t st) {
  if (g.N % BN != 0 || g.K % BK != 0) return hipErrorInvalidValue;  // tiles must cover C exactly
  uint64_t blocks = tiles_max * static_cast<uint64_t>(g.N / BN);
  uint64_t grid = (blocks + 7) / 8 * 8;
  if (grid == 0) return hipSuccess;
  const int nb = GATED ? 2 : 1;
  if (nb * g.P <= kTilePtMax) {
    hipLaunchKernelGGL((k_paged_gemm<T, BM, BN, BK, WM, WN, GM, GATED, true, NBUF>), dim3(static_cast<uint32_t>(grid)),
                       dim3(WM * WN * 64), static_cast<size_t>(nb) * g.P * sizeof(int32_t), st, g);
  } else {
    hipLaunchKernelGGL((k_paged_gemm<T, BM, BN, BK, WM, WN, GM, GATED, false, NBUF>), dim3(static_cast<uint32_t>(grid)),
                       dim3(WM * WN * 64), 0, st, g);
  }
  return hipGetLastError();
}

}  // namespace

// Column tiles are 128 wide when N allows it, else 64 (N is a multiple of 64
// by validation); fp32 tiles take a shorter K step, keeping their LDS
// footprint near the bf16 tiles'.
template <typename T, bool GATED>
hipError_t launch_tiled(int bm, const GemmArgs& g, uint64_t tiles_max, hipStream_t st) {
  constexpr bool kF32 = sizeof(T) == 4;
  constexpr int BK_TILE = kF32 ? 16 : 64;
  const bool wide = g.N % 128 == 0;
  if (bm == 64) {
    if constexpr (!kF32) {
      constexpr TileShape t = GATED ? kT64Up : kT64Dn;
      if (g.N % t.bn == 0) return launch_gemm<T, 64, t.bn, t.bk, t.wm, t.wn, 4, GATED, t.nbuf>(g, tiles_max, st);
    }
    return wide ? launch_gemm<T, 64, 128, BK_TILE, 2, 2, 4, GATED>(g, tiles_max, st)
                : launch_gemm<T, 64, 64, BK_TILE, 2, 2, 4, GATED>(g, tiles_max, st);
  }
  if (bm != 128) return hipErrorInvalidValue;
  if constexpr (!kF32) {
    constexpr TileShape t = GATED ? kT128Up : kT128Dn;
    if (g.N % t.bn == 0) return launch_gemm<T, 128, t.bn, t.bk, t.wm, t.wn, 8, GATED, t.nbuf>(g, tiles_max, st);
  }
  return wide ? launch_gemm<T, 128, 128, BK_TILE, 2, 2, 8, GATED>(g, tiles_max, st)
              : launch_gemm<T, 128, 64, BK_TILE, 2, 2, 8, GATED>(g, tiles_max, st);
}

template hipError_t launch_tiled<uint16_t, true>(int, const GemmArgs&, uint64_t, hipStream_t);
template hipError_t launch_tiled<uint16_t, false>(int, const GemmArgs&, uint64_t, hipStream_t);
template hipError_t launch_tiled<float, true>(int, const GemmArgs&, uint64_t, hipStream_t);
template hipError_t launch_tiled<float, false>(int, const GemmArgs&, uint64_t, hipStream_t);

}  // namespace rimuru
