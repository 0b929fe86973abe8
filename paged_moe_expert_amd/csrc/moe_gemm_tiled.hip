// Stages 4 and 5 of the fused MoE layer for many routed rows per expert
// (prefill): a grouped GEMM over the sorted rows whose weight tiles are read
// page by page through the expert view's page table (Rimuru paper summary,
// abstract and Figure 11, "Discrete FusedMoE"; Table 1 for the projections).
//   gemm-up    h = SiLU(x w1) * (x w3)
//   gemm-down  y_slot[t*k+j] = w[t,j] * (h w2)
#include <type_traits>

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

  // Weights of an expert whose routed rows fit one row tile are read by no
  // other tile of the launch at these columns: they stream past the caches
  // (non-temporal loads, bf16). Several row tiles of one expert share them
  // in L2 instead (plain loads).
  const bool nt_tile = sizeof(T) == 2 && a.expert_off[e + 1] - a.expert_off[e] == BM;
  auto run = [&](auto NTC) {
    constexpr bool NTW = decltype(NTC)::value;
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
          if constexpr (NTW)
            b_reg[b][j] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
          else
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
  };
  if (nt_tile) run(std::true_type{});
  else run(std::false_type{});
}

// ---------------------------------------------------------------- bf16, many rows: asynchronous pipeline

constexpr int kMtBM = 128;     // tile rows
constexpr int kMtSN = 256;     // columns of one weight sub-tile (512-byte rows)
#ifndef RIMURU_MT_GM
#define RIMURU_MT_GM 1
#endif
// row tiles walked per column tile; 1 = the column tiles of one row tile run
// back to back, sharing its A rows in L2 (measured 2% faster than 8 or 32 on
// the fragmented-prefill layer)
constexpr int kMtGM = RIMURU_MT_GM;

// One workgroup of NW wavefronts computes a 128-row tile against two
// 256-column weight sub-tiles: w1 and w3 at the same columns when GATED, else
// two adjacent column ranges of w2. Wavefront (wm, wn) owns columns
// 64wn .. 64wn+63 of each sub-tile for 128/(NW/4) rows: with NW = 4 (one per
// SIMD) 4 x 2 x 2 tiles of 32x32 (256 accumulators), with NW = 8 (two per
// SIMD, the default: one wavefront's MFMAs cover the other's copy and LDS
// read issue) 2 x 2 x 2 tiles (128 accumulators, 8 MFMAs per 16-deep K step
// against 2 A and 4 B operand reads).
//
// Operands reach LDS by asynchronous global->LDS copies (16 bytes per lane;
// each wavefront instruction fills 1 KB of LDS), STAGES stages of BK rows
// deep, with no register staging. A rows are stored row-major with their
// 16-byte K octets XOR-swizzled by row, copied as whole row pieces; weight
// rows are stored as they sit in the pool (N-contiguous) in padded two-row
// chunks; both layouts keep the operand reads free of bank conflicts (the
// weight operand is gathered by transposed LDS reads).
//
// Pipeline: the operands of K step s+1 are read from LDS while the MFMAs of
// step s run. At the last K step of a stage the workgroup waits for the next
// stage's copies, passes one barrier, refills the stage it has just finished
// reading with the stage STAGES ahead, and reads the next stage's first
// operands between the last MFMAs of the current stage.
//
// Measured on the fragmented-prefill layer (8192 tokens, 128 experts), with
// NW = 4: the wait for copies stays near 100 cycles a stage and the MFMAs
// alone take ~1180 cycles of the ~2400 a stage costs; the rest is instruction
// issue (copy, address and LDS-read instructions between MFMAs) at one
// wavefront per SIMD. NW = 8 brings a stage to ~2000-2100 cycles.
template <bool GATED, int BK, int STAGES, int NW>
__global__ __launch_bounds__(NW * 64, 1) void k_paged_gemm_mt(GemmArgs a) {
  constexpr int KS = BK / 16;                     // MFMA K steps per stage
  constexpr int A_CHUNKS = (kMtBM / 32) * KS;     // 1 KB chunks (row block, K step)
  constexpr int A_BYTES = A_CHUNKS * 1024;
  constexpr int SUB_BYTES = BK * kMtSN * 2;       // one weight sub-tile's data
  constexpr int SUB_CHUNKS = SUB_BYTES / 1024;    // 2 rows of 512 bytes each
  constexpr int CHUNK_PITCH = 1024 + 64;          // LDS bytes per chunk (padded)
  constexpr int SUB_LDS = SUB_CHUNKS * CHUNK_PITCH;
  constexpr int STAGE_BYTES = A_BYTES + 2 * SUB_LDS;
  constexpr int NT = NW * 64;
  constexpr int A_DMA = A_CHUNKS / NW;            // per wavefront per stage
  constexpr int B_DMA = 2 * SUB_CHUNKS / NW;
  constexpr int DMA = A_DMA + B_DMA;
  constexpr int NBM = GATED ? 2 : 1;              // weight matrices read
  // wavefront grid: WGM row groups x 4 column groups; TM row blocks of 32 each
  constexpr int WGM = NW / 4;
  constexpr int TM = 4 / WGM;
  constexpr int NMMA = TM * 4;                    // MFMAs per K step
  constexpr int NREAD = TM + 8;                   // operand reads per K step
  static_assert((NW == 4 || NW == 8) && A_CHUNKS % NW == 0 && (2 * SUB_CHUNKS) % NW == 0, "wavefronts");
  static_assert(KS == 2 && BK % 8 == 0, "the K-step schedule below is laid out for two K steps a stage");
  static_assert(STAGES >= 2 && (STAGES - 1) * DMA < 64, "copies in flight");

  __shared__ __attribute__((aligned(1024))) uint8_t smem[STAGES * STAGE_BYTES];
  __shared__ int32_t row_slot[kMtBM];
  __shared__ float row_w[kMtBM];
  extern __shared__ uint64_t page_base[];         // [NBM][P]: pool address of each page

  // ---- tile: XCD chunk, then kMtGM row tiles per column tile
  const int BNW = 2 * kMtSN / NBM;                // output columns per tile
  const int nN = a.N / BNW;
  const int n_tiles = a.expert_off[a.E] / kMtBM;
  const int L = n_tiles * nN;
  const int chunk = (L + 7) >> 3;
  const int xcd = blockIdx.x & 7, idx = blockIdx.x >> 3;
  if (idx >= chunk) return;
  const int logical = xcd * chunk + idx;
  if (logical >= L) return;
  const int gsz = kMtGM * nN;
  const int g = logical / gsz;
  const int rr = logical - g * gsz;
  const int gm = min(kMtGM, n_tiles - g * kMtGM);
  const int mt = g * kMtGM + rr % gm;
  const int nt = rr / gm;
  const int e = a.tile_expert[mt];
  const int r0 = mt * kMtBM;
  const int n0 = nt * BNW;

  const int tid = threadIdx.x, lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = w >> 2, wn = w & 3;              // row group, column group
  typedef __attribute__((address_space(3))) uint8_t lds_u8;
  const uint32_t smem_lds = __builtin_amdgcn_readfirstlane(
      static_cast<uint32_t>(reinterpret_cast<uintptr_t>((lds_u8*)smem)));
  const uint32_t page = a.pd.page;
  const int nk = a.K / BK;

  // ---- page addresses and the tile's row -> slot map
  for (int i = tid; i < NBM * a.P; i += NT) {
    const int b = i / a.P, q = i - b * a.P;
    const int32_t pg = a.pt[static_cast<int64_t>(e * 3 + (GATED ? b : 2)) * a.P + q];
    page_base[i] = reinterpret_cast<uint64_t>(a.pool) + static_cast<uint64_t>(static_cast<uint32_t>(pg)) * page;
  }
  if (tid < kMtBM) {
    const int slot = a.sorted_ids[r0 + tid];
    row_slot[tid] = slot;
    row_w[tid] = (!GATED && slot < a.TK) ? a.topk_w[slot] : 0.0f;
  }
  __syncthreads();

  // ---- per-lane copy sources
  // A: the stage's 128 rows x BK are stored row-major (2*BK bytes a row),
  // their 16-byte K octets XOR-swizzled by row (octet o of row r at slot
  // o ^ (r/4)%4) so the operand reads below are conflict-free. One copy
  // instruction fills 1024/(2*BK) whole rows: lane l fetches row
  // c*RPC + l/OPR, slot l%OPR of chunk c (contiguous row pieces: each copy
  // touches few cache lines).
  constexpr int OPR = BK / 8;                     // K octets per row
  constexpr int RPC = 64 / OPR;                   // rows per 1 KB chunk
  const uint8_t* asrc[A_DMA];
#pragma unroll
  for (int d = 0; d < A_DMA; ++d) {
    const int trow = (w * A_DMA + d) * RPC + lane / OPR;
    int64_t src = r0 + trow;
    if (a.kdiv > 0) {
      const int slot = row_slot[trow];
      src = slot < a.TK ? slot / a.kdiv : 0;      // padding rows read row 0
    }
    const int oct = (lane % OPR) ^ ((trow >> 2) & (OPR - 1));
    asrc[d] = a.A + (src * a.lda + 8 * oct) * 2;
  }
  // B: a weight sub-tile (BK rows of 512 bytes) is stored as BK/2 chunks of
  // two rows, chunk c holding rows 8*(c/4) + c%4 and that + 4, chunks padded
  // to 1088 bytes. The 4 consecutive rows a transposed operand read touches
  // then lie in 4 chunks whose starts differ by 64 bytes modulo 256 (distinct
  // banks), while every copy instruction still fetches two whole 512-byte row
  // pieces in lane order. Wavefront w copies chunks w*B_DMA .. +B_DMA-1 of
  // the 2 sub-tiles. Each copy tracks its page index q and
  // the offset in that page, advanced by one stage at a time (the stage
  // advance is step_q pages plus step_r bytes, step_r < page).
  uint32_t bq[B_DMA], brem[B_DMA];
  const uint32_t row_bytes = static_cast<uint32_t>(a.N) * 2;
  const uint32_t stage_step = static_cast<uint32_t>(BK) * row_bytes;
  const uint32_t step_q = __builtin_amdgcn_readfirstlane(stage_step / page);
  const uint32_t step_r = stage_step - step_q * page;
#pragma unroll
  for (int d = 0; d < B_DMA; ++d) {
    const int cb = w * B_DMA + d;
    const int b = cb / SUB_CHUNKS, c = cb % SUB_CHUNKS;
    const int r = 8 * (c >> 2) + (c & 3) + 4 * (lane >> 5);
    const int seg = lane & 31;
    const int col = GATED ? n0 + 8 * seg : n0 + b * kMtSN + 8 * seg;
    const uint32_t f = static_cast<uint32_t>(r) * row_bytes + static_cast<uint32_t>(col) * 2;
    const uint32_t q = page_index(f, a.pd);
    bq[d] = q + (GATED ? b : 0) * a.P;            // index into page_base
    brem[d] = f - q * page;
  }

  // Sources of the next stage to copy: the A rows advance by BK, each weight
  // segment by one stage. The page addresses are read from LDS one K step
  // before the copies are formed (lookup), so the copies never wait on them.
  struct Srcs { uint64_t pb[B_DMA]; uint32_t rem[B_DMA]; int st; };
  int next_st = 0;
  auto lookup_one = [&](Srcs& sr, int d) {
    sr.pb[d] = page_base[bq[d]];
    sr.rem[d] = brem[d];
  };
  auto advance_one = [&](int d) {
    uint32_t r = brem[d] + step_r;
    const bool wrap = r >= page;
    brem[d] = wrap ? r - page : r;
    bq[d] += step_q + (wrap ? 1u : 0u);
  };
  auto lookup = [&](Srcs& sr) {
    sr.st = next_st;
#pragma unroll
    for (int d = 0; d < B_DMA; ++d) lookup_one(sr, d);
  };
  auto advance = [&]() {
    ++next_st;
#pragma unroll
    for (int d = 0; d < B_DMA; ++d) advance_one(d);
  };
  auto src_of = [&](const Srcs& sr, int d) -> const void* {
    if (d < A_DMA) return asrc[d] + sr.st * BK * 2;
    return reinterpret_cast<const void*>(sr.pb[d - A_DMA] + sr.rem[d - A_DMA]);
  };
  auto copy = [&](const Srcs& sr, int st, int d) {
    const uint32_t base = smem_lds + (st % STAGES) * STAGE_BYTES;
    if (d < A_DMA) copy_to_lds16(src_of(sr, d), base + (w * A_DMA + d) * 1024);
    else {
      const int cb = w * B_DMA + d - A_DMA;
      copy_to_lds16(src_of(sr, d), base + A_BYTES + (cb / SUB_CHUNKS) * SUB_LDS + (cb % SUB_CHUNKS) * CHUNK_PITCH);
    }
  };

  // ---- per-lane operand read offsets
  const int grp = lane >> 4, sl = lane & 15;
  uint32_t boff[2];                               // B: column block jj of this wavefront
#pragma unroll
  for (int jj = 0; jj < 2; ++jj) {
    // rows 8*(grp/2) + sl/4 (+4 for the upper half): chunk 4*(grp/2) + sl/4
    const int chunk = 4 * (grp >> 1) + (sl >> 2);
    const int col = 64 * wn + 32 * jj + 16 * (grp & 1) + 4 * (sl & 3);
    boff[jj] = A_BYTES + chunk * CHUNK_PITCH + col * 2;
  }
  typedef __attribute__((address_space(3))) v4i16 lds_v4;
  struct Frags { u32x4 a[TM]; u32x4 b[2][2]; };
  // A operand of K step s, row block i: lane l reads row 32i + l%32, octet
  // 2s + l/32 (slot swizzled as stored)
  uint32_t aoff[KS];
#pragma unroll
  for (int s2 = 0; s2 < KS; ++s2) {
    const int row = lane & 31;
    const int oct = 2 * s2 + (lane >> 5);
    aoff[s2] = row * (2 * BK) + ((oct ^ ((row >> 2) & (OPR - 1))) * 16);
  }
  // operand read k (0..NREAD-1) of K step s: the wavefront's A row blocks,
  // then the lower and upper halves of the 4 B operands
  auto read_one = [&](Frags& f, int st, int s, int k) {
    const uint8_t* base = smem + (st % STAGES) * STAGE_BYTES;
    if (k < TM) {
      f.a[k] = *reinterpret_cast<const u32x4*>(base + (wm * TM + k) * 32 * (2 * BK) + aoff[s]);
    } else {
      const int b = (k - TM) >> 2, jj = ((k - TM) >> 1) & 1, half = (k - TM) & 1;
      // K step s: rows +16s = chunks +8s; the upper 4 rows: second half of each chunk
      const uint8_t* p = base + boff[jj] + b * SUB_LDS + s * 8 * CHUNK_PITCH + half * 512;
      const u32x2 v = __builtin_bit_cast(u32x2, __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4*)p));
      f.b[b][jj][2 * half] = v[0];
      f.b[b][jj][2 * half + 1] = v[1];
    }
  };
  auto read_frags = [&](Frags& f, int st, int s) {
#pragma unroll
    for (int k = 0; k < NREAD; ++k) read_one(f, st, s, k);
  };

  f32x16 acc[TM][2][2];
#pragma unroll
  for (int i = 0; i < TM; ++i)
#pragma unroll
    for (int b = 0; b < 2; ++b)
#pragma unroll
      for (int jj = 0; jj < 2; ++jj)
#pragma unroll
        for (int r = 0; r < 16; ++r) acc[i][b][jj][r] = 0.0f;
  // MFMA t (0..NMMA-1) of one K step: row block t/4, sub-tile (t/2)%2, column block t%2
  auto mma = [&](const Frags& f, int t) {
    const int i = t >> 2, b = (t >> 1) & 1, jj = t & 1;
    acc[i][b][jj] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, f.a[i]),
                                                            __builtin_bit_cast(bf16x8, f.b[b][jj]),
                                                            acc[i][b][jj], 0, 0, 0);
  };

  // prologue: STAGES stages in flight, then the first operands
  Srcs sr;
#pragma unroll
  for (int st = 0; st < STAGES; ++st)
    if (st < nk) {
      lookup(sr);
      advance();
#pragma unroll
      for (int d = 0; d < DMA; ++d) copy(sr, st, d);
    }
  if (STAGES - 1 < nk) wait_vmem<(STAGES - 1) * DMA>();
  else wait_vmem<0>();
  barrier_only();
  Frags fr[2];
  read_frags(fr[0], 0, 0);

  // Each wavefront issues everything in order, so every operand read,
  // address step and copy sits in a slot between two MFMAs (the matrix pipe
  // runs the earlier MFMA meanwhile); scheduling barriers keep that order.
  //   K step 0: the MFMAs, with the operand reads of K step 1, the refill's
  //             page-address reads (first half) and their advance (second
  //             half) spread between them.
  //   K step 1: two MFMAs, the wait for stage st+1 and the barrier, then the
  //             remaining MFMAs with the next stage's operand reads and the
  //             refill copies spread between them.
  for (int st = 0; st < nk; ++st) {
    const bool refill = st + STAGES < nk;
    const bool more = st + 1 < nk;
    if (refill) sr.st = next_st;
#pragma unroll
    for (int t = 0; t < NMMA; ++t) {
      mma(fr[0], t);
#pragma unroll
      for (int k = t * NREAD / NMMA; k < (t + 1) * NREAD / NMMA; ++k) read_one(fr[1], st, 1, k);
      if (refill) {
        constexpr int H = NMMA / 2;
        if (t < H) {
#pragma unroll
          for (int d = t * B_DMA / H; d < (t + 1) * B_DMA / H; ++d) lookup_one(sr, d);
        } else {
#pragma unroll
          for (int d = (t - H) * B_DMA / H; d < (t - H + 1) * B_DMA / H; ++d) advance_one(d);
        }
      }
      __builtin_amdgcn_sched_barrier(0);
    }
    if (refill) ++next_st;
    mma(fr[1], 0);
    mma(fr[1], 1);
    __builtin_amdgcn_sched_barrier(0);
    if (more) {
      wait_lds();
      if (st + STAGES - 1 < nk) wait_vmem<(STAGES - 2) * DMA>();
      else wait_vmem<0>();
      barrier_only();
    }
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int t = 2; t < NMMA; ++t) {
      mma(fr[1], t);
      constexpr int R = NMMA - 2;
      if (more) {
#pragma unroll
        for (int k = (t - 2) * NREAD / R; k < (t - 1) * NREAD / R; ++k) read_one(fr[0], st + 1, 0, k);
      }
      if (refill) {
#pragma unroll
        for (int d = (t - 2) * DMA / R; d < (t - 1) * DMA / R; ++d) copy(sr, st + STAGES, d);
      }
      __builtin_amdgcn_sched_barrier(0);
    }
  }

  // ---- epilogue. acc[r] of a 32x32 tile is row 8*(r/4) + 4*(lane/32) + r%4,
  // column lane%32. Results go through LDS (the stage buffers are free now)
  // as a bf16 [128][256] tile, then leave in whole 16-byte row pieces.
  // Neighbouring lanes swap one value so each lane writes two adjacent
  // columns of one row to LDS (even lane: row R, columns c and c+1; odd
  // lane: row R+1, columns c-1 and c).
  const bool odd = lane & 1;
  uint16_t* C = reinterpret_cast<uint16_t*>(a.C);
  uint32_t* tile = reinterpret_cast<uint32_t*>(smem);      // [128][128] column pairs
  constexpr int PAIRS = kMtSN / 2;
  auto stash = [&](int i, int r, int col_in_sub, float v0, float v1) {
    const float y = swap_lane_pair(odd ? v0 : v1);
    const float lo = odd ? y : v0, hi = odd ? v1 : y;
    const int trow = 32 * (wm * TM + i) + 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3) + (odd ? 1 : 0);
    const int col = col_in_sub - (odd ? 1 : 0);
    tile[trow * PAIRS + (col >> 1)] = pack_bf16x2(lo, hi);
  };
  // 16-byte pieces of the tile: 32 per row, 4096 in all
  auto drain = [&](auto&& row_dst) {
#pragma unroll 4
    for (int p = 0; p < kMtBM * kMtSN / 8 / NT; ++p) {
      const int idx = p * NT + tid;
      const int trow = idx >> 5, piece = idx & 31;
      uint16_t* dst = row_dst(trow);
      if (dst != nullptr)
        *reinterpret_cast<u32x4*>(dst + piece * 8) = *reinterpret_cast<const u32x4*>(tile + trow * PAIRS + piece * 4);
    }
  };
  // SiLU with the hardware exp2 and reciprocal
  auto silu_fast = [](float v) {
    return v * __builtin_amdgcn_rcpf(1.0f + __builtin_amdgcn_exp2f(-1.4426950408889634f * v));
  };
  __syncthreads();                                          // operand buffers are free
  if constexpr (GATED) {
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
      for (int r = 0; r < 16; r += 2)
#pragma unroll
        for (int jj = 0; jj < 2; ++jj)
          stash(i, r, 64 * wn + 32 * jj + (lane & 31),
                silu_fast(acc[i][0][jj][r]) * acc[i][1][jj][r],
                silu_fast(acc[i][0][jj][r + 1]) * acc[i][1][jj][r + 1]);
    __syncthreads();
    drain([&](int trow) { return C + static_cast<int64_t>(r0 + trow) * a.ldc + n0; });
  } else {
#pragma unroll
    for (int b = 0; b < 2; ++b) {
      if (b) __syncthreads();                               // first half drained
#pragma unroll
      for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int r = 0; r < 16; r += 2) {
          const int trow = 32 * (wm * TM + i) + 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3) + (odd ? 1 : 0);
          const float wt = row_w[trow];
#pragma unroll
          for (int jj = 0; jj < 2; ++jj) {
            // the lane's own row weight applies to both of its stored values
            const float v0 = acc[i][b][jj][r], v1 = acc[i][b][jj][r + 1];
            const float y = swap_lane_pair(odd ? v0 : v1);
            const float lo = wt * (odd ? y : v0), hi = wt * (odd ? v1 : y);
            const int col = 64 * wn + 32 * jj + (lane & 31) - (odd ? 1 : 0);
            tile[trow * PAIRS + (col >> 1)] = pack_bf16x2(lo, hi);
          }
        }
      __syncthreads();
      drain([&](int trow) -> uint16_t* {
        const int slot = row_slot[trow];
        return slot < a.TK ? C + static_cast<int64_t>(slot) * a.ldc + n0 + b * kMtSN : nullptr;
      });
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

// K rows per stage and stages of the asynchronous pipeline (compile-time
// overridable for tuning sweeps)
#ifndef RIMURU_MT
#define RIMURU_MT 32, 3, 8
#endif
#ifndef RIMURU_MT_ENABLE
#define RIMURU_MT_ENABLE 1
#endif
struct MtShape { int bk, stages, waves; };
constexpr int kMtPtMax = 2048;    // page addresses the pipelined kernel stages in LDS (16 KB)
constexpr MtShape kMt{RIMURU_MT};

// The 128-row bf16 plan's asynchronous-pipeline kernel, when the shape fits
// it; returns hipErrorNotSupported otherwise (the caller then uses the
// register-staged kernel).
template <bool GATED>
hipError_t launch_mt(const GemmArgs& g, uint64_t tiles_max, hipStream_t st) {
  const int nbm = GATED ? 2 : 1;
  const int bnw = 2 * kMtSN / nbm;
  if (!RIMURU_MT_ENABLE || g.N % bnw != 0 || g.K % kMt.bk != 0 || nbm * g.P > kMtPtMax)
    return hipErrorNotSupported;
  const uint64_t blocks = tiles_max * static_cast<uint64_t>(g.N / bnw);
  const uint64_t grid = (blocks + 7) / 8 * 8;
  if (grid == 0) return hipSuccess;
  hipLaunchKernelGGL((k_paged_gemm_mt<GATED, kMt.bk, kMt.stages, kMt.waves>), dim3(static_cast<uint32_t>(grid)),
                     dim3(kMt.waves * 64),
                     static_cast<size_t>(nbm) * g.P * sizeof(uint64_t), st, g);
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
      // The persistent GEMM on 64-row tiles takes the down projection only:
      // on the 2048-token Qwen3.5 prefill it ran the down GEMM in 140 us
      // against 155 us here, but gate/up in 290 us against 261 us here.
      if constexpr (!GATED) {
        const hipError_t ep = launch_prefill<GATED>(64, g, tiles_max, st);
        if (ep != hipErrorNotSupported) return ep;
      }
      constexpr TileShape t = GATED ? kT64Up : kT64Dn;
      if (g.N % t.bn == 0) return launch_gemm<T, 64, t.bn, t.bk, t.wm, t.wn, 4, GATED, t.nbuf>(g, tiles_max, st);
    }
    return wide ? launch_gemm<T, 64, 128, BK_TILE, 2, 2, 4, GATED>(g, tiles_max, st)
                : launch_gemm<T, 64, 64, BK_TILE, 2, 2, 4, GATED>(g, tiles_max, st);
  }
  if (bm != 128) return hipErrorInvalidValue;
  if constexpr (!kF32) {
#ifndef RIMURU_PF_DISABLE
    const hipError_t ep = launch_prefill<GATED>(128, g, tiles_max, st);
    if (ep != hipErrorNotSupported) return ep;
#endif
    const hipError_t e = launch_mt<GATED>(g, tiles_max, st);
    if (e != hipErrorNotSupported) return e;
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
