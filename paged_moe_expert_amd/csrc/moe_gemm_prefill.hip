// Stages 4 and 5 of the fused MoE layer for many routed rows per expert
// (prefill, bf16): a persistent grouped GEMM whose weight tiles are read page
// by page through the expert view's page table (Rimuru paper summary,
// abstract and Figure 11, "Discrete FusedMoE"; Table 1 for the projections).
//   gemm-up    h = SiLU(x w1) * (x w3)
//   gemm-down  y_slot[t*k+j] = w[t,j] * (h w2)
//
// One workgroup per CU walks a list of 128-row tiles (the sorted rows of one
// expert) against 512 weight columns (w1 and w3 at the same 256 columns, or
// 512 columns of w2). Operands reach LDS by asynchronous global->LDS copies,
// three stages of 32 K rows in a ring that runs on across tile boundaries:
// while a tile's last stages are multiplied, the first stages of the
// workgroup's next tile are already being copied, and its page addresses and
// row map were staged in LDS during the current tile. The stage loop has no
// branch: the compiler then counts the LDS reads in flight exactly and never
// waits for more than the operands the next MFMA needs.
#include <algorithm>
#include <type_traits>

#include "moe_common.h"

namespace rimuru {

constexpr int kPfSN = 256;        // columns of one weight sub-tile (512-byte rows)
constexpr int kPfBK = 32;         // K rows per stage
constexpr int kPfStages = 3;      // stages in the LDS ring
constexpr int kPfCtxPages = 1024; // page addresses a tile context holds
#ifndef RIMURU_PF_PRE
#define RIMURU_PF_PRE 2
#endif
constexpr int kPfPre = RIMURU_PF_PRE;  // second-K-step MFMAs issued before a stage's barrier

template <int NW, int BM>
struct PfShape {
  static constexpr int KS = kPfBK / 16;                  // MFMA K steps per stage
  static constexpr int A_CHUNKS = (BM / 32) * KS;        // 1 KB chunks of A per stage
  static constexpr int A_BYTES = A_CHUNKS * 1024;
  static constexpr int SUB_CHUNKS = kPfBK * kPfSN * 2 / 1024;  // 2-row chunks of one sub-tile
  static constexpr int CHUNK_PITCH = 1024 + 64;          // padded: 4 rows of a transpose read in 4 bank phases
  static constexpr int SUB_LDS = SUB_CHUNKS * CHUNK_PITCH;
  static constexpr int STAGE_BYTES = A_BYTES + 2 * SUB_LDS;
  static constexpr int NT = NW * 64;
  static constexpr int A_DMA = A_CHUNKS / NW;            // copies per wavefront per stage
  static constexpr int B_DMA = 2 * SUB_CHUNKS / NW;
  static constexpr int DMA = A_DMA + B_DMA;
  static constexpr int WGM = NW / 4;                     // wavefront row groups (x 4 column groups)
  static constexpr int TM = BM / 32 / WGM;               // 32-row blocks per wavefront
  static constexpr int NMMA = TM * 4;                    // MFMAs per K step
  static constexpr int NREAD = TM + 8;                   // operand reads per K step
  static constexpr int OPR = kPfBK / 8;                  // 16-byte K octets per A row
  static constexpr int RPC = 64 / OPR;                   // A rows per copy
  static_assert(NW == 4 || NW == 8, "one or two wavefronts per SIMD");
  static_assert((BM == 128 || BM == 64) && TM >= 1, "tile rows");
  static_assert(A_CHUNKS % NW == 0 && (2 * SUB_CHUNKS) % NW == 0 && KS == 2, "copy split");
  static_assert(2 * DMA < 64, "copies in flight");
};

// What a workgroup knows about one tile, in LDS (two: the tile being
// computed and the next one, filled while the current one runs).
template <int BM>
struct PfCtx {
  int32_t slot[BM];               // routed slot of each row (>= TK: padding)
  float w[BM];                    // routing weight of each row (down GEMM)
  int32_t r0, n0, pad[2];         // first sorted row, first output column
  uint64_t page[kPfCtxPages];     // pool address of each page of the tile's projections
};

// Source of the gathered x rows of padding slots: zeros (static storage, never
// written), so the padding rows' MFMAs multiply zeros rather than a copy of
// a real row, and their rows of h come out zero for the down GEMM. Measured
// on the 8192-token prefill (10.7% padding rows), alternating runs on one
// box: layer 0.827-0.830 -> 0.819-0.822 ms (zero operands presumably costing
// less power on a power-limited clock). Rows longer than the array read
// row 0 instead (padding results are never used either way).
constexpr int kPfZeroRowBytes = 65536;
__device__ __attribute__((aligned(256))) uint8_t g_pf_zero_row[kPfZeroRowBytes];

template <bool GATED, int NW, int BM>
__global__ __launch_bounds__(NW * 64, 1) void k_moe_gemm_pf(GemmArgs a) {
  typedef PfShape<NW, BM> S;
  typedef PfCtx<BM> Ctx;
  constexpr int NBM = GATED ? 2 : 1;              // weight matrices read
  constexpr int BNW = 2 * kPfSN / NBM;            // output columns per tile
  __shared__ __attribute__((aligned(1024))) uint8_t smem[kPfStages * S::STAGE_BYTES];
  __shared__ Ctx ctx[2];

  // ---- this workgroup's tiles: XCD x (dispatch deals workgroups to the 8
  // XCDs in turn) owns a contiguous chunk of the live tiles, walked by its
  // workgroups in step, so tiles running together on one XCD share weight
  // columns (row tiles of one expert) and x rows (column tiles of one row
  // tile) in its L2.
  const int nN = a.N / BNW;
  const int L = (a.expert_off[a.E] / BM) * nN;
  const int wpx = gridDim.x >> 3;
  const int xcd = blockIdx.x & 7;
  const int chunk = (L + 7) >> 3;
  const int t_end = min((xcd + 1) * chunk, L);
  int t = xcd * chunk + (blockIdx.x >> 3);
  if (t >= t_end) return;

  const int tid = threadIdx.x, lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = w >> 2, wn = w & 3;              // row group, column group
  typedef __attribute__((address_space(3))) uint8_t lds_u8;
  const uint32_t smem_lds = __builtin_amdgcn_readfirstlane(
      static_cast<uint32_t>(reinterpret_cast<uintptr_t>((lds_u8*)smem)));
  const uint32_t page = a.pd.page;
  const int nk = a.K / kPfBK;
  const uint32_t row_bytes = static_cast<uint32_t>(a.N) * 2;
  const uint32_t stage_step = static_cast<uint32_t>(kPfBK) * row_bytes;
  const int np = NBM * a.P;

  // ---- tile contexts. Loading one takes global reads whose results are
  // written to LDS later (after a wait), so the loads are split from the
  // stores: prep_load issues them, prep_store writes what they returned.
  constexpr int PREP = (kPfCtxPages + S::NT - 1) / S::NT;
  struct Prep { uint32_t pg[PREP]; int32_t slot; float w; int32_t r0, n0; };
  auto prep_load = [&](int tt, Prep& p) {
    const int mt = tt / nN, nt = tt - mt * nN;
    const int e = a.tile_expert[mt];
    p.r0 = mt * BM;
    p.n0 = nt * BNW;
#pragma unroll
    for (int j = 0; j < PREP; ++j) {
      const int i = tid + j * S::NT;
      const int ii = i < np ? i : 0;
      const int b = ii / a.P, q = ii - b * a.P;
      p.pg[j] = static_cast<uint32_t>(a.pt[static_cast<int64_t>(e * 3 + (GATED ? b : 2)) * a.P + q]);
    }
    p.slot = a.TK;
    p.w = 0.0f;
    if (tid < BM) {
      p.slot = a.sorted_ids[p.r0 + tid];
      if (!GATED && p.slot < a.TK) p.w = a.topk_w[p.slot];
    }
  };
  auto prep_store = [&](Ctx& c, const Prep& p) {
#pragma unroll
    for (int j = 0; j < PREP; ++j) {
      const int i = tid + j * S::NT;
      if (i < np) c.page[i] = reinterpret_cast<uint64_t>(a.pool) + static_cast<uint64_t>(p.pg[j]) * page;
    }
    if (tid < BM) {
      c.slot[tid] = p.slot;
      c.w[tid] = p.w;
    }
    if (tid == 0) {
      c.r0 = p.r0;
      c.n0 = p.n0;
    }
  };

  // ---- per-lane copy sources of a tile.
  // A: a stage's 128 rows x 32 K are stored row-major (64 bytes a row), their
  // 16-byte K octets XOR-swizzled by row (octet o of row r at slot
  // o ^ (r/4)%4) so operand reads are conflict-free; one copy fills 16 whole
  // row pieces: lane l fetches row RPC*c + l/4, slot l%4 of chunk c.
  // B: a weight sub-tile (32 rows of 512 bytes) is stored as 16 chunks of two
  // rows, chunk c holding rows 8(c/4) + c%4 and that + 4, padded to 1088
  // bytes; each copy fetches two whole 512-byte row pieces in lane order.
  // A weight segment's pool address is the address of its page (LDS, the
  // tile context) plus its offset in the page. A tile's stages are looked up
  // in order, so each B copy carries its segment's page index q and offset
  // in the page r for the next stage, advanced by the stage's step
  // (Qs pages and Rs bytes) with one compare instead of a division.
  struct Src { const uint8_t* a[S::A_DMA]; uint32_t q[S::B_DMA], r[S::B_DMA]; };
  auto sources = [&](const Ctx& c, Src& s) {
#pragma unroll
    for (int d = 0; d < S::A_DMA; ++d) {
      const int trow = (w * S::A_DMA + d) * S::RPC + lane / S::OPR;
      int64_t src = c.r0 + trow;
      bool zero = false;
      if (a.kdiv > 0) {
        const int slot = c.slot[trow];
        src = slot < a.TK ? slot / a.kdiv : 0;
        zero = slot >= a.TK && a.lda * 2 <= kPfZeroRowBytes;   // padding: the zero row
      }
      const int oct = (lane % S::OPR) ^ ((trow >> 2) & (S::OPR - 1));
      s.a[d] = zero ? g_pf_zero_row + 8 * oct * 2 : a.A + (src * a.lda + 8 * oct) * 2;
    }
#pragma unroll
    for (int d = 0; d < S::B_DMA; ++d) {
      const int cb = w * S::B_DMA + d;
      const int b = cb / S::SUB_CHUNKS, cc = cb % S::SUB_CHUNKS;
      const int r = 8 * (cc >> 2) + (cc & 3) + 4 * (lane >> 5);
      const int col = GATED ? c.n0 + 8 * (lane & 31) : c.n0 + b * kPfSN + 8 * (lane & 31);
      const uint32_t f = static_cast<uint32_t>(r) * row_bytes + static_cast<uint32_t>(col) * 2;
      s.q[d] = page_index(f, a.pd);
      s.r[d] = f - s.q[d] * page;
    }
  };
  // page-table row (matrix) of B copy d
  auto bmat = [&](int d) { return GATED ? (w * S::B_DMA + d) / S::SUB_CHUNKS : 0; };

  // Copy addresses of one stage, looked up one K step before the copies are
  // issued so the copies never wait on the LDS reads of the page addresses.
  // The page address and the offset stay apart until the copy: adding them
  // at lookup time would make the wavefront wait for the LDS read there.
  struct Refill { uint64_t pb[S::B_DMA]; uint32_t rem[S::B_DMA]; };
  const uint32_t Qs = stage_step / page, Rs = stage_step - Qs * page;
  auto lookup_one = [&](const Ctx& c, Src& s, Refill& r, int d) {
    r.pb[d] = c.page[bmat(d) * a.P + s.q[d]];
    r.rem[d] = s.r[d];
    const uint32_t nr = s.r[d] + Rs;              // the next stage's segment: < 2 pages on
    const bool wrap = nr >= page;
    s.r[d] = wrap ? nr - page : nr;
    s.q[d] += Qs + (wrap ? 1u : 0u);
  };
  auto copy_one = [&](const Src& s, const Refill& r, int rst, uint32_t buf_lds, int d) {
    if (d < S::A_DMA) {
      copy_to_lds16(s.a[d] + rst * kPfBK * 2, buf_lds + (w * S::A_DMA + d) * 1024);
    } else {
      const int db = d - S::A_DMA;
      const int cb = w * S::B_DMA + db;
      copy_to_lds16(reinterpret_cast<const void*>(r.pb[db] + r.rem[db]),
                    buf_lds + S::A_BYTES + (cb / S::SUB_CHUNKS) * S::SUB_LDS + (cb % S::SUB_CHUNKS) * S::CHUNK_PITCH);
    }
  };

  // ---- per-lane operand read offsets
  const int grp = lane >> 4, sl = lane & 15;
  uint32_t boff[2];                               // B: column block jj of this wavefront
#pragma unroll
  for (int jj = 0; jj < 2; ++jj) {
    const int chunk_i = 4 * (grp >> 1) + (sl >> 2);
    const int col = 64 * wn + 32 * jj + 16 * (grp & 1) + 4 * (sl & 3);
    boff[jj] = S::A_BYTES + chunk_i * S::CHUNK_PITCH + col * 2;
  }
  uint32_t aoff[S::KS];                           // A: row lane%32, octet 2s + lane/32
#pragma unroll
  for (int s2 = 0; s2 < S::KS; ++s2) {
    const int row = lane & 31;
    const int oct = 2 * s2 + (lane >> 5);
    aoff[s2] = row * (2 * kPfBK) + ((oct ^ ((row >> 2) & (S::OPR - 1))) * 16);
  }
  typedef __attribute__((address_space(3))) v4i16 lds_v4;
  struct Frags { u32x4 a[S::TM]; u32x4 b[2][2]; };
  // operand read k (0..NREAD-1) of K step s from the stage at buf: the
  // wavefront's A row blocks, then the lower and upper halves of its 4 B operands
  auto read_one = [&](Frags& f, int buf, int s, int k) {
    const uint8_t* base = smem + buf * S::STAGE_BYTES;
    if (k < S::TM) {
      f.a[k] = *reinterpret_cast<const u32x4*>(base + (wm * S::TM + k) * 32 * (2 * kPfBK) + aoff[s]);
    } else {
      const int b = (k - S::TM) >> 2, jj = ((k - S::TM) >> 1) & 1, half = (k - S::TM) & 1;
      const uint8_t* p = base + boff[jj] + b * S::SUB_LDS + s * 8 * S::CHUNK_PITCH + half * 512;
      const u32x2 v = __builtin_bit_cast(u32x2, __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4*)p));
      f.b[b][jj][2 * half] = v[0];
      f.b[b][jj][2 * half + 1] = v[1];
    }
  };

  f32x16 acc[S::TM][2][2];
  auto zero_acc = [&]() {
#pragma unroll
    for (int i = 0; i < S::TM; ++i)
#pragma unroll
      for (int b = 0; b < 2; ++b)
#pragma unroll
        for (int jj = 0; jj < 2; ++jj)
#pragma unroll
          for (int r = 0; r < 16; ++r) acc[i][b][jj][r] = 0.0f;
  };
  // MFMA t (0..NMMA-1) of one K step: row block t/4, sub-tile (t/2)%2, column block t%2
  auto mma = [&](const Frags& f, int tt) {
    const int i = tt >> 2, b = (tt >> 1) & 1, jj = tt & 1;
    acc[i][b][jj] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, f.a[i]),
                                                            __builtin_bit_cast(bf16x8, f.b[b][jj]),
                                                            acc[i][b][jj], 0, 0, 0);
  };

  // ---- one stage: the MFMAs of its two K steps, with the operand reads of
  // the next K step, the page lookups and copies of the refill, the wait for
  // the next stage's copies and the barrier spread between them. Every
  // wavefront issues in this order; the scheduling barriers keep it.
  //   RK: 0 no refill, 1 refill stage rst of this tile, 2 of the next tile
  //   VM: copies allowed in flight at the wait (the stages after the next)
  //   MORE: a next stage exists (wait and barrier); 2: also read its first
  //   operands here (1: they are read after the epilogue, which needs the
  //   registers)
  Frags fr[2];
  Src cur, nxt;
  int buf = 0;                                    // ring position of the stage being multiplied
  int cidx = 0;                                   // context of the current tile (the other: the next)
  auto stage = [&](auto RK, auto VM, auto MORE, int rst) {
    constexpr int rk = decltype(RK)::value;
    constexpr int vm = decltype(VM)::value;
    constexpr int more_k = decltype(MORE)::value;
    constexpr bool more = more_k > 0, read_next = more_k > 1;
    const Ctx& rc = ctx[(rk == 2) ? (cidx ^ 1) : cidx];
    Src& rs = (rk == 2) ? nxt : cur;
    const int nbuf = buf == kPfStages - 1 ? 0 : buf + 1;
    const uint32_t buf_lds = smem_lds + buf * S::STAGE_BYTES;   // refill target: this stage's slot
    Refill rf;
#pragma unroll
    for (int tt = 0; tt < S::NMMA; ++tt) {
      mma(fr[0], tt);
#pragma unroll
      for (int k = tt * S::NREAD / S::NMMA; k < (tt + 1) * S::NREAD / S::NMMA; ++k) read_one(fr[1], buf, 1, k);
      if constexpr (rk != 0) {
#pragma unroll
        for (int d = tt * S::B_DMA / S::NMMA; d < (tt + 1) * S::B_DMA / S::NMMA; ++d) lookup_one(rc, rs, rf, d);
      }
      __builtin_amdgcn_sched_barrier(0);
    }
    constexpr int PRE = kPfPre;                   // MFMAs of the second K step before the barrier
#pragma unroll
    for (int tt = 0; tt < PRE; ++tt) mma(fr[1], tt);
    __builtin_amdgcn_sched_barrier(0);
    if constexpr (more) {
      wait_lds();
      wait_vmem<vm>();
      barrier_only();
    }
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int tt = PRE; tt < S::NMMA; ++tt) {
      mma(fr[1], tt);
      constexpr int R = S::NMMA - PRE;
      if constexpr (read_next) {
#pragma unroll
        for (int k = (tt - PRE) * S::NREAD / R; k < (tt - PRE + 1) * S::NREAD / R; ++k) read_one(fr[0], nbuf, 0, k);
      }
      if constexpr (rk != 0) {
#pragma unroll
        for (int d = (tt - PRE) * S::DMA / R; d < (tt - PRE + 1) * S::DMA / R; ++d) copy_one(rs, rf, rst, buf_lds, d);
      }
      __builtin_amdgcn_sched_barrier(0);
    }
    buf = nbuf;
  };
  using C0 = std::integral_constant<int, 0>;
  using C1 = std::integral_constant<int, 1>;
  using C2 = std::integral_constant<int, 2>;
  using VMD = std::integral_constant<int, S::DMA>;   // in flight at a wait: the copies of the stage after next
  using T_ = std::integral_constant<int, 2>;      // next stage: wait, barrier, first operand reads
  using W_ = std::integral_constant<int, 1>;      // next stage: wait and barrier only
  using F_ = std::integral_constant<int, 0>;      // last stage of the workgroup

  // ---- epilogue: acc[r] of a 32x32 tile is row 8(r/4) + 4(lane/32) + r%4,
  // column lane%32. Neighbouring lanes swap one value so each lane stores two
  // adjacent columns of one row (even lane: row R, columns c, c+1; odd lane:
  // row R+1, columns c-1, c): 4-byte stores, 64 contiguous bytes per row.
  const bool odd = lane & 1;
  auto silu_fast = [](float v) {
    return v * __builtin_amdgcn_rcpf(1.0f + __builtin_amdgcn_exp2f(-1.4426950408889634f * v));
  };
  // Stores address the output as its uniform base plus a 32-bit byte offset
  // (the launcher checks the output spans less than 4 GiB), which keeps one
  // register per store address.
  uint8_t* const Cb = a.C;
  const uint32_t ldc2 = static_cast<uint32_t>(a.ldc) * 2;
  auto store2 = [&](uint32_t off, float lo, float hi) {
    *reinterpret_cast<uint32_t*>(Cb + off) = pack_bf16x2(lo, hi);
  };
  auto epilogue = [&](const Ctx& c) {
    const uint32_t colb = static_cast<uint32_t>(c.n0 + 64 * wn + (lane & 31) - (odd ? 1 : 0)) * 2;
#pragma unroll
    for (int i = 0; i < S::TM; ++i)
#pragma unroll
      for (int r = 0; r < 16; r += 2) {
        __builtin_amdgcn_sched_barrier(0);                 // bounds the temporaries in flight
        const int trow = 32 * (wm * S::TM + i) + 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3) + (odd ? 1 : 0);
        if constexpr (GATED) {
          const uint32_t rowb = static_cast<uint32_t>(c.r0 + trow) * ldc2 + colb;
#pragma unroll
          for (int jj = 0; jj < 2; ++jj) {
            const float v0 = silu_fast(acc[i][0][jj][r]) * acc[i][1][jj][r];
            const float v1 = silu_fast(acc[i][0][jj][r + 1]) * acc[i][1][jj][r + 1];
            const float y = swap_lane_pair(odd ? v0 : v1);
            store2(rowb + 64 * jj, odd ? y : v0, odd ? v1 : y);
          }
        } else {
          const int slot = c.slot[trow];
          const float wt = c.w[trow];
          const uint32_t rowb = static_cast<uint32_t>(slot) * ldc2 + colb;
#pragma unroll
          for (int b = 0; b < 2; ++b)
#pragma unroll
            for (int jj = 0; jj < 2; ++jj) {
              const float v0 = acc[i][b][jj][r], v1 = acc[i][b][jj][r + 1];
              const float y = swap_lane_pair(odd ? v0 : v1);
              if (slot < a.TK) store2(rowb + 2 * kPfSN * b + 64 * jj, wt * (odd ? y : v0), wt * (odd ? v1 : y));
            }
        }
      }
  };

  // ---- prologue: the first tile's context, its first three stages in flight
  {
    Prep p;
    prep_load(t, p);
    prep_store(ctx[0], p);
  }
  __syncthreads();
  sources(ctx[0], cur);
  {
    Refill rf;
#pragma unroll
    for (int st = 0; st < kPfStages; ++st) {
#pragma unroll
      for (int d = 0; d < S::B_DMA; ++d) lookup_one(ctx[0], cur, rf, d);
#pragma unroll
      for (int d = 0; d < S::DMA; ++d) copy_one(cur, rf, st, smem_lds + st * S::STAGE_BYTES, d);
    }
  }
  wait_vmem<2 * S::DMA>();
  barrier_only();
#pragma unroll
  for (int k = 0; k < S::NREAD; ++k) read_one(fr[0], 0, 0, k);
  zero_acc();

  // ---- tiles. Every tile runs the same straight-line sequence; after the
  // workgroup's last tile the "next" tile is that tile again, whose copies
  // land in the ring unread (drained before the workgroup exits).
  for (;;) {
    const int t_next = t + wpx;
    const bool has_next = t_next < t_end;
    // stage 0: the next tile's context is loaded and stored to the spare
    // context once every wavefront has passed the barrier (the spare context
    // is then free: the previous tile's epilogue, its last reader, is done);
    // it is visible after the barrier of stage 1. Stage 0's wait takes every
    // copy and store in flight, the previous tile's epilogue stores included.
    Prep p;
    prep_load(has_next ? t_next : t, p);
    stage(C1(), C0(), T_(), 3);
    prep_store(ctx[cidx ^ 1], p);
    // stages 1 .. nk-4: refill stage st+3 of this tile
    for (int st = 1; st + 3 < nk; ++st) stage(C1(), VMD(), T_(), st + 3);
    // the next tile's copy sources, then its first three stages as the
    // refills of this tile's last three
    sources(ctx[cidx ^ 1], nxt);
    stage(C2(), VMD(), T_(), 0);
    stage(C2(), VMD(), T_(), 1);
    stage(C2(), VMD(), W_(), 2);
    epilogue(ctx[cidx]);
    if (!has_next) break;
    zero_acc();
#pragma unroll
    for (int k = 0; k < S::NREAD; ++k) read_one(fr[0], buf, 0, k);
    cur = nxt;
    cidx ^= 1;
    t = t_next;
  }
  wait_vmem<0>();                                 // no copy may land after the workgroup ends
}

// ---------------------------------------------------------------- launcher

namespace {
int cu_count() {
  static int n = 0;
  if (n == 0) {
    int dev = 0, v = 0;
    if (hipGetDevice(&dev) == hipSuccess && hipDeviceGetAttribute(&v, hipDeviceAttributeMultiprocessorCount, dev) == hipSuccess && v > 0)
      n = v;
    else
      n = 256;
  }
  return n;
}
}  // namespace

// 128-row tiles: 8 wavefronts (two per SIMD, 64 rows x 128 columns each);
// 64-row tiles: 4 wavefronts (one per SIMD, the same 64 x 128 each), for
// the down projection of weight-bound layers (few rows per expert): its
// tiles carry half the padding and the copies, not the MFMAs, set its pace.
template <bool GATED>
hipError_t launch_prefill(int bm, const GemmArgs& g, uint64_t tiles_max, hipStream_t st) {
  const int nbm = GATED ? 2 : 1;
  const int bnw = 2 * kPfSN / nbm;
  if (bm != 128 && (bm != 64 || GATED)) return hipErrorNotSupported;
  // shapes this kernel covers: whole column tiles, whole stages, at least
  // five stages (the first and the last three are peeled, and the next
  // tile's context needs one barrier between them), page addresses of a tile
  // within one context
  const uint64_t out_rows = GATED ? tiles_max * bm : static_cast<uint64_t>(g.TK);
  if (g.N % bnw != 0 || g.K % kPfBK != 0 || g.K / kPfBK < 5 || nbm * g.P > kPfCtxPages ||
      out_rows * static_cast<uint64_t>(g.ldc) * 2 >= (1ull << 32))
    return hipErrorNotSupported;
  const uint64_t tiles = tiles_max * static_cast<uint64_t>(g.N / bnw);
  uint64_t grid = std::min<uint64_t>(static_cast<uint64_t>(cu_count() / 8 * 8), (tiles + 7) / 8 * 8);
  if (grid == 0) return hipSuccess;
#ifndef RIMURU_PF128_NW
#define RIMURU_PF128_NW 8
#endif
  if (bm == 128)
    hipLaunchKernelGGL((k_moe_gemm_pf<GATED, RIMURU_PF128_NW, 128>), dim3(static_cast<uint32_t>(grid)),
                       dim3(RIMURU_PF128_NW * 64), 0, st, g);
  else if constexpr (!GATED)
    hipLaunchKernelGGL((k_moe_gemm_pf<GATED, 4, 64>), dim3(static_cast<uint32_t>(grid)), dim3(4 * 64), 0, st, g);
  return hipGetLastError();
}

template hipError_t launch_prefill<true>(int, const GemmArgs&, uint64_t, hipStream_t);
template hipError_t launch_prefill<false>(int, const GemmArgs&, uint64_t, hipStream_t);

}  // namespace rimuru
