// Page-table-aware fused MoE for CDNA4 (gfx950).
//
// Rimuru paper summary (thelatestinai.com), abstract: a fused MoE kernel that
// reads non-contiguous expert weights directly through the expert view's page
// table, so no expert is ever copied into a contiguous buffer; Figure 11 names
// it "Discrete FusedMoE". Explainer "Rimuru unifies serving memory"
// (learnaivisually.com), paragraph on the two pieces that make the moving
// fence usable: the kernel reads expert pages where they sit. Table 1 of the
// summary gives the three projections per expert (w1, w3 [H, I], w2 [I, H]).
//
// Stages (one launch each, all on the caller's stream, no host sync):
//   1 gating     one wavefront per token: top-k on raw logits, then softmax
//                over the kept logits (the renormalised softmax weights)
//   2 count      one workgroup per expert: routed slots per expert
//   3 sort       one workgroup per expert: stable list of slots t*k+j,
//                padded to the tile height, tile -> expert map
//   4 gemm-up    grouped GEMM over sorted rows: h = SiLU(x w1) * (x w3),
//                w1/w3 tiles fetched page by page
//   5 gemm-down  grouped GEMM: y_slot[t*k+j] = w[t,j] * (h w2)
//   6 combine    y[t] = sum_j y_slot[t*k+j], j in rank order
//
// Every 16-byte weight segment a lane loads gets its own page lookup
// (page = offset / page_bytes by multiply-shift, then the page table); a
// segment never straddles a page because pages are multiples of 128 bytes and
// segments start on 16-byte boundaries. Results do not depend on where the
// pages sit, so the paged and the contiguous layouts give identical bits.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cstdint>

#include "rimuru.h"
#include "rimuru_internal.h"

namespace rimuru {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef short v4i16 __attribute__((ext_vector_type(4)));

constexpr int kMaxK = 32;
constexpr int kMaxE = 512;

// offset / page for offset < 2^31 by one 64-bit multiply and a shift
// (Granlund & Montgomery, "Division by Invariant Integers using
// Multiplication", 1994: m = 2^32 + floor(2^32 (2^l - d) / d) + 1, l = ceil
// log2 d, q = (n m) >> (32 + l)).
struct PageDiv {
  uint64_t mul;
  uint32_t shift;
  uint32_t page;
};

__device__ __forceinline__ uint32_t page_index(uint32_t f, const PageDiv& d) {
  return static_cast<uint32_t>((static_cast<uint64_t>(f) * d.mul) >> d.shift);
}

__device__ __forceinline__ float bf16_to_f32(uint32_t b) { return __uint_as_float(b << 16); }

// fp32 -> bf16, round to nearest even; NaN stays a quiet NaN.
__device__ __forceinline__ uint32_t f32_to_bf16(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7fffffffu) > 0x7f800000u) return (u >> 16) | 0x40u;
  u += 0x7fffu + ((u >> 16) & 1u);
  return u >> 16;
}

__device__ __forceinline__ float silu(float a) { return a / (1.0f + expf(-a)); }

// ---------------------------------------------------------------- elements

template <typename T>
struct Elt;

// bf16 stored as its 16-bit pattern.
template <>
struct Elt<uint16_t> {
  static constexpr int ES = 2;
  static constexpr int VEC = 8;  // elements per 16-byte segment
  static constexpr int KI = 32;  // K of one MFMA (v_mfma_f32_16x16x32_bf16)
  static constexpr int FE = 8;   // elements of one operand per lane
  typedef u32x4 Frag;
  static __device__ __forceinline__ Frag frag(const uint16_t* p) {
    return *reinterpret_cast<const u32x4*>(p);
  }
  static __device__ __forceinline__ f32x4 mma(Frag a, Frag b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a),
                                                   __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
  }
  static __device__ __forceinline__ float to_f32(uint32_t bits) { return bf16_to_f32(bits); }
  static __device__ __forceinline__ uint32_t from_f32(float v) { return f32_to_bf16(v); }
  static __device__ __forceinline__ void put(uint16_t* p, float v) {
    *p = static_cast<uint16_t>(f32_to_bf16(v));
  }
  // element c of a 16-byte segment
  static __device__ __forceinline__ uint32_t get(const u32x4& s, int c) {
    return (s[c >> 1] >> ((c & 1) * 16)) & 0xffffu;
  }
  // B operand of a 32x32x16 MFMA from a row-major [K][N] LDS tile (pitch in
  // elements): lane l needs B[k0 + 8*(l/32) .. +7][n0 + l%32]. Two transposed
  // LDS reads (ds_read_b64_tr_b16) deliver it: in each 16-lane group, source
  // lane s points at B[k0 + s/4][n0 + 4*(s%4)] and output lane i receives
  // B[k0 .. k0+3][n0 + i].
  static constexpr int B_PAD = 32;   // row padding (elements): 64 bytes
  static __device__ __forceinline__ Frag bfrag32(const uint16_t* tile, int pitch, int k0, int n0,
                                                 int lane) {
    const int grp = lane >> 4, s = lane & 15;
    const int row = k0 + 8 * (grp >> 1) + (s >> 2);
    const int col = n0 + 16 * (grp & 1) + 4 * (s & 3);
    // tile points into LDS: the generic -> local address-space cast is exact
    typedef __attribute__((address_space(3))) v4i16 lds_v4;
    lds_v4* p0 = (lds_v4*)(tile + row * pitch + col);
    lds_v4* p1 = (lds_v4*)(tile + (row + 4) * pitch + col);
    const v4i16 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(p0);
    const v4i16 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(p1);
    const u32x2 a = __builtin_bit_cast(u32x2, lo), b = __builtin_bit_cast(u32x2, hi);
    return u32x4{a[0], a[1], b[0], b[1]};
  }
  // 32x32 output tile, K = 16 per MFMA, 8 values of each operand per lane
  static constexpr int KI32 = 16;
  static __device__ __forceinline__ f32x16 mma32(Frag a, Frag b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a),
                                                   __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
  }
  // B operand of a 16x16x32 MFMA from a row-major [K][N] LDS tile: lane l
  // needs B[k0 + 8*(l/16) .. +7][n0 + l%16]; two transposed LDS reads (see
  // bfrag32: here each 16-lane group covers one K octet).
  static __device__ __forceinline__ void bfrag16(const uint16_t* tile, int pitch, int k0, int n0,
                                                 int lane, u32x4 (&out)[1]) {
    const int grp = lane >> 4, s = lane & 15;
    const int row = k0 + 8 * grp + (s >> 2);
    const int col = n0 + 4 * (s & 3);
    typedef __attribute__((address_space(3))) v4i16 lds_v4;
    lds_v4* p0 = (lds_v4*)(tile + row * pitch + col);
    lds_v4* p1 = (lds_v4*)(tile + (row + 4) * pitch + col);
    const u32x2 a = __builtin_bit_cast(u32x2, __builtin_amdgcn_ds_read_tr16_b64_v4i16(p0));
    const u32x2 b = __builtin_bit_cast(u32x2, __builtin_amdgcn_ds_read_tr16_b64_v4i16(p1));
    out[0] = u32x4{a[0], a[1], b[0], b[1]};
  }
  // 8 consecutive K values per lane (one 16-byte segment): one MFMA
  static constexpr int SEG8 = 1;
  static __device__ __forceinline__ f32x4 mma8(const u32x4* a, const u32x4* b, f32x4 c) {
    return mma(a[0], b[0], c);
  }
};

template <>
struct Elt<float> {
  static constexpr int ES = 4;
  static constexpr int VEC = 4;
  static constexpr int KI = 4;   // v_mfma_f32_16x16x4_f32
  static constexpr int FE = 1;
  typedef float Frag;
  static __device__ __forceinline__ Frag frag(const float* p) { return *p; }
  static __device__ __forceinline__ f32x4 mma(Frag a, Frag b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
  }
  static __device__ __forceinline__ float to_f32(uint32_t bits) { return __uint_as_float(bits); }
  static __device__ __forceinline__ uint32_t from_f32(float v) { return __float_as_uint(v); }
  static __device__ __forceinline__ void put(float* p, float v) { *p = v; }
  static __device__ __forceinline__ uint32_t get(const u32x4& s, int c) { return s[c]; }
  // B operand of a 32x32x2 MFMA from a row-major [K][N] LDS tile: lane l
  // needs B[k0 + l/32][n0 + l%32], one plain read.
  static constexpr int B_PAD = 4;    // row padding (elements): 16 bytes
  static __device__ __forceinline__ Frag bfrag32(const float* tile, int pitch, int k0, int n0, int lane) {
    return tile[(k0 + (lane >> 5)) * pitch + n0 + (lane & 31)];
  }
  // 32x32 output tile, K = 2 per MFMA, one value of each operand per lane
  static constexpr int KI32 = 2;
  static __device__ __forceinline__ f32x16 mma32(Frag a, Frag b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x2f32(a, b, c, 0, 0, 0);
  }
  // 8 consecutive K values B[k0 + 8*(l/16) + kk][n0 + l%16] per lane, plain reads
  static __device__ __forceinline__ void bfrag16(const float* tile, int pitch, int k0, int n0, int lane,
                                                 u32x4 (&out)[2]) {
    const float* src = tile + (k0 + 8 * (lane >> 4)) * pitch + n0 + (lane & 15);
#pragma unroll
    for (int kk = 0; kk < 8; ++kk) out[kk >> 2][kk & 3] = __float_as_uint(src[kk * pitch]);
  }
  // 8 consecutive K values per lane (two 16-byte segments): eight K=4 MFMAs,
  // MFMA kk taking K value kk of every lane's group.
  static constexpr int SEG8 = 2;
  static __device__ __forceinline__ f32x4 mma8(const u32x4* a, const u32x4* b, f32x4 c) {
#pragma unroll
    for (int kk = 0; kk < 8; ++kk)
      c = mma(__uint_as_float(a[kk >> 2][kk & 3]), __uint_as_float(b[kk >> 2][kk & 3]), c);
    return c;
  }
};

// ---------------------------------------------------------------- stage 1: gating

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

__device__ __forceinline__ uint64_t wave_max_u64(uint64_t v) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) {
    uint32_t lo = __shfl_xor(static_cast<uint32_t>(v), off, 64);
    uint32_t hi = __shfl_xor(static_cast<uint32_t>(v >> 32), off, 64);
    uint64_t o = (static_cast<uint64_t>(hi) << 32) | lo;
    v = o > v ? o : v;
  }
  return v;
}

__device__ __forceinline__ float wave_sum_f32(float v) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) v += __shfl_xor(v, off, 64);
  return v;
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

// ---------------------------------------------------------------- stage 2: count

// ids is 16-byte aligned (validated); 8 independent 16-byte loads per thread
// are in flight per round.
__global__ __launch_bounds__(256) void k_count(const int32_t* __restrict__ ids, int TK,
                                               int32_t* __restrict__ counts) {
  __shared__ int part[4];
  const int e = blockIdx.x;
  const int n4 = TK >> 2;
  const u32x4* v = reinterpret_cast<const u32x4*>(ids);
  const uint32_t ue = static_cast<uint32_t>(e);
  int c = 0;
  for (int base = 0; base < n4; base += 256 * 8) {
    u32x4 r[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const int i = base + u * 256 + threadIdx.x;
      r[u] = (i < n4) ? v[i] : u32x4{~0u, ~0u, ~0u, ~0u};
    }
#pragma unroll
    for (int u = 0; u < 8; ++u)
      c += (r[u][0] == ue) + (r[u][1] == ue) + (r[u][2] == ue) + (r[u][3] == ue);
  }
  for (int f = n4 * 4 + threadIdx.x; f < TK; f += 256) c += (ids[f] == e);
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) c += __shfl_xor(c, off, 64);
  if ((threadIdx.x & 63) == 0) part[threadIdx.x >> 6] = c;
  __syncthreads();
  if (threadIdx.x == 0) counts[e] = part[0] + part[1] + part[2] + part[3];
}

// ---------------------------------------------------------------- stage 3: sort + align

// Exclusive prefix of v over the 256 threads of the block; *total gets the sum.
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
  for (int i = 0; i < 4; ++i) {
    before += (i < wv) ? sh[i] : 0;
    all += sh[i];
  }
  __syncthreads();
  *total = all;
  return before + incl - v;
}

constexpr int kSortChunk = 64;  // consecutive slots per thread per round (16 x 16-byte loads)

// counts == nullptr: the workgroup builds the per-expert histogram itself in
// LDS (small batches: this saves the separate count launch).
constexpr int kSortSelfCountMax = 4096;   // routed slots

__global__ __launch_bounds__(256) void k_sort_align(const int32_t* __restrict__ ids, int TK, int E,
                                                    int BM, const int32_t* __restrict__ counts,
                                                    int32_t* __restrict__ sorted_ids,
                                                    int32_t* __restrict__ expert_off,
                                                    int32_t* __restrict__ tile_expert) {
  __shared__ int sh[4];
  __shared__ int hist[kMaxE];
  const int e = blockIdx.x;
  const int tid = threadIdx.x;
  const uint32_t ue = static_cast<uint32_t>(e);
  if (counts == nullptr) {
    for (int i = tid; i < E; i += 256) hist[i] = 0;
    __syncthreads();
    for (int f = tid; f < TK; f += 256) atomicAdd(&hist[ids[f]], 1);
    __syncthreads();
    counts = hist;
  }
  // start of this expert's padded segment, and the padded total
  int before = 0, total = 0;
  for (int e2 = tid; e2 < E; e2 += 256) {
    int pc = (counts[e2] + BM - 1) / BM * BM;
    total += pc;
    before += (e2 < e) ? pc : 0;
  }
  int sum_before, sum_total;
  block_excl_scan(before, &sum_before, sh);   // block sums of the per-thread partials
  block_excl_scan(total, &sum_total, sh);
  const int seg = sum_before;
  const int cnt = counts[e];
  if (tid == 0) {
    expert_off[e] = seg;
    if (e == 0) expert_off[E] = sum_total;
  }
  const bool vec = (TK & 3) == 0;
  int running = 0;
  for (int base = 0; base < TK; base += 256 * kSortChunk) {
    const int f0 = base + tid * kSortChunk;
    uint64_t mask = 0;
    if (vec) {
      u32x4 r[kSortChunk / 4];
#pragma unroll
      for (int u = 0; u < kSortChunk / 4; ++u)
        r[u] = (f0 + 4 * u < TK) ? *reinterpret_cast<const u32x4*>(ids + f0 + 4 * u)
                                 : u32x4{~0u, ~0u, ~0u, ~0u};
#pragma unroll
      for (int u = 0; u < kSortChunk / 4; ++u)
#pragma unroll
        for (int c = 0; c < 4; ++c) mask |= static_cast<uint64_t>(r[u][c] == ue) << (4 * u + c);
    } else {
      for (int i = 0; i < kSortChunk; ++i) {
        const int f = f0 + i;
        if (f < TK && ids[f] == e) mask |= 1ull << i;
      }
    }
    int chunk_total;
    int pos = seg + running + block_excl_scan(__popcll(mask), &chunk_total, sh);
    while (mask) {
      const int i = __ffsll(static_cast<long long>(mask)) - 1;
      sorted_ids[pos++] = f0 + i;
      mask &= mask - 1;
    }
    running += chunk_total;
  }
  const int padded = (cnt + BM - 1) / BM * BM;
  for (int i = cnt + tid; i < padded; i += 256) sorted_ids[seg + i] = TK;
  for (int i = tid; i < padded / BM; i += 256) tile_expert[seg / BM + i] = e;
}

// ---------------------------------------------------------------- stages 4, 5: paged grouped GEMM

struct GemmArgs {
  const uint8_t* A;            // GEMM-up: x [T, H]; GEMM-down: h [sorted_len, I]
  int64_t lda;                 // elements per A row
  const int32_t* sorted_ids;
  int kdiv;                    // GEMM-up: token = slot / kdiv
  const uint8_t* pool;
  const int32_t* pt;
  int P;
  PageDiv pd;
  int K, N;                    // C[M, N] = A[M, K] B[K, N]
  const int32_t* tile_expert;
  const int32_t* expert_off;
  int E;
  uint8_t* C;                  // GEMM-up: h; GEMM-down: y_slot [T*k, H]
  int64_t ldc;
  const float* topk_w;
  int TK;                      // number of routed slots; also the padding sentinel
};

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
struct StreamShape { int bn, depth; };
constexpr StreamShape kStreamUp{RIMURU_STREAM_UP}, kStreamDn{RIMURU_STREAM_DN};
constexpr int kStreamUpBN = kStreamUp.bn, kStreamUpDepth = kStreamUp.depth;
constexpr int kStreamDnBN = kStreamDn.bn, kStreamDnDepth = kStreamDn.depth;
constexpr int kStreamPtMax = 4096; // page-table entries a workgroup stages in LDS

// NSTEPS > 0: the wavefront's step count is known at compile time and the K
// loop unrolls into straight-line code (a loop back-edge makes the compiler
// wait for every load in flight at the loop head). NSTEPS == 0: runtime loop.
template <typename T, int BN, int DEPTH, bool GATED, int NSTEPS>
__global__ __launch_bounds__(kStreamMaxWaves * 64, RIMURU_STREAM_WG_PER_CU) void k_paged_gemm_stream(GemmArgs a, int ksplit) {
  typedef Elt<T> X;
  constexpr int NB = GATED ? 2 : 1;
  constexpr int VEC = X::VEC;
  constexpr int CG = BN / VEC;                 // 16-byte column groups per weight row
  constexpr int RG = 64 / CG;                  // row groups per wavefront
  constexpr int RPL = kStreamK / RG;           // consecutive weight rows per lane
  constexpr int TN = BN / 16;
  constexpr int BNP = BN + X::B_PAD;           // row pitch of the wave's weight slice
  constexpr int SEG8 = X::SEG8;
  static_assert(CG * RG == 64 && RPL * RG == kStreamK, "stream tile shape");
  static_assert(NB * 16 * BN * 4 <= NB * kStreamK * BNP * X::ES, "reduction must fit the wave buffer");

  __shared__ __attribute__((aligned(16))) T lds[kStreamMaxWaves][NB * kStreamK * BNP];
  extern __shared__ int32_t pt_lds[];          // this expert's page-table rows (NB * P)

  const int nN = a.N / BN;
  const int n_tiles = a.expert_off[a.E] / 16;
  const int L = n_tiles * nN;
  const int chunk = (L + 7) >> 3;
  const int xcd = blockIdx.x & 7, idx = blockIdx.x >> 3;
  if (idx >= chunk) return;
  const int logical = xcd * chunk + idx;
  if (logical >= L) return;
  const int mt = logical / nN;
  const int nt = logical - mt * nN;
  const int e = a.tile_expert[mt];
  const int r0 = mt * 16;
  const int n0 = nt * BN;

  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  const int fi = lane & 15, fq = lane >> 4;
  const int kw = a.K / ksplit;
  const int nsteps = kw / kStreamK;
  const int kbase = wv * kw;

  // A operand: row fi of the tile, K values fq*8 .. fq*8+7 of each step.
  // Padding rows read a valid row and are zeroed by a select, so the main
  // loop has no branch around a load (a branch there makes the compiler wait
  // for every load in flight at the join).
  const T* arow;
  bool a_ok = true;
  if (a.kdiv > 0) {
    const int slot = a.sorted_ids[r0 + fi];
    a_ok = slot < a.TK;
    arow = reinterpret_cast<const T*>(a.A) + static_cast<int64_t>(a_ok ? slot / a.kdiv : 0) * a.lda;
  } else {
    arow = reinterpret_cast<const T*>(a.A) + static_cast<int64_t>(r0 + fi) * a.lda;
  }
  const int cg = lane % CG, rg = lane / CG;
  // Page lookups read LDS: a global load here would make every weight load
  // wait for all older ones (vector-memory loads retire in order).
  for (int i = threadIdx.x; i < NB * a.P; i += blockDim.x) {
    const int b = i / a.P, q = i - b * a.P;
    pt_lds[i] = a.pt[static_cast<int64_t>(e * 3 + (GATED ? b : 2)) * a.P + q];
  }
  __syncthreads();
  const int32_t* pt_row[NB];
#pragma unroll
  for (int b = 0; b < NB; ++b) pt_row[b] = pt_lds + b * a.P;
  const uint32_t col_bytes = static_cast<uint32_t>(n0 + cg * VEC) * X::ES;
  const uint32_t row_bytes = static_cast<uint32_t>(a.N) * X::ES;

  u32x4 breg[DEPTH][NB][RPL];
  u32x4 areg[DEPTH][SEG8];
  f32x4 acc[NB][TN];
#pragma unroll
  for (int b = 0; b < NB; ++b)
#pragma unroll
    for (int j = 0; j < TN; ++j) acc[b][j] = f32x4{0.f, 0.f, 0.f, 0.f};

  T* wbuf = lds[wv];

  // Loads of step st (clamped to the last step: the surplus loads at the end
  // repeat addresses already in cache and their data is never used).
  auto issue = [&](u32x4 (&br)[NB][RPL], u32x4 (&ar)[SEG8], int st) {
    st = min(st, nsteps - 1);
    const int k0 = kbase + st * kStreamK;
#pragma unroll
    for (int u = 0; u < SEG8; ++u) ar[u] = *reinterpret_cast<const u32x4*>(arow + k0 + fq * 8 + u * VEC);
#pragma unroll
    for (int b = 0; b < NB; ++b) {
#pragma unroll
      for (int j = 0; j < RPL; ++j) {
        const uint32_t f = static_cast<uint32_t>(k0 + rg * RPL + j) * row_bytes + col_bytes;
        const uint32_t q = page_index(f, a.pd);
        const uint8_t* p = a.pool + static_cast<uint64_t>(pt_row[b][q]) * a.pd.page + (f - q * a.pd.page);
        br[b][j] = *reinterpret_cast<const u32x4*>(p);
      }
    }
  };

  // Multiply step data into the accumulators; live == false (a step past the
  // end) multiplies by a zero A operand, which adds exact zeros.
  auto consume = [&](const u32x4 (&br)[NB][RPL], const u32x4 (&ar)[SEG8], bool live) {
    // the wave's weight slice, row-major as it sits in the pool
#pragma unroll
    for (int b = 0; b < NB; ++b)
#pragma unroll
      for (int j = 0; j < RPL; ++j)
        *reinterpret_cast<u32x4*>(wbuf + b * kStreamK * BNP + (rg * RPL + j) * BNP + cg * VEC) = br[b][j];
    const bool use = live && a_ok;
    u32x4 af[SEG8];
#pragma unroll
    for (int u = 0; u < SEG8; ++u) af[u] = use ? ar[u] : u32x4{0u, 0u, 0u, 0u};
#pragma unroll
    for (int b = 0; b < NB; ++b) {
#pragma unroll
      for (int j = 0; j < TN; ++j) {
        u32x4 bf[SEG8];
        X::bfrag16(wbuf + b * kStreamK * BNP, BNP, 0, j * 16, lane, bf);
        acc[b][j] = X::mma8(af, bf, acc[b][j]);
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

  // ---- reduce the ksplit partial sums in wavefront order, then the epilogue
  __syncthreads();
  float* red = reinterpret_cast<float*>(wbuf);           // [NB][16][BN] of this wavefront
#pragma unroll
  for (int b = 0; b < NB; ++b)
#pragma unroll
    for (int j = 0; j < TN; ++j)
#pragma unroll
      for (int r = 0; r < 4; ++r) red[(b * 16 + 4 * fq + r) * BN + j * 16 + fi] = acc[b][j][r];
  __syncthreads();
  constexpr int PER = 4;                                  // outputs per thread per pass
  T* C = reinterpret_cast<T*>(a.C);
  for (int o = threadIdx.x * PER; o < 16 * BN; o += blockDim.x * PER) {
    const int row = o / BN, col = o % BN;
    float v[NB][PER];
#pragma unroll
    for (int b = 0; b < NB; ++b)
#pragma unroll
      for (int c = 0; c < PER; ++c) v[b][c] = 0.0f;
    for (int w = 0; w < ksplit; ++w) {
      const float* rw = reinterpret_cast<const float*>(lds[w]);
#pragma unroll
      for (int b = 0; b < NB; ++b)
#pragma unroll
        for (int c = 0; c < PER; ++c) v[b][c] += rw[(b * 16 + row) * BN + col + c];
    }
    if constexpr (GATED) {
      T* dst = C + static_cast<int64_t>(r0 + row) * a.ldc + n0 + col;
#pragma unroll
      for (int c = 0; c < PER; ++c) X::put(dst + c, silu(v[0][c]) * v[1][c]);
    } else {
      const int slot = a.sorted_ids[r0 + row];
      if (slot < a.TK) {
        const float wt = a.topk_w[slot];
        T* dst = C + static_cast<int64_t>(slot) * a.ldc + n0 + col;
#pragma unroll
        for (int c = 0; c < PER; ++c) X::put(dst + c, wt * v[0][c]);
      }
    }
  }
}

// ---------------------------------------------------------------- stage 6: combine

template <typename T>
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
  for (int j = 0; j < k; ++j) {
    u32x4 s = *reinterpret_cast<const u32x4*>(yslot + (static_cast<int64_t>(t) * k + j) * H + h0);
#pragma unroll
    for (int c = 0; c < VEC; ++c) acc[c] += X::to_f32(X::get(s, c));
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

__global__ __launch_bounds__(256) void k_store_pages(uint8_t* __restrict__ pool,
                                                     const int32_t* __restrict__ pt, int P,
                                                     PageDiv pd, const uint8_t* __restrict__ src,
                                                     uint64_t proj_bytes, uint64_t n_segs) {
  for (uint64_t s = blockIdx.x * 256ull + threadIdx.x; s < n_segs; s += gridDim.x * 256ull) {
    uint64_t byte = s * 16;
    uint64_t proj = byte / proj_bytes;
    uint32_t off = static_cast<uint32_t>(byte - proj * proj_bytes);
    uint32_t q = page_index(off, pd);
    uint8_t* dst = pool + static_cast<uint64_t>(pt[proj * P + q]) * pd.page + (off - q * pd.page);
    *reinterpret_cast<u32x4*>(dst) = *reinterpret_cast<const u32x4*>(src + byte);
  }
}

// ---------------------------------------------------------------- host side

namespace {

constexpr uint64_t kAlign = 256;
inline uint64_t align_up(uint64_t x) { return (x + kAlign - 1) / kAlign * kAlign; }

PageDiv make_div(uint32_t page) {
  uint32_t l = 0;
  while ((1ull << l) < page) ++l;
  unsigned __int128 num = (static_cast<unsigned __int128>(1) << 32) * ((1ull << l) - page);
  uint64_t m = static_cast<uint64_t>(num / page) + 1 + (1ull << 32);
  return PageDiv{m, 32 + l, page};
}

// Tile height by expected rows per expert (T*k/E): few rows per expert is a
// weight stream (decode), many rows is a dense grouped GEMM (prefill).
enum PlanId { kPlan16 = 0, kPlan64 = 1, kPlan128 = 2 };
struct Plan {
  PlanId id;
  int bm;
};

Plan choose_plan(int64_t T, int E, int k, int64_t P) {
  int64_t tk = T * k;
  if (tk <= 24ll * E && 2 * P <= kStreamPtMax) return {kPlan16, 16};
  if (tk <= 160ll * E) return {kPlan64, 64};
  return {kPlan128, 128};
}

struct Layout {
  uint64_t tiles_max, sorted_len;
  uint64_t off_counts, off_tiles, off_h, off_yslot, total;
};

Layout layout_for(int64_t T, int E, int k, int H, int I, int es, int bm) {
  Layout l;
  int64_t tk = T * k;
  l.tiles_max = static_cast<uint64_t>(tk / bm + (tk < E ? tk : E));
  l.sorted_len = l.tiles_max * bm;
  l.off_counts = 0;
  l.off_tiles = align_up(static_cast<uint64_t>(E) * 4);
  l.off_h = l.off_tiles + align_up(l.tiles_max * 4);
  l.off_yslot = l.off_h + align_up(l.sorted_len * static_cast<uint64_t>(I) * es);
  l.total = l.off_yslot + align_up(static_cast<uint64_t>(tk) * H * es);
  return l;
}

rimuru_status check_shapes(int64_t T, int E, int k, int H, int I, int dtype) {
  if (dtype != RIMURU_BF16 && dtype != RIMURU_F32)
    return rimuru_fail(RIMURU_EDTYPE, "dtype %d is neither RIMURU_BF16 nor RIMURU_F32", dtype);
  if (T < 0) return rimuru_fail(RIMURU_EINVAL, "T = %lld is negative", (long long)T);
  if (E < 1 || E > kMaxE) return rimuru_fail(RIMURU_EINVAL, "E = %d outside [1, %d]", E, kMaxE);
  if (k < 1 || k > E || k > kMaxK)
    return rimuru_fail(RIMURU_EINVAL, "k = %d outside [1, min(E, %d)]", k, kMaxK);
  if (H < 64 || H % 64 != 0 || I < 64 || I % 64 != 0)
    return rimuru_fail(RIMURU_EINVAL, "H = %d and I = %d must be positive multiples of 64", H, I);
  if (T * k >= (1ll << 30)) return rimuru_fail(RIMURU_EINVAL, "T*k = %lld is too large", (long long)(T * k));
  return RIMURU_OK;
}

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

template <typename T, int BN, int DEPTH, bool GATED>
hipError_t launch_stream(const GemmArgs& g, uint64_t tiles_max, hipStream_t st) {
  const int ksteps = g.K / kStreamK;
  const int max_split = GATED ? kStreamUpWaves : kStreamDnWaves;
  const int ksplit = (ksteps % 4 == 0 && max_split >= 4) ? 4 : (ksteps % 2 == 0 && max_split >= 2) ? 2 : 1;
  if (g.N % BN != 0 || g.K % kStreamK != 0) return hipErrorInvalidValue;
  uint64_t blocks = tiles_max * static_cast<uint64_t>(g.N / BN);
  uint64_t grid = (blocks + 7) / 8 * 8;
  if (grid == 0) return hipSuccess;
  const dim3 gd(static_cast<uint32_t>(grid)), bd(ksplit * 64);
  const size_t pt_bytes = static_cast<size_t>(GATED ? 2 : 1) * g.P * sizeof(int32_t);
  switch (ksteps / ksplit) {
#define RIMURU_STREAM_CASE(n) \
    case n: hipLaunchKernelGGL((k_paged_gemm_stream<T, BN, DEPTH, GATED, n>), gd, bd, pt_bytes, st, g, ksplit); break;
    RIMURU_STREAM_CASE(2)
    RIMURU_STREAM_CASE(3)
    RIMURU_STREAM_CASE(4)
    RIMURU_STREAM_CASE(6)
    RIMURU_STREAM_CASE(8)
    RIMURU_STREAM_CASE(12)
    RIMURU_STREAM_CASE(16)
#undef RIMURU_STREAM_CASE
    // other step counts: runtime loop, one step less in flight (register budget)
    default: hipLaunchKernelGGL((k_paged_gemm_stream<T, BN, 2, GATED, 0>), gd, bd, pt_bytes, st, g, ksplit);
  }
  return hipGetLastError();
}

// Few rows per expert: the streaming kernel (16-row tiles). Otherwise tiled
// GEMMs; fp32 tiles take a shorter K step, keeping their LDS footprint near the
// bf16 tiles'. Column tiles are 128 wide when N allows it, else 64 (N is a
// multiple of 64 by validation).
template <typename T, bool GATED>
hipError_t launch_plan(Plan p, const GemmArgs& g, uint64_t tiles_max, hipStream_t st) {
  constexpr bool kF32 = sizeof(T) == 4;
  constexpr int BK_TILE = kF32 ? 16 : 64;
  const bool wide = g.N % 128 == 0;
  switch (p.id) {
    case kPlan16:
      if constexpr (kF32) {
        return launch_stream<T, 64, 3, GATED>(g, tiles_max, st);
      } else {
        // Widest column tile that still yields enough workgroups to keep
        // every CU streaming when only a few experts are touched.
        const int64_t touched = std::min<int64_t>(g.E, g.TK);
        auto enough = [&](int bn, int floor_bn) {
          return g.N % bn == 0 && (bn <= floor_bn || touched * (g.N / bn) >= kStreamNarrow.min_groups);
        };
        if constexpr (GATED) {
          if (enough(kStreamUpBN, kStreamNarrow.up_bn)) return launch_stream<T, kStreamUpBN, kStreamUpDepth, true>(g, tiles_max, st);
          if (enough(64, kStreamNarrow.up_bn)) return launch_stream<T, 64, 3, true>(g, tiles_max, st);
          return launch_stream<T, 32, 3, true>(g, tiles_max, st);
        } else {
          if (enough(kStreamDnBN, kStreamNarrow.dn_bn)) return launch_stream<T, kStreamDnBN, kStreamDnDepth, false>(g, tiles_max, st);
          if (enough(128, kStreamNarrow.dn_bn)) return launch_stream<T, 128, 3, false>(g, tiles_max, st);
          return launch_stream<T, 64, 3, false>(g, tiles_max, st);
        }
      }
    case kPlan64:
      if constexpr (!kF32) {
        constexpr TileShape t = GATED ? kT64Up : kT64Dn;
        if (g.N % t.bn == 0) return launch_gemm<T, 64, t.bn, t.bk, t.wm, t.wn, 4, GATED, t.nbuf>(g, tiles_max, st);
      }
      return wide ? launch_gemm<T, 64, 128, BK_TILE, 2, 2, 4, GATED>(g, tiles_max, st)
                  : launch_gemm<T, 64, 64, BK_TILE, 2, 2, 4, GATED>(g, tiles_max, st);
    default:
      if constexpr (!kF32) {
        constexpr TileShape t = GATED ? kT128Up : kT128Dn;
        if (g.N % t.bn == 0) return launch_gemm<T, 128, t.bn, t.bk, t.wm, t.wn, 8, GATED, t.nbuf>(g, tiles_max, st);
      }
      return wide ? launch_gemm<T, 128, 128, BK_TILE, 2, 2, 8, GATED>(g, tiles_max, st)
                  : launch_gemm<T, 128, 64, BK_TILE, 2, 2, 8, GATED>(g, tiles_max, st);
  }
}

template <typename T>
hipError_t launch_layer(const rimuru_moe_args* a, Plan p, const Layout& lay, hipStream_t st) {
  const int T_ = a->T, E = a->E, k = a->k, H = a->H, I = a->I;
  const int TK = T_ * k;
  uint8_t* ws = static_cast<uint8_t*>(a->workspace);
  int32_t* counts = reinterpret_cast<int32_t*>(ws + lay.off_counts);
  int32_t* tile_expert = reinterpret_cast<int32_t*>(ws + lay.off_tiles);
  uint8_t* h = ws + lay.off_h;
  uint8_t* yslot = ws + lay.off_yslot;
  hipEvent_t* ev = a->stage_events ? reinterpret_cast<hipEvent_t*>(const_cast<void**>(a->stage_events)) : nullptr;
  hipError_t err;
  auto mark = [&](int i) -> hipError_t { return ev ? hipEventRecord(ev[i], st) : hipSuccess; };

  const int epl = (E + 63) / 64;
  if ((err = mark(0)) != hipSuccess) return err;
  {
    dim3 grid((T_ + 3) / 4);
    if (epl <= 1) hipLaunchKernelGGL(k_gating<1>, grid, dim3(256), 0, st, a->logits, T_, E, k, a->topk_ids, a->topk_w);
    else if (epl <= 2) hipLaunchKernelGGL(k_gating<2>, grid, dim3(256), 0, st, a->logits, T_, E, k, a->topk_ids, a->topk_w);
    else if (epl <= 4) hipLaunchKernelGGL(k_gating<4>, grid, dim3(256), 0, st, a->logits, T_, E, k, a->topk_ids, a->topk_w);
    else hipLaunchKernelGGL(k_gating<8>, grid, dim3(256), 0, st, a->logits, T_, E, k, a->topk_ids, a->topk_w);
    if ((err = hipGetLastError()) != hipSuccess) return err;
  }
  if ((err = mark(1)) != hipSuccess) return err;
  const bool self_count = TK <= kSortSelfCountMax;
  if (!self_count) {
    hipLaunchKernelGGL(k_count, dim3(E), dim3(256), 0, st, a->topk_ids, TK, counts);
    if ((err = hipGetLastError()) != hipSuccess) return err;
  }
  if ((err = mark(2)) != hipSuccess) return err;
  hipLaunchKernelGGL(k_sort_align, dim3(E), dim3(256), 0, st, a->topk_ids, TK, E, p.bm,
                     self_count ? nullptr : counts, a->sorted_ids, a->expert_off, tile_expert);
  if ((err = hipGetLastError()) != hipSuccess) return err;

  GemmArgs g{};
  g.sorted_ids = a->sorted_ids;
  g.pool = static_cast<const uint8_t*>(a->pool_base);
  g.pt = a->pt;
  g.P = a->P;
  g.pd = make_div(static_cast<uint32_t>(a->page_bytes));
  g.tile_expert = tile_expert;
  g.expert_off = a->expert_off;
  g.E = E;
  g.topk_w = a->topk_w;
  g.TK = TK;

  if ((err = mark(3)) != hipSuccess) return err;
  g.A = static_cast<const uint8_t*>(a->x);
  g.lda = H;
  g.kdiv = k;
  g.K = H;
  g.N = I;
  g.C = h;
  g.ldc = I;
  if ((err = launch_plan<T, true>(p, g, lay.tiles_max, st)) != hipSuccess) return err;

  if ((err = mark(4)) != hipSuccess) return err;
  g.A = h;
  g.lda = I;
  g.kdiv = 0;
  g.K = I;
  g.N = H;
  g.C = yslot;
  g.ldc = H;
  if ((err = launch_plan<T, false>(p, g, lay.tiles_max, st)) != hipSuccess) return err;

  if ((err = mark(5)) != hipSuccess) return err;
  {
    constexpr int VEC = Elt<T>::VEC;
    dim3 grid(T_, (H + 256 * VEC - 1) / (256 * VEC));
    hipLaunchKernelGGL(k_combine<T>, grid, dim3(256), 0, st, reinterpret_cast<const T*>(yslot), k, H,
                       static_cast<T*>(a->y));
    if ((err = hipGetLastError()) != hipSuccess) return err;
  }
  return mark(6);
}

bool aligned(const void* p, uintptr_t n) { return (reinterpret_cast<uintptr_t>(p) % n) == 0; }

}  // namespace
}  // namespace rimuru

using namespace rimuru;

extern "C" rimuru_status rimuru_moe_sizes(int32_t T, int32_t E, int32_t k, int32_t H, int32_t I,
                                          int32_t P, int32_t dtype, uint64_t* sorted_len,
                                          uint64_t* workspace_bytes, int32_t* block_m) {
  rimuru_status s = check_shapes(T, E, k, H, I, dtype);
  if (s != RIMURU_OK) return s;
  if (P < 1) return rimuru_fail(RIMURU_EINVAL, "P = %d must be at least 1", P);
  Plan p = choose_plan(T, E, k, P);
  Layout l = layout_for(T, E, k, H, I, dtype == RIMURU_BF16 ? 2 : 4, p.bm);
  if (sorted_len) *sorted_len = l.sorted_len;
  if (workspace_bytes) *workspace_bytes = l.total;
  if (block_m) *block_m = p.bm;
  return RIMURU_OK;
}

extern "C" rimuru_status rimuru_fused_moe_paged(const rimuru_moe_args* a, void* hip_stream) {
  if (a == nullptr) return rimuru_fail(RIMURU_EINVAL, "fused_moe_paged: args is NULL");
  rimuru_status s = check_shapes(a->T, a->E, a->k, a->H, a->I, a->dtype);
  if (s != RIMURU_OK) return s;
  if (a->renormalize != 1)
    return rimuru_fail(RIMURU_EINVAL, "renormalize must be 1 (the kept top-k weights sum to one)");
  if (a->T == 0) return RIMURU_OK;
  const int es = a->dtype == RIMURU_BF16 ? 2 : 4;
  const uint64_t proj = static_cast<uint64_t>(a->H) * a->I * es;
  if (a->page_bytes == 0 || a->page_bytes % 128 != 0)
    return rimuru_fail(RIMURU_EINVAL, "page_bytes %llu is not a positive multiple of 128",
                       (unsigned long long)a->page_bytes);
  if (a->P < 1 || static_cast<uint64_t>(a->P) * a->page_bytes < proj)
    return rimuru_fail(RIMURU_EINVAL, "P = %d pages of %llu bytes cannot hold a %llu-byte projection",
                       a->P, (unsigned long long)a->page_bytes, (unsigned long long)proj);
  if (static_cast<uint64_t>(a->P) * a->page_bytes >= (1ull << 31))
    return rimuru_fail(RIMURU_EINVAL, "a projection's pages must span less than 2 GiB");
  if (!a->x || !a->logits || !a->pool_base || !a->pt || !a->y || !a->topk_ids || !a->topk_w ||
      !a->sorted_ids || !a->expert_off || !a->workspace)
    return rimuru_fail(RIMURU_EINVAL, "fused_moe_paged: a required pointer is NULL");
  if (!aligned(a->pool_base, 256) || !aligned(a->workspace, 256) || !aligned(a->x, 16) ||
      !aligned(a->y, 16) || !aligned(a->topk_ids, 16))
    return rimuru_fail(RIMURU_EINVAL, "pool_base/workspace need 256-byte and x/y/topk_ids 16-byte alignment");
  Plan p = choose_plan(a->T, a->E, a->k, a->P);
  Layout lay = layout_for(a->T, a->E, a->k, a->H, a->I, es, p.bm);
  if (a->workspace_bytes < lay.total)
    return rimuru_fail(RIMURU_EINVAL, "workspace of %llu bytes is below the %llu needed",
                       (unsigned long long)a->workspace_bytes, (unsigned long long)lay.total);
  if ((a->stage_events == nullptr) != (a->n_stage_events == 0) ||
      (a->stage_events && a->n_stage_events != RIMURU_MOE_STAGES + 1))
    return rimuru_fail(RIMURU_EINVAL, "stage_events needs exactly %d events", RIMURU_MOE_STAGES + 1);
  hipStream_t st = static_cast<hipStream_t>(hip_stream);
  hipError_t err = (a->dtype == RIMURU_BF16) ? launch_layer<uint16_t>(a, p, lay, st)
                                             : launch_layer<float>(a, p, lay, st);
  if (err != hipSuccess) return rimuru_fail(RIMURU_EHIP, "launch failed: %s", hipGetErrorString(err));
  return RIMURU_OK;
}

extern "C" rimuru_status rimuru_pt_check(const int32_t* pt_host, int32_t E, int32_t P,
                                         uint64_t page_bytes, uint64_t pool_bytes) {
  if (pt_host == nullptr || E < 1 || P < 1 || page_bytes == 0)
    return rimuru_fail(RIMURU_EINVAL, "pt_check: bad argument");
  const uint64_t n = static_cast<uint64_t>(E) * 3 * P;
  for (uint64_t i = 0; i < n; ++i) {
    if (pt_host[i] < 0 || (static_cast<uint64_t>(pt_host[i]) + 1) * page_bytes > pool_bytes)
      return rimuru_fail(RIMURU_ERANGE, "pt entry %llu (expert %llu, projection %llu, page %llu) = %d "
                         "lies outside the pool", (unsigned long long)i,
                         (unsigned long long)(i / (3ull * P)), (unsigned long long)(i / P % 3),
                         (unsigned long long)(i % P), pt_host[i]);
  }
  return RIMURU_OK;
}

extern "C" rimuru_status rimuru_experts_store(void* pool_base, const int32_t* pt, int32_t E, int32_t P,
                                              uint64_t page_bytes, const void* src,
                                              uint64_t proj_bytes, void* hip_stream) {
  if (!pool_base || !pt || !src || E < 1 || P < 1)
    return rimuru_fail(RIMURU_EINVAL, "experts_store: bad argument");
  if (page_bytes == 0 || page_bytes % 128 != 0 || proj_bytes == 0 || proj_bytes % 16 != 0 ||
      proj_bytes > static_cast<uint64_t>(P) * page_bytes ||
      static_cast<uint64_t>(P) * page_bytes >= (1ull << 31))
    return rimuru_fail(RIMURU_EINVAL, "experts_store: page %llu / projection %llu bytes / P %d do not fit",
                       (unsigned long long)page_bytes, (unsigned long long)proj_bytes, P);
  if (!aligned(pool_base, 256) || !aligned(src, 16))
    return rimuru_fail(RIMURU_EINVAL, "experts_store: pool_base needs 256-byte, src 16-byte alignment");
  uint64_t n_segs = static_cast<uint64_t>(E) * 3 * proj_bytes / 16;
  uint64_t blocks = (n_segs + 255) / 256;
  if (blocks > 65536) blocks = 65536;
  hipLaunchKernelGGL(k_store_pages, dim3(static_cast<uint32_t>(blocks)), dim3(256), 0,
                     static_cast<hipStream_t>(hip_stream), static_cast<uint8_t*>(pool_base), pt, P,
                     make_div(static_cast<uint32_t>(page_bytes)), static_cast<const uint8_t*>(src),
                     proj_bytes, n_segs);
  hipError_t err = hipGetLastError();
  if (err != hipSuccess) return rimuru_fail(RIMURU_EHIP, "experts_store: %s", hipGetErrorString(err));
  return RIMURU_OK;
}

extern "C" rimuru_status rimuru_event_create(void** ev) {
  if (!ev) return rimuru_fail(RIMURU_EINVAL, "event_create: NULL");
  hipEvent_t e;
  hipError_t err = hipEventCreate(&e);
  if (err != hipSuccess) return rimuru_fail(RIMURU_EHIP, "hipEventCreate: %s", hipGetErrorString(err));
  *ev = e;
  return RIMURU_OK;
}

extern "C" rimuru_status rimuru_event_destroy(void* ev) {
  if (!ev) return RIMURU_OK;
  hipError_t err = hipEventDestroy(static_cast<hipEvent_t>(ev));
  if (err != hipSuccess) return rimuru_fail(RIMURU_EHIP, "hipEventDestroy: %s", hipGetErrorString(err));
  return RIMURU_OK;
}

extern "C" rimuru_status rimuru_event_record(void* ev, void* hip_stream) {
  hipError_t err = hipEventRecord(static_cast<hipEvent_t>(ev), static_cast<hipStream_t>(hip_stream));
  if (err != hipSuccess) return rimuru_fail(RIMURU_EHIP, "hipEventRecord: %s", hipGetErrorString(err));
  return RIMURU_OK;
}

extern "C" rimuru_status rimuru_event_elapsed_ms(void* start, void* stop, float* ms) {
  if (!start || !stop || !ms) return rimuru_fail(RIMURU_EINVAL, "event_elapsed_ms: NULL");
  hipError_t err = hipEventSynchronize(static_cast<hipEvent_t>(stop));
  if (err == hipSuccess) err = hipEventElapsedTime(ms, static_cast<hipEvent_t>(start), static_cast<hipEvent_t>(stop));
  if (err != hipSuccess) return rimuru_fail(RIMURU_EHIP, "event timing: %s", hipGetErrorString(err));
  return RIMURU_OK;
}
