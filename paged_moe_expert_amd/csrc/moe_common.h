// Device helpers and host launchers shared by the fused-MoE translation units.
//
// Rimuru paper summary (thelatestinai.com), abstract: a fused MoE kernel that
// reads non-contiguous expert weights directly through the expert view's page
// table, so no expert is ever copied into a contiguous buffer; Figure 11 names
// it "Discrete FusedMoE". Table 1 of the summary gives the three projections
// per expert (w1, w3 [H, I], w2 [I, H]).
//
// Every 16-byte weight segment a lane loads gets its own page lookup
// (page = offset / page_bytes by multiply-shift, then the page table); a
// segment never straddles a page because pages are multiples of 128 bytes and
// segments start on 16-byte boundaries. Results do not depend on where the
// pages sit, so the paged and the contiguous layouts give identical bits.
#pragma once

#include <hip/hip_runtime.h>

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

// Two fp32 values -> packed bf16 pair (lo in bits 15:0), round to nearest even,
// by the hardware conversion (v_cvt_pk_bf16_f32).
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2_t{lo, hi}, bf16x2_t));
}

// Value of lane l ^ 1 (a DPP quad permutation, no LDS traffic).
__device__ __forceinline__ float swap_lane_pair(float v) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0xB1, 0xF, 0xF, false));
}

// ---------------------------------------------------------------- asynchronous copies and waits

// vmcnt <= N (gfx9 encoding: vmcnt in bits 3:0 and 15:14; expcnt and lgkmcnt
// left at their "no wait" values).
template <int N>
__device__ __forceinline__ void wait_vmem() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | (7 << 4) | (15 << 8) | ((N >> 4) << 14));
}

// lgkmcnt = 0 (LDS reads issued so far have returned).
__device__ __forceinline__ void wait_lds() { __builtin_amdgcn_s_waitcnt(0xC07F); }

// Workgroup barrier without the memory fence of __syncthreads (which waits for
// every load in flight, including the prefetched stages): callers wait for
// exactly the loads they need first. The empty asm statements keep the
// compiler from moving memory accesses across it.
__device__ __forceinline__ void barrier_only() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

// Asynchronous 16-byte-per-lane copy global -> LDS (global_load_lds_dwordx4):
// lane l's 16 bytes land at LDS byte address lds + 16*l; lds must be
// wavefront-uniform. Issued through asm so the compiler does not order LDS
// reads after it (it would wait for every copy in flight); callers wait with
// wait_vmem. M0 is restored afterwards.
__device__ __forceinline__ void copy_to_lds16(const void* g, uint32_t lds) {
  uint32_t saved;
  asm volatile(
      "s_mov_b32 %0, m0\n\t"
      "s_mov_b32 m0, %2\n\t"
      "global_load_lds_dwordx4 %1, off\n\t"
      "s_mov_b32 m0, %0"
      : "=&s"(saved)
      : "v"(g), "s"(lds)
      : "memory");
}

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

// ---------------------------------------------------------------- grouped GEMM arguments

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

// ---------------------------------------------------------------- host launchers

PageDiv make_div(uint32_t page);

// The router projection run in the gating stage instead of taking given
// logits: x [T, H] and w_gate [E, H] in the layer's dtype; the logits [T, E]
// fp32 go to logits_out (caller memory, or the layer's workspace).
struct RouterArgs {
  const void* x;
  const void* w_gate;
  int H;
  bool bf16;
  float* logits_out;
};

// Slot-list ranges the count and sort of many routed slots are cut into (the
// counts buffer holds E * kCountSplits entries).
constexpr int kCountSplits = 8;

// Routing (gating top-k, per-expert sort padded to bm-row tiles) on stream st;
// counts/tile_expert live in the workspace. router == null: top-k of the given
// logits; else the logits are computed from x and w_gate first. Stage marks 1
// and 2 are recorded between the kernels when ev is not null.
hipError_t launch_routing(const float* logits, const RouterArgs* router, int T, int E, int k, int bm,
                          int32_t* topk_ids, float* topk_w, int32_t* counts, int32_t* sorted_ids,
                          int32_t* expert_off, int32_t* tile_expert, hipEvent_t* ev, hipStream_t st);

// y[t] = sum_j y_slot[t*k+j] (fixed j order)
template <typename T>
hipError_t launch_combine(const T* yslot, int T_, int k, int H, T* y, hipStream_t st);

hipError_t launch_stream_read(const void* buf, uint64_t bytes, uint32_t* sink, hipStream_t st);
hipError_t launch_store_pages(uint8_t* pool, uint64_t pool_bytes, const int32_t* pt, int P, uint32_t page_bytes,
                              const uint8_t* src, uint64_t proj_bytes, uint64_t n_segs, hipStream_t st);

// Page-table entries a streaming workgroup stages in LDS (both gated matrices).
constexpr int kStreamPtMax = 4096;

// Few rows per expert (bm = 16, or 32 for bf16): weight-streaming GEMM.
template <typename T, bool GATED>
hipError_t launch_streamed(int bm, const GemmArgs& g, uint64_t tiles_max, hipStream_t st);

// Many rows per expert, bf16, 64- or 128-row tiles: the persistent pipelined
// GEMM; hipErrorNotSupported when the shape is outside what it covers.
template <bool GATED>
hipError_t launch_prefill(int bm, const GemmArgs& g, uint64_t tiles_max, hipStream_t st);

// Many rows per expert (bm = 64 or 128): tiled MFMA GEMM.
template <typename T, bool GATED>
hipError_t launch_tiled(int bm, const GemmArgs& g, uint64_t tiles_max, hipStream_t st);

}  // namespace rimuru
