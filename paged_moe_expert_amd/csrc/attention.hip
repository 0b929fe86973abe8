// Paged decode attention over the KV view of the shared page pool.
//
// Rimuru explainer "Rimuru unifies serving memory" (learnaivisually.com),
// paragraph on moving the fence: KV blocks of 16 tokens reached through a
// block table (PagedAttention's idea) are cut from expert-sized pages of the
// same pool the experts live in. Paper summary (thelatestinai.com), Table 1:
// one token's K and V are [2, n_kv_heads, head_dim] ([2, 4, 128] for
// Qwen3-30B-A3B, [2, 2, 256] for Qwen3.5-35B-A3B).
//
// Block layout (the pages fix none; stated in rimuru.h): K of every KV head
// token-major [16][D], then V of every KV head dim-major [D][16].
//
// One workgroup = one request, one KV head, one range of blocks (a split);
// its 4 wavefronts take the range's blocks in turn, two at a time. All G
// query heads of the KV head share each K/V read (grouped-query attention):
//   S^T[t][h] = K[t] . q[h]       v_mfma_f32_16x16x32_bf16, A = K rows, B = q
//   O^T[d][h] += V^T[d][t] P[h][t] v_mfma_f32_16x16x16_bf16, A = V^T rows, B = P^T
// S^T's output layout (head = lane % 16, tokens 4*(lane/16) + r) is exactly
// the B operand the second product needs, and O^T keeps the head on lane % 16
// too, so the online-softmax state of head h lives on the lanes h, h+16,
// h+32, h+48 and rescaling needs no data movement. G < 16 pads q with zeros.
// Splits write unnormalised partials (O, m, l); a second kernel merges them.
// With a single split the first kernel normalises and writes the output.
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdint>

#include "moe_common.h"

namespace rimuru {
namespace {

constexpr int kBT = 16;        // tokens per KV block
constexpr int kWaves = 4;
constexpr int kMinWorkgroups = 1024;
constexpr int kMaxChunk = 1024;  // blocks per split: the split's block-table slice fits LDS
constexpr int kRound = 2;        // blocks a wavefront loads per round

__device__ __forceinline__ float wave_shfl_xor(float v, int m) {
  return __shfl_xor(v, m, 64);
}

template <int D>
struct AttnFrags {
  u32x4 k[D / 32];   // K rows: token lane%16, dims 32c + 8(lane/16) .. +7
  u32x2 v[D / 16];   // V^T rows: dim 16c + lane%16, tokens 4(lane/16) .. +3
};

template <int D>
__device__ __forceinline__ void load_block(AttnFrags<D>& f, const uint8_t* blk, int j, int n_kv, int lane) {
  const int i16 = lane & 15, g4 = lane >> 4;
  const uint16_t* kp = reinterpret_cast<const uint16_t*>(blk) + (j * kBT + i16) * D + 8 * g4;
#pragma unroll
  for (int c = 0; c < D / 32; ++c) f.k[c] = *reinterpret_cast<const u32x4*>(kp + 32 * c);
  const uint16_t* vp = reinterpret_cast<const uint16_t*>(blk) + n_kv * kBT * D + (j * D + i16) * kBT + 4 * g4;
#pragma unroll
  for (int c = 0; c < D / 16; ++c) f.v[c] = *reinterpret_cast<const u32x2*>(vp + 16 * kBT * c);
}

template <int D>
struct SoftmaxState {
  float m;            // running max (log2 domain) of head lane%16
  float l;            // this lane's share of the running denominator
  f32x4 o[D / 16];    // O^T: dims 16c + 4(lane/16) + r, head lane%16
};

template <int D>
__device__ __forceinline__ void attend_block(SoftmaxState<D>& st, const AttnFrags<D>& f, const u32x4 (&qf)[D / 32],
                                             int tok0, int L, float scale_log2, int lane) {
  f32x4 s = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int c = 0; c < D / 32; ++c) s = Elt<uint16_t>::mma(f.k[c], qf[c], s);
  const int t0 = tok0 + 4 * (lane >> 4);
  float mb = -INFINITY;
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    s[r] = (t0 + r < L) ? s[r] * scale_log2 : -INFINITY;
    mb = fmaxf(mb, s[r]);
  }
  mb = fmaxf(mb, wave_shfl_xor(mb, 16));
  mb = fmaxf(mb, wave_shfl_xor(mb, 32));
  const float mn = fmaxf(st.m, mb);      // finite: the block holds a valid token
  const float alpha = exp2f(st.m - mn);   // 0 on the first block (m = -inf)
  float p[4], ps = 0.f;
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    p[r] = exp2f(s[r] - mn);
    ps += p[r];
  }
  st.l = st.l * alpha + ps;
  st.m = mn;
  const u32x2 pb = {pack_bf16x2(p[0], p[1]), pack_bf16x2(p[2], p[3])};
  const v4i16 pv = __builtin_bit_cast(v4i16, pb);
  // V values of tokens at or past the context end are selected to zero, not
  // multiplied by p = 0: the tail of a request's last block holds whatever
  // the page held before (pages move between tensor types), and a NaN there
  // times zero would still be NaN. This lane's V values are tokens t0 .. t0+3,
  // token r in bits 16(r%2) of word r/2.
  const u32x2 vmask = {(t0 < L ? 0x0000ffffu : 0u) | (t0 + 1 < L ? 0xffff0000u : 0u),
                       (t0 + 2 < L ? 0x0000ffffu : 0u) | (t0 + 3 < L ? 0xffff0000u : 0u)};
#pragma unroll
  for (int c = 0; c < D / 16; ++c) {
    f32x4 o = st.o[c] * alpha;
    const u32x2 vv = f.v[c] & vmask;
    st.o[c] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(__builtin_bit_cast(v4i16, vv), pv, o, 0, 0, 0);
  }
}

template <int D>
__global__ __launch_bounds__(kWaves * 64) void k_paged_attn(const uint16_t* __restrict__ q,
                                                            const uint8_t* __restrict__ pool,
                                                            const int32_t* __restrict__ block_table,
                                                            const int32_t* __restrict__ ctx_lens, int n_q,
                                                            int n_kv, int max_blocks, int chunk, int n_split,
                                                            float scale_log2, float* __restrict__ part_o,
                                                            float* __restrict__ part_ml,
                                                            uint16_t* __restrict__ out) {
  const int split = blockIdx.x, j = blockIdx.y, b = blockIdx.z;
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int G = n_q / n_kv;
  const int L = min(max(ctx_lens[b], 0), max_blocks * kBT);
  const int nblk = (L + kBT - 1) / kBT;
  const int blk0 = split * chunk, blk1 = min(blk0 + chunk, nblk);
  if (blk0 >= blk1) {             // nothing of this request in this split
    if (out != nullptr) {         // one split: an empty context gives zeros
      uint16_t* o = out + (static_cast<int64_t>(b) * n_q + j * G) * D;
      for (int i = threadIdx.x; i < G * D; i += kWaves * 64) o[i] = 0;
    }
    return;
  }
  const uint64_t bbytes = static_cast<uint64_t>(2) * n_kv * kBT * D * 2;
  const int32_t* bt = block_table + static_cast<int64_t>(b) * max_blocks;

  // q rows of the group as the B operand (zeros for padded heads)
  const int h = lane & 15;
  u32x4 qf[D / 32];
  {
    const uint16_t* qp = q + (static_cast<int64_t>(b) * n_q + j * G + min(h, G - 1)) * D + 8 * (lane >> 4);
#pragma unroll
    for (int c = 0; c < D / 32; ++c) {
      const u32x4 v = *reinterpret_cast<const u32x4*>(qp + 32 * c);
      qf[c] = (h < G) ? v : u32x4{0u, 0u, 0u, 0u};
    }
  }
  SoftmaxState<D> st;
  st.m = -INFINITY;
  st.l = 0.f;
#pragma unroll
  for (int c = 0; c < D / 16; ++c) st.o[c] = f32x4{0.f, 0.f, 0.f, 0.f};

  // The split's block indices, staged in LDS once: a block's address is then
  // an LDS read away instead of a dependent global load per round.
  __shared__ int32_t sbt[kMaxChunk];
  for (int i = threadIdx.x; i < blk1 - blk0; i += kWaves * 64) sbt[i] = bt[blk0 + i];
  __syncthreads();

  // blocks blk0 + w, + 4, ... kRound per round, all loaded before the first
  // is multiplied; a block past the range re-reads the round's first and is
  // skipped
  for (int i = blk0 + w; i < blk1; i += kRound * kWaves) {
    AttnFrags<D> f[kRound];
#pragma unroll
    for (int u = 0; u < kRound; ++u) {
      const int iu = i + u * kWaves < blk1 ? i + u * kWaves : i;
      load_block<D>(f[u], pool + static_cast<uint64_t>(sbt[iu - blk0]) * bbytes, j, n_kv, lane);
    }
    attend_block<D>(st, f[0], qf, i * kBT, L, scale_log2, lane);
#pragma unroll
    for (int u = 1; u < kRound; ++u)
      if (i + u * kWaves < blk1) attend_block<D>(st, f[u], qf, (i + u * kWaves) * kBT, L, scale_log2, lane);
  }
  st.l += wave_shfl_xor(st.l, 16);
  st.l += wave_shfl_xor(st.l, 32);

  // merge the wavefronts: waves 1..3 leave their registers in LDS as they
  // are (lane-major, conflict-free), wave 0 folds them into its own
  __shared__ f32x4 so[kWaves - 1][D / 16][64];
  __shared__ float sm[kWaves - 1][64], sl[kWaves - 1][64];
  if (w > 0) {
#pragma unroll
    for (int c = 0; c < D / 16; ++c) so[w - 1][c][lane] = st.o[c];
    sm[w - 1][lane] = st.m;
    sl[w - 1][lane] = st.l;
  }
  __syncthreads();
  if (w != 0) return;
  float M = st.m;                 // finite: wave 0 holds the split's first block
#pragma unroll
  for (int v = 0; v < kWaves - 1; ++v) M = fmaxf(M, sm[v][lane]);
  const float a0 = exp2f(st.m - M);
  float l = st.l * a0;
#pragma unroll
  for (int c = 0; c < D / 16; ++c) st.o[c] = st.o[c] * a0;
#pragma unroll
  for (int v = 0; v < kWaves - 1; ++v) {
    const float mv = sm[v][lane];
    const float av = (mv == -INFINITY) ? 0.f : exp2f(mv - M);   // a wave without blocks adds nothing
    l += av * sl[v][lane];
#pragma unroll
    for (int c = 0; c < D / 16; ++c) st.o[c] += av * so[v][c][lane];
  }
  if (out != nullptr) {
    // one split: normalise and write the output here (the merge kernel would
    // scale by 2^0 = 1 and divide the same values)
    if (h < G) {
      uint16_t* po = out + (static_cast<int64_t>(b) * n_q + j * G + h) * D + 4 * (lane >> 4);
#pragma unroll
      for (int c = 0; c < D / 16; ++c)
#pragma unroll
        for (int r = 0; r < 4; ++r) po[16 * c + r] = static_cast<uint16_t>(f32_to_bf16(st.o[c][r] / l));
    }
    return;
  }
  if (h < G) {
    const int64_t r = ((static_cast<int64_t>(b) * n_q + j * G + h) * n_split + split);
    float* po = part_o + r * D + 4 * (lane >> 4);
#pragma unroll
    for (int c = 0; c < D / 16; ++c) *reinterpret_cast<f32x4*>(po + 16 * c) = st.o[c];
    if (lane < 16) {
      part_ml[2 * r] = M;
      part_ml[2 * r + 1] = l;
    }
  }
}

// out[b, h] = sum_s 2^(m_s - M) O_s / sum_s 2^(m_s - M) l_s over the splits
// that hold blocks of the request; zeros for an empty context.
template <int D>
__global__ __launch_bounds__(D) void k_attn_merge(const float* __restrict__ part_o, const float* __restrict__ part_ml,
                                                  const int32_t* __restrict__ ctx_lens, int n_q, int max_blocks,
                                                  int chunk, int n_split, uint16_t* __restrict__ out) {
  const int row = blockIdx.x, b = row / n_q, d = threadIdx.x;
  const int L = min(max(ctx_lens[b], 0), max_blocks * kBT);
  const int ns = min(n_split, ((L + kBT - 1) / kBT + chunk - 1) / chunk);
  float M = -INFINITY;
  for (int s = 0; s < ns; ++s) M = fmaxf(M, part_ml[2 * (static_cast<int64_t>(row) * n_split + s)]);
  float o = 0.f, l = 0.f;
  for (int s = 0; s < ns; ++s) {
    const int64_t r = static_cast<int64_t>(row) * n_split + s;
    const float a = exp2f(part_ml[2 * r] - M);
    o += a * part_o[r * D + d];
    l += a * part_ml[2 * r + 1];
  }
  out[static_cast<int64_t>(row) * D + d] = static_cast<uint16_t>(f32_to_bf16(ns > 0 ? o / l : 0.f));
}

int pick_split(int B, int n_kv, int max_blocks) {
  const int64_t pairs = static_cast<int64_t>(B) * n_kv;
  if (pairs == 0) return 1;
  int ns = static_cast<int>((kMinWorkgroups + pairs - 1) / pairs);
  const int most = (max_blocks + kRound * kWaves - 1) / (kRound * kWaves);   // at least one round per wavefront
  if (ns > most) ns = most;
  const int fewest = (max_blocks + kMaxChunk - 1) / kMaxChunk;     // each split's table fits LDS
  if (ns < fewest) ns = fewest;
  return ns < 1 ? 1 : ns;
}

template <int D>
hipError_t launch_attn(const rimuru_attn_args* a, int n_split, hipStream_t st) {
  const int chunk = (a->max_blocks + n_split - 1) / n_split;
  float* part_o = static_cast<float*>(a->workspace);
  float* part_ml = part_o + static_cast<int64_t>(a->B) * a->n_q * n_split * D;
  const float scale_log2 = a->scale * 1.4426950408889634f;
  hipLaunchKernelGGL(k_paged_attn<D>, dim3(n_split, a->n_kv, a->B), dim3(kWaves * 64), 0, st,
                     static_cast<const uint16_t*>(a->q), static_cast<const uint8_t*>(a->pool_base),
                     a->block_table, a->context_lens, a->n_q, a->n_kv, a->max_blocks, chunk, n_split,
                     scale_log2, part_o, part_ml, n_split == 1 ? static_cast<uint16_t*>(a->out) : nullptr);
  hipError_t err = hipGetLastError();
  if (err != hipSuccess || n_split == 1) return err;
  hipLaunchKernelGGL(k_attn_merge<D>, dim3(a->B * a->n_q), dim3(D), 0, st, part_o, part_ml, a->context_lens,
                     a->n_q, a->max_blocks, chunk, n_split, static_cast<uint16_t*>(a->out));
  return hipGetLastError();
}

rimuru_status attn_shape(int32_t B, int32_t n_q, int32_t n_kv, int32_t head_dim, int32_t max_blocks) {
  if (B < 0 || n_kv < 1 || n_q < n_kv || n_q % n_kv != 0 || n_q / n_kv > 16)
    return rimuru_fail(RIMURU_EINVAL, "attention: need n_q a multiple of n_kv with at most 16 query heads per KV head");
  if (head_dim != 128 && head_dim != 256)
    return rimuru_fail(RIMURU_EINVAL, "attention: head_dim %d (128 or 256)", head_dim);
  if (max_blocks < 1) return rimuru_fail(RIMURU_EINVAL, "attention: max_blocks must be >= 1");
  return RIMURU_OK;
}

}  // namespace
}  // namespace rimuru

using namespace rimuru;

extern "C" rimuru_status rimuru_attn_sizes(int32_t B, int32_t n_q, int32_t n_kv, int32_t head_dim,
                                           int32_t max_blocks, uint64_t* workspace_bytes, int32_t* n_split,
                                           uint64_t* block_bytes) {
  const rimuru_status s = attn_shape(B, n_q, n_kv, head_dim, max_blocks);
  if (s != RIMURU_OK) return s;
  const int ns = pick_split(B, n_kv, max_blocks);
  const uint64_t rows = static_cast<uint64_t>(B) * n_q * ns;
  if (workspace_bytes) *workspace_bytes = rows * (head_dim + 2) * 4;
  if (n_split) *n_split = ns;
  if (block_bytes) *block_bytes = static_cast<uint64_t>(2) * n_kv * kBT * head_dim * 2;
  return RIMURU_OK;
}

extern "C" rimuru_status rimuru_paged_decode_attention(const rimuru_attn_args* a, void* hip_stream) {
  if (a == nullptr) return rimuru_fail(RIMURU_EINVAL, "attention: NULL args");
  rimuru_status s = attn_shape(a->B, a->n_q, a->n_kv, a->head_dim, a->max_blocks);
  if (s != RIMURU_OK) return s;
  if (a->B == 0) return RIMURU_OK;
  if (a->q == nullptr || a->pool_base == nullptr || a->block_table == nullptr || a->context_lens == nullptr ||
      a->out == nullptr || a->workspace == nullptr)
    return rimuru_fail(RIMURU_EINVAL, "attention: NULL pointer");
  auto aligned = [](const void* p, uintptr_t n) { return reinterpret_cast<uintptr_t>(p) % n == 0; };
  if (!aligned(a->q, 16) || !aligned(a->pool_base, 256) || !aligned(a->workspace, 16) || !aligned(a->out, 2))
    return rimuru_fail(RIMURU_EINVAL, "attention: q/workspace need 16-byte, pool_base 256-byte alignment");
  if (!(a->scale > 0.f) || !std::isfinite(a->scale))
    return rimuru_fail(RIMURU_EINVAL, "attention: scale must be positive and finite");
  uint64_t need = 0;
  int32_t ns = 0;
  rimuru_attn_sizes(a->B, a->n_q, a->n_kv, a->head_dim, a->max_blocks, &need, &ns, nullptr);
  if (a->workspace_bytes < need)
    return rimuru_fail(RIMURU_EINVAL, "attention: workspace of %llu bytes, %llu needed",
                       (unsigned long long)a->workspace_bytes, (unsigned long long)need);
  hipStream_t st = static_cast<hipStream_t>(hip_stream);
  const hipError_t err = a->head_dim == 128 ? launch_attn<128>(a, ns, st) : launch_attn<256>(a, ns, st);
  if (err != hipSuccess) return rimuru_fail(RIMURU_EHIP, "attention: launch failed: %s", hipGetErrorString(err));
  return RIMURU_OK;
}

extern "C" rimuru_status rimuru_block_table_check(const int32_t* table, int32_t B, int32_t max_blocks,
                                                  const int32_t* context_lens, uint64_t block_bytes,
                                                  uint64_t pool_bytes) {
  if (table == nullptr || context_lens == nullptr || B < 0 || max_blocks < 1 || block_bytes == 0)
    return rimuru_fail(RIMURU_EINVAL, "block_table_check: bad argument");
  const uint64_t n_blocks = pool_bytes / block_bytes;
  for (int32_t b = 0; b < B; ++b) {
    const int32_t L = context_lens[b];
    if (L < 0 || L > max_blocks * kBT)
      return rimuru_fail(RIMURU_ERANGE, "block_table_check: context_lens[%d] = %d outside [0, %d]", b, L,
                         max_blocks * kBT);
    for (int32_t i = 0; i < (L + kBT - 1) / kBT; ++i) {
      const int32_t v = table[static_cast<int64_t>(b) * max_blocks + i];
      if (v < 0 || static_cast<uint64_t>(v) >= n_blocks)
        return rimuru_fail(RIMURU_ERANGE, "block_table_check: block_table[%d][%d] = %d outside [0, %llu)", b, i, v,
                           (unsigned long long)n_blocks);
    }
  }
  return RIMURU_OK;
}
