// The fused MoE layer's C entry points: validation, tile plan, workspace
// layout and the six stages enqueued on the caller's stream, no host sync
// (Rimuru paper summary, abstract and Figure 11, "Discrete FusedMoE").
//
//   1 gating     top-k on raw logits, softmax over the kept logits
//   2 count      routed slots per expert (skipped for small batches: the sort
//                kernel counts for itself)
//   3 sort       stable per-expert slot lists padded to the tile height
//   4 gemm-up    h = SiLU(x w1) * (x w3), w1/w3 read through the page table
//   5 gemm-down  y_slot[t*k+j] = w[t,j] * (h w2), w2 through the page table
//   6 combine    y[t] = sum_j y_slot[t*k+j], j in rank order
#include <atomic>
#include <mutex>

#include "moe_common.h"
#include "moe_topk.h"

namespace rimuru {
namespace {

constexpr uint64_t kAlign = 256;
inline uint64_t align_up(uint64_t x) { return (x + kAlign - 1) / kAlign * kAlign; }

// Tile height by expected rows per expert (T*k/E): few rows per expert is a
// weight stream (decode), many rows is a dense grouped GEMM (prefill).
enum PlanId { kPlan16 = 0, kPlan64 = 1, kPlan128 = 2, kPlan32 = 3 };
struct Plan {
  PlanId id;
  int bm;
};

#ifndef RIMURU_PLAN64_MAX_ROWS
#define RIMURU_PLAN64_MAX_ROWS 160
#endif
// Weight streaming up to 24 rows per expert: 16-row tiles up to 8 (most
// experts one tile), bf16 32-row tiles above (an expert with 9 to 32 rows
// still one tile, its weights read once: 256-token decode layer, 16 rows an
// expert on average, half of the experts past 16).
Plan choose_plan(int64_t T, int E, int k, int64_t P, int dtype) {
  int64_t tk = T * k;
  if (tk <= 24ll * E && 2 * P <= kStreamPtMax) {
#ifndef RIMURU_PLAN32_MIN_ROWS
#define RIMURU_PLAN32_MIN_ROWS 8
#endif
    if (dtype == RIMURU_BF16 && tk > static_cast<int64_t>(RIMURU_PLAN32_MIN_ROWS) * E) return {kPlan32, 32};
    return {kPlan16, 16};
  }
  if (tk <= static_cast<int64_t>(RIMURU_PLAN64_MAX_ROWS) * E) return {kPlan64, 64};
  return {kPlan128, 128};
}

struct Layout {
  uint64_t tiles_max, sorted_len;
  uint64_t off_counts, off_tiles, off_logits, off_h, off_yslot, total;
};

Layout layout_for(int64_t T, int E, int k, int H, int I, int es, int bm) {
  Layout l;
  int64_t tk = T * k;
  l.tiles_max = static_cast<uint64_t>(tk / bm + (tk < E ? tk : E));
  l.sorted_len = l.tiles_max * bm;
  l.off_counts = 0;
  l.off_tiles = align_up(static_cast<uint64_t>(E) * kCountSplits * 4);   // counts [E][splits]
  l.off_logits = l.off_tiles + align_up(l.tiles_max * 4);        // router logits [T, E] fp32
  l.off_h = l.off_logits + align_up(static_cast<uint64_t>(T) * E * 4);
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

template <typename T>
hipError_t launch_layer(const rimuru_moe_args* a, const RouterArgs* router, Plan p, const Layout& lay,
                        hipStream_t st) {
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
  auto gemm = [&](bool gated, const GemmArgs& g) -> hipError_t {
    if (p.id == kPlan16 || p.id == kPlan32)
      return gated ? launch_streamed<T, true>(p.bm, g, lay.tiles_max, st)
                   : launch_streamed<T, false>(p.bm, g, lay.tiles_max, st);
    return gated ? launch_tiled<T, true>(p.bm, g, lay.tiles_max, st)
                 : launch_tiled<T, false>(p.bm, g, lay.tiles_max, st);
  };

  // a tiny batch on 16-row tiles with given logits: the gate/up stream
  // routes it itself (one launch less); its time then counts as gate/up
  const bool routed = p.id == kPlan16 && router == nullptr &&
                      streamed_routed_fits(static_cast<int>(sizeof(T)), T_, k, E, H, lay.tiles_max);
  if ((err = mark(0)) != hipSuccess) return err;
  if (routed) {
    if ((err = mark(1)) != hipSuccess || (err = mark(2)) != hipSuccess) return err;
  } else if ((err = launch_routing(a->logits, router, T_, E, k, p.bm, a->topk_ids, a->topk_w, counts, a->sorted_ids,
                                   a->expert_off, tile_expert, ev, st)) != hipSuccess) {
    return err;
  }

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
  if (routed) {
    const TinyRoute rt{a->logits, T_, k, a->topk_ids, a->topk_w, a->sorted_ids, a->expert_off, tile_expert};
    if ((err = launch_streamed_routed<T>(g, lay.tiles_max, rt, st)) != hipSuccess) return err;
  } else if ((err = gemm(true, g)) != hipSuccess) {
    return err;
  }

  if ((err = mark(4)) != hipSuccess) return err;
  g.A = h;
  g.lda = I;
  g.kdiv = 0;
  g.K = I;
  g.N = H;
  g.C = yslot;
  g.ldc = H;
  if ((err = gemm(false, g)) != hipSuccess) return err;

  if ((err = mark(5)) != hipSuccess) return err;
  if ((err = launch_combine<T>(reinterpret_cast<const T*>(yslot), T_, k, H, static_cast<T*>(a->y), st)) != hipSuccess)
    return err;
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
  Plan p = choose_plan(T, E, k, P, dtype);
  Layout l = layout_for(T, E, k, H, I, dtype == RIMURU_BF16 ? 2 : 4, p.bm);
  if (sorted_len) *sorted_len = l.sorted_len;
  if (workspace_bytes) *workspace_bytes = l.total;
  if (block_m) *block_m = p.bm;
  return RIMURU_OK;
}

namespace rimuru {
namespace {

// Host-side validation and launch shared by the two layer entry points;
// router == null: the logits are an input.
rimuru_status run_layer(const rimuru_moe_args* a, const RouterArgs* router, void* hip_stream) {
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
  if (!a->x || (!router && !a->logits) || !a->pool_base || !a->pt || !a->y || !a->topk_ids || !a->topk_w ||
      !a->sorted_ids || !a->expert_off || !a->workspace)
    return rimuru_fail(RIMURU_EINVAL, "fused_moe_paged: a required pointer is NULL");
  if (!aligned(a->pool_base, 256) || !aligned(a->workspace, 256) || !aligned(a->x, 16) ||
      !aligned(a->y, 16) || !aligned(a->topk_ids, 16))
    return rimuru_fail(RIMURU_EINVAL, "pool_base/workspace need 256-byte and x/y/topk_ids 16-byte alignment");
  Plan p = choose_plan(a->T, a->E, a->k, a->P, a->dtype);
  Layout lay = layout_for(a->T, a->E, a->k, a->H, a->I, es, p.bm);
  if (a->workspace_bytes < lay.total)
    return rimuru_fail(RIMURU_EINVAL, "workspace of %llu bytes is below the %llu needed",
                       (unsigned long long)a->workspace_bytes, (unsigned long long)lay.total);
  if ((a->stage_events == nullptr) != (a->n_stage_events == 0) ||
      (a->stage_events && a->n_stage_events != RIMURU_MOE_STAGES + 1))
    return rimuru_fail(RIMURU_EINVAL, "stage_events needs exactly %d events", RIMURU_MOE_STAGES + 1);
  hipStream_t st = static_cast<hipStream_t>(hip_stream);
  RouterArgs r2;
  if (router != nullptr) {
    r2 = *router;
    if (r2.logits_out == nullptr)
      r2.logits_out = reinterpret_cast<float*>(static_cast<uint8_t*>(a->workspace) + lay.off_logits);
    router = &r2;
  }
  hipError_t err = (a->dtype == RIMURU_BF16) ? launch_layer<uint16_t>(a, router, p, lay, st)
                                             : launch_layer<float>(a, router, p, lay, st);
  if (err != hipSuccess) return rimuru_fail(RIMURU_EHIP, "launch failed: %s", hipGetErrorString(err));
  return RIMURU_OK;
}

}  // namespace
}  // namespace rimuru

extern "C" rimuru_status rimuru_fused_moe_paged(const rimuru_moe_args* a, void* hip_stream) {
  return run_layer(a, nullptr, hip_stream);
}

extern "C" rimuru_status rimuru_fused_moe_paged_router(const rimuru_moe_args* a, const void* w_gate,
                                                       float* logits_out, void* hip_stream) {
  if (a == nullptr) return rimuru_fail(RIMURU_EINVAL, "fused_moe_paged_router: args is NULL");
  if (w_gate == nullptr || !aligned(w_gate, 16))
    return rimuru_fail(RIMURU_EINVAL, "fused_moe_paged_router: w_gate must be a 16-byte aligned device pointer");
  RouterArgs r{a->x, w_gate, a->H, a->dtype == RIMURU_BF16, logits_out};
  return run_layer(a, &r, hip_stream);   // logits_out == NULL: run_layer points it at the workspace
}

// ---------------------------------------------------------------- the layer without a caller workspace

// Scratch of rimuru_fused_moe_paged_noalloc: the layer's workspace (tile map,
// router logits, h, y_slot) in a fixed device array, for callers that cannot
// allocate. Every GPU the library runs on holds its own copy until the process
// ends. In host code the array's name is not a device address: its address on
// a device comes from hipGetSymbolAddress, taken once per device with that
// device current and kept below. Nothing in the workspace has to start at
// zero (every kernel writes what it later reads), so the scratch is never
// cleared.
namespace rimuru {

static __device__ __attribute__((aligned(256))) uint8_t scratch[RIMURU_NOALLOC_SCRATCH_BYTES];

namespace {

constexpr int kMaxDevices = 64;
std::atomic<void*> g_scratch[kMaxDevices];
std::mutex g_scratch_mu;

rimuru_status scratch_of_current_device(void** out) {
  int dev = -1;
  hipError_t err = hipGetDevice(&dev);
  if (err != hipSuccess) return rimuru_fail(RIMURU_EHIP, "fused_moe_paged_noalloc: hipGetDevice: %s", hipGetErrorString(err));
  if (dev < 0 || dev >= kMaxDevices)
    return rimuru_fail(RIMURU_EINVAL, "fused_moe_paged_noalloc: device %d beyond the %d this library tracks", dev, kMaxDevices);
  void* p = g_scratch[dev].load(std::memory_order_acquire);
  if (p == nullptr) {
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    p = g_scratch[dev].load(std::memory_order_relaxed);
    if (p == nullptr) {
      err = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
      if (err != hipSuccess || p == nullptr)
        return rimuru_fail(RIMURU_EHIP, "fused_moe_paged_noalloc: hipGetSymbolAddress of the scratch on device %d: %s",
                           dev, hipGetErrorString(err));
      g_scratch[dev].store(p, std::memory_order_release);
    }
  }
  *out = p;
  return RIMURU_OK;
}

}  // namespace
}  // namespace rimuru

extern "C" rimuru_status rimuru_fused_moe_paged_noalloc(const rimuru_moe_args* a, void* hip_stream) {
  if (a == nullptr) return rimuru_fail(RIMURU_EINVAL, "fused_moe_paged_noalloc: args is NULL");
  rimuru_status s = check_shapes(a->T, a->E, a->k, a->H, a->I, a->dtype);
  if (s != RIMURU_OK) return s;
  if (a->T == 0) return RIMURU_OK;
  if (a->P < 1) return rimuru_fail(RIMURU_EINVAL, "fused_moe_paged_noalloc: P = %d must be at least 1", a->P);
  const Plan p = choose_plan(a->T, a->E, a->k, a->P, a->dtype);
  const Layout lay = layout_for(a->T, a->E, a->k, a->H, a->I, a->dtype == RIMURU_BF16 ? 2 : 4, p.bm);
  if (lay.total > RIMURU_NOALLOC_SCRATCH_BYTES)
    return rimuru_fail(RIMURU_ENOMEM, "fused_moe_paged_noalloc: this shape needs %llu bytes of workspace, above the "
                       "%llu-byte scratch of the no-allocation entry point (use rimuru_fused_moe_paged with a "
                       "workspace)", (unsigned long long)lay.total, (unsigned long long)RIMURU_NOALLOC_SCRATCH_BYTES);
  void* ptr = nullptr;
  if ((s = scratch_of_current_device(&ptr)) != RIMURU_OK) return s;
  rimuru_moe_args b = *a;
  b.workspace = ptr;
  b.workspace_bytes = RIMURU_NOALLOC_SCRATCH_BYTES;
  return run_layer(&b, nullptr, hip_stream);
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

extern "C" rimuru_status rimuru_experts_store(void* pool_base, uint64_t pool_bytes, const int32_t* pt, int32_t E,
                                              int32_t P, uint64_t page_bytes, const void* src,
                                              uint64_t proj_bytes, void* hip_stream) {
  if (!pool_base || !pt || !src || E < 1 || P < 1)
    return rimuru_fail(RIMURU_EINVAL, "experts_store: bad argument");
  if (pool_bytes < page_bytes)
    return rimuru_fail(RIMURU_EINVAL, "experts_store: a pool of %llu bytes holds no page of %llu bytes",
                       (unsigned long long)pool_bytes, (unsigned long long)page_bytes);
  if (page_bytes == 0 || page_bytes % 128 != 0 || proj_bytes == 0 || proj_bytes % 16 != 0 ||
      proj_bytes > static_cast<uint64_t>(P) * page_bytes ||
      static_cast<uint64_t>(P) * page_bytes >= (1ull << 31))
    return rimuru_fail(RIMURU_EINVAL, "experts_store: page %llu / projection %llu bytes / P %d do not fit",
                       (unsigned long long)page_bytes, (unsigned long long)proj_bytes, P);
  if (!aligned(pool_base, 256) || !aligned(src, 16))
    return rimuru_fail(RIMURU_EINVAL, "experts_store: pool_base needs 256-byte, src 16-byte alignment");
  uint64_t n_segs = static_cast<uint64_t>(E) * 3 * proj_bytes / 16;
  hipError_t err = launch_store_pages(static_cast<uint8_t*>(pool_base), pool_bytes, pt, P,
                                      static_cast<uint32_t>(page_bytes),
                                      static_cast<const uint8_t*>(src), proj_bytes, n_segs,
                                      static_cast<hipStream_t>(hip_stream));
  if (err != hipSuccess) return rimuru_fail(RIMURU_EHIP, "experts_store: %s", hipGetErrorString(err));
  return RIMURU_OK;
}

extern "C" rimuru_status rimuru_stream_read(const void* buf, uint64_t bytes, uint32_t* sink, void* hip_stream) {
  if (buf == nullptr || sink == nullptr) return rimuru_fail(RIMURU_EINVAL, "stream_read: NULL pointer");
  if (reinterpret_cast<uintptr_t>(buf) % 16 != 0 || bytes % 16 != 0)
    return rimuru_fail(RIMURU_EINVAL, "stream_read: buf must be 16-byte aligned and bytes a multiple of 16");
  const hipError_t err = launch_stream_read(buf, bytes, sink, static_cast<hipStream_t>(hip_stream));
  if (err != hipSuccess) return rimuru_fail(RIMURU_EHIP, "stream_read: launch failed: %s", hipGetErrorString(err));
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
