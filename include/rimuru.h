/*
 * rimuru.h -- C ABI of the paged fused-MoE library (librimuru.so) for MI355X.
 *
 * The library has two halves:
 *
 *  1. A host-side page allocator over one shared page pool, with one memory
 *     view per tensor type. Rimuru paper summary ("Rimuru: Unified Memory
 *     Management for Modern LLM Serving via Elastic Expert Offloading",
 *     thelatestinai.com), abstract and Figures 6-7; explainer "Rimuru unifies
 *     serving memory" (learnaivisually.com), paragraph on moving the fence.
 *     The allocator only hands out byte offsets; it never touches device
 *     memory.
 *
 *  2. The page-table-aware fused MoE layer: routing (softmax top-k,
 *     renormalised), grouping of routed slots by expert, and the gated SiLU
 *     expert MLP with a weighted top-k combine, reading every expert weight
 *     in place through the expert view's page table, never copying an expert
 *     into a contiguous buffer (paper summary, abstract; explainer, paragraph
 *     on the two pieces that make the moving fence usable; Figure 11's
 *     "Discrete FusedMoE").
 *
 * Conventions for every call:
 *  - Every function returns a status; 0 is success, negative values are the
 *    RIMURU_E* codes below. rimuru_last_error() returns a thread-local
 *    message for the last failing call on the calling thread.
 *  - Nothing crosses this ABI but C types, plain host pointers, device
 *    pointers given as void* / typed pointers, and hipStream_t given as void*.
 *    No exception escapes; the library never aborts the process.
 *  - Device memory is always owned by the caller. The library never
 *    allocates or frees device memory.
 *  - Host objects (pools and views) are owned by the library between their
 *    create call and rimuru_pool_destroy(). A pool and its views must not
 *    be used from two threads at once.
 */
#ifndef RIMURU_H
#define RIMURU_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef int32_t rimuru_status;

enum {
  RIMURU_OK = 0,
  RIMURU_EINVAL = -1, /* bad argument, unknown owner, double free */
  RIMURU_ENOMEM = -2, /* pool exhausted or a view budget exceeded */
  RIMURU_ERANGE = -3, /* a page-table entry outside the pool (checked call) */
  RIMURU_EDTYPE = -4, /* unsupported element type */
  RIMURU_EHIP = -5,   /* a HIP runtime call failed (launch, event) */
  RIMURU_EBUSY = -6   /* a budget change would cut into resident pages */
};

enum { RIMURU_F32 = 0, RIMURU_BF16 = 1 };

/* Tensor types that own a view (Table 1 of the paper summary: expert
 * projections, KV cache, SSM state, conv state). */
enum { RIMURU_VIEW_EXPERT = 0, RIMURU_VIEW_KV = 1, RIMURU_VIEW_SSM = 2, RIMURU_VIEW_CONV = 3 };

typedef struct rimuru_pool rimuru_pool; /* opaque, host side */
typedef struct rimuru_view rimuru_view; /* opaque, host side */

/* Thread-local text for the last failing call on this thread ("" if none).
 * The pointer stays valid until the next failing call on the same thread. */
const char* rimuru_last_error(void);

/* ABI revision of this header; bumped on any incompatible change. */
int32_t rimuru_abi_version(void);
#define RIMURU_ABI_VERSION 1

/* ------------------------------------------------------------------------ */
/* Page pool and views                                                      */
/* ------------------------------------------------------------------------ */

/* Create host state for a shared page pool of pool_bytes bytes cut into
 * floor(pool_bytes / huge_page_bytes) huge pages (paper summary, abstract:
 * a shared page pool with huge-page alignment; explainer: huge pages are a
 * common multiple of the expert and state page sizes). Bytes past the last
 * whole huge page are unused and reported as waste.
 *   huge_page_bytes: > 0, a multiple of 128, <= pool_bytes.
 *   out: receives the pool; free it with rimuru_pool_destroy().
 * Errors: EINVAL. */
rimuru_status rimuru_pool_create(uint64_t pool_bytes, uint64_t huge_page_bytes,
                                 rimuru_pool** out);

/* Destroy a pool and every view mapped on it. NULL is a no-op. */
rimuru_status rimuru_pool_destroy(rimuru_pool* pool);

/* Register a memory view: one tensor type's own page size over the shared
 * pool (paper summary, abstract and Figure 6).
 *   kind: RIMURU_VIEW_*.
 *   page_bytes: > 0, a multiple of 128.
 *   parent: NULL to cut this view's pages straight from huge pages
 *     (page_bytes must then divide huge_page_bytes), or another view of the
 *     same pool whose pages are split into pages of this one (page_bytes <=
 *     the parent's page size; floor(parent / page) pages per parent page,
 *     the rest is waste). Figure 7: huge -> expert-sized -> KV-sized.
 *   A KV view may not be cut straight from huge pages unless its page is a
 *   whole huge page (explainer: a huge page is never cut straight into KV
 *   blocks).
 *   out: receives the view, owned by the pool.
 * A new view has no budget limit.
 * Errors: EINVAL. */
rimuru_status rimuru_view_map(rimuru_pool* pool, int32_t kind, uint64_t page_bytes,
                              rimuru_view* parent, rimuru_view** out);

/* Allocate n_pages pages of view v for one owner (a request, or one expert
 * projection) and write their pool byte offsets, in allocation order, to
 * out_offsets[0..n_pages). Owner ids >= 2^63 are reserved. Calling again for
 * the same owner appends pages.
 * Placement, one page at a time: the lowest-address parent page of v that
 * already holds a page of this owner and has a free slot; else the
 * lowest-address parent with a free slot; else a new parent (the
 * lowest-address free huge page, or a page of the parent view allocated by
 * these same rules). Within a parent, the lowest free slot (explainer: one
 * request's small pages are cut from the same parent when possible).
 * All or nothing: on failure the pool is left exactly as it was.
 * Errors: EINVAL (n_pages == 0, reserved owner, NULL out_offsets),
 *         ENOMEM (no room, or the view's budget would be exceeded). */
rimuru_status rimuru_view_alloc(rimuru_view* v, uint64_t owner, uint64_t n_pages,
                                int64_t* out_offsets);

/* Free every page of owner in view v. A parent page whose last slot is freed
 * merges back into its own level, recursively up to the huge page
 * (explainer: reclaiming takes the same path in reverse).
 * Errors: EINVAL (owner holds no page in v, e.g. a double free). */
rimuru_status rimuru_view_free(rimuru_view* v, uint64_t owner);

/* Copy the pool byte offsets of owner's pages in v, in allocation order, to
 * out_offsets (capacity cap entries); *n_out receives the page count even
 * when it exceeds cap (then nothing is copied and EINVAL is returned). An
 * owner with no page yields *n_out = 0 and OK. */
rimuru_status rimuru_view_pages(const rimuru_view* v, uint64_t owner, int64_t* out_offsets,
                                uint64_t cap, uint64_t* n_out);

/* Workload-aware adjuster mechanism (paper summary, abstract; explainer,
 * paragraph on the adjuster): capacity moves between views by budget.
 * A budget caps the bytes a view's owners may hold (pages * page_bytes);
 * UINT64_MAX means no limit. Resident pages never move.
 *   rimuru_view_set_budget: EBUSY if bytes is below what the owners hold.
 *   rimuru_pool_transfer: moves bytes of budget from one view to another
 *     view of the same pool; both must have a finite budget (EINVAL);
 *     EBUSY if the source would drop below what its owners hold. */
rimuru_status rimuru_view_set_budget(rimuru_view* v, uint64_t bytes);
rimuru_status rimuru_pool_transfer(rimuru_pool* pool, rimuru_view* from, rimuru_view* to,
                                   uint64_t bytes);
/* Bytes held by the view's owners, and its budget (UINT64_MAX = none). */
rimuru_status rimuru_view_usage(const rimuru_view* v, uint64_t* used_bytes,
                                uint64_t* budget_bytes);
/* The pool a view belongs to, its kind and its page size; any output may be
 * NULL. Errors: EINVAL (NULL view). */
rimuru_status rimuru_view_info(const rimuru_view* v, rimuru_pool** pool, int32_t* kind,
                               uint64_t* page_bytes);

typedef struct {
  uint64_t huge_pages;        /* whole huge pages in the pool */
  uint64_t huge_free;         /* huge pages not split for any view */
  uint64_t bytes_per_kind[4]; /* bytes held by owners, per RIMURU_VIEW_* kind */
  uint64_t bytes_free;        /* free huge pages + free slots of split pages */
  uint64_t waste_bytes;       /* pool tail + split remainders */
  uint64_t split_parents;     /* parent pages currently split, all views */
} rimuru_pool_stats_t;
/* bytes_per_kind summed + bytes_free + waste_bytes == pool_bytes. */
rimuru_status rimuru_pool_stats(const rimuru_pool* pool, rimuru_pool_stats_t* out);

/* Full internal consistency check (slow; for tests). EINVAL with a message
 * naming the first broken invariant. */
rimuru_status rimuru_pool_check(const rimuru_pool* pool);

/* ------------------------------------------------------------------------ */
/* Workload-aware adjuster policy                                           */
/* ------------------------------------------------------------------------ */

/* The policy that moves the fence between the expert view and the KV view
 * (paper summary: abstract, "workload-aware adjuster", and Figure 8;
 * explainer "Rimuru unifies serving memory", paragraph on the two pieces that
 * make the moving fence usable: rising request counts shift budget toward the
 * KV view, KV blocks freed by finished requests shift it back, and the
 * prefetch path's uploads are never evicted mid-flight). The pages give no
 * rule beyond that; the rule below is this library's reading.
 *
 * Experts are expert-view owners 3e + p (p = 0, 1, 2 for w1, w3, w2), P pages
 * each; expert e is resident when all three hold P pages. Each expert has an
 * integer popularity score, s <- s - (s >> shift) + (routed << 16) per step.
 * Pinned experts (needed by the next layer call, or with an upload in
 * flight) are never evicted. "Coldest" = lowest score, ties to the lower id.
 * One step, given D = KV blocks demanded:
 *   1. each needed, non-resident expert (ascending id) gets pages: while the
 *      expert view's free budget is short of one expert, evict the coldest
 *      unpinned resident expert; with none left, move the shortfall from the
 *      KV view's unused budget, else fail (ENOMEM); if the pool itself has
 *      no room, evict the next coldest and retry;
 *   2. W = (D + headroom_blocks) KV blocks. Below W: the KV view takes the
 *      shortfall, capped so that the expert view keeps a budget of
 *      min_resident experts; coldest unpinned experts are evicted until the
 *      expert view's free budget covers that amount (or none is left), then
 *      the free amount moves. Above W by more than return_blocks blocks:
 *      everything above max(W, KV bytes held) moves back to the experts;
 *   3. prefetch: while a whole expert of budget is free and fewer than
 *      max_prefetch prefetches were made, the most popular non-resident
 *      expert with a positive score not evicted in this step gets pages
 *      (ties to the lower id); the first that does not fit ends the step.
 * Loads are reported demand loads first, then prefetches; each loaded
 * expert is "in flight" until rimuru_adjuster_upload_done: the caller fills
 * its pages (rimuru_view_pages gives them; rimuru_expert_upload copies from
 * host memory) and must finish the demand loads before the layer runs.
 * Page moves never happen: only budgets move and experts come and go. */
typedef struct rimuru_adjuster rimuru_adjuster; /* opaque, host side */
typedef struct {
  int32_t E;               /* experts, >= 1 */
  int32_t P;               /* expert-view pages per projection, >= 1 */
  int32_t min_resident;    /* expert budget kept when KV grows, in experts;
                              must cover the experts one step needs plus the
                              uploads in flight, or steps can fail */
  int32_t headroom_blocks; /* KV blocks of slack above the demand */
  int32_t return_blocks;   /* surplus KV blocks tolerated before giving back */
  int32_t shift;           /* popularity decay, 0..16 (keeps scores < 2^63) */
  int32_t max_prefetch;    /* prefetch loads per step, >= 0 */
} rimuru_adjuster_params;

/* Create the adjuster over two views of one pool; both need finite budgets
 * (rimuru_view_set_budget). Experts whose three projections already hold P
 * pages start resident; a partly placed expert is EINVAL. The adjuster does
 * not own the pool: destroy it before the pool.
 * Errors: EINVAL. */
rimuru_status rimuru_adjuster_create(rimuru_pool* pool, rimuru_view* expert_view, rimuru_view* kv_view,
                                     const rimuru_adjuster_params* params, rimuru_adjuster** out);
rimuru_status rimuru_adjuster_destroy(rimuru_adjuster* adj); /* NULL is a no-op */

/* One policy step.
 *   demand_blocks  KV blocks the running and admitted requests need.
 *   routed         host int32 [E] routed slots per expert in the last step
 *                  (>= 0), or NULL for none.
 *   needed         host uint8 [E], nonzero = the next layer call reads the expert.
 *   evicted, loaded  host int32 arrays of capacity E; *n_evicted and *n_loaded
 *                  receive the counts (an expert appears at most once in each).
 *   kv_moved       bytes of budget moved toward the KV view (negative: toward
 *                  the experts), net over the step; may be NULL.
 * Errors: EINVAL (bad argument); ENOMEM (the needed experts do not fit):
 * the evictions and loads made before the failure stand and are reported. */
rimuru_status rimuru_adjuster_step(rimuru_adjuster* adj, uint64_t demand_blocks, const int32_t* routed,
                                   const uint8_t* needed, int32_t* evicted, int32_t* n_evicted,
                                   int32_t* loaded, int32_t* n_loaded, int64_t* kv_moved);

/* The upload into expert e's pages has finished: e is no longer pinned by
 * it. Errors: EINVAL (no upload of e in flight). */
rimuru_status rimuru_adjuster_upload_done(rimuru_adjuster* adj, int32_t e);

/* Copy the state out: resident and in_flight as uint8 [E], score as uint64
 * [E]; any may be NULL. */
rimuru_status rimuru_adjuster_state(const rimuru_adjuster* adj, uint8_t* resident, uint8_t* in_flight,
                                    uint64_t* score);

/* ------------------------------------------------------------------------ */
/* Paged decode attention over the KV view                                   */
/* ------------------------------------------------------------------------ */

/* The second workload on the same pool: decode attention reading the KV
 * cache where its blocks sit in the KV view (explainer "Rimuru unifies
 * serving memory", paragraph on moving the fence: 16-token KV blocks through
 * a block table, cut from expert-sized pages; paper summary, Table 1: one
 * token's K and V are [2, n_kv_heads, head_dim]).
 *
 * KV block layout (bf16, 16 tokens; the pages fix no order inside a block):
 * K of KV heads 0..n_kv-1, each token-major [16][head_dim], then V of KV
 * heads 0..n_kv-1, each dim-major [head_dim][16]. block_bytes =
 * 2 * n_kv * 16 * head_dim * 2 (32 KiB for [2, 4, 128]).
 *
 * For request b and query head h (KV head h / (n_q / n_kv)):
 *   out[b, h] = softmax_t(scale * q[b, h] . K_b[t]) V_b, t < context_lens[b],
 * accumulated in fp32 (probabilities rounded to bf16 for the second
 * product), written as bf16; context length 0 gives zeros. Token slots past
 * the context in a request's last block may hold any bytes (NaN and Inf
 * included: blocks are cut from pages that held other tensors): their scores
 * and their V values are selected away, never multiplied in. */
typedef struct {
  int32_t B;               /* requests (one query token each), >= 0 */
  int32_t n_q;             /* query heads: a multiple of n_kv, <= 16 * n_kv */
  int32_t n_kv;            /* KV heads, >= 1 */
  int32_t head_dim;        /* 128 or 256 */
  int32_t max_blocks;      /* columns of block_table, >= 1 */
  float scale;             /* softmax scale (> 0), e.g. 1/sqrt(head_dim) */
  const void* q;           /* device bf16 [B, n_q, head_dim], 16-byte aligned */
  const void* pool_base;   /* device pool, 256-byte aligned */
  const int32_t* block_table; /* device [B, max_blocks]: block indices in units
                              of block_bytes from pool_base (the KV view's
                              page offsets / block_bytes); entries past a
                              request's context are not read. Not checked on
                              the device: rimuru_block_table_check checks a
                              host copy. */
  const int32_t* context_lens; /* device [B], 0 .. 16 * max_blocks (clamped) */
  void* out;               /* device bf16 [B, n_q, head_dim] */
  void* workspace;         /* device, 16-byte aligned, workspace_bytes from
                              rimuru_attn_sizes; partials of the splits */
  uint64_t workspace_bytes;
} rimuru_attn_args;

/* Workspace bytes, number of context splits and block bytes for a shape.
 * Any output may be NULL. Errors: EINVAL (unsupported shape). */
rimuru_status rimuru_attn_sizes(int32_t B, int32_t n_q, int32_t n_kv, int32_t head_dim, int32_t max_blocks,
                                uint64_t* workspace_bytes, int32_t* n_split, uint64_t* block_bytes);

/* Enqueue the attention (two kernels: the splits, then their merge; the
 * first alone when every context fits one split, e.g. 256 or more requests
 * over 4 KV heads) on the
 * stream; returns without a host sync. Errors: EINVAL, EHIP. */
rimuru_status rimuru_paged_decode_attention(const rimuru_attn_args* args, void* hip_stream);

/* Host check of a host copy of block_table and context_lens: every block a
 * request's context covers lies inside a pool of pool_bytes. ERANGE names the
 * first bad entry or length. */
rimuru_status rimuru_block_table_check(const int32_t* block_table, int32_t B, int32_t max_blocks,
                                       const int32_t* context_lens, uint64_t block_bytes, uint64_t pool_bytes);

/* ------------------------------------------------------------------------ */
/* Page-table-aware fused MoE                                               */
/* ------------------------------------------------------------------------ */

/* Arguments of rimuru_fused_moe_paged. All pointers are device pointers
 * unless stated; all arrays are row-major and densely packed.
 *
 * Expert weights live in the pool. Expert e owns three projections, in this
 * order: w1 [H, I] (gate), w3 [H, I] (up), w2 [I, H] (down) (Table 1 of the
 * paper summary gives the shapes; the gate/up/down roles are this library's
 * reading). Byte f of projection p of expert e lives at
 *     pool_base + pt[(e*3 + p)*P + f / page_bytes] * page_bytes + f % page_bytes.
 */
typedef struct {
  int32_t T;           /* tokens, >= 0 (0 is a no-op) */
  int32_t E;           /* experts, 1..512 */
  int32_t k;           /* experts per token, 1..min(E, 32) */
  int32_t H;           /* hidden size, a positive multiple of 64 */
  int32_t I;           /* intermediate size, a positive multiple of 64 */
  int32_t P;           /* pages per projection in pt; P*page_bytes >= H*I*es */
  int32_t dtype;       /* RIMURU_BF16 or RIMURU_F32: x, weights and y share it */
  int32_t renormalize; /* must be 1: the kept top-k weights sum to one */
  const void* x;       /* [T, H] tokens, 16-byte aligned */
  const float* logits; /* [T, E] fp32 router logits; finite (precondition) */
  const void* pool_base; /* pool start, 256-byte aligned */
  const int32_t* pt;   /* [E][3][P] page indices in units of page_bytes; every
                          entry an expert with routed tokens uses must lie in
                          the pool (precondition, not checked per call) */
  uint64_t page_bytes; /* expert-view page, a multiple of 128 */
  void* y;             /* [T, H] output, dtype, 16-byte aligned */
  int32_t* topk_ids;   /* [T, k] out: expert ids in rank order, 16-byte aligned */
  float* topk_w;       /* [T, k] out: renormalised weights */
  int32_t* sorted_ids; /* [sorted_len] out: routed slots t*k + j grouped by expert
                          (ascending expert, ascending slot), each expert's
                          segment padded with T*k to a multiple of block_m */
  int32_t* expert_off; /* [E + 1] out: start of each expert's padded segment;
                          expert_off[E] = total padded length */
  void* workspace;     /* scratch, workspace_bytes from rimuru_moe_sizes,
                          256-byte aligned; contents undefined on return */
  uint64_t workspace_bytes;
  void* const* stage_events; /* optional host array of hipEvent_t (NULL = none):
                          n_stage_events == RIMURU_MOE_STAGES + 1; event i is
                          recorded on the stream before stage i, the last one
                          after the last stage */
  int32_t n_stage_events;
} rimuru_moe_args;

/* Stages, in launch order: gating top-k, per-expert count, sort + tile align,
 * gate/up GEMM with SiLU, down GEMM with routing weight, top-k combine. Some
 * stages share a kernel, and then the events around the later ones are
 * recorded back to back: the count runs inside the sort up to 4096 routed
 * slots, one kernel routes batches of up to 16 tokens, and for bf16 batches
 * of at most 4 tokens (16-row tiles, given logits, H a multiple of 128) the
 * gate/up stream does the routing itself, whose time then falls in the
 * gate/up stage. */
#define RIMURU_MOE_STAGES 6

/* Buffer sizes for a call with these shapes and P pages per projection:
 * sorted_len (entries of sorted_ids), workspace_bytes, and the tile height
 * block_m the segments are padded to. Any output pointer may be NULL. The
 * workspace does not depend on the size of the expert weights: the layer
 * never copies them.
 * Errors: EINVAL, EDTYPE. */
rimuru_status rimuru_moe_sizes(int32_t T, int32_t E, int32_t k, int32_t H, int32_t I, int32_t P,
                               int32_t dtype, uint64_t* sorted_len,
                               uint64_t* workspace_bytes, int32_t* block_m);

/* Enqueue the fused MoE layer on hip_stream (a hipStream_t; NULL = the null
 * stream) and return without synchronising. Arguments are validated on the
 * host first; nothing is enqueued on error. Device faults from a broken
 * precondition surface at the caller's next synchronisation.
 * Errors: EINVAL, EDTYPE, EHIP (a launch or event record failed). */
rimuru_status rimuru_fused_moe_paged(const rimuru_moe_args* a, void* hip_stream);

/* The same layer with the router projection inside the gating stage (the
 * upstream step the pages leave implicit): logits[t, e] = x[t] . w_gate[e],
 * accumulated in fp32 with MFMA tiles by one small GEMM kernel, then the same
 * top-k and softmax. The logits go to logits_out, or to the workspace (its
 * size from rimuru_moe_sizes covers them) when logits_out is NULL.
 *   w_gate      device [E, H] row-major (a Linear layer's weight layout), in
 *               the layer's dtype, 16-byte aligned.
 *   logits_out  device [T, E] fp32, or NULL.
 *   a->logits   not read (may be NULL); every other field as above.
 * Ties in the top-k are decided on these fp32 logits.
 * Errors: EINVAL, EDTYPE, EHIP. */
rimuru_status rimuru_fused_moe_paged_router(const rimuru_moe_args* a, const void* w_gate,
                                            float* logits_out, void* hip_stream);

/* Bytes of the fixed device scratch rimuru_fused_moe_paged_noalloc uses as
 * its workspace (one array per GPU, held until the process ends). */
#define RIMURU_NOALLOC_SCRATCH_BYTES (64ull << 20)

/* The same layer for callers that cannot allocate device memory (code under
 * HIP graph capture, tight serving loops, harnesses that forbid hipMalloc):
 * it takes no workspace (a->workspace and a->workspace_bytes are ignored) and
 * uses a fixed scratch array of RIMURU_NOALLOC_SCRATCH_BYTES on the current
 * device instead; the caller still passes x, logits, the pool, pt and the
 * outputs. It calls no allocating routine. Every call on one GPU shares that
 * GPU's scratch: calls that overlap on one GPU (on different streams, or
 * from several threads) race and must be ordered by the caller. The scratch
 * needs no clearing between calls.
 * Errors: ENOMEM (the shape's workspace, rimuru_moe_sizes' workspace_bytes,
 * exceeds the scratch; nothing is enqueued), EINVAL, EDTYPE, EHIP. */
rimuru_status rimuru_fused_moe_paged_noalloc(const rimuru_moe_args* a, void* hip_stream);

/* Host-side check that every entry of a host copy of pt (E*3*P entries)
 * names a page inside a pool of pool_bytes bytes. ERANGE names the first bad
 * entry. */
rimuru_status rimuru_pt_check(const int32_t* pt_host, int32_t E, int32_t P,
                              uint64_t page_bytes, uint64_t pool_bytes);

/* Load expert weights into their pages: copy src (device, [E][3][proj_bytes]
 * contiguous) into the pool pages pt (device [E][3][P]) names, page by page,
 * on hip_stream. This is how weights reach the pool (the reverse of the
 * contiguous copy the layer avoids); it is not part of the layer.
 * pool_bytes is the pool's size: a pt entry naming a page outside
 * [0, pool_bytes) is skipped on the device (that page's bytes are not
 * stored; nothing outside the pool is written). pt lives on the device and
 * is not read on the host here: check a host copy with rimuru_pt_check first
 * to have such entries reported (the Python binding does). proj_bytes <=
 * P*page_bytes, proj_bytes a multiple of 16, page_bytes a multiple of 128.
 * Errors: EINVAL, EHIP. */
rimuru_status rimuru_experts_store(void* pool_base, uint64_t pool_bytes, const int32_t* pt, int32_t E,
                                   int32_t P, uint64_t page_bytes, const void* src, uint64_t proj_bytes,
                                   void* hip_stream);

/* Elastic expert offloading, dual-buffer upload (Rimuru paper summary,
 * Figure 8: expert prefetch overlapped with execution, no device-to-device
 * copy): copy one expert's three projections from host memory straight into
 * fresh expert-view pages, one host-to-device copy per run of pages that are
 * consecutive in the pool and in the projection, on hip_stream
 * (typically a copy stream beside the stream running the layer). The pages
 * are written where they sit; since the layer reads every weight through the
 * page table, the expert is usable as soon as its page-table rows name these
 * pages and the copies have completed on hip_stream.
 *   pool_base   device, 256-byte aligned; pool_bytes its size.
 *   pt_rows     host int32 [3][P]: destination page indices (units of
 *               page_bytes) for w1, w3, w2, as the expert view allocated
 *               them; every page must lie inside the pool (else ERANGE).
 *   host_src    host memory, [3][proj_bytes] contiguous, 16-byte aligned;
 *               page-locked (hipHostMalloc, or pinned by its allocator) so
 *               the copies run asynchronously. The caller keeps it alive and
 *               unmodified until the copies complete.
 *   proj_bytes  bytes of one projection, <= P*page_bytes, a multiple of 16;
 *               page_bytes a multiple of 128.
 * Errors: EINVAL, ERANGE (checked before anything is enqueued), EHIP (a copy
 * could not be enqueued; earlier pages of this call may have been). */
rimuru_status rimuru_expert_upload(void* pool_base, uint64_t pool_bytes, const int32_t* pt_rows,
                                   int32_t P, uint64_t page_bytes, const void* host_src,
                                   uint64_t proj_bytes, void* hip_stream);

/* Small event helpers so callers can time stages without linking HIP:
 * create/destroy a timing-enabled hipEvent_t, and the elapsed milliseconds
 * between two recorded events (synchronises on the second). */
rimuru_status rimuru_event_create(void** ev);
rimuru_status rimuru_event_destroy(void* ev);
rimuru_status rimuru_event_record(void* ev, void* hip_stream);
rimuru_status rimuru_event_elapsed_ms(void* start, void* stop, float* ms);

/* Calibration read: enqueue one plain streaming read of buf (every 16-byte
 * piece loaded once, non-temporally, by a grid-stride loop with eight loads
 * in flight per thread), the practical read bound of the GPU beside its
 * datasheet peak.
 * Nothing is written except, if the XOR of all the data equals 0x5A5A5A5A,
 * that value to *sink (a device uint32; the store keeps the loads live).
 *   buf: device, 16-byte aligned; bytes: a multiple of 16.
 * Errors: EINVAL, EHIP. */
rimuru_status rimuru_stream_read(const void* buf, uint64_t bytes, uint32_t* sink, void* hip_stream);

#ifdef __cplusplus
}
#endif

#endif /* RIMURU_H */
