// Workload-aware adjuster policy over the page allocator's expert and KV views.
//
// Rimuru paper summary (thelatestinai.com), abstract (a workload-aware
// adjuster reallocates pages across tensor types by runtime demand) and
// Figure 8 (expert prefetch overlapped with execution); explainer "Rimuru
// unifies serving memory" (learnaivisually.com), paragraph on the two pieces
// that make the moving fence usable. The decision rule is stated in rimuru.h.
//
// The adjuster moves budget between the two views and makes experts come and
// go through the allocator's public calls; it never moves a resident page.
#include <cstdint>
#include <new>
#include <vector>

#include "rimuru.h"
#include "rimuru_internal.h"

struct rimuru_adjuster {
  rimuru_pool* pool = nullptr;
  rimuru_view* xv = nullptr;     // expert view
  rimuru_view* kv = nullptr;     // KV view
  rimuru_adjuster_params prm{};
  uint64_t expert_bytes = 0;     // 3 projections x P pages
  uint64_t kv_page = 0;
  std::vector<uint8_t> resident, inflight;
  std::vector<uint64_t> score;
  std::vector<int64_t> scratch;  // page offsets (allocator output, unused)
};

namespace {

struct Usage {
  uint64_t used, budget;
};

Usage usage(const rimuru_view* v) {
  Usage u{0, 0};
  rimuru_view_usage(v, &u.used, &u.budget);
  return u;
}

uint64_t free_budget(const rimuru_view* v) {
  const Usage u = usage(v);
  return u.budget - u.used;
}

// Step-local bookkeeping: pins, and the lists handed back to the caller.
struct StepState {
  std::vector<uint8_t> pinned, evicted_now;
  int32_t* evicted;
  int32_t n_evicted = 0;
  int32_t* loaded;
  int32_t n_loaded = 0;
  int64_t moved = 0;
};

// Coldest resident expert that is not pinned, or -1.
int coldest(const rimuru_adjuster* a, const StepState& st) {
  int best = -1;
  for (int e = 0; e < a->prm.E; ++e)
    if (a->resident[e] && !st.pinned[e] && (best < 0 || a->score[e] < a->score[best])) best = e;
  return best;
}

rimuru_status evict(rimuru_adjuster* a, int e, StepState& st) {
  for (int p = 0; p < 3; ++p) {
    const rimuru_status s = rimuru_view_free(a->xv, 3ull * e + p);
    if (s != RIMURU_OK) return s;
  }
  a->resident[e] = 0;
  st.evicted_now[e] = 1;
  st.evicted[st.n_evicted++] = e;
  return RIMURU_OK;
}

// Pages for the three projections of e, all or nothing.
rimuru_status load(rimuru_adjuster* a, int e) {
  for (int p = 0; p < 3; ++p) {
    const rimuru_status s = rimuru_view_alloc(a->xv, 3ull * e + p, a->prm.P, a->scratch.data());
    if (s != RIMURU_OK) {
      for (int q = 0; q < p; ++q) rimuru_view_free(a->xv, 3ull * e + q);
      return s;
    }
  }
  return RIMURU_OK;
}

void mark_loaded(rimuru_adjuster* a, int e, StepState& st) {
  a->resident[e] = 1;
  a->inflight[e] = 1;
  st.loaded[st.n_loaded++] = e;
}

// Step 1: the needed experts that are not resident.
rimuru_status demand_loads(rimuru_adjuster* a, const uint8_t* needed, StepState& st) {
  for (int e = 0; e < a->prm.E; ++e) {
    if (!needed[e] || a->resident[e]) continue;
    for (;;) {
      if (free_budget(a->xv) < a->expert_bytes) {
        const int v = coldest(a, st);
        if (v >= 0) {
          const rimuru_status s = evict(a, v, st);
          if (s != RIMURU_OK) return s;
          continue;
        }
        const uint64_t short_by = a->expert_bytes - free_budget(a->xv);
        if (free_budget(a->kv) < short_by)
          return rimuru_fail(RIMURU_ENOMEM, "adjuster_step: no room for needed expert %d", e);
        const rimuru_status s = rimuru_pool_transfer(a->pool, a->kv, a->xv, short_by);
        if (s != RIMURU_OK) return s;
        st.moved -= static_cast<int64_t>(short_by);
      }
      const rimuru_status s = load(a, e);
      if (s == RIMURU_OK) break;
      if (s != RIMURU_ENOMEM) return s;
      const int v = coldest(a, st);   // budget allows, the pool has no room
      if (v < 0)
        return rimuru_fail(RIMURU_ENOMEM, "adjuster_step: the pool has no room for needed expert %d", e);
      const rimuru_status s2 = evict(a, v, st);
      if (s2 != RIMURU_OK) return s2;
    }
    mark_loaded(a, e, st);
  }
  return RIMURU_OK;
}

// Step 2: the KV budget toward W = (D + headroom) blocks.
rimuru_status move_fence(rimuru_adjuster* a, uint64_t demand_blocks, StepState& st) {
  const uint64_t want = (demand_blocks + a->prm.headroom_blocks) * a->kv_page;
  const Usage k = usage(a->kv);
  if (k.budget < want) {
    const uint64_t floor = static_cast<uint64_t>(a->prm.min_resident) * a->expert_bytes;
    const uint64_t bx = usage(a->xv).budget;
    uint64_t goal = want - k.budget;
    const uint64_t cap = bx > floor ? bx - floor : 0;
    if (goal > cap) goal = cap;
    while (free_budget(a->xv) < goal) {
      const int v = coldest(a, st);
      if (v < 0) break;
      const rimuru_status s = evict(a, v, st);
      if (s != RIMURU_OK) return s;
    }
    const uint64_t fx = free_budget(a->xv);
    const uint64_t take = goal < fx ? goal : fx;
    if (take > 0) {
      const rimuru_status s = rimuru_pool_transfer(a->pool, a->xv, a->kv, take);
      if (s != RIMURU_OK) return s;
      st.moved += static_cast<int64_t>(take);
    }
  } else if (k.budget - want > static_cast<uint64_t>(a->prm.return_blocks) * a->kv_page) {
    const uint64_t keep = want > k.used ? want : k.used;
    if (k.budget > keep) {
      const rimuru_status s = rimuru_pool_transfer(a->pool, a->kv, a->xv, k.budget - keep);
      if (s != RIMURU_OK) return s;
      st.moved -= static_cast<int64_t>(k.budget - keep);
    }
  }
  return RIMURU_OK;
}

// Step 3: prefetch the most popular experts into free expert budget.
rimuru_status prefetch(rimuru_adjuster* a, StepState& st) {
  for (int n = 0; n < a->prm.max_prefetch && free_budget(a->xv) >= a->expert_bytes; ++n) {
    int best = -1;
    for (int e = 0; e < a->prm.E; ++e)
      if (!a->resident[e] && a->score[e] > 0 && !st.evicted_now[e] &&
          (best < 0 || a->score[e] > a->score[best]))
        best = e;
    if (best < 0) break;
    const rimuru_status s = load(a, best);
    if (s == RIMURU_ENOMEM) break;
    if (s != RIMURU_OK) return s;
    mark_loaded(a, best, st);
  }
  return RIMURU_OK;
}

}  // namespace

extern "C" rimuru_status rimuru_adjuster_create(rimuru_pool* pool, rimuru_view* expert_view,
                                                rimuru_view* kv_view, const rimuru_adjuster_params* prm,
                                                rimuru_adjuster** out) {
  if (pool == nullptr || expert_view == nullptr || kv_view == nullptr || prm == nullptr || out == nullptr)
    return rimuru_fail(RIMURU_EINVAL, "adjuster_create: NULL argument");
  *out = nullptr;
  if (prm->E < 1 || prm->P < 1 || prm->min_resident < 0 || prm->headroom_blocks < 0 ||
      prm->return_blocks < 0 || prm->shift < 0 || prm->shift > 16 || prm->max_prefetch < 0)
    return rimuru_fail(RIMURU_EINVAL, "adjuster_create: bad parameter");
  rimuru_pool *px = nullptr, *pk = nullptr;
  uint64_t xpage = 0, kpage = 0;
  rimuru_view_info(expert_view, &px, nullptr, &xpage);
  rimuru_view_info(kv_view, &pk, nullptr, &kpage);
  if (px != pool || pk != pool || expert_view == kv_view)
    return rimuru_fail(RIMURU_EINVAL, "adjuster_create: the views must be two views of this pool");
  if (usage(expert_view).budget == ~0ull || usage(kv_view).budget == ~0ull)
    return rimuru_fail(RIMURU_EINVAL, "adjuster_create: both views need a finite budget");
  rimuru_adjuster* a = new (std::nothrow) rimuru_adjuster;
  if (a == nullptr) return rimuru_fail(RIMURU_ENOMEM, "adjuster_create: host allocation failed");
  a->pool = pool;
  a->xv = expert_view;
  a->kv = kv_view;
  a->prm = *prm;
  a->expert_bytes = 3ull * prm->P * xpage;
  a->kv_page = kpage;
  a->resident.assign(prm->E, 0);
  a->inflight.assign(prm->E, 0);
  a->score.assign(prm->E, 0);
  a->scratch.assign(prm->P, 0);
  for (int e = 0; e < prm->E; ++e) {
    uint64_t held[3];
    for (int p = 0; p < 3; ++p) {
      held[p] = 0;
      rimuru_view_pages(expert_view, 3ull * e + p, nullptr, 0, &held[p]);
    }
    const uint64_t P = static_cast<uint64_t>(prm->P);
    if (held[0] == P && held[1] == P && held[2] == P) {
      a->resident[e] = 1;
    } else if (held[0] || held[1] || held[2]) {
      delete a;
      return rimuru_fail(RIMURU_EINVAL, "adjuster_create: expert %d is partly resident", e);
    }
  }
  *out = a;
  return RIMURU_OK;
}

extern "C" rimuru_status rimuru_adjuster_destroy(rimuru_adjuster* adj) {
  delete adj;
  return RIMURU_OK;
}

extern "C" rimuru_status rimuru_adjuster_step(rimuru_adjuster* a, uint64_t demand_blocks, const int32_t* routed,
                                              const uint8_t* needed, int32_t* evicted, int32_t* n_evicted,
                                              int32_t* loaded, int32_t* n_loaded, int64_t* kv_moved) {
  if (a == nullptr || needed == nullptr || evicted == nullptr || n_evicted == nullptr || loaded == nullptr ||
      n_loaded == nullptr)
    return rimuru_fail(RIMURU_EINVAL, "adjuster_step: NULL argument");
  const int E = a->prm.E;
  if (routed != nullptr)
    for (int e = 0; e < E; ++e)
      if (routed[e] < 0) return rimuru_fail(RIMURU_EINVAL, "adjuster_step: routed[%d] < 0", e);
  if (demand_blocks > ~0ull / a->kv_page - static_cast<uint64_t>(a->prm.headroom_blocks))
    return rimuru_fail(RIMURU_EINVAL, "adjuster_step: demand_blocks out of range");
  for (int e = 0; e < E; ++e) {
    const uint64_t s = a->score[e];
    a->score[e] = s - (s >> a->prm.shift) + (routed ? static_cast<uint64_t>(routed[e]) << 16 : 0);
  }
  StepState st;
  st.pinned.resize(E);
  st.evicted_now.assign(E, 0);
  for (int e = 0; e < E; ++e) st.pinned[e] = (needed[e] || a->inflight[e]) ? 1 : 0;
  st.evicted = evicted;
  st.loaded = loaded;
  rimuru_status s = demand_loads(a, needed, st);
  if (s == RIMURU_OK) s = move_fence(a, demand_blocks, st);
  if (s == RIMURU_OK) s = prefetch(a, st);
  *n_evicted = st.n_evicted;
  *n_loaded = st.n_loaded;
  if (kv_moved) *kv_moved = st.moved;
  return s;
}

extern "C" rimuru_status rimuru_adjuster_upload_done(rimuru_adjuster* a, int32_t e) {
  if (a == nullptr || e < 0 || e >= a->prm.E || !a->inflight[e])
    return rimuru_fail(RIMURU_EINVAL, "adjuster_upload_done: expert %d has no upload in flight", e);
  a->inflight[e] = 0;
  return RIMURU_OK;
}

extern "C" rimuru_status rimuru_adjuster_state(const rimuru_adjuster* a, uint8_t* resident, uint8_t* in_flight,
                                               uint64_t* score) {
  if (a == nullptr) return rimuru_fail(RIMURU_EINVAL, "adjuster_state: NULL adjuster");
  for (int e = 0; e < a->prm.E; ++e) {
    if (resident) resident[e] = a->resident[e];
    if (in_flight) in_flight[e] = a->inflight[e];
    if (score) score[e] = a->score[e];
  }
  return RIMURU_OK;
}
