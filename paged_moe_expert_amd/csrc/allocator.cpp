// Multi-level split/merge page allocator over one shared page pool.
//
// Rimuru paper summary (thelatestinai.com), abstract and Figures 6-7: one
// shared page pool, a memory view per tensor type with its own page size, and
// huge-page alignment with a multi-level allocator that splits and merges
// pages. Explainer "Rimuru unifies serving memory" (learnaivisually.com),
// paragraph on moving the fence: a huge page splits into expert-sized pages,
// which may split into KV-sized pages; reclaiming merges back the same way; a
// huge page is never cut straight into KV blocks; one request's pages come
// from one parent when possible.
//
// The allocator hands out byte offsets into the pool and never touches device
// memory. All policy choices (lowest-address parent, lowest free slot, all-or
// nothing requests, budgets) are stated in rimuru.h.
#include <cstdarg>
#include <cstdio>
#include <map>
#include <memory>
#include <new>
#include <set>
#include <string>
#include <unordered_map>
#include <vector>

#include "rimuru.h"
#include "rimuru_internal.h"

namespace {

constexpr uint64_t kSplit = 1ull << 63;   // owners >= kSplit: split owner of a child view
constexpr uint64_t kFree = ~0ull;          // empty slot marker
constexpr uint64_t kNoBudget = ~0ull;

struct Parent {
  uint64_t base = 0;
  std::vector<uint64_t> slots;             // owner per slot or kFree
  uint32_t used = 0;
};

}  // namespace

struct rimuru_view {
  rimuru_pool* pool = nullptr;
  int id = 0;
  int kind = 0;
  uint64_t page = 0;
  rimuru_view* parent = nullptr;           // nullptr: cut from huge pages
  uint64_t parent_size = 0;
  uint32_t nslots = 0;
  std::map<uint64_t, Parent> parents;      // base -> parent
  std::set<uint64_t> avail;                // bases with a free slot
  std::unordered_map<uint64_t, std::vector<uint64_t>> owner_pages;
  std::unordered_map<uint64_t, std::map<uint64_t, uint32_t>> owner_parents;
  std::unordered_map<uint64_t, uint64_t> page_parent;  // page offset -> parent base
  uint64_t used = 0;                       // pages held by real owners
  uint64_t budget = kNoBudget;
};

struct rimuru_pool {
  uint64_t pool_bytes = 0;
  uint64_t huge = 0;
  uint64_t n_huge = 0;
  std::set<uint64_t> free_huge;            // huge page indices
  std::vector<std::unique_ptr<rimuru_view>> views;
};

namespace {

thread_local std::string g_err;

}  // namespace

rimuru_status rimuru_fail(rimuru_status code, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  g_err = buf;
  return code;
}

extern "C" const char* rimuru_last_error(void) { return g_err.c_str(); }
extern "C" int32_t rimuru_abi_version(void) { return RIMURU_ABI_VERSION; }

namespace {

bool take_page(rimuru_view* v, uint64_t owner, uint64_t* off_out);

// Obtain a new parent page for view v and register it as a parent of v.
bool new_parent(rimuru_view* v, uint64_t* base_out) {
  rimuru_pool* p = v->pool;
  uint64_t base;
  if (v->parent == nullptr) {
    if (p->free_huge.empty()) return false;
    auto it = p->free_huge.begin();
    base = *it * p->huge;
    p->free_huge.erase(it);
  } else {
    if (!take_page(v->parent, kSplit | static_cast<uint64_t>(v->id), &base)) return false;
  }
  Parent par;
  par.base = base;
  par.slots.assign(v->nslots, kFree);
  v->parents.emplace(base, std::move(par));
  v->avail.insert(base);
  *base_out = base;
  return true;
}

// One page for owner: a parent the owner already uses, else the lowest
// parent with a free slot, else a new parent; lowest free slot within it.
bool take_page(rimuru_view* v, uint64_t owner, uint64_t* off_out) {
  bool found = false;
  uint64_t base = 0;
  auto op = v->owner_parents.find(owner);
  if (op != v->owner_parents.end()) {
    for (auto& kv : op->second) {          // std::map: ascending base
      if (v->parents.at(kv.first).used < v->nslots) {
        base = kv.first;
        found = true;
        break;
      }
    }
  }
  if (!found && !v->avail.empty()) {
    base = *v->avail.begin();
    found = true;
  }
  if (!found && !new_parent(v, &base)) return false;
  Parent& par = v->parents.at(base);
  uint32_t slot = 0;
  while (par.slots[slot] != kFree) ++slot;
  par.slots[slot] = owner;
  par.used += 1;
  if (par.used == v->nslots) v->avail.erase(base);
  v->owner_parents[owner][base] += 1;
  uint64_t off = base + static_cast<uint64_t>(slot) * v->page;
  v->page_parent[off] = base;
  if (owner >= kSplit) v->owner_pages[owner].push_back(off);
  *off_out = off;
  return true;
}

void release_page(rimuru_view* v, uint64_t off, uint64_t owner) {
  auto pp = v->page_parent.find(off);
  uint64_t base = pp->second;
  v->page_parent.erase(pp);
  Parent& par = v->parents.at(base);
  uint32_t slot = static_cast<uint32_t>((off - base) / v->page);
  par.slots[slot] = kFree;
  if (par.used == v->nslots) v->avail.insert(base);
  par.used -= 1;
  auto& cnt = v->owner_parents[owner];
  if (--cnt[base] == 0) {
    cnt.erase(base);
    if (cnt.empty()) v->owner_parents.erase(owner);
  }
  if (par.used == 0) {                     // merge back into the parent level
    v->parents.erase(base);
    v->avail.erase(base);
    if (v->parent == nullptr) {
      v->pool->free_huge.insert(base / v->pool->huge);
    } else {
      uint64_t so = kSplit | static_cast<uint64_t>(v->id);
      auto& lst = v->parent->owner_pages[so];
      for (size_t i = 0; i < lst.size(); ++i) {
        if (lst[i] == base) {
          lst.erase(lst.begin() + static_cast<long>(i));
          break;
        }
      }
      if (lst.empty()) v->parent->owner_pages.erase(so);
      release_page(v->parent, base, so);
    }
  }
}

}  // namespace

extern "C" rimuru_status rimuru_pool_create(uint64_t pool_bytes, uint64_t huge_page_bytes,
                                            rimuru_pool** out) {
  if (out == nullptr) return rimuru_fail(RIMURU_EINVAL, "pool_create: out is NULL");
  *out = nullptr;
  if (huge_page_bytes == 0 || huge_page_bytes % 128 != 0 || pool_bytes < huge_page_bytes)
    return rimuru_fail(RIMURU_EINVAL, "pool_create: huge page %llu must be a positive multiple "
                       "of 128 and <= pool %llu", (unsigned long long)huge_page_bytes,
                       (unsigned long long)pool_bytes);
  try {
    auto* p = new rimuru_pool;
    p->pool_bytes = pool_bytes;
    p->huge = huge_page_bytes;
    p->n_huge = pool_bytes / huge_page_bytes;
    for (uint64_t i = 0; i < p->n_huge; ++i) p->free_huge.insert(p->free_huge.end(), i);
    *out = p;
  } catch (const std::bad_alloc&) {
    return rimuru_fail(RIMURU_ENOMEM, "pool_create: host allocation failed");
  }
  return RIMURU_OK;
}

extern "C" rimuru_status rimuru_pool_destroy(rimuru_pool* pool) {
  delete pool;
  return RIMURU_OK;
}

extern "C" rimuru_status rimuru_view_map(rimuru_pool* pool, int32_t kind, uint64_t page_bytes,
                                         rimuru_view* parent, rimuru_view** out) {
  if (pool == nullptr || out == nullptr) return rimuru_fail(RIMURU_EINVAL, "view_map: NULL argument");
  *out = nullptr;
  if (kind < 0 || kind > 3) return rimuru_fail(RIMURU_EINVAL, "view_map: unknown kind %d", kind);
  if (page_bytes == 0 || page_bytes % 128 != 0)
    return rimuru_fail(RIMURU_EINVAL, "view_map: page %llu is not a positive multiple of 128",
                       (unsigned long long)page_bytes);
  uint64_t psize;
  if (parent == nullptr) {
    psize = pool->huge;
    if (psize % page_bytes != 0)
      return rimuru_fail(RIMURU_EINVAL, "view_map: page %llu does not divide the huge page %llu",
                         (unsigned long long)page_bytes, (unsigned long long)psize);
    if (kind == RIMURU_VIEW_KV && page_bytes != psize)
      return rimuru_fail(RIMURU_EINVAL, "view_map: a KV view may not be cut straight from huge "
                         "pages; give it an expert-sized parent view");
  } else {
    if (parent->pool != pool) return rimuru_fail(RIMURU_EINVAL, "view_map: parent is from another pool");
    psize = parent->page;
    if (page_bytes > psize)
      return rimuru_fail(RIMURU_EINVAL, "view_map: page %llu exceeds its parent page %llu",
                         (unsigned long long)page_bytes, (unsigned long long)psize);
  }
  try {
    auto v = std::make_unique<rimuru_view>();
    v->pool = pool;
    v->id = static_cast<int>(pool->views.size());
    v->kind = kind;
    v->page = page_bytes;
    v->parent = parent;
    v->parent_size = psize;
    v->nslots = static_cast<uint32_t>(psize / page_bytes);
    *out = v.get();
    pool->views.push_back(std::move(v));
  } catch (const std::bad_alloc&) {
    return rimuru_fail(RIMURU_ENOMEM, "view_map: host allocation failed");
  }
  return RIMURU_OK;
}

extern "C" rimuru_status rimuru_view_alloc(rimuru_view* v, uint64_t owner, uint64_t n_pages,
                                           int64_t* out_offsets) {
  if (v == nullptr || out_offsets == nullptr || n_pages == 0 || owner >= kSplit)
    return rimuru_fail(RIMURU_EINVAL, "view_alloc: bad argument (view %p, owner %llu, n %llu)",
                       (void*)v, (unsigned long long)owner, (unsigned long long)n_pages);
  if (v->budget != kNoBudget && (v->used + n_pages) * v->page > v->budget)
    return rimuru_fail(RIMURU_ENOMEM, "view_alloc: %llu pages exceed the view budget",
                       (unsigned long long)n_pages);
  std::vector<uint64_t> got;
  try {
    got.reserve(n_pages);
    for (uint64_t i = 0; i < n_pages; ++i) {
      uint64_t off;
      if (!take_page(v, owner, &off)) {
        for (size_t j = got.size(); j-- > 0;) release_page(v, got[j], owner);
        return rimuru_fail(RIMURU_ENOMEM, "view_alloc: pool exhausted after %llu of %llu pages",
                           (unsigned long long)i, (unsigned long long)n_pages);
      }
      got.push_back(off);
    }
    auto& lst = v->owner_pages[owner];
    lst.insert(lst.end(), got.begin(), got.end());
  } catch (const std::bad_alloc&) {
    return rimuru_fail(RIMURU_ENOMEM, "view_alloc: host allocation failed");
  }
  v->used += n_pages;
  for (uint64_t i = 0; i < n_pages; ++i) out_offsets[i] = static_cast<int64_t>(got[i]);
  return RIMURU_OK;
}

extern "C" rimuru_status rimuru_view_free(rimuru_view* v, uint64_t owner) {
  if (v == nullptr || owner >= kSplit) return rimuru_fail(RIMURU_EINVAL, "view_free: bad argument");
  auto it = v->owner_pages.find(owner);
  if (it == v->owner_pages.end() || it->second.empty())
    return rimuru_fail(RIMURU_EINVAL, "view_free: owner %llu holds no page in this view",
                       (unsigned long long)owner);
  std::vector<uint64_t> pages = std::move(it->second);
  v->owner_pages.erase(it);
  for (uint64_t off : pages) release_page(v, off, owner);
  v->used -= pages.size();
  return RIMURU_OK;
}

extern "C" rimuru_status rimuru_view_pages(const rimuru_view* v, uint64_t owner,
                                           int64_t* out_offsets, uint64_t cap, uint64_t* n_out) {
  if (v == nullptr || n_out == nullptr) return rimuru_fail(RIMURU_EINVAL, "view_pages: NULL argument");
  auto it = v->owner_pages.find(owner);
  uint64_t n = (it == v->owner_pages.end()) ? 0 : it->second.size();
  *n_out = n;
  if (n == 0) return RIMURU_OK;
  if (n > cap || out_offsets == nullptr)
    return rimuru_fail(RIMURU_EINVAL, "view_pages: %llu pages exceed capacity %llu",
                       (unsigned long long)n, (unsigned long long)cap);
  for (uint64_t i = 0; i < n; ++i) out_offsets[i] = static_cast<int64_t>(it->second[i]);
  return RIMURU_OK;
}

extern "C" rimuru_status rimuru_view_set_budget(rimuru_view* v, uint64_t bytes) {
  if (v == nullptr) return rimuru_fail(RIMURU_EINVAL, "view_set_budget: NULL view");
  if (bytes != kNoBudget && bytes < v->used * v->page)
    return rimuru_fail(RIMURU_EBUSY, "view_set_budget: %llu bytes is below the %llu held",
                       (unsigned long long)bytes, (unsigned long long)(v->used * v->page));
  v->budget = bytes;
  return RIMURU_OK;
}

extern "C" rimuru_status rimuru_pool_transfer(rimuru_pool* pool, rimuru_view* from, rimuru_view* to,
                                              uint64_t bytes) {
  if (pool == nullptr || from == nullptr || to == nullptr || from == to || from->pool != pool ||
      to->pool != pool)
    return rimuru_fail(RIMURU_EINVAL, "pool_transfer: bad views");
  if (from->budget == kNoBudget || to->budget == kNoBudget)
    return rimuru_fail(RIMURU_EINVAL, "pool_transfer: both views need a finite budget");
  if (from->budget < bytes || from->budget - bytes < from->used * from->page)
    return rimuru_fail(RIMURU_EBUSY, "pool_transfer: the source view holds too much to give %llu",
                       (unsigned long long)bytes);
  if (to->budget + bytes < to->budget) return rimuru_fail(RIMURU_EINVAL, "pool_transfer: overflow");
  from->budget -= bytes;
  to->budget += bytes;
  return RIMURU_OK;
}

extern "C" rimuru_status rimuru_view_usage(const rimuru_view* v, uint64_t* used_bytes,
                                           uint64_t* budget_bytes) {
  if (v == nullptr) return rimuru_fail(RIMURU_EINVAL, "view_usage: NULL view");
  if (used_bytes) *used_bytes = v->used * v->page;
  if (budget_bytes) *budget_bytes = v->budget;
  return RIMURU_OK;
}

extern "C" rimuru_status rimuru_view_info(const rimuru_view* v, rimuru_pool** pool, int32_t* kind,
                                          uint64_t* page_bytes) {
  if (v == nullptr) return rimuru_fail(RIMURU_EINVAL, "view_info: NULL view");
  if (pool) *pool = v->pool;
  if (kind) *kind = v->kind;
  if (page_bytes) *page_bytes = v->page;
  return RIMURU_OK;
}

extern "C" rimuru_status rimuru_pool_stats(const rimuru_pool* pool, rimuru_pool_stats_t* out) {
  if (pool == nullptr || out == nullptr) return rimuru_fail(RIMURU_EINVAL, "pool_stats: NULL argument");
  rimuru_pool_stats_t s{};
  s.huge_pages = pool->n_huge;
  s.huge_free = pool->free_huge.size();
  s.bytes_free = s.huge_free * pool->huge;
  s.waste_bytes = pool->pool_bytes - pool->n_huge * pool->huge;
  for (const auto& vp : pool->views) {
    const rimuru_view* v = vp.get();
    s.bytes_per_kind[v->kind] += v->used * v->page;
    s.split_parents += v->parents.size();
    for (const auto& kv : v->parents) {
      s.bytes_free += static_cast<uint64_t>(v->nslots - kv.second.used) * v->page;
      s.waste_bytes += v->parent_size - static_cast<uint64_t>(v->nslots) * v->page;
    }
  }
  *out = s;
  return RIMURU_OK;
}

extern "C" rimuru_status rimuru_pool_check(const rimuru_pool* pool) {
  if (pool == nullptr) return rimuru_fail(RIMURU_EINVAL, "pool_check: NULL pool");
  // Intervals held by real owners must not overlap.
  std::map<uint64_t, uint64_t> iv;
  for (const auto& vp : pool->views) {
    const rimuru_view* v = vp.get();
    uint64_t n_real = 0;
    for (const auto& op : v->owner_pages) {
      if (op.first >= kSplit) continue;
      n_real += op.second.size();
      for (uint64_t off : op.second) {
        auto pp = v->page_parent.find(off);
        if (pp == v->page_parent.end())
          return rimuru_fail(RIMURU_EINVAL, "pool_check: page %llu has no parent", (unsigned long long)off);
        const Parent& par = v->parents.at(pp->second);
        uint64_t slot = (off - par.base) / v->page;
        if ((off - par.base) % v->page != 0 || slot >= v->nslots || par.slots[slot] != op.first)
          return rimuru_fail(RIMURU_EINVAL, "pool_check: page %llu is misplaced", (unsigned long long)off);
        if (!iv.emplace(off, off + v->page).second)
          return rimuru_fail(RIMURU_EINVAL, "pool_check: page %llu held twice", (unsigned long long)off);
      }
    }
    if (n_real != v->used) return rimuru_fail(RIMURU_EINVAL, "pool_check: used count drifted");
    for (const auto& kv : v->parents) {
      const Parent& par = kv.second;
      uint32_t u = 0;
      for (uint64_t s : par.slots) u += (s != kFree);
      if (u != par.used || u == 0) return rimuru_fail(RIMURU_EINVAL, "pool_check: parent count drifted");
      if (v->parent == nullptr) {
        if (par.base % pool->huge != 0 || pool->free_huge.count(par.base / pool->huge))
          return rimuru_fail(RIMURU_EINVAL, "pool_check: parent on a free or unaligned huge page");
      } else {
        auto it = v->parent->owner_pages.find(kSplit | static_cast<uint64_t>(v->id));
        bool ok = false;
        if (it != v->parent->owner_pages.end())
          for (uint64_t b : it->second) ok |= (b == par.base);
        if (!ok) return rimuru_fail(RIMURU_EINVAL, "pool_check: parent not split from its parent view");
      }
      if ((par.used < v->nslots) != (v->avail.count(par.base) == 1))
        return rimuru_fail(RIMURU_EINVAL, "pool_check: free-slot index drifted");
    }
  }
  uint64_t prev_end = 0;
  for (const auto& kv : iv) {
    if (kv.first < prev_end) return rimuru_fail(RIMURU_EINVAL, "pool_check: overlapping pages");
    prev_end = kv.second;
  }
  rimuru_pool_stats_t s;
  rimuru_pool_stats(pool, &s);
  uint64_t sum = s.bytes_free + s.waste_bytes;
  for (int i = 0; i < 4; ++i) sum += s.bytes_per_kind[i];
  if (sum != pool->pool_bytes) return rimuru_fail(RIMURU_EINVAL, "pool_check: bytes not conserved");
  return RIMURU_OK;
}
