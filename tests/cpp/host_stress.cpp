// Seeded stress of the host side of librimuru (pool, views, split/merge
// allocator, budget transfers, adjuster policy) through its C ABI, built
// with AddressSanitizer and UndefinedBehaviorSanitizer by
// tests/test_host_sanitizers.py. Every step runs the pool's full internal
// consistency check; the run ends with every page freed and the pool merged
// back to whole huge pages.
#include <cstdint>
#include <cstdio>
#include <cstdlib>
#include <map>
#include <vector>

#include "rimuru.h"

namespace {

uint64_t lcg_state = 0x9E3779B97F4A7C15ull;
uint64_t next_u64() {                       // SplitMix64
  uint64_t z = (lcg_state += 0x9E3779B97F4A7C15ull);
  z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
  z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
  return z ^ (z >> 31);
}
uint64_t below(uint64_t n) { return next_u64() % n; }

int fails = 0;
void expect(bool ok, const char* what) {
  if (!ok) {
    std::fprintf(stderr, "FAIL: %s (%s)\n", what, rimuru_last_error());
    ++fails;
  }
}

void allocator_stress(uint64_t seed) {
  lcg_state = seed;
  const uint64_t KIB = 1024, MIB = 1024 * KIB;
  rimuru_pool* pool = nullptr;
  expect(rimuru_pool_create(256 * MIB + 512 * KIB, 3 * MIB, &pool) == RIMURU_OK, "pool_create");
  rimuru_view *xv = nullptr, *kv = nullptr;
  expect(rimuru_view_map(pool, RIMURU_VIEW_EXPERT, 64 * KIB, nullptr, &xv) == RIMURU_OK, "map expert");
  expect(rimuru_view_map(pool, RIMURU_VIEW_KV, 32 * KIB, xv, &kv) == RIMURU_OK, "map kv");
  std::map<uint64_t, uint64_t> live_x, live_k;   // owner -> pages
  std::vector<int64_t> offs(4096);
  for (int step = 0; step < 2000; ++step) {
    const uint64_t r = below(100);
    if (r < 35) {                                // KV request
      const uint64_t owner = 1000000 + below(400), n = 1 + below(64);
      const rimuru_status s = rimuru_view_alloc(kv, owner, n, offs.data());
      expect(s == RIMURU_OK || s == RIMURU_ENOMEM, "kv alloc status");
      if (s == RIMURU_OK) live_k[owner] += n;
    } else if (r < 55) {                         // expert projection (48 pages)
      const uint64_t owner = below(300);
      if (!live_x.count(owner)) {
        const rimuru_status s = rimuru_view_alloc(xv, owner, 48, offs.data());
        expect(s == RIMURU_OK || s == RIMURU_ENOMEM, "expert alloc status");
        if (s == RIMURU_OK) live_x[owner] = 48;
      }
    } else if (r < 80 && !live_k.empty()) {      // free a KV request
      auto it = live_k.begin();
      std::advance(it, static_cast<long>(below(live_k.size())));
      expect(rimuru_view_free(kv, it->first) == RIMURU_OK, "kv free");
      live_k.erase(it);
    } else if (r < 95 && !live_x.empty()) {      // free an expert projection
      auto it = live_x.begin();
      std::advance(it, static_cast<long>(below(live_x.size())));
      expect(rimuru_view_free(xv, it->first) == RIMURU_OK, "expert free");
      live_x.erase(it);
    } else {                                     // budgets: cap, move, lift
      uint64_t used_k = 0, budget_k = 0, used_x = 0, budget_x = 0;
      rimuru_view_usage(kv, &used_k, &budget_k);
      rimuru_view_usage(xv, &used_x, &budget_x);
      rimuru_view_set_budget(kv, used_k + 64 * 32 * KIB);
      rimuru_view_set_budget(xv, used_x + 96 * 64 * KIB);
      const rimuru_status s = rimuru_pool_transfer(pool, kv, xv, 32 * 32 * KIB);
      expect(s == RIMURU_OK || s == RIMURU_EBUSY, "transfer status");
      rimuru_view_set_budget(kv, UINT64_MAX);
      rimuru_view_set_budget(xv, UINT64_MAX);
    }
    // error paths leave the pool as it was
    expect(rimuru_view_free(kv, 999) == RIMURU_EINVAL, "free of an unknown owner");
    expect(rimuru_view_alloc(kv, 1, 0, offs.data()) == RIMURU_EINVAL, "zero pages");
    expect(rimuru_pool_check(pool) == RIMURU_OK, "pool_check");
    if (fails) break;
  }
  for (auto& o : live_k) expect(rimuru_view_free(kv, o.first) == RIMURU_OK, "final kv free");
  for (auto& o : live_x) expect(rimuru_view_free(xv, o.first) == RIMURU_OK, "final expert free");
  rimuru_pool_stats_t st{};
  expect(rimuru_pool_stats(pool, &st) == RIMURU_OK, "stats");
  expect(st.huge_free == st.huge_pages && st.split_parents == 0, "everything merged back");
  expect(rimuru_pool_check(pool) == RIMURU_OK, "final pool_check");
  expect(rimuru_pool_destroy(pool) == RIMURU_OK, "pool_destroy");
}

void adjuster_stress(uint64_t seed) {
  lcg_state = seed;
  const uint64_t KIB = 1024, MIB = 1024 * KIB;
  const int E = 32, P = 1;
  const uint64_t page = 3 * MIB, block = 32 * KIB;
  rimuru_pool* pool = nullptr;
  expect(rimuru_pool_create(160 * page, page, &pool) == RIMURU_OK, "adj pool_create");
  rimuru_view *xv = nullptr, *kv = nullptr;
  rimuru_view_map(pool, RIMURU_VIEW_EXPERT, page, nullptr, &xv);
  rimuru_view_map(pool, RIMURU_VIEW_KV, block, xv, &kv);
  std::vector<int64_t> offs(8);
  for (int e = 0; e < E; ++e)
    for (int p = 0; p < 3; ++p) expect(rimuru_view_alloc(xv, 3 * e + p, P, offs.data()) == RIMURU_OK, "place");
  rimuru_view_set_budget(xv, static_cast<uint64_t>(E) * 3 * page);
  rimuru_view_set_budget(kv, 160 * page - static_cast<uint64_t>(E) * 3 * page);
  rimuru_adjuster_params prm{E, P, 20, 64, 512, 3, 2};
  rimuru_adjuster* adj = nullptr;
  expect(rimuru_adjuster_create(pool, xv, kv, &prm, &adj) == RIMURU_OK, "adjuster_create");
  std::vector<int32_t> routed(E), ev(E), ld(E);
  std::vector<uint8_t> needed(E);
  uint64_t demand = 0;
  for (int step = 0; step < 400; ++step) {
    demand = (step % 100 < 60) ? demand + below(200) : (demand > 300 ? demand - below(300) : 0);
    for (int e = 0; e < E; ++e) {
      routed[e] = static_cast<int32_t>(below(4) == 0 ? below(20) : 0);
      needed[e] = 0;
    }
    for (int i = 0; i < 4; ++i) needed[below(E)] = 1;
    int32_t ne = 0, nl = 0;
    int64_t moved = 0;
    const rimuru_status s = rimuru_adjuster_step(adj, demand, routed.data(), needed.data(), ev.data(), &ne,
                                                 ld.data(), &nl, &moved);
    expect(s == RIMURU_OK || s == RIMURU_ENOMEM, "adjuster_step status");
    expect(ne >= 0 && ne <= E && nl >= 0 && nl <= E, "adjuster counts");
    for (int i = 0; i < nl; ++i) expect(rimuru_adjuster_upload_done(adj, ld[i]) == RIMURU_OK, "upload_done");
    expect(rimuru_pool_check(pool) == RIMURU_OK, "adj pool_check");
    if (fails) break;
  }
  expect(rimuru_adjuster_destroy(adj) == RIMURU_OK, "adjuster_destroy");
  expect(rimuru_pool_destroy(pool) == RIMURU_OK, "adj pool_destroy");
}

}  // namespace

int main(int argc, char** argv) {
  const uint64_t seed = argc > 1 ? std::strtoull(argv[1], nullptr, 10) : 1;
  allocator_stress(seed);
  adjuster_stress(seed + 1);
  if (fails) return 1;
  std::printf("host stress ok (seed %llu)\n", static_cast<unsigned long long>(seed));
  return 0;
}
