// Dual-buffer expert upload (Rimuru paper summary, Figure 8): an evicted
// expert comes back from host memory directly into fresh expert-view pages
// by asynchronous host-to-device copies on the caller's stream (one per run
// of consecutive pages), so the upload overlaps the layer running on another
// stream and no staging buffer or device-to-device copy is involved.
#include <hip/hip_runtime.h>

#include <cstdint>

#include "rimuru.h"
#include "rimuru_internal.h"

extern "C" rimuru_status rimuru_expert_upload(void* pool_base, uint64_t pool_bytes, const int32_t* pt_rows,
                                              int32_t P, uint64_t page_bytes, const void* host_src,
                                              uint64_t proj_bytes, void* hip_stream) {
  if (pool_base == nullptr || pt_rows == nullptr || host_src == nullptr)
    return rimuru_fail(RIMURU_EINVAL, "expert_upload: a required pointer is NULL");
  if (reinterpret_cast<uintptr_t>(pool_base) % 256 != 0 || reinterpret_cast<uintptr_t>(host_src) % 16 != 0)
    return rimuru_fail(RIMURU_EINVAL, "expert_upload: pool_base needs 256-byte, host_src 16-byte alignment");
  if (P < 1 || page_bytes == 0 || page_bytes % 128 != 0 || proj_bytes == 0 || proj_bytes % 16 != 0 ||
      proj_bytes > static_cast<uint64_t>(P) * page_bytes)
    return rimuru_fail(RIMURU_EINVAL, "expert_upload: page %llu / projection %llu bytes / P %d do not fit",
                       (unsigned long long)page_bytes, (unsigned long long)proj_bytes, P);
  // every destination page inside the pool, before anything is enqueued
  for (int64_t i = 0; i < 3ll * P; ++i) {
    const int32_t pg = pt_rows[i];
    if (pg < 0 || (static_cast<uint64_t>(pg) + 1) * page_bytes > pool_bytes)
      return rimuru_fail(RIMURU_ERANGE, "expert_upload: projection %lld, page %lld = %d lies outside the pool",
                         (long long)(i / P), (long long)(i % P), pg);
  }
  hipStream_t st = static_cast<hipStream_t>(hip_stream);
  uint8_t* pool = static_cast<uint8_t*>(pool_base);
  const uint8_t* src = static_cast<const uint8_t*>(host_src);
  // one copy per run of pages that are consecutive in the pool as well as
  // in the projection (the allocator gives an owner's pages from the same
  // parent when it can, so a projection is often a few runs rather than P
  // pages); pages past the projection's end stay unused
  for (int p = 0; p < 3; ++p) {
    const int32_t* row = pt_rows + static_cast<int64_t>(p) * P;
    for (int32_t q = 0; q < P;) {
      const uint64_t off = static_cast<uint64_t>(q) * page_bytes;
      if (off >= proj_bytes) break;
      int32_t r = q + 1;
      while (r < P && static_cast<uint64_t>(r) * page_bytes < proj_bytes && row[r] == row[r - 1] + 1) ++r;
      const uint64_t end = static_cast<uint64_t>(r) * page_bytes < proj_bytes ? static_cast<uint64_t>(r) * page_bytes
                                                                               : proj_bytes;
      const hipError_t err = hipMemcpyAsync(pool + static_cast<uint64_t>(row[q]) * page_bytes,
                                            src + static_cast<uint64_t>(p) * proj_bytes + off, end - off,
                                            hipMemcpyHostToDevice, st);
      if (err != hipSuccess)
        return rimuru_fail(RIMURU_EHIP, "expert_upload: copy of projection %d pages %d..%d: %s", p, q, r - 1,
                           hipGetErrorString(err));
      q = r;
    }
  }
  return RIMURU_OK;
}
