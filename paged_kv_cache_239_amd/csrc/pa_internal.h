// Internal definitions shared by the host manager (pa_host.cpp) and the
// device launchers (pa_attention.hip, pa_cache.hip).  Not part of the public ABI.
#pragma once

#include <cstddef>
#include <cstdint>
#include <string>
#include <vector>

#include "pa.h"

struct pa_pool {
  // shape
  int L = 0, Hkv = 0, d = 0, B = 0, P = 0;
  pa_dtype dtype = PA_F16;
  // device memory (caller-owned)
  char* base = nullptr;
  size_t bytes = 0;
  size_t tile_bytes = 0;  // one block of one layer's K (or V): Hkv * B * d * 2
  size_t slab_bytes = 0;  // P * tile_bytes
  // host manager state
  std::vector<int32_t> ref;   // refcount per physical block
  std::vector<int32_t> ring;  // FIFO free list storage (capacity P)
  int64_t head = 0;           // index of the free list's head in ring
  int32_t nfree = 0;          // entries on the free list
  // counters
  int64_t allocs = 0, cows = 0, releases = 0;
  int32_t live_high_water = 0;

  char* k_slab(int layer) const { return base + (size_t)(2 * layer) * slab_bytes; }
  char* v_slab(int layer) const { return base + (size_t)(2 * layer + 1) * slab_bytes; }
};

namespace pa_detail {

// Records `msg` as the calling thread's last error and returns `st`.
pa_status fail(pa_status st, const std::string& msg);
void clear_error();

}  // namespace pa_detail
