// Helpers shared by the device translation units (pa_attention.hip,
// pa_cache.hip).  Internal; not part of the public ABI.
#pragma once

#include <hip/hip_runtime.h>

#include <cstdint>
#include <cstdlib>
#include <string>

#include "pa_internal.h"

namespace {

constexpr int kD = 128;            // head dimension of every compiled kernel
constexpr int kRowBytes = kD * 2;  // one token of one head: 256 bytes

typedef unsigned int u32x4_t __attribute__((ext_vector_type(4)));

// 16-byte load with the non-temporal (streaming) cache hint
__device__ __forceinline__ uint4 nt_load16(const char* p) {
  const u32x4_t v = __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(p));
  return make_uint4(v.x, v.y, v.z, v.w);
}

// 16-byte store with the non-temporal hint
__device__ __forceinline__ void nt_store16(char* p, const uint4 x) {
  const u32x4_t v = {x.x, x.y, x.z, x.w};
  __builtin_nontemporal_store(v, reinterpret_cast<u32x4_t*>(p));
}

inline pa_status hip_check(hipError_t e, const char* what) {
  if (e == hipSuccess) return PA_OK;
  return pa_detail::fail(PA_ERR_HIP, std::string(what) + ": " + hipGetErrorString(e));
}

inline bool aligned(const void* p, size_t a) { return reinterpret_cast<uintptr_t>(p) % a == 0; }

}  // namespace
