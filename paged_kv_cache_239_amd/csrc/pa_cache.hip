// Cache maintenance kernels for gfx950: the cache write of new tokens and
// whole-block copies.
//
// Sources (page title, section):
//   "vLLM PagedAttention and continuous batching" -- "PagedAttention: fixed
//     blocks, non-contiguous physical memory" (a token's keys and values go
//     to the slot its block table entry names), "Sharing with reference
//     counts and copy-on-write" (a write into a block that others map
//     copies that one block first).

#include "pa_device_common.h"

using pa_detail::fail;

namespace {

// ---------------------------------------------------------------------------
// write_kv: one workgroup per token
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void write_kv_kernel(char* kslab, char* vslab, const uint4* k, const uint4* v,
                                                       const int64_t* slots, int Hkv, int B, int64_t nslots,
                                                       uint64_t tile_bytes) {
  const int s = blockIdx.x;
  const int64_t slot = slots[s];
  if (slot < 0 || slot >= nslots) return;
  const int64_t blk = slot / B;
  const int off = (int)(slot % B);
  const int chunks_per_row = kRowBytes / 16;  // 16
  const int chunks = Hkv * chunks_per_row;
  for (int i = threadIdx.x; i < chunks; i += blockDim.x) {
    const int h = i / chunks_per_row;
    const int w = i % chunks_per_row;
    const uint64_t dst = (uint64_t)blk * tile_bytes + ((uint64_t)h * B + off) * kRowBytes + (uint64_t)w * 16;
    *reinterpret_cast<uint4*>(kslab + dst) = k[(size_t)s * chunks + i];
    *reinterpret_cast<uint4*>(vslab + dst) = v[(size_t)s * chunks + i];
  }
}

// ---------------------------------------------------------------------------
// copy_blocks: one workgroup per (pair, slab); it streams the whole tile with
// kCopyUnroll 16-byte non-temporal loads per thread in flight
// ---------------------------------------------------------------------------
constexpr int kCopyUnroll = 8;
constexpr int kCopyThreads = 256;

__global__ __launch_bounds__(kCopyThreads) void copy_blocks_kernel(char* base, const int32_t* pairs, int P,
                                                                   uint64_t tile_bytes, uint64_t slab_bytes) {
  const int pr = blockIdx.y;
  const int32_t src = pairs[2 * pr];
  const int32_t dst = pairs[2 * pr + 1];
  if (src < 0 || src >= P || dst < 0 || dst >= P || src == dst) return;
  char* slab = base + (uint64_t)blockIdx.x * slab_bytes;
  const char* from = slab + (uint64_t)src * tile_bytes;
  char* to = slab + (uint64_t)dst * tile_bytes;
  const uint64_t nchunks = tile_bytes / 16;
  for (uint64_t first = threadIdx.x; first < nchunks; first += (uint64_t)kCopyThreads * kCopyUnroll) {
    uint4 tmp[kCopyUnroll];
#pragma unroll
    for (int u = 0; u < kCopyUnroll; ++u) {
      const uint64_t i = first + (uint64_t)u * kCopyThreads;
      if (i < nchunks) tmp[u] = nt_load16(from + i * 16);
    }
#pragma unroll
    for (int u = 0; u < kCopyUnroll; ++u) {
      const uint64_t i = first + (uint64_t)u * kCopyThreads;
      if (i < nchunks) {
        nt_store16(to + i * 16, tmp[u]);
      }
    }
  }
}

// ---------------------------------------------------------------------------
// swap_blocks: copy_blocks between two pools (one may be pinned host memory,
// read or written by the GPU through its device-mapped address)
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(kCopyThreads) void swap_blocks_kernel(const char* from, char* to, const int32_t* pairs,
                                                                   int P_from, int P_to, uint64_t tile_bytes,
                                                                   uint64_t slab_from, uint64_t slab_to) {
  const int pr = blockIdx.y;
  const int32_t src = pairs[2 * pr];
  const int32_t dst = pairs[2 * pr + 1];
  if (src < 0 || src >= P_from || dst < 0 || dst >= P_to) return;
  const char* a = from + (uint64_t)blockIdx.x * slab_from + (uint64_t)src * tile_bytes;
  char* b = to + (uint64_t)blockIdx.x * slab_to + (uint64_t)dst * tile_bytes;
  const uint64_t nchunks = tile_bytes / 16;
  for (uint64_t first = threadIdx.x; first < nchunks; first += (uint64_t)kCopyThreads * kCopyUnroll) {
    uint4 tmp[kCopyUnroll];
#pragma unroll
    for (int u = 0; u < kCopyUnroll; ++u) {
      const uint64_t i = first + (uint64_t)u * kCopyThreads;
      if (i < nchunks) tmp[u] = nt_load16(a + i * 16);
    }
#pragma unroll
    for (int u = 0; u < kCopyUnroll; ++u) {
      const uint64_t i = first + (uint64_t)u * kCopyThreads;
      if (i < nchunks) nt_store16(b + i * 16, tmp[u]);
    }
  }
}

// The address at which kernels reach a pool's memory: the memory itself for
// device memory, the mapped alias for pinned host memory.
pa_status device_view(const pa_pool* pool, char** out) {
  hipPointerAttribute_t attr;
  const hipError_t e = hipPointerGetAttributes(&attr, pool->base);
  if (e != hipSuccess) {
    (void)hipGetLastError();
    return fail(PA_ERR_INVALID_ARG, "pool memory is neither device memory nor pinned host memory");
  }
  if (attr.type == hipMemoryTypeDevice) {
    *out = pool->base;
    return PA_OK;
  }
  if (attr.type == hipMemoryTypeHost && attr.devicePointer != nullptr) {
    // only memory from hipHostMalloc has host-allocation flags
    unsigned int flags = 0;
    if (hipHostGetFlags(&flags, pool->base) != hipSuccess) {
      (void)hipGetLastError();
      return fail(PA_ERR_INVALID_ARG, "host pool memory was not allocated with hipHostMalloc");
    }
    *out = static_cast<char*>(attr.devicePointer);
    return PA_OK;
  }
  return fail(PA_ERR_INVALID_ARG, "pool memory is not mapped into the device's address space");
}

}  // namespace

extern "C" {

pa_status pa_write_kv(pa_pool* pool, int layer, const void* k, const void* v, const int64_t* slot_mapping, int S,
                      hipStream_t stream) {
  pa_detail::clear_error();
  if (!pool) return fail(PA_ERR_INVALID_ARG, "pool is NULL");
  if (layer < 0 || layer >= pool->L) return fail(PA_ERR_INVALID_ARG, "layer out of range");
  if (S < 0) return fail(PA_ERR_INVALID_ARG, "negative S");
  if (S == 0) return PA_OK;
  if (pool->d != kD) return fail(PA_ERR_UNSUPPORTED, "head dimension must be 128");
  if (!k || !v || !slot_mapping) return fail(PA_ERR_INVALID_ARG, "NULL device pointer");
  if (!aligned(k, 16) || !aligned(v, 16) || !aligned(slot_mapping, 8))
    return fail(PA_ERR_INVALID_ARG, "k and v must be 16-byte aligned, slot_mapping 8-byte aligned");
  if (S > 2147483647) return fail(PA_ERR_INVALID_ARG, "S too large");
  hipLaunchKernelGGL(write_kv_kernel, dim3(S), dim3(256), 0, stream, pool->k_slab(layer), pool->v_slab(layer),
                     static_cast<const uint4*>(k), static_cast<const uint4*>(v), slot_mapping, pool->Hkv, pool->B,
                     (int64_t)pool->P * pool->B, (uint64_t)pool->tile_bytes);
  return hip_check(hipGetLastError(), "write_kv launch");
}

pa_status pa_copy_blocks(pa_pool* pool, const int32_t* pairs, int N, hipStream_t stream) {
  pa_detail::clear_error();
  if (!pool) return fail(PA_ERR_INVALID_ARG, "pool is NULL");
  if (N < 0) return fail(PA_ERR_INVALID_ARG, "negative N");
  if (N == 0) return PA_OK;
  if (!pairs || !aligned(pairs, 4)) return fail(PA_ERR_INVALID_ARG, "pairs must be a 4-byte aligned device pointer");
  if (N > 65535) return fail(PA_ERR_INVALID_ARG, "at most 65535 pairs per call");
  if (pool->tile_bytes % 16) return fail(PA_ERR_UNSUPPORTED, "block size in bytes must be a multiple of 16");
  const dim3 grid((unsigned)(2 * pool->L), (unsigned)N);
  hipLaunchKernelGGL(copy_blocks_kernel, grid, dim3(kCopyThreads), 0, stream, pool->base, pairs, pool->P,
                     (uint64_t)pool->tile_bytes, (uint64_t)pool->slab_bytes);
  return hip_check(hipGetLastError(), "copy_blocks launch");
}

pa_status pa_swap_blocks(pa_pool* from, pa_pool* to, const int32_t* pairs, int N, hipStream_t stream) {
  pa_detail::clear_error();
  if (!from || !to) return fail(PA_ERR_INVALID_ARG, "pool is NULL");
  if (from->L != to->L || from->Hkv != to->Hkv || from->d != to->d || from->B != to->B || from->dtype != to->dtype)
    return fail(PA_ERR_INVALID_ARG, "pools differ in shape");
  if (N < 0) return fail(PA_ERR_INVALID_ARG, "negative N");
  if (N == 0) return PA_OK;
  if (!pairs || !aligned(pairs, 4)) return fail(PA_ERR_INVALID_ARG, "pairs must be a 4-byte aligned device pointer");
  if (N > 65535) return fail(PA_ERR_INVALID_ARG, "at most 65535 pairs per call");
  if (from->tile_bytes % 16) return fail(PA_ERR_UNSUPPORTED, "block size in bytes must be a multiple of 16");
  char* a = nullptr;
  char* b = nullptr;
  if (pa_status st = device_view(from, &a)) return st;
  if (pa_status st = device_view(to, &b)) return st;
  const dim3 grid((unsigned)(2 * from->L), (unsigned)N);
  hipLaunchKernelGGL(swap_blocks_kernel, grid, dim3(kCopyThreads), 0, stream, a, b, pairs, from->P, to->P,
                     (uint64_t)from->tile_bytes, (uint64_t)from->slab_bytes, (uint64_t)to->slab_bytes);
  return hip_check(hipGetLastError(), "swap_blocks launch");
}

}  // extern "C"
