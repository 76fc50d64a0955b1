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

}  // extern "C"
