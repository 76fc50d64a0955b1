// Cache maintenance kernels for gfx950: the cache write of new tokens and
// whole-block copies.
//
// Sources (page title, section):
//   "vLLM PagedAttention and continuous batching" -- "PagedAttention: fixed
//     blocks, non-contiguous physical memory" (a token's keys and values go
//     to the slot its block table entry names), "Sharing with reference
//     counts and copy-on-write" (a write into a block that others map
//     copies that one block first).

#include <atomic>

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

// ---------------------------------------------------------------------------
// stream_tiles: the key and value rows decode attention reads (positions
// 0 .. n-1 of every sequence and head, through its block table) with the
// same 16-byte non-temporal loads and no arithmetic but an XOR of every
// word.  The work item is one mapped block of one sequence: its key tile and
// value tile of all heads, each Hkv * B * 256 contiguous bytes, read by the
// workgroup's threads in 4 KiB instructions (rows past the sequence's
// length skipped).  Items are numbered sequence by sequence and cut into
// one contiguous, equal range per workgroup, so every workgroup moves the
// same bytes; a workgroup first builds the prefix of block counts over the
// sequences in LDS (at most kStreamMaxSeqs), finds its first item by
// bisection and then walks its range.
// ---------------------------------------------------------------------------
constexpr int kStreamThreads = 256;
constexpr int kStreamUnroll = 8;       // 16-byte loads per thread per tile issued together
constexpr int kStreamMaxSeqs = 2048;   // 16 KiB of LDS for the prefix and lengths
constexpr int kStreamWgPerCu = 1;      // config-3 batch: 94 us per layer at 1, 97-100 at 2, 105-111 at 4

struct StreamArgs {
  const char* kslab;
  const char* vslab;
  const int32_t* tables;
  const int32_t* lens;
  uint32_t* checksum;     // [1]
  uint64_t tile_bytes;    // Hkv * B * 256: one block of one layer's keys (or values)
  int S, Hkv, P, maxb, max_ctx;
};

template <int BS>
__global__ __launch_bounds__(kStreamThreads) void stream_tiles_kernel(const StreamArgs a) {
  __shared__ int s_pre[kStreamMaxSeqs + 1];   // mapped blocks of sequences 0 .. s-1
  __shared__ int s_len[kStreamMaxSeqs];
  const int t = threadIdx.x;
  if (t < 64) {
    int carry = 0;
    for (int base = 0; base < a.S; base += 64) {
      const int s = base + t;
      int n = s < a.S ? a.lens[s] : 0;
      n = n < 0 ? 0 : (n > a.max_ctx ? a.max_ctx : n);
      int v = (n + BS - 1) / BS;
#pragma unroll
      for (int o = 1; o < 64; o <<= 1) {
        const int y = __shfl_up(v, o);
        if (t >= o) v += y;
      }
      if (s < a.S) {
        s_pre[s + 1] = carry + v;
        s_len[s] = n;
      }
      carry += __shfl(v, 63);
    }
    if (t == 0) s_pre[0] = 0;
  }
  __syncthreads();
  const int items = s_pre[a.S];
  const int per_wg = (items + (int)gridDim.x - 1) / (int)gridDim.x;
  const int i0 = (int)blockIdx.x * per_wg;
  const int i1 = min(items, i0 + per_wg);
  if (i0 >= i1) return;
  int lo = 0, hi = a.S - 1;
  while (lo < hi) {                   // the sequence holding item i0: last s with s_pre[s] <= i0
    const int mid = (lo + hi + 1) >> 1;
    if (s_pre[mid] <= i0) lo = mid; else hi = mid - 1;
  }
  // the walk is uniform: keep it in scalar registers, so that each block's
  // table entry is a scalar (constant-cache) load rather than a vector
  // memory round trip before the block's data loads
  int s = __builtin_amdgcn_readfirstlane(lo);
  const int nch = (int)(a.tile_bytes / 16);   // 16-byte chunks per tile; chunk k is row (k / 16) % BS
  uint32_t x = 0;
  for (int i = i0; i < i1; ++i) {
    while (__builtin_amdgcn_readfirstlane(s_pre[s + 1]) <= i) ++s;
    const int j = i - __builtin_amdgcn_readfirstlane(s_pre[s]);
    const int rows = min(BS, __builtin_amdgcn_readfirstlane(s_len[s]) - j * BS);
    int e = a.tables[(size_t)s * a.maxb + (j < a.maxb ? j : a.maxb - 1)];
    e = __builtin_amdgcn_readfirstlane(e < 0 ? 0 : (e >= a.P ? a.P - 1 : e));
    const char* kb = a.kslab + (uint64_t)e * a.tile_bytes;
    const char* vb = a.vslab + (uint64_t)e * a.tile_bytes;
    for (int k0 = t; k0 < nch; k0 += kStreamThreads * kStreamUnroll) {
      uint4 K[kStreamUnroll], V[kStreamUnroll];
#pragma unroll
      for (int u = 0; u < kStreamUnroll; ++u) {
        const int k = k0 + u * kStreamThreads;
        K[u] = make_uint4(0, 0, 0, 0);
        V[u] = make_uint4(0, 0, 0, 0);
        if (k < nch && ((k >> 4) % BS) < rows) {
          K[u] = nt_load16(kb + (uint64_t)k * 16);
          V[u] = nt_load16(vb + (uint64_t)k * 16);
        }
      }
#pragma unroll
      for (int u = 0; u < kStreamUnroll; ++u)
        x ^= K[u].x ^ K[u].y ^ K[u].z ^ K[u].w ^ V[u].x ^ V[u].y ^ V[u].z ^ V[u].w;
    }
  }
#pragma unroll
  for (int sh = 32; sh >= 1; sh >>= 1) x ^= __shfl_xor(x, sh);
  if ((t & 63) == 0 && x != 0) atomicXor(a.checksum, x);
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

pa_status pa_stream_tiles(pa_pool* pool, int layer, const int32_t* block_tables, int maxb,
                          const int32_t* context_lens, int S, int max_ctx, uint32_t* checksum, hipStream_t stream) {
  pa_detail::clear_error();
  if (!pool) return fail(PA_ERR_INVALID_ARG, "pool is NULL");
  if (layer < 0 || layer >= pool->L) return fail(PA_ERR_INVALID_ARG, "layer out of range");
  if (S < 0 || maxb <= 0 || max_ctx < 0) return fail(PA_ERR_INVALID_ARG, "bad S, maxb or max_ctx");
  if (S == 0 || max_ctx == 0) return PA_OK;
  if (S > kStreamMaxSeqs) return fail(PA_ERR_UNSUPPORTED, "at most 2048 sequences");
  if (pool->d != kD) return fail(PA_ERR_UNSUPPORTED, "head dimension must be 128");
  if ((int64_t)max_ctx > (int64_t)maxb * pool->B) return fail(PA_ERR_INVALID_ARG, "max_ctx exceeds maxb * B");
  if ((int64_t)S * maxb > 0x7fffffffLL) return fail(PA_ERR_UNSUPPORTED, "too many blocks");
  if (!block_tables || !context_lens || !checksum) return fail(PA_ERR_INVALID_ARG, "NULL device pointer");
  if (!aligned(block_tables, 4) || !aligned(context_lens, 4) || !aligned(checksum, 4))
    return fail(PA_ERR_INVALID_ARG, "block_tables, context_lens and checksum must be 4-byte aligned");
  static std::atomic<int> cus[64];     // compute units per device, looked up once
  int dev = 0;
  if (pa_status st = hip_check(hipGetDevice(&dev), "hipGetDevice")) return st;
  if (dev < 0 || dev >= 64) return fail(PA_ERR_UNSUPPORTED, "device index above 63");
  if (cus[dev].load() == 0) {
    int n = 0;
    if (pa_status st = hip_check(hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev),
                                 "hipDeviceGetAttribute"))
      return st;
    cus[dev].store(n > 0 ? n : 256);
  }
  StreamArgs a;
  a.kslab = pool->k_slab(layer);
  a.vslab = pool->v_slab(layer);
  a.tables = block_tables;
  a.lens = context_lens;
  a.checksum = checksum;
  a.tile_bytes = pool->tile_bytes;
  a.S = S;
  a.Hkv = pool->Hkv;
  a.P = pool->P;
  a.maxb = maxb;
  a.max_ctx = max_ctx;
  const dim3 grid((unsigned)(cus[dev].load() * kStreamWgPerCu)), block(kStreamThreads);
  switch (pool->B) {
    case 8: hipLaunchKernelGGL(stream_tiles_kernel<8>, grid, block, 0, stream, a); break;
    case 16: hipLaunchKernelGGL(stream_tiles_kernel<16>, grid, block, 0, stream, a); break;
    case 32: hipLaunchKernelGGL(stream_tiles_kernel<32>, grid, block, 0, stream, a); break;
    case 64: hipLaunchKernelGGL(stream_tiles_kernel<64>, grid, block, 0, stream, a); break;
    case 128: hipLaunchKernelGGL(stream_tiles_kernel<128>, grid, block, 0, stream, a); break;
    default: return fail(PA_ERR_UNSUPPORTED, "block size must be 8, 16, 32, 64 or 128");
  }
  return hip_check(hipGetLastError(), "stream_tiles launch");
}

}  // extern "C"
