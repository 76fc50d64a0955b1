// Paged decode attention for gfx950 (CDNA4, wave64): single-query attention
// over block tables, split into context partitions merged by the
// online-softmax rescale, optionally with the step's cache write fused in.
// (The cache write and block copies on their own are in pa_cache.hip.)
//
// Sources (page title, section):
//   "vLLM PagedAttention and continuous batching" -- "PagedAttention: fixed
//     blocks, non-contiguous physical memory" (score one block, then the
//     next, and combine; blocks need not be adjacent), "Sharing with
//     reference counts and copy-on-write" (copy the one shared block before
//     the write), "The kernel page, and what the 2023 runs measured" (one
//     query token per sequence, separate key and value caches, compile-time
//     block size), "How it works" (decode re-reads the whole cache every
//     step and is memory-bound).
//   "Serving Language Models Within a Memory Budget" -- section 6 (scaled
//     scores, softmax, weighted values; extreme logits must not overflow)
//     and eq. (4) (running maximum m' = max(m, max_j s_j), normaliser
//     l' = e^(m-m') l + sum_j e^(s_j-m'), accumulator rescaled by the same
//     factor).
//   "PagedAttention and Online Inference" -- section 1 (grouped-query
//     attention: several query heads read one key/value head).
//
// Kernel design (memory-bound: 2G flops per 2-byte key or value element):
//   * One workgroup of NW wave64s per (sequence, key/value head, context
//     partition).  The G query heads of the group are staged once in LDS and
//     then held in registers as packed 16-bit pairs.
//   * A wave consumes 16 tokens per step: four 16-byte loads per lane for K
//     and four for V.  Lane = (row r = lane/16, chunk c = lane%16): load j
//     reads token 4j+r, dims 8c..8c+7, so every load instruction covers 1 KiB
//     of contiguous cache.  The next 16 tokens are in flight while the
//     current ones are scored.
//   * Scores: v_dot2 (fp16 or bf16 pairs, fp32 accumulation) gives 4G
//     partial dot products per lane; a DPP reduce-scatter over the 16 lanes
//     of a row (row_mirror, row_half_mirror, quad xor 2, quad xor 1) leaves
//     each lane with complete scores of distinct (head, token) pairs, so
//     each exponential is evaluated by one lane only.  The probabilities are
//     exchanged through a small per-wave LDS buffer for the P.V products.
//   * Online softmax per (row, head) in the base-2 domain (scale * log2 e
//     folded into the scores).  The running maximum is raised only when a
//     block's maximum exceeds it by more than 2^8; the kept weights are then
//     at most 2^8 and the result is unchanged (numerator and denominator
//     share the offset).
//   * Partition end: rows combine with lane shuffles, waves through LDS.
//     One partition: normalise and store.  Several: store (m, l, acc) to the
//     workspace; a second, small kernel merges the partitions of every
//     (sequence, head) by the eq. (4) rescale.  The kernel boundary makes the
//     partials visible across the chip's L2 caches without a device-scope
//     fence per workgroup (such a fence writes back a whole L2).
//   * Launch order.  Given host copies of the context lengths (the block
//     manager holds them), the host splits each sequence into partitions of
//     equal length, lists the (sequence, partition) units longest first and
//     passes the list in the kernel arguments.  Workgroups start in id
//     order, so the device stays full until the shortest units at the end,
//     and no workgroup is launched past a sequence's end.  Without host
//     lengths every partition but a sequence's last has part_tokens
//     positions, the grid gives every sequence max_ctx's partition count,
//     and the surplus workgroups exit after reading the length.

#include <algorithm>
#include <cmath>
#include <mutex>
#include <string>
#include <type_traits>
#include <vector>

#include "pa_device_common.h"

using pa_detail::fail;

namespace {

constexpr float kRescaleSlack = 8.0f;  // log2 of the largest kept weight


typedef _Float16 half2_t __attribute__((ext_vector_type(2)));
typedef __bf16 bf162_t __attribute__((ext_vector_type(2)));

// ---------------------------------------------------------------------------
// small helpers
// ---------------------------------------------------------------------------
template <bool BF16>
__device__ __forceinline__ float dot8(const uint4 q, const uint4 k, float acc) {
  if constexpr (BF16) {
    acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf162_t, k.x), __builtin_bit_cast(bf162_t, q.x), acc, false);
    acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf162_t, k.y), __builtin_bit_cast(bf162_t, q.y), acc, false);
    acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf162_t, k.z), __builtin_bit_cast(bf162_t, q.z), acc, false);
    acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf162_t, k.w), __builtin_bit_cast(bf162_t, q.w), acc, false);
  } else {
    acc = __builtin_amdgcn_fdot2(__builtin_bit_cast(half2_t, k.x), __builtin_bit_cast(half2_t, q.x), acc, false);
    acc = __builtin_amdgcn_fdot2(__builtin_bit_cast(half2_t, k.y), __builtin_bit_cast(half2_t, q.y), acc, false);
    acc = __builtin_amdgcn_fdot2(__builtin_bit_cast(half2_t, k.z), __builtin_bit_cast(half2_t, q.z), acc, false);
    acc = __builtin_amdgcn_fdot2(__builtin_bit_cast(half2_t, k.w), __builtin_bit_cast(half2_t, q.w), acc, false);
  }
  return acc;
}

// 8 packed 16-bit values -> 8 floats (exact)
template <bool BF16>
__device__ __forceinline__ void widen8(const uint4 v, float (&f)[8]) {
  const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    if constexpr (BF16) {
      f[2 * i] = __builtin_bit_cast(float, w[i] << 16);
      f[2 * i + 1] = __builtin_bit_cast(float, w[i] & 0xffff0000u);
    } else {
      const half2_t h = __builtin_bit_cast(half2_t, w[i]);
      f[2 * i] = (float)h.x;
      f[2 * i + 1] = (float)h.y;
    }
  }
}

// float -> fp16 bit pattern, round to nearest even
__device__ __forceinline__ uint32_t f16_bits(float x) {
  return (uint32_t)__builtin_bit_cast(uint16_t, (_Float16)x);
}

// two floats -> two 16-bit patterns (a in the low half), round to nearest
// even; bf16 through the packed hardware conversion (one instruction)
typedef float f32x2_t __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
template <bool BF16>
__device__ __forceinline__ uint32_t pack2(float a, float b) {
  if constexpr (BF16)
    return __builtin_bit_cast(uint32_t, __builtin_convertvector((f32x2_t{a, b}), bf16x2_t));
  else
    return f16_bits(a) | (f16_bits(b) << 16);
}

template <bool BF16>
__device__ __forceinline__ uint4 narrow8(const float (&f)[8]) {
  uint4 r;
  r.x = pack2<BF16>(f[0], f[1]);
  r.y = pack2<BF16>(f[2], f[3]);
  r.z = pack2<BF16>(f[4], f[5]);
  r.w = pack2<BF16>(f[6], f[7]);
  return r;
}

// DPP lane exchange inside a row of 16 lanes.  Every pattern used here is an
// xor of the lane index: row_mirror = xor 15, row_half_mirror = xor 7,
// quad_perm [2,3,0,1] = xor 2, quad_perm [1,0,3,2] = xor 1.
constexpr int kDppMirror = 0x140;
constexpr int kDppHalfMirror = 0x141;
constexpr int kDppXor2 = 0x4E;
constexpr int kDppXor1 = 0xB1;

template <int CTRL>
__device__ __forceinline__ float dpp(float x) {
  return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), CTRL, 0xF, 0xF, false));
}

// Stage k of the reduction over the 16 lanes of a row: partner = lane ^ mask_k
// with mask = 15, 7, 2, 1; the partner differs in bit (3-k) and agrees on the
// higher bits.
template <int K> struct Stage;
template <> struct Stage<0> { static constexpr int ctrl = kDppMirror;     static constexpr int bit = 3; };
template <> struct Stage<1> { static constexpr int ctrl = kDppHalfMirror; static constexpr int bit = 2; };
template <> struct Stage<2> { static constexpr int ctrl = kDppXor2;       static constexpr int bit = 1; };
template <> struct Stage<3> { static constexpr int ctrl = kDppXor1;       static constexpr int bit = 0; };

// One reduce-scatter stage: NV values per lane -> NV/2, each now summed over
// the lane and its partner.  The lane keeps the half selected by its bit.
template <int NV, int K>
__device__ __forceinline__ void rs_stage(float* x, int c) {
  const bool hi = (c >> Stage<K>::bit) & 1;
#pragma unroll
  for (int i = 0; i < NV / 2; ++i) {
    const float lo = x[i], up = x[i + NV / 2];
    const float keep = hi ? up : lo;
    const float send = hi ? lo : up;
    x[i] = keep + dpp<Stage<K>::ctrl>(send);
  }
}

template <int K>
__device__ __forceinline__ void ar_stage(float* x) {
  x[0] = x[0] + dpp<Stage<K>::ctrl>(x[0]);
}

constexpr int ilog2(int v) { return v <= 1 ? 0 : 1 + ilog2(v / 2); }

// Per GQA group size G: the 4G partial dot products of a lane (index
// v = 4h + j: head h, load j) are summed over the 16 lanes of the row.
// Afterwards lane c holds E = max(1, 4G/16) complete scores with indices
// value_index(c, e).
template <int G>
struct Scores {
  static constexpr int NV = 4 * G;
  static constexpr int LOGNV = ilog2(NV);
  static constexpr int NRS = LOGNV < 4 ? LOGNV : 4;   // reduce-scatter stages
  static constexpr int E = NV >> NRS;                  // scores left per lane
  static constexpr int LANES_PER_HEAD = 16 / G;        // lanes of a row owning one head

  __device__ static __forceinline__ void reduce(float (&x)[NV], int c) {
    if constexpr (NRS >= 1) rs_stage<NV, 0>(x, c); else ar_stage<0>(x);
    if constexpr (NRS >= 2) rs_stage<NV / 2, 1>(x, c); else ar_stage<1>(x);
    if constexpr (NRS >= 3) rs_stage<NV / 4, 2>(x, c); else ar_stage<2>(x);
    if constexpr (NRS >= 4) rs_stage<NV / 8, 3>(x, c); else ar_stage<3>(x);
  }
  __device__ static __forceinline__ int value_index(int c, int e) {
    return ((c >> (4 - NRS)) << (LOGNV - NRS)) + e;
  }
  // max / sum over the lanes of a row that hold the same head but other tokens
  template <bool MAX>
  __device__ static __forceinline__ float across_tokens(float x) {
    auto op = [](float a, float b) { return MAX ? fmaxf(a, b) : a + b; };
    if constexpr (G == 1) {        // tokens on lane bits 3,2
      x = op(x, dpp<kDppMirror>(x));
      x = op(x, dpp<kDppHalfMirror>(x));
    } else if constexpr (G == 2) { // tokens on lane bits 2,1
      x = op(x, dpp<kDppXor2>(x));
      x = op(x, dpp<kDppHalfMirror>(x));
    } else if constexpr (G == 4) { // tokens on lane bits 1,0
      x = op(x, dpp<kDppXor1>(x));
      x = op(x, dpp<kDppXor2>(x));
    } else {                       // G == 8: tokens on lane bit 0 (and e)
      x = op(x, dpp<kDppXor1>(x));
    }
    return x;
  }
};

__device__ __forceinline__ float exp2_fast(float x) { return __builtin_amdgcn_exp2f(x); }

// (M, L, A) := the eq. (4) combination of (M, L, A) and the partial (m, l, acc)
__device__ __forceinline__ void fold_partial(float& M, float& L, float (&A)[8], const float* ml, const float* acc) {
  const float2 x = *reinterpret_cast<const float2*>(ml);
  if (x.x == -INFINITY) return;
  const float4 a0 = *reinterpret_cast<const float4*>(acc);
  const float4 a1 = *reinterpret_cast<const float4*>(acc + 4);
  const float Mn = fmaxf(M, x.x);
  const float fo = (M == -INFINITY) ? 0.0f : exp2_fast(M - Mn);
  const float fn = exp2_fast(x.x - Mn);
  L = fo * L + fn * x.y;
  A[0] = fo * A[0] + fn * a0.x; A[1] = fo * A[1] + fn * a0.y;
  A[2] = fo * A[2] + fn * a0.z; A[3] = fo * A[3] + fn * a0.w;
  A[4] = fo * A[4] + fn * a1.x; A[5] = fo * A[5] + fn * a1.y;
  A[6] = fo * A[6] + fn * a1.z; A[7] = fo * A[7] + fn * a1.w;
  M = Mn;
}

// the same with the partial already in registers
__device__ __forceinline__ void fold_partial_regs(float& M, float& L, float (&A)[8], const float2 x, const float4 a0,
                                                  const float4 a1) {
  if (x.x == -INFINITY) return;
  const float Mn = fmaxf(M, x.x);
  const float fo = (M == -INFINITY) ? 0.0f : exp2_fast(M - Mn);
  const float fn = exp2_fast(x.x - Mn);
  L = fo * L + fn * x.y;
  A[0] = fo * A[0] + fn * a0.x; A[1] = fo * A[1] + fn * a0.y;
  A[2] = fo * A[2] + fn * a0.z; A[3] = fo * A[3] + fn * a0.w;
  A[4] = fo * A[4] + fn * a1.x; A[5] = fo * A[5] + fn * a1.y;
  A[6] = fo * A[6] + fn * a1.z; A[7] = fo * A[7] + fn * a1.w;
  M = Mn;
}

// shared positions of group g as every pass of the grouped decode reads them
__device__ __forceinline__ int shared_positions(const int32_t* grp_len, int ngroups, int max_shared, int g) {
  if (g < 0 || g >= ngroups) return 0;
  const int L = min(max(grp_len[g], 0), max_shared);
  return L & ~15;
}

// ---------------------------------------------------------------------------
// decode attention
// ---------------------------------------------------------------------------
struct DecodeArgs {
  const char* kslab;        // layer's key slab   [P][Hkv][B][d]
  const char* vslab;        // layer's value slab [P][Hkv][B][d]
  uint64_t tile_bytes;      // Hkv * B * d * 2: stride of one physical block
  const uint16_t* q;        // [S][Hq][d]; several queries per sequence: [T][Hq][d]
  uint16_t* out;            // same shape as q
  const int32_t* tables;    // [S][maxb]
  const int32_t* lens;      // [S]
  float* ws_ml;             // [S][ntiles][Hkv][nparts_max][G][2]  (max, normaliser)
  float* ws_acc;            // [S][ntiles][Hkv][nparts_max][G][d]
  const int32_t* q_start;   // [S+1] first query row of each sequence (several queries), or null
  int ntiles;               // query tiles per sequence (1 for single-query decode)
  int T;                    // query rows in q and out (several queries; row indices are clamped to it)
  // shared prefixes read once (grouped decode): sequences of group g are
  // q_start[g] .. q_start[g+1]-1 in the group pass, their first grp_len[g]
  // positions (rounded down to 16, at most max_shared) mapped to the same
  // blocks; seq_group[s] names the group of sequence s (or < 0)
  const int32_t* grp_len = nullptr;
  const int32_t* seq_group = nullptr;
  int ngroups = 0, max_shared = 0;
  float* gws_ml = nullptr;  // group pass partials [ngroups][gntiles][Hkv][gparts_max][16][2]
  float* gws_acc = nullptr; // [ngroups][gntiles][Hkv][gparts_max][16][d]
  int gpart_tokens = 1, gparts_max = 1, gntiles = 0;
  int fold = 0;             // suffix pass: every suffix is one partition, so fold the group partials in here
  const uint4* knew;        // [S][Hkv][d] this step's keys (fused cache write) or null
  const uint4* vnew;        // [S][Hkv][d] this step's values, or null
  const int64_t* slots;     // [S] their slots, or null
  int64_t nslots;           // P * B
  int S, Hq, Hkv, P, maxb, max_ctx, part_tokens, nparts_max;
  float scale_log2;         // softmax scale * log2(e)
};

// the group-pass partials of sequence s (query head wh of key/value head kvh)
// folded into (M, L, A): the partitions of its group's L shared positions
template <int G>
__device__ __forceinline__ void fold_group_partials(const DecodeArgs& a, int s, int g, int L, int kvh, int wh, int wc,
                                                    float& M, float& Lsum, float (&A)[8]) {
  if (L <= 0) return;
  const int first = min(max(a.q_start[g], 0), a.S);
  const int w = s - first;
  const int r = w * G + wh;                     // row among the group's rows
  const int tile = r / 16, row = r % 16;
  if (w < 0 || tile >= a.gntiles) return;
  const int np = (L + a.gpart_tokens - 1) / a.gpart_tokens;
  const size_t base = (((size_t)g * a.gntiles + tile) * a.Hkv + kvh) * (size_t)a.gparts_max;
  for (int pp = 0; pp < np; ++pp)
    fold_partial(M, Lsum, A, a.gws_ml + ((base + pp) * 16 + row) * 2, a.gws_acc + ((base + pp) * 16 + row) * kD + 8 * wc);
}

// Longest-first order of a decode launch, built on the host from host
// copies of the context lengths: unit u = (sequence << 16) | (first
// position / 16), and workgroup id = u * Hkv + head.  Passed by value
// (kernel arguments), so a workgroup finds its partition with one scalar
// load and the grid holds exactly the partitions that have work.
constexpr int kMaxUnits = 512;
constexpr int kUnitStepBits = 16;
template <bool ON> struct UnitList { int unused; };
template <> struct UnitList<true> { int count; uint32_t unit[kMaxUnits]; };


// QT = 0: one query token per sequence (decode); the G rows are the query
// heads of one key/value head.  QT > 0: several query tokens per sequence
// at its last positions, each attending causally (up to its own position);
// a workgroup takes QT of them, and its G rows are (token t, head g) =
// (row / GQ, row % GQ) with GQ = G / QT query heads per key/value head.
// SUF: the suffix pass of the grouped decode -- sequence s attends only to
// its own positions from the end of its group's shared prefix, and always
// leaves partials for the cascade merge.
// SCHED (one query per sequence): the workgroup's (sequence, partition)
// comes from the unit list instead of the fixed grid order.
template <bool BF16, int G, int BS, int NW, int QT, bool SUF = false, bool SCHED = false>
__global__ __launch_bounds__(NW * 64) void decode_attention_kernel(const DecodeArgs a,
                                                                                const UnitList<SCHED> ul) {
  static_assert(!SCHED || (QT == 0 && !SUF), "unit lists order single-query decode launches");
  using SC = Scores<G>;
  constexpr int GQ = QT > 0 ? G / QT : G;
  static_assert(QT == 0 || GQ * QT == G, "rows = query tokens x query heads");
  static_assert(NW * 64 >= G * 16, "query staging and the combine use G * 16 threads");
  constexpr int E = SC::E;
  // A 16-token step lies inside one block when 16 | BS; with 8-token blocks
  // it covers two (loads 0-1 read the first, loads 2-3 the second).
  static_assert(BS % 16 == 0 || BS == 8, "block size must be 8 or a multiple of 16");
  constexpr int BPG = BS >= 16 ? 1 : 16 / BS;   // blocks per 16-token step

  // 1-D grid; the dispatcher deals consecutive workgroups round-robin to the
  // 8 XCDs, so the order decides each XCD's share of the work.  Head fastest:
  // XCD = head mod 8 when 8 | Hkv, an equal share of every sequence for
  // every XCD.
  int kvh, s, p, tile = 0;
  {
    const uint32_t id = blockIdx.x;
    if constexpr (SCHED) {
      kvh = id % a.Hkv;
      const uint32_t w = ul.unit[min(id / a.Hkv, (uint32_t)kMaxUnits - 1)];
      s = (int)(w >> kUnitStepBits);
      p = (int)(w & ((1u << kUnitStepBits) - 1));   // first 16-token step; the partition index follows from n
      if (s >= a.S) return;
    } else if (QT > 0) {                      // head, then query tile, sequence, partition
      kvh = id % a.Hkv;
      uint32_t t = id / a.Hkv;
      tile = t % a.ntiles;
      t /= a.ntiles;
      s = t % a.S;
      p = t / a.S;
    } else {
      kvh = id % a.Hkv;
      const uint32_t t = id / a.Hkv;
      s = t % a.S;
      p = t / a.S;
    }
  }
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int r = lane >> 4;   // row: token offset inside a 4-token load
  const int c = lane & 15;   // 16-byte chunk: dims 8c..8c+7

  // Requests that do not depend on the context length go out first: the
  // query group and this lane's block-table entry (index clamped into the
  // table row; an entry past the sequence is never used).
  int start = 0;   // first position of this pass (the suffix pass starts after the shared prefix)
  int grp = -1;
  if constexpr (SUF) {
    int n0 = a.lens[s];
    n0 = n0 < 0 ? 0 : (n0 > a.max_ctx ? a.max_ctx : n0);
    grp = __builtin_amdgcn_readfirstlane(a.seq_group[s]);
    start = __builtin_amdgcn_readfirstlane(min(shared_positions(a.grp_len, a.ngroups, a.max_shared, grp), n0));
  }
  const int t_begin = SCHED ? p * 16 : start + p * a.part_tokens;
  const int g_first = t_begin / 16 + wave;
  const int32_t* table = a.tables + (size_t)s * a.maxb;
  uint4 qv = make_uint4(0, 0, 0, 0);
  int q0 = 0, nq = 1;   // several queries: first row of the sequence, its query count
  if constexpr (QT == 0) {
    const uint4* qg = reinterpret_cast<const uint4*>(a.q + ((size_t)s * a.Hq + (size_t)kvh * G) * kD);
    if (threadIdx.x < G * 16) qv = qg[threadIdx.x];
  } else {
    // row offsets are clamped into [0, T] so that q and out stay in bounds
    q0 = min(max(a.q_start[s], 0), a.T);
    nq = min(max(a.q_start[s + 1], q0), a.T) - q0;
    const int row = threadIdx.x >> 4;
    const int tq = tile * QT + row / GQ;
    if (threadIdx.x < G * 16 && tq < nq)
      qv = reinterpret_cast<const uint4*>(
          a.q + ((size_t)(q0 + tq) * a.Hq + (size_t)kvh * GQ + row % GQ) * kD)[threadIdx.x & 15];
  }
  int entry[BPG];
#pragma unroll
  for (int b = 0; b < BPG; ++b) {
    const int idx = ((g_first + lane * NW) * 16) / BS + b;
    entry[b] = table[idx < a.maxb ? idx : a.maxb - 1];
  }

  int n = a.lens[s];
  n = n < 0 ? 0 : (n > a.max_ctx ? a.max_ctx : n);
  // Several queries: query t of the sequence sits at position n - nq + t and
  // sees positions 0 .. n - nq + t.  This tile's rows see at least lim_min
  // and at most n (now the tile's context) positions.
  int lim_min = n;
  if constexpr (QT > 0) {
    nq = __builtin_amdgcn_readfirstlane(nq);
    if (tile * QT >= nq || nq > n) return;
    lim_min = n - nq + tile * QT + 1;
    n = n - nq + min(tile * QT + QT, nq);
  }
  n = __builtin_amdgcn_readfirstlane(n);
  const int nparts = SUF ? (n - start + a.part_tokens - 1) / a.part_tokens
                         : (n > 0 ? (n + a.part_tokens - 1) / a.part_tokens : 1);
  // Partition length: part_tokens, or from a unit list, the sequence's
  // nparts partitions share its length (rounded up to 16 tokens).
  int plen = a.part_tokens;
  if constexpr (SCHED) {
    if (nparts > 1) plen = ((n + nparts - 1) / nparts + 15) & ~15;
    if (t_begin % plen) return;   // not a partition start of this length
    p = t_begin / plen;
  }
  // Suffix pass that stores the output itself (fold): a sequence with no
  // positions of its own (an empty one) still needs its row written, from
  // the group partials alone -- partition 0 runs with an empty range.
  const bool empty_fold = SUF && a.fold && nparts == 0 && p == 0;
  if (p >= nparts && !empty_fold) return;
  const int t_end = empty_fold ? t_begin : min(n, t_begin + plen);

  // Suffix pass that stores the output itself: the first two group-pass
  // partials of this thread's row are requested now, so that they arrive
  // while the suffix's own positions load (folded in the same order as the
  // rest, after the suffix)
  constexpr int kPre = 2;
  float2 gp_ml[kPre];
  float4 gp_a0[kPre], gp_a1[kPre];
  int gp_np = 0, gp_row = 0;
  size_t gp_base = 0;
  if constexpr (SUF) {
    if (a.fold && threadIdx.x < G * 16 && start > 0) {
      const int first = min(max(a.q_start[grp], 0), a.S);
      const int w = s - first;
      const int r = w * G + (int)(threadIdx.x >> 4);   // row among the group's rows
      if (w >= 0 && r / 16 < a.gntiles) {
        gp_np = (start + a.gpart_tokens - 1) / a.gpart_tokens;
        gp_row = r % 16;
        gp_base = (((size_t)grp * a.gntiles + r / 16) * a.Hkv + kvh) * (size_t)a.gparts_max;
        const int wc0 = threadIdx.x & 15;
#pragma unroll
        for (int pp = 0; pp < kPre; ++pp) {
          if (pp < gp_np) {
            gp_ml[pp] = *reinterpret_cast<const float2*>(a.gws_ml + ((gp_base + pp) * 16 + gp_row) * 2);
            const float4* ga = reinterpret_cast<const float4*>(a.gws_acc + ((gp_base + pp) * 16 + gp_row) * kD + 8 * wc0);
            gp_a0[pp] = ga[0];
            gp_a1[pp] = ga[1];
          }
        }
      }
    }
  }

  __shared__ uint4 s_q[G * 16];
  __shared__ __attribute__((aligned(16))) float s_p[NW][2][4][4 * G];
  __shared__ float s_f[NW][4][G];
  __shared__ __attribute__((aligned(16))) float s_acc[NW][G][kD];
  __shared__ float s_m[NW][G];
  __shared__ float s_l[NW][G];

  const uint64_t head_off = (uint64_t)kvh * BS * kRowBytes;
  const uint32_t lane_off = (uint32_t)(r * kRowBytes + c * 16);

  // running state of this lane's (row, head)
  float m = -INFINITY;
  float ell = 0.0f;
  float acc[G][8];
#pragma unroll
  for (int h = 0; h < G; ++h)
#pragma unroll
    for (int i = 0; i < 8; ++i) acc[h][i] = 0.0f;

  int hown;  // head owned by this lane after the reduction
  {
    const int v0 = SC::value_index(c, 0);
    hown = v0 >> 2;
  }

  // groups of 16 tokens in this partition, dealt round-robin to the waves:
  // the k-th group of this wave is g_first + k * NW, and lane k holds that
  // group's physical block (one lane read per group later).
  // groups [.., g_full) are full and seen whole by every row
  int g_full = (QT > 0 ? min(t_end, lim_min) : t_end) / 16;
  const int g_last = (t_end + 15) / 16;        // a tail group exists if g_full < g_last
  uint4 qr[G];
  int my_phys[BPG];
#pragma unroll
  for (int b = 0; b < BPG; ++b) {
    my_phys[b] = 0;
    if (g_first + lane * NW < g_last) my_phys[b] = entry[b] < 0 ? 0 : (entry[b] >= a.P ? a.P - 1 : entry[b]);
  }

  // Fused cache write of this step's token: the workgroup of the sequence's
  // last partition stores k_new / v_new of its head into the token's slot,
  // and when that slot is the one position n-1 maps to, uses them directly
  // from registers for that position (the cache load of the slot is
  // replaced), so no other workgroup depends on the store.  (Reading them
  // again at that step instead puts a load under a branch inside the loop,
  // which coarsens every wait on the prefetched loads.)
  int g_new = -1, j_new = 0, r_new = 0;
  uint4 k_reg = make_uint4(0, 0, 0, 0), v_reg = make_uint4(0, 0, 0, 0);
  if (QT == 0 && a.slots != nullptr && p == nparts - 1) {
    const int64_t slot = a.slots[s];
    if (slot >= 0 && slot < a.nslots) {
      const size_t src = ((size_t)s * a.Hkv + kvh) * 16 + c;
      k_reg = a.knew[src];
      v_reg = a.vnew[src];
      const int64_t blk = slot / BS;
      const int off = (int)(slot % BS);
      if (wave == 0 && r == 0) {
        const uint64_t dst = (uint64_t)blk * a.tile_bytes + head_off + (uint64_t)off * kRowBytes + (uint64_t)c * 16;
        *reinterpret_cast<uint4*>(const_cast<char*>(a.kslab) + dst) = k_reg;
        *reinterpret_cast<uint4*>(const_cast<char*>(a.vslab) + dst) = v_reg;
      }
      if (n > 0) {
        const int pos = n - 1;
        int e = table[pos / BS];
        e = e < 0 ? 0 : (e >= a.P ? a.P - 1 : e);
        if ((int64_t)e * BS + pos % BS == slot) {
          g_new = pos / 16;
          j_new = (pos % 16) / 4;
          r_new = pos % 4;
        }
      }
    }
  }

  // The step holding position n-1 is the partition's last one; it always
  // takes the peeled tail path, so the substitution above costs nothing in
  // the main loop.
  if (g_new >= 0) g_full = g_new;

  auto load_group = [&](int k, uint4 (&K)[4], uint4 (&V)[4], bool tail) {
    const int g = g_first + k * NW;
    const int tok0 = g * 16;
    uint64_t off[BPG];
#pragma unroll
    for (int b = 0; b < BPG; ++b) {
      const int phys = __builtin_amdgcn_readlane(my_phys[b], k);
      off[b] = (uint64_t)phys * a.tile_bytes + head_off + (uint64_t)(tok0 % BS) * kRowBytes;
    }
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      // token 4j + r of the step: block (4j) / BS of the step, row (4j) % BS
      // inside it when BS < 16, else row 4j after the step's first token
      constexpr int kStepRows = BS >= 16 ? 16 : BS;
      const char* kb = a.kslab + off[(4 * j) / kStepRows] + (uint64_t)((4 * j) % kStepRows) * kRowBytes;
      const char* vb = a.vslab + off[(4 * j) / kStepRows] + (uint64_t)((4 * j) % kStepRows) * kRowBytes;
      if (!tail || tok0 + 4 * j < n) {
        // read once per step: the streaming (non-temporal) hint keeps them
        // from displacing reusable lines
        K[j] = nt_load16(kb + lane_off);
        V[j] = nt_load16(vb + lane_off);
      } else {
        K[j] = make_uint4(0, 0, 0, 0);
        V[j] = make_uint4(0, 0, 0, 0);
      }
    }
  };

  int buf = 0;
  auto process_group = [&](int g, const uint4 (&Kin)[4], const uint4 (&Vin)[4], bool tail) {
    const int tok0 = g * 16;
    uint4 K[4], V[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      K[j] = Kin[j];
      V[j] = Vin[j];
    }
    if (tail && g == g_new) {
#pragma unroll
      for (int j = 0; j < 4; ++j)
        if (j == j_new && r == r_new) {
          K[j] = k_reg;
          V[j] = v_reg;
        }
    }
    // partial dot products: x[4h + j] = q_h . k(token 4j + r) over this lane's 8 dims
    float x[4 * G];
#pragma unroll
    for (int h = 0; h < G; ++h)
#pragma unroll
      for (int j = 0; j < 4; ++j) x[4 * h + j] = dot8<BF16>(qr[h], K[j], 0.0f);
    SC::reduce(x, c);

    float sc[E];
    float mx = -INFINITY;
#pragma unroll
    for (int e = 0; e < E; ++e) {
      sc[e] = x[e] * a.scale_log2;
      if (tail) {
        const int j = SC::value_index(c, e) & 3;
        // row (t, g) sees positions below lim_min + t (QT > 0), all rows below n (QT = 0)
        const int lim = QT > 0 ? lim_min + (SC::value_index(c, e) >> 2) / GQ : n;
        if (tok0 + 4 * j + r >= lim) sc[e] = -INFINITY;
      }
      mx = fmaxf(mx, sc[e]);
    }
    mx = SC::template across_tokens<true>(mx);

    // raise the running maximum only when the block would exceed it by > 2^8
    if (__builtin_amdgcn_ballot_w64(mx > m + kRescaleSlack) != 0) {
      const float m_new = fmaxf(m, mx);
      const float f = (m_new == m) ? 1.0f : exp2_fast(m - m_new);
      m = m_new;
      ell *= f;
      s_f[wave][r][hown] = f;
      __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
      __builtin_amdgcn_wave_barrier();
      __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
#pragma unroll
      for (int h = 0; h < G; ++h) {
        const float fh = s_f[wave][r][h];
#pragma unroll
        for (int i = 0; i < 8; ++i) acc[h][i] *= fh;
      }
    }

#pragma unroll
    for (int e = 0; e < E; ++e) {
      const float pe = (tail && sc[e] == -INFINITY) ? 0.0f : exp2_fast(sc[e] - m);
      ell += pe;
      s_p[wave][buf][r][SC::value_index(c, e)] = pe;
    }
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    float pv[4 * G];
#pragma unroll
    for (int i = 0; i < G; ++i) {
      const float4 t = *reinterpret_cast<const float4*>(&s_p[wave][buf][r][4 * i]);
      pv[4 * i] = t.x; pv[4 * i + 1] = t.y; pv[4 * i + 2] = t.z; pv[4 * i + 3] = t.w;
    }
    buf ^= 1;

#pragma unroll
    for (int j = 0; j < 4; ++j) {
      float vf[8];
      widen8<BF16>(V[j], vf);
      if (tail && tok0 + 4 * j + r >= n) {
#pragma unroll
        for (int i = 0; i < 8; ++i) vf[i] = 0.0f;
      }
#pragma unroll
      for (int h = 0; h < G; ++h) {
        const float w = pv[4 * h + j];
#pragma unroll
        for (int i = 0; i < 8; ++i) acc[h][i] = fmaf(w, vf[i], acc[h][i]);
      }
    }
  };

  {
    // Two register buffers; the next group's loads are issued before the
    // current group is scored.  The prefetch index is clamped instead of
    // skipped, so every path through the loop has the same loads in flight
    // and the wait before scoring covers exactly the current group.
    const int ng = g_full > g_first ? (g_full - g_first + NW - 1) / NW : 0;
    uint4 K0[4], V0[4], K1[4], V1[4];
    // unconditional, so that every path has the same loads in flight (a wave
    // without a full group reads an in-bounds stand-in block and ignores it);
    // in the suffix pass, whose suffixes are mostly shorter than one group,
    // only when there is a full group, so the tail is not read twice
    if (!SUF || ng > 0) load_group(0, K0, V0, false);
    if (threadIdx.x < G * 16) s_q[threadIdx.x] = qv;
    __syncthreads();
#pragma unroll
    for (int h = 0; h < G; ++h) qr[h] = s_q[h * 16 + c];
    if (ng > 0) {
      // invariant at the top of every iteration: buffer 0 holds group k's
      // loads (issued, maybe not complete) and nothing else is in flight
      int k = 0;
      for (; k + 2 < ng; k += 2) {
        load_group(k + 1, K1, V1, false);
        process_group(g_first + k * NW, K0, V0, false);
        load_group(k + 2, K0, V0, false);
        process_group(g_first + (k + 1) * NW, K1, V1, false);
      }
      // the last one or two groups: no loads beyond this wave's groups
      if (k + 2 == ng) {
        load_group(k + 1, K1, V1, false);
        process_group(g_first + k * NW, K0, V0, false);
        process_group(g_first + (k + 1) * NW, K1, V1, false);
      } else {
        process_group(g_first + k * NW, K0, V0, false);
      }
    }
    if constexpr (QT == 0) {
      if (g_full < g_last && g_full >= g_first && (g_full - g_first) % NW == 0) {
        const int kt = (g_full - g_first) / NW;
        load_group(kt, K0, V0, true);
        process_group(g_full, K0, V0, true);
      }
    } else {
      // the steps where some rows stop (the causal edge), with per-row masks
      int g = g_full > g_first ? g_first + (g_full - g_first + NW - 1) / NW * NW : g_first;
      for (; g < g_last; g += NW) {
        load_group((g - g_first) / NW, K0, V0, true);
        process_group(g, K0, V0, true);
      }
    }
  }

  // ---- combine: tokens of a row, then rows, then waves ---------------------
  ell = SC::template across_tokens<false>(ell);
  float mh[G], lh[G];
#pragma unroll
  for (int h = 0; h < G; ++h) {
    const int owner = (lane & 0x30) | (h * SC::LANES_PER_HEAD);
    mh[h] = __shfl(m, owner);
    lh[h] = __shfl(ell, owner);
  }
#pragma unroll
  for (int sh = 16; sh <= 32; sh <<= 1) {
#pragma unroll
    for (int h = 0; h < G; ++h) {
      const float mo = __shfl_xor(mh[h], sh);
      const float lo = __shfl_xor(lh[h], sh);
      const float M = fmaxf(mh[h], mo);
      const float wa = (mh[h] == -INFINITY) ? 0.0f : exp2_fast(mh[h] - M);
      const float wb = (mo == -INFINITY) ? 0.0f : exp2_fast(mo - M);
      lh[h] = wa * lh[h] + wb * lo;
#pragma unroll
      for (int i = 0; i < 8; ++i) acc[h][i] = wa * acc[h][i] + wb * __shfl_xor(acc[h][i], sh);
      mh[h] = M;
    }
  }
  if (lane < 16) {
#pragma unroll
    for (int h = 0; h < G; ++h) {
      float4* dst = reinterpret_cast<float4*>(&s_acc[wave][h][8 * c]);
      dst[0] = make_float4(acc[h][0], acc[h][1], acc[h][2], acc[h][3]);
      dst[1] = make_float4(acc[h][4], acc[h][5], acc[h][6], acc[h][7]);
    }
    if (lane == 0) {
#pragma unroll
      for (int h = 0; h < G; ++h) {
        s_m[wave][h] = mh[h];
        s_l[wave][h] = lh[h];
      }
    }
  }
  __syncthreads();

  const int t = threadIdx.x;
  const bool worker = t < G * 16;     // one thread per (head, 8-dim chunk)
  const int wh = t >> 4;
  const int wc = t & 15;
  float A[8];
  float M = -INFINITY, Lsum = 0.0f;
  if (worker) {
#pragma unroll
    for (int w = 0; w < NW; ++w) M = fmaxf(M, s_m[w][wh]);
#pragma unroll
    for (int i = 0; i < 8; ++i) A[i] = 0.0f;
#pragma unroll
    for (int w = 0; w < NW; ++w) {
      const float mw = s_m[w][wh];
      const float wt = (mw == -INFINITY) ? 0.0f : exp2_fast(mw - M);
      Lsum += wt * s_l[w][wh];
      const float4 a0 = *reinterpret_cast<const float4*>(&s_acc[w][wh][8 * wc]);
      const float4 a1 = *reinterpret_cast<const float4*>(&s_acc[w][wh][8 * wc + 4]);
      A[0] += wt * a0.x; A[1] += wt * a0.y; A[2] += wt * a0.z; A[3] += wt * a0.w;
      A[4] += wt * a1.x; A[5] += wt * a1.y; A[6] += wt * a1.z; A[7] += wt * a1.w;
    }
  }

  size_t orow = (size_t)s * a.Hq + (size_t)kvh * G + wh;
  bool live = worker;
  if constexpr (QT > 0) {
    const int tq = tile * QT + wh / GQ;
    orow = (size_t)(q0 + tq) * a.Hq + (size_t)kvh * GQ + wh % GQ;
    live = worker && tq < nq;
  }
  uint4* out_row = reinterpret_cast<uint4*>(a.out + orow * kD) + wc;
  if constexpr (SUF) {
    if (a.fold) {
      // one suffix partition: add the group's shared-prefix partials (the
      // group pass finished one launch earlier) and store the result
      if (worker) {
#pragma unroll
        for (int pp = 0; pp < kPre; ++pp)
          if (pp < gp_np) fold_partial_regs(M, Lsum, A, gp_ml[pp], gp_a0[pp], gp_a1[pp]);
        for (int pp = kPre; pp < gp_np; ++pp)
          fold_partial(M, Lsum, A, a.gws_ml + ((gp_base + pp) * 16 + gp_row) * 2,
                       a.gws_acc + ((gp_base + pp) * 16 + gp_row) * kD + 8 * wc);
        const float inv = Lsum > 0.0f ? 1.0f / Lsum : 0.0f;
        float o[8];
#pragma unroll
        for (int i = 0; i < 8; ++i) o[i] = A[i] * inv;
        *out_row = narrow8<BF16>(o);
      }
      return;
    }
  }
  if (!SUF && nparts == 1) {
    if (live) {
      const float inv = Lsum > 0.0f ? 1.0f / Lsum : 0.0f;
      float o[8];
#pragma unroll
      for (int i = 0; i < 8; ++i) o[i] = A[i] * inv;
      *out_row = narrow8<BF16>(o);
    }
    return;
  }

  // ---- several partitions: store this partition's (m, l, acc) --------------
  if (worker) {
    const size_t pbase = (((size_t)s * a.ntiles + tile) * a.Hkv + kvh) * (size_t)a.nparts_max;
    float4* dst = reinterpret_cast<float4*>(a.ws_acc + ((pbase + p) * G + wh) * kD + 8 * wc);
    dst[0] = make_float4(A[0], A[1], A[2], A[3]);
    dst[1] = make_float4(A[4], A[5], A[6], A[7]);
    if (wc == 0) *reinterpret_cast<float2*>(a.ws_ml + ((pbase + p) * G + wh) * 2) = make_float2(M, Lsum);
  }
}

// ---------------------------------------------------------------------------
// merge of the context partitions (eq. (4) rescale): one wave per
// (sequence, key/value head); thread = (head, 8-dim chunk)
// ---------------------------------------------------------------------------
template <bool BF16, int G, int QT>
__global__ __launch_bounds__(G * 16) void decode_merge_kernel(const DecodeArgs a) {
  constexpr int GQ = QT > 0 ? G / QT : G;
  const int kvh = blockIdx.x;
  const int s = blockIdx.y;
  const int tile = QT > 0 ? (int)blockIdx.z : 0;
  const int wh = threadIdx.x >> 4;
  const int wc = threadIdx.x & 15;
  const size_t pbase = (((size_t)s * a.ntiles + tile) * a.Hkv + kvh) * (size_t)a.nparts_max;
  // Partitions are read CHUNK at a time with all loads of a chunk in flight;
  // the first chunk is requested together with the context length (its
  // indices are clamped into the workspace; unused entries are ignored).
  constexpr int CHUNK = 4;
  float2 ml[CHUNK];
  float4 x0[CHUNK], x1[CHUNK];
  auto fetch = [&](int p0) {
#pragma unroll
    for (int k = 0; k < CHUNK; ++k) {
      const int pp = p0 + k < a.nparts_max ? p0 + k : a.nparts_max - 1;
      ml[k] = *reinterpret_cast<const float2*>(a.ws_ml + ((pbase + pp) * G + wh) * 2);
      const float4* src = reinterpret_cast<const float4*>(a.ws_acc + ((pbase + pp) * G + wh) * kD + 8 * wc);
      x0[k] = src[0];
      x1[k] = src[1];
    }
  };
  fetch(0);
  int n = a.lens[s];
  n = n < 0 ? 0 : (n > a.max_ctx ? a.max_ctx : n);
  size_t orow = (size_t)s * a.Hq + (size_t)kvh * G + wh;
  if constexpr (QT > 0) {
    // the same tile context and rows as the partition kernel
    const int q0 = min(max(a.q_start[s], 0), a.T);
    const int nq = min(max(a.q_start[s + 1], q0), a.T) - q0;
    if (tile * QT >= nq || nq > n) return;
    n = n - nq + min(tile * QT + QT, nq);
    const int tq = tile * QT + wh / GQ;
    if (tq >= nq) return;
    orow = (size_t)(q0 + tq) * a.Hq + (size_t)kvh * GQ + wh % GQ;
  }
  const int nparts = n > 0 ? (n + a.part_tokens - 1) / a.part_tokens : 1;
  if (nparts <= 1) return;  // written directly by the partition kernel
  float Mg = -INFINITY, Lg = 0.0f, Ag[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) Ag[i] = 0.0f;
  for (int p0 = 0; p0 < nparts; p0 += CHUNK) {
    if (p0 > 0) fetch(p0);
    float mc = Mg;
#pragma unroll
    for (int k = 0; k < CHUNK; ++k)
      if (p0 + k < nparts) mc = fmaxf(mc, ml[k].x);
    const float f = (Mg == -INFINITY) ? 0.0f : exp2_fast(Mg - mc);
    Lg *= f;
#pragma unroll
    for (int i = 0; i < 8; ++i) Ag[i] *= f;
#pragma unroll
    for (int k = 0; k < CHUNK; ++k) {
      if (p0 + k >= nparts) break;
      const float wt = (ml[k].x == -INFINITY) ? 0.0f : exp2_fast(ml[k].x - mc);
      Lg += wt * ml[k].y;
      Ag[0] += wt * x0[k].x; Ag[1] += wt * x0[k].y; Ag[2] += wt * x0[k].z; Ag[3] += wt * x0[k].w;
      Ag[4] += wt * x1[k].x; Ag[5] += wt * x1[k].y; Ag[6] += wt * x1[k].z; Ag[7] += wt * x1[k].w;
    }
    Mg = mc;
  }
  const float inv = Lg > 0.0f ? 1.0f / Lg : 0.0f;
  float o[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) o[i] = Ag[i] * inv;
  uint4* out_row = reinterpret_cast<uint4*>(a.out + orow * kD) + wc;
  *out_row = narrow8<BF16>(o);
}

// ---------------------------------------------------------------------------
// cascade merge of the grouped decode: for sequence s and each query head of
// key/value head kvh, the partials of its group's shared prefix (rows
// member * G + head of the group pass) and of its own suffix, combined by the
// eq. (4) rescale; thread = (head, 8-dim chunk)
// ---------------------------------------------------------------------------
template <bool BF16, int G>
__global__ __launch_bounds__(G * 16) void cascade_merge_kernel(const DecodeArgs a) {
  const int kvh = blockIdx.x;
  const int s = blockIdx.y;
  const int wh = threadIdx.x >> 4;
  const int wc = threadIdx.x & 15;
  int n = a.lens[s];
  n = n < 0 ? 0 : (n > a.max_ctx ? a.max_ctx : n);
  const int g = a.seq_group[s];
  const int L = min(shared_positions(a.grp_len, a.ngroups, a.max_shared, g), n);
  float Mg = -INFINITY, Lg = 0.0f, Ag[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) Ag[i] = 0.0f;
  fold_group_partials<G>(a, s, g, L, kvh, wh, wc, Mg, Lg, Ag);
  if (n > L) {
    const int np = (n - L + a.part_tokens - 1) / a.part_tokens;
    const size_t base = ((size_t)s * a.Hkv + kvh) * (size_t)a.nparts_max;
    for (int pp = 0; pp < np; ++pp)
      fold_partial(Mg, Lg, Ag, a.ws_ml + ((base + pp) * G + wh) * 2, a.ws_acc + ((base + pp) * G + wh) * kD + 8 * wc);
  }
  const float inv = Lg > 0.0f ? 1.0f / Lg : 0.0f;
  float o[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) o[i] = Ag[i] * inv;
  *(reinterpret_cast<uint4*>(a.out + ((size_t)s * a.Hq + (size_t)kvh * G + wh) * kD) + wc) = narrow8<BF16>(o);
}

// ---------------------------------------------------------------------------
// several queries per sequence on the matrix cores
//
// A workgroup's 16 rows are QT = 16 / GQ query tokens x GQ query heads of one
// key/value head.  Lane = (row = lane % 16, quarter kq = lane / 16).  Per
// 16-token step of a wave the key and value tiles are loaded as whole
// 256-byte rows (lane: tokens 4j + kq, dims 8 row .. +7; each instruction
// reads 1 KiB contiguous) into per-wave LDS tiles, then
//   S^T[token][row] = K[token][:] . Q[row][:]   4 x mfma 16x16x32: A = the
//       key tile read back row-major (lane: token `row`, dims 32ks + 8kq ..
//       +7; 272-byte rows), B = Q^T held in registers (lane: query row
//       `row`, the same dims); the result gives lane (row, kq) the scores of
//       tokens 4kq .. 4kq+3 for its row;
//   O^T[dim][row] += V^T[dim][token] . P^T[token][row]   8 x mfma 16x16x16:
//       B = the lane's own four probabilities (the layout S^T came out in),
//       A = V^T, from a per-wave LDS copy of the value tile (token order,
//       288-byte rows) by one transposing read (ds_read_b64_tr_b16) per 16
//       dims; lane (row, kq) accumulates dims 16nb + 4kq .. +3 of its row, so
//       the softmax state of a row and its rescale stay inside the lane.
// Probabilities enter the P.V products in the storage type (the products
// accumulate in fp32); for bf16 as a rounded part plus the rounded remainder.
// ---------------------------------------------------------------------------
typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8_t __attribute__((ext_vector_type(8)));
typedef short i16x4_t __attribute__((ext_vector_type(4)));
typedef _Float16 f16x4_t __attribute__((ext_vector_type(4)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));

template <bool BF16>
__device__ __forceinline__ f32x4_t mfma_k32(const uint4 a, const uint4 b, f32x4_t c) {
  if constexpr (BF16)
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, a), __builtin_bit_cast(bf16x8_t, b), c,
                                                   0, 0, 0);
  else
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8_t, a), __builtin_bit_cast(f16x8_t, b), c,
                                                  0, 0, 0);
}

template <bool BF16>
__device__ __forceinline__ f32x4_t mfma_k16(const uint2 a, const uint2 b, f32x4_t c) {
  if constexpr (BF16)
    return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(__builtin_bit_cast(i16x4_t, a), __builtin_bit_cast(i16x4_t, b), c,
                                                     0, 0, 0);
  else
    return __builtin_amdgcn_mfma_f32_16x16x16f16(__builtin_bit_cast(f16x4_t, a), __builtin_bit_cast(f16x4_t, b), c, 0,
                                                 0, 0);
}

constexpr int kVRow = 288;   // bytes per token row of the LDS value tile (256 + 32 pad)

// operand of the transposing LDS read (ds_read_b64_tr_b16)
typedef short v4i16_t __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) v4i16_t lds_v4i16_t;

constexpr int kKRow = 272;   // bytes per token row of an LDS key tile (256 + 16 pad)


// GRP: the group pass of the grouped decode -- "sequence" s is group s, its
// query tokens are the group's sequences (one query each), every row sees the
// group's shared positions, read through the first member's table, and the
// result is always left as partials for the cascade merge.
template <bool BF16, int GQ, int BS, int NW, bool GRP = false, bool SCHED = false>
__global__ __launch_bounds__(NW * 64) void mq_mfma_kernel(const DecodeArgs a, const UnitList<SCHED> ul) {
  // unit lists order the group pass, and several queries per sequence when
  // a sequence's rows fit one tile (its tile context is then its length)
  constexpr int R = 16;             // rows per workgroup
  constexpr int QT = R / GQ;        // query tokens per workgroup
  static_assert(BS % 16 == 0 || BS == 8, "block size must be 8 or a multiple of 16");
  constexpr int BPG = BS >= 16 ? 1 : 16 / BS;

  int kvh, s, p, tile;
  {
    const uint32_t id = blockIdx.x;   // head, then query tile, sequence, partition
    kvh = id % a.Hkv;
    uint32_t t = id / a.Hkv;
    tile = t % a.ntiles;
    t /= a.ntiles;
    if constexpr (SCHED) {            // unit = (group, first 16-token step), longest first
      const uint32_t w = ul.unit[min(t, (uint32_t)kMaxUnits - 1)];
      s = (int)(w >> kUnitStepBits);
      p = (int)(w & ((1u << kUnitStepBits) - 1));
      if (s >= a.S) return;
    } else {
      s = t % a.S;
      p = t / a.S;
    }
  }
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int row = lane & 15;
  const int kq = lane >> 4;

  const int t_begin = SCHED ? p * 16 : p * a.part_tokens;
  const int g_first = t_begin / 16 + wave;
  const int q0 = min(max(a.q_start[s], 0), a.T);
  int nq = min(max(a.q_start[s + 1], q0), a.T) - q0;
  // a group reads its shared positions through its first member's table
  const int32_t* table = a.tables + (size_t)(GRP ? min(q0, a.T - 1) : s) * a.maxb;
  int entry[BPG];
#pragma unroll
  for (int b = 0; b < BPG; ++b) {
    const int idx = ((g_first + lane * NW) * 16) / BS + b;
    entry[b] = table[idx < a.maxb ? idx : a.maxb - 1];
  }
  const int tq = tile * QT + row / GQ;    // this lane's query token
  uint4 qb[4];
  {
    const bool live = tq < nq;
    const uint4* qrow = reinterpret_cast<const uint4*>(
        a.q + ((size_t)(live ? q0 + tq : 0) * a.Hq + (size_t)kvh * GQ + row % GQ) * kD);
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) qb[ks] = live ? qrow[4 * ks + kq] : make_uint4(0, 0, 0, 0);
  }

  int n, lim_min;
  nq = __builtin_amdgcn_readfirstlane(nq);
  if constexpr (GRP) {
    n = __builtin_amdgcn_readfirstlane(shared_positions(a.grp_len, a.ngroups, a.max_shared, s));
    if (tile * QT >= nq || n == 0) return;
    lim_min = n;                                        // no causal edge: every row sees all n
  } else {
    n = a.lens[s];
    n = n < 0 ? 0 : (n > a.max_ctx ? a.max_ctx : n);
    if (tile * QT >= nq || nq > n) return;
    lim_min = n - nq + tile * QT + 1;
    n = __builtin_amdgcn_readfirstlane(n - nq + min(tile * QT + QT, nq));
  }
  const int nparts = (n + a.part_tokens - 1) / a.part_tokens;
  int plen = a.part_tokens;
  if constexpr (SCHED) {              // the group's nparts partitions share its length
    if (nparts > 1) plen = ((n + nparts - 1) / nparts + 15) & ~15;
    if (t_begin % plen) return;
    p = t_begin / plen;
  }
  if (p >= nparts) return;
  const int t_end = min(n, t_begin + plen);
  const int lim = tq < nq ? (GRP ? n : lim_min + row / GQ) : 0;   // positions this row sees
  const int g_full = min(t_end, lim_min) / 16;        // steps every row sees whole
  const int g_last = (t_end + 15) / 16;
  int my_phys[BPG];
#pragma unroll
  for (int b = 0; b < BPG; ++b) {
    my_phys[b] = 0;
    if (g_first + lane * NW < g_last) my_phys[b] = entry[b] < 0 ? 0 : (entry[b] >= a.P ? a.P - 1 : entry[b]);
  }

  // value tiles during the loop; the cross-wave combine reuses the space
  __shared__ __attribute__((aligned(16))) char s_v[NW][2][16 * kVRow];
  __shared__ __attribute__((aligned(16))) char s_k[NW][2][16 * kKRow];
  static_assert(sizeof(s_v) >= sizeof(float) * NW * R * kD, "combine buffer must fit");
  float (*s_acc)[R][kD] = reinterpret_cast<float (*)[R][kD]>(&s_v[0][0][0]);
  __shared__ float s_m[NW][R];
  __shared__ float s_l[NW][R];

  const uint64_t head_off = (uint64_t)kvh * BS * kRowBytes;
  float m = -INFINITY;
  float ell = 0.0f;
  f32x4_t acc[8];
#pragma unroll
  for (int nb = 0; nb < 8; ++nb) acc[nb] = f32x4_t{0.0f, 0.0f, 0.0f, 0.0f};

  // lane loads tokens 4j + kq of the step, dims 8 row .. +7: each load
  // instruction reads four whole 256-byte rows
  auto load_group = [&](int k, uint4 (&K)[4], uint4 (&V)[4], bool tail) {
    const int g = g_first + k * NW;
    const int tok0 = g * 16;
    uint64_t base[BPG];
#pragma unroll
    for (int b = 0; b < BPG; ++b)
      base[b] = (uint64_t)__builtin_amdgcn_readlane(my_phys[b], k) * a.tile_bytes + head_off + row * 16;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int t = 4 * j + kq;                        // token of the step
      const int b = BPG == 2 ? j / 2 : 0;              // its block when BS = 8
      const int rib = BS >= 16 ? tok0 % BS + t : t % BS;
      const uint64_t off = base[b] + (uint64_t)rib * kRowBytes;
      if (!tail || tok0 + t < n) {
        K[j] = nt_load16(a.kslab + off);
        V[j] = nt_load16(a.vslab + off);
      } else {
        K[j] = make_uint4(0, 0, 0, 0);
        V[j] = make_uint4(0, 0, 0, 0);
      }
    }
  };

  // this lane's transposing value read: token 4 kq + (lane / 4) % 4, dims 4 (lane % 4) ..
  const int tr_lane = (4 * kq + ((lane >> 2) & 3)) * kVRow + (lane & 3) * 8;
  int buf = 0;
  auto process_group = [&](int g, const uint4 (&K)[4], const uint4 (&V)[4], bool tail) {
    const int tok0 = g * 16;
    char* vb = s_v[wave][buf];
    char* kb = s_k[wave][buf];
    buf ^= 1;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      // token t = 4j + kq: key row t, value row t
      *reinterpret_cast<uint4*>(kb + (4 * j + kq) * kKRow + row * 16) = K[j];
      *reinterpret_cast<uint4*>(vb + (4 * j + kq) * kVRow + row * 16) = V[j];
    }
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    f32x4_t st = f32x4_t{0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
      const uint4 kx = *reinterpret_cast<const uint4*>(kb + row * kKRow + (32 * ks + 8 * kq) * 2);
      st = mfma_k32<BF16>(kx, qb[ks], st);
    }

    float sc[4];
    float mx = -INFINITY;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      sc[i] = st[i] * a.scale_log2;
      if (tail && tok0 + 4 * kq + i >= lim) sc[i] = -INFINITY;
      mx = fmaxf(mx, sc[i]);
    }
    mx = fmaxf(mx, __shfl_xor(mx, 16));
    mx = fmaxf(mx, __shfl_xor(mx, 32));
    if (__builtin_amdgcn_ballot_w64(mx > m + kRescaleSlack) != 0) {
      const float m_new = fmaxf(m, mx);
      const float f = (m_new == m) ? 1.0f : exp2_fast(m - m_new);
      m = m_new;
      ell *= f;
#pragma unroll
      for (int nb = 0; nb < 8; ++nb) acc[nb] *= f;
    }
    float pe[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      pe[i] = (tail && sc[i] == -INFINITY) ? 0.0f : exp2_fast(sc[i] - m);
      ell += pe[i];
    }
    // probabilities as the MFMA's 16-bit operand; bf16 keeps 8 significant
    // bits, so there the remainder goes in a second product (error ~2^-17)
    uint2 pb, pl = make_uint2(0, 0);
    pb.x = pack2<BF16>(pe[0], pe[1]);
    pb.y = pack2<BF16>(pe[2], pe[3]);
    if constexpr (BF16) {
      // what the rounding left out: p - bf16(p), itself rounded to bf16
      pl.x = pack2<true>(pe[0] - __builtin_bit_cast(float, pb.x << 16), pe[1] - __builtin_bit_cast(float, pb.x & 0xffff0000u));
      pl.y = pack2<true>(pe[2] - __builtin_bit_cast(float, pb.y << 16), pe[3] - __builtin_bit_cast(float, pb.y & 0xffff0000u));
    }
    // the value tile written above by all lanes of the wave
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    // V^T operand of dims 16 nb + row, tokens 4 kq .. +3: one transposing
    // read (lane a + 4 e of the 16-lane group kq addresses token 4 kq + e,
    // dims 16 nb + 4 a .. +3; lane 4 a + b receives dim 16 nb + 4 a + b of the
    // four tokens); the 32-byte row padding spreads each half-wave over all banks
    const char* vtr = vb + tr_lane;
#pragma unroll
    for (int nb = 0; nb < 8; ++nb) {
      const uint2 va = __builtin_bit_cast(uint2, __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4i16_t*)(vtr + 32 * nb)));
      acc[nb] = mfma_k16<BF16>(va, pb, acc[nb]);
      if constexpr (BF16) acc[nb] = mfma_k16<BF16>(va, pl, acc[nb]);
    }
  };

  {
    const int ng = g_full > g_first ? (g_full - g_first + NW - 1) / NW : 0;
    uint4 K0[4], V0[4], K1[4], V1[4];
    load_group(0, K0, V0, false);
    if (ng > 0) {
      int k = 0;
      for (; k + 2 < ng; k += 2) {
        load_group(k + 1, K1, V1, false);
        process_group(g_first + k * NW, K0, V0, false);
        load_group(k + 2, K0, V0, false);
        process_group(g_first + (k + 1) * NW, K1, V1, false);
      }
      if (k + 2 == ng) {
        load_group(k + 1, K1, V1, false);
        process_group(g_first + k * NW, K0, V0, false);
        process_group(g_first + (k + 1) * NW, K1, V1, false);
      } else {
        process_group(g_first + k * NW, K0, V0, false);
      }
    }
    // the steps at the causal edge and the context end, with per-row masks
    int g = g_full > g_first ? g_first + (g_full - g_first + NW - 1) / NW * NW : g_first;
    for (; g < g_last; g += NW) {
      load_group((g - g_first) / NW, K0, V0, true);
      process_group(g, K0, V0, true);
    }
  }

  // ---- combine: the four quarters of a row, then waves ----------------------
  ell += __shfl_xor(ell, 16);
  ell += __shfl_xor(ell, 32);
  __syncthreads();   // every wave is done with its value tiles
#pragma unroll
  for (int nb = 0; nb < 8; ++nb)
    *reinterpret_cast<float4*>(&s_acc[wave][row][16 * nb + 4 * kq]) =
        make_float4(acc[nb][0], acc[nb][1], acc[nb][2], acc[nb][3]);
  if (kq == 0) {
    s_m[wave][row] = m;
    s_l[wave][row] = ell;
  }
  __syncthreads();

  // one thread per (row, 8-dim chunk); fewer than 4 waves loop over them
  for (int t = threadIdx.x; t < R * 16; t += NW * 64) {
    const int wh = t >> 4;
    const int wc = t & 15;
    float A[8];
    float M = -INFINITY, Lsum = 0.0f;
#pragma unroll
    for (int w = 0; w < NW; ++w) M = fmaxf(M, s_m[w][wh]);
#pragma unroll
    for (int i = 0; i < 8; ++i) A[i] = 0.0f;
#pragma unroll
    for (int w = 0; w < NW; ++w) {
      const float mw = s_m[w][wh];
      const float wt = (mw == -INFINITY) ? 0.0f : exp2_fast(mw - M);
      Lsum += wt * s_l[w][wh];
      const float4 a0 = *reinterpret_cast<const float4*>(&s_acc[w][wh][8 * wc]);
      const float4 a1 = *reinterpret_cast<const float4*>(&s_acc[w][wh][8 * wc + 4]);
      A[0] += wt * a0.x; A[1] += wt * a0.y; A[2] += wt * a0.z; A[3] += wt * a0.w;
      A[4] += wt * a1.x; A[5] += wt * a1.y; A[6] += wt * a1.z; A[7] += wt * a1.w;
    }
    const int otq = tile * QT + wh / GQ;
    if (otq >= nq) continue;   // rows past the last query hold nothing anyone reads
    if (!GRP && nparts == 1) {
      const size_t orow = (size_t)(q0 + otq) * a.Hq + (size_t)kvh * GQ + wh % GQ;
      const float inv = Lsum > 0.0f ? 1.0f / Lsum : 0.0f;
      float o[8];
#pragma unroll
      for (int i = 0; i < 8; ++i) o[i] = A[i] * inv;
      *(reinterpret_cast<uint4*>(a.out + orow * kD) + wc) = narrow8<BF16>(o);
      continue;
    }
    const size_t pbase = (((size_t)s * a.ntiles + tile) * a.Hkv + kvh) * (size_t)a.nparts_max;
    float4* dst = reinterpret_cast<float4*>(a.ws_acc + ((pbase + p) * R + wh) * kD + 8 * wc);
    dst[0] = make_float4(A[0], A[1], A[2], A[3]);
    dst[1] = make_float4(A[4], A[5], A[6], A[7]);
    if (wc == 0) *reinterpret_cast<float2*>(a.ws_ml + ((pbase + p) * R + wh) * 2) = make_float2(M, Lsum);
  }
}

// Many rows per sequence (a chunk of a split prefill): one workgroup takes
// up to 64 RT rows of a (sequence, key/value head) -- query tokens x query
// heads -- and walks the sequence's whole context once, so there are no
// partial results to merge; further row tiles of the same sequence and head
// are further workgroups, dealt to the same XCD (head fastest in the grid),
// whose reads of the context mostly hit its L2.  Four waves own RT 16-row
// tiles each (wave w: rows 16 RT w ..); all waves share the 32-token steps.
// Keys and values travel from HBM straight into a ring of four LDS slots
// (direct-to-LDS loads, no registers in between): while step k's softmax
// and P.V run and step k+1's scores are taken, steps k+2 and k+3 are in
// flight; one barrier per step both publishes the step that landed and
// frees the slot the step before used.  A load
// instruction fills 1 KB of LDS (four token rows), lane by lane.  Key rows:
// token t's 16-byte chunk c sits at position c ^ (t % 16), so the 16 tokens
// whose rows one MFMA operand reads spread over all banks.  Values: each
// group of four token rows (one load instruction) 128 bytes past the last,
// and row e's chunk c at position c ^ 2e, so that the transposing LDS read
// (ds_read_b64_tr_b16: lane a + 4e of a 16-lane group addresses four
// elements of row e, lane 4a + b receives element b of rows 0..3) that
// builds a V^T operand touches distinct banks.  Per step and row tile, on
// the matrix cores (16x16x32 for both products):
//   S^T[token][row] = K[token][:] . Q[row][:] for the step's two 16-token
//       halves h: A = K rows of half h (lane: token lane % 16, dims
//       32 ks + 8 kq .. +7, read from LDS), B = Q^T held in registers; lane
//       (row, kq) gets the scores of tokens 16 h + 4 kq .. +3 of its row;
//   O^T[dim][row] += V^T[dim][token] . P^T[token][row] with the step's 32
//       tokens ordered so that lane (row, kq) supplies exactly its own eight
//       probabilities (tokens 4 kq .. +3 and 16 + 4 kq .. +3) as B; A = V^T in
//       the same token order, two transposing reads per operand;
//       lane (row, kq) accumulates dims 16 nb + 4 kq .. +3 of its row.
// The row's running maximum and normaliser live in the four lanes of the
// row (one per kq); bf16 probabilities enter P.V as a rounded part plus the
// rounded remainder (two products), fp16 ones as one.
constexpr int kWideTok = 32;                    // tokens per step
constexpr int kWideBufs = 4;                    // LDS ring slots: step k and the three after it
constexpr int kWideTabMax = 2048;               // table entries cached in LDS
constexpr int kWideVGroup = 72;                 // 16-byte chunks per group of four value rows (+8 pad)
constexpr int kWideSlot = kWideTok * 16 + (kWideTok / 4) * kWideVGroup;   // chunks per slot: keys, then values
// direct-to-LDS loads per lane and step: two key and two value chunks
constexpr int kWideLoadsPerStep = 4;

typedef __attribute__((address_space(3))) void lds_void_t;

// s_waitcnt immediate (gfx9 layout): vector-memory count vm, LDS count lgkm,
// export count left at its maximum
constexpr int waitcnt_imm(int vm, int lgkm) { return (vm & 0xF) | ((vm >> 4) << 14) | (0x7 << 4) | (lgkm << 8); }


template <bool BF16, int GQ, int BS, int RT, bool SCHED>
__global__ __launch_bounds__(256, 2) void mq_wide_kernel(const DecodeArgs a, const UnitList<SCHED> ul) {
  constexpr int NW = 4;
  constexpr int R = 16 * RT * NW;                 // rows per workgroup
  constexpr int QT = R / GQ;                      // query tokens per workgroup
  static_assert(QT * GQ == R, "rows = query tokens x query heads");
  static_assert(BS % 16 == 0 || BS == 8, "block size must be 8 or a multiple of 16");

  int kvh, s, tile;
  {
    const uint32_t id = blockIdx.x;               // head, then row tile, then sequence
    kvh = id % a.Hkv;
    uint32_t t = id / a.Hkv;
    tile = t % a.ntiles;
    t /= a.ntiles;
    if constexpr (SCHED) {                        // sequences longest first
      s = (int)ul.unit[min(t, (uint32_t)kMaxUnits - 1)];
    } else {
      s = (int)t;
    }
    if (s >= a.S) return;
  }
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int row = lane & 15;
  const int kq = lane >> 4;

  const int q0 = min(max(a.q_start[s], 0), a.T);
  const int nq = __builtin_amdgcn_readfirstlane(min(max(a.q_start[s + 1], q0), a.T) - q0);
  int n = a.lens[s];
  n = n < 0 ? 0 : (n > a.max_ctx ? a.max_ctx : n);
  n = __builtin_amdgcn_readfirstlane(n);
  if (tile * QT >= nq || nq > n) return;
  // positions the workgroup reads: up to what its last query sees
  const int n_wg = n - nq + min(tile * QT + QT, nq);
  const int nsteps = (n_wg + kWideTok - 1) / kWideTok;

  // query rows of this wave: Q^T operands, and each row tile's visible limit
  uint4 qb[RT][4];
  int lim[RT];
#pragma unroll
  for (int rt = 0; rt < RT; ++rt) {
    const int wrow = (wave * RT + rt) * 16 + row;     // row of the workgroup
    const int tq = tile * QT + wrow / GQ;
    const bool live = tq < nq;
    lim[rt] = live ? n - nq + tq + 1 : 0;
    const uint4* qrow = reinterpret_cast<const uint4*>(
        a.q + ((size_t)(live ? q0 + tq : 0) * a.Hq + (size_t)kvh * GQ + wrow % GQ) * kD);
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) qb[rt][ks] = live ? qrow[4 * ks + kq] : make_uint4(0, 0, 0, 0);
  }
  // scores enter the exponent as fma(s, c, -m) with c > 0: for a negative
  // scale the query changes sign instead (exact in 16-bit floats)
  const float c_log2 = fabsf(a.scale_log2);
  if (a.scale_log2 < 0.0f) {
#pragma unroll
    for (int rt = 0; rt < RT; ++rt)
#pragma unroll
      for (int ks = 0; ks < 4; ++ks) {
        qb[rt][ks].x ^= 0x80008000u;
        qb[rt][ks].y ^= 0x80008000u;
        qb[rt][ks].z ^= 0x80008000u;
        qb[rt][ks].w ^= 0x80008000u;
      }
  }
  // the first position some row of this wave cannot see: steps before it need no mask
  int wave_lim_min;
  {
    // the smallest limit over the wave's live rows (dead rows have limit 0)
    int v = 0x7fffffff;
#pragma unroll
    for (int rt = 0; rt < RT; ++rt) if (lim[rt] > 0) v = min(v, lim[rt]);
#pragma unroll
    for (int sh = 32; sh >= 1; sh >>= 1) v = min(v, __shfl_xor(v, sh));
    wave_lim_min = __builtin_amdgcn_readfirstlane(v);
  }

  // The ring slots are separate objects: the compiler then sees that a read
  // of one slot does not depend on the loads still landing in the others,
  // and leaves their waits to the explicit counts below.
  __shared__ __attribute__((aligned(16))) uint4 ring0[kWideSlot];
  __shared__ __attribute__((aligned(16))) uint4 ring1[kWideSlot];
  __shared__ __attribute__((aligned(16))) uint4 ring2[kWideSlot];
  __shared__ __attribute__((aligned(16))) uint4 ring3[kWideSlot];
  // the sequence's table row (physical blocks, clamped into the pool)
  __shared__ int s_tab[kWideTabMax];

  const uint64_t head_off = (uint64_t)kvh * BS * kRowBytes;
  const int32_t* table = a.tables + (size_t)s * a.maxb;
  const int nblk = (n_wg + BS - 1) / BS;
  const bool tab_lds = nblk <= kWideTabMax;    // else blocks come from the table in memory
  if (tab_lds) {
    for (int i = tid; i < nblk; i += 256) {
      const int e = table[i < a.maxb ? i : a.maxb - 1];
      s_tab[i] = e < 0 ? 0 : (e >= a.P ? a.P - 1 : e);
    }
  }
  __syncthreads();

  // Step k into a slot: each wave fills token rows 8 wave .. +7, one load
  // instruction per four rows and tensor; lane l lands in position l % 16 of
  // row l / 16, so it fetches the chunk that belongs there.  Every call
  // issues the same four loads (the step and the position are clamped; rows
  // past n_wg repeat a position the workgroup reads, and no row sees them),
  // so the wait counts below are exact.
  const int my_t = 8 * wave + (lane >> 4);
  const int kc16 = (lane & 15) ^ (my_t & 15);          // key: chunk at position ^ (t % 16), t = my_t + 4 j
  const int kc16b = (lane & 15) ^ ((my_t + 4) & 15);
  const int vc16 = (lane & 15) ^ (2 * (lane >> 4));    // value: row t % 4 = lane / 16
  // a whole step's token t: with B < 32 block 32 step / B + t / B, row t % B;
  // with B >= 32 the step's tokens share block 32 step / B, rows 32 step % B + t
  int lane_blk[2];
  uint32_t lane_k[2], lane_v[2];
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    const int t = my_t + 4 * j;
    lane_blk[j] = BS < kWideTok ? t / BS : 0;
    const uint32_t row_b = (uint32_t)head_off + (uint32_t)(BS < kWideTok ? t % BS : t) * kRowBytes;
    lane_k[j] = row_b + (j ? kc16b : kc16) * 16;
    lane_v[j] = row_b + vc16 * 16;
  }
  auto issue = [&](int k, uint4* slot) {
    const int kc = min(k, nsteps - 1);
    if (tab_lds && kc * kWideTok + kWideTok <= n_wg) {
      const int blk0 = kc * kWideTok / BS;
      const uint32_t step_row = BS < kWideTok ? 0u : (uint32_t)(kc * kWideTok % BS) * kRowBytes;
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        const uint64_t base = (uint64_t)s_tab[blk0 + lane_blk[j]] * a.tile_bytes + step_row;
        __builtin_amdgcn_global_load_lds(a.kslab + base + lane_k[j], (lds_void_t*)(slot + (8 * wave + 4 * j) * 16), 16, 0, 0);
        __builtin_amdgcn_global_load_lds(a.vslab + base + lane_v[j],
                                         (lds_void_t*)(slot + kWideTok * 16 + (2 * wave + j) * kWideVGroup), 16, 0, 0);
      }
      return;
    }
    // the last step (positions clamped to n_wg - 1: rows past it repeat a
    // position the workgroup reads, and no row sees them), or a table too
    // long for LDS
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const int t = my_t + 4 * j;
      const int tok = min(kc * kWideTok + t, n_wg - 1);
      int phys;
      if (tab_lds) {
        phys = s_tab[tok / BS];
      } else {
        const int e = table[tok / BS];
        phys = e < 0 ? 0 : (e >= a.P ? a.P - 1 : e);
      }
      const uint64_t row_off = (uint64_t)phys * a.tile_bytes + head_off + (uint64_t)(tok % BS) * kRowBytes;
      __builtin_amdgcn_global_load_lds(a.kslab + row_off + (j ? kc16b : kc16) * 16,
                                       (lds_void_t*)(slot + (8 * wave + 4 * j) * 16), 16, 0, 0);
      __builtin_amdgcn_global_load_lds(a.vslab + row_off + vc16 * 16,
                                       (lds_void_t*)(slot + kWideTok * 16 + (2 * wave + j) * kWideVGroup), 16, 0, 0);
    }
  };

  float m[RT], ell[RT];
  f32x4_t acc[RT][8];
#pragma unroll
  for (int rt = 0; rt < RT; ++rt) {
    m[rt] = -INFINITY;
    ell[rt] = 0.0f;
#pragma unroll
    for (int nb = 0; nb < 8; ++nb) acc[rt][nb] = f32x4_t{0.0f, 0.0f, 0.0f, 0.0f};
  }

  // scores of a step: two 16-token halves x RT row tiles
  auto scores = [&](const uint4* slot, f32x4_t (&sc)[RT][2]) {
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      uint4 kx[4];
#pragma unroll
      for (int ks = 0; ks < 4; ++ks) kx[ks] = slot[(16 * h + row) * 16 + ((4 * ks + kq) ^ row)];
#pragma unroll
      for (int rt = 0; rt < RT; ++rt) {
        f32x4_t st = f32x4_t{0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
        for (int ks = 0; ks < 4; ++ks) st = mfma_k32<BF16>(kx[ks], qb[rt][ks], st);
        sc[rt][h] = st;
      }
    }
  };

  // One step: the softmax of step k (its scores sc were taken in the step
  // before) and its P.V from slot cur, while the matrix cores already take
  // step k+1's scores from slot nxt; free: the slot of step k-1, refilled
  // with step k+3.  EDGE: some row of the wave stops inside step k
  // (per-row masks, and a row may have seen no position yet); otherwise
  // every score is finite.
  // this lane's transposing reads: source lane a + 4 e of its 16-lane group
  // addresses row e of the value group, dims 16 nb + 4 a .. +3, that is
  // chunk 2 nb + a / 2 (stored at 2 (nb ^ e) + a / 2) and its half a % 2
  const int tr_a = lane & 3, tr_e = (lane >> 2) & 3;
  const int tr_lane = kq * (kWideVGroup * 16) + tr_e * 256 + (tr_a >> 1) * 16 + (tr_a & 1) * 8;
  int voff[4];
#pragma unroll
  for (int q = 0; q < 4; ++q) voff[q] = tr_lane + 32 * (q ^ tr_e);
  f32x4_t sc[RT][2];
  auto run_step = [&](int k, const uint4* cur, const uint4* nxt, uint4* free_slot, auto edge_tag) {
    constexpr bool EDGE = decltype(edge_tag)::value;
    const char* vcol = reinterpret_cast<const char*>(cur + kWideTok * 16);
    // this lane's loads of step k+1 have landed (step k+2 may still be in
    // flight) and its reads of step k-1 are done; after the barrier the same
    // holds for every lane
    __builtin_amdgcn_s_waitcnt(waitcnt_imm((kWideBufs - 3) * kWideLoadsPerStep, 0));
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
    issue(k + kWideBufs - 1, free_slot);
    const int tok0 = k * kWideTok;
    // the row maxima of step k first (its scores sc were taken in the step
    // before; masked ones become -inf), and any rescale they call for
#pragma unroll
    for (int rt = 0; rt < RT; ++rt) {
      float mr = -INFINITY;
#pragma unroll
      for (int h = 0; h < 2; ++h)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          if (EDGE && tok0 + 16 * h + 4 * kq + i >= lim[rt]) sc[rt][h][i] = -INFINITY;
          mr = fmaxf(mr, sc[rt][h][i]);
        }
      mr = fmaxf(mr, __shfl_xor(mr, 16));     // the row's four lanes
      mr = fmaxf(mr, __shfl_xor(mr, 32));
      const float mx = (EDGE && mr == -INFINITY) ? -INFINITY : mr * c_log2;
      if (__builtin_amdgcn_ballot_w64(mx > m[rt] + kRescaleSlack) != 0) {
        const float m_new = fmaxf(m[rt], mx);
        const float f = (m_new == m[rt]) ? 1.0f : exp2_fast(m[rt] - m_new);
        m[rt] = m_new;
        ell[rt] *= f;
#pragma unroll
        for (int nb = 0; nb < 8; ++nb) acc[rt][nb] *= f;
      }
    }

    // step k+1's scores on the matrix cores (slot nxt has landed; after the
    // last step it holds a repeat, whose scores nobody uses), interleaved
    // with step k's exponentials and their packing on the vector unit
    f32x4_t sn[RT][2];
    scores(nxt, sn);
    uint4 pb[RT], pl[RT];
#pragma unroll
    for (int rt = 0; rt < RT; ++rt) {
      float pe[8];
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const float v = sc[rt][i >> 2][i & 3];
        pe[i] = (EDGE && v == -INFINITY) ? 0.0f : exp2_fast(fmaf(v, c_log2, -m[rt]));
        ell[rt] += pe[i];
      }
      pb[rt].x = pack2<BF16>(pe[0], pe[1]);
      pb[rt].y = pack2<BF16>(pe[2], pe[3]);
      pb[rt].z = pack2<BF16>(pe[4], pe[5]);
      pb[rt].w = pack2<BF16>(pe[6], pe[7]);
      if constexpr (BF16) {
        // what the rounding left out: p - bf16(p), itself rounded to bf16
        const uint32_t w[4] = {pb[rt].x, pb[rt].y, pb[rt].z, pb[rt].w};
        uint32_t r[4];
#pragma unroll
        for (int i = 0; i < 4; ++i)
          r[i] = pack2<true>(pe[2 * i] - __builtin_bit_cast(float, w[i] << 16),
                             pe[2 * i + 1] - __builtin_bit_cast(float, w[i] & 0xffff0000u));
        pl[rt] = make_uint4(r[0], r[1], r[2], r[3]);
      }
    }
    // one score product, then a share of the vector work, 16 RT times
#pragma unroll
    for (int i = 0; i < 8 * RT; ++i) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
      __builtin_amdgcn_sched_group_barrier(0x002, BF16 ? 6 : 3, 0);
    }

    // P.V: V^T operand of dims 16 nb + row, tokens 4 kq .. +3 (value group
    // kq) and 16 + 4 kq .. +3 (group 4 + kq), one transposing read each
#pragma unroll
    for (int nb = 0; nb < 8; ++nb) {
      const char* g = vcol + (nb >> 2) * 128 + voff[nb & 3];
      const v4i16_t lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4i16_t*)g);
      const v4i16_t hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4i16_t*)(g + 4 * kWideVGroup * 16));
      const uint2 l2 = __builtin_bit_cast(uint2, lo);
      const uint2 h2 = __builtin_bit_cast(uint2, hi);
      const uint4 va = make_uint4(l2.x, l2.y, h2.x, h2.y);
#pragma unroll
      for (int rt = 0; rt < RT; ++rt) {
        acc[rt][nb] = mfma_k32<BF16>(va, pb[rt], acc[rt][nb]);
        if constexpr (BF16) acc[rt][nb] = mfma_k32<BF16>(va, pl[rt], acc[rt][nb]);
      }
    }
#pragma unroll
    for (int rt = 0; rt < RT; ++rt) {
      sc[rt][0] = sn[rt][0];
      sc[rt][1] = sn[rt][1];
    }
  };

  // prologue: steps 0 .. 2 in flight, then step 0's scores
  issue(0, ring0);
  issue(1, ring1);
  issue(2, ring2);
  __builtin_amdgcn_s_waitcnt(waitcnt_imm((kWideBufs - 2) * kWideLoadsPerStep, 0));
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
  scores(ring0, sc);
  // steps every live row of the wave sees whole, four at a time so that each
  // slot is a fixed object; then the rest with masks
  const int k_edge = min(nsteps, wave_lim_min / kWideTok);
  int k = 0;
  for (; k + 4 <= k_edge; k += 4) {
    run_step(k, ring0, ring1, ring3, std::false_type{});
    run_step(k + 1, ring1, ring2, ring0, std::false_type{});
    run_step(k + 2, ring2, ring3, ring1, std::false_type{});
    run_step(k + 3, ring3, ring0, ring2, std::false_type{});
  }
  for (; k < nsteps; ++k) {
    switch (k & 3) {
      case 0: run_step(k, ring0, ring1, ring3, std::true_type{}); break;
      case 1: run_step(k, ring1, ring2, ring0, std::true_type{}); break;
      case 2: run_step(k, ring2, ring3, ring1, std::true_type{}); break;
      default: run_step(k, ring3, ring0, ring2, std::true_type{}); break;
    }
  }
  // the clamped loads issued past the last step land before the workgroup's
  // LDS is released
  __builtin_amdgcn_s_waitcnt(waitcnt_imm(0, 0));

  // each row: normaliser over its four lanes, then store
#pragma unroll
  for (int rt = 0; rt < RT; ++rt) {
    float l = ell[rt];
    l += __shfl_xor(l, 16);
    l += __shfl_xor(l, 32);
    if (lim[rt] == 0) continue;                  // a padding row: no query
    const int wrow = (wave * RT + rt) * 16 + row;
    const int tq = tile * QT + wrow / GQ;
    const float inv = l > 0.0f ? 1.0f / l : 0.0f;
    uint16_t* orow = a.out + ((size_t)(q0 + tq) * a.Hq + (size_t)kvh * GQ + wrow % GQ) * kD;
#pragma unroll
    for (int nb = 0; nb < 8; ++nb) {
      uint2 w;
      w.x = pack2<BF16>(acc[rt][nb][0] * inv, acc[rt][nb][1] * inv);
      w.y = pack2<BF16>(acc[rt][nb][2] * inv, acc[rt][nb][3] * inv);
      *reinterpret_cast<uint2*>(orow + 16 * nb + 4 * kq) = w;
    }
  }
}

__global__ void zero_kernel(uint4* p, uint64_t n16, uint8_t* tail, uint64_t ntail) {
  const uint64_t i = (uint64_t)blockIdx.x * blockDim.x + threadIdx.x;
  const uint64_t stride = (uint64_t)gridDim.x * blockDim.x;
  for (uint64_t k = i; k < n16; k += stride) p[k] = make_uint4(0, 0, 0, 0);
  if (i < ntail) tail[i] = 0;
}

// ---------------------------------------------------------------------------
// host-side launch configuration
// ---------------------------------------------------------------------------
constexpr int kWaves = 4;  // waves per workgroup

struct LaunchCfg {
  int part_tokens = 0;
  int nparts_max = 1;
};

// Partition length: as long as possible (fewer partials to merge) while the
// grid still has several workgroups per compute unit.  With long contexts a
// partition keeps at least 6 steps per wave (384 tokens): shorter ones spend
// more in start-up and in the merge than the extra workgroups gain (one
// key/value head over 64 sequences of 512-4096 tokens: 64-token partitions
// take 1.8x as long per layer as 384-token ones).
// Launches in longest-first order (unit lists) split each sequence into
// ceil(n / part) partitions of equal length and start from 24 steps per
// wave (1,536 tokens).  A workgroup is latency-bound: its first loads wait
// for two memory round trips, so a short partition moves its bytes at a
// fraction of a full one's rate; equal partitions have no short remainders
// (config-3 batch: 98 us per layer at 24 steps per wave, 101 at 12, against
// 100-101 with full partitions plus a remainder at 16-24 steps per wave,
// and 103-105 at 6-8).
LaunchCfg choose_launch(int S, int Hkv, int max_ctx, bool ordered = false) {
  int gpw = ordered ? 24 : 12;
  {
    // workgroups: 256 CUs x 8 for the fixed grid, whose workgroups past a
    // sequence's end cost little; a unit list holds live units only, and its
    // partitions are worth keeping long down to about one per CU (one GPU's
    // share of the GQA batch, 16/4 heads: 55.0 us per layer at 24 steps per
    // wave, 58.0 at 6; 4/1 heads: 21.6 at 12, 23.7 at 6)
    const int64_t target = ordered ? 256 : 2048;
    const int floor_gpw = max_ctx >= 2 * 16 * kWaves * 6 ? 6 : 1;
    while (gpw > floor_gpw) {
      const int64_t part = 16LL * kWaves * gpw;
      const int64_t wgs = (int64_t)S * Hkv * ((max_ctx + part - 1) / part);
      if (wgs >= target) break;
      gpw = std::max(gpw / 2, floor_gpw);
    }
  }
  LaunchCfg cfg;
  cfg.part_tokens = 16 * kWaves * gpw;
  cfg.nparts_max = max_ctx > 0 ? (max_ctx + cfg.part_tokens - 1) / cfg.part_tokens : 1;
  return cfg;
}

size_t align_up(size_t x, size_t a) { return (x + a - 1) / a * a; }

struct WsLayout {
  size_t ml_off = 0, acc_off = 0, total = 0;
};

WsLayout ws_layout(int S, int Hkv, int G, const LaunchCfg& cfg) {
  WsLayout w;
  if (cfg.nparts_max <= 1) return w;
  const size_t units = (size_t)S * Hkv;
  w.ml_off = 0;
  w.acc_off = w.ml_off + align_up(units * cfg.nparts_max * G * 2 * sizeof(float), 256);
  w.total = w.acc_off + align_up(units * cfg.nparts_max * G * kD * sizeof(float), 256);
  return w;
}

template <bool BF16, int G, int BS, int QT>
void launch_decode(const DecodeArgs& args, dim3 grid, hipStream_t stream) {
  hipLaunchKernelGGL((decode_attention_kernel<BF16, G, BS, kWaves, QT>), grid, dim3(kWaves * 64), 0, stream, args,
                     UnitList<false>{});
  if (args.nparts_max > 1)
    hipLaunchKernelGGL((decode_merge_kernel<BF16, G, QT>), dim3(args.Hkv, args.S, args.ntiles), dim3(G * 16), 0,
                       stream, args);
}

template <bool BF16, int G, int BS>
void launch_decode_ordered(const DecodeArgs& args, const UnitList<true>& ul, hipStream_t stream) {
  hipLaunchKernelGGL((decode_attention_kernel<BF16, G, BS, kWaves, 0, false, true>),
                     dim3((unsigned)(ul.count * args.Hkv)), dim3(kWaves * 64), 0, stream, args, ul);
  if (args.nparts_max > 1)
    hipLaunchKernelGGL((decode_merge_kernel<BF16, G, 0>), dim3(args.Hkv, args.S, 1), dim3(G * 16), 0, stream, args);
}

template <bool BF16, int BS>
bool dispatch_ordered(int G, const DecodeArgs& args, const UnitList<true>& ul, hipStream_t stream) {
  switch (G) {
    case 1: launch_decode_ordered<BF16, 1, BS>(args, ul, stream); return true;
    case 2: launch_decode_ordered<BF16, 2, BS>(args, ul, stream); return true;
    case 4: launch_decode_ordered<BF16, 4, BS>(args, ul, stream); return true;
    case 8: launch_decode_ordered<BF16, 8, BS>(args, ul, stream); return true;
    default: return false;
  }
}

// The units of a decode launch, longest first.  A sequence of n positions
// gets np = ceil(n / part) partitions of equal length (ceil(n / np) rounded
// up to 16; the last may be shorter by the rounding), so no partition is a
// short remainder.  An empty sequence is one unit of length 0 (it writes
// zeros) unless `keep_empty` is false.  Workgroups start in id order, so the
// device stays full until the shortest units, which start last.  Returns
// the count, or -1 when they do not fit one list.
// No heap use: a fixed array and an in-place sort whose key (length
// descending, then position in the list) orders like a stable sort.
int order_units(const int32_t* host_lens, int S, int max_ctx, int part, UnitList<true>& ul,
                bool keep_empty = true) {
  struct U { int len, idx; uint32_t word; };
  static thread_local U units[kMaxUnits];
  int cnt = 0;
  for (int s = 0; s < S; ++s) {
    const int n = std::min(std::max(host_lens[s], 0), max_ctx);
    if (n == 0 && !keep_empty) continue;
    const int np = n > 0 ? (n + part - 1) / part : 1;
    const int plen = np > 1 ? ((n + np - 1) / np + 15) / 16 * 16 : part;
    if ((int64_t)n > ((int64_t)1 << kUnitStepBits) * 16 - plen) return -1;
    if (cnt + np > kMaxUnits) return -1;
    for (int p = 0; p < np; ++p, ++cnt)
      units[cnt] = {std::max(std::min(plen, n - p * plen), 0), cnt,
                    ((uint32_t)s << kUnitStepBits) | (uint32_t)(p * plen / 16)};
  }
  std::sort(units, units + cnt, [](const U& x, const U& y) { return x.len != y.len ? x.len > y.len : x.idx < y.idx; });
  for (int c = 0; c < cnt; ++c) ul.unit[c] = units[c].word;
  ul.count = cnt;
  return cnt;
}

// G query heads per key/value head.  One query per sequence: the rows of a
// workgroup are those G heads.  Several: 8 rows = 8 / G query tokens x G heads.
template <bool BF16, int BS>
bool dispatch_g(int G, bool multi, const DecodeArgs& args, dim3 grid, hipStream_t stream) {
  if (multi) {
    switch (G) {
      case 1: launch_decode<BF16, 8, BS, 8>(args, grid, stream); return true;
      case 2: launch_decode<BF16, 8, BS, 4>(args, grid, stream); return true;
      case 4: launch_decode<BF16, 8, BS, 2>(args, grid, stream); return true;
      case 8: launch_decode<BF16, 8, BS, 1>(args, grid, stream); return true;
      default: return false;
    }
  }
  switch (G) {
    case 1: launch_decode<BF16, 1, BS, 0>(args, grid, stream); return true;
    case 2: launch_decode<BF16, 2, BS, 0>(args, grid, stream); return true;
    case 4: launch_decode<BF16, 4, BS, 0>(args, grid, stream); return true;
    case 8: launch_decode<BF16, 8, BS, 0>(args, grid, stream); return true;
    default: return false;
  }
}

// Several queries per sequence: rows = query tokens x G query heads per
// workgroup.  Up to 8 rows per sequence run on the vector path (the decode
// kernel with a query tile); up to 32 on the matrix cores with 16 rows per
// workgroup, its waves splitting the context; more on the matrix cores with
// 64 rows per workgroup, its waves splitting the rows over shared LDS tiles.
// 16-row tiles per wave of the wide kernel at most: two keep two waves per
// SIMD (four row tiles need one wave per SIMD, and at 64 queries per sequence
// with four query heads per key/value head took 472-504 us per call against
// 397-409 us for two)
constexpr int kWideMaxRt = 2;

struct MqPlan {
  bool mfma = false, wide = false;
  int rows = 8, qt = 1, ntiles = 1;
  int rt = 1;   // wide: 16-row tiles per wave (rows = 64 rt)
};

MqPlan mq_plan(int G, int max_q) {
  MqPlan p;
  const int64_t need = (int64_t)max_q * G;
  p.mfma = need > 8;
  p.wide = need > 32;
  if (p.wide) p.rt = need > kWideMaxRt * 32 ? kWideMaxRt : (need > 64 ? 2 : 1);
  p.rows = p.wide ? 16 * kWaves * p.rt : (p.mfma ? 16 : 8);
  p.qt = p.rows / G;
  p.ntiles = (int)((max_q + p.qt - 1) / p.qt);
  return p;
}

// Sequences longest first (unit = sequence index) for the wide kernel, which
// walks each sequence's whole context in one workgroup: the longest start
// first, the shortest fill in at the end.  Returns the count, or -1 when S
// exceeds one list.
int order_sequences(const int32_t* host_lens, int S, int max_ctx, UnitList<true>& ul) {
  if (S > kMaxUnits) return -1;
  struct U { int len, s; };
  static thread_local U units[kMaxUnits];
  for (int s = 0; s < S; ++s) units[s] = {std::min(std::max(host_lens[s], 0), max_ctx), s};
  std::sort(units, units + S, [](const U& x, const U& y) { return x.len != y.len ? x.len > y.len : x.s < y.s; });
  for (int c = 0; c < S; ++c) ul.unit[c] = (uint32_t)units[c].s;
  ul.count = S;
  return S;
}

template <bool BF16, int GQ, int BS, int RT, bool SCHED>
void launch_mq_wide(const DecodeArgs& args, const UnitList<SCHED>& ul, hipStream_t stream) {
  const dim3 grid((unsigned)((uint64_t)args.S * args.ntiles * args.Hkv));
  hipLaunchKernelGGL((mq_wide_kernel<BF16, GQ, BS, RT, SCHED>), grid, dim3(256), 0, stream, args, ul);
}

template <bool BF16, int BS, bool SCHED>
bool dispatch_mq_wide(int G, int rt, const DecodeArgs& args, const UnitList<SCHED>& ul, hipStream_t stream) {
#define PA_WIDE_CASE(GG)                                                   \
  case GG:                                                                 \
    if (rt == 1) launch_mq_wide<BF16, GG, BS, 1, SCHED>(args, ul, stream); \
    else launch_mq_wide<BF16, GG, BS, 2, SCHED>(args, ul, stream);         \
    return true;
  switch (G) {
    PA_WIDE_CASE(1)
    PA_WIDE_CASE(2)
    PA_WIDE_CASE(4)
    PA_WIDE_CASE(8)
    default: return false;
  }
#undef PA_WIDE_CASE
}

template <bool BF16, int GQ, int BS>
void launch_mq_mfma_ordered(const DecodeArgs& args, const UnitList<true>& ul, hipStream_t stream) {
  hipLaunchKernelGGL((mq_mfma_kernel<BF16, GQ, BS, kWaves, false, true>),
                     dim3((unsigned)(ul.count * args.ntiles * args.Hkv)), dim3(kWaves * 64), 0, stream, args, ul);
  if (args.nparts_max > 1)
    hipLaunchKernelGGL((decode_merge_kernel<BF16, 16, 16 / GQ>), dim3(args.Hkv, args.S, args.ntiles), dim3(16 * 16),
                       0, stream, args);
}

template <bool BF16, int BS>
bool dispatch_mq_ordered(int G, const DecodeArgs& args, const UnitList<true>& ul, hipStream_t stream) {
  switch (G) {
    case 1: launch_mq_mfma_ordered<BF16, 1, BS>(args, ul, stream); return true;
    case 2: launch_mq_mfma_ordered<BF16, 2, BS>(args, ul, stream); return true;
    case 4: launch_mq_mfma_ordered<BF16, 4, BS>(args, ul, stream); return true;
    case 8: launch_mq_mfma_ordered<BF16, 8, BS>(args, ul, stream); return true;
    default: return false;
  }
}

template <bool BF16, int GQ, int BS>
void launch_mq_mfma(const DecodeArgs& args, dim3 grid, hipStream_t stream) {
  hipLaunchKernelGGL((mq_mfma_kernel<BF16, GQ, BS, kWaves>), grid, dim3(kWaves * 64), 0, stream, args,
                     UnitList<false>{});
  if (args.nparts_max > 1)
    hipLaunchKernelGGL((decode_merge_kernel<BF16, 16, 16 / GQ>), dim3(args.Hkv, args.S, args.ntiles), dim3(16 * 16),
                       0, stream, args);
}

template <bool BF16, int BS>
bool dispatch_mfma(int G, const DecodeArgs& args, dim3 grid, hipStream_t stream) {
  switch (G) {
    case 1: launch_mq_mfma<BF16, 1, BS>(args, grid, stream); return true;
    case 2: launch_mq_mfma<BF16, 2, BS>(args, grid, stream); return true;
    case 4: launch_mq_mfma<BF16, 4, BS>(args, grid, stream); return true;
    case 8: launch_mq_mfma<BF16, 8, BS>(args, grid, stream); return true;
    default: return false;
  }
}

}  // namespace

namespace {

// q_start == nullptr: one query per sequence (decode).  Otherwise sequence s
// has queries q_start[s] .. q_start[s+1]-1 of T rows, at most max_q of them.
pa_status decode_launch(pa_pool* pool, int layer, void* out, const void* q, int S, int Hq,
                        const int32_t* block_tables, int maxb, const int32_t* context_lens, int max_ctx, float scale,
                        void* workspace, size_t ws_bytes, const void* k_new, const void* v_new,
                        const int64_t* slot_mapping, const int32_t* q_start, int T, int max_q, hipStream_t stream,
                        const int32_t* host_lens = nullptr, bool static_scratch = false) {
  if (!pool) return fail(PA_ERR_INVALID_ARG, "pool is NULL");
  if (layer < 0 || layer >= pool->L) return fail(PA_ERR_INVALID_ARG, "layer out of range");
  if (S < 0) return fail(PA_ERR_INVALID_ARG, "negative S");
  if (S == 0) return PA_OK;
  if (Hq <= 0 || Hq % pool->Hkv) return fail(PA_ERR_INVALID_ARG, "Hq must be a positive multiple of Hkv");
  const int G = Hq / pool->Hkv;
  if (G != 1 && G != 2 && G != 4 && G != 8) return fail(PA_ERR_UNSUPPORTED, "Hq / Hkv must be 1, 2, 4 or 8");
  if (pool->d != kD) return fail(PA_ERR_UNSUPPORTED, "head dimension must be 128");
  if (pool->B != 8 && pool->B != 16 && pool->B != 32 && pool->B != 64 && pool->B != 128)
    return fail(PA_ERR_UNSUPPORTED, "block size must be 8, 16, 32, 64 or 128");
  if (!out || !q || !block_tables || !context_lens) return fail(PA_ERR_INVALID_ARG, "NULL device pointer");
  if (!aligned(out, 16) || !aligned(q, 16)) return fail(PA_ERR_INVALID_ARG, "q and out must be 16-byte aligned");
  if (!aligned(block_tables, 4) || !aligned(context_lens, 4))
    return fail(PA_ERR_INVALID_ARG, "block_tables and context_lens must be 4-byte aligned");
  if (maxb <= 0 || max_ctx < 0) return fail(PA_ERR_INVALID_ARG, "bad maxb or max_ctx");
  if ((int64_t)max_ctx > (int64_t)maxb * pool->B) return fail(PA_ERR_INVALID_ARG, "max_ctx exceeds maxb * B");
  if (!std::isfinite(scale)) return fail(PA_ERR_INVALID_ARG, "scale must be finite");
  if (S > 65535 || pool->Hkv > 65535) return fail(PA_ERR_UNSUPPORTED, "at most 65535 sequences and heads");
  const bool multi = q_start != nullptr;
  MqPlan plan;
  if (multi) {
    if (!aligned(q_start, 4)) return fail(PA_ERR_INVALID_ARG, "q_start must be 4-byte aligned");
    if (T < 0 || max_q < 0) return fail(PA_ERR_INVALID_ARG, "negative T or max_q");
    if (T == 0 || max_q == 0) return PA_OK;
    plan = mq_plan(G, max_q);
    if (plan.ntiles > 65535) return fail(PA_ERR_UNSUPPORTED, "max_q too large");
  }
  const int ntiles = plan.ntiles;
  const int rows = multi ? plan.rows : G;

  // A unit list (longest first) when host lengths are given and the shape
  // allows one: single-query decode, or several queries whose rows fit one
  // 16-row matrix tile.  If the units do not fit a list, the launch is the
  // unordered one, with its own partition length.
  const bool want_list = host_lens != nullptr && (!multi || (plan.mfma && !plan.wide && ntiles == 1));
  static thread_local UnitList<true> ul;
  LaunchCfg cfg = choose_launch(S * ntiles, pool->Hkv, max_ctx, want_list);
  const bool use_list = want_list && order_units(host_lens, S, max_ctx, cfg.part_tokens, ul) > 0;
  if (want_list && !use_list) cfg = choose_launch(S * ntiles, pool->Hkv, max_ctx, false);
  // The wide kernel walks a sequence's whole context in one workgroup: no
  // partitions, no workspace; with host lengths the sequences go longest first.
  bool wide_list = false;
  if (multi && plan.wide) {
    cfg.part_tokens = max_ctx > 0 ? max_ctx : 1;
    cfg.nparts_max = 1;
    wide_list = host_lens != nullptr && order_sequences(host_lens, S, max_ctx, ul) > 0;
  }
  const WsLayout wl = ws_layout(S * ntiles, pool->Hkv, rows, cfg);
  char* ws = static_cast<char*>(workspace);
  if (wl.total > 0) {
    if (static_scratch && ws_bytes < wl.total)
      return fail(PA_ERR_INVALID_ARG, "this call needs " + std::to_string(wl.total) +
                                          " bytes of partial results; the static scratch holds " +
                                          std::to_string(ws_bytes) + " (use pa_decode_attention_ordered)");
    if (!ws || !aligned(ws, 256)) return fail(PA_ERR_INVALID_ARG, "workspace must be a 256-byte aligned device pointer");
    if (ws_bytes < wl.total) return fail(PA_ERR_INVALID_ARG, "workspace smaller than pa_decode_workspace_bytes");
  }

  DecodeArgs args;
  args.kslab = pool->k_slab(layer);
  args.vslab = pool->v_slab(layer);
  args.tile_bytes = pool->tile_bytes;
  args.q = static_cast<const uint16_t*>(q);
  args.out = static_cast<uint16_t*>(out);
  args.tables = block_tables;
  args.lens = context_lens;
  args.ws_ml = wl.total ? reinterpret_cast<float*>(ws + wl.ml_off) : nullptr;
  args.ws_acc = wl.total ? reinterpret_cast<float*>(ws + wl.acc_off) : nullptr;
  args.S = S;
  args.Hq = Hq;
  args.Hkv = pool->Hkv;
  args.P = pool->P;
  args.maxb = maxb;
  args.max_ctx = max_ctx;
  args.part_tokens = cfg.part_tokens;
  args.nparts_max = cfg.nparts_max;
  args.scale_log2 = (float)((double)scale * 1.4426950408889634);
  args.knew = static_cast<const uint4*>(k_new);
  args.vnew = static_cast<const uint4*>(v_new);
  args.slots = slot_mapping;
  args.nslots = (int64_t)pool->P * pool->B;
  args.q_start = q_start;
  args.ntiles = ntiles;
  args.T = T;

  const uint64_t nwg = (uint64_t)pool->Hkv * S * ntiles * cfg.nparts_max;
  if (nwg > 0x7fffffffULL) return fail(PA_ERR_UNSUPPORTED, "grid too large");
  const dim3 grid((unsigned)nwg);
  bool ok;
  const bool bf16 = pool->dtype == PA_BF16;
  if (multi && plan.wide) {      // many rows per sequence: one workgroup walks the whole context
#define PA_WIDE_B(BB)                                                                          \
  case BB:                                                                                     \
    if (wide_list)                                                                             \
      ok = bf16 ? dispatch_mq_wide<true, BB, true>(G, plan.rt, args, ul, stream)               \
                : dispatch_mq_wide<false, BB, true>(G, plan.rt, args, ul, stream);             \
    else                                                                                       \
      ok = bf16 ? dispatch_mq_wide<true, BB, false>(G, plan.rt, args, UnitList<false>{}, stream) \
                : dispatch_mq_wide<false, BB, false>(G, plan.rt, args, UnitList<false>{}, stream); \
    break;
    switch (pool->B) {
      PA_WIDE_B(8)
      PA_WIDE_B(16)
      PA_WIDE_B(32)
      PA_WIDE_B(64)
      default:
      PA_WIDE_B(128)
    }
#undef PA_WIDE_B
    if (!ok) return fail(PA_ERR_UNSUPPORTED, "no kernel for this shape");
    return hip_check(hipGetLastError(), "multi-query attention launch");
  }
  if (use_list && multi) {       // several queries per sequence, one tile each
    switch (pool->B) {
      case 8: ok = bf16 ? dispatch_mq_ordered<true, 8>(G, args, ul, stream) : dispatch_mq_ordered<false, 8>(G, args, ul, stream); break;
      case 16: ok = bf16 ? dispatch_mq_ordered<true, 16>(G, args, ul, stream) : dispatch_mq_ordered<false, 16>(G, args, ul, stream); break;
      case 32: ok = bf16 ? dispatch_mq_ordered<true, 32>(G, args, ul, stream) : dispatch_mq_ordered<false, 32>(G, args, ul, stream); break;
      case 64: ok = bf16 ? dispatch_mq_ordered<true, 64>(G, args, ul, stream) : dispatch_mq_ordered<false, 64>(G, args, ul, stream); break;
      default: ok = bf16 ? dispatch_mq_ordered<true, 128>(G, args, ul, stream) : dispatch_mq_ordered<false, 128>(G, args, ul, stream); break;
    }
    if (!ok) return fail(PA_ERR_UNSUPPORTED, "no kernel for this shape");
    return hip_check(hipGetLastError(), "multi-query attention launch");
  }
  if (use_list) {
    switch (pool->B) {
      case 8: ok = bf16 ? dispatch_ordered<true, 8>(G, args, ul, stream) : dispatch_ordered<false, 8>(G, args, ul, stream); break;
      case 16: ok = bf16 ? dispatch_ordered<true, 16>(G, args, ul, stream) : dispatch_ordered<false, 16>(G, args, ul, stream); break;
      case 32: ok = bf16 ? dispatch_ordered<true, 32>(G, args, ul, stream) : dispatch_ordered<false, 32>(G, args, ul, stream); break;
      case 64: ok = bf16 ? dispatch_ordered<true, 64>(G, args, ul, stream) : dispatch_ordered<false, 64>(G, args, ul, stream); break;
      default: ok = bf16 ? dispatch_ordered<true, 128>(G, args, ul, stream) : dispatch_ordered<false, 128>(G, args, ul, stream); break;
    }
    if (!ok) return fail(PA_ERR_UNSUPPORTED, "no kernel for this shape");
    return hip_check(hipGetLastError(), "decode attention launch");
  }
  if (multi && plan.mfma) {
    switch (pool->B) {
      case 8: ok = bf16 ? dispatch_mfma<true, 8>(G, args, grid, stream) : dispatch_mfma<false, 8>(G, args, grid, stream); break;
      case 16: ok = bf16 ? dispatch_mfma<true, 16>(G, args, grid, stream) : dispatch_mfma<false, 16>(G, args, grid, stream); break;
      case 32: ok = bf16 ? dispatch_mfma<true, 32>(G, args, grid, stream) : dispatch_mfma<false, 32>(G, args, grid, stream); break;
      case 64: ok = bf16 ? dispatch_mfma<true, 64>(G, args, grid, stream) : dispatch_mfma<false, 64>(G, args, grid, stream); break;
      default: ok = bf16 ? dispatch_mfma<true, 128>(G, args, grid, stream) : dispatch_mfma<false, 128>(G, args, grid, stream); break;
    }
    if (!ok) return fail(PA_ERR_UNSUPPORTED, "no kernel for this shape");
    return hip_check(hipGetLastError(), "multi-query attention launch");
  }
  switch (pool->B) {
    case 8: ok = bf16 ? dispatch_g<true, 8>(G, multi, args, grid, stream) : dispatch_g<false, 8>(G, multi, args, grid, stream); break;
    case 16: ok = bf16 ? dispatch_g<true, 16>(G, multi, args, grid, stream) : dispatch_g<false, 16>(G, multi, args, grid, stream); break;
    case 32: ok = bf16 ? dispatch_g<true, 32>(G, multi, args, grid, stream) : dispatch_g<false, 32>(G, multi, args, grid, stream); break;
    case 64: ok = bf16 ? dispatch_g<true, 64>(G, multi, args, grid, stream) : dispatch_g<false, 64>(G, multi, args, grid, stream); break;
    default: ok = bf16 ? dispatch_g<true, 128>(G, multi, args, grid, stream) : dispatch_g<false, 128>(G, multi, args, grid, stream); break;
  }
  if (!ok) return fail(PA_ERR_UNSUPPORTED, "no kernel for this shape");
  return hip_check(hipGetLastError(), "decode attention launch");
}

// Grouped decode: the group pass (shared prefixes, 16-row matrix-core
// kernel over each group's members), the suffix pass (the decode kernel from
// each sequence's first own position, with the fused cache write when slots
// are given), then the cascade merge.
struct GroupedLayout {
  LaunchCfg gcfg, scfg;
  int gntiles = 0;
  size_t g_ml = 0, g_acc = 0, s_ml = 0, s_acc = 0, total = 0;
};

// The group pass runs two-wave workgroups: shared prompts are short, and
// with four waves each would get only a few steps.
constexpr int kGroupWaves = 2;

// The suffix pass runs one-wave workgroups (two for G = 8: the kernel stages
// the query and combines with G * 16 threads): suffixes are short (the tail
// of a prompt's last block plus the tokens generated since the fork).
constexpr int suffix_waves(int G) { return G <= 4 ? 1 : 2; }
constexpr int kSuffixPart = 16 * 16;   // 16 steps of 16 tokens per partition

GroupedLayout grouped_layout(int S, int Hkv, int G, int max_suffix, int ngroups, int max_group, int max_shared,
                             bool shortest, bool ordered = false) {
  GroupedLayout w;
  w.gntiles = ngroups > 0 ? (int)(((int64_t)max_group * G + 15) / 16) : 0;
  if (shortest) {   // the shortest partition the launcher can pick: a bound for every call
    w.gcfg.part_tokens = 16 * kWaves;
  } else {
    w.gcfg = choose_launch(ngroups * w.gntiles, Hkv, max_shared, ordered);
    // a lane of a group-pass wave holds the block of one of its steps
    w.gcfg.part_tokens = std::min(w.gcfg.part_tokens, 16 * 64 * kGroupWaves);
  }
  w.scfg.part_tokens = kSuffixPart;
  w.gcfg.nparts_max = max_shared > 0 ? (max_shared + w.gcfg.part_tokens - 1) / w.gcfg.part_tokens : 1;
  w.scfg.nparts_max = max_suffix > 0 ? (max_suffix + w.scfg.part_tokens - 1) / w.scfg.part_tokens : 1;
  const size_t gunits = (size_t)ngroups * w.gntiles * Hkv * w.gcfg.nparts_max * 16;
  const size_t sunits = (size_t)S * Hkv * w.scfg.nparts_max * G;
  w.g_ml = 0;
  w.g_acc = w.g_ml + align_up(gunits * 2 * sizeof(float), 256);
  w.s_ml = w.g_acc + align_up(gunits * kD * sizeof(float), 256);
  w.s_acc = w.s_ml + align_up(sunits * 2 * sizeof(float), 256);
  w.total = w.s_acc + align_up(sunits * kD * sizeof(float), 256);
  return w;
}

template <bool BF16, int G, int BS>
void launch_grouped(const DecodeArgs& ga, dim3 ggrid, const DecodeArgs& sa, dim3 sgrid, const DecodeArgs& ma,
                    const UnitList<true>* gul, hipStream_t stream) {
  if (gul != nullptr)
    hipLaunchKernelGGL((mq_mfma_kernel<BF16, G, BS, kGroupWaves, true, true>),
                       dim3((unsigned)(gul->count * ga.ntiles * ga.Hkv)), dim3(kGroupWaves * 64), 0, stream, ga, *gul);
  else if (ggrid.x > 0)
    hipLaunchKernelGGL((mq_mfma_kernel<BF16, G, BS, kGroupWaves, true>), ggrid, dim3(kGroupWaves * 64), 0, stream, ga,
                       UnitList<false>{});
  constexpr int NWS = suffix_waves(G);
  static_assert(NWS * 64 >= G * 16, "the decode kernel needs G * 16 threads");
  hipLaunchKernelGGL((decode_attention_kernel<BF16, G, BS, NWS, 0, true>), sgrid, dim3(NWS * 64), 0, stream, sa,
                     UnitList<false>{});
  if (!sa.fold) hipLaunchKernelGGL((cascade_merge_kernel<BF16, G>), dim3(ma.Hkv, ma.S), dim3(G * 16), 0, stream, ma);
}

template <bool BF16, int BS>
bool dispatch_grouped(int G, const DecodeArgs& ga, dim3 ggrid, const DecodeArgs& sa, dim3 sgrid, const DecodeArgs& ma,
                      const UnitList<true>* gul,
                      hipStream_t stream) {
  switch (G) {
    case 1: launch_grouped<BF16, 1, BS>(ga, ggrid, sa, sgrid, ma, gul, stream); return true;
    case 2: launch_grouped<BF16, 2, BS>(ga, ggrid, sa, sgrid, ma, gul, stream); return true;
    case 4: launch_grouped<BF16, 4, BS>(ga, ggrid, sa, sgrid, ma, gul, stream); return true;
    case 8: launch_grouped<BF16, 8, BS>(ga, ggrid, sa, sgrid, ma, gul, stream); return true;
    default: return false;
  }
}

pa_status grouped_launch(pa_pool* pool, int layer, void* out, const void* q, int S, int Hq,
                         const int32_t* block_tables, int maxb, const int32_t* context_lens, int max_ctx,
                         const int32_t* group_start, const int32_t* group_len, const int32_t* seq_group, int ngroups,
                         int max_group, int max_shared, int max_suffix, float scale, void* workspace, size_t ws_bytes,
                         const void* k_new, const void* v_new, const int64_t* slot_mapping, hipStream_t stream,
                         const int32_t* host_group_len = nullptr) {
  if (!pool) return fail(PA_ERR_INVALID_ARG, "pool is NULL");
  if (layer < 0 || layer >= pool->L) return fail(PA_ERR_INVALID_ARG, "layer out of range");
  if (S < 0) return fail(PA_ERR_INVALID_ARG, "negative S");
  if (S == 0) return PA_OK;
  if (Hq <= 0 || Hq % pool->Hkv) return fail(PA_ERR_INVALID_ARG, "Hq must be a positive multiple of Hkv");
  const int G = Hq / pool->Hkv;
  if (G != 1 && G != 2 && G != 4 && G != 8) return fail(PA_ERR_UNSUPPORTED, "Hq / Hkv must be 1, 2, 4 or 8");
  if (pool->d != kD) return fail(PA_ERR_UNSUPPORTED, "head dimension must be 128");
  if (pool->B != 8 && pool->B != 16 && pool->B != 32 && pool->B != 64 && pool->B != 128)
    return fail(PA_ERR_UNSUPPORTED, "block size must be 8, 16, 32, 64 or 128");
  if (!out || !q || !block_tables || !context_lens || !seq_group) return fail(PA_ERR_INVALID_ARG, "NULL device pointer");
  if (!aligned(out, 16) || !aligned(q, 16)) return fail(PA_ERR_INVALID_ARG, "q and out must be 16-byte aligned");
  if (!aligned(block_tables, 4) || !aligned(context_lens, 4) || !aligned(seq_group, 4))
    return fail(PA_ERR_INVALID_ARG, "int32 arrays must be 4-byte aligned");
  if (maxb <= 0 || max_ctx < 0) return fail(PA_ERR_INVALID_ARG, "bad maxb or max_ctx");
  if ((int64_t)max_ctx > (int64_t)maxb * pool->B) return fail(PA_ERR_INVALID_ARG, "max_ctx exceeds maxb * B");
  if (!std::isfinite(scale)) return fail(PA_ERR_INVALID_ARG, "scale must be finite");
  if (S > 65535 || pool->Hkv > 65535) return fail(PA_ERR_UNSUPPORTED, "at most 65535 sequences and heads");
  if (ngroups < 0 || max_group < 0 || max_shared < 0) return fail(PA_ERR_INVALID_ARG, "negative group sizes");
  if (ngroups > 0 && (!group_start || !group_len || !aligned(group_start, 4) || !aligned(group_len, 4)))
    return fail(PA_ERR_INVALID_ARG, "group_start and group_len must be 4-byte aligned device pointers");
  if (ngroups > 65535 || max_group > S) return fail(PA_ERR_INVALID_ARG, "bad ngroups or max_group");
  if (max_shared > max_ctx) return fail(PA_ERR_INVALID_ARG, "max_shared exceeds max_ctx");
  if (max_suffix < 0 || max_suffix > max_ctx) return fail(PA_ERR_INVALID_ARG, "bad max_suffix");
  if (k_new || v_new || slot_mapping) {
    if (!k_new || !v_new || !slot_mapping) return fail(PA_ERR_INVALID_ARG, "k, v and slot_mapping go together");
    if (!aligned(k_new, 16) || !aligned(v_new, 16) || !aligned(slot_mapping, 8))
      return fail(PA_ERR_INVALID_ARG, "k and v must be 16-byte aligned, slot_mapping 8-byte aligned");
  }
  // group pass in longest-first order over equal partitions of each group's
  // shared positions (as the kernels count them: capped at max_shared and
  // rounded down to 16); if they do not fit one list, the unordered layout
  static thread_local UnitList<true> gunits;
  bool use_list = false;
  GroupedLayout wl;
  if (host_group_len != nullptr && ngroups > 0 && max_shared >= 16) {
    wl = grouped_layout(S, pool->Hkv, G, max_suffix, ngroups, max_group, max_shared, false, true);
    std::vector<int32_t> shared(ngroups);
    for (int g = 0; g < ngroups; ++g) shared[g] = std::min(std::max(host_group_len[g], 0), max_shared) & ~15;
    use_list = order_units(shared.data(), ngroups, max_shared, wl.gcfg.part_tokens, gunits, false) > 0 &&
               (int64_t)gunits.count * wl.gntiles * pool->Hkv <= 0x7fffffffLL;
  }
  if (!use_list) wl = grouped_layout(S, pool->Hkv, G, max_suffix, ngroups, max_group, max_shared, false);
  char* ws = static_cast<char*>(workspace);
  if (!ws || !aligned(ws, 256)) return fail(PA_ERR_INVALID_ARG, "workspace must be a 256-byte aligned device pointer");
  if (ws_bytes < wl.total) return fail(PA_ERR_INVALID_ARG, "workspace smaller than pa_decode_grouped_workspace_bytes");

  DecodeArgs args;
  args.kslab = pool->k_slab(layer);
  args.vslab = pool->v_slab(layer);
  args.tile_bytes = pool->tile_bytes;
  args.q = static_cast<const uint16_t*>(q);
  args.out = static_cast<uint16_t*>(out);
  args.tables = block_tables;
  args.lens = context_lens;
  args.S = S;
  args.Hq = Hq;
  args.Hkv = pool->Hkv;
  args.P = pool->P;
  args.maxb = maxb;
  args.max_ctx = max_ctx;
  args.scale_log2 = (float)((double)scale * 1.4426950408889634);
  args.knew = nullptr;
  args.vnew = nullptr;
  args.slots = nullptr;
  args.nslots = (int64_t)pool->P * pool->B;
  args.q_start = group_start;   // the merge finds each group's first member here
  args.ntiles = 1;
  args.T = S;
  args.grp_len = group_len;
  args.seq_group = seq_group;
  args.ngroups = ngroups;
  args.max_shared = max_shared;
  args.gws_ml = reinterpret_cast<float*>(ws + wl.g_ml);
  args.gws_acc = reinterpret_cast<float*>(ws + wl.g_acc);
  args.gpart_tokens = wl.gcfg.part_tokens;
  args.gparts_max = wl.gcfg.nparts_max;
  args.gntiles = wl.gntiles;
  args.ws_ml = reinterpret_cast<float*>(ws + wl.s_ml);
  args.ws_acc = reinterpret_cast<float*>(ws + wl.s_acc);
  args.part_tokens = wl.scfg.part_tokens;
  args.nparts_max = wl.scfg.nparts_max;

  // group pass: "sequences" are the groups, query tokens their members
  DecodeArgs ga = args;
  ga.S = ngroups;
  ga.q_start = group_start;
  ga.ntiles = wl.gntiles;
  ga.part_tokens = wl.gcfg.part_tokens;
  ga.nparts_max = wl.gcfg.nparts_max;
  ga.ws_ml = args.gws_ml;
  ga.ws_acc = args.gws_acc;
  const uint64_t gwg = (ngroups > 0 && max_shared >= 16)
                           ? (uint64_t)pool->Hkv * ngroups * wl.gntiles * wl.gcfg.nparts_max : 0;
  // suffix pass (with this step's cache write, if given)
  DecodeArgs sa = args;
  sa.fold = wl.scfg.nparts_max <= 1 ? 1 : 0;   // every suffix fits one partition: no merge launch
  sa.knew = static_cast<const uint4*>(k_new);
  sa.vnew = static_cast<const uint4*>(v_new);
  sa.slots = slot_mapping;
  const uint64_t swg = (uint64_t)pool->Hkv * S * wl.scfg.nparts_max;
  if (gwg > 0x7fffffffULL || swg > 0x7fffffffULL) return fail(PA_ERR_UNSUPPORTED, "grid too large");
  const dim3 ggrid((unsigned)gwg), sgrid((unsigned)swg);
  const UnitList<true>* gul = use_list ? &gunits : nullptr;
  bool ok;
  const bool bf16 = pool->dtype == PA_BF16;
  switch (pool->B) {
    case 8: ok = bf16 ? dispatch_grouped<true, 8>(G, ga, ggrid, sa, sgrid, args, gul, stream)
                      : dispatch_grouped<false, 8>(G, ga, ggrid, sa, sgrid, args, gul, stream); break;
    case 16: ok = bf16 ? dispatch_grouped<true, 16>(G, ga, ggrid, sa, sgrid, args, gul, stream)
                       : dispatch_grouped<false, 16>(G, ga, ggrid, sa, sgrid, args, gul, stream); break;
    case 32: ok = bf16 ? dispatch_grouped<true, 32>(G, ga, ggrid, sa, sgrid, args, gul, stream)
                       : dispatch_grouped<false, 32>(G, ga, ggrid, sa, sgrid, args, gul, stream); break;
    case 64: ok = bf16 ? dispatch_grouped<true, 64>(G, ga, ggrid, sa, sgrid, args, gul, stream)
                       : dispatch_grouped<false, 64>(G, ga, ggrid, sa, sgrid, args, gul, stream); break;
    default: ok = bf16 ? dispatch_grouped<true, 128>(G, ga, ggrid, sa, sgrid, args, gul, stream)
                       : dispatch_grouped<false, 128>(G, ga, ggrid, sa, sgrid, args, gul, stream); break;
  }
  if (!ok) return fail(PA_ERR_UNSUPPORTED, "no kernel for this shape");
  return hip_check(hipGetLastError(), "grouped decode attention launch");
}

}  // namespace

// ---------------------------------------------------------------------------
// Static scratch for pa_decode_attention_ordered_noalloc: the split-K
// partials live in this file-scope device array instead of a caller's
// workspace.  Each device that runs the call holds its own copy until the
// process ends; kernels reach it through the address hipGetSymbolAddress
// returns on that device (the array's name in host code is only a stand-in).
// ---------------------------------------------------------------------------
constexpr size_t kStaticScratchBytes = (size_t)32 << 20;
static __device__ __align__(256) unsigned char scratch[kStaticScratchBytes];

namespace {

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

// The current device's address of `scratch`, looked up once per device.
pa_status static_scratch_ptr(void** out) {
  int dev = -1;
  if (pa_status st = hip_check(hipGetDevice(&dev), "hipGetDevice")) return st;
  if (dev < 0 || dev >= kMaxDevices) return fail(PA_ERR_UNSUPPORTED, "device index above 63");
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    if (pa_status st = hip_check(hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)), "hipGetSymbolAddress(scratch)"))
      return st;
    if (!p) return fail(PA_ERR_HIP, "hipGetSymbolAddress(scratch) returned NULL");
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return PA_OK;
}

}  // namespace

extern "C" {

size_t pa_decode_workspace_bytes(const pa_pool* pool, int S, int Hq, int max_ctx) {
  if (!pool || S <= 0 || Hq <= 0 || max_ctx < 0 || Hq % pool->Hkv) return 0;
  // Sized for the shortest partition the launcher can pick, so the result
  // never decreases with S or max_ctx and one allocation serves every call
  // up to these sizes.
  LaunchCfg cfg;
  cfg.part_tokens = 16 * kWaves;
  cfg.nparts_max = max_ctx > 0 ? (max_ctx + cfg.part_tokens - 1) / cfg.part_tokens : 1;
  if (cfg.nparts_max <= 1 && max_ctx > 0) cfg.nparts_max = 2;
  return ws_layout(S, pool->Hkv, Hq / pool->Hkv, cfg).total;
}

pa_status pa_decode_workspace_init(void* workspace, size_t ws_bytes, hipStream_t stream) {
  pa_detail::clear_error();
  if (ws_bytes == 0) return PA_OK;
  if (!workspace || !aligned(workspace, 16)) return fail(PA_ERR_INVALID_ARG, "workspace must be 16-byte aligned");
  const uint64_t n16 = ws_bytes / 16;
  const uint64_t ntail = ws_bytes % 16;
  uint64_t blocks = (n16 + 255) / 256;
  if (blocks < 1) blocks = 1;
  if (blocks > 65535) blocks = 65535;
  hipLaunchKernelGGL(zero_kernel, dim3((unsigned)blocks), dim3(256), 0, stream, static_cast<uint4*>(workspace), n16,
                     static_cast<uint8_t*>(workspace) + n16 * 16, ntail);
  return hip_check(hipGetLastError(), "workspace init launch");
}

pa_status pa_decode_attention(pa_pool* pool, int layer, void* out, const void* q, int S, int Hq,
                              const int32_t* block_tables, int maxb, const int32_t* context_lens, int max_ctx,
                              float scale, void* workspace, size_t ws_bytes, hipStream_t stream) {
  pa_detail::clear_error();
  return decode_launch(pool, layer, out, q, S, Hq, block_tables, maxb, context_lens, max_ctx, scale, workspace,
                       ws_bytes, nullptr, nullptr, nullptr, nullptr, 0, 0, stream);
}

pa_status pa_decode_attention_ordered(pa_pool* pool, int layer, const void* k, const void* v,
                                      const int64_t* slot_mapping, void* out, const void* q, int S, int Hq,
                                      const int32_t* block_tables, int maxb, const int32_t* context_lens,
                                      const int32_t* host_context_lens, int max_ctx, float scale, void* workspace,
                                      size_t ws_bytes, hipStream_t stream) {
  pa_detail::clear_error();
  if (S > 0 && !host_context_lens) return fail(PA_ERR_INVALID_ARG, "NULL host_context_lens");
  const bool fused = k != nullptr || v != nullptr || slot_mapping != nullptr;
  if (S > 0 && fused) {
    if (!k || !v || !slot_mapping) return fail(PA_ERR_INVALID_ARG, "k, v and slot_mapping must all be given or all NULL");
    if (!aligned(k, 16) || !aligned(v, 16) || !aligned(slot_mapping, 8))
      return fail(PA_ERR_INVALID_ARG, "k and v must be 16-byte aligned, slot_mapping 8-byte aligned");
  }
  return decode_launch(pool, layer, out, q, S, Hq, block_tables, maxb, context_lens, max_ctx, scale, workspace,
                       ws_bytes, fused ? k : nullptr, fused ? v : nullptr, fused ? slot_mapping : nullptr, nullptr, 0,
                       0, stream, host_context_lens);
}

pa_status pa_decode_attention_ordered_noalloc(pa_pool* pool, int layer, const void* k, const void* v,
                                              const int64_t* slot_mapping, void* out, const void* q, int S, int Hq,
                                              const int32_t* block_tables, int maxb, const int32_t* context_lens,
                                              const int32_t* host_context_lens, int max_ctx, float scale,
                                              hipStream_t stream) {
  pa_detail::clear_error();
  if (S > 0 && !host_context_lens) return fail(PA_ERR_INVALID_ARG, "NULL host_context_lens");
  const bool fused = k != nullptr || v != nullptr || slot_mapping != nullptr;
  if (S > 0 && fused) {
    if (!k || !v || !slot_mapping) return fail(PA_ERR_INVALID_ARG, "k, v and slot_mapping must all be given or all NULL");
    if (!aligned(k, 16) || !aligned(v, 16) || !aligned(slot_mapping, 8))
      return fail(PA_ERR_INVALID_ARG, "k and v must be 16-byte aligned, slot_mapping 8-byte aligned");
  }
  void* ws = nullptr;
  if (S > 0)
    if (pa_status st = static_scratch_ptr(&ws)) return st;
  return decode_launch(pool, layer, out, q, S, Hq, block_tables, maxb, context_lens, max_ctx, scale, ws,
                       kStaticScratchBytes, fused ? k : nullptr, fused ? v : nullptr, fused ? slot_mapping : nullptr,
                       nullptr, 0, 0, stream, host_context_lens, true);
}

size_t pa_multi_query_workspace_bytes(const pa_pool* pool, int S, int Hq, int max_ctx, int max_q) {
  if (!pool || S <= 0 || Hq <= 0 || max_ctx < 0 || max_q <= 0 || Hq % pool->Hkv) return 0;
  const int G = Hq / pool->Hkv;
  if (G != 1 && G != 2 && G != 4 && G != 8) return 0;
  const MqPlan plan = mq_plan(G, max_q);
  if ((int64_t)plan.ntiles * S > 0x7fffffff) return 0;
  // as pa_decode_workspace_bytes: the shortest partition, so the size never
  // decreases with any argument
  LaunchCfg cfg;
  cfg.part_tokens = 16 * kWaves;
  cfg.nparts_max = max_ctx > 0 ? (max_ctx + cfg.part_tokens - 1) / cfg.part_tokens : 1;
  if (cfg.nparts_max <= 1 && max_ctx > 0) cfg.nparts_max = 2;
  return ws_layout(S * plan.ntiles, pool->Hkv, plan.rows, cfg).total;
}

pa_status pa_multi_query_attention(pa_pool* pool, int layer, void* out, const void* q, const int32_t* q_start, int T,
                                   int S, int Hq, const int32_t* block_tables, int maxb, const int32_t* context_lens,
                                   int max_ctx, int max_q, float scale, void* workspace, size_t ws_bytes,
                                   hipStream_t stream) {
  pa_detail::clear_error();
  if (S > 0 && !q_start) return fail(PA_ERR_INVALID_ARG, "NULL q_start");
  return decode_launch(pool, layer, out, q, S, Hq, block_tables, maxb, context_lens, max_ctx, scale, workspace,
                       ws_bytes, nullptr, nullptr, nullptr, q_start, T, max_q, stream);
}

pa_status pa_multi_query_attention_ordered(pa_pool* pool, int layer, void* out, const void* q,
                                           const int32_t* q_start, int T, int S, int Hq,
                                           const int32_t* block_tables, int maxb, const int32_t* context_lens,
                                           const int32_t* host_context_lens, int max_ctx, int max_q, float scale,
                                           void* workspace, size_t ws_bytes, hipStream_t stream) {
  pa_detail::clear_error();
  if (S > 0 && !q_start) return fail(PA_ERR_INVALID_ARG, "NULL q_start");
  if (S > 0 && !host_context_lens) return fail(PA_ERR_INVALID_ARG, "NULL host_context_lens");
  return decode_launch(pool, layer, out, q, S, Hq, block_tables, maxb, context_lens, max_ctx, scale, workspace,
                       ws_bytes, nullptr, nullptr, nullptr, q_start, T, max_q, stream, host_context_lens);
}

pa_status pa_write_kv_decode_attention(pa_pool* pool, int layer, const void* k, const void* v,
                                       const int64_t* slot_mapping, void* out, const void* q, int S, int Hq,
                                       const int32_t* block_tables, int maxb, const int32_t* context_lens,
                                       int max_ctx, float scale, void* workspace, size_t ws_bytes,
                                       hipStream_t stream) {
  pa_detail::clear_error();
  if (S > 0) {
    if (!k || !v || !slot_mapping) return fail(PA_ERR_INVALID_ARG, "NULL device pointer");
    if (!aligned(k, 16) || !aligned(v, 16) || !aligned(slot_mapping, 8))
      return fail(PA_ERR_INVALID_ARG, "k and v must be 16-byte aligned, slot_mapping 8-byte aligned");
  }
  return decode_launch(pool, layer, out, q, S, Hq, block_tables, maxb, context_lens, max_ctx, scale, workspace,
                       ws_bytes, k, v, slot_mapping, nullptr, 0, 0, stream);
}

pa_status pa_decode_attention_grouped_ordered(pa_pool* pool, int layer, const void* k, const void* v,
                                              const int64_t* slot_mapping, void* out, const void* q, int S, int Hq,
                                              const int32_t* block_tables, int maxb, const int32_t* context_lens,
                                              int max_ctx, const int32_t* group_start, const int32_t* group_len,
                                              const int32_t* seq_group, const int32_t* host_group_len, int n_groups,
                                              int max_group, int max_shared, int max_suffix, float scale,
                                              void* workspace, size_t ws_bytes, hipStream_t stream) {
  pa_detail::clear_error();
  if (n_groups > 0 && !host_group_len) return fail(PA_ERR_INVALID_ARG, "NULL host_group_len");
  return grouped_launch(pool, layer, out, q, S, Hq, block_tables, maxb, context_lens, max_ctx, group_start, group_len,
                        seq_group, n_groups, max_group, max_shared, max_suffix, scale, workspace, ws_bytes, k, v,
                        slot_mapping, stream, host_group_len);
}

size_t pa_decode_grouped_workspace_bytes(const pa_pool* pool, int S, int Hq, int max_ctx, int n_groups,
                                        int max_group, int max_shared, int max_suffix) {
  if (!pool || S <= 0 || Hq <= 0 || max_ctx < 0 || Hq % pool->Hkv || n_groups < 0 || max_group < 0 ||
      max_shared < 0 || max_group > S || max_shared > max_ctx || max_suffix < 0 || max_suffix > max_ctx)
    return 0;
  return grouped_layout(S, pool->Hkv, Hq / pool->Hkv, max_suffix, n_groups, max_group, max_shared, true).total;
}

pa_status pa_decode_attention_grouped(pa_pool* pool, int layer, const void* k, const void* v,
                                      const int64_t* slot_mapping, void* out, const void* q, int S, int Hq,
                                      const int32_t* block_tables, int maxb, const int32_t* context_lens, int max_ctx,
                                      const int32_t* group_start, const int32_t* group_len, const int32_t* seq_group,
                                      int n_groups, int max_group, int max_shared, int max_suffix, float scale,
                                      void* workspace, size_t ws_bytes, hipStream_t stream) {
  pa_detail::clear_error();
  return grouped_launch(pool, layer, out, q, S, Hq, block_tables, maxb, context_lens, max_ctx, group_start, group_len,
                        seq_group, n_groups, max_group, max_shared, max_suffix, scale, workspace, ws_bytes, k, v,
                        slot_mapping, stream);
}

}  // extern "C"
