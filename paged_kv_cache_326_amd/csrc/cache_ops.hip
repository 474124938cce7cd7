// Slot mapping and the KV scatter into the paged pool (gfx950).
//
// Sources: [P1] "大模型推理内存优化从 KV Cache 分页到连续批处理的工程实践",
// section "KV Cache 的内存开销与分页机制" (block table maps logical to
// physical blocks; a new token goes into the current block or a new one).
#include "pa_common.h"
#include "pa_launch.h"

namespace pa {

// One workgroup per sequence; its threads walk that sequence's new tokens.
__global__ void __launch_bounds__(256) slot_mapping_kernel(
    const int32_t* __restrict__ block_tables, int32_t max_blocks, const int32_t* __restrict__ seq_lens,
    const int32_t* __restrict__ cu_q_lens, int32_t block_size, int64_t* __restrict__ slots,
    int32_t num_tokens) {
  const int s = blockIdx.x;
  const int t0 = cu_q_lens[s];
  const int t1 = cu_q_lens[s + 1];
  const int L = seq_lens[s];
  const int q = t1 - t0;
  for (int i = threadIdx.x; i < q; i += blockDim.x) {
    const int t = t0 + i;
    if (t < 0 || t >= num_tokens) continue;
    const int pos = L - q + i;
    int64_t slot = -1;
    if (pos >= 0) {
      const int logical = pos / block_size;
      if (logical < max_blocks) {
        const int64_t phys = block_tables[(int64_t)s * max_blocks + logical];
        slot = phys * block_size + pos % block_size;
      }
    }
    slots[t] = slot;
  }
}

// The scatter works on groups of up to kGroup consecutive entries of the
// token list; one workgroup per group.  A token row of one KV head is
// head_dim elements.  The key tile of (block, KV head) holds block_size rows
// in 64-byte column chunks (row `offset` becomes one 64-byte piece of every
// chunk), the value tile is [head_dim][block_size] (the row becomes column
// `offset`).  Key rows move as 16-byte chunks.  Value rows: when the group's kGroup
// slots are consecutive and the first is a multiple of kGroup (so they lie
// in one block, block_size being a multiple of kGroup; the usual case for a
// prefill chunk), each thread loads one 16-byte chunk (VEC dims) of all
// kGroup tokens, transposes them in registers and writes, for each of its
// dims, the kGroup tokens' values as one contiguous piece of the value-tile
// row; otherwise every element is stored into its column on its own.
constexpr int kGroup = 8;
constexpr int kScatterThreads = 256;

template <typename T>
struct ScatterArgs {
  T* key_cache;
  T* value_cache;
  const typename Src<T>::type* key;
  const typename Src<T>::type* value;
  int32_t num_kv_heads, head_dim, block_size;
  int64_t pool_slots;
  float k_scale, v_scale;
};

// kGroup values of dim e (one per token, token order) -> one piece of a
// value-tile row at p: 16-bit types 16 bytes, float32 32 bytes, FP8 codes
// 8 bytes (quantised like every other FP8 store).
template <typename T>
__device__ __forceinline__ void store_row_piece(T* p, const u32x4 (&d)[kGroup], int e, float scale);
template <>
__device__ __forceinline__ void store_row_piece<float>(float* p, const u32x4 (&d)[kGroup], int e, float) {
  u32x4* q = reinterpret_cast<u32x4*>(p);
  q[0] = u32x4{d[0][e], d[1][e], d[2][e], d[3][e]};
  q[1] = u32x4{d[4][e], d[5][e], d[6][e], d[7][e]};
}
__device__ __forceinline__ void store_row_piece16(uint16_t* p, const u32x4 (&d)[kGroup], int e) {
  const int w = e / 2, sh = 16 * (e % 2);
  u32x4 r;
#pragma unroll
  for (int j = 0; j < 4; ++j) r[j] = ((d[2 * j][w] >> sh) & 0xffffu) | (((d[2 * j + 1][w] >> sh) & 0xffffu) << 16);
  *reinterpret_cast<u32x4*>(p) = r;
}
template <>
__device__ __forceinline__ void store_row_piece<f16_t>(f16_t* p, const u32x4 (&d)[kGroup], int e, float) {
  store_row_piece16(reinterpret_cast<uint16_t*>(p), d, e);
}
template <>
__device__ __forceinline__ void store_row_piece<bf16_t>(bf16_t* p, const u32x4 (&d)[kGroup], int e, float) {
  store_row_piece16(reinterpret_cast<uint16_t*>(p), d, e);
}
template <>
__device__ __forceinline__ void store_row_piece<fp8_t>(fp8_t* p, const u32x4 (&d)[kGroup], int e, float scale) {
  const int w = e / 2;
  uint32_t r[2] = {0u, 0u};
#pragma unroll
  for (int i = 0; i < kGroup; ++i) {
    const float x = e % 2 ? f16_hi(d[i][w]) : f16_lo(d[i][w]);
    r[i / 4] |= f32_to_e4m3(x / scale) << (8 * (i % 4));
  }
  *reinterpret_cast<u32x2*>(p) = u32x2{r[0], r[1]};
}

// Scatter of tokens t0 .. t0+n-1 (n <= kGroup) by one workgroup.  slot_of(i)
// gives token t0+i's slot (or -1 to skip it); it is called once per token,
// by thread i, while the other threads' first K/V loads are in flight.
template <typename T, typename SlotFn>
__device__ __forceinline__ void scatter_group(const ScatterArgs<T>& a, int64_t t0, int n, SlotFn slot_of) {
  using S = typename Src<T>::type;
  constexpr int VEC = vec16<S>();
  __shared__ int64_t s_slot[kGroup];
  const int tid = threadIdx.x;
  const int cpr = a.head_dim / VEC;             // 16-byte chunks per head row
  const int nk = n * a.num_kv_heads * cpr;      // key chunks of the group
  const int nv = a.num_kv_heads * cpr;          // value items: one chunk of every token
  auto src = [&](const S* base, int i, int h, int ch) {
    return *reinterpret_cast<const u32x4*>(base + ((t0 + i) * a.num_kv_heads + h) * a.head_dim + ch * VEC);
  };
  // First loads before the slots are known.
  u32x4 kpre = {0, 0, 0, 0};
  if (tid < nk) kpre = src(a.key, tid / (a.num_kv_heads * cpr), (tid / cpr) % a.num_kv_heads, tid % cpr);
  u32x4 vpre[kGroup];
#pragma unroll
  for (int i = 0; i < kGroup; ++i) vpre[i] = (tid < nv && i < n) ? src(a.value, i, tid / cpr, tid % cpr) : u32x4{0, 0, 0, 0};
  if (tid < n) {
    const int64_t sl = slot_of(tid);
    s_slot[tid] = (sl >= 0 && sl < a.pool_slots) ? sl : -1;
  }
  __syncthreads();
  bool run = n == kGroup && s_slot[0] >= 0 && s_slot[0] % kGroup == 0;
#pragma unroll
  for (int i = 1; i < kGroup; ++i) run = run && s_slot[i] == s_slot[0] + i;

  // Key chunks in batches of kKeyBatch per thread, every load of a batch
  // issued before its stores (a store into the pool could alias a later
  // source row as far as the compiler knows, so loads are not moved across
  // stores).
  constexpr int kKeyBatch = 4;
  for (int base = tid; base < nk; base += kKeyBatch * kScatterThreads) {
    u32x4 x[kKeyBatch];
#pragma unroll
    for (int j = 0; j < kKeyBatch; ++j) {
      const int idx = base + j * kScatterThreads;
      x[j] = idx == tid ? kpre
                        : (idx < nk ? src(a.key, idx / (a.num_kv_heads * cpr), (idx / cpr) % a.num_kv_heads, idx % cpr)
                                    : u32x4{0, 0, 0, 0});
    }
#pragma unroll
    for (int j = 0; j < kKeyBatch; ++j) {
      const int idx = base + j * kScatterThreads;
      if (idx >= nk) break;
      const int i = idx / (a.num_kv_heads * cpr), h = (idx / cpr) % a.num_kv_heads, ch = idx % cpr;
      const int64_t sl = s_slot[i];
      if (sl < 0) continue;
      store_kv_chunk<T>(a.key_cache, a.value_cache, 0, sl / a.block_size, (int)(sl % a.block_size), h, ch, VEC,
                        a.num_kv_heads, a.head_dim, a.block_size, x[j], a.k_scale, a.v_scale);
    }
  }
  for (int it = tid; it < nv; it += kScatterThreads) {
    const int h = it / cpr, ch = it % cpr;
    u32x4 d[kGroup];
#pragma unroll
    for (int i = 0; i < kGroup; ++i) d[i] = it == tid ? vpre[i] : (i < n ? src(a.value, i, h, ch) : u32x4{0, 0, 0, 0});
    if (run) {
      const int64_t blk = s_slot[0] / a.block_size;
      const int off = (int)(s_slot[0] % a.block_size);
      T* row = a.value_cache + ((blk * a.num_kv_heads + h) * a.head_dim + ch * VEC) * a.block_size + off;
#pragma unroll
      for (int e = 0; e < VEC; ++e) store_row_piece<T>(row + (int64_t)e * a.block_size, d, e, a.v_scale);
    } else {
#pragma unroll
      for (int i = 0; i < kGroup; ++i) {
        const int64_t sl = i < n ? s_slot[i] : -1;
        if (sl < 0) continue;
        store_kv_chunk<T>(a.key_cache, a.value_cache, 1, sl / a.block_size, (int)(sl % a.block_size), h, ch, VEC,
                          a.num_kv_heads, a.head_dim, a.block_size, d[i], a.k_scale, a.v_scale);
      }
    }
  }
}

// Scatter by an explicit slot mapping: workgroup x takes tokens
// x*kGroup .. x*kGroup+kGroup-1; slots < 0 (or past the pool) are skipped.
template <typename T>
__global__ void __launch_bounds__(kScatterThreads) reshape_and_cache_kernel(ScatterArgs<T> a,
                                                                           const int64_t* __restrict__ slots,
                                                                           int32_t num_tokens) {
  const int64_t t0 = (int64_t)blockIdx.x * kGroup;
  const int n = num_tokens - t0 < kGroup ? (int)(num_tokens - t0) : kGroup;
  scatter_group<T>(a, t0, n, [&](int i) { return slots[t0 + i]; });
}

// Slot mapping and scatter in one pass.  Workgroup (x, s) covers new tokens
// x*kGroup .. of sequence s: the slot of each comes from the block table
// (and is recorded in slots[]), and its rows are scattered as above.
template <typename T>
__global__ void __launch_bounds__(kScatterThreads) append_kernel(
    ScatterArgs<T> a, const int32_t* __restrict__ block_tables, int32_t max_blocks,
    const int32_t* __restrict__ seq_lens, const int32_t* __restrict__ cu_q_lens, int64_t* __restrict__ slots,
    int32_t num_tokens) {
  const int s = blockIdx.y;
  const int tq = cu_q_lens[s];
  const int q = cu_q_lens[s + 1] - tq;
  const int L = seq_lens[s];
  const int first = blockIdx.x * kGroup;
  // Tokens outside the list are not touched.
  const int64_t t0 = (int64_t)tq + first;
  int64_t n64 = q - first < kGroup ? q - first : kGroup;
  if (n64 > num_tokens - t0) n64 = num_tokens - t0;
  if (n64 <= 0 || t0 < 0) return;
  const int n = (int)n64;
  // The slot is recorded as computed (a block id outside the pool gives a
  // slot past the pool, which the scatter skips).
  scatter_group<T>(a, t0, n, [&](int i) -> int64_t {
    const int pos = L - q + first + i;
    int64_t slot = -1;
    if (pos >= 0 && pos / a.block_size < max_blocks)
      slot = (int64_t)block_tables[(int64_t)s * max_blocks + pos / a.block_size] * a.block_size + pos % a.block_size;
    slots[t0 + i] = slot;
    return slot;
  });
}

template <typename T>
static ScatterArgs<T> scatter_args(const KvCacheArgs& c, const void* key, const void* value) {
  ScatterArgs<T> a;
  a.key_cache = static_cast<T*>(c.key_cache);
  a.value_cache = static_cast<T*>(c.value_cache);
  a.key = static_cast<const typename Src<T>::type*>(key);
  a.value = static_cast<const typename Src<T>::type*>(value);
  a.num_kv_heads = c.num_kv_heads;
  a.head_dim = c.head_dim;
  a.block_size = c.block_size;
  a.pool_slots = (int64_t)c.num_blocks * c.block_size;
  a.k_scale = c.k_scale;
  a.v_scale = c.v_scale;
  return a;
}

template <typename T>
static hipError_t launch_append_t(const KvCacheArgs& c, const void* key, const void* value,
                                  const int32_t* block_tables, int32_t max_blocks, const int32_t* seq_lens,
                                  const int32_t* cu_q_lens, int32_t num_seqs, int32_t max_q_len, int64_t* slots,
                                  int32_t num_tokens, hipStream_t stream) {
  if (num_seqs == 0 || max_q_len == 0) return hipSuccess;
  dim3 grid((max_q_len + kGroup - 1) / kGroup, num_seqs);
  hipLaunchKernelGGL(append_kernel<T>, grid, dim3(kScatterThreads), 0, stream, scatter_args<T>(c, key, value),
                     block_tables, max_blocks, seq_lens, cu_q_lens, slots, num_tokens);
  return hipGetLastError();
}

hipError_t launch_append(const KvCacheArgs& c, const void* key, const void* value, const int32_t* block_tables,
                         int32_t max_blocks, const int32_t* seq_lens, const int32_t* cu_q_lens, int32_t num_seqs,
                         int32_t max_q_len, int64_t* slots, int32_t num_tokens, hipStream_t stream) {
  switch (c.dtype) {
    case DType::kF32:
      return launch_append_t<float>(c, key, value, block_tables, max_blocks, seq_lens, cu_q_lens, num_seqs, max_q_len,
                                    slots, num_tokens, stream);
    case DType::kF16:
      return launch_append_t<f16_t>(c, key, value, block_tables, max_blocks, seq_lens, cu_q_lens, num_seqs, max_q_len,
                                    slots, num_tokens, stream);
    case DType::kBF16:
      return launch_append_t<bf16_t>(c, key, value, block_tables, max_blocks, seq_lens, cu_q_lens, num_seqs,
                                     max_q_len, slots, num_tokens, stream);
    case DType::kFP8:
      return launch_append_t<fp8_t>(c, key, value, block_tables, max_blocks, seq_lens, cu_q_lens, num_seqs,
                                    max_q_len, slots, num_tokens, stream);
  }
  return hipErrorInvalidValue;
}

// Whole-block moves, 16 bytes per thread, K and V alike.  Mode 0: pool block
// src[i] -> pool block dst[i] (copy-on-write); mode 1: pool block ids[i] ->
// row i of a staging buffer; mode 2: row i of a staging buffer -> pool block
// ids[i].  A staging buffer is [n][num_kv_heads][block_size][head_dim] and may
// live in pinned host memory (then the move is a swap over the bus).  Block
// ids outside the pool are skipped.
__global__ void __launch_bounds__(256) block_move_kernel(uint8_t* __restrict__ kc, uint8_t* __restrict__ vc,
                                                         const int32_t* __restrict__ src, const int32_t* __restrict__ dst,
                                                         uint8_t* __restrict__ kbuf, uint8_t* __restrict__ vbuf,
                                                         int32_t n, int64_t block_bytes, int32_t num_blocks, int mode) {
  const int64_t chunks = block_bytes / 16;
  const int64_t gid = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  const int64_t total = (int64_t)n * chunks * 2;
  if (gid >= total) return;
  const int which = (int)(gid / ((int64_t)n * chunks));  // 0 = K, 1 = V
  const int64_t rem = gid - (int64_t)which * n * chunks;
  const int i = (int)(rem / chunks);
  const int64_t c = rem % chunks;
  uint8_t* pool = which ? vc : kc;
  uint8_t* buf = which ? vbuf : kbuf;
  const uint8_t* from;
  uint8_t* to;
  if (mode == 0) {
    const int32_t a = src[i], b = dst[i];
    if (a < 0 || a >= num_blocks || b < 0 || b >= num_blocks || a == b) return;
    from = pool + a * block_bytes;
    to = pool + b * block_bytes;
  } else if (mode == 1) {
    const int32_t a = src[i];
    if (a < 0 || a >= num_blocks) return;
    from = pool + a * block_bytes;
    to = buf + i * block_bytes;
  } else {
    const int32_t b = src[i];
    if (b < 0 || b >= num_blocks) return;
    from = buf + i * block_bytes;
    to = pool + b * block_bytes;
  }
  reinterpret_cast<u32x4*>(to)[c] = reinterpret_cast<const u32x4*>(from)[c];
}

hipError_t launch_block_move(const KvCacheArgs& c, const int32_t* src, const int32_t* dst, void* kbuf, void* vbuf,
                             int32_t n, int mode, hipStream_t stream) {
  if (n == 0) return hipSuccess;
  const int64_t eb = c.dtype == DType::kF32 ? 4 : c.dtype == DType::kFP8 ? 1 : 2;
  const int64_t block_bytes = (int64_t)c.num_kv_heads * c.block_size * c.head_dim * eb;
  const int64_t total = (int64_t)n * (block_bytes / 16) * 2;
  hipLaunchKernelGGL(block_move_kernel, dim3((unsigned)((total + 255) / 256)), dim3(256), 0, stream,
                     (uint8_t*)c.key_cache, (uint8_t*)c.value_cache, src, dst, (uint8_t*)kbuf, (uint8_t*)vbuf, n,
                     block_bytes, c.num_blocks, mode);
  return hipGetLastError();
}

hipError_t launch_slot_mapping(const int32_t* block_tables, int32_t max_blocks, const int32_t* seq_lens,
                               const int32_t* cu_q_lens, int32_t num_seqs, int32_t block_size,
                               int64_t* slots, int32_t num_tokens, hipStream_t stream) {
  if (num_seqs == 0) return hipSuccess;
  hipLaunchKernelGGL(slot_mapping_kernel, dim3(num_seqs), dim3(256), 0, stream, block_tables, max_blocks,
                     seq_lens, cu_q_lens, block_size, slots, num_tokens);
  return hipGetLastError();
}

template <typename T>
static hipError_t launch_rac(const KvCacheArgs& c, const void* key, const void* value, const int64_t* slots,
                             int32_t num_tokens, hipStream_t stream) {
  if (num_tokens <= 0) return hipSuccess;
  const int64_t groups = ((int64_t)num_tokens + kGroup - 1) / kGroup;
  hipLaunchKernelGGL(reshape_and_cache_kernel<T>, dim3((unsigned)groups), dim3(kScatterThreads), 0, stream,
                     scatter_args<T>(c, key, value), slots, num_tokens);
  return hipGetLastError();
}

hipError_t launch_reshape_and_cache(const KvCacheArgs& c, const void* key, const void* value,
                                    const int64_t* slots, int32_t num_tokens, hipStream_t stream) {
  switch (c.dtype) {
    case DType::kF32:
      return launch_rac<float>(c, key, value, slots, num_tokens, stream);
    case DType::kF16:
      return launch_rac<f16_t>(c, key, value, slots, num_tokens, stream);
    case DType::kBF16:
      return launch_rac<bf16_t>(c, key, value, slots, num_tokens, stream);
    case DType::kFP8:
      return launch_rac<fp8_t>(c, key, value, slots, num_tokens, stream);
  }
  return hipErrorInvalidValue;
}

}  // namespace pa
