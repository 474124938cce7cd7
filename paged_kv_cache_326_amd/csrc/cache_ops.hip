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

// Each thread moves one 16-byte chunk of one token's K or V row.  A token row
// of one KV head is head_dim elements.  The key tile of (block, KV head) is
// [block_size][head_dim] (the row lands at
//   ((block * num_kv_heads + head) * block_size + offset) * head_dim),
// the value tile [head_dim][block_size] (the row becomes column `offset`).
template <typename T>
__global__ void __launch_bounds__(256) reshape_and_cache_kernel(
    T* __restrict__ key_cache, T* __restrict__ value_cache, const typename Src<T>::type* __restrict__ key,
    const typename Src<T>::type* __restrict__ value, const int64_t* __restrict__ slots, int32_t num_tokens,
    int32_t num_kv_heads, int32_t head_dim, int32_t block_size, int64_t pool_slots, float k_scale, float v_scale) {
  using S = typename Src<T>::type;
  constexpr int VEC = vec16<S>();
  const int chunks_per_row = head_dim / VEC;          // 16-byte chunks per head row
  const int chunks_per_tok = num_kv_heads * chunks_per_row;
  const int64_t gid = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  const int64_t total = (int64_t)num_tokens * chunks_per_tok * 2;
  if (gid >= total) return;
  const int which = (int)(gid / ((int64_t)num_tokens * chunks_per_tok));  // 0 = K, 1 = V
  const int64_t rem = gid - (int64_t)which * num_tokens * chunks_per_tok;
  const int t = (int)(rem / chunks_per_tok);
  const int c = (int)(rem % chunks_per_tok);
  const int64_t slot = slots[t];
  if (slot < 0 || slot >= pool_slots) return;
  const int h = c / chunks_per_row;
  const int ch = c % chunks_per_row;
  const int64_t blk = slot / block_size;
  const int off = (int)(slot % block_size);
  const S* src = (which ? value : key) + ((int64_t)t * num_kv_heads + h) * head_dim + ch * VEC;
  store_kv_chunk<T>(key_cache, value_cache, which, blk, off, h, ch, VEC, num_kv_heads, head_dim, block_size,
                    *reinterpret_cast<const u32x4*>(src), k_scale, v_scale);
}

// Slot mapping and scatter in one pass.  Workgroup (x, s) covers new tokens
// x*kAppendTok .. of sequence s; thread (token, chunk) fetches its 16-byte
// K or V chunk (independent of the slot, so the load overlaps the table
// lookup), computes the slot and stores.  The chunk-0 thread of each token
// also records the slot.
constexpr int kAppendTok = 8;

template <typename T>
__global__ void __launch_bounds__(256) append_kernel(
    T* __restrict__ key_cache, T* __restrict__ value_cache, const typename Src<T>::type* __restrict__ key,
    const typename Src<T>::type* __restrict__ value, const int32_t* __restrict__ block_tables, int32_t max_blocks,
    const int32_t* __restrict__ seq_lens, const int32_t* __restrict__ cu_q_lens, int64_t* __restrict__ slots,
    int32_t num_tokens, int32_t num_kv_heads, int32_t head_dim, int32_t block_size, int32_t num_blocks,
    float k_scale, float v_scale) {
  using S = typename Src<T>::type;
  constexpr int VEC = vec16<S>();
  const int s = blockIdx.y;
  const int t0 = cu_q_lens[s];
  const int q = cu_q_lens[s + 1] - t0;
  const int L = seq_lens[s];
  const int chunks_per_row = head_dim / VEC;
  const int chunks_per_tok = num_kv_heads * chunks_per_row * 2;  // K and V
  const int first = blockIdx.x * kAppendTok;
  for (int idx = threadIdx.x; idx < kAppendTok * chunks_per_tok; idx += blockDim.x) {
    const int i = first + idx / chunks_per_tok;
    if (i >= q) break;
    const int t = t0 + i;
    if (t < 0 || t >= num_tokens) continue;
    const int c = idx % chunks_per_tok;
    const int which = c / (num_kv_heads * chunks_per_row);
    const int h = (c / chunks_per_row) % num_kv_heads;
    const int ch = c % chunks_per_row;
    const S* src = (which ? value : key) + ((int64_t)t * num_kv_heads + h) * head_dim + ch * VEC;
    const u32x4 data = *reinterpret_cast<const u32x4*>(src);
    const int pos = L - q + i;
    int64_t slot = -1, phys = -1;
    if (pos >= 0 && pos / block_size < max_blocks) {
      phys = block_tables[(int64_t)s * max_blocks + pos / block_size];
      slot = phys * block_size + pos % block_size;
    }
    if (c == 0) slots[t] = slot;
    if (slot < 0 || phys >= num_blocks) continue;
    const int64_t blk = slot / block_size;
    const int off = (int)(slot % block_size);
    store_kv_chunk<T>(key_cache, value_cache, which, blk, off, h, ch, VEC, num_kv_heads, head_dim, block_size, data,
                      k_scale, v_scale);
  }
}

template <typename T>
static hipError_t launch_append_t(const KvCacheArgs& c, const void* key, const void* value,
                                  const int32_t* block_tables, int32_t max_blocks, const int32_t* seq_lens,
                                  const int32_t* cu_q_lens, int32_t num_seqs, int32_t max_q_len, int64_t* slots,
                                  int32_t num_tokens, hipStream_t stream) {
  if (num_seqs == 0 || max_q_len == 0) return hipSuccess;
  dim3 grid((max_q_len + kAppendTok - 1) / kAppendTok, num_seqs);
  using S = typename Src<T>::type;
  hipLaunchKernelGGL(append_kernel<T>, grid, dim3(256), 0, stream, (T*)c.key_cache, (T*)c.value_cache, (const S*)key,
                     (const S*)value, block_tables, max_blocks, seq_lens, cu_q_lens, slots, num_tokens, c.num_kv_heads,
                     c.head_dim, c.block_size, c.num_blocks, c.k_scale, c.v_scale);
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
  using S = typename Src<T>::type;
  constexpr int VEC = vec16<S>();
  const int64_t total = (int64_t)num_tokens * c.num_kv_heads * (c.head_dim / VEC) * 2;
  if (total == 0) return hipSuccess;
  const int64_t blocks = (total + 255) / 256;
  hipLaunchKernelGGL(reshape_and_cache_kernel<T>, dim3((unsigned)blocks), dim3(256), 0, stream,
                     (T*)c.key_cache, (T*)c.value_cache, (const S*)key, (const S*)value, slots, num_tokens,
                     c.num_kv_heads, c.head_dim, c.block_size, (int64_t)c.num_blocks * c.block_size, c.k_scale,
                     c.v_scale);
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
