// Internal launcher interface between the C ABI (api.hip) and the kernels.
// Arguments reaching these functions have already been validated.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace pa {

enum class DType : int { kF32 = 0, kF16 = 1, kBF16 = 2, kFP8 = 3 };

struct KvCacheArgs {
  void* key_cache;
  void* value_cache;
  int32_t num_blocks, num_kv_heads, head_dim, block_size;
  DType dtype;
  float k_scale, v_scale;  // FP8 pools: code c stands for value(c) * scale
};

struct DecodeArgs {
  KvCacheArgs cache;
  void* out;
  const void* query;
  const int32_t* block_tables;
  int32_t max_blocks;
  const int32_t* seq_lens;
  int32_t num_seqs, num_heads, max_seq_len;
  float scale;
  int32_t partition;      // tokens per partition, multiple of block_size
  int32_t num_partitions; // ceil(max_seq_len / partition)
  int32_t waves;          // wavefronts per partition workgroup: 4 or 8
  hipEvent_t t0, t1;      // optional: the partition kernel's own start / end
  // Optional fused append: token seq_lens[s]-1 of every sequence, rows
  // [num_seqs][num_kv_heads][head_dim] (float16 for an FP8 pool), is written
  // into its pool slot first; slots[s] receives the slot or -1.
  const void* new_key;
  const void* new_value;
  int64_t* slots;
  // Optional plan: work[i] = sequence * num_partitions + partition for the
  // num_work launched units (else the grid covers every partition).
  const int32_t* work;
  int32_t num_work;
  // Without a plan, for batches of at most kDevicePlanSeqs sequences: each
  // workgroup reads every length and takes the unit of its rank in the
  // longest-first order itself (see decode.hip); the merge then reads only
  // the partitions a sequence has.
  int32_t device_plan;
  float* ws_m;            // [num_seqs][num_heads][num_partitions]
  float* ws_l;            // same
  float* ws_o;            // [num_seqs][num_heads][num_partitions][head_dim]
};

struct PrefillArgs {
  KvCacheArgs cache;
  void* out;
  const void* query;
  const int32_t* cu_q_lens;
  const int32_t* seq_lens;
  const int32_t* block_tables;
  int32_t max_blocks;
  int32_t num_seqs, num_heads;
  int32_t num_qtiles;  // query tiles per (sequence, KV head)
  float scale;
};

constexpr int kMaxPartition = 4096;
constexpr int kDevicePlanSeqs = 64;  // one length per lane of a wave

hipError_t launch_slot_mapping(const int32_t* block_tables, int32_t max_blocks, const int32_t* seq_lens,
                               const int32_t* cu_q_lens, int32_t num_seqs, int32_t block_size,
                               int64_t* slots, int32_t num_tokens, hipStream_t stream);

hipError_t launch_reshape_and_cache(const KvCacheArgs& c, const void* key, const void* value,
                                    const int64_t* slots, int32_t num_tokens, hipStream_t stream);

hipError_t launch_append(const KvCacheArgs& c, const void* key, const void* value, const int32_t* block_tables,
                         int32_t max_blocks, const int32_t* seq_lens, const int32_t* cu_q_lens, int32_t num_seqs,
                         int32_t max_q_len, int64_t* slots, int32_t num_tokens, hipStream_t stream);

// mode 0: pool -> pool (src[i] -> dst[i]); 1: pool src[i] -> buffer row i;
// 2: buffer row i -> pool src[i].
hipError_t launch_block_move(const KvCacheArgs& c, const int32_t* src, const int32_t* dst, void* kbuf, void* vbuf,
                             int32_t n, int mode, hipStream_t stream);

// stage 1: partition kernel; 2: merge of the partials; 0: both.
hipError_t launch_decode(const DecodeArgs& a, int stage, hipStream_t stream);

// A plain streaming read of `bytes` (a multiple of 16) by `workgroups`
// workgroups of `threads` threads; sink[w] receives workgroup w's XOR.
hipError_t launch_stream_read(const void* src, int64_t bytes, int workgroups, int threads, uint32_t* sink,
                              hipStream_t stream);

// Query positions one prefill workgroup covers for a head group of `group`
// (the same for every pool dtype).
int prefill_positions_per_tile(int group);
hipError_t launch_prefill(const PrefillArgs& a, hipStream_t stream);
// The FP8-pool kernel (prefill_fp8.hip); launch_prefill dispatches to it.
hipError_t launch_prefill_fp8(const PrefillArgs& a, hipStream_t stream);

}  // namespace pa
