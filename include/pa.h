/*
 * pa.h -- C ABI of libpa.so: paged KV-cache attention for AMD Instinct MI355X
 * (gfx950).
 *
 * Sources (web pages on paged KV caches):
 *   [P1] "大模型推理内存优化从 KV Cache 分页到连续批处理的工程实践"
 *        (seekfood.cn/news/1660747)
 *   [P2] "KV Cache管理优化：大模型推理显存瓶颈突破"
 *        (intelliparadigm.com/article/weixin_33178839/2255646)
 *
 * Memory model.  Every pointer argument except `cache` (a host struct) is a
 * DEVICE pointer owned by the caller; the library never allocates, frees or
 * synchronises.  Arrays are dense and row-major.  Work is enqueued on
 * `stream` (0 = the legacy default stream) and runs asynchronously: the
 * caller synchronises before reading results.
 *
 * KV pool ([P1] "KV Cache 的内存开销与分页机制", fixed-size physical blocks;
 * [P2] section 2.1, one pool preallocated up front).  One layer's pool is two
 * arrays
 *     key_cache   : [num_blocks][num_kv_heads][head_dim / kc][block_size][kc]
 *     value_cache : [num_blocks][num_kv_heads][head_dim][block_size]
 * (kc = 64 bytes of elements: 16 float32, 32 float16 / bfloat16, 64 FP8
 * codes) so that the block_size token vectors of one (block, KV head) are
 * one contiguous tile ([P1] "PagedAttention 的 CUDA Kernel 实现": vectors of
 * a block sit together so that reads coalesce); inside a tile the key rows
 * are cut into 64-byte column chunks and the value tile is transposed (see
 * pa_kv_cache).  A slot numbers token positions in the pool:
 * slot = physical_block * block_size + offset.
 *
 * Block tables ([P1] "KV Cache 的内存开销与分页机制": one table per request,
 * logical block -> physical block) are int32 [num_seqs][max_blocks_per_seq];
 * only the first ceil(seq_len / block_size) entries of a row are read.
 *
 * seq_lens counts the tokens a sequence holds in the pool INCLUDING the
 * tokens written this step (so a decode token attends to itself).
 *
 * Errors.  Argument checks run on the host before anything is enqueued; on
 * failure nothing is launched and outputs are untouched.  A failed launch
 * returns PA_ERR_LAUNCH.  Device-resident contents (block IDs, seq_lens,
 * slots) are the caller's contract; kernels nonetheless skip block IDs
 * outside [0, num_blocks), slots outside the pool, and clamp seq_lens to the
 * host-side bounds, so a bad table gives a wrong result, never an
 * out-of-bounds access.  (The Python binding's PA_DEBUG=1 mode copies those
 * contents to the host and rejects bad ones before each call.)
 *
 * Supported: head_dim in {64, 128}; block_size in {16, 32};
 * num_heads / num_kv_heads in {1, 2, 4, 8}; dtype f32, f16, bf16
 * (prefill: f16, bf16, FP8).
 *
 * Thread safety: no global mutable state; calls on different streams may run
 * concurrently as long as their output buffers do not overlap.
 */
#ifndef PA_H_
#define PA_H_

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Storage dtype of a pool.  PA_FP8_E4M3 stores OCP E4M3 codes (1 sign, 4
 * exponent bits with bias 7, 3 mantissa bits; no infinities; largest finite
 * 448) under one float32 scale per pool: [P1] "工程边界与架构取舍" names
 * FP8 KV quantisation as the conservative way to halve KV memory.  Its
 * queries, outputs and new K/V rows are float16. */
typedef enum {
  PA_F32 = 0,
  PA_F16 = 1,
  PA_BF16 = 2,
  PA_FP8_E4M3 = 3,
} pa_dtype;

typedef enum {
  PA_OK = 0,
  PA_ERR_NULL = 1,        /* a required pointer is NULL */
  PA_ERR_SHAPE = 2,       /* inconsistent sizes (e.g. num_heads % num_kv_heads != 0) */
  PA_ERR_UNSUPPORTED = 3, /* head_dim / block_size / dtype / group size not built */
  PA_ERR_WORKSPACE = 4,   /* workspace missing or smaller than pa_decode_workspace_bytes() */
  PA_ERR_LAUNCH = 5,      /* the HIP runtime rejected a kernel launch */
  PA_ERR_NO_BLOCKS = 6,   /* block manager: the pool cannot supply the blocks (caller preempts) */
  PA_ERR_NOT_FOUND = 7,   /* block manager: unknown sequence id */
  PA_ERR_EXISTS = 8,      /* block manager: sequence id already in use */
} pa_status;

/* One layer's paged KV pool.  Both arrays are device memory owned by the
 * caller, in `dtype`: key_cache [num_blocks][num_kv_heads][head_dim / kc]
 * [block_size][kc] with kc = 64 / (bytes per element), and value_cache
 * [num_blocks][num_kv_heads][head_dim][block_size].  Every (block, KV head)
 * tile is contiguous ([P1] "PagedAttention 的 CUDA Kernel 实现": a block's
 * vectors are adjacent so its reads coalesce).  Inside a key tile, key
 * element (offset t, dim d) sits at (d / kc) * block_size * kc + t * kc +
 * d % kc: the rows are cut into 64-byte column chunks, so a matrix-core
 * operand (64 bytes of each of 16 rows) is whole 128-byte lines.  Value
 * tiles are stored transposed so that the tokens of one dimension are
 * adjacent, which makes the PV product's operand a contiguous load.
 * k_scale and v_scale are read only for PA_FP8_E4M3 (must then be positive
 * and finite, else PA_ERR_SHAPE): a key code c stands for value(c) * k_scale,
 * a value code for value(c) * v_scale.  New rows are quantised as
 * round-to-nearest-even(x / scale) in float32, saturating at +-448. */
typedef struct {
  void* key_cache;
  void* value_cache;
  int32_t num_blocks;
  int32_t num_kv_heads;
  int32_t head_dim;
  int32_t block_size;
  pa_dtype dtype;
  float k_scale;
  float v_scale;
} pa_kv_cache;

/* Slot of every new token.  [P1] "KV Cache 的内存开销与分页机制": a token at
 * position pos of sequence s lives in logical block pos / block_size at offset
 * pos % block_size; a step's new tokens go into the current (or a freshly
 * appended) block of the table.
 *
 * block_tables  int32 [num_seqs][max_blocks_per_seq]
 * seq_lens      int32 [num_seqs], tokens after this step
 * cu_q_lens     int32 [num_seqs + 1], prefix sums of new-token counts
 *               (sequence s writes positions seq_lens[s] - q_s .. seq_lens[s] - 1)
 * slot_mapping  int64 [num_tokens] out, num_tokens = cu_q_lens[num_seqs];
 *               slot = block_tables[s][pos / block_size] * block_size
 *                      + pos % block_size, or -1 when pos is negative or its
 *               logical block is beyond max_blocks_per_seq.
 */
pa_status pa_slot_mapping(const int32_t* block_tables, int32_t max_blocks_per_seq,
                          const int32_t* seq_lens, const int32_t* cu_q_lens,
                          int32_t num_seqs, int32_t block_size,
                          int64_t* slot_mapping, int32_t num_tokens,
                          hipStream_t stream);

/* Scatter new tokens' K and V into their pool slots (bit-exact copy; a
 * token's value row becomes column `offset` of its block's value tile).
 * [P1] "KV Cache 的内存开销与分页机制": the new token's vectors are stored in
 * the current block, or in a block appended to the table when it is full.
 *
 * key, value    [num_tokens][num_kv_heads][head_dim], cache->dtype (float16
 *               for an FP8 pool, which stores the quantised codes)
 * slot_mapping  int64 [num_tokens]; a negative slot marks a padding token and
 *               is skipped.  Two tokens must not share a slot.
 */
pa_status pa_reshape_and_cache(const pa_kv_cache* cache, const void* key, const void* value,
                               const int64_t* slot_mapping, int32_t num_tokens,
                               hipStream_t stream);

/* pa_slot_mapping and pa_reshape_and_cache in one launch: computes every new
 * token's slot from the block table (same definition and -1 rule as
 * pa_slot_mapping), stores it to slot_mapping, and copies the token's K and V
 * there; tokens whose slot is -1 or whose physical block lies outside the
 * pool are not written.  Arguments as in the two calls; max_q_len is a
 * host-side upper bound of the per-sequence new-token counts and num_tokens
 * = cu_q_lens[num_seqs].
 */
pa_status pa_append_kv(const pa_kv_cache* cache, const void* key, const void* value,
                       const int32_t* block_tables, int32_t max_blocks_per_seq,
                       const int32_t* seq_lens, const int32_t* cu_q_lens, int32_t num_seqs,
                       int32_t max_q_len, int64_t* slot_mapping, int32_t num_tokens,
                       hipStream_t stream);

/* Partition length (tokens) that pa_decode picks when partition_size is 0:
 * with at most 256 (sequence, KV head) pairs, each sequence is cut into the
 * equal parts that give about one workgroup per compute unit (one part when
 * the pairs alone fill the chip); with more pairs, 1024 tokens, halved while
 * that leaves fewer than two workgroups per compute unit.  At most 4096. */
int32_t pa_decode_auto_partition(int32_t num_seqs, int32_t num_kv_heads, int32_t max_seq_len,
                                 int32_t block_size);

/* Bytes of float32 scratch pa_decode needs to keep per-partition softmax
 * statistics and partial outputs of sequences longer than one partition.
 * partition_size 0 means the automatic choice (pass the same value to the
 * decode call).  Returns 0 on invalid arguments. */
size_t pa_decode_workspace_bytes(int32_t num_seqs, int32_t num_heads, int32_t num_kv_heads,
                                 int32_t head_dim, int32_t block_size, int32_t max_seq_len,
                                 int32_t partition_size);

/* Decode attention over the paged cache: one query token per sequence.
 * [P1] "PagedAttention 的 CUDA Kernel 实现": for each logical block, look up
 * the physical block in the table and read its K/V vectors; [P1]
 * "工程边界与架构取舍": decode reads the whole cache of a sequence for one
 * token.  Computes, for every query head h of KV group g = h / (num_heads /
 * num_kv_heads),
 *     out[s][h] = softmax_t(scale * q[s][h] . K[s][t][g]) . V[s][t][g],
 * t over 0 .. seq_lens[s]-1; a sequence of length 0 yields zeros.
 *
 * out, query    [num_seqs][num_heads][head_dim], cache->dtype, float16 for
 *               an FP8 pool (out is rounded from float32 to nearest-even).
 *               An FP8 pool's codes are widened exactly to float16 in
 *               registers and its scales applied to the float32 logits and
 *               outputs.
 * max_seq_len   host-side upper bound of seq_lens (<= max_blocks_per_seq *
 *               block_size); longer device values are clamped to it
 * workspace     device scratch of at least pa_decode_workspace_bytes(); may
 *               be NULL when that size is 0.  Overwritten; must not overlap
 *               out, query or the cache.
 */
pa_status pa_decode(const pa_kv_cache* cache, void* out, const void* query,
                    const int32_t* block_tables, int32_t max_blocks_per_seq,
                    const int32_t* seq_lens, int32_t num_seqs, int32_t num_heads,
                    int32_t max_seq_len, float scale, void* workspace,
                    size_t workspace_bytes, hipStream_t stream);

/* pa_decode with an explicit partition length in tokens: a positive multiple
 * of block_size no larger than 4096 (0 = automatic). */
pa_status pa_decode_ex(const pa_kv_cache* cache, void* out, const void* query,
                       const int32_t* block_tables, int32_t max_blocks_per_seq,
                       const int32_t* seq_lens, int32_t num_seqs, int32_t num_heads,
                       int32_t max_seq_len, float scale, void* workspace,
                       size_t workspace_bytes, int32_t partition_size, hipStream_t stream);

/* The two launches of pa_decode_ex, for callers that time or interleave
 * them.  stage 1: the partition kernel (writes the output of every sequence
 * that fits one partition and the partials of the others to the workspace);
 * stage 2: the merge of those partials (launches nothing when max_seq_len
 * fits one partition).  Arguments as for pa_decode_ex, identical for both
 * stages; stage 2 must follow stage 1 on the same stream.  Any other stage
 * value returns PA_ERR_SHAPE. */
pa_status pa_decode_stage(const pa_kv_cache* cache, void* out, const void* query,
                          const int32_t* block_tables, int32_t max_blocks_per_seq,
                          const int32_t* seq_lens, int32_t num_seqs, int32_t num_heads,
                          int32_t max_seq_len, float scale, void* workspace,
                          size_t workspace_bytes, int32_t partition_size, int32_t stage,
                          hipStream_t stream);

/* pa_decode_ex with the partition kernel's own start and end recorded into
 * two caller-created HIP events (hipExtLaunchKernel): the duration of the
 * dominant launch, measured without a marker packet between the partition
 * and merge launches.  Either event may be NULL. */
pa_status pa_decode_timed(const pa_kv_cache* cache, void* out, const void* query,
                          const int32_t* block_tables, int32_t max_blocks_per_seq,
                          const int32_t* seq_lens, int32_t num_seqs, int32_t num_heads,
                          int32_t max_seq_len, float scale, void* workspace,
                          size_t workspace_bytes, int32_t partition_size, hipEvent_t kernel_start,
                          hipEvent_t kernel_stop, hipStream_t stream);

/* One decode step in one call: every sequence's new token (position
 * seq_lens[s] - 1, rows new_key / new_value [num_seqs][num_kv_heads]
 * [head_dim] in the cache dtype, float16 for an FP8 pool) is written into
 * its pool slot exactly as pa_append_kv writes a one-token step (the slot,
 * or -1 when its block is missing from the table or the pool, goes to
 * slot_mapping [num_seqs], int64), then decode attention runs as in
 * pa_decode_timed.  The write is done by the partition workgroup that owns
 * that position, so no separate scatter launch is needed.  seq_lens are
 * clamped to max_seq_len for both parts.  Events may be NULL. */
pa_status pa_decode_append(const pa_kv_cache* cache, const void* new_key, const void* new_value,
                           int64_t* slot_mapping, void* out, const void* query,
                           const int32_t* block_tables, int32_t max_blocks_per_seq,
                           const int32_t* seq_lens, int32_t num_seqs, int32_t num_heads,
                           int32_t max_seq_len, float scale, void* workspace,
                           size_t workspace_bytes, int32_t partition_size, hipEvent_t kernel_start,
                           hipEvent_t kernel_stop, hipStream_t stream);

/* All decode options in one call.  Fields as in pa_decode_ex; the optional
 * ones are NULL / 0 when unused:
 *   stage            0 both launches, 1 the partition kernel, 2 the merge
 *   new_key, new_value, slot_mapping   the fused append of pa_decode_append
 *                    (all three or none)
 *   work, num_work   a plan from pa_decode_plan for the same seq_lens,
 *                    max_seq_len and partition_size (uploaded to device
 *                    memory): only the listed partitions are launched, in
 *                    that order, and the merge reads only the partitions
 *                    each sequence has.  Without a plan the grid covers
 *                    ceil(max_seq_len / partition) partitions of every
 *                    sequence and empty ones exit at once.
 *   kernel_start, kernel_stop   events that the partition kernel records
 *                    its own start and end into
 */
typedef struct {
  const pa_kv_cache* cache;
  void* out;
  const void* query;
  const int32_t* block_tables;
  int32_t max_blocks_per_seq;
  const int32_t* seq_lens;
  int32_t num_seqs;
  int32_t num_heads;
  int32_t max_seq_len;
  float scale;
  void* workspace;
  size_t workspace_bytes;
  int32_t partition_size;
  int32_t stage;
  const void* new_key;
  const void* new_value;
  int64_t* slot_mapping;
  const int32_t* work;
  int32_t num_work;
  hipEvent_t kernel_start;
  hipEvent_t kernel_stop;
} pa_decode_args;

pa_status pa_decode_run(const pa_decode_args* args, hipStream_t stream);

/* pa_decode_ex for callers that cannot allocate device memory (code under
 * HIP graph capture, tight serving loops, harnesses that forbid hipMalloc):
 * no workspace argument.  The per-partition partials live in a fixed
 * library-owned scratch array of PA_NOALLOC_SCRATCH_BYTES in each GPU's
 * memory (held until the process ends); the call allocates nothing.  A
 * batch whose partials need more than that (pa_decode_workspace_bytes with
 * the same arguments) is refused with PA_ERR_WORKSPACE before any launch.
 * Every call on one GPU shares that GPU's scratch, so calls that overlap in
 * time on one GPU (different streams, or other threads) race and must be
 * serialised by the caller; calls on one stream are ordered.  The scratch
 * needs no clearing: every partition writes its partials (or an absent
 * marker) before the merge reads them. */
#define PA_NOALLOC_SCRATCH_BYTES (16u << 20)
pa_status pa_decode_noalloc(const pa_kv_cache* cache, void* out, const void* query,
                            const int32_t* block_tables, int32_t max_blocks_per_seq,
                            const int32_t* seq_lens, int32_t num_seqs, int32_t num_heads,
                            int32_t max_seq_len, float scale, int32_t partition_size,
                            hipStream_t stream);

/* Host-side work list for decode batches of mixed lengths (no device
 * memory; the caller's scheduler knows the lengths).  Lists, for the host
 * copy of seq_lens (clamped to [0, max_seq_len]), every partition that
 * holds a token (and partition 0 of empty sequences, which writes their
 * zeros), longest first -- full partitions in sequence order, then the
 * last partial ones by decreasing length -- each as
 * sequence * ceil(max_seq_len / partition_size) + partition.  Writes the
 * list only if capacity suffices; returns its length, or -1 on bad
 * arguments.  partition_size must be the one the decode call uses (e.g.
 * pa_decode_auto_partition's). */
int32_t pa_decode_plan(const int32_t* seq_lens_host, int32_t num_seqs, int32_t max_seq_len,
                       int32_t partition_size, int32_t* work, int32_t capacity);

/* Chunked-prefill attention over the paged cache (causal).  [P1]
 * "工程边界与架构取舍": prefill is a compute-bound matrix product and a long
 * prompt is processed in chunks interleaved with decode steps; the chunk
 * reads the cached prefix through the block table like decode does.
 *
 * Sequence s has q_s = cu_q_lens[s+1] - cu_q_lens[s] chunk tokens, already
 * written to the pool (pa_reshape_and_cache), at positions ctx .. ctx+q_s-1
 * with ctx = seq_lens[s] - q_s.  Chunk token i, head h attends to positions
 * 0 .. ctx+i of KV head h / (num_heads / num_kv_heads):
 *     out[t][h] = softmax_j(scale * q[t][h] . K[s][j]) . V[s][j],  j <= ctx+i.
 *
 * out, query   [cu_q_lens[num_seqs]][num_heads][head_dim], cache->dtype
 *              for f16 and bf16 pools, float16 for an FP8 pool (whose codes
 *              are converted exactly to f16 on chip and whose scales apply
 *              as in pa_decode); rounded to nearest-even; float32 pools
 *              return PA_ERR_UNSUPPORTED
 * cu_q_lens    int32 [num_seqs + 1]
 * seq_lens     int32 [num_seqs], >= the sequence's chunk length
 * max_q_len    host-side upper bound of the chunk lengths
 * Products run on v_mfma_f32_32x32x16 with fp32 accumulation; the softmax
 * probabilities enter the PV product rounded to the operand dtype (f16 for
 * an FP8 pool; bf16 as a head and remainder pair).
 */
pa_status pa_prefill_chunk(const pa_kv_cache* cache, void* out, const void* query,
                           const int32_t* cu_q_lens, const int32_t* seq_lens,
                           const int32_t* block_tables, int32_t max_blocks_per_seq,
                           int32_t num_seqs, int32_t num_heads, int32_t max_q_len, float scale,
                           hipStream_t stream);

/* Whole-block moves (K and V, all KV heads of a block; bit-exact copies).
 * [P1] "KV Cache 的内存开销与分页机制": sequences may share a prefix's
 * physical blocks; a sequence that must write into a shared, partly filled
 * block first gets a private copy (pa_bm_append_tokens reports the pair).
 * [P2] section 3.2: blocks can be moved out of HBM and back.
 *
 * pa_copy_blocks     pool block src[i] -> pool block dst[i], i < num_pairs
 *                    (src, dst: device int32 arrays; dst must not repeat and
 *                    must not be any src of the same call)
 * pa_gather_blocks   pool block block_ids[i] -> row i of key_out/value_out
 * pa_scatter_blocks  row i of key_in/value_in -> pool block block_ids[i]
 * Buffers are laid out like the pool's blocks (key: [n][num_kv_heads]
 * [head_dim / kc][block_size][kc], value: [n][num_kv_heads][head_dim]
 * [block_size]) in
 * the cache dtype, device memory or pinned host memory (hipHostMalloc), so a gather or
 * scatter through a pinned buffer swaps blocks out of or into HBM; other
 * host memory is refused with PA_ERR_UNSUPPORTED.  Ids outside
 * [0, cache->num_blocks) are skipped.
 */
pa_status pa_copy_blocks(const pa_kv_cache* cache, const int32_t* src, const int32_t* dst,
                         int32_t num_pairs, hipStream_t stream);
pa_status pa_gather_blocks(const pa_kv_cache* cache, const int32_t* block_ids, int32_t num_blocks,
                           void* key_out, void* value_out, hipStream_t stream);
pa_status pa_scatter_blocks(const pa_kv_cache* cache, const int32_t* block_ids, int32_t num_blocks,
                            const void* key_in, const void* value_in, hipStream_t stream);

/* Host-side block manager (no device memory, thread-safe per manager).
 * [P1] "生产级推理引擎的内存管理与调度": a FIFO pool of physical block ids,
 * taken from the front and returned to the back; a sequence of n tokens owns
 * ceil(n / block_size) blocks; when the pool cannot supply them the call
 * fails with PA_ERR_NO_BLOCKS and changes nothing (the caller preempts).
 * [P2] section 4.1: blocks shared by several sequences carry a reference
 * count and return to the pool when the last reference is released.
 *
 * pa_bm_create          free_order: optional permutation of 0..num_blocks-1
 *                       giving the initial free-list order (NULL = ascending);
 *                       returns NULL on bad arguments
 * pa_bm_add_sequence    new sequence holding num_tokens tokens
 * pa_bm_fork            child shares all of parent's blocks (refcount + 1)
 * pa_bm_append_tokens   grow by num_new tokens, taking blocks as needed; if
 *                       the partly filled last block is shared it is replaced
 *                       by a fresh block first and (old, new) is written to
 *                       copy_src[0], copy_dst[0], *num_copies = 1 (else 0):
 *                       copy it with pa_copy_blocks before scattering
 * pa_bm_free_sequence   release every block reference of the sequence
 * pa_bm_block_table     copies up to capacity entries; returns the table
 *                       length (blocks), -1 if unknown
 * pa_bm_free_list       copies up to capacity free ids in pool order;
 *                       returns the number of free blocks
 *
 * Prefix cache.  [P1] "工程边界与架构取舍": requests sharing a system prompt
 * reuse the prefix's physical blocks; cached prefixes are marked by hash and
 * carry a version, and a hash collision must not produce a wrong hit.
 * A full block is cached once pa_bm_commit reports its K/V written; its key
 * is (version, the exact token prefix it ends).  Lookups go through a
 * chained 64-bit hash (parent hash, version, the block's token ids) and
 * accept a candidate only if version, parent block and token ids match.
 * Every cached block's parent is cached; a cached block whose references
 * are all released stays cached in the free list until a fresh allocation
 * pops it, which uncaches it and every cached block extending it.
 *
 * pa_bm_add_sequence_tokens  new sequence with token ids; its leading full
 *                       blocks that are cached for this version are shared
 *                       (taken back from the free list if needed) and
 *                       *num_cached_tokens = their tokens (the caller skips
 *                       their K/V); the rest are fresh.  The search stops
 *                       one token short of the end, so at least the last
 *                       token is always computed, into a private block (a
 *                       prompt of k whole cached blocks reuses k - 1).
 *                       All or nothing.
 * pa_bm_append_token_ids  pa_bm_append_tokens with the new tokens' ids
 *                       (PA_ERR_SHAPE if the sequence's ids are not known;
 *                       pa_bm_append_tokens forgets them)
 * pa_bm_commit          the first num_computed_tokens tokens' K/V are in
 *                       the pool: cache their full blocks, in order,
 *                       stopping at a block whose parent is not cached or
 *                       whose key another block already holds
 * pa_bm_drop_version    uncache every block of a version (a changed system
 *                       prompt); returns how many
 * pa_bm_cached_blocks   number of cached blocks; pa_bm_is_cached: 1 / 0
 * pa_bm_set_hash_bits   keep only the low bits of the hash (1..64, default
 *                       64; only while nothing is cached): forces collisions
 *                       so the exact-match check can be exercised
 */
typedef struct pa_block_manager pa_block_manager;
pa_block_manager* pa_bm_create(int32_t num_blocks, int32_t block_size, const int32_t* free_order);
void pa_bm_destroy(pa_block_manager* bm);
int32_t pa_bm_available(pa_block_manager* bm);
int32_t pa_bm_refcount(pa_block_manager* bm, int32_t block);
pa_status pa_bm_add_sequence(pa_block_manager* bm, int64_t seq_id, int32_t num_tokens);
pa_status pa_bm_fork(pa_block_manager* bm, int64_t parent, int64_t child);
pa_status pa_bm_append_tokens(pa_block_manager* bm, int64_t seq_id, int32_t num_new, int32_t* copy_src,
                              int32_t* copy_dst, int32_t* num_copies);
pa_status pa_bm_free_sequence(pa_block_manager* bm, int64_t seq_id);
int32_t pa_bm_block_table(pa_block_manager* bm, int64_t seq_id, int32_t* out, int32_t capacity);
int64_t pa_bm_num_tokens(pa_block_manager* bm, int64_t seq_id);
int32_t pa_bm_free_list(pa_block_manager* bm, int32_t* out, int32_t capacity);
pa_status pa_bm_add_sequence_tokens(pa_block_manager* bm, int64_t seq_id, const int32_t* token_ids,
                                    int32_t num_tokens, uint64_t version, int32_t* num_cached_tokens);
pa_status pa_bm_append_token_ids(pa_block_manager* bm, int64_t seq_id, const int32_t* token_ids, int32_t num_new,
                                 int32_t* copy_src, int32_t* copy_dst, int32_t* num_copies);
pa_status pa_bm_commit(pa_block_manager* bm, int64_t seq_id, int32_t num_computed_tokens);
int32_t pa_bm_drop_version(pa_block_manager* bm, uint64_t version);
int32_t pa_bm_cached_blocks(pa_block_manager* bm);
int32_t pa_bm_is_cached(pa_block_manager* bm, int32_t block);
pa_status pa_bm_set_hash_bits(pa_block_manager* bm, int32_t bits);
int32_t pa_bm_block_size(pa_block_manager* bm);

/* Continuous-batching step arithmetic (host only, thread-safe per scheduler).
 * [P1] "生产级推理引擎的内存管理与调度": one scheduling call per iteration
 * decides which requests take part, in three steps:
 *   1. every decoding request whose prompt + generated tokens need more
 *      blocks than it owns (ceil(tokens / block_size) > owned) takes one
 *      more block from the pool and is scheduled; if the pool is empty the
 *      request is preempted for this iteration (not scheduled, keeps its
 *      blocks); a request needing no block is scheduled;
 *   2. while fewer than max_batch_size requests are scheduled, the front of
 *      the FIFO waiting queue is admitted (its ceil(prompt / block_size)
 *      blocks allocated, state decoding) if the pool holds them, else it
 *      stays at the front and admission stops for this iteration;
 *   3. requests that have generated max_tokens tokens release their blocks.
 * Active requests are visited in admission order.  The scheduler keeps its
 * requests' blocks in the block manager it is given (sequence id = request
 * id; their tables are read with pa_bm_block_table); it does not own the
 * manager, which must outlive it.
 *
 * pa_sched_create       NULL on bad arguments (max_batch_size < 1)
 * pa_sched_add_request  queue a request; max_tokens >= 1 and prompt_len >= 0
 *                       (PA_ERR_SHAPE), id unused in the scheduler and the
 *                       manager (PA_ERR_EXISTS)
 * pa_sched_schedule     run one iteration's three steps; writes up to
 *                       capacity scheduled ids (decoding requests in
 *                       admission order, then the newly admitted) and their
 *                       count to *num_scheduled
 * pa_sched_copies       the copy-on-write pairs of the last
 *                       pa_sched_schedule call: a scheduled request whose
 *                       partly filled last block another sequence shares
 *                       (pa_bm_fork) was given a private block; copy
 *                       copy_src[i] -> copy_dst[i] with pa_copy_blocks
 *                       before the step writes its tokens.  Copies up to
 *                       capacity pairs, returns their number (-1 on bad
 *                       arguments)
 * pa_sched_step         one token generated by a decoding request
 *                       (PA_ERR_NOT_FOUND for any other id); reaching
 *                       max_tokens finishes it (released by the next
 *                       pa_sched_schedule)
 * pa_sched_state        0 waiting, 1 decoding, 2 finished, -1 unknown or
 *                       released
 * pa_sched_generated    tokens generated so far, -1 unknown or released
 */
typedef struct pa_scheduler pa_scheduler;
pa_scheduler* pa_sched_create(pa_block_manager* bm, int32_t max_batch_size);
void pa_sched_destroy(pa_scheduler* sched);
pa_status pa_sched_add_request(pa_scheduler* sched, int64_t request_id, int32_t prompt_len, int32_t max_tokens);
pa_status pa_sched_schedule(pa_scheduler* sched, int64_t* scheduled, int32_t capacity, int32_t* num_scheduled);
int32_t pa_sched_copies(pa_scheduler* sched, int32_t* copy_src, int32_t* copy_dst, int32_t capacity);
pa_status pa_sched_step(pa_scheduler* sched, int64_t request_id);
int32_t pa_sched_state(pa_scheduler* sched, int64_t request_id);
int32_t pa_sched_generated(pa_scheduler* sched, int64_t request_id);
int32_t pa_sched_num_waiting(pa_scheduler* sched);
int32_t pa_sched_num_active(pa_scheduler* sched);

/* Measurement helper, not part of the attention path: a plain streaming
 * read of `bytes` bytes of device memory at `src` (16-byte aligned, bytes a
 * multiple of 16) by `workgroups` workgroups of `threads` threads (a
 * multiple of 64, at most 1024), each reading one contiguous share with
 * 16-byte non-temporal loads, two batches of eight per thread in flight.
 * sink: device uint32 [workgroups], XOR-ed with what each workgroup read
 * (so the loads are kept).  Timing it beside pa_decode on the same number
 * of bytes gives the read bandwidth the chip reaches at a launch shape. */
pa_status pa_stream_read(const void* src, size_t bytes, int32_t workgroups, int32_t threads, uint32_t* sink,
                         hipStream_t stream);

const char* pa_status_string(pa_status status);
const char* pa_version(void);

#ifdef __cplusplus
}
#endif

#endif /* PA_H_ */
