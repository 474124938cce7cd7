// Slot mapping and the KV scatter into the paged pool (gfx950).
//
// Sources: [P1] "大模型推理内存优化从 KV Cache 分页到连续批处理的工程实践",
// section "KV Cache 的内存开销与分页机制" (block table maps logical to
// physical blocks; a new token goes into the current block or a new one).
#include <algorithm>

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
// token list; one workgroup per group and KV head.  A token row of one KV head is
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

// Scatter of tokens t0 .. t0+n-1 (n <= kGroup), KV heads h0 .. h0+nh-1, by
// one workgroup.  slot_of(i) gives token t0+i's slot (or -1 to skip it); it
// is called once per token, by thread i, while the other threads' first K/V
// loads are in flight.
template <typename T, typename SlotFn>
__device__ __forceinline__ void scatter_group(const ScatterArgs<T>& a, int64_t t0, int n, int h0, int nh,
                                              SlotFn slot_of) {
  using S = typename Src<T>::type;
  constexpr int VEC = vec16<S>();
  __shared__ int64_t s_slot[kGroup];
  const int tid = threadIdx.x;
  const int cpr = a.head_dim / VEC;             // 16-byte chunks per head row
  const int nk = n * nh * cpr;                  // key chunks of the group
  const int nv = nh * cpr;                      // value items: one chunk of every token
  auto src = [&](const S* base, int i, int h, int ch) {
    return *reinterpret_cast<const u32x4*>(base + ((t0 + i) * a.num_kv_heads + h) * a.head_dim + ch * VEC);
  };
  // First loads before the slots are known.
  u32x4 kpre = {0, 0, 0, 0};
  if (tid < nk) kpre = src(a.key, tid / (nh * cpr), h0 + (tid / cpr) % nh, tid % cpr);
  u32x4 vpre[kGroup];
#pragma unroll
  for (int i = 0; i < kGroup; ++i) vpre[i] = (tid < nv && i < n) ? src(a.value, i, h0 + tid / cpr, tid % cpr) : u32x4{0, 0, 0, 0};
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
                        : (idx < nk ? src(a.key, idx / (nh * cpr), h0 + (idx / cpr) % nh, idx % cpr)
                                    : u32x4{0, 0, 0, 0});
    }
#pragma unroll
    for (int j = 0; j < kKeyBatch; ++j) {
      const int idx = base + j * kScatterThreads;
      if (idx >= nk) break;
      const int i = idx / (nh * cpr), h = h0 + (idx / cpr) % nh, ch = idx % cpr;
      const int64_t sl = s_slot[i];
      if (sl < 0) continue;
      store_kv_chunk<T>(a.key_cache, a.value_cache, 0, sl / a.block_size, (int)(sl % a.block_size), h, ch, VEC,
                        a.num_kv_heads, a.head_dim, a.block_size, x[j], a.k_scale, a.v_scale);
    }
  }
  for (int it = tid; it < nv; it += kScatterThreads) {
    const int h = h0 + it / cpr, ch = it % cpr;
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
// (x / H) * kGroup .. + kGroup - 1 of KV head x % H (one head per workgroup:
// eight times the workgroups of one per token group, 10.2 against 14.1 us
// on 2096 tokens of 8 KV heads); slots < 0 (or past the pool) are skipped.
template <typename T>
__global__ void __launch_bounds__(kScatterThreads) reshape_and_cache_kernel(ScatterArgs<T> a,
                                                                           const int64_t* __restrict__ slots,
                                                                           int32_t num_tokens) {
  const int64_t t0 = (int64_t)(blockIdx.x / a.num_kv_heads) * kGroup;
  const int n = num_tokens - t0 < kGroup ? (int)(num_tokens - t0) : kGroup;
  scatter_group<T>(a, t0, n, (int)(blockIdx.x % a.num_kv_heads), 1, [&](int i) { return slots[t0 + i]; });
}

// Slot mapping and scatter in one pass, by tiles.  The new tokens of one
// sequence occupy consecutive positions, so those that fall into one
// logical block share its physical block and fill consecutive rows of its
// key tile and consecutive columns of its value tile.  One workgroup per
// (block touched by a sequence's new tokens, KV head): it computes the
// block's slots (recorded by the head-0 workgroup), copies the tokens' key
// rows into the key tile (each wave writing runs of whole 64-byte chunk
// rows), and transposes their values through LDS into the value tile,
// writing each tile row's covered part in 16-byte pieces.  A prefill chunk
// that fills a block thus writes both tiles of every (block, KV head) whole
// and contiguous.
//
// Which block: for batches of at most 64 sequences every workgroup reads
// all the chunk lengths (one per lane) and numbers the (sequence, block)
// pairs in order, so the grid needs only an upper bound on their count,
// (num_tokens + n (2B - 2)) / B; larger batches take a grid of (block
// slot k, sequence, head), k slowest, whose slots past a sequence's blocks
// leave at once.  Workgroups that find no block cost their launch, and in a
// batch of long chunks and one-token steps those launches were most of the
// time (7.5 of 12.4 us for the (k, sequence, head) grid on 4 chunks of 512
// and 48 steps).
constexpr int kAppendSeqs = 64;           // sequences numbered by one wave
constexpr int kMaxTileWords = 32 * 128;   // one value tile of 32-bit source words at most (32 x 128)

template <typename T>
__global__ void __launch_bounds__(kScatterThreads) append_kernel(
    ScatterArgs<T> a, const int32_t* __restrict__ block_tables, int32_t max_blocks,
    const int32_t* __restrict__ seq_lens, const int32_t* __restrict__ cu_q_lens, int64_t* __restrict__ slots,
    int32_t num_tokens, int32_t num_seqs, int32_t numbered) {
  using S = typename Src<T>::type;
  constexpr int VEC = vec16<S>();             // source elements per 16-byte chunk
  constexpr int KC = key_chunk<T>();          // elements per 64-byte key chunk
  constexpr int CPC = KC / VEC;               // source chunks per key chunk
  constexpr int PE = 16 / Elem<T>::kBytes;    // value-tile elements per 16-byte piece
  constexpr int SW = sizeof(S) == 4 ? 1 : 2;  // source elements per 32-bit word
  constexpr int kItems = kMaxTileWords / 4 / kScatterThreads;  // 16-byte items per thread at most
  static_assert(KC % VEC == 0, "a source chunk lies inside one key chunk");
  __shared__ uint32_t s_v[kMaxTileWords];
  const int H = a.num_kv_heads, D = a.head_dim, B = a.block_size;
  const int tid = threadIdx.x;
  const int h = (int)(blockIdx.x % H);
  int s, k, tq, q, L;
  if (numbered) {
    // Blocks touched by sequence l's chunk: positions L - q .. L - 1.
    const int lane = tid & 63;
    int nb = 0, tl = 0, ql = 0, Ll = 0;
    if (lane < num_seqs) {
      tl = cu_q_lens[lane];
      ql = cu_q_lens[lane + 1] - tl;
      Ll = seq_lens[lane];
      const int64_t pl = (int64_t)Ll - ql;
      if (ql > 0) {
        const int64_t first = pl >= 0 ? pl / B : -((-pl + B - 1) / B);
        const int64_t last = (pl + ql - 1) >= 0 ? (pl + ql - 1) / B : -((-(pl + ql - 1) + B - 1) / B);
        nb = (int)(last - first + 1);
      }
    }
    // Inclusive prefix sum over the lanes.
    int incl = nb;
#pragma unroll
    for (int d = 1; d < 64; d *= 2) {
      const int y = __shfl_up(incl, d, 64);
      incl += lane >= d ? y : 0;
    }
    const int r = (int)(blockIdx.x / H);
    const uint64_t past = __ballot(incl <= r);  // sequences wholly before pair r
    s = __builtin_popcountll(past);
    if (s >= num_seqs) return;  // past the last pair
    s = __builtin_amdgcn_readfirstlane(s);
    k = r - (s > 0 ? __builtin_amdgcn_readlane(incl, s - 1) : 0);
    tq = __builtin_amdgcn_readlane(tl, s);
    q = __builtin_amdgcn_readlane(ql, s);
    L = __builtin_amdgcn_readlane(Ll, s);
  } else {
    const int sk = (int)(blockIdx.x / H);
    s = sk % num_seqs;
    k = sk / num_seqs;
    tq = cu_q_lens[s];
    q = cu_q_lens[s + 1] - tq;
    L = seq_lens[s];
  }
  if (q <= 0) return;
  // Positions pf .. pf+q-1 (token rows tq ..); this workgroup takes the
  // k-th block they touch, j, clipped to the token rows that exist.
  const int64_t pf = (int64_t)L - q;
  const int64_t j = (pf >= 0 ? pf / B : -((-pf + B - 1) / B)) + k;
  int64_t lo = pf > j * B ? pf : j * B;
  int64_t hi = pf + q < (j + 1) * B ? pf + q : (j + 1) * B;
  const int64_t t_lo = tq + (lo - pf);
  if (t_lo < 0) lo -= t_lo;
  if (tq + (hi - pf) > num_tokens) hi -= tq + (hi - pf) - num_tokens;
  if (lo >= hi) return;
  const int n = (int)(hi - lo);
  const int64_t t0 = tq + (lo - pf);  // token row of position lo
  const int o0 = (int)(lo - j * B);   // its row of the tile
  const bool in_table = j >= 0 && j < max_blocks;
  const int64_t phys = in_table ? (int64_t)block_tables[(int64_t)s * max_blocks + j] : -1;

  // Every source load of the segment is issued before anything is stored
  // (a store into the pool could alias a source row as far as the compiler
  // knows) and without waiting for the table entry.  Key items it = (chunk
  // c, token o, piece sub), sub fastest, so a wave stores whole chunk rows
  // of consecutive tokens; value items (token o, piece ch) as the rows lie.
  const int cpr = D / VEC;
  const int nk = n * cpr;
  u32x4 kx[kItems], vx[kItems];
#pragma unroll
  for (int b = 0; b < kItems; ++b) {
    const int it = tid + b * kScatterThreads;
    if (it < nk) {
      const int sub = it % CPC, o = (it / CPC) % n, c = it / (CPC * n);
      kx[b] = *reinterpret_cast<const u32x4*>(a.key + ((t0 + o) * H + h) * D + (c * CPC + sub) * VEC);
      vx[b] = *reinterpret_cast<const u32x4*>(a.value + ((t0 + it / cpr) * H + h) * D + (it % cpr) * VEC);
    }
  }
  // The values staged in LDS as they come ([token][dim], D / SW words a
  // row) for the transposed writes below.
  const int W = D / SW;
#pragma unroll
  for (int b = 0; b < kItems; ++b) {
    const int it = tid + b * kScatterThreads;
    if (it < nk) {
#pragma unroll
      for (int e = 0; e < 4; ++e) s_v[(it / cpr) * W + (it % cpr) * 4 + e] = vx[b][e];
    }
  }
  if (h == 0) {
    for (int i = tid; i < n; i += kScatterThreads) slots[t0 + i] = in_table ? phys * B + o0 + i : -1;
  }
  if (!in_table || phys < 0 || phys * B >= a.pool_slots) return;  // not written
#pragma unroll
  for (int b = 0; b < kItems; ++b) {
    const int it = tid + b * kScatterThreads;
    if (it < nk) {
      const int sub = it % CPC, o = (it / CPC) % n, c = it / (CPC * n);
      store_kv_chunk<T>(a.key_cache, a.value_cache, 0, phys, o0 + o, h, c * CPC + sub, VEC, H, D, B, kx[b],
                        a.k_scale, a.v_scale);
    }
  }
  __syncthreads();
  // Piece p of value-tile row d holds tokens p*PE .. p*PE+PE-1 of the block.
  const int p0 = o0 / PE, p1 = (o0 + n - 1) / PE;
  const int npc = p1 - p0 + 1;
  T* tile = a.value_cache + (phys * H + h) * (int64_t)D * B;
  for (int it = tid; it < D * npc; it += kScatterThreads) {
    const int p = p0 + it % npc, d = it / npc;
    T* row = tile + (int64_t)d * B;
    // Source element (token o of the block, dim d) as raw bits (16-bit
    // types in the low half).
    auto elem = [&](int o) -> uint32_t {
      const uint32_t w = s_v[(o - o0) * W + d / SW];
      return SW == 1 ? w : (w >> (16 * (d % 2))) & 0xffffu;
    };
    const int e0 = p * PE;
    if (e0 >= o0 && e0 + PE <= o0 + n) {
      u32x4 r = {0u, 0u, 0u, 0u};
      if constexpr (Elem<T>::kBytes == 4) {
#pragma unroll
        for (int e = 0; e < 4; ++e) r[e] = elem(e0 + e);
      } else if constexpr (Elem<T>::kBytes == 2) {
#pragma unroll
        for (int e = 0; e < 4; ++e) r[e] = elem(e0 + 2 * e) | (elem(e0 + 2 * e + 1) << 16);
      } else {
#pragma unroll
        for (int e = 0; e < 16; ++e) r[e / 4] |= f32_to_e4m3(f16_lo(elem(e0 + e)) / a.v_scale) << (8 * (e % 4));
      }
      *reinterpret_cast<u32x4*>(row + e0) = r;
    } else {
      for (int e = 0; e < PE; ++e) {
        const int o = e0 + e;
        if (o < o0 || o >= o0 + n) continue;
        const uint32_t bits = elem(o);
        if constexpr (Elem<T>::kBytes == 4) {
          reinterpret_cast<uint32_t*>(row)[o] = bits;
        } else if constexpr (Elem<T>::kBytes == 2) {
          reinterpret_cast<uint16_t*>(row)[o] = (uint16_t)bits;
        } else {
          reinterpret_cast<uint8_t*>(row)[o] = (uint8_t)f32_to_e4m3(f16_lo(bits) / a.v_scale);
        }
      }
    }
  }
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
  const int tile_words = c.block_size * c.head_dim / (sizeof(typename Src<T>::type) == 4 ? 1 : 2);
  if (tile_words > kMaxTileWords) return hipErrorInvalidValue;
  // (sequence, block) pairs: numbered on the device for small batches,
  // else every sequence's chunk may touch up to ceil((B - 1 + q) / B)
  // blocks.
  const int B = c.block_size;
  const bool numbered = num_seqs <= kAppendSeqs;
  const int64_t pairs = numbered ? ((int64_t)num_tokens + (int64_t)num_seqs * (2 * B - 2)) / B
                                 : ((int64_t)max_q_len + 2 * B - 2) / B * num_seqs;
  const int64_t groups = pairs * c.num_kv_heads;
  if (groups > INT32_MAX) return hipErrorInvalidValue;
  hipLaunchKernelGGL(append_kernel<T>, dim3((unsigned)groups), dim3(kScatterThreads), 0, stream,
                     scatter_args<T>(c, key, value), block_tables, max_blocks, seq_lens, cu_q_lens, slots, num_tokens,
                     num_seqs, (int32_t)numbered);
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
  const int64_t groups = ((int64_t)num_tokens + kGroup - 1) / kGroup * c.num_kv_heads;
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
