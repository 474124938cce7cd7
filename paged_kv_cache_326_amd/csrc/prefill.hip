// Chunked-prefill attention over a float16 / bfloat16 paged cache on gfx950
// matrix cores (FP8 pools: prefill_fp8.hip).
//
// Sources: [P1] "大模型推理内存优化从 KV Cache 分页到连续批处理的工程实践",
// section "工程边界与架构取舍" (prefill is a compute-bound matrix product; a
// long prompt is processed in chunks interleaved with decode steps) and
// section "PagedAttention 的 CUDA Kernel 实现" (K/V reached block by block
// through the table).
//
// A chunk of q_s new tokens of sequence s sits at positions ctx .. ctx+q_s-1
// (ctx = seq_len - q_s; the chunk's own K/V are already in the pool) and
// attends causally: position ctx+i sees keys 0 .. ctx+i.
//
// Work decomposition.  A workgroup of 8 waves (two per SIMD) owns 256 query
// rows that share one KV head: the G heads of the group times 256/G
// consecutive positions; each wave owns 32 of them.  Keys stream through in
// tiles of 32; per wave
//   S^T[32 keys x 32 rows] = K . Q^T      v_mfma_f32_32x32x16 over D
//   online softmax down each column (a column is one query row, held by a
//   lane pair), P^T rounded to the storage type in registers
//   O^T[D x 32 rows]     += V^T . P^T    v_mfma_f32_32x32x16 over the tile
// Each step multiplies the scores of tile t+1 while it exponentiates and
// rounds tile t's probabilities, then runs tile t's PV product while it
// finds tile t+1's maxima and rescale factors; the two waves of a SIMD fill
// each other's waits.  Masks (the causal diagonal, blocks missing from the
// pool), the accumulator rescale and the rounding remainder below run only
// on the tiles that need them.  A workgroup serves two query tiles of one
// (sequence, KV head), j and n-1-j, so that every workgroup carries about
// the same causal work.
//
// Staging.  Tiles move from the pool straight into LDS (16 bytes per lane,
// no registers on the way) through six stages, each its own array so that
// the compiler waits only for the loads this code waits for.  A pass covers
// two tiles between barriers: it starts the loads of tiles t+3 and t+4,
// computes tiles t and t+1, and by its end those loads have landed.  A
// stage holds the tile's K as the pool stores it (column chunks of 32
// dimensions, one 64-byte row per key) and its V^T (one 64-byte row of 32
// keys per dimension); the 16-byte columns of each row are permuted (kswz,
// vswz) so that the operand reads hit every bank group once.
//
// Computing the transposed products keeps every operand a 16-byte LDS or
// register read: the accumulator layout of S^T is directly the B operand of
// the PV product once the S^T rows (keys) are permuted by swapping index bits
// 2 and 3, and each lane's accumulators of O^T belong to one query row, so
// the softmax rescale is a per-lane scalar.
//
// Operand layouts of v_mfma_f32_32x32x16 (lane l, e = 0..7, j = 0..15):
//   A[m][k]: m = l % 32, k = 8 (l / 32) + e
//   B[k][n]: k = 8 (l / 32) + e, n = l % 32
//   C[m][n]: m = 8 (j / 4) + 4 (l / 32) + j % 4, n = l % 32
#include <math.h>

#include <type_traits>

#include "pa_common.h"
#include "pa_launch.h"

namespace pa {

namespace {

#ifndef PA_PREFILL_WAVE_ROWS
#define PA_PREFILL_WAVE_ROWS 32
#endif
constexpr int kWR = PA_PREFILL_WAVE_ROWS;  // query rows per wave (halves of 32)
constexpr int kHalves = kWR / 32;
constexpr int kRows = 256;                 // query rows per workgroup
constexpr int kPW = kRows / kWR;           // waves per workgroup
constexpr int kKT = 32;           // keys per tile
constexpr int kStages = 6;        // key tiles resident in LDS
constexpr int kBtStage = 2048;    // table entries staged in LDS (32K tokens at block size 16)
// The running maximum of a row is moved only when a tile's maximum exceeds
// it by more than this (log2 units), so probabilities stay below 2^8 and the
// accumulator rescale is rare; the final division by the row sum cancels
// whichever reference maximum was used.
constexpr float kLazy = 8.f;
// bf16 keeps 8 significant bits of a probability.  Rounding p once is
// accurate enough for keys that can hold only a small share of their row's
// final weight; a tile in which some row's largest probability could reach
// more than this share (judged against the row's sum before the tile, so
// the first tiles of every row qualify) also multiplies the rounding
// remainder bf16(p - bf16(p)), which restores about 16 bits.
constexpr float kSplitShare = 1.f / 16.f;
// Logit scales are taken as at least this large in magnitude, so that a
// masked logit (-inf) times the scale stays -inf; every smaller scale gives
// probabilities that round to those of a zero scale.
constexpr float kMinScale = 1e-30f;

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef __attribute__((address_space(3))) void lds_void;

// 16 bytes per lane from global memory straight into LDS (lane i's bytes
// land at lds + 16 i).  The host pass never runs device code, and with the
// builtin in its view it silently drops the kernels' launch stubs, so it
// sees an empty body.
__device__ __forceinline__ void load16_to_lds(const void* src, void* lds) {
#if defined(__HIP_DEVICE_COMPILE__)
  __builtin_amdgcn_global_load_lds(src, (lds_void*)lds, 16, 0, 0);
#endif
}

template <typename T>
__device__ __forceinline__ f32x16 mfma32(const u32x4& a, const u32x4& b, const f32x16& c);
template <>
__device__ __forceinline__ f32x16 mfma32<bf16_t>(const u32x4& a, const u32x4& b, const f32x16& c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a), __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
}
template <>
__device__ __forceinline__ f32x16 mfma32<f16_t>(const u32x4& a, const u32x4& b, const f32x16& c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(f16x8, a), __builtin_bit_cast(f16x8, b), c, 0, 0, 0);
}

// Two floats -> one packed pair of storage elements (round to nearest even).
template <typename T>
__device__ __forceinline__ uint32_t pack2(float lo, float hi);
template <>
__device__ __forceinline__ uint32_t pack2<bf16_t>(float lo, float hi) {
  return pack_bf16x2(lo, hi);
}
template <>
__device__ __forceinline__ uint32_t pack2<f16_t>(float lo, float hi) {
  return pack_f16x2(lo, hi);
}

// The two elements of a packed pair as floats.
template <typename T>
__device__ __forceinline__ float lo_value(uint32_t w);
template <typename T>
__device__ __forceinline__ float hi_value(uint32_t w);
template <>
__device__ __forceinline__ float lo_value<bf16_t>(uint32_t w) {
  return bf16_lo(w);
}
template <>
__device__ __forceinline__ float hi_value<bf16_t>(uint32_t w) {
  return bf16_hi(w);
}
template <>
__device__ __forceinline__ float lo_value<f16_t>(uint32_t w) {
  return f16_lo(w);
}
template <>
__device__ __forceinline__ float hi_value<f16_t>(uint32_t w) {
  return f16_hi(w);
}

// acc + both elements of a packed pair: the row sum is taken over the very
// values the PV product multiplies.
template <typename T>
__device__ __forceinline__ float add_pair(uint32_t w, float acc);
template <>
__device__ __forceinline__ float add_pair<bf16_t>(uint32_t w, float acc) {
  return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, w), __builtin_bit_cast(bf16x2, 0x3f803f80u), acc,
                                         false);
}
template <>
__device__ __forceinline__ float add_pair<f16_t>(uint32_t w, float acc) {
  return __builtin_amdgcn_fdot2(__builtin_bit_cast(f16x2, w), __builtin_bit_cast(f16x2, 0x3c003c00u), acc, false);
}

// Column permutation of the 64-byte LDS rows (four 16-byte columns).  K rows
// are read by lanes n = 0..31 in the order of keys with index bits 2 and 3
// swapped, V^T rows in plain order; either way the eight (sixteen) lanes that
// the LDS serves together then touch eight (sixteen) distinct 16-byte slots.
__device__ __forceinline__ int kswz(int key) { return (((key >> 1) ^ (key >> 2)) & 1) | (((key >> 3) & 1) << 1); }
__device__ __forceinline__ int vswz(int d) { return (((d >> 1) ^ (d >> 3)) & 1) | (((d >> 2) & 1) << 1); }

// s_waitcnt immediate (gfx9 encoding: vmcnt in bits 3:0 and 15:14, expcnt
// 6:4, lgkmcnt 11:8): at most `vm` vector-memory and `lgkm` LDS/scalar
// operations of this wave left outstanding.
constexpr int waitcnt(int vm, int lgkm) { return (vm & 15) | (7 << 4) | ((lgkm & 15) << 8) | (((vm >> 4) & 3) << 14); }
constexpr int kNoWait = 63;

// Wait, then meet the workgroup at a barrier.  The loads straight into LDS
// count as vector-memory operations; the caller states how many of them may
// still be in flight.  The empty asm statements keep the compiler from
// moving memory accesses across.
template <int VM, int LGKM>
__device__ __forceinline__ void wait_barrier() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_waitcnt(waitcnt(VM, LGKM));
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

template <int S>
using Stage = std::integral_constant<int, S>;

// acc *= alpha, in place.  Written as assembly so that the rescaled values
// keep the accumulator's registers: as plain code the compiler may give them
// new ones and then carry two copies of the whole accumulator set around the
// rarely taken branch (or spill).  The leading no-ops cover the wait states
// between a matrix product's result and a vector read of it (at most 18 for
// a 16-pass product), the trailing ones those between a vector write and the
// next product's accumulator read.
__device__ __forceinline__ void rescale_acc(f32x16& acc, float alpha) {
  asm volatile("s_nop 7\n s_nop 7\n s_nop 7" : "+v"(acc));
#pragma unroll
  for (int j = 0; j < 16; ++j) asm volatile("v_mul_f32 %0, %0, %1" : "+v"(acc[j]) : "v"(alpha));
  asm volatile("s_nop 7" : "+v"(acc));
}

template <typename T, int D, int B, int G>
__global__ void __launch_bounds__(kPW * 64) __attribute__((amdgpu_waves_per_eu(kPW / 4, kPW / 4)))
prefill_kernel(PrefillArgs a) {
  static_assert(Elem<T>::kBytes == 2, "16-bit pools");
  constexpr int QP = kRows / G;          // positions per workgroup
  constexpr int KSTEPS = D / 16;         // QK contraction steps
  constexpr int DT = D / 32;             // O^T row tiles
  constexpr int NT = kPW * 64;
  // Share of a row's weight above which a tile also multiplies the rounding
  // remainders: bf16 probabilities (8 significant bits) need them for large
  // shares; f16 ones (11 bits) never do, so theirs is 1, which no tile's
  // test can exceed (0 * p_max > l never holds).  Both types run the same
  // code, whose register use the compiler then lays out the same way.
  constexpr float kShare = std::is_same<T, bf16_t>::value ? kSplitShare : 1.f;
  static_assert(B == kKT || 2 * B == kKT, "a key tile spans one or two blocks");
  constexpr int kTileBytes = kKT * D * 2;     // K (and V) bytes of one tile
  constexpr int kStageBytes = 2 * kTileBytes; // K, then V^T
  constexpr int kPieces = kTileBytes / 1024;  // 1 KB wave loads per K (or V) tile
  static_assert(2 * kPieces % kPW == 0, "every wave issues the same loads");
  constexpr int kLoadsPerTile = 2 * kPieces / kPW;  // vector-memory instructions per wave per tile

  // One array per stage, always addressed with a compile-time stage number:
  // the compiler can then tell that reads of one stage do not touch the
  // loads still landing in another, and waits for them only where this code
  // says so (with a single array it waits for every load in flight before
  // any LDS read).
  static_assert(kStages == 6, "six stage arrays below");
  __shared__ __align__(1024) unsigned char stage0[kStageBytes], stage1[kStageBytes], stage2[kStageBytes],
      stage3[kStageBytes], stage4[kStageBytes], stage5[kStageBytes];
  auto stage = [&](auto S) -> unsigned char* {
    constexpr int k = decltype(S)::value % kStages;
    return k == 0 ? stage0 : k == 1 ? stage1 : k == 2 ? stage2 : k == 3 ? stage3 : k == 4 ? stage4 : stage5;
  };
  __shared__ int s_bt[kBtStage];

  // Work item: a pair of query tiles of one sequence and KV head, j and
  // nqt-1-j.  Under the causal mask a tile's key range grows with its
  // position, so every pair holds about the same work and one round of
  // workgroups (one per compute unit at the mixed config) ends together;
  // both tiles read the same K/V.  Workgroup ids are dealt to the 8 XCDs
  // round-robin; remap so that consecutive pairs (of one sequence and KV
  // head) land on the same XCD and share its L2.
  const int nqt = a.num_qtiles;
  const int npair = (nqt + 1) / 2;
  const int total = a.num_seqs * a.cache.num_kv_heads * npair;
  const int per_xcd = (total + 7) / 8;
  const int u = (blockIdx.x % 8) * per_xcd + blockIdx.x / 8;
  if (u >= total) return;
  const int jp = u % npair;
  const int g = (u / npair) % a.cache.num_kv_heads;
  const int s = u / npair / a.cache.num_kv_heads;

  // One query tile: rows q0 .. q0+QP-1 of the chunk (QP positions of the
  // group's G heads).
  auto process = [&](const int qt) {
  const int qbeg = a.cu_q_lens[s];
  // Rows stay below the call's token count (the query and output length),
  // whatever the other prefix sums hold.
  const int qend = min(a.cu_q_lens[s + 1], a.cu_q_lens[a.num_seqs]);
  const int q_len = qend - qbeg;
  const int q0 = qt * QP;
  if (qbeg < 0 || q0 >= q_len) return;
  int L = a.seq_lens[s];
  const int Lmax = a.max_blocks * B;
  L = L > Lmax ? Lmax : L;
  const int ctx = L - q_len;
  if (ctx < 0) return;  // inconsistent lengths: nothing defined to compute
  const int nvalid = min(QP, q_len - q0);
  const int kend = ctx + q0 + nvalid;  // keys 0 .. kend-1 are visible to some row
  const int ntiles = (kend + kKT - 1) / kKT;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int w = tid >> 6;
  const int n = lane & 31;
  const int hi = lane >> 5;
  const int Hkv = a.cache.num_kv_heads;
  const int Hq = a.num_heads;

  // This lane's query rows: column n of the wave's two S^T / O^T halves.
  bool row_ok[kHalves];
  int limit[kHalves], hq[kHalves];
  int64_t tok[kHalves];
  // The smallest causal limit among this wave's rows that exist: a key tile
  // that ends at or below it is visible to all of them, unmasked.
  int lim_min = 0x7fffffff;
#pragma unroll
  for (int hf = 0; hf < kHalves; ++hf) {
    const int r = w * kWR + 32 * hf + n;
    const int h = r / QP;
    const int p = r % QP;
    row_ok[hf] = q0 + p < q_len;
    limit[hf] = row_ok[hf] ? ctx + q0 + p : -1;
    tok[hf] = (int64_t)qbeg + q0 + p;
    hq[hf] = g * G + h;
    if (row_ok[hf]) lim_min = min(lim_min, limit[hf]);
  }
#pragma unroll
  for (int m = 1; m < 64; m <<= 1) lim_min = min(lim_min, __shfl_xor(lim_min, m, 64));
  lim_min = __builtin_amdgcn_readfirstlane(lim_min);  // wave-uniform: scalar branches below

  // Q rows as B operands.  A negative scale is moved into Q (negation is
  // exact), so the logit scale below is positive and the maximum of the
  // scaled logits is the scaled maximum.
  const uint32_t qflip = a.scale < 0.f ? 0x80008000u : 0u;
  u32x4 qreg[kHalves][KSTEPS];
#pragma unroll
  for (int hf = 0; hf < kHalves; ++hf) {
    const T* qrow = reinterpret_cast<const T*>(a.query) + (tok[hf] * Hq + hq[hf]) * D;
#pragma unroll
    for (int ks = 0; ks < KSTEPS; ++ks) {
      qreg[hf][ks] = row_ok[hf] ? *reinterpret_cast<const u32x4*>(qrow + 16 * ks + 8 * hi) : u32x4{0, 0, 0, 0};
      qreg[hf][ks] ^= qflip;
    }
  }

  const T* kc = reinterpret_cast<const T*>(a.cache.key_cache);
  const T* vc = reinterpret_cast<const T*>(a.cache.value_cache);
  const int32_t* bt = a.block_tables + (int64_t)s * a.max_blocks;
  // The table entries this workgroup needs are staged in LDS once (the tile
  // loop would otherwise pay a dependent global read before every K/V load);
  // tables longer than the staging area are read from global memory.
  const int nbk = (kend + B - 1) / B;
  const bool staged = nbk <= kBtStage;
  if (staged) {
    for (int j = tid; j < nbk; j += NT) {
      const int id = bt[j];
      s_bt[j] = (id >= 0 && id < a.cache.num_blocks) ? id : -1;
    }
  }
  __syncthreads();
  // Table entry j as a pool block, -1 past the keys any row sees or outside
  // the pool (only validated entries are ever used as addresses).
  auto block_at = [&](int j) -> int {
    if (j >= nbk) return -1;
    if (staged) return s_bt[j];
    const int id = bt[j];
    return (id >= 0 && id < a.cache.num_blocks) ? id : -1;
  };
  // The one or two blocks of key tile t: fetched one iteration before they
  // are needed (the LDS read then completes under the barrier's wait instead
  // of stalling the tile loop), made wave-uniform when used.
  struct TileBlocks {
    int b0, b1;
  };
  auto fetch_blocks = [&](int t) -> TileBlocks {
    const int b0 = block_at(t * kKT / B);
    return {b0, B == kKT ? b0 : block_at(t * kKT / B + 1)};
  };
  auto uniform = [](TileBlocks x) -> TileBlocks {
    return {__builtin_amdgcn_readfirstlane(x.b0), __builtin_amdgcn_readfirstlane(x.b1)};
  };

  // Pool -> LDS for tile t into its stage: 2 * kPieces 1 KB pieces (K, then
  // V^T), kLoadsPerTile per wave.  Lane i writes bytes 16i .. 16i+15 of its
  // piece, i.e. row i / 4, stored column i % 4, which holds the pool's
  // column (i % 4) ^ swizzle(row).  Keys in blocks missing from the pool, or
  // past the table entries any row needs, load from block 0 (the pool is
  // never empty): their logits are masked and their V^T columns zeroed
  // before use (fix_values).
  // Per lane, the byte offset of its 16 bytes inside a block's K (V^T) tile
  // and which of the tile's two blocks they come from; only the block ids
  // change from tile to tile.
  int lane_off[kLoadsPerTile];
  bool lane_hi[kLoadsPerTile];
#pragma unroll
  for (int k = 0; k < kLoadsPerTile; ++k) {
    // Piece q (wave-uniform): K, chunk q / 2, keys 16 (q % 2) .., or V^T,
    // dimensions 16 (q - kPieces) ..
    const int q = w * kLoadsPerTile + k;
    if (q < kPieces) {
      const int key = 16 * (q % 2) + lane / 4;
      const int col = (lane % 4) ^ kswz(key);
      lane_off[k] = 2 * ((q / 2) * (B * 32) + (key % B) * 32 + col * 8);
      lane_hi[k] = B != kKT && key >= B;
    } else {
      const int d = 16 * (q - kPieces) + lane / 4;
      const int col = (lane % 4) ^ vswz(d);
      lane_off[k] = 2 * (d * B + (8 * col) % B);
      lane_hi[k] = B != kKT && 8 * col >= B;
    }
  }
  const int64_t head_off = (int64_t)g * (B * D) * 2;  // bytes of head g inside a block
  auto load_tile = [&](auto S, TileBlocks tb) {
    unsigned char* st = stage(S);
    const int64_t blk_bytes = (int64_t)Hkv * (B * D) * 2;
    // Missing blocks (-1) read block 0 (the pool is never empty).
    const int64_t off0 = (tb.b0 >= 0 ? tb.b0 : 0) * blk_bytes + head_off;
    const int64_t off1 = (tb.b1 >= 0 ? tb.b1 : 0) * blk_bytes + head_off;
#pragma unroll
    for (int k = 0; k < kLoadsPerTile; ++k) {
      const int q = w * kLoadsPerTile + k;
      const unsigned char* base =
          reinterpret_cast<const unsigned char*>(q < kPieces ? kc : vc) + (lane_hi[k] ? off1 : off0);
      load16_to_lds(base + lane_off[k], st + q * 1024);
    }
  };


  // Zero the V^T entries of tile t's keys that no row may see (at or past
  // kend, or in a missing block), so that 0 * V stays finite whatever the
  // pool holds there.
  auto fix_values = [&](auto S, int t, uint32_t gaps) {
    unsigned char* vt = stage(S) + kTileBytes;
    const int nvis = kend - t * kKT;  // keys of the tile below kend
    for (int c = tid; c < D * 4; c += NT) {
      const int d = c / 4, col = c % 4;
      const int key0 = 8 * (col ^ vswz(d));
      u32x4* piece = reinterpret_cast<u32x4*>(vt + d * 64 + col * 16);
      u32x4 x = *piece;
      const bool gone = (gaps >> (key0 / 16)) & 1u;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int k = key0 + 2 * e;
        const uint32_t keep = gone || k >= nvis ? 0u : (k + 1 >= nvis ? 0xffffu : 0xffffffffu);
        x[e] &= keep;
      }
      *piece = x;
    }
  };

  f32x16 o[kHalves][DT];
#pragma unroll
  for (int hf = 0; hf < kHalves; ++hf)
#pragma unroll
    for (int dt = 0; dt < DT; ++dt)
#pragma unroll
      for (int j = 0; j < 16; ++j) o[hf][dt][j] = 0.f;
  float m_run[kHalves], l_run[kHalves];
#pragma unroll
  for (int hf = 0; hf < kHalves; ++hf) {
    m_run[hf] = -INFINITY;
    l_run[hf] = 0.f;
  }
  const float qscale = fmaxf(fabsf(a.scale) * kLog2e, kMinScale);

  // LDS operand addresses of this lane.  K: key krow (bits 2 and 3 of n
  // swapped), dimensions 16 ks + 8 hi .. +8 = chunk ks / 2, column
  // 2 (ks % 2) + hi.  V^T: dimension 32 dt + n, keys 16 ks + 8 hi .. +8 =
  // column 2 ks + hi.
  const int krow = (n & ~12) | ((n & 4) << 1) | ((n & 8) >> 1);
  const int koff[2] = {krow * 64 + ((hi ^ kswz(krow)) * 16), krow * 64 + (((2 + hi) ^ kswz(krow)) * 16)};
  const int voff[2] = {n * 64 + ((hi ^ vswz(n)) * 16), n * 64 + (((2 + hi) ^ vswz(n)) * 16)};

  // S^T = K . Q^T for the tile in stage st, both halves.
  auto scores = [&](auto S, f32x16 (&acc)[kHalves]) {
#pragma unroll
    for (int hf = 0; hf < kHalves; ++hf)
#pragma unroll
      for (int j = 0; j < 16; ++j) acc[hf][j] = 0.f;
    const unsigned char* kb = stage(S);
#pragma unroll
    for (int ks = 0; ks < KSTEPS; ++ks) {
      const u32x4 ka = *reinterpret_cast<const u32x4*>(kb + (ks / 2) * (kKT * 64) + koff[ks % 2]);
#pragma unroll
      for (int hf = 0; hf < kHalves; ++hf) acc[hf] = mfma32<T>(ka, qreg[hf][ks], acc[hf]);
    }
  };

  // Masks of tile t's scores: -inf for keys past the row's causal limit or
  // in a missing block (`gaps` bit h: keys 16h .. 16h+15 of the tile lie in
  // a block outside the pool; such keys hold no vector, so they are masked,
  // never read as zeros, which would still add to the row's normaliser).
  // Accumulator j holds key t*32 + 16 (j / 8) + 8 hi + j % 8 (after the row
  // permutation).
  auto mask = [&](f32x16 (&sv)[kHalves], int t, uint32_t gaps) {
    const int kt0 = t * kKT + 8 * hi;
#pragma unroll
    for (int hf = 0; hf < kHalves; ++hf)
#pragma unroll
      for (int j = 0; j < 16; ++j) {
        const int key = kt0 + 16 * (j >> 3) + (j & 7);
        const bool gone = (gaps >> (j >> 3)) & 1u;
        sv[hf][j] = key <= limit[hf] && !gone ? sv[hf][j] : -INFINITY;
      }
  };

  // Softmax, first part, for a tile's (unscaled) scores: row maxima, the
  // lazy move of the running maximum and the rescale factor it implies, and
  // whether the tile needs the rounding remainder.
  auto phase1 = [&](const f32x16 (&sv)[kHalves], float (&alpha)[kHalves], float (&mref)[kHalves], bool& split_next,
                    bool& rescale) {
    bool split = false, moved = false;
#pragma unroll
    for (int hf = 0; hf < kHalves; ++hf) {
      float mt = sv[hf][0];
#pragma unroll
      for (int j = 1; j < 16; ++j) mt = fmaxf(mt, sv[hf][j]);
      mt = max_across_halves(mt * qscale);
      const bool move = mt > m_run[hf] + kLazy;
      const float m_new = move ? mt : m_run[hf];
      alpha[hf] = move ? fast_exp2(m_run[hf] - m_new) : 1.f;  // 0 from -inf
      m_run[hf] = m_new;
      // A row that has seen no key yet (m_run = -inf) only holds masked
      // logits: exp2(-inf) = 0 with any finite reference.
      mref[hf] = m_new == -INFINITY ? 0.f : m_new;
      moved = moved || move;
      // The row's largest probability in this tile against a lower bound of
      // the row's sum including it: the sum so far (both lanes of the row,
      // at the new reference; l_run itself is rescaled with the
      // accumulators when the tile's step begins) plus that probability.
      const float pmax = fast_exp2(mt - mref[hf]);
      split = split || pmax * (1.f - kShare) > kShare * sum_across_halves(l_run[hf] * alpha[hf]);
    }
    split_next = __any(split);
    rescale = __any(moved);
  };

  // Softmax, second part: probabilities rounded into the P^T operands, and
  // their sum.
  auto phase2 = [&](const f32x16 (&sv)[kHalves], const float (&mref)[kHalves], u32x4 (&pb)[kHalves][2]) {
#pragma unroll
    for (int hf = 0; hf < kHalves; ++hf) {
      float ps[2] = {0.f, 0.f};
#pragma unroll
      for (int ks = 0; ks < 2; ++ks)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int j = 8 * ks + 2 * i;
          pb[hf][ks][i] = pack2<T>(fast_exp2(fmaf(sv[hf][j], qscale, -mref[hf])),
                                   fast_exp2(fmaf(sv[hf][j + 1], qscale, -mref[hf])));
          ps[ks] = add_pair<T>(pb[hf][ks][i], ps[ks]);
        }
      l_run[hf] += ps[0] + ps[1];
    }
  };
  // The rounding remainders p - bf16(p) of a tile that needs them (the
  // probabilities are recomputed: the tile is rare), added to the sum.
  auto remainders = [&](const f32x16 (&sv)[kHalves], const float (&mref)[kHalves], const u32x4 (&pb)[kHalves][2],
                        u32x4 (&pl)[kHalves][2]) {
#pragma unroll
    for (int hf = 0; hf < kHalves; ++hf) {
      float ps = 0.f;
#pragma unroll
      for (int ks = 0; ks < 2; ++ks)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int j = 8 * ks + 2 * i;
          const float x0 = fast_exp2(fmaf(sv[hf][j], qscale, -mref[hf]));
          const float x1 = fast_exp2(fmaf(sv[hf][j + 1], qscale, -mref[hf]));
          pl[hf][ks][i] = pack2<T>(x0 - lo_value<T>(pb[hf][ks][i]), x1 - hi_value<T>(pb[hf][ks][i]));
          ps = add_pair<T>(pl[hf][ks][i], ps);
        }
      l_run[hf] += ps;
    }
  };

  // O^T += V^T . P^T for the tile in stage st, both halves (P^T: the
  // rounded probabilities, or their remainders).
  auto accumulate = [&](auto S, const u32x4 (&pb)[kHalves][2]) {
    const unsigned char* vb = stage(S) + kTileBytes;
#pragma unroll
    for (int dt = 0; dt < DT; ++dt)
#pragma unroll
      for (int ks = 0; ks < 2; ++ks) {
        const u32x4 va = *reinterpret_cast<const u32x4*>(vb + dt * (32 * 64) + voff[ks]);
#pragma unroll
        for (int hf = 0; hf < kHalves; ++hf) o[hf][dt] = mfma32<T>(va, pb[hf][ks], o[hf][dt]);
      }
  };

  auto tile_gaps = [](TileBlocks tb) -> uint32_t { return (tb.b0 < 0 ? 1u : 0u) | (tb.b1 < 0 ? 2u : 0u); };
  // Tiles that reach past the wave's smallest limit or touch a missing
  // block are masked (every tile past the last holds only keys >= kend).
  auto tile_masked = [&](int t, uint32_t gaps) { return t * kKT + kKT - 1 > lim_min || gaps != 0; };
  // Tiles whose V^T needs fix_values.
  auto tile_fixed = [&](int t, uint32_t gaps) { return t * kKT + kKT > kend || gaps != 0; };

  // Prologue: tiles 0, 1, 2 landed (and fixed), tile 0's scores and first
  // softmax part.
  TileBlocks tb1 = uniform(fetch_blocks(1)), tb2 = uniform(fetch_blocks(2)), tb3 = uniform(fetch_blocks(3)),
             tb4 = uniform(fetch_blocks(4));
  const TileBlocks tb0 = uniform(fetch_blocks(0));
  load_tile(Stage<0>(), tb0);
  load_tile(Stage<1>(), tb1);
  load_tile(Stage<2>(), tb2);
  wait_barrier<0, kNoWait>();
  // Two score buffers alternate between tiles (the loop below handles an
  // even number of tiles per pass), so neither is ever copied into the other.
  f32x16 sa[kHalves], sb[kHalves];
  float alpha[kHalves], mref[kHalves];
  bool split, rescale;
  {
    const uint32_t g0 = tile_gaps(tb0), g1 = tile_gaps(tb1), g2 = tile_gaps(tb2);
    if (tile_fixed(0, g0)) fix_values(Stage<0>(), 0, g0);
    if (tile_fixed(1, g1)) fix_values(Stage<1>(), 1, g1);
    if (tile_fixed(2, g2)) fix_values(Stage<2>(), 2, g2);
    scores(Stage<0>(), sa);
    if (tile_masked(0, g0)) mask(sa, 0, g0);
    phase1(sa, alpha, mref, split, rescale);
  }
  rescale = false;  // the accumulators are still zero
  wait_barrier<kNoWait, 0>();  // the fixed V^T of tiles 0 .. 2

  // One tile (t in stage S, its scores in `cur`): the scores of tile t+1
  // (whose blocks are tb_next) are multiplied into `nxt` while tile t's
  // probabilities are formed, then tile t's PV product runs while tile
  // t+1's first softmax part is computed.  Past the last tile the stages
  // hold stale data: tile t+1's keys then lie beyond every row's limit, its
  // mask removes all of them, and the results go unused.
  auto step = [&](auto S, int t, f32x16 (&cur)[kHalves], f32x16 (&nxt)[kHalves], TileBlocks tb_next) {
    constexpr int st = decltype(S)::value;
    const uint32_t gaps = tile_gaps(tb_next);
    if (rescale) {
#pragma unroll
      for (int hf = 0; hf < kHalves; ++hf)
#pragma unroll
        for (int dt = 0; dt < DT; ++dt) rescale_acc(o[hf][dt], alpha[hf]);
    }
#pragma unroll
    for (int hf = 0; hf < kHalves; ++hf) l_run[hf] *= alpha[hf];
    u32x4 pb[kHalves][2];
    scores(Stage<st + 1>(), nxt);
    phase2(cur, mref, pb);
    // Tile t's probabilities are formed here, beside tile t+1's score
    // products, not sunk past the mask branch below to their first use.
#pragma unroll
    for (int hf = 0; hf < kHalves; ++hf)
#pragma unroll
      for (int ks = 0; ks < 2; ++ks) asm volatile("" ::"v"(pb[hf][ks]));
    if (tile_masked(t + 1, gaps)) mask(nxt, t + 1, gaps);
    // Tile t's PV product and tile t+1's maxima share one stretch of code
    // (no branch between them), so the vector work fills the matrix
    // products' issue gaps; tile t's own split flag and reference are kept
    // for its remainder product, which follows.
    const bool split_cur = split;
    float mref_cur[kHalves];
#pragma unroll
    for (int hf = 0; hf < kHalves; ++hf) mref_cur[hf] = mref[hf];
    accumulate(S, pb);
    phase1(nxt, alpha, mref, split, rescale);
    if (split_cur) {
      u32x4 pl[kHalves][2];
      remainders(cur, mref_cur, pb, pl);
      accumulate(S, pl);
    }
  };

  // A pass covers tiles t and t+1 (in stages S and S+1) between two
  // barriers: tiles t+3 and t+4 start loading (into the stages last read as
  // tiles t-3 and t-2), then the two tiles run; at the end every load of the
  // pass has landed (it had the two tiles' time), tiles whose values need
  // it are fixed, and a barrier publishes them.  tb1 .. tb4: the blocks of
  // tiles t+1 .. t+4 (uniform).
  auto pass = [&](auto S, int t) {
    constexpr int st = decltype(S)::value;
    load_tile(Stage<st + 3>(), tb3);
    load_tile(Stage<st + 4>(), tb4);
    const TileBlocks tb5_raw = fetch_blocks(t + 5), tb6_raw = fetch_blocks(t + 6);  // used after the barrier
    step(S, t, sa, sb, tb1);
    if (t + 1 < ntiles) step(Stage<st + 1>(), t + 1, sb, sa, tb2);
    const uint32_t g3 = tile_gaps(tb3), g4 = tile_gaps(tb4);
    const bool fix3 = tile_fixed(t + 3, g3), fix4 = tile_fixed(t + 4, g4);
    if (fix3 || fix4) {
      // Every wave's loads must have landed before any wave fixes them.
      wait_barrier<0, 0>();
      if (fix3) fix_values(Stage<st + 3>(), t + 3, g3);
      if (fix4) fix_values(Stage<st + 4>(), t + 4, g4);
    }
    wait_barrier<0, 0>();
    tb1 = tb3;
    tb2 = tb4;
    tb3 = uniform(tb5_raw);
    tb4 = uniform(tb6_raw);
  };
  for (int t = 0; t < ntiles; t += 6) {
    pass(Stage<0>(), t);
    if (t + 2 >= ntiles) break;
    pass(Stage<2>(), t + 2);
    if (t + 4 >= ntiles) break;
    pass(Stage<4>(), t + 4);
  }

  // Normalise and store this lane's rows: accumulator j of tile dt is
  // dimension 32 dt + 8 (j / 4) + 4 hi + j % 4.
#pragma unroll
  for (int hf = 0; hf < kHalves; ++hf) {
    const float l_tot = sum_across_halves(l_run[hf]);
    if (row_ok[hf]) {
      const float inv = l_tot > 0.f ? 1.f / l_tot : 0.f;
      uint16_t* orow = reinterpret_cast<uint16_t*>(a.out) + (tok[hf] * Hq + hq[hf]) * D;
#pragma unroll
      for (int dt = 0; dt < DT; ++dt)
#pragma unroll
        for (int j4 = 0; j4 < 4; ++j4) {
          const int d = 32 * dt + 8 * j4 + 4 * hi;
          u32x2 pk;
          pk[0] = pack2<T>(o[hf][dt][4 * j4] * inv, o[hf][dt][4 * j4 + 1] * inv);
          pk[1] = pack2<T>(o[hf][dt][4 * j4 + 2] * inv, o[hf][dt][4 * j4 + 3] * inv);
          *reinterpret_cast<u32x2*>(orow + d) = pk;
        }
    }
  }
  // Loads of the tiles past the last may still be in flight: let them land
  // before the workgroup's LDS is reused or released.
  __builtin_amdgcn_s_waitcnt(waitcnt(0, kNoWait));
  };

  // The longer tile first.
  process(nqt - 1 - jp);
  if (jp != nqt - 1 - jp) {
    __syncthreads();  // every wave is done with the stages and the table
    process(jp);
  }
}

template <typename T, int D, int B, int G>
hipError_t launch_prefill_typed(const PrefillArgs& a, hipStream_t stream) {
  const int total = a.num_seqs * a.cache.num_kv_heads * ((a.num_qtiles + 1) / 2);
  const int grid = ((total + 7) / 8) * 8;
  hipLaunchKernelGGL((prefill_kernel<T, D, B, G>), dim3(grid), dim3(kPW * 64), 0, stream, a);
  return hipGetLastError();
}

template <typename T, int D, int B>
hipError_t prefill_g(const PrefillArgs& a, int G, hipStream_t stream) {
  switch (G) {
    case 1: return launch_prefill_typed<T, D, B, 1>(a, stream);
    case 2: return launch_prefill_typed<T, D, B, 2>(a, stream);
    case 4: return launch_prefill_typed<T, D, B, 4>(a, stream);
    case 8: return launch_prefill_typed<T, D, B, 8>(a, stream);
  }
  return hipErrorInvalidValue;
}

template <typename T, int D>
hipError_t prefill_b(const PrefillArgs& a, int G, hipStream_t stream) {
  switch (a.cache.block_size) {
    case 16: return prefill_g<T, D, 16>(a, G, stream);
    case 32: return prefill_g<T, D, 32>(a, G, stream);
  }
  return hipErrorInvalidValue;
}

template <typename T>
hipError_t prefill_d(const PrefillArgs& a, int G, hipStream_t stream) {
  switch (a.cache.head_dim) {
    case 64: return prefill_b<T, 64>(a, G, stream);
    case 128: return prefill_b<T, 128>(a, G, stream);
  }
  return hipErrorInvalidValue;
}

}  // namespace

int prefill_positions_per_tile(int group) { return kRows / group; }

hipError_t launch_prefill(const PrefillArgs& a, hipStream_t stream) {
  if (a.num_seqs == 0 || a.num_qtiles == 0) return hipSuccess;
  const int G = a.num_heads / a.cache.num_kv_heads;
  switch (a.cache.dtype) {
    case DType::kF16: return prefill_d<f16_t>(a, G, stream);
    case DType::kBF16: return prefill_d<bf16_t>(a, G, stream);
    case DType::kFP8: return launch_prefill_fp8(a, stream);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace pa
