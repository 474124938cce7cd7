// Paged decode attention for gfx950 (MI355X) on the matrix cores.
//
// Sources: [P1] "大模型推理内存优化从 KV Cache 分页到连续批处理的工程实践",
// sections "PagedAttention 的 CUDA Kernel 实现" (look up each logical block's
// physical ID in the block table, then read the block's contiguous K/V; the
// table sits on chip; in-block reads coalesce; the next block is fetched
// while the current one is used) and "工程边界与架构取舍" (decode is bound by
// reading the whole KV cache for one token).
//
// Work decomposition.  One workgroup of kNW wavefronts handles one
// (partition, KV head, sequence): a partition is `partition` consecutive
// tokens of the sequence (a multiple of the block size).  All G query heads
// that share the KV head are served together, so every K/V byte is read from
// HBM once.  The partition is cut into steps of 32 tokens, dealt to the waves
// round-robin (rotated so that the partition's last step falls to wave 0);
// each wave keeps its next steps' K/V loads in flight (a register ring)
// while it computes the current one.
//
// Per step, with the G heads as the 16-wide N side of v_mfma_f32_16x16x*
// (heads G..15 are zero columns):
//   S[token][head]    = K . Q^T     two 16-token halves; K rows are plain
//                                   16-byte loads of the key tile
//   online softmax per head (running max and sum per lane, rescale of the
//   accumulators when the max grows)
//   O^T[dim][head]   += V^T . P^T   V^T comes straight from the transposed
//                                   value tile (8 tokens of one dimension per
//                                   lane), P^T straight from the lane's own
//                                   logits
// The 16 K rows of the first half are tokens 8(r/4) + r%4 and of the second
// half 8(r/4) + 4 + r%4 (r = row): the logits that land in lane (head r,
// group g) are then exactly tokens 8g .. 8g+7 of the step, which is the
// k-slice the same lane holds in the PV product, and the one its value load
// fetches; nothing moves between lanes except the per-head maximum.
//
// Operand layouts (lane l, r = l % 16, g = l / 16, j = 0..3):
//   16x16x32 f16/bf16: A[m][k] m = r, k = 8g + e (e < 8); B[k][n] k = 8g + e, n = r
//   16x16x4 f32:       A[m][k] m = r, k = g;             B[k][n] k = g, n = r
//   C[m][n]: m = 4g + j, n = r
// FP8 codes are converted exactly to f16 (v_cvt_scalef32_pk_f16_fp8, two
// codes per instruction) on the way into the f16 products; bf16 probabilities enter the PV product as a bf16 hi + lo
// pair (two products), f16 ones rounded to f16 with the normaliser summing
// the same rounded values.
//
// A sequence that fits one partition is normalised and written directly.
// Longer sequences write (max, sum, unnormalised o) per partition to the
// workspace and a second kernel merges them:
//   M = max_p m_p,  out = sum_p 2^(m_p - M) o_p / sum_p 2^(m_p - M) l_p.
#include <math.h>

#include <type_traits>

#include <hip/hip_ext.h>

#include "pa_common.h"
#include "pa_launch.h"

namespace pa {

namespace {

constexpr int kStep = 32;  // tokens per step

typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));

// Per storage type: CE elements per 16-byte K load, KE k-elements per lane
// per product, VW 32-bit words of V^T per lane per 16-dim tile and step (8
// tokens), NBUF steps in the register ring.
template <typename T>
struct Dec;
template <>
struct Dec<f16_t> {
  typedef f16_t Q;
  static constexpr int CE = 8, KE = 8, VW = 4, NBUF = 2;
};
template <>
struct Dec<bf16_t> {
  typedef bf16_t Q;
  static constexpr int CE = 8, KE = 8, VW = 4, NBUF = 2;
};
template <>
struct Dec<float> {
  typedef float Q;
  static constexpr int CE = 4, KE = 1, VW = 8, NBUF = 1;
};
template <>
struct Dec<fp8_t> {
  typedef f16_t Q;
  static constexpr int CE = 16, KE = 8, VW = 2, NBUF = 2;
};

__device__ __forceinline__ f32x4 mma_f16(const u32x4& a, const u32x4& b, const f32x4& c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8, a), __builtin_bit_cast(f16x8, b), c, 0, 0, 0);
}
__device__ __forceinline__ f32x4 mma_bf16(const u32x4& a, const u32x4& b, const f32x4& c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a), __builtin_bit_cast(bf16x8, b), c, 0, 0,
                                                 0);
}
__device__ __forceinline__ f32x4 mma_f32(float a, float b, const f32x4& c) {
  return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
}

// Four E4M3 codes (one word) -> two f16x2 words holding their values
// (bytes 0, 1 in lo, 2, 3 in hi, low byte in the low half).  Every E4M3 value
// (magnitudes 2^-9 .. 448) is an f16 normal number, so the conversion at
// scale 1 is exact.
__device__ __forceinline__ void widen4(uint32_t w, uint32_t& lo, uint32_t& hi) {
  lo = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(w, 1.0f, false));
  hi = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(w, 1.0f, true));
}

// Two floats -> packed pair in the operand type, round to nearest even.
__device__ __forceinline__ uint32_t pack_f16(float a, float b) { return pack_f16x2(a, b); }
__device__ __forceinline__ uint32_t pack_bf16(float a, float b) { return pack_bf16x2(a, b); }

// LDS of one workgroup of NW waves: the partition's block-table slice, and
// per wave its partial output [G][D], maximum and sum per head for the
// final merge.
struct SmemLayout {
  int bt_off, o_off, m_off, l_off, bytes;
};

__host__ __device__ inline SmemLayout smem_layout(int partition, int B, int G, int D, int NW) {
  SmemLayout s;
  int off = 0;
  s.bt_off = off;
  off += ((partition / B) * 4 + 15) & ~15;
  s.o_off = off;
  off += NW * G * D * 4;
  s.m_off = off;
  off += NW * G * 4;
  s.l_off = off;
  off += NW * G * 4;
  s.bytes = off;
  return s;
}

// Combine the per-partition partials of one (sequence, query head, dim):
//   M = max_p m_p,  out = sum_p 2^(m_p - M) o_p / sum_p 2^(m_p - M) l_p.
// Every one of the call's partitions is fetched (empty ones carry
// m = -inf and contribute nothing), in batches of kMergeBatch whose loads are
// all issued before any is used; batches combine with a running rescale.
constexpr int kMergeBatch = 16;

// Lazy rescale threshold of the online softmax (log2 units).
constexpr float kLazy = 8.f;

// np partitions of the sequence are merged for dims d .. d+3 of query head
// hq; rows are num_partitions apart.
template <int D>
__device__ __forceinline__ f32x4 merge_partials(const DecodeArgs& a, int s, int hq, int d, int np) {
  const int64_t row0 = ((int64_t)s * a.num_heads + hq) * a.num_partitions;
  float M = -INFINITY, den = 0.f;
  f32x4 num = {0.f, 0.f, 0.f, 0.f};
  for (int p0 = 0; p0 < np; p0 += kMergeBatch) {
    float mv[kMergeBatch], lv[kMergeBatch];
    f32x4 ov[kMergeBatch];
#pragma unroll
    for (int i = 0; i < kMergeBatch; ++i) {
      const bool ok = p0 + i < np;
      const int64_t row = row0 + p0 + i;
      mv[i] = ok ? a.ws_m[row] : -INFINITY;
      lv[i] = ok ? a.ws_l[row] : 0.f;
      ov[i] = ok ? *reinterpret_cast<const f32x4*>(a.ws_o + row * D + d) : f32x4{0.f, 0.f, 0.f, 0.f};
    }
    float Mb = M;
#pragma unroll
    for (int i = 0; i < kMergeBatch; ++i) Mb = fmaxf(Mb, mv[i]);
    if (Mb == -INFINITY) continue;
    if (M != -INFINITY) {
      const float f = fast_exp2(M - Mb);
#pragma unroll
      for (int k = 0; k < 4; ++k) num[k] *= f;
      den *= f;
    }
#pragma unroll
    for (int i = 0; i < kMergeBatch; ++i) {
      // Absent partitions are skipped by select: their l and o are stale.
      const bool live = mv[i] != -INFINITY;
      const float wgt = live ? fast_exp2(mv[i] - Mb) : 0.f;
#pragma unroll
      for (int k = 0; k < 4; ++k) num[k] = live ? fmaf(wgt, ov[i][k], num[k]) : num[k];
      den = live ? fmaf(wgt, lv[i], den) : den;
    }
    M = Mb;
  }
  f32x4 r = {0.f, 0.f, 0.f, 0.f};
  if (den > 0.f) {
#pragma unroll
    for (int k = 0; k < 4; ++k) r[k] = num[k] / den;
  }
  return r;
}

// Four consecutive output elements from float32.
template <typename T>
__device__ __forceinline__ void store4(T* p, const f32x4& v);
template <>
__device__ __forceinline__ void store4<float>(float* p, const f32x4& v) {
  *reinterpret_cast<f32x4*>(p) = v;
}
template <>
__device__ __forceinline__ void store4<f16_t>(f16_t* p, const f32x4& v) {
  *reinterpret_cast<u32x2*>(p) = u32x2{pack_f16x2(v[0], v[1]), pack_f16x2(v[2], v[3])};
}
template <>
__device__ __forceinline__ void store4<bf16_t>(bf16_t* p, const f32x4& v) {
  *reinterpret_cast<u32x2*>(p) = u32x2{pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3])};
}

// 8-wave workgroups (one per compute unit) keep two steps in flight per
// wave at 2 waves per SIMD; 4-wave workgroups of 16-bit types keep one and
// fit 3 waves per SIMD, i.e. three workgroups per compute unit, which serves
// batches of many short or mixed-length sequences better (FP8 steps are
// small enough to keep two either way; float32 is a correctness path).
template <int kNW, typename T>
struct WaveCfg {
  static constexpr bool kThree = kNW == 4 && Elem<T>::kBytes <= 2;
  static constexpr int kWavesPerEU = kThree ? 3 : 2;
  static constexpr int kRing = kThree && Elem<T>::kBytes == 2 ? 1 : Dec<T>::NBUF;
};

template <int kNW, typename T, int D, int B, int G>
__global__ void __launch_bounds__(kNW * 64) __attribute__((amdgpu_waves_per_eu(WaveCfg<kNW, T>::kWavesPerEU)))
decode_partition_kernel(DecodeArgs a) {
  using QT = typename Dec<T>::Q;
  constexpr bool kFp8 = std::is_same<T, fp8_t>::value;
  constexpr bool kF32 = std::is_same<T, float>::value;
  constexpr bool kBf16 = std::is_same<T, bf16_t>::value;
  constexpr int CE = Dec<T>::CE, KE = Dec<T>::KE, VW = Dec<T>::VW;
  constexpr int NBUF = WaveCfg<kNW, T>::kRing;
  constexpr int NLK = D / (4 * CE);                 // K loads per lane per 16-token half
  constexpr int KC = key_chunk<T>();                // elements per 64-byte key chunk (= 4 * CE)
  static_assert(KC == 4 * CE, "one key load instruction covers one 64-byte chunk of 16 rows");
  constexpr int NSUB = CE / KE;                     // products per K load
  constexpr int QW = CE * (int)sizeof(QT) / 16;     // 16-byte query pieces per K load
  constexpr int NDT = D / 16;                       // 16-dim tiles of the PV product
  constexpr int NT = kNW * 64;
  static_assert(NLK >= 1 && QW >= 1 && B % 8 == 0 && G <= 16, "unsupported shape");

  extern __shared__ __align__(16) unsigned char smem[];
  // 1-D grid, (sequence, KV head) fastest and partition slowest, last
  // partition first: workgroup ids are dealt to the 8 XCDs round-robin, so
  // each XCD gets whole (sequence, KV head) pairs and short sequences spread
  // over all XCDs; the late partitions exist only for long sequences, and
  // starting them first keeps the longest chains of work off the tail.
  // With a plan, workgroup i serves KV head i % H_kv of the listed unit
  // i / H_kv (a sequence's partition), so the heads of a unit spread over
  // the XCDs.
  int s, g, part;
  if (a.work) {
    const int unit = blockIdx.x / a.cache.num_kv_heads;
    g = blockIdx.x % a.cache.num_kv_heads;
    const int wi = unit < a.num_work ? a.work[unit] : -1;
    if (wi < 0 || wi >= a.num_seqs * a.num_partitions) return;  // not a unit of this call
    s = wi / a.num_partitions;
    part = wi % a.num_partitions;
  } else if (a.device_plan) {
    // The plan computed on the device (a batch of at most 64 sequences, one
    // length per lane; every wave computes the same): workgroup i serves KV
    // head i % H_kv of the unit of rank i / H_kv in the order full
    // partitions first (partition-major), then each sequence's last, partial
    // one by decreasing size in eighths of a partition (and the partition 0
    // of empty sequences, which writes their zeros).  Ranks past the last
    // unit exit: they come last in the grid, behind all the work.
    const int lane = threadIdx.x & 63;
    if ((int)(blockIdx.x / a.cache.num_kv_heads) >= a.num_seqs) {
      // Every sequence has at least one unit, so ranks below the batch size
      // always find one.  Past that, a bound on the number of units from the
      // lengths read through the scalar cache (the sum of ceil(max(L, 1) / P)
      // is at most the sum of max(L, 1), plus n (P - 1), over P) lets most
      // workgroups past the end of the work leave without a vector load,
      // which would queue behind the key and value streams of the
      // workgroups still running (about 2 us on a 64-sequence batch whose
      // grid is two-thirds such workgroups).
      const int rank = (int)(blockIdx.x / a.cache.num_kv_heads);
      const int n = a.num_seqs;
      int64_t tot = (int64_t)n * (a.partition - 1);
      auto len1 = [&](int v) -> int64_t {
        v = v > a.max_seq_len ? a.max_seq_len : v;
        return v < 1 ? 1 : v;
      };
      int i = 0;
      for (; i + 16 <= n; i += 16) {
#pragma unroll
        for (int j = 0; j < 16; ++j) tot += len1(a.seq_lens[i + j]);
      }
      for (; i < n; ++i) tot += len1(a.seq_lens[i]);
      if (tot < (int64_t)(rank + 1) * a.partition) return;  // rank >= floor(tot / P) >= the unit count
    }
    int Ls = lane < a.num_seqs ? a.seq_lens[lane] : -1;
    Ls = Ls < 0 ? (lane < a.num_seqs ? 0 : -1) : (Ls > a.max_seq_len ? a.max_seq_len : Ls);
    const int full = Ls > 0 ? Ls / a.partition : 0;
    const int rem = Ls >= 0 ? Ls - full * a.partition : 0;
    const bool partial = Ls == 0 || rem > 0;
    int u = (int)(blockIdx.x / a.cache.num_kv_heads);
    g = blockIdx.x % a.cache.num_kv_heads;
    s = -1;
    part = 0;
    // The unit of rank u among the lanes set in m: the u-th set lane.
    auto pick = [&](uint64_t m) -> int {
      const int below = __builtin_amdgcn_mbcnt_hi((uint32_t)(m >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)m, 0u));
      const uint64_t hit = __ballot(((m >> lane) & 1u) && below == u);
      return hit ? (int)__builtin_ctzll(hit) : -1;
    };
    for (int q = 0;; ++q) {
      const uint64_t m = __ballot(full > q);
      if (!m) break;
      const int c = __builtin_popcountll(m);
      if (u < c) {
        s = pick(m);
        part = q;
        break;
      }
      u -= c;
    }
    if (s < 0) {
      for (int b = 7; b >= 0; --b) {
        const uint64_t m = __ballot(partial && (rem * 8) / a.partition == b);
        const int c = __builtin_popcountll(m);
        if (u < c) {
          s = pick(m);
          part = __builtin_amdgcn_readlane(full, s);
          break;
        }
        u -= c;
      }
    }
    s = __builtin_amdgcn_readfirstlane(s);
    part = __builtin_amdgcn_readfirstlane(part);
    if (s < 0) return;  // past the last unit of this call
  } else {
    const int sg = blockIdx.x % (a.num_seqs * a.cache.num_kv_heads);
    part = a.num_partitions - 1 - (int)(blockIdx.x / (a.num_seqs * a.cache.num_kv_heads));
    g = sg % a.cache.num_kv_heads;
    s = sg / a.cache.num_kv_heads;
  }
  const int P = a.partition;
  const int nbp = P / B;
  const SmemLayout lay = smem_layout(P, B, G, D, kNW);

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int w = tid >> 6;
  const int r = lane & 15;   // MFMA row / column index of this lane
  const int grp = lane >> 4; // MFMA k group of this lane
  const int Hkv = a.cache.num_kv_heads;
  const int Hq = a.num_heads;
  const int tok0 = part * P;
  const int blk0 = tok0 / B;

  // The first NT entries of the partition's table slice are fetched without
  // waiting for seq_len (they lie inside the table row either way), so the
  // two loads overlap.
  int bt_id = -1;
  if (tid < nbp && blk0 + tid < a.max_blocks) bt_id = a.block_tables[(int64_t)s * a.max_blocks + blk0 + tid];
  int L = a.seq_lens[s];
  L = L < 0 ? 0 : (L > a.max_seq_len ? a.max_seq_len : L);
  const bool direct = L <= P;
  if (part > 0 && tok0 >= L) {
    // An empty partition of a split sequence marks its partials as absent
    // (m = -inf) so the merge can fetch every partition unconditionally.
    if (!direct && tid < G) a.ws_m[((int64_t)s * Hq + g * G + tid) * a.num_partitions + part] = -INFINITY;
    return;
  }
  const int ntok = min(P, L - tok0) > 0 ? min(P, L - tok0) : 0;

  int* s_bt = reinterpret_cast<int*>(smem + lay.bt_off);
  float* s_o = reinterpret_cast<float*>(smem + lay.o_off);
  float* s_m = reinterpret_cast<float*>(smem + lay.m_off);
  float* s_l = reinterpret_cast<float*>(smem + lay.l_off);

  // 1. Block-table slice -> LDS.  Entries outside the pool become -1.
  if (tid < nbp) s_bt[tid] = (bt_id < 0 || bt_id >= a.cache.num_blocks) ? -1 : bt_id;
  for (int j = tid + NT; j < nbp; j += NT) {
    const int id = blk0 + j < a.max_blocks ? a.block_tables[(int64_t)s * a.max_blocks + blk0 + j] : -1;
    s_bt[j] = (id < 0 || id >= a.cache.num_blocks) ? -1 : id;
  }

  // 2. Query operand: lane (head r, group grp) holds, for K load ls, the
  // query elements 4*CE*ls + CE*grp .. + CE-1 of head r (zero for r >= G).
  u32x4 qw[NLK][QW];
  {
    const QT* qrow = reinterpret_cast<const QT*>(a.query) + ((int64_t)s * Hq + g * G + (r < G ? r : 0)) * D;
#pragma unroll
    for (int ls = 0; ls < NLK; ++ls)
#pragma unroll
      for (int q = 0; q < QW; ++q)
        qw[ls][q] = r < G ? *reinterpret_cast<const u32x4*>(qrow + 4 * CE * ls + CE * grp + q * (16 / (int)sizeof(QT)))
                          : u32x4{0, 0, 0, 0};
  }
  __syncthreads();  // table slice visible

  // Steps go to the waves round-robin, rotated so that the partition's last
  // step (which holds a sequence's newest position) falls to wave 0, the
  // first wave on its SIMD: the first wave of each SIMD issues ahead of the
  // second (on the benchmark layer waves 0-3 finish their steps about 9 us
  // before waves 4-7), so the appending wave's wait below costs nothing.
  const int nsteps = (ntok + kStep - 1) / kStep;
  const int rot = nsteps > 0 ? (kNW - (nsteps - 1) % kNW) % kNW : 0;
  const int first = (w + kNW - rot) % kNW;  // this wave's steps: first, first + kNW, ...

  // Fused append: in the workgroup whose partition holds the sequence's last
  // position, wave 0 (which processes the partition's last step) writes this
  // step's token (KV head g) into its slot, exactly as the scatter does.
  // The key row is stored now, and the wave waits until those stores have
  // completed before it issues any load; no other wave reads that token's
  // block (the last block belongs to the last step only), so the other
  // waves start streaming at once.  The value row is a column of the
  // transposed value tile, i.e. head_dim scattered element stores; instead
  // the wave patches it into the block's value tile once it has loaded that
  // tile for its last step, and writes the tile back whole (every other slot
  // bit for bit as loaded), which the memory system takes as full lines.
  using S = typename Src<T>::type;
  const int jnew = ntok > 0 ? (ntok - 1) / B : 0;  // the new token's block in the table slice
  const bool apnd = a.new_key != nullptr && ntok > 0 && tok0 + ntok == L && w == 0 && s_bt[jnew] >= 0;
  uint32_t nvb[NDT];  // the new value's element for dims 16 dd + r (storage bits)
  if (a.new_key != nullptr && ntok > 0 && tok0 + ntok == L && w == 0) {
    constexpr int VS = vec16<S>();
    constexpr int NCH = D / VS;  // 16-byte source chunks per row
    static_assert(NCH <= 64, "one wave writes the key row");
    const int pb = s_bt[jnew];
    const int off = (L - 1) % B;
    const S* vrow = reinterpret_cast<const S*>(a.new_value) + ((int64_t)s * Hkv + g) * D;
#pragma unroll
    for (int dd = 0; dd < NDT; ++dd) {
      const S x = vrow[16 * dd + r];
      if constexpr (kFp8) {
        nvb[dd] = f32_to_e4m3((float)x / a.cache.v_scale);
      } else if constexpr (kF32) {
        nvb[dd] = __float_as_uint(x);
      } else {
        nvb[dd] = __builtin_bit_cast(uint16_t, x);
      }
    }
    if (lane < NCH && pb >= 0) {
      const S* src = reinterpret_cast<const S*>(a.new_key) + ((int64_t)s * Hkv + g) * D + lane * VS;
      store_kv_chunk<T>(reinterpret_cast<T*>(a.cache.key_cache), reinterpret_cast<T*>(a.cache.value_cache), 0, pb,
                        off, g, lane, VS, Hkv, D, B, *reinterpret_cast<const u32x4*>(src), a.cache.k_scale,
                        a.cache.v_scale);
    }
    if (lane == 0 && g == 0) a.slots[s] = pb >= 0 ? (int64_t)pb * B + off : -1;
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  }

  const int64_t blk_stride = (int64_t)Hkv * B * D;
  const T* kbase = reinterpret_cast<const T*>(a.cache.key_cache) + (int64_t)g * B * D;
  const T* vbase = reinterpret_cast<const T*>(a.cache.value_cache) + (int64_t)g * D * B;
  // FP8: the widened K values are the codes' values; the pool scale joins
  // the logit scale.
  const float qscale = kFp8 ? a.scale * kLog2e * a.cache.k_scale : a.scale * kLog2e;

  struct Buf {
    u32x4 k[2][NLK];        // K rows of the two 16-token halves
    uint32_t v[NDT][VW];    // V^T: 8 tokens of dim 16*dd + r
  };
  auto load = [&](Buf& b, int st) {
    const int stok = st * kStep;
#pragma unroll
    for (int c = 0; c < 2; ++c) {
      const int t = stok + 8 * (r >> 2) + 4 * c + (r & 3);
      const int j = t / B;
      const int pb = (t < ntok && j < nbp) ? s_bt[j] : -1;
      // Key load ls reads 64-byte chunk ls of the 16 rows: rows 8(r/4) +
      // 4c .. +3 are adjacent in a chunk, so the wave reads whole 128-byte
      // lines, each once.  K and V are streamed with non-temporal loads,
      // except FP8 keys: ordinary loads measured faster there (28.4 against
      // 29.8 us on the benchmark layer).
      const T* src = kbase + (int64_t)pb * blk_stride + (t % B) * KC + CE * grp;
#pragma unroll
      for (int ls = 0; ls < NLK; ++ls) {
        const u32x4* p = reinterpret_cast<const u32x4*>(src + (int64_t)ls * B * KC);
        if constexpr (kFp8)
          b.k[c][ls] = pb >= 0 ? *p : u32x4{0, 0, 0, 0};
        else
          b.k[c][ls] = pb >= 0 ? __builtin_nontemporal_load(p) : u32x4{0, 0, 0, 0};
      }
    }
    const int t0 = stok + 8 * grp;
    const int j = t0 / B;
    // The appending wave loads the new token's whole block in its last step
    // (past the sequence's end too): it writes that value tile back.
    const bool whole = apnd && st == nsteps - 1 && j == jnew;
    const int pb = ((t0 < ntok || whole) && j < nbp) ? s_bt[j] : -1;
    const T* vsrc = vbase + (int64_t)pb * blk_stride + r * B + (t0 % B);
#pragma unroll
    for (int dd = 0; dd < NDT; ++dd) {
      const T* p = vsrc + dd * 16 * B;
      if constexpr (VW == 2) {
        const u32x2 x = pb >= 0 ? __builtin_nontemporal_load(reinterpret_cast<const u32x2*>(p)) : u32x2{0, 0};
        b.v[dd][0] = x[0], b.v[dd][1] = x[1];
      } else {
#pragma unroll
        for (int h = 0; h < VW / 4; ++h) {
          const u32x4 x = pb >= 0 ? __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p) + h) : u32x4{0, 0, 0, 0};
          b.v[dd][4 * h] = x[0], b.v[dd][4 * h + 1] = x[1], b.v[dd][4 * h + 2] = x[2], b.v[dd][4 * h + 3] = x[3];
        }
      }
    }
  };

  f32x4 o[NDT];
#pragma unroll
  for (int dd = 0; dd < NDT; ++dd) o[dd] = f32x4{0.f, 0.f, 0.f, 0.f};
  float m_run = -INFINITY, l_run = 0.f;

  auto compute = [&](Buf& b, int st) {
    // S = K . Q^T for the two halves: lane (head r, group grp) receives the
    // logits of tokens 8*grp + 4*c + jj.
    f32x4 sc[2];
#pragma unroll
    for (int c = 0; c < 2; ++c) {
      f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int ls = 0; ls < NLK; ++ls) {
        if constexpr (kF32) {
#pragma unroll
          for (int sub = 0; sub < 4; ++sub) {
            const uint32_t kv = b.k[c][ls][sub], qv = qw[ls][0][sub];
            acc = mma_f32(__uint_as_float(kv), __uint_as_float(qv), acc);
          }
        } else if constexpr (kFp8) {
#pragma unroll
          for (int sub = 0; sub < NSUB; ++sub) {
            u32x4 ka;
            uint32_t x0, x1, x2, x3;
            widen4(b.k[c][ls][2 * sub], x0, x1);
            widen4(b.k[c][ls][2 * sub + 1], x2, x3);
            ka = u32x4{x0, x1, x2, x3};
            acc = mma_f16(ka, qw[ls][sub], acc);
          }
        } else if constexpr (kBf16) {
          acc = mma_bf16(b.k[c][ls], qw[ls][0], acc);
        } else {
          acc = mma_f16(b.k[c][ls], qw[ls][0], acc);
        }
      }
      sc[c] = acc;
    }

    // Online softmax.  Tokens of this lane: 8*grp + e, e = 4*c + jj.
    const int t0 = st * kStep + 8 * grp;
    const int jb = t0 / B;
    const bool blk_ok = t0 < ntok && jb < nbp && s_bt[jb] >= 0;
    const int nvalid = blk_ok ? min(8, ntok - t0) : 0;
    float z[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) z[e] = e < nvalid ? sc[e / 4][e % 4] * qscale : -INFINITY;
    float mx = z[0];
#pragma unroll
    for (int e = 1; e < 8; ++e) mx = fmaxf(mx, z[e]);
    mx = max_across_rows(mx);  // the four k groups of head r
    // The reference maximum moves only when the step exceeds it by more
    // than kLazy (log2 units), so probabilities stay below 2^kLazy and the
    // accumulator rescale is rare; the final division by the sum cancels
    // whichever reference was used.
    const bool move = mx > m_run + kLazy;
    const float m_new = move ? mx : m_run;
    const float alpha = move ? fast_exp2(m_run - m_new) : 1.f;  // 0 from -inf
    float p[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) p[e] = z[e] == -INFINITY ? 0.f : fast_exp2(z[e] - m_new);
    m_run = m_new;
    if (__any(move)) {
#pragma unroll
      for (int dd = 0; dd < NDT; ++dd) o[dd] *= alpha;
    }

    // The appending wave's last step: put the new token's value into the
    // loaded value tile of its block and store the tile's pieces back.
    if (apnd && st == nsteps - 1 && t0 / B == jnew) {
      const int e = (ntok - 1) - t0;  // the new token's place in this lane's 8 tokens, if 0..7
      T* vdst = reinterpret_cast<T*>(a.cache.value_cache) + (int64_t)g * D * B +
                (int64_t)s_bt[jnew] * blk_stride + r * B + (t0 % B);
#pragma unroll
      for (int dd = 0; dd < NDT; ++dd) {
        // Selects over the words (a runtime index into the register array
        // would move it to scratch memory).
#pragma unroll
        for (int q = 0; q < VW; ++q) {
          if constexpr (VW == 8) {
            b.v[dd][q] = q == e ? nvb[dd] : b.v[dd][q];
          } else if constexpr (VW == 4) {
            const uint32_t sh = 16u * (uint32_t)(e & 1);
            const uint32_t put = (b.v[dd][q] & ~(0xffffu << sh)) | (nvb[dd] << sh);
            b.v[dd][q] = (e >= 0 && q == (e >> 1)) ? put : b.v[dd][q];
          } else {
            const uint32_t sh = 8u * (uint32_t)(e & 3);
            const uint32_t put = (b.v[dd][q] & ~(0xffu << sh)) | (nvb[dd] << sh);
            b.v[dd][q] = (e >= 0 && q == (e >> 2)) ? put : b.v[dd][q];
          }
        }
        T* p = vdst + dd * 16 * B;
        if constexpr (VW == 8) {
          reinterpret_cast<u32x4*>(p)[0] = u32x4{b.v[dd][0], b.v[dd][1], b.v[dd][2], b.v[dd][3]};
          reinterpret_cast<u32x4*>(p)[1] = u32x4{b.v[dd][4], b.v[dd][5], b.v[dd][6], b.v[dd][7]};
        } else if constexpr (VW == 4) {
          *reinterpret_cast<u32x4*>(p) = u32x4{b.v[dd][0], b.v[dd][1], b.v[dd][2], b.v[dd][3]};
        } else {
          *reinterpret_cast<u32x2*>(p) = u32x2{b.v[dd][0], b.v[dd][1]};
        }
      }
    }

    // Value tokens past the end (or in a block outside the pool) are zeroed:
    // their probabilities are 0 and 0 * NaN would poison the sums.
    if (nvalid < 8) {
#pragma unroll
      for (int q = 0; q < VW; ++q) {
        uint32_t keep;
        if constexpr (VW == 8) {
          keep = q < nvalid ? 0xffffffffu : 0u;
        } else if constexpr (VW == 4) {
          keep = 2 * q >= nvalid ? 0u : (2 * q + 1 >= nvalid ? 0xffffu : 0xffffffffu);
        } else {
          keep = 0;
#pragma unroll
          for (int bb = 0; bb < 4; ++bb) keep |= (4 * q + bb < nvalid ? 0xffu : 0u) << (8 * bb);
        }
#pragma unroll
        for (int dd = 0; dd < NDT; ++dd) b.v[dd][q] &= keep;
      }
    }

    // O^T += V^T . P^T
    float lstep = 0.f;
    if constexpr (kF32) {
#pragma unroll
      for (int e = 0; e < 8; ++e) lstep += p[e];
#pragma unroll
      for (int dd = 0; dd < NDT; ++dd)
#pragma unroll
        for (int e = 0; e < 8; ++e) o[dd] = mma_f32(__uint_as_float(b.v[dd][e]), p[e], o[dd]);
    } else if constexpr (kBf16) {
      // p = hi + lo, both bf16: the product keeps ~16 bits of p.
      uint32_t ph[4], pl[4];
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const float a0 = p[2 * q], a1 = p[2 * q + 1];
        const uint32_t h = pack_bf16(a0, a1);
        ph[q] = h;
        pl[q] = pack_bf16(a0 - bf16_lo(h), a1 - bf16_hi(h));
        lstep += a0 + a1;
      }
      const u32x4 pa = {ph[0], ph[1], ph[2], ph[3]}, pb = {pl[0], pl[1], pl[2], pl[3]};
#pragma unroll
      for (int dd = 0; dd < NDT; ++dd) {
        const u32x4 va = {b.v[dd][0], b.v[dd][1], b.v[dd][2], b.v[dd][3]};
        o[dd] = mma_bf16(va, pa, o[dd]);
        o[dd] = mma_bf16(va, pb, o[dd]);
      }
    } else {
      // f16 (and widened FP8): p rounded to f16; the normaliser sums the
      // same rounded values.
      uint32_t ph[4];
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const uint32_t h = pack_f16(p[2 * q], p[2 * q + 1]);
        ph[q] = h;
        lstep += f16_lo(h) + f16_hi(h);
      }
      const u32x4 pa = {ph[0], ph[1], ph[2], ph[3]};
#pragma unroll
      for (int dd = 0; dd < NDT; ++dd) {
        u32x4 va;
        if constexpr (kFp8) {
          uint32_t x0, x1, x2, x3;
          widen4(b.v[dd][0], x0, x1);
          widen4(b.v[dd][1], x2, x3);
          va = u32x4{x0, x1, x2, x3};
        } else {
          va = u32x4{b.v[dd][0], b.v[dd][1], b.v[dd][2], b.v[dd][3]};
        }
        o[dd] = mma_f16(va, pa, o[dd]);
      }
    }
    l_run = l_run * alpha + lstep;
  };

  // 3. The wave's steps first, first + kNW, ..., NBUF of them in flight,
  // walked from a starting point that depends on the sequence and the
  // partition.  When sequences occupy contiguous runs of the pool, streams
  // that start at the same offset of their runs and advance in lockstep
  // meet the same memory channels at the same time (a contiguous layout ran
  // 21 % slower than a random one on the benchmark layer); staggered starts
  // make the walk indifferent to how blocks are laid out.
  const int nmine = nsteps > first ? (nsteps - first + kNW - 1) / kNW : 0;
  const int off = nmine > 1 ? (5 * s + 3 * part) % nmine : 0;
  auto step_of = [&](int i) {
    const int k = i + off;
    return first + (k >= nmine ? k - nmine : k) * kNW;
  };
  Buf buf[NBUF];
#pragma unroll
  for (int i = 0; i < NBUF; ++i)
    if (i < nmine) load(buf[i], step_of(i));
  for (int i0 = 0; i0 < nmine; i0 += NBUF) {
#pragma unroll
    for (int bi = 0; bi < NBUF; ++bi) {
      const int i = i0 + bi;
      if (i < nmine) {
        compute(buf[bi], step_of(i));
        if (i + NBUF < nmine) load(buf[bi], step_of(i + NBUF));
      }
    }
  }

  // 4. The wave's partials -> LDS, then merge the waves.  Lane (head r,
  // group grp) holds dims 16*dd + 4*grp + jj; the four groups' sums add up.
  const float l_tot = sum_across_rows(l_run);
  if (r < G) {
#pragma unroll
    for (int dd = 0; dd < NDT; ++dd)
#pragma unroll
      for (int jj = 0; jj < 4; ++jj) s_o[(w * G + r) * D + 16 * dd + 4 * grp + jj] = o[dd][jj];
    if (grp == 0) {
      s_m[w * G + r] = m_run;
      s_l[w * G + r] = l_tot;
    }
  }
  __syncthreads();

  // FP8: the widened V values are the codes' values.
  const float vfac = kFp8 ? a.cache.v_scale : 1.f;
  for (int idx = tid; idx < G * D; idx += NT) {
    const int h = idx / D;
    const int d = idx % D;
    float Mx = -INFINITY;
#pragma unroll
    for (int ww = 0; ww < kNW; ++ww) Mx = fmaxf(Mx, s_m[ww * G + h]);
    float acc = 0.f, l = 0.f;
    if (Mx != -INFINITY) {
#pragma unroll
      for (int ww = 0; ww < kNW; ++ww) {
        const float mw = s_m[ww * G + h];
        const float f = mw == -INFINITY ? 0.f : fast_exp2(mw - Mx);
        acc = fmaf(f, s_o[(ww * G + h) * D + d], acc);
        l = fmaf(f, s_l[ww * G + h], l);
      }
    }
    acc *= vfac;
    const int hq = g * G + h;
    if (direct) {
      QT* out = reinterpret_cast<QT*>(a.out) + ((int64_t)s * Hq + hq) * D + d;
      store_elem<QT>(out, l > 0.f ? acc / l : 0.f);
    } else {
      const int64_t row = ((int64_t)s * Hq + hq) * a.num_partitions + part;
      a.ws_o[row * D + d] = acc;
      if (d == 0) {
        a.ws_m[row] = Mx;
        a.ws_l[row] = l;
      }
    }
  }
}

// Merge kernel for sequences longer than one partition.  Fused variants (the
// last partition workgroup of a sequence and KV head merging, after either
// an agent-scope release/acquire or device-coherent partial stores and an
// arrival counter) were correct but no faster: every workgroup then waits
// for its partials to reach memory.  grid (num_kv_heads, num_seqs), one
// thread per 4 dims of each of the G query heads of the KV head.
template <typename T, int D, int G>
__global__ void __launch_bounds__(G * D / 4) decode_reduce_kernel(DecodeArgs a) {
  const int s = blockIdx.y;
  const int hq = blockIdx.x * G + (int)threadIdx.x / (D / 4);
  const int d = ((int)threadIdx.x % (D / 4)) * 4;
  int L = a.seq_lens[s];
  L = L < 0 ? 0 : (L > a.max_seq_len ? a.max_seq_len : L);
  // Without a plan every partition wrote its partials or an m = -inf marker,
  // so the loads need not wait for seq_len; with one (from the host or made
  // on the device), only the sequence's own partitions ran.
  const int np = a.work || a.device_plan ? (L + a.partition - 1) / a.partition : a.num_partitions;
  const f32x4 v = merge_partials<D>(a, s, hq, d, np);
  if (L <= a.partition) return;  // written directly by the partition kernel
  store4<T>(reinterpret_cast<T*>(a.out) + ((int64_t)s * a.num_heads + hq) * D + d, v);
}

// With events, the kernel's own start and end are recorded into them
// (hipExtLaunchKernel): its execution time, with no packet of its own
// between this launch and the next.
template <int NW, typename T, int D, int B, int G>
hipError_t launch_partitions(const DecodeArgs& a, hipStream_t stream, hipEvent_t t0, hipEvent_t t1) {
  const SmemLayout lay = smem_layout(a.partition, B, G, D, NW);
  dim3 grid((unsigned)((a.work ? a.num_work : (a.num_partitions > 0 ? a.num_partitions : 1) * a.num_seqs) *
                       a.cache.num_kv_heads));
  if (t0 || t1) {
    hipExtLaunchKernelGGL((decode_partition_kernel<NW, T, D, B, G>), grid, dim3(NW * 64), (uint32_t)lay.bytes, stream,
                          t0, t1, 0u, a);
  } else {
    hipLaunchKernelGGL((decode_partition_kernel<NW, T, D, B, G>), grid, dim3(NW * 64), lay.bytes, stream, a);
  }
  return hipGetLastError();
}

// stage 1: partition kernel; stage 2: merge (only when some sequence can be
// longer than one partition); 0: both.
template <typename T, int D, int B, int G>
hipError_t launch_typed(const DecodeArgs& a, int stage, hipStream_t stream) {
  if (stage != 2) {
    const hipError_t e = a.waves == 8 ? launch_partitions<8, T, D, B, G>(a, stream, a.t0, a.t1)
                                      : launch_partitions<4, T, D, B, G>(a, stream, a.t0, a.t1);
    if (e != hipSuccess) return e;
  }
  if (stage != 1 && a.max_seq_len > a.partition) {
    hipLaunchKernelGGL((decode_reduce_kernel<typename Dec<T>::Q, D, G>), dim3(a.cache.num_kv_heads, a.num_seqs),
                       dim3(G * D / 4), 0, stream, a);
    return hipGetLastError();
  }
  return hipSuccess;
}

template <typename T, int D, int B>
hipError_t dispatch_g(const DecodeArgs& a, int G, int stage, hipStream_t stream) {
  switch (G) {
    case 1: return launch_typed<T, D, B, 1>(a, stage, stream);
    case 2: return launch_typed<T, D, B, 2>(a, stage, stream);
    case 4: return launch_typed<T, D, B, 4>(a, stage, stream);
    case 8: return launch_typed<T, D, B, 8>(a, stage, stream);
  }
  return hipErrorInvalidValue;
}

template <typename T, int D>
hipError_t dispatch_b(const DecodeArgs& a, int G, int stage, hipStream_t stream) {
  switch (a.cache.block_size) {
    case 16: return dispatch_g<T, D, 16>(a, G, stage, stream);
    case 32: return dispatch_g<T, D, 32>(a, G, stage, stream);
  }
  return hipErrorInvalidValue;
}

template <typename T>
hipError_t dispatch_d(const DecodeArgs& a, int G, int stage, hipStream_t stream) {
  switch (a.cache.head_dim) {
    case 64: return dispatch_b<T, 64>(a, G, stage, stream);
    case 128: return dispatch_b<T, 128>(a, G, stage, stream);
  }
  return hipErrorInvalidValue;
}

}  // namespace

hipError_t launch_decode(const DecodeArgs& a, int stage, hipStream_t stream) {
  if (a.num_seqs == 0) return hipSuccess;
  const int G = a.num_heads / a.cache.num_kv_heads;
  switch (a.cache.dtype) {
    case DType::kF32: return dispatch_d<float>(a, G, stage, stream);
    case DType::kF16: return dispatch_d<f16_t>(a, G, stage, stream);
    case DType::kBF16: return dispatch_d<bf16_t>(a, G, stage, stream);
    case DType::kFP8: return dispatch_d<fp8_t>(a, G, stage, stream);
  }
  return hipErrorInvalidValue;
}

}  // namespace pa
