// Chunked-prefill attention over an FP8 (E4M3) paged cache on gfx950 matrix
// cores.  The codes are converted to f16 as they are staged in LDS (every
// E4M3 value is exact in f16), so the products, the query and the output are
// f16; the 16-bit pools run the kernel in prefill.hip.
//
// Sources: [P1] "大模型推理内存优化从 KV Cache 分页到连续批处理的工程实践",
// section "工程边界与架构取舍" (prefill is a compute-bound matrix product; a
// long prompt is processed in chunks interleaved with decode steps) and
// section "PagedAttention 的 CUDA Kernel 实现" (K/V reached block by block
// through the table); the FP8 cache format as in decode.hip.
//
// A chunk of q_s new tokens of sequence s sits at positions ctx .. ctx+q_s-1
// (ctx = seq_len - q_s; the chunk's own K/V are already in the pool) and
// attends causally: position ctx+i sees keys 0 .. ctx+i.
//
// Work decomposition.  A workgroup (8 waves) owns 256 query rows that share
// one KV head: the G heads of the group times 256/G consecutive positions.
// Each wave owns 32 rows.  Keys stream through in tiles of 32: the tile's K
// rows ([32][D]) and V^T ([D][32], as the pool stores value tiles) are
// converted and staged in LDS, then per wave
//   S^T[32 keys x 32 rows] = K . Q^T      v_mfma_f32_32x32x16_f16 over D
//   online softmax down each column (a column is one query row, held by a
//   lane pair), P^T rounded to f16 in registers
//   O^T[D x 32 rows]     += V^T . P^T    v_mfma_f32_32x32x16_f16 over the tile
// The loop is software-pipelined so that matrix and vector work of one wave
// overlap: while tile t's softmax runs on the vector ALU, the scores of tile
// t+1 are computed on the matrix cores.  LDS holds three tile stages (t,
// t+1 and t+2, written while t is used), and a ring of register sets keeps
// the global loads of later tiles in flight.
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

constexpr int kPW = 8;          // waves per workgroup
constexpr int kRows = 32 * kPW; // query rows per workgroup
constexpr int kKT = 32;         // keys per tile
constexpr int kRing = 3;        // key tiles in flight in registers
constexpr int kBtStage = 2048;  // table entries staged in LDS (32K tokens at block size 16)
// The running maximum of a row is moved only when a tile's maximum exceeds
// it by more than this (log2 units), so probabilities stay below 2^8 and the
// accumulator rescale is rare; the final division by the row sum cancels
// whichever reference maximum was used.
constexpr float kLazy = 8.f;

typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

template <typename T>
__device__ __forceinline__ f32x16 mfma32(const u32x4& a, const u32x4& b, const f32x16& c);
template <>
__device__ __forceinline__ f32x16 mfma32<f16_t>(const u32x4& a, const u32x4& b, const f32x16& c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(f16x8, a), __builtin_bit_cast(f16x8, b), c, 0, 0, 0);
}

// Two floats -> one packed pair of storage elements (round to nearest even).
template <typename T>
__device__ __forceinline__ uint32_t pack2(float lo, float hi);
template <>
__device__ __forceinline__ uint32_t pack2<f16_t>(float lo, float hi) {
  return pack_f16x2(lo, hi);
}

template <int D>
struct PrefillSmem {
  static constexpr int kKStride = D + 8;     // K row stride (elements): 16-byte pad
  static constexpr int kVStride = kKT + 8;   // V^T row stride (elements)
  static constexpr int kKElems = kKT * kKStride;
  static constexpr int kVElems = D * kVStride;
  static constexpr int kStage = kKElems + kVElems;  // one tile: K rows, then V^T
  static constexpr int kStages = 3;
  static constexpr int kBytes = kStages * kStage * 2;
};

template <typename T, int D, int B, int G>
__global__ void __launch_bounds__(kPW * 64) __attribute__((amdgpu_waves_per_eu(2))) prefill_fp8_kernel(PrefillArgs a) {
  constexpr int QP = kRows / G;          // positions per workgroup
  constexpr int KSTEPS = D / 16;         // QK contraction steps
  constexpr int DT = D / 32;             // O^T row tiles
  constexpr int NT = kPW * 64;
  // An FP8 pool's codes are converted to f16 as they are staged in LDS; the
  // products, the query and the output are f16 then.
  using CT = typename Src<T>::type;
  constexpr bool kFp8 = std::is_same<T, fp8_t>::value;
  constexpr int CE = 16 / Elem<T>::kBytes;  // pool elements per 16-byte chunk
  static_assert(B % CE == 0, "a chunk of one value row never crosses a block");
  constexpr int NCHK = kKT * D / CE;     // 16-byte chunks per tile (K, and V)
  constexpr int CPT = (NCHK + NT - 1) / NT;  // per thread
  constexpr int RD = kRing;
  static_assert(RD >= 2, "the prologue stages two tiles from the ring");
  using S = PrefillSmem<D>;

  __shared__ __align__(16) uint16_t smem[S::kBytes / 2];
  auto Ks = [&](int st) { return smem + st * S::kStage; };
  auto Vt = [&](int st) { return smem + st * S::kStage + S::kKElems; };

  // Work item.  Workgroup ids are dealt to the 8 XCDs round-robin; remap so
  // that consecutive work items (the query tiles of one sequence and KV head,
  // which read the same K/V) land on the same XCD and share its L2.
  const int nqt = a.num_qtiles;
  const int total = a.num_seqs * a.cache.num_kv_heads * nqt;
  const int per_xcd = (total + 7) / 8;
  const int u = (blockIdx.x % 8) * per_xcd + blockIdx.x / 8;
  if (u >= total) return;
  const int qt = u % nqt;
  const int g = (u / nqt) % a.cache.num_kv_heads;
  const int s = u / nqt / a.cache.num_kv_heads;

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

  // This lane's query row (column n of the wave's S^T / O^T tiles).
  const int r = w * 32 + n;
  const int h = r / QP;
  const int p = r % QP;
  const bool row_ok = q0 + p < q_len;
  const int limit = row_ok ? ctx + q0 + p : -1;
  const int64_t tok = (int64_t)qbeg + q0 + p;
  const int hq = g * G + h;
  // The smallest causal limit among this wave's rows that exist: a key tile
  // that ends at or below it is visible to all of them, unmasked.
  int lim_min = row_ok ? limit : 0x7fffffff;
#pragma unroll
  for (int m = 1; m < 64; m <<= 1) lim_min = min(lim_min, __shfl_xor(lim_min, m, 64));
  lim_min = __builtin_amdgcn_readfirstlane(lim_min);  // wave-uniform: scalar branches below

  // Q rows as B operands.  A negative scale is moved into Q (negation is
  // exact), so the logit scale below is never negative and the maximum of
  // the scaled logits is the scaled maximum.
  const uint32_t qflip = a.scale < 0.f ? 0x80008000u : 0u;
  u32x4 qreg[KSTEPS];
  {
    const CT* qrow = reinterpret_cast<const CT*>(a.query) + (tok * Hq + hq) * D;
#pragma unroll
    for (int ks = 0; ks < KSTEPS; ++ks) {
      qreg[ks] = row_ok ? *reinterpret_cast<const u32x4*>(qrow + 16 * ks + 8 * hi) : u32x4{0, 0, 0, 0};
      qreg[ks] ^= qflip;
    }
  }

  const T* kc = reinterpret_cast<const T*>(a.cache.key_cache);
  const T* vc = reinterpret_cast<const T*>(a.cache.value_cache);
  const int32_t* bt = a.block_tables + (int64_t)s * a.max_blocks;
  // The table entries this workgroup needs are staged in LDS once (the tile
  // loop would otherwise pay a dependent global read before every K/V load);
  // tables longer than the staging area are read from global memory.
  __shared__ int s_bt[kBtStage];
  const int nbk = (kend + B - 1) / B;
  const bool staged = nbk <= kBtStage;
  if (staged) {
    for (int j = tid; j < nbk; j += NT) {
      const int id = bt[j];
      s_bt[j] = (id >= 0 && id < a.cache.num_blocks) ? id : -1;
    }
  }
  __syncthreads();
  // Callers pass pos < kend, so pos / B < nbk; the bound is checked anyway
  // so that no index outside the staged (validated) entries is ever used.
  auto block_of = [&](int pos) -> int {
    const int j = pos / B;
    if (j >= nbk) return -1;
    if (staged) return s_bt[j];
    const int id = bt[j];
    return (id >= 0 && id < a.cache.num_blocks) ? id : -1;
  };

  // K piece c of a tile: 16 bytes (dims dch*CE ..) of key `key`, numbered
  // in the pool's order (the four pieces of a key's 64-byte chunk, then the
  // tile's keys, then the chunks), so consecutive threads read consecutive
  // memory.
  constexpr int KPC = key_chunk<T>() / CE;  // 16-byte pieces per 64-byte chunk
  auto key_piece = [&](int c, int& key, int& dch) {
    key = (c / KPC) % kKT;
    dch = (c / (KPC * kKT)) * KPC + c % KPC;
  };
  // Global -> registers for one tile.  K chunks in pool order (coalesced);
  // V chunks: CE keys of one dimension from the transposed value tile (a
  // tile of 32 keys never splits such a piece across blocks, since CE
  // divides the block size).  Keys no row of this workgroup sees (>= kend),
  // or in blocks outside the pool, read as zeros (their probabilities are
  // zero; a zero V keeps 0 * V finite).  Up to RD tiles are in flight in
  // registers at once.
  u32x4 kregs[RD][CPT], vregs[RD][CPT];
  auto fetch = [&](u32x4 (&kreg)[CPT], u32x4 (&vreg)[CPT], int t) {
#pragma unroll
    for (int i = 0; i < CPT; ++i) {
      const int c = tid + i * NT;
      if (NCHK % NT != 0 && c >= NCHK) continue;
      {
        int key, dch;
        key_piece(c, key, dch);
        const int pos = t * kKT + key;
        u32x4 x = {0, 0, 0, 0};
        if (pos < kend) {  // keys >= kend are masked for every row of this tile
          const int pb = block_of(pos);
          if (pb >= 0)
            x = *reinterpret_cast<const u32x4*>(kc + ((int64_t)pb * Hkv + g) * B * D +
                                                key_tile_offset<T>(pos % B, dch * CE, B));
        }
        kreg[i] = x;
      }
      {
        const int kg = c % (kKT / CE), d = c / (kKT / CE);
        const int pos = t * kKT + kg * CE;
        u32x4 x = {0, 0, 0, 0};
        if (pos < kend) {  // keys >= kend are masked for every row of this tile
          const int pb = block_of(pos);
          if (pb >= 0) {
            x = *reinterpret_cast<const u32x4*>(vc + (((int64_t)pb * Hkv + g) * D + d) * B + pos % B);
            const int nv = kend - pos;  // keys of this piece that some row sees
            if (nv < CE) {
#pragma unroll
              for (int e = 0; e < 4; ++e) {
                uint32_t keep;
                if constexpr (kFp8) {
                  keep = 0;
#pragma unroll
                  for (int b = 0; b < 4; ++b) keep |= (4 * e + b < nv ? 0xffu : 0u) << (8 * b);
                } else {
                  keep = 2 * e >= nv ? 0u : (2 * e + 1 >= nv ? 0xffffu : 0xffffffffu);
                }
                x[e] &= keep;
              }
            }
          }
        }
        vreg[i] = x;
      }
    }
  };
  // Registers -> LDS (as f16 for an FP8 pool: sixteen codes become two
  // 16-byte pieces, every E4M3 value being exact in f16).
  auto put = [&](uint16_t* dst, const u32x4& x) {
    if constexpr (kFp8) {
      u32x4 lo, hi;
#pragma unroll
      for (int e = 0; e < 2; ++e) {
        lo[2 * e] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(x[e], 1.0f, false));
        lo[2 * e + 1] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(x[e], 1.0f, true));
        hi[2 * e] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(x[e + 2], 1.0f, false));
        hi[2 * e + 1] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(x[e + 2], 1.0f, true));
      }
      *reinterpret_cast<u32x4*>(dst) = lo;
      *reinterpret_cast<u32x4*>(dst + 8) = hi;
    } else {
      *reinterpret_cast<u32x4*>(dst) = x;
    }
  };
  auto stash = [&](const u32x4 (&kreg)[CPT], const u32x4 (&vreg)[CPT], int st) {
#pragma unroll
    for (int i = 0; i < CPT; ++i) {
      const int c = tid + i * NT;
      if (NCHK % NT != 0 && c >= NCHK) continue;
      {
        int key, dch;
        key_piece(c, key, dch);
        put(Ks(st) + key * S::kKStride + dch * CE, kreg[i]);
      }
      {
        const int kg = c % (kKT / CE), d = c / (kKT / CE);
        put(Vt(st) + d * S::kVStride + kg * CE, vreg[i]);
      }
    }
  };

  f32x16 o[DT];
#pragma unroll
  for (int dt = 0; dt < DT; ++dt)
#pragma unroll
    for (int j = 0; j < 16; ++j) o[dt][j] = 0.f;
  float m_run = -INFINITY, l_run = 0.f;
  // FP8: the staged K values are the codes' values; the pool scale joins
  // the logit scale (and V's the output factor).
  const float qscale = fabsf(a.scale) * kLog2e * (kFp8 ? a.cache.k_scale : 1.f);
  // S^T row slot of this lane's A operand, with bits 2 and 3 swapped.
  const int krow = (n & ~12) | ((n & 4) << 1) | ((n & 8) >> 1);

  // S^T = K . Q^T for the tile in stage st.
  auto scores = [&](int st) {
    f32x16 acc;
#pragma unroll
    for (int j = 0; j < 16; ++j) acc[j] = 0.f;
    const uint16_t* krp = Ks(st) + krow * S::kKStride + 8 * hi;
#pragma unroll
    for (int ks = 0; ks < KSTEPS; ++ks)
      acc = mfma32<CT>(*reinterpret_cast<const u32x4*>(krp + 16 * ks), qreg[ks], acc);
    return acc;
  };

  // Online softmax of tile t's scores down the column, in log2 units, into
  // the P^T operands.  Accumulator j holds key t*32 + 16 (j / 8) + 8 hi +
  // j % 8 (after the row permutation).  Only tiles that reach past the
  // wave's smallest limit (the causal diagonal) mask per key.  The running
  // maximum moves only where the tile exceeds it by more than kLazy; the
  // probabilities are taken against the moved maximum and the accumulator
  // rescale (rare) is left to the caller through alpha.
  u32x4 pb[2];
  // `gaps` bit h (h = 0, 1): keys 16h .. 16h+15 of the tile lie in a block
  // missing from the pool (table entry outside it).  Such keys hold no
  // vector, so they are masked like keys past the diagonal, never read as
  // zeros (a zero key would still add to the row's normaliser).
  auto softmax = [&](f32x16 sc, int t, bool masked, uint32_t gaps, float& alpha) {
    float mt = -INFINITY;
    if (masked) {
      const int kt0 = t * kKT + 8 * hi;
#pragma unroll
      for (int j = 0; j < 16; ++j) {
        const int key = kt0 + 16 * (j >> 3) + (j & 7);
        const bool gone = (gaps >> (j >> 3)) & 1u;
        sc[j] = key <= limit && !gone ? sc[j] * qscale : -INFINITY;
        mt = fmaxf(mt, sc[j]);
      }
    } else {
#pragma unroll
      for (int j = 0; j < 16; ++j) mt = fmaxf(mt, sc[j]);
      mt *= qscale;
    }
    mt = max_across_halves(mt);
    const bool move = mt > m_run + kLazy;
    const float m_new = move ? mt : m_run;
    alpha = move ? fast_exp2(m_run - m_new) : 1.f;  // 0 from -inf
    m_run = m_new;
    // A row that has seen no key yet (m_run = -inf) only holds masked
    // logits: exp2(-inf) = 0 with any finite reference.
    const float m_ref = m_run == -INFINITY ? 0.f : m_run;
    float pj[16];
    if (masked) {
#pragma unroll
      for (int j = 0; j < 16; ++j) pj[j] = fast_exp2(sc[j] - m_ref);
    } else {
#pragma unroll
      for (int j = 0; j < 16; ++j) pj[j] = fast_exp2(fmaf(sc[j], qscale, -m_ref));
    }
    float ps = 0.f;
#pragma unroll
    for (int j = 0; j < 16; ++j) ps += pj[j];
    l_run = l_run * alpha + ps;
    // P^T as B operands (f16 keeps 11 significant bits of a probability).
#pragma unroll
    for (int ks = 0; ks < 2; ++ks)
#pragma unroll
      for (int i = 0; i < 4; ++i) pb[ks][i] = pack2<CT>(pj[8 * ks + 2 * i], pj[8 * ks + 2 * i + 1]);
  };

  // O^T += V^T . P^T for the tile in stage st.
  auto accumulate = [&](int st) {
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) {
      const uint16_t* vrp = Vt(st) + (32 * dt + n) * S::kVStride + 8 * hi;
#pragma unroll
      for (int ks = 0; ks < 2; ++ks) {
        const u32x4 va = *reinterpret_cast<const u32x4*>(vrp + 16 * ks);
        o[dt] = mfma32<CT>(va, pb[ks], o[dt]);
      }
    }
  };

  // Prologue: tiles 0 .. RD-1 load into the register sets, tiles 0 and 1 go
  // to stages 0 and 1 and their sets are refilled with tiles RD and RD+1.
#pragma unroll
  for (int i = 0; i < RD; ++i)
    if (i < ntiles) fetch(kregs[i], vregs[i], i);
  stash(kregs[0], vregs[0], 0);
  if (1 < ntiles) stash(kregs[1], vregs[1], 1);
  if (RD < ntiles) fetch(kregs[0], vregs[0], RD);
  if (RD + 1 < ntiles) fetch(kregs[1], vregs[1], RD + 1);
  __syncthreads();
  f32x16 sc = scores(0);

  // Iteration t: scores of tile t+1 (stage (t+1) % 3; past the last tile
  // the stage holds stale data and the result goes unused) with tile t's
  // softmax, then tile t's PV product (stage t % 3), then tile t+2 from its
  // register set into stage (t+2) % 3, whose last reader was tile t-1, and
  // the set refilled with tile t+2+RD.
  for (int t0 = 0; t0 < ntiles; t0 += RD) {
#pragma unroll
    for (int i = 0; i < RD; ++i) {
      const int t = t0 + i;
      if (t < ntiles) {
        // Stage of tile t (a constant when RD is a multiple of 3).
        const int st0 = RD % 3 == 0 ? i % 3 : t % 3;
        const int st1 = st0 == 2 ? 0 : st0 + 1;
        const int st2 = st1 == 2 ? 0 : st1 + 1;
        float alpha;
        f32x16 sn;
        // Wave-uniform: the tile's two 16-key halves each lie in one block.
        const uint32_t gaps = __builtin_amdgcn_readfirstlane((block_of(t * kKT) < 0 ? 1u : 0u) |
                                                             (block_of(t * kKT + 16) < 0 ? 2u : 0u));
        if (t * kKT + kKT - 1 > lim_min || gaps) {
          sn = scores(st1);
          softmax(sc, t, true, gaps, alpha);
        } else {
          sn = scores(st1);
          softmax(sc, t, false, 0u, alpha);
        }
        if (__any(alpha != 1.f)) {
#pragma unroll
          for (int dt = 0; dt < DT; ++dt)
#pragma unroll
            for (int j = 0; j < 16; ++j) o[dt][j] *= alpha;
        }
        accumulate(st0);
        if (t + 2 < ntiles) {
          stash(kregs[(i + 2) % RD], vregs[(i + 2) % RD], st2);
          if (t + 2 + RD < ntiles) fetch(kregs[(i + 2) % RD], vregs[(i + 2) % RD], t + 2 + RD);
        }
        __syncthreads();
        sc = sn;
      }
    }
  }

  // Normalise and store this lane's row: accumulator j of tile dt is
  // dimension 32 dt + 8 (j / 4) + 4 hi + j % 4.
  const float l_tot = sum_across_halves(l_run);
  if (row_ok) {
    const float inv = l_tot > 0.f ? (kFp8 ? a.cache.v_scale : 1.f) / l_tot : 0.f;
    uint16_t* orow = reinterpret_cast<uint16_t*>(a.out) + (tok * Hq + hq) * D;
#pragma unroll
    for (int dt = 0; dt < DT; ++dt)
#pragma unroll
      for (int j4 = 0; j4 < 4; ++j4) {
        const int d = 32 * dt + 8 * j4 + 4 * hi;
        u32x2 pk;
        pk[0] = pack2<CT>(o[dt][4 * j4] * inv, o[dt][4 * j4 + 1] * inv);
        pk[1] = pack2<CT>(o[dt][4 * j4 + 2] * inv, o[dt][4 * j4 + 3] * inv);
        *reinterpret_cast<u32x2*>(orow + d) = pk;
      }
  }
}

template <typename T, int D, int B, int G>
hipError_t launch_prefill_typed(const PrefillArgs& a, hipStream_t stream) {
  const int total = a.num_seqs * a.cache.num_kv_heads * a.num_qtiles;
  const int grid = ((total + 7) / 8) * 8;
  hipLaunchKernelGGL((prefill_fp8_kernel<T, D, B, G>), dim3(grid), dim3(kPW * 64), 0, stream, a);
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

hipError_t launch_prefill_fp8(const PrefillArgs& a, hipStream_t stream) {
  if (a.num_seqs == 0 || a.num_qtiles == 0) return hipSuccess;
  return prefill_d<fp8_t>(a, a.num_heads / a.cache.num_kv_heads, stream);
}

}  // namespace pa
