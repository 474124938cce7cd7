// Paged decode attention for gfx950 (MI355X).
//
// Sources: [P1] "大模型推理内存优化从 KV Cache 分页到连续批处理的工程实践",
// sections "PagedAttention 的 CUDA Kernel 实现" (look up each logical block's
// physical ID in the block table, then read the block's contiguous K/V; the
// table sits on chip; in-block reads coalesce) and "工程边界与架构取舍"
// (decode is bound by reading the whole KV cache for one token).
//
// Work decomposition.  One workgroup of NW (8) wavefronts handles one
// (partition, KV head, sequence): a partition is `partition` consecutive
// tokens of the sequence (a multiple of the block size).  All G query heads
// that share the KV head are served by the same workgroup, so every K/V block
// is read from HBM once per KV head.
//
//   1. The partition's block-table entries are staged in LDS.
//   2. QK: each wave takes blocks w, w+NW, ...  A token's K row is split over
//      8 lanes (16-byte loads, 128 contiguous bytes per 8 lanes), every lane
//      dots its slice with the G query heads (v_dot2 for f16/bf16), and a
//      3-step DPP reduce-scatter over the 8 lanes leaves each lane with the
//      full logit of one head.  Logits, pre-multiplied by scale*log2(e), go
//      to LDS as [token][head].
//   3. Softmax: per-head maximum over the partition, p = 2^(z - max) written
//      back in place, per-head sums.
//   4. PV: a token's V row is split over D/VEC lanes (16 bytes each), each
//      lane accumulates p * v for all G heads in fp32; lanes holding the same
//      dims are summed with cross-lane moves, waves through LDS.
//   5. A sequence that fits one partition is normalised and written directly.
//      Longer sequences write (max, sum, unnormalised o) per partition to the
//      workspace and a second kernel merges them:
//        M = max_p m_p,  out = sum_p 2^(m_p - M) o_p / sum_p 2^(m_p - M) l_p.
#include <math.h>

#include <type_traits>

#include "pa_common.h"
#include "pa_launch.h"

namespace pa {

namespace {

constexpr int kNW = 8;  // wavefronts per workgroup (two workgroups per CU at 4 waves per SIMD)

template <int G>
struct Log2 {
  static constexpr int v = G == 1 ? 0 : G == 2 ? 1 : G == 4 ? 2 : 3;
};

// Dot product of two 16-byte chunks (8 x f16 / 8 x bf16 / 4 x f32) into fp32.
template <typename T>
__device__ __forceinline__ float dot16(const u32x4& q, const u32x4& k, float acc);

template <>
__device__ __forceinline__ float dot16<f16_t>(const u32x4& q, const u32x4& k, float acc) {
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    // Copy the lane out of the vector first: bit-casting a vector element
    // lvalue in place reads the vector's first element.
    const uint32_t qi = q[i], ki = k[i];
    acc = __builtin_amdgcn_fdot2(__builtin_bit_cast(f16x2, qi), __builtin_bit_cast(f16x2, ki), acc, false);
  }
  return acc;
}

template <>
__device__ __forceinline__ float dot16<bf16_t>(const u32x4& q, const u32x4& k, float acc) {
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const uint32_t qi = q[i], ki = k[i];
    acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(i16x2, qi), __builtin_bit_cast(i16x2, ki), acc, false);
  }
  return acc;
}

template <>
__device__ __forceinline__ float dot16<float>(const u32x4& q, const u32x4& k, float acc) {
#pragma unroll
  for (int i = 0; i < 4; ++i) acc = fmaf(__uint_as_float(q[i]), __uint_as_float(k[i]), acc);
  return acc;
}

// Query/output type of a pool dtype: FP8 pools take float16 queries.
template <typename T>
struct QType {
  using type = T;
};
template <>
struct QType<fp8_t> {
  using type = f16_t;
};

// A 16-byte K chunk as dot-product operands in the query type: itself, or
// for FP8 its 16 codes widened to two chunks of f16 pairs (values * 2^-8,
// exact; the 2^8 goes into the logit scale).
template <typename T>
struct KOps {
  static constexpr int kW = 1;
  __device__ static __forceinline__ void widen(const u32x4& k, u32x4* out) { out[0] = k; }
};
template <>
struct KOps<fp8_t> {
  static constexpr int kW = 2;
  __device__ static __forceinline__ void widen(const u32x4& k, u32x4* out) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const uint32_t w = k[i];
      out[i / 2][2 * (i % 2)] = e4m3_pair_to_f16x2(__builtin_amdgcn_perm(w, w, kPermBytes01));
      out[i / 2][2 * (i % 2) + 1] = e4m3_pair_to_f16x2(__builtin_amdgcn_perm(w, w, kPermBytes23));
    }
  }
};

// V chunk one PV lane loads per token: 16 bytes, or 8 for FP8 (8 dims, so
// that the lane's accumulators stay G * 8).
template <typename T>
struct VOps {
  typedef u32x4 load_t;
  static constexpr int kDims = vec16<T>();
};
template <>
struct VOps<fp8_t> {
  typedef u32x2 load_t;
  static constexpr int kDims = 8;
};

// 16 bytes of storage -> VEC floats.
template <typename T>
__device__ __forceinline__ void unpack16(const u32x4& v, float* f);

template <>
__device__ __forceinline__ void unpack16<f16_t>(const u32x4& v, float* f) {
#pragma unroll
  for (int i = 0; i < 4; ++i) unpack2<f16_t>(v[i], f[2 * i], f[2 * i + 1]);
}
template <>
__device__ __forceinline__ void unpack16<bf16_t>(const u32x4& v, float* f) {
#pragma unroll
  for (int i = 0; i < 4; ++i) unpack2<bf16_t>(v[i], f[2 * i], f[2 * i + 1]);
}
template <>
__device__ __forceinline__ void unpack16<float>(const u32x4& v, float* f) {
#pragma unroll
  for (int i = 0; i < 4; ++i) f[i] = __uint_as_float(v[i]);
}

// One butterfly step of the 8-lane reduce-scatter.  N values per lane; the
// partner lane differs in the bit selected by `hi`.  The lane keeps the upper
// half of its values when `hi` is set, sends the other half, and adds what
// the partner sent.  With N == 1 the step is a plain pairwise all-reduce.
template <int N, int kCtrl>
__device__ __forceinline__ void rs_step(float* a, bool hi) {
  if constexpr (N > 1) {
    constexpr int H = N / 2;
#pragma unroll
    for (int j = 0; j < H; ++j) {
      const float send = hi ? a[j] : a[j + H];
      const float keep = hi ? a[j + H] : a[j];
      a[j] = keep + dpp_mov<kCtrl>(send);
    }
  } else {
    a[0] += dpp_mov<kCtrl>(a[0]);
  }
}

// Sum G per-lane partial logits over the 8 lanes of one token; afterwards lane
// `sub` holds the full logit of head (sub >> (3 - log2 G)).
template <int G>
__device__ __forceinline__ float reduce_scatter8(float* a, int sub) {
  rs_step<G, kDppHalfMirror>(a, (sub >> 2) & 1);
  rs_step<(G >= 2 ? G / 2 : 1), kDppQuadXor2>(a, (sub >> 1) & 1);
  rs_step<(G >= 4 ? G / 4 : 1), kDppQuadXor1>(a, sub & 1);
  return a[0];
}

// LDS layout of one workgroup.  Each wave owns one region that first holds
// its logits/probabilities and, once its PV pass is done, its partial output
// (only the owning wave ever touches its region, so the reuse needs no
// barrier); f16 probability pairs, the per-wave (m, l), the block-table
// slice and the query rows are separate.  At the benchmark shape the total
// is ~27 KiB, so LDS never limits the four workgroups per CU that the VGPR
// budget allows.
struct SmemLayout {
  int bt_off, p_off, p_wave, h_off, h_wave, m_off, l_off, q_off, bytes;
};

__host__ __device__ inline SmemLayout smem_layout(int partition, int B, int G, int D) {
  SmemLayout s;
  const int nblk = partition / B;
  const int bpw = (nblk + kNW - 1) / kNW;  // blocks per wave
  int off = 0;
  s.bt_off = off;
  off += (nblk * 4 + 15) & ~15;
  s.p_off = off;
  const int logits = bpw * B * G;  // floats
  s.p_wave = logits > G * D ? logits : G * D;
  off += kNW * s.p_wave * 4;
  s.h_off = off;
  s.h_wave = bpw * B / 2 * G;  // dwords per wave: f16 probability pairs
  off += kNW * s.h_wave * 4;
  s.m_off = off;
  off += kNW * G * 4;
  s.l_off = off;
  off += kNW * G * 4;
  s.q_off = off;  // the G query rows, as stored (at most 8 x 128 x 4 bytes)
  off += G * D * 4;
  s.bytes = off;
  return s;
}

// Sum the per-lane PV accumulators x[NV] over the TS token slots of a wave
// (the lanes that hold the same dims).  gfx950's row swaps do the first two
// halvings: v_permlane32_swap exchanges the two 32-lane halves of a pair of
// registers, v_permlane16_swap the odd rows of one with the even rows of the
// other, so every swap-and-add halves the register count.  Afterwards lane
// (row q, column c) holds full sums x[q * NV/R + j], j < NV/R, R = min(TS, 4),
// rows counted in units of 64/R lanes; a third step (TS == 8) folds the two
// slots that share a 16-lane row with a DPP rotate.
template <int NV, int TS>
__device__ __forceinline__ void reduce_slots(float* x) {
  static_assert(TS == 2 || TS == 4 || TS == 8, "token slots");
#pragma unroll
  for (int j = 0; j < NV / 2; ++j) {
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x[j]), __float_as_uint(x[j + NV / 2]), false, false);
    x[j] = __uint_as_float(r[0]) + __uint_as_float(r[1]);
  }
  if constexpr (TS >= 4) {
#pragma unroll
    for (int j = 0; j < NV / 4; ++j) {
      const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x[j]), __float_as_uint(x[j + NV / 4]), false, false);
      x[j] = __uint_as_float(r[0]) + __uint_as_float(r[1]);
    }
  }
  if constexpr (TS == 8) {
#pragma unroll
    for (int j = 0; j < NV / 4; ++j) x[j] += dpp_mov<kDppRowRor8>(x[j]);
  }
}

// Wave-local LDS ordering: the compiler may not move LDS accesses across this
// point, and the wave's own earlier LDS writes are complete before later reads.
__device__ __forceinline__ void wave_lds_sync() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

// Combine the per-partition partials of one (sequence, query head, dim):
//   M = max_p m_p,  out = sum_p 2^(m_p - M) o_p / sum_p 2^(m_p - M) l_p.
// Every one of the call's partitions is fetched (empty ones carry
// m = -inf and contribute nothing), in batches of kMergeBatch whose loads are
// all issued before any is used; batches combine with a running rescale.
constexpr int kMergeBatch = 16;

template <int D>
__device__ __forceinline__ float merge_partials(const DecodeArgs& a, int s, int hq, int d) {
  const int np = a.num_partitions;
  const int64_t row0 = ((int64_t)s * a.num_heads + hq) * np;
  float M = -INFINITY, num = 0.f, den = 0.f;
  for (int p0 = 0; p0 < np; p0 += kMergeBatch) {
    float mv[kMergeBatch], lv[kMergeBatch], ov[kMergeBatch];
#pragma unroll
    for (int i = 0; i < kMergeBatch; ++i) {
      const bool ok = p0 + i < np;
      const int64_t row = row0 + p0 + i;
      mv[i] = ok ? a.ws_m[row] : -INFINITY;
      lv[i] = ok ? a.ws_l[row] : 0.f;
      ov[i] = ok ? a.ws_o[row * D + d] : 0.f;
    }
    float Mb = M;
#pragma unroll
    for (int i = 0; i < kMergeBatch; ++i) Mb = fmaxf(Mb, mv[i]);
    if (Mb == -INFINITY) continue;
    if (M != -INFINITY) {
      const float f = fast_exp2(M - Mb);
      num *= f;
      den *= f;
    }
#pragma unroll
    for (int i = 0; i < kMergeBatch; ++i) {
      // Absent partitions are skipped by select: their l and o are stale.
      const bool live = mv[i] != -INFINITY;
      const float wgt = live ? fast_exp2(mv[i] - Mb) : 0.f;
      num = live ? fmaf(wgt, ov[i], num) : num;
      den = live ? fmaf(wgt, lv[i], den) : den;
    }
    M = Mb;
  }
  return den > 0.f ? num / den : 0.f;
}

template <typename T, int G>
struct Occupancy {
  // 1- and 2-byte types fit in 128 VGPRs (4 waves per SIMD); f32 is a
  // correctness path and keeps the compiler's choice.
  static constexpr int kWaves = Elem<T>::kBytes <= 2 ? 4 : 1;
};

template <typename T, int D, int B, int G>
__global__ void __launch_bounds__(kNW * 64) __attribute__((amdgpu_waves_per_eu(Occupancy<T, G>::kWaves)))
decode_partition_kernel(DecodeArgs a) {
  using QT = typename QType<T>::type;
  using VLoad = typename VOps<T>::load_t;
  constexpr bool kFp8 = std::is_same<T, fp8_t>::value;
  constexpr int VEC = vec16<T>();   // K dims per 16-byte load
  constexpr int QVEC = vec16<QT>(); // query elements per 16 bytes
  constexpr int KW = KOps<T>::kW;   // operand chunks per K chunk
  constexpr int LPT = 8;            // lanes per token (QK)
  constexpr int DL = D / LPT;       // dims per lane (QK)
  constexpr int NCK = DL / VEC;     // 16-byte chunks per lane per token (QK)
  constexpr int CH = 16;            // tokens per pipeline stage (a chunk; B is 16 or 32)
  constexpr int CPB = B / CH;       // chunks per block
  constexpr int TPG = 64 / LPT;     // tokens per load group (QK)
  constexpr int GPC = CH / TPG;     // load groups per chunk (QK)
  constexpr int VV = VOps<T>::kDims; // dims per lane (PV)
  constexpr int LPV = D / VV;       // lanes per token (PV)
  constexpr int TS = 64 / LPV;      // token slots per load (PV)
  constexpr int IPC = CH / TS;      // loads per chunk (PV)
  constexpr int NT = kNW * 64;
  constexpr int SHIFT = 3 - Log2<G>::v;
  constexpr int NV = G * VV;        // PV accumulators per lane
  static_assert(B % CH == 0 && NCK >= 1 && GPC >= 1 && IPC >= 1, "unsupported shape");
  static_assert(64 % G == 0, "group size must divide the wave");

  extern __shared__ __align__(16) unsigned char smem[];
  // 1-D grid, (sequence, KV head) fastest and partition slowest.  Workgroup
  // ids are dealt to the 8 XCDs round-robin, so this hands each XCD whole
  // (sequence, KV head) pairs; with the partition fastest, XCD x would get
  // partitions x and x+8 of everything and every short sequence's only
  // partition would pile onto XCD 0.
  const int sg = blockIdx.x % (a.num_seqs * a.cache.num_kv_heads);
  const int part = blockIdx.x / (a.num_seqs * a.cache.num_kv_heads);
  const int g = sg % a.cache.num_kv_heads;
  const int s = sg / a.cache.num_kv_heads;
  const int P = a.partition;
  const SmemLayout lay = smem_layout(P, B, G, D);

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int w = tid >> 6;
  const int Hkv = a.cache.num_kv_heads;
  const int Hq = a.num_heads;
  const int tok0 = part * P;
  const int blk0 = tok0 / B;

  // The table slice of the whole partition range is fetched without waiting
  // for seq_len (it lies inside the table row either way), so the two loads
  // overlap; entries past the sequence's end are never used.
  int bt_id = -1;
  if (tid < P / B && blk0 + tid < a.max_blocks) bt_id = a.block_tables[(int64_t)s * a.max_blocks + blk0 + tid];
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
  const int nblk = (ntok + B - 1) / B;

  int* s_bt = reinterpret_cast<int*>(smem + lay.bt_off);
  float* s_p = reinterpret_cast<float*>(smem + lay.p_off) + w * lay.p_wave;
  // f16 path: probabilities of token pairs (t, t + TS) packed as f16x2, one
  // dword per (pair, head), pair index jc*CH/2 + (i/2)*TS + ts for the token
  // loaded by PV load i of chunk jc in slot ts.
  uint32_t* s_h = reinterpret_cast<uint32_t*>(smem + lay.h_off) + w * lay.h_wave;
  constexpr bool kDot2PV = std::is_same<QT, f16_t>::value;
  // Wave w's partial output, once its PV pass is done: [G][D] floats at the
  // start of region w.
  float* s_o = reinterpret_cast<float*>(smem + lay.p_off);
  float* s_m = reinterpret_cast<float*>(smem + lay.m_off);
  float* s_l = reinterpret_cast<float*>(smem + lay.l_off);

  // 1. Block-table slice -> LDS.  Entries outside the pool become -1.
  if (tid < P / B) s_bt[tid] = (bt_id < 0 || bt_id >= a.cache.num_blocks) ? -1 : bt_id;

  // The G query rows of this KV head are fetched once per workgroup into LDS
  // (G*D elements, 16 bytes per thread); every lane then reads its slices
  // from there, eight lanes per address.
  QT* s_q = reinterpret_cast<QT*>(smem + lay.q_off);
  {
    const QT* qb = reinterpret_cast<const QT*>(a.query) + ((int64_t)s * Hq + g * G) * D;
    for (int c = tid; c < G * D / QVEC; c += NT)
      *reinterpret_cast<u32x4*>(s_q + c * QVEC) = *reinterpret_cast<const u32x4*>(qb + c * QVEC);
  }
  __syncthreads();

  // Query slices for the QK layout: lane `sub` of a token holds, for each
  // head, dims c*LPT*VEC + sub*VEC .. +VEC of every chunk c.
  const int sub = lane & (LPT - 1);
  const int tq = lane / LPT;
  u32x4 qv[G][NCK * KW];
#pragma unroll
  for (int h = 0; h < G; ++h)
#pragma unroll
    for (int c = 0; c < NCK; ++c)
#pragma unroll
      for (int w2 = 0; w2 < KW; ++w2)
        qv[h][c * KW + w2] = *reinterpret_cast<const u32x4*>(s_q + h * D + c * LPT * VEC + sub * VEC + w2 * QVEC);

  // This wave's blocks: local index jl -> partition block w + jl*NW.
  const int nbw = nblk > w ? (nblk - w + kNW - 1) / kNW : 0;
  const int64_t blk_stride = (int64_t)Hkv * B * D;
  const T* kbase = reinterpret_cast<const T*>(a.cache.key_cache) + (int64_t)g * B * D;
  const T* vbase = reinterpret_cast<const T*>(a.cache.value_cache) + (int64_t)g * B * D;
  // FP8: widened K values are the codes' values * 2^-8.
  const float qscale = kFp8 ? a.scale * kLog2e * 256.f * a.cache.k_scale : a.scale * kLog2e;
  const int myhead = sub >> SHIFT;
  const bool writer = (sub & ((1 << SHIFT) - 1)) == 0;

  // 2. QK with the next chunk's K in flight while the current one is used.
  // Wave-local chunk jc is chunk jc % CPB of partition block w + (jc / CPB)*NW;
  // its logits live at wave-local tokens jc*CH ...
  const int nch = nbw * CPB;
  float run_max = -INFINITY;
  auto chunk_src = [&](const T* base, int jc, int& t0) -> const T* {
    const int jb = w + (jc / CPB) * kNW;
    t0 = jb * B + (jc % CPB) * CH;  // first token of the chunk, partition-relative
    const int pb = s_bt[jb];
    return pb >= 0 ? base + pb * blk_stride + (jc % CPB) * CH * D : nullptr;
  };
  auto k_load = [&](u32x4 (&kb)[GPC][NCK], int jc) {
    int t0;
    const T* src = chunk_src(kbase, jc, t0);
    if (src) {
#pragma unroll
      for (int gi = 0; gi < GPC; ++gi)
#pragma unroll
        for (int c = 0; c < NCK; ++c)
          kb[gi][c] = __builtin_nontemporal_load(
              reinterpret_cast<const u32x4*>(src + (gi * TPG + tq) * D + c * LPT * VEC + sub * VEC));
    }
  };
  auto qk_block = [&](const u32x4 (&kb)[GPC][NCK], int jc) {
    int t0;
    const bool valid = chunk_src(kbase, jc, t0) != nullptr;
#pragma unroll
    for (int gi = 0; gi < GPC; ++gi) {
      u32x4 ko[NCK * KW];
#pragma unroll
      for (int c = 0; c < NCK; ++c) KOps<T>::widen(kb[gi][c], ko + c * KW);
      float acc[G];
#pragma unroll
      for (int h = 0; h < G; ++h) {
        float x = 0.f;
#pragma unroll
        for (int c = 0; c < NCK * KW; ++c) x = dot16<QT>(qv[h][c], ko[c], x);
        acc[h] = x;
      }
      float z = reduce_scatter8<G>(acc, sub);
      const int tl = t0 + gi * TPG + tq;
      z = (valid && tl < ntok) ? z * qscale : -INFINITY;
      run_max = fmaxf(run_max, z);
      if (writer) s_p[(jc * CH + gi * TPG + tq) * G + myhead] = z;
    }
  };
  {
    u32x4 kb0[GPC][NCK], kb1[GPC][NCK];
    if (nch > 0) k_load(kb0, 0);
    for (int jc = 0; jc < nch; jc += 2) {
      if (jc + 1 < nch) k_load(kb1, jc + 1);
      qk_block(kb0, jc);
      if (jc + 2 < nch) k_load(kb0, jc + 2);
      if (jc + 1 < nch) qk_block(kb1, jc + 1);
    }
  }

  // The first V chunk goes out before the softmax so HBM stays busy.
  auto v_load = [&](VLoad (&vb)[IPC], int jc) {
    int t0;
    const T* src = chunk_src(vbase, jc, t0);
    if (src) {
      const int ts = lane / LPV, dc = lane % LPV;
#pragma unroll
      for (int i = 0; i < IPC; ++i)
        vb[i] = __builtin_nontemporal_load(reinterpret_cast<const VLoad*>(src + (i * TS + ts) * D + dc * VV));
    }
  };
  VLoad vb0[IPC], vb1[IPC];
  if (nch > 0) v_load(vb0, 0);

  // 3. Wave-local softmax.  Lanes with equal `sub` hold the same head.
  run_max = fmaxf(run_max, shfl_xor(run_max, 8));
  run_max = fmaxf(run_max, shfl_xor(run_max, 16));
  run_max = fmaxf(run_max, shfl_xor(run_max, 32));
  // Lane `lane` now serves head lane % G (64 % G == 0): fetch that head's max.
  const float M = __shfl(run_max, (lane % G) << SHIFT, 64);
  wave_lds_sync();
  float lsum = 0.f;
  {
    const int ne = nch * CH * G;
    for (int e = lane; e < ne; e += 64) {
      const float z = s_p[e];
      float pr = z == -INFINITY ? 0.f : fast_exp2(z - M);
      if constexpr (kDot2PV) {
        // The PV product sees p rounded to f16; the normaliser sums the
        // same rounded values.
        const _Float16 ph = (_Float16)pr;
        pr = (float)ph;
        const int tw = e / G, hh = e % G;        // wave-local token, head
        const int jc = tw / CH, tb = tw % CH;    // chunk, token within chunk
        const int i = tb / TS, tsl = tb % TS;    // PV load index, slot
        const int pair = jc * (CH / 2) + (i / 2) * TS + tsl;
        reinterpret_cast<uint16_t*>(s_h)[(pair * G + hh) * 2 + (i & 1)] = __builtin_bit_cast(uint16_t, ph);
      } else {
        s_p[e] = pr;
      }
      lsum += pr;
    }
  }
#pragma unroll
  for (int m = G; m < 64; m <<= 1) lsum += shfl_xor(lsum, m);
  wave_lds_sync();

  // 4. PV, double-buffered like QK.
  float o[NV];
#pragma unroll
  for (int k = 0; k < NV; ++k) o[k] = 0.f;
  const int ts = lane / LPV;
  auto pv_block = [&](const VLoad (&vb)[IPC], int jc) {
    int t0;
    if (!chunk_src(vbase, jc, t0)) return;
    if constexpr (kDot2PV) {
      // Token pairs (load i, load i+1) of this slot: build (v_t0[d], v_t1[d])
      // halves with v_perm and dot them with the packed (p_t0, p_t1).
#pragma unroll
      for (int i = 0; i < IPC; i += 2) {
        VLoad va = vb[i], vz = vb[i + 1];
        // Tail of the last block: zero V of tokens past the end (p is 0
        // there, and 0 * NaN would poison the sum).
        if (t0 + i * TS + ts >= ntok) va = VLoad(0u);
        if (t0 + (i + 1) * TS + ts >= ntok) vz = VLoad(0u);
        uint32_t X[VV];
        if constexpr (kFp8) {
          // Byte j of each token's word -> bits 15:8 / 31:24, then widen.
#pragma unroll
          for (int q = 0; q < 2; ++q) {
            const uint32_t lo = va[q], hi = vz[q];
#pragma unroll
            for (int j = 0; j < 4; ++j)
              X[4 * q + j] = e4m3_pair_to_f16x2(
                  __builtin_amdgcn_perm(hi, lo, ((4u + j) << 24) | (0x0cu << 16) | ((uint32_t)j << 8) | 0x0cu));
          }
        } else {
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            const uint32_t lo = va[q], hi = vz[q];
            X[2 * q] = __builtin_amdgcn_perm(hi, lo, 0x05040100u);
            X[2 * q + 1] = __builtin_amdgcn_perm(hi, lo, 0x07060302u);
          }
        }
        const int pair = jc * (CH / 2) + (i / 2) * TS + ts;
        uint32_t pw[G];
        const uint32_t* pp = s_h + pair * G;
        if constexpr (G % 4 == 0) {
#pragma unroll
          for (int h = 0; h < G; h += 4) {
            const u32x4 v4 = *reinterpret_cast<const u32x4*>(pp + h);
            pw[h] = v4[0], pw[h + 1] = v4[1], pw[h + 2] = v4[2], pw[h + 3] = v4[3];
          }
        } else {
#pragma unroll
          for (int h = 0; h < G; ++h) pw[h] = pp[h];
        }
#pragma unroll
        for (int h = 0; h < G; ++h) {
          const f16x2 ph = __builtin_bit_cast(f16x2, pw[h]);
#pragma unroll
          for (int v = 0; v < VV; ++v)
            o[h * VV + v] = __builtin_amdgcn_fdot2(ph, __builtin_bit_cast(f16x2, X[v]), o[h * VV + v], false);
        }
      }
    } else {
#pragma unroll
    for (int i = 0; i < IPC; ++i) {
      const int tb = i * TS + ts;  // token within the chunk
      if (t0 + tb >= ntok) continue;  // tail of the last block: never touch its contents
      float pr[G];
      const float* pp = s_p + (jc * CH + tb) * G;
      if constexpr (G % 4 == 0) {
#pragma unroll
        for (int h = 0; h < G; h += 4) {
          const f32x4 v4 = *reinterpret_cast<const f32x4*>(pp + h);
          pr[h] = v4[0], pr[h + 1] = v4[1], pr[h + 2] = v4[2], pr[h + 3] = v4[3];
        }
      } else {
#pragma unroll
        for (int h = 0; h < G; ++h) pr[h] = pp[h];
      }
      float vf[VV];
      unpack16<T>(vb[i], vf);
#pragma unroll
      for (int h = 0; h < G; ++h)
#pragma unroll
        for (int v = 0; v < VV; ++v) o[h * VV + v] = fmaf(pr[h], vf[v], o[h * VV + v]);
    }
    }
  };
  for (int jc = 0; jc < nch; jc += 2) {
    if (jc + 1 < nch) v_load(vb1, jc + 1);
    pv_block(vb0, jc);
    if (jc + 2 < nch) v_load(vb0, jc + 2);
    if (jc + 1 < nch) pv_block(vb1, jc + 1);
  }

  // 5. Fold token slots, park the wave's partial in LDS, merge the waves.
  reduce_slots<NV, TS>(o);
  wave_lds_sync();  // this wave's probability reads are done before its region is reused
  {
    constexpr int R = TS < 4 ? TS : 4;
    constexpr int PER = NV / R;  // values per lane after the fold
    const int q = lane / (64 / R);
    const int col = lane % (64 / R);
    if (col < LPV) {
#pragma unroll
      for (int j = 0; j < PER; ++j) {
        const int k = q * PER + j;
        const int h = k / VV, v = k % VV;
        s_o[w * lay.p_wave + h * D + col * VV + v] = o[j];
      }
    }
  }
  if (lane < G) {
    s_m[w * G + lane] = M;
    s_l[w * G + lane] = lsum;
  }
  __syncthreads();

  // FP8: widened V values are the codes' values * 2^-8.
  const float vfac = kFp8 ? 256.f * a.cache.v_scale : 1.f;
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
        const float sc = mw == -INFINITY ? 0.f : fast_exp2(mw - Mx);
        acc = fmaf(sc, s_o[ww * lay.p_wave + h * D + d], acc);
        l = fmaf(sc, s_l[ww * G + h], l);
      }
    }
    const int hq = g * G + h;
    acc *= vfac;
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

// Merge kernel for sequences longer than one partition.  A fused variant
// (the last workgroup of a sequence and KV head merging after an agent-scope
// release/acquire on an arrival counter) is correct but on gfx950 every such
// release writes back the XCD's L2, which cost far more than this launch.
// grid (num_heads, num_seqs), D threads.
template <typename T, int D>
__global__ void __launch_bounds__(D) decode_reduce_kernel(DecodeArgs a) {
  const int s = blockIdx.y, hq = blockIdx.x, d = threadIdx.x;
  int L = a.seq_lens[s];  // independent of the partial loads below
  const float v = merge_partials<D>(a, s, hq, d);
  L = L < 0 ? 0 : (L > a.max_seq_len ? a.max_seq_len : L);
  if (L <= a.partition) return;  // written directly by the partition kernel
  store_elem<T>(reinterpret_cast<T*>(a.out) + ((int64_t)s * a.num_heads + hq) * D + d, v);
}

template <typename T, int D, int B, int G>
hipError_t launch_typed(const DecodeArgs& a, hipStream_t stream) {
  const SmemLayout lay = smem_layout(a.partition, B, G, D);
  dim3 grid((unsigned)((a.num_partitions > 0 ? a.num_partitions : 1) * a.cache.num_kv_heads * a.num_seqs));
  hipLaunchKernelGGL((decode_partition_kernel<T, D, B, G>), grid, dim3(kNW * 64), lay.bytes, stream, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  if (a.max_seq_len > a.partition) {
    hipLaunchKernelGGL((decode_reduce_kernel<typename QType<T>::type, D>), dim3(a.num_heads, a.num_seqs), dim3(D), 0,
                       stream, a);
    e = hipGetLastError();
  }
  return e;
}

template <typename T, int D, int B>
hipError_t dispatch_g(const DecodeArgs& a, int G, hipStream_t stream) {
  switch (G) {
    case 1: return launch_typed<T, D, B, 1>(a, stream);
    case 2: return launch_typed<T, D, B, 2>(a, stream);
    case 4: return launch_typed<T, D, B, 4>(a, stream);
    case 8: return launch_typed<T, D, B, 8>(a, stream);
  }
  return hipErrorInvalidValue;
}

template <typename T, int D>
hipError_t dispatch_b(const DecodeArgs& a, int G, hipStream_t stream) {
  switch (a.cache.block_size) {
    case 16: return dispatch_g<T, D, 16>(a, G, stream);
    case 32: return dispatch_g<T, D, 32>(a, G, stream);
  }
  return hipErrorInvalidValue;
}

template <typename T>
hipError_t dispatch_d(const DecodeArgs& a, int G, hipStream_t stream) {
  if constexpr (Elem<T>::kBytes == 1) {
    // 16 codes per lane per token need 8 x 16 = 128 dims.
    return a.cache.head_dim == 128 ? dispatch_b<T, 128>(a, G, stream) : hipErrorInvalidValue;
  } else {
    switch (a.cache.head_dim) {
      case 64: return dispatch_b<T, 64>(a, G, stream);
      case 128: return dispatch_b<T, 128>(a, G, stream);
    }
    return hipErrorInvalidValue;
  }
}

}  // namespace

size_t decode_smem_bytes(int partition, int block_size, int group, int head_dim) {
  return (size_t)smem_layout(partition, block_size, group, head_dim).bytes;
}

hipError_t launch_decode(const DecodeArgs& a, hipStream_t stream) {
  if (a.num_seqs == 0) return hipSuccess;
  const int G = a.num_heads / a.cache.num_kv_heads;
  switch (a.cache.dtype) {
    case DType::kF32: return dispatch_d<float>(a, G, stream);
    case DType::kF16: return dispatch_d<f16_t>(a, G, stream);
    case DType::kBF16: return dispatch_d<bf16_t>(a, G, stream);
    case DType::kFP8: return dispatch_d<fp8_t>(a, G, stream);
  }
  return hipErrorInvalidValue;
}

}  // namespace pa
