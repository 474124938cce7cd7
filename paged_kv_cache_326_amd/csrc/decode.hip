// Paged decode attention for gfx950 (MI355X).
//
// Sources: [P1] "大模型推理内存优化从 KV Cache 分页到连续批处理的工程实践",
// sections "PagedAttention 的 CUDA Kernel 实现" (look up each logical block's
// physical ID in the block table, then read the block's contiguous K/V; the
// table sits on chip; in-block reads coalesce) and "工程边界与架构取舍"
// (decode is bound by reading the whole KV cache for one token).
//
// Work decomposition.  One workgroup of NW wavefronts handles one
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

#include "pa_common.h"
#include "pa_launch.h"

namespace pa {

namespace {

constexpr int kNW = 4;  // wavefronts per workgroup

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

struct SmemLayout {
  int bt_off, p_off, o_off, wmax_off, wsum_off, bytes;
};

__host__ __device__ inline SmemLayout smem_layout(int partition, int B, int G, int D) {
  SmemLayout s;
  int off = 0;
  s.bt_off = off;
  off += ((partition / B) * 4 + 15) & ~15;
  s.p_off = off;
  off += partition * G * 4;
  s.o_off = off;
  off += kNW * G * D * 4;
  s.wmax_off = off;
  off += kNW * G * 4;
  s.wsum_off = off;
  off += kNW * G * 4;
  s.bytes = off;
  return s;
}

template <typename T, int D, int B, int G>
__global__ void __launch_bounds__(kNW * 64) decode_partition_kernel(DecodeArgs a) {
  constexpr int VEC = vec16<T>();
  constexpr int LPT = 8;            // lanes per token (QK)
  constexpr int DL = D / LPT;       // dims per lane (QK)
  constexpr int NCK = DL / VEC;     // 16-byte chunks per lane per token (QK)
  constexpr int TPG = 64 / LPT;     // tokens per load group (QK)
  constexpr int GPB = B / TPG;      // load groups per block (QK)
  constexpr int LPV = D / VEC;      // lanes per token (PV)
  constexpr int TS = 64 / LPV;      // token slots per load (PV)
  constexpr int IPB = B / TS;       // loads per block (PV)
  constexpr int NT = kNW * 64;
  constexpr int SHIFT = 3 - Log2<G>::v;
  static_assert(NCK >= 1 && GPB >= 1 && IPB >= 1, "unsupported shape");
  static_assert(NT % G == 0, "thread count must be a multiple of the group size");

  extern __shared__ __align__(16) unsigned char smem[];
  const int part = blockIdx.x;
  const int g = blockIdx.y;
  const int s = blockIdx.z;
  const int P = a.partition;
  const SmemLayout lay = smem_layout(P, B, G, D);
  int* s_bt = reinterpret_cast<int*>(smem + lay.bt_off);
  float* s_p = reinterpret_cast<float*>(smem + lay.p_off);
  float* s_o = reinterpret_cast<float*>(smem + lay.o_off);
  float* s_wmax = reinterpret_cast<float*>(smem + lay.wmax_off);
  float* s_wsum = reinterpret_cast<float*>(smem + lay.wsum_off);

  int L = a.seq_lens[s];
  L = L < 0 ? 0 : (L > a.max_seq_len ? a.max_seq_len : L);
  const int tok0 = part * P;
  if (part > 0 && tok0 >= L) return;
  const int ntok = min(P, L - tok0) > 0 ? min(P, L - tok0) : 0;
  const int nblk = (ntok + B - 1) / B;
  const bool direct = L <= P;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int w = tid >> 6;
  const int Hkv = a.cache.num_kv_heads;
  const int Hq = a.num_heads;

  // 1. Block-table slice -> LDS.  Entries outside the pool become -1.
  {
    const int blk0 = tok0 / B;
    for (int j = tid; j < nblk; j += NT) {
      const int lj = blk0 + j;
      int id = lj < a.max_blocks ? a.block_tables[(int64_t)s * a.max_blocks + lj] : -1;
      if (id < 0 || id >= a.cache.num_blocks) id = -1;
      s_bt[j] = id;
    }
  }

  // Query slices for the QK layout: lane `sub` of a token holds, for each
  // head, dims c*LPT*VEC + sub*VEC .. +VEC of every chunk c.
  const int sub = lane & (LPT - 1);
  const int tq = lane / LPT;
  u32x4 qv[G][NCK];
  {
    const T* qb = reinterpret_cast<const T*>(a.query) + ((int64_t)s * Hq + g * G) * D;
#pragma unroll
    for (int h = 0; h < G; ++h)
#pragma unroll
      for (int c = 0; c < NCK; ++c)
        qv[h][c] = *reinterpret_cast<const u32x4*>(qb + h * D + c * LPT * VEC + sub * VEC);
  }
  __syncthreads();

  const float qscale = a.scale * kLog2e;
  const int myhead = sub >> SHIFT;
  const bool writer = (sub & ((1 << SHIFT) - 1)) == 0;
  const int64_t blk_stride = (int64_t)Hkv * B * D;
  const T* kbase = reinterpret_cast<const T*>(a.cache.key_cache) + (int64_t)g * B * D;
  const T* vbase = reinterpret_cast<const T*>(a.cache.value_cache) + (int64_t)g * B * D;

  // 2. QK.
  float run_max = -INFINITY;
  for (int j = w; j < nblk; j += kNW) {
    const int pb = s_bt[j];
    if (pb < 0) {
      if (writer)
        for (int gi = 0; gi < GPB; ++gi) s_p[(j * B + gi * TPG + tq) * G + myhead] = -INFINITY;
      continue;
    }
    const T* kb = kbase + pb * blk_stride;
    u32x4 kv[GPB][NCK];
#pragma unroll
    for (int gi = 0; gi < GPB; ++gi)
#pragma unroll
      for (int c = 0; c < NCK; ++c)
        kv[gi][c] = *reinterpret_cast<const u32x4*>(kb + (gi * TPG + tq) * D + c * LPT * VEC + sub * VEC);
#pragma unroll
    for (int gi = 0; gi < GPB; ++gi) {
      float acc[G];
#pragma unroll
      for (int h = 0; h < G; ++h) {
        float x = 0.f;
#pragma unroll
        for (int c = 0; c < NCK; ++c) x = dot16<T>(qv[h][c], kv[gi][c], x);
        acc[h] = x;
      }
      float z = reduce_scatter8<G>(acc, sub);
      const int tl = j * B + gi * TPG + tq;
      z = tl < ntok ? z * qscale : -INFINITY;
      run_max = fmaxf(run_max, z);
      if (writer) s_p[tl * G + myhead] = z;
    }
  }
  // Per-wave, per-head maximum: lanes with equal `sub` hold the same head.
  run_max = fmaxf(run_max, shfl_xor(run_max, 8));
  run_max = fmaxf(run_max, shfl_xor(run_max, 16));
  run_max = fmaxf(run_max, shfl_xor(run_max, 32));
  if (lane < LPT && writer) s_wmax[w * G + myhead] = run_max;
  __syncthreads();

  // 3. Softmax numerators and per-head sums.  NT % G == 0, so a thread always
  // sees the same head.
  const int hh = tid % G;
  float M = -INFINITY;
#pragma unroll
  for (int ww = 0; ww < kNW; ++ww) M = fmaxf(M, s_wmax[ww * G + hh]);
  float lsum = 0.f;
  {
    const int ne = nblk * B * G;
    for (int e = tid; e < ne; e += NT) {
      const float z = s_p[e];
      const float pr = z == -INFINITY ? 0.f : fast_exp2(z - M);
      s_p[e] = pr;
      lsum += pr;
    }
  }
#pragma unroll
  for (int m = G; m < 64; m <<= 1) lsum += shfl_xor(lsum, m);
  if (lane < G) s_wsum[w * G + lane] = lsum;
  __syncthreads();

  // 4. PV.
  const int ts = lane / LPV;
  const int dc = lane % LPV;
  float o[G][VEC];
#pragma unroll
  for (int h = 0; h < G; ++h)
#pragma unroll
    for (int v = 0; v < VEC; ++v) o[h][v] = 0.f;

  for (int j = w; j < nblk; j += kNW) {
    const int pb = s_bt[j];
    if (pb < 0) continue;
    const T* vb = vbase + pb * blk_stride;
    u32x4 vv[IPB];
#pragma unroll
    for (int i = 0; i < IPB; ++i) vv[i] = *reinterpret_cast<const u32x4*>(vb + (i * TS + ts) * D + dc * VEC);
#pragma unroll
    for (int i = 0; i < IPB; ++i) {
      const int tl = j * B + i * TS + ts;
      if (tl >= ntok) continue;  // tail of the last block: never touch its (arbitrary) contents
      float pr[G];
#pragma unroll
      for (int h = 0; h < G; ++h) pr[h] = s_p[tl * G + h];
      float vf[VEC];
      unpack16<T>(vv[i], vf);
#pragma unroll
      for (int h = 0; h < G; ++h)
#pragma unroll
        for (int v = 0; v < VEC; ++v) o[h][v] = fmaf(pr[h], vf[v], o[h][v]);
    }
  }
  // Sum the token slots of the wave (lanes that hold the same dims).
#pragma unroll
  for (int m = LPV; m < 64; m <<= 1)
#pragma unroll
    for (int h = 0; h < G; ++h)
#pragma unroll
      for (int v = 0; v < VEC; ++v) o[h][v] += shfl_xor(o[h][v], m);
  if (lane < LPV) {
#pragma unroll
    for (int h = 0; h < G; ++h)
#pragma unroll
      for (int v = 0; v < VEC; ++v) s_o[(w * G + h) * D + dc * VEC + v] = o[h][v];
  }
  __syncthreads();

  // 5. Combine the waves; normalise and store, or park the partial.
  for (int idx = tid; idx < G * D; idx += NT) {
    const int h = idx / D;
    const int d = idx % D;
    float acc = 0.f, l = 0.f, m = -INFINITY;
#pragma unroll
    for (int ww = 0; ww < kNW; ++ww) {
      acc += s_o[(ww * G + h) * D + d];
      l += s_wsum[ww * G + h];
      m = fmaxf(m, s_wmax[ww * G + h]);
    }
    const int hq = g * G + h;
    if (direct) {
      T* out = reinterpret_cast<T*>(a.out) + ((int64_t)s * Hq + hq) * D + d;
      store_elem<T>(out, l > 0.f ? acc / l : 0.f);
    } else {
      const int64_t row = ((int64_t)s * Hq + hq) * a.num_partitions + part;
      a.ws_o[row * D + d] = acc;
      if (d == 0) {
        a.ws_m[row] = m;
        a.ws_l[row] = l;
      }
    }
  }
}

// Merge the partitions of sequences longer than one partition.
// grid (num_heads, num_seqs), D threads.
template <typename T, int D>
__global__ void __launch_bounds__(D) decode_reduce_kernel(DecodeArgs a) {
  const int hq = blockIdx.x;
  const int s = blockIdx.y;
  const int d = threadIdx.x;
  int L = a.seq_lens[s];
  L = L < 0 ? 0 : (L > a.max_seq_len ? a.max_seq_len : L);
  if (L <= a.partition) return;  // written directly by the partition kernel
  const int np = (L + a.partition - 1) / a.partition;
  const int64_t row0 = ((int64_t)s * a.num_heads + hq) * a.num_partitions;
  float M = -INFINITY;
  for (int p = 0; p < np; ++p) M = fmaxf(M, a.ws_m[row0 + p]);
  float num = 0.f, den = 0.f;
  if (M != -INFINITY) {
    for (int p = 0; p < np; ++p) {
      const float wgt = fast_exp2(a.ws_m[row0 + p] - M);
      num = fmaf(wgt, a.ws_o[(row0 + p) * D + d], num);
      den = fmaf(wgt, a.ws_l[row0 + p], den);
    }
  }
  T* out = reinterpret_cast<T*>(a.out) + ((int64_t)s * a.num_heads + hq) * D + d;
  store_elem<T>(out, den > 0.f ? num / den : 0.f);
}

template <typename T, int D, int B, int G>
hipError_t launch_typed(const DecodeArgs& a, hipStream_t stream) {
  const SmemLayout lay = smem_layout(a.partition, B, G, D);
  dim3 grid(a.num_partitions > 0 ? a.num_partitions : 1, a.cache.num_kv_heads, a.num_seqs);
  hipLaunchKernelGGL((decode_partition_kernel<T, D, B, G>), grid, dim3(kNW * 64), lay.bytes, stream, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  if (a.max_seq_len > a.partition) {
    hipLaunchKernelGGL((decode_reduce_kernel<T, D>), dim3(a.num_heads, a.num_seqs), dim3(D), 0, stream, a);
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
  switch (a.cache.head_dim) {
    case 64: return dispatch_b<T, 64>(a, G, stream);
    case 128: return dispatch_b<T, 128>(a, G, stream);
  }
  return hipErrorInvalidValue;
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
  }
  return hipErrorInvalidValue;
}

}  // namespace pa
