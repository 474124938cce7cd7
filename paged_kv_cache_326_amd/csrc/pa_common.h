// Device helpers shared by the gfx950 kernels of libpa.so: storage dtypes,
// 16-byte vector types, conversions and wave64 cross-lane primitives.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace pa {

// Storage element types.  bf16 is carried as raw 16-bit patterns so every
// conversion below is explicit.
struct bf16_t {
  uint16_t bits;
};
typedef _Float16 f16_t;
// OCP E4M3 code (FP8 pools): 1 sign, 4 exponent bits (bias 7), 3 mantissa bits.
struct fp8_t {
  uint8_t bits;
};

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
typedef short i16x2 __attribute__((ext_vector_type(2)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

constexpr float kLog2e = 1.4426950408889634f;

template <typename T>
struct Elem;
template <>
struct Elem<float> {
  static constexpr int kBytes = 4;
};
template <>
struct Elem<f16_t> {
  static constexpr int kBytes = 2;
};
template <>
struct Elem<bf16_t> {
  static constexpr int kBytes = 2;
};
template <>
struct Elem<fp8_t> {
  static constexpr int kBytes = 1;
};

// Elements of T per 16-byte load.
template <typename T>
constexpr int vec16() {
  return 16 / Elem<T>::kBytes;
}

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }
__device__ __forceinline__ float f16_lo(uint32_t w) {
  return (float)__builtin_bit_cast(_Float16, (uint16_t)(w & 0xffffu));
}
__device__ __forceinline__ float f16_hi(uint32_t w) {
  return (float)__builtin_bit_cast(_Float16, (uint16_t)(w >> 16));
}

// float32 -> bf16 bits, round to nearest, ties to even (the hardware
// conversion in the default rounding mode); NaN stays NaN.
__device__ __forceinline__ uint16_t f32_to_bf16_bits(float x) {
  return __builtin_bit_cast(uint16_t, (__bf16)x);
}

// Two floats -> one packed pair (a in the low half), round to nearest even:
// one v_cvt_pk_f16_f32 / v_cvt_pk_bf16_f32.
__device__ __forceinline__ uint32_t pack_f16x2(float a, float b) {
  return __builtin_bit_cast(uint32_t, __builtin_convertvector((f32x2{a, b}), f16x2));
}
__device__ __forceinline__ uint32_t pack_bf16x2(float a, float b) {
  return __builtin_bit_cast(uint32_t, __builtin_convertvector((f32x2{a, b}), bf16x2));
}

// float32 -> E4M3 code (in the low byte): nearest value, ties to the even
// code, magnitudes from 448 up (infinity included) saturate to 448, NaN
// stays NaN, the sign of zero is kept.
__device__ __forceinline__ uint32_t f32_to_e4m3(float x) {
  const uint32_t u = __float_as_uint(x);
  const uint32_t sign = (u >> 24) & 0x80u;
  const uint32_t a = u & 0x7fffffffu;
  if (a > 0x7f800000u) return sign | 0x7fu;   // NaN
  if (a >= 0x43e00000u) return sign | 0x7eu;  // |x| >= 448
  if (a < 0x3c800000u) {
    // Below 2^-6 the codes are multiples of 2^-9 (subnormals); scaling by
    // 2^9 is exact and v_rndne rounds half to even, giving 0..8 (8 is the
    // smallest normal, code 0x08).
    return sign | (uint32_t)__builtin_rintf(__uint_as_float(a) * 512.0f);
  }
  // Normal: keep 3 of the 23 mantissa bits, rounding the 20 dropped bits to
  // nearest even; the carry may step into the exponent, which is still right.
  // Rebias the exponent from 127 to 7.
  const uint32_t r = (a + 0x7ffffu + ((a >> 20) & 1u)) >> 20;
  return sign | (r - (120u << 3));
}

// Store one float as a storage element.
template <typename T>
__device__ __forceinline__ void store_elem(T* p, float x);
template <>
__device__ __forceinline__ void store_elem<float>(float* p, float x) {
  *p = x;
}
template <>
__device__ __forceinline__ void store_elem<f16_t>(f16_t* p, float x) {
  *p = (_Float16)x;  // v_cvt_f16_f32 rounds to nearest-even
}
template <>
__device__ __forceinline__ void store_elem<bf16_t>(bf16_t* p, float x) {
  p->bits = f32_to_bf16_bits(x);
}

// New K/V rows are stored as they come, except into an FP8 pool, whose rows
// arrive as float16 and are quantised on the way: code = E4M3(x / scale),
// the division in float32 (IEEE, rounded to nearest).
template <typename T>
struct Src {
  using type = T;
};
template <>
struct Src<fp8_t> {
  using type = f16_t;
};

// Store the VEC = vec16<Src<T>> source elements of one 16-byte chunk (a
// piece of a key row).
template <typename T>
__device__ __forceinline__ void store_chunk(T* dst, const u32x4 data, float) {
  *reinterpret_cast<u32x4*>(dst) = data;
}
template <>
__device__ __forceinline__ void store_chunk<fp8_t>(fp8_t* dst, const u32x4 data, float scale) {
  uint32_t w[2];
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    uint32_t acc = 0;
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const uint32_t word = data[2 * i + j];
      const uint32_t lo = f32_to_e4m3(f16_lo(word) / scale);
      const uint32_t hi = f32_to_e4m3(f16_hi(word) / scale);
      acc |= (lo | (hi << 8)) << (16 * j);
    }
    w[i] = acc;
  }
  *reinterpret_cast<u32x2*>(dst) = u32x2{w[0], w[1]};
}

// Store the same chunk as one column piece of a transposed value tile:
// element e goes to p[e * stride].
template <typename T>
__device__ __forceinline__ void store_column(T* p, int64_t stride, const u32x4 data, float scale) {
  if constexpr (Elem<T>::kBytes == 4) {
    uint32_t* q = reinterpret_cast<uint32_t*>(p);
#pragma unroll
    for (int e = 0; e < 4; ++e) q[e * stride] = data[e];
  } else if constexpr (Elem<T>::kBytes == 2) {
    uint16_t* q = reinterpret_cast<uint16_t*>(p);
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const uint32_t word = data[e / 2];
      q[e * stride] = (uint16_t)(word >> (16 * (e % 2)));
    }
  } else {
    uint8_t* q = reinterpret_cast<uint8_t*>(p);
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const uint32_t word = data[e / 2];
      const float x = e % 2 ? f16_hi(word) : f16_lo(word);
      q[e * stride] = (uint8_t)f32_to_e4m3(x / scale);
    }
  }
}

// Key tiles.  The key tile of one (block, KV head), block_size rows of
// head_dim elements, is stored as 64-byte column chunks: chunk q holds dims
// q*KC .. q*KC+KC-1 (KC = 64 bytes of elements) of every row, row after row,
// so element (row t, dim d) sits at (d / KC) * block_size * KC + t * KC +
// d % KC of the tile.  A wave that reads a 64-byte piece of each of 16 rows
// (one matrix-core operand) then reads whole 128-byte lines.
template <typename T>
constexpr int key_chunk() {
  return 64 / Elem<T>::kBytes;
}

// Offset (elements) of (row t, dim d) inside a key tile.
template <typename T>
__host__ __device__ __forceinline__ int64_t key_tile_offset(int t, int d, int block_size) {
  constexpr int KC = key_chunk<T>();
  return (int64_t)(d / KC) * block_size * KC + (int64_t)t * KC + d % KC;
}

// The destination of one 16-byte source chunk (dims ch*VEC ..) of token
// slot (blk, off), KV head h: a key row piece (inside one 64-byte key
// chunk, VEC dividing it), or a value column piece.
template <typename T>
__device__ __forceinline__ void store_kv_chunk(T* key_cache, T* value_cache, int which, int64_t blk, int off, int h,
                                               int ch, int vec, int num_kv_heads, int head_dim, int block_size,
                                               const u32x4 data, float k_scale, float v_scale) {
  if (which == 0) {
    T* dst = key_cache + (blk * num_kv_heads + h) * (int64_t)block_size * head_dim +
             key_tile_offset<T>(off, ch * vec, block_size);
    store_chunk<T>(dst, data, k_scale);
  } else {
    T* dst = value_cache + ((blk * num_kv_heads + h) * head_dim + ch * vec) * block_size + off;
    store_column<T>(dst, block_size, data, v_scale);
  }
}

// ---------------------------------------------------------------------------
// Cross-lane reductions over the four 16-lane rows of a wave, on the vector
// ALU (no LDS round trip).  v_permlane16_swap with both operands x swaps the
// odd rows of one copy with the even rows of the other, so the two results
// hold rows (0, 0, 2, 2) and (1, 1, 3, 3): combining them pairs row 0 with
// row 1 and row 2 with row 3.  v_permlane32_swap does the same for the two
// 32-lane halves.
// ---------------------------------------------------------------------------
__device__ __forceinline__ float max_across_halves(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}

__device__ __forceinline__ float sum_across_halves(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// Maximum (sum) of x over the lanes l, l ^ 16, l ^ 32, l ^ 48.
__device__ __forceinline__ float max_across_rows(float x) {
  const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return max_across_halves(fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1])));
}

__device__ __forceinline__ float sum_across_rows(float x) {
  const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return sum_across_halves(__uint_as_float(r[0]) + __uint_as_float(r[1]));
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

}  // namespace pa
