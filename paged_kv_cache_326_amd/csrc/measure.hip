// Measurement helper of libpa.so: a plain streaming read, the bandwidth a
// kernel that only reads can reach at a given launch shape, against which
// the decode kernel (which must read the same bytes) is judged.  Not part
// of the attention path.
#include "pa_common.h"
#include "pa_launch.h"

namespace pa {

namespace {

constexpr int kReadUnroll = 8;  // 16-byte loads per thread per batch (two batches in flight)

// Workgroup w reads bytes [w * per, min((w + 1) * per, total)) of src in
// 16-byte non-temporal loads, lane-contiguous (a wave reads 1 KiB per
// instruction), kReadUnroll loads per thread per batch with the next batch
// issued before the current one is folded into an XOR.  sink[w] receives the
// XOR so the loads cannot be dropped.
__global__ void __launch_bounds__(1024) stream_read_kernel(const u32x4* __restrict__ src, int64_t chunks,
                                                           int64_t per_wg, uint32_t* __restrict__ sink) {
  const int64_t lo = (int64_t)blockIdx.x * per_wg;
  const int64_t hi = lo + per_wg < chunks ? lo + per_wg : chunks;
  const int nt = blockDim.x;
  u32x4 acc = {0, 0, 0, 0};
  u32x4 cur[kReadUnroll], nxt[kReadUnroll];
  auto batch = [&](u32x4 (&b)[kReadUnroll], int64_t base) {
#pragma unroll
    for (int u = 0; u < kReadUnroll; ++u) {
      const int64_t c = base + (int64_t)u * nt + threadIdx.x;
      b[u] = c < hi ? __builtin_nontemporal_load(src + c) : u32x4{0, 0, 0, 0};
    }
  };
  const int64_t step = (int64_t)kReadUnroll * nt;
  batch(cur, lo);
  for (int64_t base = lo; base < hi; base += step) {
    if (base + step < hi) batch(nxt, base + step);
#pragma unroll
    for (int u = 0; u < kReadUnroll; ++u) acc ^= cur[u];
#pragma unroll
    for (int u = 0; u < kReadUnroll; ++u) cur[u] = nxt[u];
  }
  uint32_t x = acc[0] ^ acc[1] ^ acc[2] ^ acc[3];
#pragma unroll
  for (int m = 1; m < 64; m <<= 1) x ^= (uint32_t)__shfl_xor((int)x, m, 64);
  if ((threadIdx.x & 63) == 0) atomicXor(sink + blockIdx.x, x);
}

}  // namespace

hipError_t launch_stream_read(const void* src, int64_t bytes, int workgroups, int threads, uint32_t* sink,
                              hipStream_t stream) {
  const int64_t chunks = bytes / 16;
  const int64_t per = (chunks + workgroups - 1) / workgroups;
  hipLaunchKernelGGL(stream_read_kernel, dim3(workgroups), dim3(threads), 0, stream,
                     reinterpret_cast<const u32x4*>(src), chunks, per, sink);
  return hipGetLastError();
}

}  // namespace pa
