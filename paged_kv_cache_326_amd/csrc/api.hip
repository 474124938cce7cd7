// C ABI of libpa.so: host-side argument checks, partition choice, workspace
// layout and dispatch to the gfx950 kernels.  Every check runs before any
// launch; a failed check launches nothing.
#include <algorithm>
#include <climits>
#include <mutex>
#include <vector>

#include "../../include/pa.h"
#include "pa_launch.h"

namespace {

constexpr int kCUs = 256;  // MI355X compute units

bool supported_shape(int head_dim, int block_size) {
  return (head_dim == 64 || head_dim == 128) && (block_size == 16 || block_size == 32);
}

bool supported_group(int num_heads, int num_kv_heads) {
  if (num_kv_heads <= 0 || num_heads <= 0 || num_heads % num_kv_heads) return false;
  const int g = num_heads / num_kv_heads;
  return g == 1 || g == 2 || g == 4 || g == 8;
}

pa_status check_cache(const pa_kv_cache* c) {
  if (!c || !c->key_cache || !c->value_cache) return PA_ERR_NULL;
  if (c->num_blocks <= 0 || c->num_kv_heads <= 0) return PA_ERR_SHAPE;
  if (!supported_shape(c->head_dim, c->block_size)) return PA_ERR_UNSUPPORTED;
  if (c->dtype != PA_F32 && c->dtype != PA_F16 && c->dtype != PA_BF16 && c->dtype != PA_FP8_E4M3)
    return PA_ERR_UNSUPPORTED;
  if (c->dtype == PA_FP8_E4M3) {
    // Positive and finite (a NaN fails both comparisons).
    if (!(c->k_scale > 0.f && c->k_scale <= 3.4e38f) || !(c->v_scale > 0.f && c->v_scale <= 3.4e38f))
      return PA_ERR_SHAPE;
  }
  return PA_OK;
}

pa::KvCacheArgs to_args(const pa_kv_cache* c) {
  pa::KvCacheArgs a;
  a.key_cache = c->key_cache;
  a.value_cache = c->value_cache;
  a.num_blocks = c->num_blocks;
  a.num_kv_heads = c->num_kv_heads;
  a.head_dim = c->head_dim;
  a.block_size = c->block_size;
  a.dtype = static_cast<pa::DType>(c->dtype);
  a.k_scale = c->dtype == PA_FP8_E4M3 ? c->k_scale : 1.f;
  a.v_scale = c->dtype == PA_FP8_E4M3 ? c->v_scale : 1.f;
  return a;
}

int ceil_div(int64_t a, int64_t b) { return (int)((a + b - 1) / b); }

size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

struct WsLayout {
  size_t m_off, l_off, o_off, bytes;
};

WsLayout ws_layout(int num_seqs, int num_heads, int head_dim, int num_partitions) {
  const size_t rows = (size_t)num_seqs * num_heads * num_partitions;
  WsLayout w;
  w.m_off = 0;
  w.l_off = align256(rows * 4);
  w.o_off = w.l_off + align256(rows * 4);
  w.bytes = w.o_off + align256(rows * head_dim * 4);
  return w;
}

// Decode partials of pa_decode_noalloc: one fixed array per GPU, held until
// the process ends.  Host code never passes this name to a kernel (on the
// host it is a stand-in, not a device address); it uses the address that
// hipGetSymbolAddress reports for the current device.
static __device__ __align__(256) unsigned char scratch[PA_NOALLOC_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

// The scratch address on the current device (looked up once per device),
// or nullptr if the runtime cannot give it.
void* scratch_on_current_device() {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) {
    (void)hipGetLastError();
    return nullptr;
  }
  std::lock_guard<std::mutex> g(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) {
      (void)hipGetLastError();
      return nullptr;
    }
    g_scratch_ptr[dev] = p;
  }
  return g_scratch_ptr[dev];
}

}  // namespace

extern "C" {

const char* pa_status_string(pa_status s) {
  switch (s) {
    case PA_OK: return "ok";
    case PA_ERR_NULL: return "a required pointer is NULL";
    case PA_ERR_SHAPE: return "inconsistent sizes or an invalid scale";
    case PA_ERR_UNSUPPORTED: return "unsupported head_dim, block_size, dtype or head grouping";
    case PA_ERR_WORKSPACE: return "workspace missing or too small";
    case PA_ERR_LAUNCH: return "kernel launch failed";
    case PA_ERR_NO_BLOCKS: return "not enough free blocks in the pool";
    case PA_ERR_NOT_FOUND: return "unknown sequence id";
    case PA_ERR_EXISTS: return "sequence id already in use";
  }
  return "unknown status";
}

const char* pa_version(void) { return "pa-mi355x 0.1.0 (gfx950)"; }

pa_status pa_slot_mapping(const int32_t* block_tables, int32_t max_blocks_per_seq, const int32_t* seq_lens,
                          const int32_t* cu_q_lens, int32_t num_seqs, int32_t block_size, int64_t* slot_mapping,
                          int32_t num_tokens, hipStream_t stream) {
  if (num_seqs < 0 || num_tokens < 0 || max_blocks_per_seq <= 0 || block_size <= 0) return PA_ERR_SHAPE;
  if (num_seqs == 0 || num_tokens == 0) return PA_OK;
  if (!block_tables || !seq_lens || !cu_q_lens || !slot_mapping) return PA_ERR_NULL;
  const hipError_t e = pa::launch_slot_mapping(block_tables, max_blocks_per_seq, seq_lens, cu_q_lens, num_seqs,
                                               block_size, slot_mapping, num_tokens, stream);
  return e == hipSuccess ? PA_OK : PA_ERR_LAUNCH;
}

pa_status pa_reshape_and_cache(const pa_kv_cache* cache, const void* key, const void* value,
                               const int64_t* slot_mapping, int32_t num_tokens, hipStream_t stream) {
  const pa_status st = check_cache(cache);
  if (st != PA_OK) return st;
  if (num_tokens < 0) return PA_ERR_SHAPE;
  if (num_tokens == 0) return PA_OK;
  if (!key || !value || !slot_mapping) return PA_ERR_NULL;
  const hipError_t e = pa::launch_reshape_and_cache(to_args(cache), key, value, slot_mapping, num_tokens, stream);
  return e == hipSuccess ? PA_OK : PA_ERR_LAUNCH;
}

pa_status pa_append_kv(const pa_kv_cache* cache, const void* key, const void* value, const int32_t* block_tables,
                       int32_t max_blocks_per_seq, const int32_t* seq_lens, const int32_t* cu_q_lens,
                       int32_t num_seqs, int32_t max_q_len, int64_t* slot_mapping, int32_t num_tokens,
                       hipStream_t stream) {
  const pa_status st = check_cache(cache);
  if (st != PA_OK) return st;
  if (num_seqs < 0 || num_tokens < 0 || max_q_len < 0 || max_blocks_per_seq <= 0) return PA_ERR_SHAPE;
  if (num_seqs == 0 || num_tokens == 0 || max_q_len == 0) return PA_OK;
  if (!key || !value || !block_tables || !seq_lens || !cu_q_lens || !slot_mapping) return PA_ERR_NULL;
  const hipError_t e = pa::launch_append(to_args(cache), key, value, block_tables, max_blocks_per_seq, seq_lens,
                                         cu_q_lens, num_seqs, max_q_len, slot_mapping, num_tokens, stream);
  return e == hipSuccess ? PA_OK : PA_ERR_LAUNCH;
}

// A staging buffer must be device memory or pinned host memory; the kernel
// reaches pinned memory through its device mapping.  Pageable memory is
// refused here rather than faulting in the kernel.
static bool device_view(void** p) {
  hipPointerAttribute_t at;
  if (hipPointerGetAttributes(&at, *p) != hipSuccess) {
    (void)hipGetLastError();
    return false;
  }
  if (at.type == hipMemoryTypeDevice || at.type == hipMemoryTypeManaged) return true;
  if (at.type != hipMemoryTypeHost) return false;
  void* d = nullptr;
  if (hipHostGetDevicePointer(&d, *p, 0) != hipSuccess || !d) {
    (void)hipGetLastError();
    return false;
  }
  *p = d;
  return true;
}

static pa_status block_move(const pa_kv_cache* cache, const int32_t* a, const int32_t* b, void* kbuf, void* vbuf,
                            int32_t n, int mode, hipStream_t stream) {
  const pa_status st = check_cache(cache);
  if (st != PA_OK) return st;
  if (n < 0) return PA_ERR_SHAPE;
  if (n == 0) return PA_OK;
  if (!a || (mode == 0 && !b) || (mode != 0 && (!kbuf || !vbuf))) return PA_ERR_NULL;
  if (mode != 0 && (!device_view(&kbuf) || !device_view(&vbuf))) return PA_ERR_UNSUPPORTED;
  const hipError_t e = pa::launch_block_move(to_args(cache), a, b, kbuf, vbuf, n, mode, stream);
  return e == hipSuccess ? PA_OK : PA_ERR_LAUNCH;
}

pa_status pa_copy_blocks(const pa_kv_cache* cache, const int32_t* src, const int32_t* dst, int32_t num_pairs,
                         hipStream_t stream) {
  return block_move(cache, src, dst, nullptr, nullptr, num_pairs, 0, stream);
}

pa_status pa_gather_blocks(const pa_kv_cache* cache, const int32_t* block_ids, int32_t num_blocks, void* key_out,
                           void* value_out, hipStream_t stream) {
  return block_move(cache, block_ids, nullptr, key_out, value_out, num_blocks, 1, stream);
}

pa_status pa_scatter_blocks(const pa_kv_cache* cache, const int32_t* block_ids, int32_t num_blocks,
                            const void* key_in, const void* value_in, hipStream_t stream) {
  return block_move(cache, block_ids, nullptr, const_cast<void*>(key_in), const_cast<void*>(value_in), num_blocks, 2,
                    stream);
}

int32_t pa_decode_auto_partition(int32_t num_seqs, int32_t num_kv_heads, int32_t max_seq_len, int32_t block_size) {
  // Few (sequence, KV head) pairs: split every sequence into as many equal
  // partitions as make about one 8-wave workgroup per compute unit, so that
  // one round of workgroups covers the batch with the fewest partials to
  // merge (a single partition when the pairs alone fill the chip).  Many
  // pairs: 1024-token partitions on 4-wave workgroups, halved while that
  // gives fewer than two workgroups per compute unit.
  if (block_size <= 0) return 0;
  const int64_t pairs = (int64_t)(num_seqs > 0 ? num_seqs : 1) * (num_kv_heads > 0 ? num_kv_heads : 1);
  const int64_t L = max_seq_len > 0 ? max_seq_len : 1;
  int64_t p;
  if (pairs <= kCUs) {
    const int64_t np = kCUs / pairs;
    p = (L + np - 1) / np;
    if (p > pa::kMaxPartition) p = pa::kMaxPartition;
  } else {
    p = 1024;
    while (p > 128 && pairs * ((L + p - 1) / p) < 2 * kCUs) p /= 2;
  }
  p = (p + block_size - 1) / block_size * block_size;
  if (p > pa::kMaxPartition) p -= block_size;
  return (int32_t)p;
}

size_t pa_decode_workspace_bytes(int32_t num_seqs, int32_t num_heads, int32_t num_kv_heads, int32_t head_dim,
                                 int32_t block_size, int32_t max_seq_len, int32_t partition_size) {
  if (num_seqs < 0 || num_heads <= 0 || head_dim <= 0 || block_size <= 0 || max_seq_len < 0) return 0;
  int p = partition_size;
  if (p == 0) p = pa_decode_auto_partition(num_seqs, num_kv_heads, max_seq_len, block_size);
  if (p <= 0 || max_seq_len <= p) return 0;
  return ws_layout(num_seqs, num_heads, head_dim, ceil_div(max_seq_len, p)).bytes;
}

static pa_status decode_run(const pa_decode_args* d, hipStream_t stream) {
  if (!d) return PA_ERR_NULL;
  const pa_kv_cache* cache = d->cache;
  const pa_status st = check_cache(cache);
  if (st != PA_OK) return st;
  if (d->stage < 0 || d->stage > 2) return PA_ERR_SHAPE;
  const int32_t num_seqs = d->num_seqs, num_heads = d->num_heads, max_seq_len = d->max_seq_len;
  if (num_seqs < 0 || max_seq_len < 0 || d->max_blocks_per_seq <= 0 || d->num_work < 0) return PA_ERR_SHAPE;
  if (!supported_group(num_heads, cache->num_kv_heads)) {
    return (num_heads > 0 && num_heads % cache->num_kv_heads == 0) ? PA_ERR_UNSUPPORTED : PA_ERR_SHAPE;
  }
  if ((int64_t)max_seq_len > (int64_t)d->max_blocks_per_seq * cache->block_size) return PA_ERR_SHAPE;
  int p = d->partition_size;
  if (p == 0) p = pa_decode_auto_partition(num_seqs, cache->num_kv_heads, max_seq_len, cache->block_size);
  if (p <= 0 || p % cache->block_size || p > pa::kMaxPartition) return PA_ERR_SHAPE;
  if (num_seqs == 0) return PA_OK;
  if (!d->out || !d->query || !d->block_tables || !d->seq_lens) return PA_ERR_NULL;
  const bool append = d->new_key || d->new_value || d->slot_mapping;
  if (append && (!d->new_key || !d->new_value || !d->slot_mapping)) return PA_ERR_NULL;
  if (d->work && d->num_work == 0) return PA_ERR_SHAPE;  // a plan always holds partition 0 of every sequence

  pa::DecodeArgs a{};
  a.cache = to_args(cache);
  a.out = d->out;
  a.query = d->query;
  a.block_tables = d->block_tables;
  a.max_blocks = d->max_blocks_per_seq;
  a.seq_lens = d->seq_lens;
  a.num_seqs = num_seqs;
  a.num_heads = num_heads;
  a.max_seq_len = max_seq_len;
  a.scale = d->scale;
  a.partition = p;
  a.num_partitions = max_seq_len > 0 ? ceil_div(max_seq_len, p) : 1;
  a.work = d->work;
  a.num_work = d->work ? d->num_work : 0;
  // With at most two partitions per sequence the full grid's order (last
  // partitions first) is already longest-first; the order made on the device
  // pays off from three on.
  a.device_plan = !d->work && a.num_partitions > 2 && num_seqs <= pa::kDevicePlanSeqs;
  // 8-wave workgroups (one per compute unit) when the workgroups fit in one
  // round of the chip, else 4-wave ones (three per compute unit).
  const int64_t units = d->work ? (int64_t)d->num_work : (int64_t)num_seqs * a.num_partitions;
  a.waves = units * cache->num_kv_heads <= kCUs ? 8 : 4;
  a.t0 = d->kernel_start;
  a.t1 = d->kernel_stop;
  a.new_key = d->new_key;
  a.new_value = d->new_value;
  a.slots = d->slot_mapping;
  if (max_seq_len > p) {
    const WsLayout wl = ws_layout(num_seqs, num_heads, cache->head_dim, a.num_partitions);
    if (!d->workspace || d->workspace_bytes < wl.bytes) return PA_ERR_WORKSPACE;
    char* base = static_cast<char*>(d->workspace);
    a.ws_m = reinterpret_cast<float*>(base + wl.m_off);
    a.ws_l = reinterpret_cast<float*>(base + wl.l_off);
    a.ws_o = reinterpret_cast<float*>(base + wl.o_off);
  }
  const hipError_t e = pa::launch_decode(a, d->stage, stream);
  return e == hipSuccess ? PA_OK : PA_ERR_LAUNCH;
}

static pa_decode_args basic_args(const pa_kv_cache* cache, void* out, const void* query, const int32_t* block_tables,
                                 int32_t max_blocks_per_seq, const int32_t* seq_lens, int32_t num_seqs,
                                 int32_t num_heads, int32_t max_seq_len, float scale, void* workspace,
                                 size_t workspace_bytes, int32_t partition_size) {
  pa_decode_args d{};
  d.cache = cache;
  d.out = out;
  d.query = query;
  d.block_tables = block_tables;
  d.max_blocks_per_seq = max_blocks_per_seq;
  d.seq_lens = seq_lens;
  d.num_seqs = num_seqs;
  d.num_heads = num_heads;
  d.max_seq_len = max_seq_len;
  d.scale = scale;
  d.workspace = workspace;
  d.workspace_bytes = workspace_bytes;
  d.partition_size = partition_size;
  return d;
}

pa_status pa_decode_run(const pa_decode_args* args, hipStream_t stream) { return decode_run(args, stream); }

int32_t pa_decode_plan(const int32_t* seq_lens_host, int32_t num_seqs, int32_t max_seq_len, int32_t partition_size,
                       int32_t* work, int32_t capacity) {
  if (num_seqs < 0 || max_seq_len < 0 || partition_size <= 0 || (num_seqs > 0 && !seq_lens_host)) return -1;
  const int64_t P = partition_size;
  const int64_t np = max_seq_len > 0 ? (max_seq_len + P - 1) / P : 1;
  struct Unit {
    int64_t size, s, part;
  };
  std::vector<Unit> units;
  for (int32_t s = 0; s < num_seqs; ++s) {
    int64_t L = seq_lens_host[s];
    L = L < 0 ? 0 : (L > max_seq_len ? max_seq_len : L);
    const int64_t parts = L > 0 ? (L + P - 1) / P : 1;  // partition 0 even when empty: it writes the zeros
    for (int64_t q = 0; q < parts; ++q) units.push_back({std::min(P, L - q * P), s, q});
  }
  if (units.size() > (size_t)INT32_MAX / 2 || (int64_t)num_seqs * np > INT32_MAX) return -1;
  std::stable_sort(units.begin(), units.end(), [](const Unit& x, const Unit& y) { return x.size > y.size; });
  const int32_t n = (int32_t)units.size();
  if (work && capacity >= n)
    for (int32_t k = 0; k < n; ++k) work[k] = (int32_t)(units[k].s * np + units[k].part);
  return n;
}

pa_status pa_decode_noalloc(const pa_kv_cache* cache, void* out, const void* query, const int32_t* block_tables,
                            int32_t max_blocks_per_seq, const int32_t* seq_lens, int32_t num_seqs, int32_t num_heads,
                            int32_t max_seq_len, float scale, int32_t partition_size, hipStream_t stream) {
  const pa_status st = check_cache(cache);
  if (st != PA_OK) return st;
  if (num_seqs < 0 || max_seq_len < 0 || num_heads <= 0) return PA_ERR_SHAPE;
  const size_t need = pa_decode_workspace_bytes(num_seqs, num_heads, cache->num_kv_heads, cache->head_dim,
                                                cache->block_size, max_seq_len, partition_size);
  if (need > PA_NOALLOC_SCRATCH_BYTES) return PA_ERR_WORKSPACE;
  pa_decode_args d = basic_args(cache, out, query, block_tables, max_blocks_per_seq, seq_lens, num_seqs, num_heads,
                                max_seq_len, scale, nullptr, 0, partition_size);
  if (need > 0 && num_seqs > 0) {
    void* ws = scratch_on_current_device();
    if (!ws) return PA_ERR_LAUNCH;
    d.workspace = ws;
    d.workspace_bytes = PA_NOALLOC_SCRATCH_BYTES;
  }
  return decode_run(&d, stream);
}

pa_status pa_stream_read(const void* src, size_t bytes, int32_t workgroups, int32_t threads, uint32_t* sink,
                         hipStream_t stream) {
  if (workgroups <= 0 || threads <= 0 || threads > 1024 || threads % 64 || bytes % 16) return PA_ERR_SHAPE;
  if (bytes == 0) return PA_OK;
  if (!src || !sink) return PA_ERR_NULL;
  if (reinterpret_cast<uintptr_t>(src) % 16) return PA_ERR_SHAPE;
  const hipError_t e = pa::launch_stream_read(src, (int64_t)bytes, workgroups, threads, sink, stream);
  return e == hipSuccess ? PA_OK : PA_ERR_LAUNCH;
}

pa_status pa_decode_ex(const pa_kv_cache* cache, void* out, const void* query, const int32_t* block_tables,
                       int32_t max_blocks_per_seq, const int32_t* seq_lens, int32_t num_seqs, int32_t num_heads,
                       int32_t max_seq_len, float scale, void* workspace, size_t workspace_bytes,
                       int32_t partition_size, hipStream_t stream) {
  const pa_decode_args d = basic_args(cache, out, query, block_tables, max_blocks_per_seq, seq_lens, num_seqs,
                                      num_heads, max_seq_len, scale, workspace, workspace_bytes, partition_size);
  return decode_run(&d, stream);
}

pa_status pa_decode_timed(const pa_kv_cache* cache, void* out, const void* query, const int32_t* block_tables,
                          int32_t max_blocks_per_seq, const int32_t* seq_lens, int32_t num_seqs, int32_t num_heads,
                          int32_t max_seq_len, float scale, void* workspace, size_t workspace_bytes,
                          int32_t partition_size, hipEvent_t kernel_start, hipEvent_t kernel_stop,
                          hipStream_t stream) {
  pa_decode_args d = basic_args(cache, out, query, block_tables, max_blocks_per_seq, seq_lens, num_seqs, num_heads,
                                max_seq_len, scale, workspace, workspace_bytes, partition_size);
  d.kernel_start = kernel_start;
  d.kernel_stop = kernel_stop;
  return decode_run(&d, stream);
}

pa_status pa_decode_stage(const pa_kv_cache* cache, void* out, const void* query, const int32_t* block_tables,
                          int32_t max_blocks_per_seq, const int32_t* seq_lens, int32_t num_seqs, int32_t num_heads,
                          int32_t max_seq_len, float scale, void* workspace, size_t workspace_bytes,
                          int32_t partition_size, int32_t stage, hipStream_t stream) {
  if (stage != 1 && stage != 2) return PA_ERR_SHAPE;
  pa_decode_args d = basic_args(cache, out, query, block_tables, max_blocks_per_seq, seq_lens, num_seqs, num_heads,
                                max_seq_len, scale, workspace, workspace_bytes, partition_size);
  d.stage = stage;
  return decode_run(&d, stream);
}

pa_status pa_decode(const pa_kv_cache* cache, void* out, const void* query, const int32_t* block_tables,
                    int32_t max_blocks_per_seq, const int32_t* seq_lens, int32_t num_seqs, int32_t num_heads,
                    int32_t max_seq_len, float scale, void* workspace, size_t workspace_bytes,
                    hipStream_t stream) {
  return pa_decode_ex(cache, out, query, block_tables, max_blocks_per_seq, seq_lens, num_seqs, num_heads,
                      max_seq_len, scale, workspace, workspace_bytes, 0, stream);
}

pa_status pa_prefill_chunk(const pa_kv_cache* cache, void* out, const void* query, const int32_t* cu_q_lens,
                           const int32_t* seq_lens, const int32_t* block_tables, int32_t max_blocks_per_seq,
                           int32_t num_seqs, int32_t num_heads, int32_t max_q_len, float scale, hipStream_t stream) {
  const pa_status st = check_cache(cache);
  if (st != PA_OK) return st;
  if (cache->dtype != PA_F16 && cache->dtype != PA_BF16 && cache->dtype != PA_FP8_E4M3) return PA_ERR_UNSUPPORTED;
  if (num_seqs < 0 || max_q_len < 0 || max_blocks_per_seq <= 0) return PA_ERR_SHAPE;
  if (!supported_group(num_heads, cache->num_kv_heads)) {
    return (num_heads > 0 && num_heads % cache->num_kv_heads == 0) ? PA_ERR_UNSUPPORTED : PA_ERR_SHAPE;
  }
  if (num_seqs == 0 || max_q_len == 0) return PA_OK;
  if (!out || !query || !cu_q_lens || !seq_lens || !block_tables) return PA_ERR_NULL;
  pa::PrefillArgs a{};
  a.cache = to_args(cache);
  a.out = out;
  a.query = query;
  a.cu_q_lens = cu_q_lens;
  a.seq_lens = seq_lens;
  a.block_tables = block_tables;
  a.max_blocks = max_blocks_per_seq;
  a.num_seqs = num_seqs;
  a.num_heads = num_heads;
  a.num_qtiles = ceil_div(max_q_len, pa::prefill_positions_per_tile(num_heads / cache->num_kv_heads));
  a.scale = scale;
  const hipError_t e = pa::launch_prefill(a, stream);
  return e == hipSuccess ? PA_OK : PA_ERR_LAUNCH;
}

pa_status pa_decode_append(const pa_kv_cache* cache, const void* new_key, const void* new_value,
                           int64_t* slot_mapping, void* out, const void* query, const int32_t* block_tables,
                           int32_t max_blocks_per_seq, const int32_t* seq_lens, int32_t num_seqs, int32_t num_heads,
                           int32_t max_seq_len, float scale, void* workspace, size_t workspace_bytes,
                           int32_t partition_size, hipEvent_t kernel_start, hipEvent_t kernel_stop,
                           hipStream_t stream) {
  if (num_seqs > 0 && (!new_key || !new_value || !slot_mapping)) return PA_ERR_NULL;
  pa_decode_args d = basic_args(cache, out, query, block_tables, max_blocks_per_seq, seq_lens, num_seqs, num_heads,
                                max_seq_len, scale, workspace, workspace_bytes, partition_size);
  d.kernel_start = kernel_start;
  d.kernel_stop = kernel_stop;
  d.new_key = new_key;
  d.new_value = new_value;
  d.slot_mapping = slot_mapping;
  return decode_run(&d, stream);
}

}  // extern "C"
