// Host-side block manager of libpa.so: the physical-block pool, per-sequence
// block tables, reference-counted sharing and copy-on-write.
//
// Sources:
//   [P1] "大模型推理内存优化从 KV Cache 分页到连续批处理的工程实践", section
//        "生产级推理引擎的内存管理与调度": a FIFO pool of block IDs (take from
//        the front, return to the back); a sequence of n tokens needs
//        ceil(n / block_size) blocks; a request that cannot get a block is
//        preempted (here: the call fails and changes nothing).
//        Section "KV Cache 的内存开销与分页机制": block-level sharing of a
//        common prefix between the outputs of parallel sampling.
//   [P2] "KV Cache管理优化：大模型推理显存瓶颈突破", section 4.1: a shared
//        block carries a reference count and returns to the pool when the
//        last reference is released.
//
// Copy-on-write is the reading taken where the pages are silent: a sequence
// that shares its partly filled last block and is about to write into it
// first gets a private copy (the caller copies the block's contents with
// pa_copy_blocks before the scatter).
#include <cstdint>
#include <deque>
#include <mutex>
#include <unordered_map>
#include <vector>

#include "../../include/pa.h"

struct pa_block_manager {
  int32_t num_blocks = 0;
  int32_t block_size = 0;
  std::deque<int32_t> free_list;
  std::vector<int32_t> refcount;
  struct Seq {
    std::vector<int32_t> table;
    int64_t num_tokens = 0;
  };
  std::unordered_map<int64_t, Seq> seqs;
  std::mutex mu;
};

namespace {

int64_t blocks_for(int64_t tokens, int32_t block_size) { return (tokens + block_size - 1) / block_size; }

int32_t take(pa_block_manager* m) {
  const int32_t b = m->free_list.front();
  m->free_list.pop_front();
  m->refcount[b] = 1;
  return b;
}

void release(pa_block_manager* m, int32_t b) {
  if (--m->refcount[b] == 0) m->free_list.push_back(b);
}

}  // namespace

extern "C" {

pa_block_manager* pa_bm_create(int32_t num_blocks, int32_t block_size, const int32_t* free_order) {
  if (num_blocks <= 0 || block_size <= 0) return nullptr;
  auto* m = new pa_block_manager;
  m->num_blocks = num_blocks;
  m->block_size = block_size;
  m->refcount.assign(num_blocks, 0);
  if (free_order) {
    // Must be a permutation of 0 .. num_blocks-1.
    std::vector<char> seen(num_blocks, 0);
    for (int32_t i = 0; i < num_blocks; ++i) {
      const int32_t b = free_order[i];
      if (b < 0 || b >= num_blocks || seen[b]) {
        delete m;
        return nullptr;
      }
      seen[b] = 1;
      m->free_list.push_back(b);
    }
  } else {
    for (int32_t b = 0; b < num_blocks; ++b) m->free_list.push_back(b);
  }
  return m;
}

void pa_bm_destroy(pa_block_manager* m) { delete m; }

int32_t pa_bm_available(pa_block_manager* m) {
  if (!m) return -1;
  std::lock_guard<std::mutex> g(m->mu);
  return (int32_t)m->free_list.size();
}

int32_t pa_bm_refcount(pa_block_manager* m, int32_t block) {
  if (!m || block < 0 || block >= m->num_blocks) return -1;
  std::lock_guard<std::mutex> g(m->mu);
  return m->refcount[block];
}

pa_status pa_bm_add_sequence(pa_block_manager* m, int64_t seq_id, int32_t num_tokens) {
  if (!m) return PA_ERR_NULL;
  if (num_tokens < 0) return PA_ERR_SHAPE;
  std::lock_guard<std::mutex> g(m->mu);
  if (m->seqs.count(seq_id)) return PA_ERR_EXISTS;
  const int64_t need = blocks_for(num_tokens, m->block_size);
  if (need > (int64_t)m->free_list.size()) return PA_ERR_NO_BLOCKS;
  auto& s = m->seqs[seq_id];
  s.num_tokens = num_tokens;
  s.table.reserve(need);
  for (int64_t i = 0; i < need; ++i) s.table.push_back(take(m));
  return PA_OK;
}

pa_status pa_bm_fork(pa_block_manager* m, int64_t parent, int64_t child) {
  if (!m) return PA_ERR_NULL;
  std::lock_guard<std::mutex> g(m->mu);
  auto it = m->seqs.find(parent);
  if (it == m->seqs.end()) return PA_ERR_NOT_FOUND;
  if (m->seqs.count(child)) return PA_ERR_EXISTS;
  const auto copy = it->second;  // table and length
  for (int32_t b : copy.table) ++m->refcount[b];
  m->seqs[child] = copy;
  return PA_OK;
}

pa_status pa_bm_append_tokens(pa_block_manager* m, int64_t seq_id, int32_t num_new, int32_t* copy_src,
                              int32_t* copy_dst, int32_t* num_copies) {
  if (!m) return PA_ERR_NULL;
  if (num_new < 0) return PA_ERR_SHAPE;
  std::lock_guard<std::mutex> g(m->mu);
  auto it = m->seqs.find(seq_id);
  if (it == m->seqs.end()) return PA_ERR_NOT_FOUND;
  auto& s = it->second;
  if (num_copies) *num_copies = 0;
  if (num_new == 0) return PA_OK;
  const int32_t B = m->block_size;
  // A partly filled last block that other sequences share is written next:
  // it needs a private copy first.
  const bool cow = s.num_tokens % B != 0 && m->refcount[s.table.back()] > 1;
  const int64_t grow = blocks_for(s.num_tokens + num_new, B) - (int64_t)s.table.size();
  const int64_t need = grow + (cow ? 1 : 0);
  if (need > (int64_t)m->free_list.size()) return PA_ERR_NO_BLOCKS;  // nothing changed: the caller preempts
  if (cow && (!copy_src || !copy_dst || !num_copies)) return PA_ERR_NULL;
  if (cow) {
    const int32_t old = s.table.back();
    const int32_t fresh = take(m);
    release(m, old);
    s.table.back() = fresh;
    copy_src[0] = old;
    copy_dst[0] = fresh;
    *num_copies = 1;
  }
  for (int64_t i = 0; i < grow; ++i) s.table.push_back(take(m));
  s.num_tokens += num_new;
  return PA_OK;
}

pa_status pa_bm_free_sequence(pa_block_manager* m, int64_t seq_id) {
  if (!m) return PA_ERR_NULL;
  std::lock_guard<std::mutex> g(m->mu);
  auto it = m->seqs.find(seq_id);
  if (it == m->seqs.end()) return PA_ERR_NOT_FOUND;
  for (int32_t b : it->second.table) release(m, b);
  m->seqs.erase(it);
  return PA_OK;
}

int32_t pa_bm_block_table(pa_block_manager* m, int64_t seq_id, int32_t* out, int32_t capacity) {
  if (!m) return -1;
  std::lock_guard<std::mutex> g(m->mu);
  auto it = m->seqs.find(seq_id);
  if (it == m->seqs.end()) return -1;
  const auto& t = it->second.table;
  for (int32_t i = 0; i < capacity && i < (int32_t)t.size(); ++i) out[i] = t[i];
  return (int32_t)t.size();
}

int64_t pa_bm_num_tokens(pa_block_manager* m, int64_t seq_id) {
  if (!m) return -1;
  std::lock_guard<std::mutex> g(m->mu);
  auto it = m->seqs.find(seq_id);
  return it == m->seqs.end() ? -1 : it->second.num_tokens;
}

int32_t pa_bm_free_list(pa_block_manager* m, int32_t* out, int32_t capacity) {
  if (!m) return -1;
  std::lock_guard<std::mutex> g(m->mu);
  int32_t i = 0;
  for (auto it = m->free_list.begin(); it != m->free_list.end() && i < capacity; ++it) out[i++] = *it;
  return (int32_t)m->free_list.size();
}

}  // extern "C"
