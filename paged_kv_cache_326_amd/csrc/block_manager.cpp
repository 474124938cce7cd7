// Host-side block manager of libpa.so: the physical-block pool, per-sequence
// block tables, reference-counted sharing, copy-on-write and a prefix cache.
//
// Sources:
//   [P1] "大模型推理内存优化从 KV Cache 分页到连续批处理的工程实践", section
//        "生产级推理引擎的内存管理与调度": a FIFO pool of block IDs (take from
//        the front, return to the back); a sequence of n tokens needs
//        ceil(n / block_size) blocks; a request that cannot get a block is
//        preempted (here: the call fails and changes nothing).
//        Section "KV Cache 的内存开销与分页机制": block-level sharing of a
//        common prefix between the outputs of parallel sampling.
//        Section "工程边界与架构取舍": requests with the same system prompt
//        reuse the prefix's blocks; cached prefixes are marked by hash values
//        and carry a version, and a hash collision must not produce a wrong
//        hit.
//   [P2] "KV Cache管理优化：大模型推理显存瓶颈突破", section 4.1: a shared
//        block carries a reference count and returns to the pool when the
//        last reference is released.
//
// Readings where the pages are silent:
//   * Copy-on-write: a sequence that shares its partly filled last block and
//     is about to write into it first gets a private copy (the caller copies
//     the block's contents with pa_copy_blocks before the scatter).
//   * Prefix cache: only full blocks are cached, and only once the caller
//     reports their K/V written (pa_bm_commit).  A block's key is the exact
//     token prefix it ends plus a version; it is found through a chained
//     64-bit hash (parent hash, version, the block's token ids), and a hit is
//     accepted only if version, parent block and token ids all match, so a
//     collision can only cost a miss.  Every cached block's parent is cached:
//     uncaching a block uncaches its descendants.  A cached block whose last
//     reference goes stays cached in the free list; a lookup hit takes it
//     back out, and a fresh allocation that pops it from the front uncaches
//     it (FIFO eviction).
#include <cstdint>
#include <mutex>
#include <unordered_map>
#include <vector>

#include "../../include/pa.h"

struct pa_block_manager {
  int32_t num_blocks = 0;
  int32_t block_size = 0;

  // FIFO free list, doubly linked through the block ids so that a block the
  // prefix cache revives leaves it in O(1) while the order of the rest stays.
  std::vector<int32_t> next, prev;
  std::vector<char> in_free;
  int32_t head = -1, tail = -1, nfree = 0;

  std::vector<int32_t> refcount;

  struct Cached {
    bool reg = false;
    uint64_t hash = 0;
    uint64_t version = 0;
    int32_t parent = -1;
    std::vector<int32_t> tokens;    // the block's token ids
    std::vector<int32_t> children;  // cached blocks whose parent this is
  };
  std::vector<Cached> cache;  // per block
  std::unordered_multimap<uint64_t, int32_t> index;
  int32_t num_cached = 0;
  int hash_bits = 64;

  struct Seq {
    std::vector<int32_t> table;
    int64_t num_tokens = 0;
    std::vector<int32_t> ids;  // token ids, complete when has_ids
    bool has_ids = false;
    uint64_t version = 0;
  };
  std::unordered_map<int64_t, Seq> seqs;
  std::mutex mu;
};

namespace {

using M = pa_block_manager;

int64_t blocks_for(int64_t tokens, int32_t block_size) { return (tokens + block_size - 1) / block_size; }

void push_back(M* m, int32_t b) {
  m->next[b] = -1;
  m->prev[b] = m->tail;
  if (m->tail >= 0) m->next[m->tail] = b;
  else m->head = b;
  m->tail = b;
  m->in_free[b] = 1;
  ++m->nfree;
}

void unlink(M* m, int32_t b) {
  const int32_t p = m->prev[b], n = m->next[b];
  if (p >= 0) m->next[p] = n;
  else m->head = n;
  if (n >= 0) m->prev[n] = p;
  else m->tail = p;
  m->in_free[b] = 0;
  --m->nfree;
}

// Uncache block b and every cached descendant (the cache keeps no child
// whose parent is gone).
void uncache(M* m, int32_t b) {
  std::vector<int32_t> stack{b};
  const int32_t parent = m->cache[b].parent;
  if (parent >= 0) {
    auto& ch = m->cache[parent].children;
    for (size_t i = 0; i < ch.size(); ++i)
      if (ch[i] == b) {
        ch[i] = ch.back();
        ch.pop_back();
        break;
      }
  }
  while (!stack.empty()) {
    const int32_t x = stack.back();
    stack.pop_back();
    auto& c = m->cache[x];
    if (!c.reg) continue;
    auto range = m->index.equal_range(c.hash);
    for (auto it = range.first; it != range.second; ++it)
      if (it->second == x) {
        m->index.erase(it);
        break;
      }
    for (int32_t k : c.children) stack.push_back(k);
    c = M::Cached{};
    --m->num_cached;
  }
}

// A fresh block from the front of the free list (the caller checked nfree).
int32_t take(M* m) {
  const int32_t b = m->head;
  unlink(m, b);
  if (m->cache[b].reg) uncache(m, b);
  m->refcount[b] = 1;
  return b;
}

void add_ref(M* m, int32_t b) {
  if (m->refcount[b] == 0) unlink(m, b);  // a cached block back from the free list
  ++m->refcount[b];
}

void release(M* m, int32_t b) {
  if (--m->refcount[b] == 0) push_back(m, b);
}

uint64_t mix(uint64_t x) {  // splitmix64 finaliser
  x += 0x9e3779b97f4a7c15ull;
  x = (x ^ (x >> 30)) * 0xbf58476d1ce4e5b9ull;
  x = (x ^ (x >> 27)) * 0x94d049bb133111ebull;
  return x ^ (x >> 31);
}

uint64_t block_hash(const M* m, uint64_t parent_hash, uint64_t version, const int32_t* t) {
  uint64_t h = mix(parent_hash ^ mix(version));
  for (int32_t i = 0; i < m->block_size; ++i) h = mix(h ^ (uint64_t)(uint32_t)t[i] ^ ((uint64_t)i << 32));
  return m->hash_bits >= 64 ? h : (h & ((1ull << m->hash_bits) - 1));
}

// The cached block holding `t` after `parent` (-1: first block) for this
// version, or -1.
int32_t lookup(const M* m, uint64_t h, uint64_t version, int32_t parent, const int32_t* t) {
  auto range = m->index.equal_range(h);
  for (auto it = range.first; it != range.second; ++it) {
    const auto& c = m->cache[it->second];
    if (c.version != version || c.parent != parent) continue;
    bool same = true;
    for (int32_t i = 0; i < m->block_size && same; ++i) same = c.tokens[i] == t[i];
    if (same) return it->second;
  }
  return -1;
}

}  // namespace

extern "C" {

pa_block_manager* pa_bm_create(int32_t num_blocks, int32_t block_size, const int32_t* free_order) {
  if (num_blocks <= 0 || block_size <= 0) return nullptr;
  auto* m = new pa_block_manager;
  m->num_blocks = num_blocks;
  m->block_size = block_size;
  m->refcount.assign(num_blocks, 0);
  m->next.assign(num_blocks, -1);
  m->prev.assign(num_blocks, -1);
  m->in_free.assign(num_blocks, 0);
  m->cache.resize(num_blocks);
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
    }
    for (int32_t i = 0; i < num_blocks; ++i) push_back(m, free_order[i]);
  } else {
    for (int32_t b = 0; b < num_blocks; ++b) push_back(m, b);
  }
  return m;
}

void pa_bm_destroy(pa_block_manager* m) { delete m; }

int32_t pa_bm_block_size(pa_block_manager* m) { return m ? m->block_size : -1; }

int32_t pa_bm_available(pa_block_manager* m) {
  if (!m) return -1;
  std::lock_guard<std::mutex> g(m->mu);
  return m->nfree;
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
  if (need > m->nfree) return PA_ERR_NO_BLOCKS;
  auto& s = m->seqs[seq_id];
  s.num_tokens = num_tokens;
  s.table.reserve(need);
  for (int64_t i = 0; i < need; ++i) s.table.push_back(take(m));
  return PA_OK;
}

pa_status pa_bm_add_sequence_tokens(pa_block_manager* m, int64_t seq_id, const int32_t* token_ids,
                                    int32_t num_tokens, uint64_t version, int32_t* num_cached_tokens) {
  if (!m) return PA_ERR_NULL;
  if (num_tokens < 0) return PA_ERR_SHAPE;
  if (num_tokens > 0 && !token_ids) return PA_ERR_NULL;
  std::lock_guard<std::mutex> g(m->mu);
  if (m->seqs.count(seq_id)) return PA_ERR_EXISTS;
  const int32_t B = m->block_size;
  const int64_t need = blocks_for(num_tokens, B);
  // Leading full blocks already cached for this version and prefix.  The
  // search stops one token short of the end: the prompt's last token is
  // always computed (its logits start generation), so the block it lies in
  // must be private, never a shared cached block.
  std::vector<int32_t> hits;
  int64_t revived = 0;
  int32_t parent = -1;
  uint64_t ph = 0;
  const int64_t searchable = num_tokens > 0 ? (num_tokens - 1) / B : 0;
  for (int64_t i = 0; i < searchable; ++i) {
    const int32_t* t = token_ids + i * B;
    const uint64_t h = block_hash(m, ph, version, t);
    const int32_t c = lookup(m, h, version, parent, t);
    if (c < 0) break;
    hits.push_back(c);
    revived += m->refcount[c] == 0;
    parent = c;
    ph = h;
  }
  if (need - (int64_t)hits.size() > m->nfree - revived) return PA_ERR_NO_BLOCKS;  // nothing changed
  for (int32_t c : hits) add_ref(m, c);
  auto& s = m->seqs[seq_id];
  s.table = hits;
  for (int64_t i = (int64_t)hits.size(); i < need; ++i) s.table.push_back(take(m));
  s.num_tokens = num_tokens;
  s.ids.assign(token_ids, token_ids + num_tokens);
  s.has_ids = true;
  s.version = version;
  if (num_cached_tokens) *num_cached_tokens = (int32_t)hits.size() * B;
  return PA_OK;
}

pa_status pa_bm_fork(pa_block_manager* m, int64_t parent, int64_t child) {
  if (!m) return PA_ERR_NULL;
  std::lock_guard<std::mutex> g(m->mu);
  auto it = m->seqs.find(parent);
  if (it == m->seqs.end()) return PA_ERR_NOT_FOUND;
  if (m->seqs.count(child)) return PA_ERR_EXISTS;
  const auto copy = it->second;  // table, length, token ids, version
  for (int32_t b : copy.table) ++m->refcount[b];
  m->seqs[child] = copy;
  return PA_OK;
}

static pa_status append(pa_block_manager* m, int64_t seq_id, int32_t num_new, const int32_t* ids, int32_t* copy_src,
                        int32_t* copy_dst, int32_t* num_copies) {
  if (!m) return PA_ERR_NULL;
  if (num_new < 0) return PA_ERR_SHAPE;
  std::lock_guard<std::mutex> g(m->mu);
  auto it = m->seqs.find(seq_id);
  if (it == m->seqs.end()) return PA_ERR_NOT_FOUND;
  auto& s = it->second;
  if (ids && !s.has_ids) return PA_ERR_SHAPE;  // earlier tokens have no ids
  if (num_copies) *num_copies = 0;
  if (num_new == 0) return PA_OK;
  const int32_t B = m->block_size;
  // A partly filled last block that other sequences share is written next:
  // it needs a private copy first.  (A partly filled block is never cached.)
  const bool cow = s.num_tokens % B != 0 && m->refcount[s.table.back()] > 1;
  const int64_t grow = blocks_for(s.num_tokens + num_new, B) - (int64_t)s.table.size();
  const int64_t need = grow + (cow ? 1 : 0);
  if (need > m->nfree) return PA_ERR_NO_BLOCKS;  // nothing changed: the caller preempts
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
  if (ids) s.ids.insert(s.ids.end(), ids, ids + num_new);
  else s.has_ids = false;
  return PA_OK;
}

pa_status pa_bm_append_tokens(pa_block_manager* m, int64_t seq_id, int32_t num_new, int32_t* copy_src,
                              int32_t* copy_dst, int32_t* num_copies) {
  return append(m, seq_id, num_new, nullptr, copy_src, copy_dst, num_copies);
}

pa_status pa_bm_append_token_ids(pa_block_manager* m, int64_t seq_id, const int32_t* token_ids, int32_t num_new,
                                 int32_t* copy_src, int32_t* copy_dst, int32_t* num_copies) {
  if (num_new > 0 && !token_ids) return PA_ERR_NULL;
  return append(m, seq_id, num_new, num_new > 0 ? token_ids : nullptr, copy_src, copy_dst, num_copies);
}

pa_status pa_bm_commit(pa_block_manager* m, int64_t seq_id, int32_t num_computed_tokens) {
  if (!m) return PA_ERR_NULL;
  std::lock_guard<std::mutex> g(m->mu);
  auto it = m->seqs.find(seq_id);
  if (it == m->seqs.end()) return PA_ERR_NOT_FOUND;
  auto& s = it->second;
  if (num_computed_tokens < 0 || num_computed_tokens > s.num_tokens) return PA_ERR_SHAPE;
  const int32_t B = m->block_size;
  const int64_t full = num_computed_tokens / B;
  if (full > 0 && !s.has_ids) return PA_ERR_SHAPE;
  for (int64_t i = 0; i < full; ++i) {
    const int32_t b = s.table[i];
    if (m->cache[b].reg) continue;  // a hit, or committed before
    const int32_t parent = i > 0 ? s.table[i - 1] : -1;
    if (parent >= 0 && !m->cache[parent].reg) break;  // its parent is not cached
    const int32_t* t = s.ids.data() + i * B;
    const uint64_t h = block_hash(m, parent >= 0 ? m->cache[parent].hash : 0, s.version, t);
    if (lookup(m, h, s.version, parent, t) >= 0) break;  // the same prefix is cached in another block
    auto& c = m->cache[b];
    c.reg = true;
    c.hash = h;
    c.version = s.version;
    c.parent = parent;
    c.tokens.assign(t, t + B);
    c.children.clear();
    if (parent >= 0) m->cache[parent].children.push_back(b);
    m->index.emplace(h, b);
    ++m->num_cached;
  }
  return PA_OK;
}

int32_t pa_bm_drop_version(pa_block_manager* m, uint64_t version) {
  if (!m) return -1;
  std::lock_guard<std::mutex> g(m->mu);
  const int32_t before = m->num_cached;
  for (int32_t b = 0; b < m->num_blocks; ++b)
    if (m->cache[b].reg && m->cache[b].version == version) uncache(m, b);
  return before - m->num_cached;
}

int32_t pa_bm_cached_blocks(pa_block_manager* m) {
  if (!m) return -1;
  std::lock_guard<std::mutex> g(m->mu);
  return m->num_cached;
}

int32_t pa_bm_is_cached(pa_block_manager* m, int32_t block) {
  if (!m || block < 0 || block >= m->num_blocks) return -1;
  std::lock_guard<std::mutex> g(m->mu);
  return m->cache[block].reg ? 1 : 0;
}

pa_status pa_bm_set_hash_bits(pa_block_manager* m, int32_t bits) {
  if (!m) return PA_ERR_NULL;
  if (bits < 1 || bits > 64) return PA_ERR_SHAPE;
  std::lock_guard<std::mutex> g(m->mu);
  if (m->num_cached > 0) return PA_ERR_EXISTS;  // keys already hashed at the old width
  m->hash_bits = bits;
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
  for (int32_t b = m->head; b >= 0 && i < capacity; b = m->next[b]) out[i++] = b;
  return m->nfree;
}

}  // extern "C"
