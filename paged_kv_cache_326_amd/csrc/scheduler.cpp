// Host-side continuous-batching step arithmetic of libpa.so, on top of the
// block manager: which requests take part in an iteration, the blocks each
// one needs, admission from a FIFO waiting queue, preemption when the pool
// runs dry, and the release of finished requests.
//
// Source: [P1] "大模型推理内存优化从 KV Cache 分页到连续批处理的工程实践",
// section "生产级推理引擎的内存管理与调度" (the scheduler's three steps per
// iteration):
//   1. Every decoding request whose tokens (prompt + generated) need more
//      blocks than it owns (ceil(tokens / block_size) > owned) gets one more
//      block if the pool has any, and is scheduled; if the pool is empty it
//      is preempted for this iteration (not scheduled, keeps its blocks).
//      A request that needs no new block is scheduled.
//   2. While fewer than max_batch_size requests are scheduled, the front of
//      the waiting queue is admitted if the pool holds the
//      ceil(prompt / block_size) blocks of its prompt; otherwise it stays at
//      the front and admission stops for this iteration.
//   3. Requests that have generated max_tokens tokens release their blocks.
//   A step of a request adds one generated token; reaching max_tokens
//   finishes it.
// Readings where the page is silent or leaves the order open: active
// requests are visited in admission order (steps 1 and 3); max_tokens must
// be at least 1 (a request admitted with nothing to generate would be
// scheduled and released in the same iteration).
#include <cstdint>
#include <deque>
#include <mutex>
#include <unordered_map>
#include <vector>

#include "../../include/pa.h"

namespace {

enum State : int32_t { kWaiting = 0, kDecoding = 1, kFinished = 2 };

struct Request {
  int32_t prompt_len = 0;
  int32_t max_tokens = 0;
  int32_t generated = 0;
  State state = kWaiting;
};

int64_t blocks_for(int64_t tokens, int32_t block_size) { return (tokens + block_size - 1) / block_size; }

}  // namespace

struct pa_scheduler {
  pa_block_manager* bm = nullptr;
  int32_t block_size = 0;
  int32_t max_batch = 0;
  std::mutex mu;
  std::unordered_map<int64_t, Request> reqs;  // waiting and active requests
  std::deque<int64_t> waiting;                // FIFO
  std::vector<int64_t> active;                // admission order
  // Copy-on-write pairs of the last pa_sched_schedule call: a scheduled
  // request whose partly filled last block is shared (pa_bm_fork) received
  // a private block; the caller copies old -> new before the step's scatter.
  std::vector<int32_t> copy_src, copy_dst;
};

extern "C" {

pa_scheduler* pa_sched_create(pa_block_manager* bm, int32_t max_batch_size) {
  if (!bm || max_batch_size <= 0) return nullptr;
  auto* s = new pa_scheduler;
  s->bm = bm;
  s->block_size = pa_bm_block_size(bm);
  s->max_batch = max_batch_size;
  return s;
}

void pa_sched_destroy(pa_scheduler* s) { delete s; }

pa_status pa_sched_add_request(pa_scheduler* s, int64_t id, int32_t prompt_len, int32_t max_tokens) {
  if (!s) return PA_ERR_NULL;
  if (prompt_len < 0 || max_tokens < 1) return PA_ERR_SHAPE;
  std::lock_guard<std::mutex> g(s->mu);
  if (s->reqs.count(id) || pa_bm_num_tokens(s->bm, id) >= 0) return PA_ERR_EXISTS;
  Request r;
  r.prompt_len = prompt_len;
  r.max_tokens = max_tokens;
  s->reqs.emplace(id, r);
  s->waiting.push_back(id);
  return PA_OK;
}

pa_status pa_sched_schedule(pa_scheduler* s, int64_t* scheduled, int32_t capacity, int32_t* num_scheduled) {
  if (!s || !num_scheduled || (capacity > 0 && !scheduled)) return PA_ERR_NULL;
  std::lock_guard<std::mutex> g(s->mu);
  std::vector<int64_t> out;
  s->copy_src.clear();
  s->copy_dst.clear();

  // 1. Decoding requests: one more block when their tokens outgrow the
  // blocks they own, or preemption for this iteration.
  for (int64_t id : s->active) {
    Request& r = s->reqs[id];
    if (r.state != kDecoding) continue;
    const int64_t tokens = (int64_t)r.prompt_len + r.generated;
    const int64_t owned = pa_bm_block_table(s->bm, id, nullptr, 0);
    const int64_t have = pa_bm_num_tokens(s->bm, id);
    if (owned < 0 || have < 0) return PA_ERR_NOT_FOUND;  // released behind the scheduler's back
    if (blocks_for(tokens, s->block_size) > owned && pa_bm_available(s->bm) <= 0) continue;  // preempted
    if (tokens > have) {
      int32_t src, dst, ncopy;
      const pa_status st = pa_bm_append_tokens(s->bm, id, (int32_t)(tokens - have), &src, &dst, &ncopy);
      if (st == PA_ERR_NO_BLOCKS) continue;  // preempted
      if (st != PA_OK) return st;
      if (ncopy > 0) {
        s->copy_src.push_back(src);
        s->copy_dst.push_back(dst);
      }
    }
    out.push_back(id);
  }

  // 2. Admission from the front of the waiting queue.
  while ((int32_t)out.size() < s->max_batch && !s->waiting.empty()) {
    const int64_t id = s->waiting.front();
    Request& r = s->reqs[id];
    if (blocks_for(r.prompt_len, s->block_size) > pa_bm_available(s->bm)) break;  // waits at the front
    const pa_status st = pa_bm_add_sequence(s->bm, id, r.prompt_len);
    if (st == PA_ERR_NO_BLOCKS) break;
    if (st != PA_OK) return st;
    s->waiting.pop_front();
    r.state = kDecoding;
    s->active.push_back(id);
    out.push_back(id);
  }

  // 3. Finished requests release their blocks.
  std::vector<int64_t> keep;
  keep.reserve(s->active.size());
  for (int64_t id : s->active) {
    const Request& r = s->reqs[id];
    if (r.generated >= r.max_tokens) {
      pa_bm_free_sequence(s->bm, id);
      s->reqs.erase(id);
    } else {
      keep.push_back(id);
    }
  }
  s->active.swap(keep);

  *num_scheduled = (int32_t)out.size();
  for (int32_t i = 0; i < capacity && i < (int32_t)out.size(); ++i) scheduled[i] = out[i];
  return PA_OK;
}

int32_t pa_sched_copies(pa_scheduler* s, int32_t* copy_src, int32_t* copy_dst, int32_t capacity) {
  if (!s || (capacity > 0 && (!copy_src || !copy_dst))) return -1;
  std::lock_guard<std::mutex> g(s->mu);
  const int32_t n = (int32_t)s->copy_src.size();
  for (int32_t i = 0; i < capacity && i < n; ++i) {
    copy_src[i] = s->copy_src[i];
    copy_dst[i] = s->copy_dst[i];
  }
  return n;
}

pa_status pa_sched_step(pa_scheduler* s, int64_t id) {
  if (!s) return PA_ERR_NULL;
  std::lock_guard<std::mutex> g(s->mu);
  auto it = s->reqs.find(id);
  if (it == s->reqs.end() || it->second.state != kDecoding) return PA_ERR_NOT_FOUND;
  Request& r = it->second;
  r.generated += 1;
  if (r.generated >= r.max_tokens) r.state = kFinished;
  return PA_OK;
}

int32_t pa_sched_state(pa_scheduler* s, int64_t id) {
  if (!s) return -1;
  std::lock_guard<std::mutex> g(s->mu);
  auto it = s->reqs.find(id);
  return it == s->reqs.end() ? -1 : (int32_t)it->second.state;
}

int32_t pa_sched_generated(pa_scheduler* s, int64_t id) {
  if (!s) return -1;
  std::lock_guard<std::mutex> g(s->mu);
  auto it = s->reqs.find(id);
  return it == s->reqs.end() ? -1 : it->second.generated;
}

int32_t pa_sched_num_waiting(pa_scheduler* s) {
  if (!s) return -1;
  std::lock_guard<std::mutex> g(s->mu);
  return (int32_t)s->waiting.size();
}

int32_t pa_sched_num_active(pa_scheduler* s) {
  if (!s) return -1;
  std::lock_guard<std::mutex> g(s->mu);
  return (int32_t)s->active.size();
}

}  // extern "C"
