"""Reference model of the continuous-batching step arithmetic, for checking
the library's host scheduler.  Test infrastructure only.

Source: [P1] "大模型推理内存优化从 KV Cache 分页到连续批处理的工程实践",
section "生产级推理引擎的内存管理与调度".  One scheduling call per
iteration, in three steps:
  1. a decoding request whose prompt + generated tokens need more blocks
     than it holds gets one block if the pool has one (scheduled), else it is
     preempted for the iteration (not scheduled, keeps its blocks); one that
     needs none is scheduled;
  2. while fewer than max_batch_size requests are scheduled, the front of the
     FIFO waiting queue is admitted if the pool can give all the blocks of its
     prompt, else it stays at the front and admission stops;
  3. requests that have generated max_tokens tokens give their blocks back.
A step adds one generated token; reaching max_tokens finishes the request.
Readings: active requests are visited in admission order (the page iterates a
hash map); max_tokens >= 1.  Blocks come from BlockPoolModel (FIFO pool).
"""

from collections import deque

from .block_pool import BlockPoolModel, NoBlocks
from .paging import blocks_needed

WAITING, DECODING, FINISHED = 0, 1, 2


class SchedulerModel:
    def __init__(self, pool: BlockPoolModel, max_batch_size: int):
        assert max_batch_size >= 1
        self.pool = pool
        self.max_batch = max_batch_size
        self.waiting = deque()
        self.active = []  # admission order
        self.req = {}     # id -> dict(prompt, max_tokens, generated, state)
        self.copies = []  # copy-on-write (old, new) pairs of the last schedule()

    def add_request(self, rid, prompt_len, max_tokens):
        if prompt_len < 0 or max_tokens < 1:
            raise ValueError("bad request")
        if rid in self.req or rid in self.pool.tables:
            raise KeyError(rid)
        self.req[rid] = {"prompt": prompt_len, "max_tokens": max_tokens, "generated": 0, "state": WAITING}
        self.waiting.append(rid)

    def schedule(self):
        B = self.pool.block_size
        scheduled = []
        self.copies = []
        # Step 1: decoding requests.
        for rid in self.active:
            r = self.req[rid]
            if r["state"] != DECODING:
                continue
            tokens = r["prompt"] + r["generated"]
            owned = len(self.pool.tables[rid])
            if blocks_needed(tokens, B) > owned:
                if len(self.pool.free) == 0:
                    continue  # preempted this iteration
            grow = tokens - self.pool.lengths[rid]
            if grow > 0:
                try:
                    # A shared, partly filled last block (a forked request)
                    # is replaced by a private one: the pair is reported.
                    self.copies += self.pool.append_tokens(rid, grow)
                except NoBlocks:
                    continue
            scheduled.append(rid)
        # Step 2: admissions from the front of the queue.
        while len(scheduled) < self.max_batch and self.waiting:
            rid = self.waiting[0]
            r = self.req[rid]
            if len(self.pool.free) < blocks_needed(r["prompt"], B):
                break
            self.pool.add_sequence(rid, r["prompt"])
            self.waiting.popleft()
            r["state"] = DECODING
            self.active.append(rid)
            scheduled.append(rid)
        # Step 3: finished requests release their blocks.
        keep = []
        for rid in self.active:
            r = self.req[rid]
            if r["generated"] >= r["max_tokens"]:
                self.pool.free_sequence(rid)
                del self.req[rid]
            else:
                keep.append(rid)
        self.active = keep
        return scheduled

    def step(self, rid):
        r = self.req.get(rid)
        if r is None or r["state"] != DECODING:
            raise KeyError(rid)
        r["generated"] += 1
        if r["generated"] >= r["max_tokens"]:
            r["state"] = FINISHED

    def state(self, rid):
        r = self.req.get(rid)
        return -1 if r is None else r["state"]
