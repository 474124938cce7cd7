"""Reference model of the physical-block pool and per-sequence tables, for
checking the library's host block manager.  Test infrastructure only.

Sources:
  [P1] "大模型推理内存优化从 KV Cache 分页到连续批处理的工程实践", section
       "生产级推理引擎的内存管理与调度": the pool hands out block IDs from the
       front of a FIFO free list and takes them back at the end; n tokens
       need ceil(n / block_size) blocks; a request that cannot be given its
       blocks waits or is preempted.
  [P2] "KV Cache管理优化：大模型推理显存瓶颈突破", section 2.1 (the same
       FIFO allocator) and section 4.1 (a shared block counts its users and
       goes back to the pool when the count reaches zero).
Where the pages are silent the model takes these readings: a failed request
changes nothing; a sequence about to write into a partly filled block that
other sequences share first receives a private copy (copy-on-write).
"""

from collections import deque

from .paging import blocks_needed


class NoBlocks(Exception):
    pass


class BlockPoolModel:
    def __init__(self, num_blocks, block_size, free_order=None):
        order = list(range(num_blocks)) if free_order is None else [int(b) for b in free_order]
        assert sorted(order) == list(range(num_blocks))
        self.block_size = block_size
        self.free = deque(order)
        self.refs = [0] * num_blocks
        self.tables = {}
        self.lengths = {}

    def _take(self):
        b = self.free.popleft()
        self.refs[b] = 1
        return b

    def _release(self, b):
        self.refs[b] -= 1
        if self.refs[b] == 0:
            self.free.append(b)

    def add_sequence(self, sid, n):
        assert sid not in self.tables
        need = blocks_needed(n, self.block_size)
        if need > len(self.free):
            raise NoBlocks
        self.tables[sid] = [self._take() for _ in range(need)]
        self.lengths[sid] = n

    def fork(self, parent, child):
        assert child not in self.tables
        self.tables[child] = list(self.tables[parent])
        self.lengths[child] = self.lengths[parent]
        for b in self.tables[child]:
            self.refs[b] += 1

    def append_tokens(self, sid, n):
        """Returns the copy-on-write (old, new) pairs."""
        if n == 0:
            return []
        t, L, B = self.tables[sid], self.lengths[sid], self.block_size
        shared_tail = L % B != 0 and self.refs[t[-1]] > 1
        grow = blocks_needed(L + n, B) - len(t)
        if grow + shared_tail > len(self.free):
            raise NoBlocks
        pairs = []
        if shared_tail:
            old = t[-1]
            new = self._take()
            self._release(old)
            t[-1] = new
            pairs.append((old, new))
        t.extend(self._take() for _ in range(grow))
        self.lengths[sid] = L + n
        return pairs

    def free_sequence(self, sid):
        for b in self.tables.pop(sid):
            self._release(b)
        del self.lengths[sid]


def copy_blocks(pool, src, dst):
    """Pool block src[i] -> pool block dst[i] for each pair, in place."""
    pool[list(dst)] = pool[list(src)]


def gather_blocks(pool, ids):
    return pool[list(ids)].copy()


def scatter_blocks(pool, ids, rows):
    pool[list(ids)] = rows
