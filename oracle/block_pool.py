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
  [P1] section "工程边界与架构取舍": requests that share a system prompt can
       reuse the prefix's physical blocks; cached prefixes carry a version
       (an updated prompt must not hit the old cache), and a hash collision
       must never produce a wrong hit.
Where the pages are silent the model takes these readings: a failed request
changes nothing; a sequence about to write into a partly filled block that
other sequences share first receives a private copy (copy-on-write).

Prefix cache (readings): a full block becomes cached when the caller
reports its K/V written (commit); its key is the version plus the exact
token prefix the block ends.  A new sequence reuses the cached blocks of its
longest cached run of leading full blocks.  A cached block stays cached
after its last reference goes (it sits in the free list) until a fresh
allocation pops it, which uncaches it together with every cached key that
extends it.  The model keys its dict by the full token tuple, so no hash is
involved at all: the library's hashed lookup must behave exactly like it.
"""

from collections import deque

import numpy as np

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
        self.ids = {}        # sequence -> token ids (None when not all known)
        self.version = {}    # sequence -> version
        self.cached = {}     # (version, token prefix tuple) -> block
        self.key_of = {}     # block -> its key

    def _uncache(self, b):
        version, prefix = self.key_of.pop(b)
        del self.cached[(version, prefix)]
        n = len(prefix)
        for (v2, p2), b2 in list(self.cached.items()):
            if v2 == version and len(p2) > n and p2[:n] == prefix and b2 in self.key_of:
                self._uncache(b2)

    def _take(self):
        b = self.free.popleft()
        if b in self.key_of:
            self._uncache(b)
        self.refs[b] = 1
        return b

    def _ref(self, b):
        if self.refs[b] == 0:
            self.free.remove(b)
        self.refs[b] += 1

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
        self.ids[sid] = None
        self.version[sid] = 0

    def add_sequence_tokens(self, sid, ids, version=0):
        """Returns how many leading tokens were found cached.

        Lookups stop one token short of the end: the prompt's last token is
        always computed (its logits start generation), so the block holding
        it must be private, never a shared cached block.  A prompt that is a
        whole number of cached blocks therefore reuses all but its last
        block."""
        assert sid not in self.tables
        ids, B = [int(x) for x in ids], self.block_size
        hits = []
        for i in range(max(len(ids) - 1, 0) // B):
            b = self.cached.get((version, tuple(ids[: (i + 1) * B])))
            if b is None:
                break
            hits.append(b)
        need = blocks_needed(len(ids), B) - len(hits)
        if need > len(self.free) - sum(1 for b in hits if self.refs[b] == 0):
            raise NoBlocks
        for b in hits:
            self._ref(b)
        self.tables[sid] = hits + [self._take() for _ in range(need)]
        self.lengths[sid] = len(ids)
        self.ids[sid] = ids
        self.version[sid] = version
        return len(hits) * B

    def commit(self, sid, n):
        """The first n tokens' K/V are written: cache the full blocks among them."""
        t, ids, B, v = self.tables[sid], self.ids[sid], self.block_size, self.version[sid]
        for i in range(n // B):
            if t[i] in self.key_of:
                continue
            if i > 0 and t[i - 1] not in self.key_of:
                break
            key = (v, tuple(ids[: (i + 1) * B]))
            if key in self.cached:
                break
            self.cached[key] = t[i]
            self.key_of[t[i]] = key

    def drop_version(self, version):
        gone = [b for b, (v, _) in self.key_of.items() if v == version]
        for b in gone:
            if b in self.key_of:
                self._uncache(b)
        return len(gone)

    def fork(self, parent, child):
        assert child not in self.tables
        self.tables[child] = list(self.tables[parent])
        self.lengths[child] = self.lengths[parent]
        self.ids[child] = None if self.ids[parent] is None else list(self.ids[parent])
        self.version[child] = self.version[parent]
        for b in self.tables[child]:
            self.refs[b] += 1

    def append_tokens(self, sid, n, ids=None):
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
        if ids is None or self.ids[sid] is None:
            self.ids[sid] = None
        else:
            self.ids[sid].extend(int(x) for x in ids)
        return pairs

    def free_sequence(self, sid):
        for b in self.tables.pop(sid):
            self._release(b)
        del self.lengths[sid], self.ids[sid], self.version[sid]


def _in_pool(b, num_blocks):
    return 0 <= int(b) < num_blocks


def copy_blocks(pool, src, dst):
    """Pool block src[i] -> pool block dst[i] for each pair, in place.

    [P1] "KV Cache 的内存开销与分页机制" and [P2] section 4.1: sequences share
    physical blocks; a sequence about to write into a shared block first
    gets a private copy of it.  ``pool`` is one pool array whose first axis
    numbers the blocks (the key pool or the value pool: the per-block layout
    does not matter to a copy).

    Contract (the library's): a pair with an id outside the pool, or with
    src == dst, is skipped; among the remaining pairs no destination may
    repeat and no destination may also be a source, so the result does not
    depend on the order of the copies.  A violation raises ValueError and
    leaves the pool unchanged.
    """
    src, dst = [int(x) for x in src], [int(x) for x in dst]
    if len(src) != len(dst):
        raise ValueError("src and dst differ in length")
    nb = pool.shape[0]
    pairs = [(a, b) for a, b in zip(src, dst) if _in_pool(a, nb) and _in_pool(b, nb) and a != b]
    dsts = [b for _, b in pairs]
    if len(set(dsts)) != len(dsts):
        raise ValueError("a destination block repeats")
    if set(dsts) & {a for a, _ in pairs}:
        raise ValueError("a destination block is also a source")
    for a, b in pairs:
        pool[b] = pool[a].copy()


def gather_blocks(pool, ids, out=None):
    """Pool block ids[i] -> row i of a staging array (swap out).

    [P2] section 3: blocks are moved out of device memory and back.  Rows
    of ids outside the pool are left as they are (zeros when ``out`` is not
    given).
    """
    ids = [int(x) for x in ids]
    nb = pool.shape[0]
    if out is None:
        out = np.zeros((len(ids),) + pool.shape[1:], dtype=pool.dtype)
    for i, b in enumerate(ids):
        if _in_pool(b, nb):
            out[i] = pool[b]
    return out


def scatter_blocks(pool, ids, rows):
    """Row i of a staging array -> pool block ids[i], in place (swap in).
    Ids outside the pool are skipped; a repeated id raises ValueError (the
    result would depend on the order of the writes)."""
    ids = [int(x) for x in ids]
    nb = pool.shape[0]
    live = [b for b in ids if _in_pool(b, nb)]
    if len(set(live)) != len(live):
        raise ValueError("a destination block repeats")
    for i, b in enumerate(ids):
        if _in_pool(b, nb):
            pool[b] = rows[i]
