"""Seeded synthetic workloads for paged-attention decode and chunked prefill.

This module only draws random inputs and lays them out; it holds none of the
method's arithmetic (no slot mapping, no attention, no softmax).  Both the
CPU oracle and the HIP path consume what it produces.

Sources (web pages on paged KV caches):
  [P1] "大模型推理内存优化从 KV Cache 分页到连续批处理的工程实践"
       (seekfood.cn/news/1660747)
  [P2] "KV Cache管理优化：大模型推理显存瓶颈突破"
       (intelliparadigm.com/article/weixin_33178839/2255646)

Layout (one layer's pool, [P1] "KV Cache 的内存开销与分页机制": fixed-size
physical blocks, a per-request block table):
  key_cache              : [num_blocks, num_kv_heads, head_dim // kc,
                            block_size, kc]: each key tile's rows cut into
                           column chunks of kc = 64 bytes of elements
                           (16 float32, 32 float16 / bfloat16)
  value_cache            : [num_blocks, num_kv_heads, head_dim, block_size]
                           (each value tile transposed)
  block_tables           : int32 [num_seqs, max_blocks_per_seq]
  seq_lens               : int32 [num_seqs], tokens in the cache after this
                           step's new tokens are written (they are counted)
  q_lens / cu_q_lens     : new tokens per sequence and their prefix sums
  new_key, new_value     : [num_new_tokens, num_kv_heads, head_dim]
  query                  : [num_new_tokens, num_heads, head_dim]

Block tables are filled from a FIFO free list whose order is a random
permutation of the pool, popping from the front in (sequence, logical block)
order, as the block pools on [P1] "生产级推理引擎的内存管理与调度" and [P2]
section 2.1 hand out blocks.

Storage dtypes: 'f32' -> float32, 'f16' -> float16, 'bf16' -> uint16 bit
patterns of bfloat16 (numpy has no bfloat16).  Every value is drawn as float32
N(0, 1) and rounded to the storage dtype to nearest-even.
"""

from __future__ import annotations

import dataclasses
import math
from typing import List, Optional, Sequence

import numpy as np

DTYPES = ("f32", "f16", "bf16")
BYTES = {"f32": 4, "f16": 2, "bf16": 2}


def key_chunk(elem_bytes: int) -> int:
    """Elements per 64-byte column chunk of a key tile."""
    return 64 // int(elem_bytes)


def key_chunks_of(rows: np.ndarray, elem_bytes: int) -> np.ndarray:
    """Key rows [NB, H, B, D] laid out as key tiles [NB, H, D // kc, B, kc]."""
    NB, H, B, D = rows.shape
    kc = key_chunk(elem_bytes)
    return np.ascontiguousarray(rows.reshape(NB, H, B, D // kc, kc).transpose(0, 1, 3, 2, 4))


def f32_to_storage(x: np.ndarray, dtype: str) -> np.ndarray:
    """Round float32 values to the storage dtype, nearest-even."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    if dtype == "f32":
        return x
    if dtype == "f16":
        return x.astype(np.float16)
    if dtype == "bf16":
        bits = x.view(np.uint32).astype(np.uint64)
        lsb = (bits >> 16) & 1
        rounded = ((bits + 0x7FFF + lsb) >> 16).astype(np.uint16)
        nan = np.isnan(x)
        if nan.any():
            rounded[nan] = 0x7FC0
        return rounded
    raise ValueError(f"unknown dtype {dtype!r}")


def nan_value(dtype: str):
    """A quiet NaN in the storage representation."""
    if dtype == "bf16":
        return np.uint16(0x7FC0)
    return np.nan


@dataclasses.dataclass
class Workload:
    """One batch of paged-attention work over a shared pool."""

    name: str
    dtype: str
    num_heads: int
    num_kv_heads: int
    head_dim: int
    block_size: int
    num_blocks: int
    scale: float
    seq_lens: np.ndarray  # int32 [S]
    q_lens: np.ndarray  # int32 [S]
    block_tables: np.ndarray  # int32 [S, MB]
    key_cache: np.ndarray  # storage [NB, Hkv, D // kc, B, kc], new-token slots not yet written
    value_cache: np.ndarray
    new_key: np.ndarray  # storage [T, Hkv, D]
    new_value: np.ndarray
    query: np.ndarray  # storage [T, Hq, D]
    refcounts: np.ndarray  # int32 [NB], how many tables reference each block

    @property
    def num_seqs(self) -> int:
        return int(self.seq_lens.shape[0])

    @property
    def cu_q_lens(self) -> np.ndarray:
        cu = np.zeros(self.num_seqs + 1, dtype=np.int32)
        cu[1:] = np.cumsum(self.q_lens)
        return cu

    @property
    def num_new_tokens(self) -> int:
        return int(self.q_lens.sum())

    @property
    def max_blocks_per_seq(self) -> int:
        return int(self.block_tables.shape[1])

    @property
    def max_seq_len(self) -> int:
        return int(self.seq_lens.max()) if self.num_seqs else 0

    @property
    def elem_bytes(self) -> int:
        return BYTES[self.dtype]

    def subset(self, seqs: Sequence[int]) -> "Workload":
        """The same pool with only some sequences (and their new tokens)."""
        seqs = np.asarray(seqs, dtype=np.int64)
        cu = self.cu_q_lens
        tok = np.concatenate([np.arange(cu[s], cu[s + 1]) for s in seqs]) if len(seqs) else np.zeros(0, np.int64)
        return dataclasses.replace(
            self,
            seq_lens=self.seq_lens[seqs].copy(),
            q_lens=self.q_lens[seqs].copy(),
            block_tables=self.block_tables[seqs].copy(),
            new_key=self.new_key[tok].copy(),
            new_value=self.new_value[tok].copy(),
            query=self.query[tok].copy(),
        )


def _fifo_tables(
    free_list: np.ndarray, blocks_per_seq: Sequence[int], max_blocks: int, pad: int
) -> np.ndarray:
    """Pop blocks from the front of the free list, sequence by sequence."""
    tables = np.full((len(blocks_per_seq), max_blocks), pad, dtype=np.int32)
    cursor = 0
    for s, n in enumerate(blocks_per_seq):
        if cursor + n > free_list.shape[0]:
            raise MemoryError("pool exhausted while building block tables")
        tables[s, :n] = free_list[cursor : cursor + n]
        cursor += n
    return tables


def _ceil_div(a: int, b: int) -> int:
    return -(-int(a) // int(b))


def build(
    *,
    name: str,
    seed: int,
    dtype: str,
    num_heads: int,
    num_kv_heads: int,
    head_dim: int,
    block_size: int,
    seq_lens: Sequence[int],
    q_lens: Optional[Sequence[int]] = None,
    num_blocks: Optional[int] = None,
    pool_factor: float = 1.0,
    shared_prefix: Optional[Sequence[int]] = None,
    prefix_len: int = 0,
    poison_unused: bool = True,
    max_blocks_per_seq: Optional[int] = None,
    rng: Optional[np.random.Generator] = None,
) -> Workload:
    """Draw one workload.

    Draw order: free-list permutation, K pool, V pool, new K, new V, query
    (lengths, when random, are drawn by the caller from the same generator
    beforehand).

    ``shared_prefix[s]`` names a group id: sequences of one group reference the
    same physical blocks for their first ``prefix_len`` tokens (which must be a
    whole number of blocks), as in parallel sampling.
    """
    if dtype not in DTYPES:
        raise ValueError(dtype)
    if num_heads % num_kv_heads:
        raise ValueError("num_heads must be a multiple of num_kv_heads")
    rng = rng if rng is not None else np.random.default_rng(seed)
    seq_lens = np.asarray(seq_lens, dtype=np.int32)
    S = seq_lens.shape[0]
    q_lens = np.ones(S, np.int32) if q_lens is None else np.asarray(q_lens, np.int32)
    if np.any(q_lens > seq_lens):
        raise ValueError("a sequence cannot have more new tokens than tokens")
    B = block_size
    nblk = [_ceil_div(L, B) for L in seq_lens]

    # Which logical blocks are private and which are shared prefix blocks.
    groups = None
    if shared_prefix is not None:
        if prefix_len % B:
            raise ValueError("shared prefix must be whole blocks")
        groups = np.asarray(shared_prefix, np.int64)
    pb = prefix_len // B
    need = 0
    if groups is None:
        need = int(sum(nblk))
    else:
        need = int(len(np.unique(groups)) * pb + sum(n - pb for n in nblk))
    NB = int(num_blocks) if num_blocks is not None else int(math.ceil(need * pool_factor))
    if NB < need:
        raise MemoryError(f"pool of {NB} blocks cannot hold {need}")
    MB = max_blocks_per_seq if max_blocks_per_seq is not None else max(max(nblk, default=1), 1)
    if MB < max(nblk, default=0):
        raise ValueError("max_blocks_per_seq too small")

    free_list = rng.permutation(NB).astype(np.int32)
    pad = int(free_list[need]) if need < NB else 0  # an unused (poisoned) block when one exists

    if groups is None:
        tables = _fifo_tables(free_list, nblk, MB, pad)
    else:
        tables = np.full((S, MB), pad, np.int32)
        cursor = 0
        prefix_of = {}
        for s in range(S):
            gid = int(groups[s])
            if gid not in prefix_of:
                prefix_of[gid] = free_list[cursor : cursor + pb]
                cursor += pb
            tables[s, :pb] = prefix_of[gid]
            n_priv = nblk[s] - pb
            tables[s, pb : pb + n_priv] = free_list[cursor : cursor + n_priv]
            cursor += n_priv
        assert cursor == need

    refcounts = np.zeros(NB, np.int32)
    for s in range(S):
        np.add.at(refcounts, tables[s, : nblk[s]], 1)

    Hkv, D, Hq = num_kv_heads, head_dim, num_heads
    shape = (NB, Hkv, B, D)
    if D % key_chunk(BYTES[dtype]):
        raise ValueError("head_dim must be a multiple of the 64-byte key chunk")
    # Keys are drawn in (block, head, token, dim) order and stored as key
    # tiles of 64-byte column chunks.
    kc = key_chunks_of(f32_to_storage(rng.standard_normal(shape, dtype=np.float32), dtype), BYTES[dtype])
    # Values are drawn in the same (block, head, token, dim) order as keys
    # and stored with each tile transposed: [NB, Hkv, D, B].
    vc = np.ascontiguousarray(f32_to_storage(rng.standard_normal(shape, dtype=np.float32), dtype).transpose(0, 1, 3, 2))
    T = int(q_lens.sum())
    nk = f32_to_storage(rng.standard_normal((T, Hkv, D), dtype=np.float32), dtype)
    nv = f32_to_storage(rng.standard_normal((T, Hkv, D), dtype=np.float32), dtype)
    q = f32_to_storage(rng.standard_normal((T, Hq, D), dtype=np.float32), dtype)

    if poison_unused:
        # Every slot that holds no cached token (unused blocks, the tail of a
        # sequence's last block, and the slots this step's tokens will fill)
        # gets NaN, so that any read of them shows up in the output.
        live = np.zeros((NB, B), bool)
        for s in range(S):
            cached = int(seq_lens[s] - q_lens[s])
            for j in range(_ceil_div(cached, B)):
                n = min(B, cached - j * B)
                live[tables[s, j], :n] = True
        dead = ~live
        nanv = nan_value(dtype)
        kc.transpose(0, 3, 1, 2, 4)[dead] = nanv
        vc.transpose(0, 3, 1, 2)[dead] = nanv

    return Workload(
        name=name,
        dtype=dtype,
        num_heads=Hq,
        num_kv_heads=Hkv,
        head_dim=D,
        block_size=B,
        num_blocks=NB,
        scale=1.0 / math.sqrt(D),
        seq_lens=seq_lens,
        q_lens=q_lens,
        block_tables=tables,
        key_cache=kc,
        value_cache=vc,
        new_key=nk,
        new_value=nv,
        query=q,
        refcounts=refcounts,
    )


# ---------------------------------------------------------------------------
# The five named workloads.  Config k draws from default_rng(326000 + k).
# ---------------------------------------------------------------------------

CONFIG_NAMES = {
    1: "tiny",
    2: "llama2-70b-layer-bs16x4096",
    3: "mixed-64xloguniform-50-8000",
    4: "shared-prefix-8x4",
    5: "chunked-prefill-decode-mix",
}


def config(k: int, *, poison_unused: bool = True, scale_down: int = 1, dtype: Optional[str] = None) -> Workload:
    """Workload for config ``k`` (1..5).

    ``scale_down`` > 1 shrinks sequence lengths (and the pool with them) by
    that factor, keeping heads, head_dim, block size, dtype and the length
    mix; it exists so that full-comparison parity runs stay small.
    ``dtype`` replaces the config's storage dtype (same draws, rounded to the
    other type): FP8 pools are filled from float16 rows.
    """
    return _config(k, poison_unused=poison_unused, scale_down=scale_down, dtype=dtype)


def _config(k: int, *, poison_unused: bool, scale_down: int, dtype: Optional[str]) -> Workload:
    rng = np.random.default_rng(326000 + k)
    sd = int(scale_down)

    def make(**kw):
        if dtype is not None:
            kw["dtype"] = dtype
        return build(**kw)

    if k == 1:
        return make(
            name=CONFIG_NAMES[1], seed=0, rng=rng, dtype="f32", num_heads=8, num_kv_heads=2,
            head_dim=64, block_size=16, seq_lens=[5, 17, 33, 50], num_blocks=64,
            poison_unused=poison_unused,
        )
    if k == 2:
        L = max(4096 // sd, 1)
        return make(
            name=CONFIG_NAMES[2], seed=0, rng=rng, dtype="f16", num_heads=64, num_kv_heads=8,
            head_dim=128, block_size=16, seq_lens=[L] * 16, poison_unused=poison_unused,
        )
    if k == 3:
        lens = np.exp(rng.uniform(math.log(50), math.log(8000), size=64))
        lens = np.maximum(np.rint(lens / sd).astype(np.int64), 1)
        return make(
            name=CONFIG_NAMES[3], seed=0, rng=rng, dtype="bf16", num_heads=32, num_kv_heads=8,
            head_dim=128, block_size=16, seq_lens=lens, pool_factor=1.2,
            poison_unused=poison_unused,
        )
    if k == 4:
        prefix = max(1024 // sd // 16, 1) * 16
        private = max(256 // sd, 1)
        groups = np.repeat(np.arange(8), 4)
        return make(
            name=CONFIG_NAMES[4], seed=0, rng=rng, dtype="f16", num_heads=32, num_kv_heads=8,
            head_dim=128, block_size=16, seq_lens=[prefix + private] * 32,
            shared_prefix=groups, prefix_len=prefix, poison_unused=poison_unused,
        )
    if k == 5:
        chunk = max(512 // sd, 1)
        ctx = max(3584 // sd, 0)
        dec = max(2048 // sd, 1)
        lens = [ctx + chunk] * 4 + [dec] * 48
        qls = [chunk] * 4 + [1] * 48
        return make(
            name=CONFIG_NAMES[5], seed=0, rng=rng, dtype="bf16", num_heads=64, num_kv_heads=8,
            head_dim=128, block_size=32, seq_lens=lens, q_lens=qls, poison_unused=poison_unused,
        )
    raise ValueError(f"no config {k}")


def prefill_decode_split(w: Workload):
    """Indices of the chunked-prefill sequences (q_len > 1) and the decode ones."""
    pre = np.nonzero(w.q_lens > 1)[0]
    dec = np.nonzero(w.q_lens == 1)[0]
    return pre, dec


def blocks_in_use(w: Workload) -> int:
    return int((w.refcounts > 0).sum())


def custom(
    *,
    seed: int,
    dtype: str,
    num_heads: int,
    num_kv_heads: int,
    head_dim: int,
    block_size: int,
    seq_lens: Sequence[int],
    q_lens: Optional[Sequence[int]] = None,
    pool_factor: float = 1.0,
    poison_unused: bool = True,
    max_blocks_per_seq: Optional[int] = None,
    name: str = "custom",
) -> Workload:
    """Any shape, for edge-case and sweep tests."""
    return build(
        name=name, seed=seed, dtype=dtype, num_heads=num_heads, num_kv_heads=num_kv_heads,
        head_dim=head_dim, block_size=block_size, seq_lens=seq_lens, q_lens=q_lens,
        pool_factor=pool_factor, poison_unused=poison_unused,
        max_blocks_per_seq=max_blocks_per_seq,
    )


def layout_tables(w: Workload, kind: str = "identity") -> Workload:
    """The same logical content with the sequences' blocks placed in the
    pool in a fixed pattern instead of the generator's random permutation
    (the blocks no sequence uses follow, in their old order):

    * ``identity``: each sequence's blocks contiguous, sequence 0 first;
    * ``rotated``: contiguous runs as in ``identity``, but sequence s's run
      starts at its block (37 s) mod n_s and wraps around;
    * ``interleaved``: block i of every sequence before block i + 1 of any
      (round-robin over the sequences that still have a block i).

    Used to measure what the block layout costs the decode."""
    S, MB = w.block_tables.shape
    B = w.block_size
    nblk = [_ceil_div(L, B) for L in w.seq_lens]
    used = int(sum(nblk))
    if w.refcounts.max() > 1:
        raise ValueError("a fixed layout needs private blocks")
    if kind == "identity":
        order = [w.block_tables[s, i] for s in range(S) for i in range(nblk[s])]
    elif kind == "rotated":
        order = [w.block_tables[s, (i + 37 * s) % nblk[s]] for s in range(S) for i in range(nblk[s])]
    elif kind == "interleaved":
        order = [w.block_tables[s, i] for i in range(max(nblk, default=0)) for s in range(S) if i < nblk[s]]
    else:
        raise ValueError(f"unknown layout {kind!r}")
    order = np.asarray(order, np.int32)
    rest = np.setdiff1d(np.arange(w.num_blocks, dtype=np.int32), order)
    new_of_old = np.empty(w.num_blocks, np.int32)
    new_of_old[order] = np.arange(used, dtype=np.int32)
    new_of_old[rest] = np.arange(used, w.num_blocks, dtype=np.int32)
    perm = np.empty(w.num_blocks, np.int64)
    perm[new_of_old] = np.arange(w.num_blocks)
    tables = w.block_tables.copy()
    for s in range(S):
        tables[s, : nblk[s]] = new_of_old[w.block_tables[s, : nblk[s]]]
        tables[s, nblk[s]:] = new_of_old[w.block_tables[s, nblk[s]:]]
    return dataclasses.replace(
        w,
        block_tables=tables,
        key_cache=np.ascontiguousarray(w.key_cache[perm]),
        value_cache=np.ascontiguousarray(w.value_cache[perm]),
        refcounts=w.refcounts[perm].copy(),
    )


def identity_tables(w: Workload) -> Workload:
    """Each sequence's blocks contiguous in pool order (sequence 0 first):
    the unpermuted layout against which indirection overhead is measured."""
    return layout_tables(w, "identity")
