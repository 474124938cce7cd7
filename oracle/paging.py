"""Paging arithmetic of the oracle: block counts, KV size, slot mapping, the
KV scatter into pool slots and the gather back out.  Test infrastructure only.

Sources:
  [P1] "大模型推理内存优化从 KV Cache 分页到连续批处理的工程实践"
  [P2] "KV Cache管理优化：大模型推理显存瓶颈突破"
  [P3] "大语言模型KV Cache内存优化与PagedAttention实践"
"""

from __future__ import annotations

import numpy as np


def blocks_needed(num_tokens: int, block_size: int) -> int:
    """Physical blocks a sequence of ``num_tokens`` tokens occupies.

    [P1] "生产级推理引擎的内存管理与调度": the scheduler's block need is the
    token count divided by the block size, rounded up (a partly filled last
    block is still a whole block).
    """
    if num_tokens < 0 or block_size <= 0:
        raise ValueError("negative token count or non-positive block size")
    return (int(num_tokens) + int(block_size) - 1) // int(block_size)


def kv_cache_bytes(
    num_layers: int, seq_len: int, num_kv_heads: int, head_dim: int, dtype_size: int, batch_size: int
) -> int:
    """Bytes of K plus V for a batch.

    [P1] "KV Cache 的内存开销与分页机制": the cache holds one key and one value
    vector per layer, token, and KV head, each ``head_dim`` elements wide, for
    every request of the batch; the factor 2 counts K and V.
    """
    return 2 * num_layers * seq_len * num_kv_heads * head_dim * dtype_size * batch_size


def preallocation_waste(num_tokens: int, slots: int):
    """Fraction of a contiguous per-request cache left unused, or None when
    the request does not fit.

    [P1] "KV Cache 的内存开销与分页机制": a traditional engine reserves the
    maximum length for every request; the unused share of that reservation
    is the reserved slots minus the request's tokens, over the reserved
    slots, and a request longer than the reservation overflows it.
    """
    if num_tokens < 0 or slots <= 0:
        raise ValueError("negative token count or non-positive reservation")
    if num_tokens > slots:
        return None
    return (slots - num_tokens) / slots


def paged_waste(num_tokens: int, block_size: int) -> int:
    """Token slots allocated but unused when a request holds whole blocks.

    [P1] "KV Cache 的内存开销与分页机制": paged allocation hands out
    fixed-size blocks on demand, so only the last block can be partly empty.
    """
    return blocks_needed(num_tokens, block_size) * block_size - num_tokens


def slot_mapping(
    block_tables: np.ndarray, seq_lens: np.ndarray, q_lens: np.ndarray, block_size: int
) -> np.ndarray:
    """Pool slot of every new token, in sequence order.

    [P1] "KV Cache 的内存开销与分页机制": a request's block table maps its
    logical blocks to physical blocks; a token at position ``pos`` lives in
    logical block ``pos // block_size`` at offset ``pos % block_size``, and the
    new token of a step goes into the current (or a newly allocated) block.
    A slot numbers the pool's token positions: physical block times the block
    size plus the offset.  Sequence ``s`` writes ``q_lens[s]`` new tokens at
    positions ``seq_lens[s] - q_lens[s]`` .. ``seq_lens[s] - 1`` (its length
    counts this step's tokens).
    """
    block_tables = np.asarray(block_tables)
    out = []
    for s in range(len(seq_lens)):
        L, q = int(seq_lens[s]), int(q_lens[s])
        for pos in range(L - q, L):
            logical = pos // block_size
            physical = int(block_tables[s, logical])
            out.append(physical * block_size + pos % block_size)
    return np.asarray(out, dtype=np.int64)


# Pool layouts.  Each (block, KV head) tile is one contiguous piece of memory,
# the property that lets in-block KV reads coalesce ([P1] "PagedAttention 的
# CUDA Kernel 实现").  Values: [num_blocks, num_kv_heads, head_dim,
# block_size] (a dimension's block_size values adjacent).  Keys:
# [num_blocks, num_kv_heads, head_dim // kc, block_size, kc]: the tile's
# block_size rows cut into column chunks of kc dims (64 bytes of the storage
# type: 16 float32, 32 float16/bfloat16, 64 FP8 codes), chunk after chunk,
# each chunk row after row.  Key element (block b, head h, offset t, dim d)
# is key_cache[b, h, d // kc, t, d % kc].


def key_rows(key_cache: np.ndarray) -> np.ndarray:
    """Key tiles [NB, H, head_dim // kc, B, kc] -> rows [NB, H, B, head_dim]."""
    NB, H, NC, B, KC = key_cache.shape
    out = np.empty((NB, H, B, NC * KC), dtype=key_cache.dtype)
    for q in range(NC):
        out[:, :, :, q * KC:(q + 1) * KC] = key_cache[:, :, q, :, :]
    return out


def key_tiles(rows: np.ndarray, kc: int) -> np.ndarray:
    """Rows [NB, H, B, head_dim] -> key tiles [NB, H, head_dim // kc, B, kc]."""
    NB, H, B, D = rows.shape
    if D % kc:
        raise ValueError("head_dim must be a multiple of the key chunk")
    out = np.empty((NB, H, D // kc, B, kc), dtype=rows.dtype)
    for q in range(D // kc):
        out[:, :, q, :, :] = rows[:, :, :, q * kc:(q + 1) * kc]
    return out


def reshape_and_cache(
    key_cache: np.ndarray,
    value_cache: np.ndarray,
    key: np.ndarray,
    value: np.ndarray,
    slots: np.ndarray,
) -> None:
    """Write each new token's K and V (all KV heads) into its pool slot, in place.

    Pool layouts as above: the key row lands as one kc-wide piece of every
    chunk of its block's key tile, the value row as column `offset` of the
    value tile.  A negative slot marks a padding token and is skipped; two
    tokens may not share a slot.  Values are copied bit for bit.
    """
    NC, B, KC = key_cache.shape[2:]
    slots = np.asarray(slots, dtype=np.int64)
    valid = slots[slots >= 0]
    if len(np.unique(valid)) != len(valid):
        raise ValueError("two tokens map to the same slot")
    for t, slot in enumerate(slots):
        if slot < 0:
            continue
        block, offset = int(slot) // B, int(slot) % B
        for q in range(NC):
            key_cache[block, :, q, offset, :] = key[t][:, q * KC:(q + 1) * KC]
        value_cache[block, :, :, offset] = value[t]


def gather_kv_present(key_cache: np.ndarray, value_cache: np.ndarray, table_row: np.ndarray, seq_len: int):
    """K, V [n, num_kv_heads, head_dim] and positions [n] of the tokens of one
    sequence whose table entry names a block inside the pool.

    The library's contract for a table entry outside [0, num_blocks) (a
    missing block): its positions hold no key, so they are left out of the
    attention entirely, as if the sequence had no token there; the other
    tokens keep their positions (and so their causal visibility).  Built
    token by token from the definition of the table walk.
    """
    nb, Hkv, NC, B, KC = key_cache.shape
    ks, vs, pos = [], [], []
    for t in range(seq_len):
        phys = int(table_row[t // B])
        if 0 <= phys < nb:
            ks.append(np.concatenate([key_cache[phys, :, q, t % B, :] for q in range(NC)], axis=1))
            vs.append(value_cache[phys, :, :, t % B])
            pos.append(t)
    D = NC * KC
    if not pos:
        return np.zeros((0, Hkv, D)), np.zeros((0, Hkv, D)), np.zeros(0, dtype=np.int64)
    return np.stack(ks), np.stack(vs), np.asarray(pos, dtype=np.int64)


def gather_kv(key_cache: np.ndarray, value_cache: np.ndarray, table_row: np.ndarray, seq_len: int):
    """Contiguous K and V [seq_len, num_kv_heads, head_dim] of one sequence.

    [P1] "PagedAttention 的 CUDA Kernel 实现": for each logical block, look up
    its physical block ID in the block table, then read that block's vectors.
    Only the first ``blocks_needed(seq_len)`` table entries are read, and of
    the last block only the filled offsets.
    """
    B = key_cache.shape[3]
    n = blocks_needed(seq_len, B)
    phys = np.asarray(table_row[:n], dtype=np.int64)
    if ((phys < 0) | (phys >= key_cache.shape[0])).any():
        raise ValueError("a table entry names a block outside the pool")
    # Logical order is block-major, offset-minor:
    # keys -> rows [n, Hkv, B, D] -> [n, B, Hkv, D]; values [n, Hkv, D, B] -> [n, B, Hkv, D].
    rows = key_rows(key_cache[phys])
    K = rows.transpose(0, 2, 1, 3).reshape(n * B, rows.shape[1], rows.shape[3])
    V = value_cache[phys].transpose(0, 3, 1, 2).reshape(n * B, value_cache.shape[1], value_cache.shape[2])
    return K[:seq_len], V[:seq_len]
