"""Paged attention of the oracle: gather, then dense softmax attention in
float64.  Test infrastructure only.

Sources:
  [P1] "大模型推理内存优化从 KV Cache 分页到连续批处理的工程实践"

Readings where the pages are silent (each is listed in the design notes):
  * GQA: query head h reads KV head h // (num_heads // num_kv_heads).
  * Softmax is stabilised by subtracting the row maximum; this is exact in
    real arithmetic.
  * A sequence of length 0 attends to nothing and yields zeros.
  * Chunked prefill is causal and inclusive: query i of a chunk of q tokens
    appended to ctx cached tokens sees keys 0 .. ctx + i.
"""

from __future__ import annotations

import numpy as np

from .paging import gather_kv, gather_kv_present


def _attend(qh: np.ndarray, K: np.ndarray, V: np.ndarray, scale: float) -> np.ndarray:
    """softmax(scale * K qh) V for one query vector over L keys (float64)."""
    z = scale * (K @ qh)
    p = np.exp(z - z.max())
    return (p @ V) / p.sum()


def decode_attention(
    query: np.ndarray,
    key_cache: np.ndarray,
    value_cache: np.ndarray,
    block_tables: np.ndarray,
    seq_lens: np.ndarray,
    scale: float,
    drop_missing_blocks: bool = False,
) -> np.ndarray:
    """One new token per sequence attends over all of that sequence's cached
    tokens (its own included), read through the block table.

    [P1] "KV Cache 的内存开销与分页机制": generating a token needs the keys and
    values of every earlier token, held in the cache; [P1] "工程边界与架构取舍":
    a decode step reads the whole cache for one token.  Paging changes only
    where the vectors are read from ([P1] "PagedAttention 的 CUDA Kernel 实现").

    query [S, Hq, D], caches [NB, Hkv, B, D], all float64.  Returns [S, Hq, D].
    With ``drop_missing_blocks`` a table entry outside the pool contributes
    no keys (the library's contract for such entries); a sequence left with
    no key yields zeros.  Without it such an entry raises.
    """
    S, Hq, D = query.shape
    Hkv = key_cache.shape[1]
    G = Hq // Hkv
    out = np.zeros((S, Hq, D), dtype=np.float64)
    for s in range(S):
        L = int(seq_lens[s])
        if L == 0:
            continue
        if drop_missing_blocks:
            K, V, _ = gather_kv_present(key_cache, value_cache, block_tables[s], L)
            if len(K) == 0:
                continue
        else:
            K, V = gather_kv(key_cache, value_cache, block_tables[s], L)
        for h in range(Hq):
            g = h // G
            out[s, h] = _attend(query[s, h], K[:, g, :], V[:, g, :], scale)
    return out


def prefill_attention(
    query: np.ndarray,
    cu_q_lens: np.ndarray,
    key_cache: np.ndarray,
    value_cache: np.ndarray,
    block_tables: np.ndarray,
    seq_lens: np.ndarray,
    scale: float,
    drop_missing_blocks: bool = False,
) -> np.ndarray:
    """A chunk of new tokens per sequence attends causally over the cache.

    [P1] "工程边界与架构取舍": a long prompt is processed in chunks.  The chunk's
    own K/V are already in the cache (written by the scatter first), so
    sequence s holds seq_lens[s] tokens of which the last q_s are the chunk;
    chunk token i sits at position ctx + i with ctx = seq_lens[s] - q_s and
    attends to positions 0 .. ctx + i.

    query [T, Hq, D] float64 with T = cu_q_lens[-1].  Returns [T, Hq, D].
    ``drop_missing_blocks`` as in decode_attention: the positions of a
    missing block hold no key; the rest keep their causal visibility, and a
    row that sees no key yields zeros.
    """
    T, Hq, D = query.shape
    Hkv = key_cache.shape[1]
    G = Hq // Hkv
    out = np.zeros((T, Hq, D), dtype=np.float64)
    for s in range(len(seq_lens)):
        L = int(seq_lens[s])
        t0, t1 = int(cu_q_lens[s]), int(cu_q_lens[s + 1])
        q = t1 - t0
        if q == 0:
            continue
        ctx = L - q
        if drop_missing_blocks:
            K, V, pos = gather_kv_present(key_cache, value_cache, block_tables[s], L)
        else:
            K, V = gather_kv(key_cache, value_cache, block_tables[s], L)
            pos = np.arange(L)
        for h in range(Hq):
            g = h // G
            Kh, Vh = K[:, g, :], V[:, g, :]
            Z = scale * (query[t0:t1, h, :] @ Kh.T)  # [q, number of keys]
            visible = pos[None, :] <= (ctx + np.arange(q))[:, None]
            rows = visible.any(axis=1)  # a row that sees no key stays zero
            if not rows.any():
                continue
            Z = np.where(visible[rows], Z[rows], -np.inf)
            P = np.exp(Z - Z.max(axis=1, keepdims=True))
            out[t0:t1, h, :][rows] = (P @ Vh) / P.sum(axis=1, keepdims=True)
    return out
