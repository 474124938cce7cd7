"""ctypes binding of libpa.so.  Argument marshalling only: every step of the
paged path runs in the library's HIP kernels.  torch supplies device memory
and the current HIP stream.

The functions carry the C names.  Tensors must live on the GPU, be contiguous
and have the dtypes the C header states; the caller owns every buffer.
Errors raise :class:`PaError` carrying the library's status.
"""

from __future__ import annotations

import ctypes
import os
from typing import Optional

import torch

# PA_LIB may name another build of the library: the sanitizer run of the
# host C++ loads one that holds only the block manager and the scheduler.
_LIB_PATH = os.environ.get("PA_LIB") or os.path.join(os.path.dirname(os.path.abspath(__file__)), "libpa.so")

PA_F32, PA_F16, PA_BF16, PA_FP8_E4M3 = 0, 1, 2, 3
# An FP8 (OCP E4M3) pool is a uint8 (or float8_e4m3fn) tensor of codes; its
# queries, outputs and new K/V rows are float16.
_DTYPE = {torch.float32: PA_F32, torch.float16: PA_F16, torch.bfloat16: PA_BF16, torch.uint8: PA_FP8_E4M3}
if hasattr(torch, "float8_e4m3fn"):
    _DTYPE[torch.float8_e4m3fn] = PA_FP8_E4M3
_STATUS = {0: "PA_OK", 1: "PA_ERR_NULL", 2: "PA_ERR_SHAPE", 3: "PA_ERR_UNSUPPORTED", 4: "PA_ERR_WORKSPACE", 5: "PA_ERR_LAUNCH",
           6: "PA_ERR_NO_BLOCKS", 7: "PA_ERR_NOT_FOUND", 8: "PA_ERR_EXISTS"}
PA_ERR_SHAPE = 2
PA_ERR_WORKSPACE = 4
PA_ERR_NO_BLOCKS = 6
PA_ERR_NOT_FOUND = 7
PA_ERR_EXISTS = 8


class PaError(RuntimeError):
    def __init__(self, status: int, what: str):
        self.status = status
        try:
            detail = lib().pa_status_string(status).decode()
        except RuntimeError:  # a partial build (PA_LIB) without pa_status_string
            detail = "no description in this build"
        super().__init__(f"{what}: {_STATUS.get(status, status)} ({detail})")


class pa_kv_cache(ctypes.Structure):
    _fields_ = [
        ("key_cache", ctypes.c_void_p),
        ("value_cache", ctypes.c_void_p),
        ("num_blocks", ctypes.c_int32),
        ("num_kv_heads", ctypes.c_int32),
        ("head_dim", ctypes.c_int32),
        ("block_size", ctypes.c_int32),
        ("dtype", ctypes.c_int32),
        ("k_scale", ctypes.c_float),
        ("v_scale", ctypes.c_float),
    ]


class pa_decode_args(ctypes.Structure):
    _fields_ = [
        ("cache", ctypes.POINTER(pa_kv_cache)),
        ("out", ctypes.c_void_p),
        ("query", ctypes.c_void_p),
        ("block_tables", ctypes.c_void_p),
        ("max_blocks_per_seq", ctypes.c_int32),
        ("seq_lens", ctypes.c_void_p),
        ("num_seqs", ctypes.c_int32),
        ("num_heads", ctypes.c_int32),
        ("max_seq_len", ctypes.c_int32),
        ("scale", ctypes.c_float),
        ("workspace", ctypes.c_void_p),
        ("workspace_bytes", ctypes.c_size_t),
        ("partition_size", ctypes.c_int32),
        ("stage", ctypes.c_int32),
        ("new_key", ctypes.c_void_p),
        ("new_value", ctypes.c_void_p),
        ("slot_mapping", ctypes.c_void_p),
        ("work", ctypes.c_void_p),
        ("num_work", ctypes.c_int32),
        ("kernel_start", ctypes.c_void_p),
        ("kernel_stop", ctypes.c_void_p),
    ]


_lib = None


class _Absent:
    """Stands for an entry point that a partial build (PA_LIB) lacks: its
    signature may be declared, a call raises."""

    def __init__(self, name: str):
        self.__dict__["_name"] = name

    def __call__(self, *args):
        raise RuntimeError(f"{self._name} is not in {_LIB_PATH}")


class _Partial:
    """A library loaded through PA_LIB that may lack some entry points."""

    def __init__(self, L: ctypes.CDLL):
        self._L = L

    def __getattr__(self, name: str):
        try:
            f = getattr(self._L, name)
        except AttributeError:
            f = _Absent(name)
        setattr(self, name, f)
        return f

EXPORTS = (
    "pa_slot_mapping",
    "pa_reshape_and_cache",
    "pa_append_kv",
    "pa_decode_auto_partition",
    "pa_decode_workspace_bytes",
    "pa_decode",
    "pa_decode_ex",
    "pa_decode_stage",
    "pa_decode_timed",
    "pa_decode_append",
    "pa_decode_run",
    "pa_decode_plan",
    "pa_decode_noalloc",
    "pa_prefill_chunk",
    "pa_stream_read",
    "pa_copy_blocks",
    "pa_gather_blocks",
    "pa_scatter_blocks",
    "pa_bm_create",
    "pa_bm_destroy",
    "pa_bm_available",
    "pa_bm_refcount",
    "pa_bm_add_sequence",
    "pa_bm_fork",
    "pa_bm_append_tokens",
    "pa_bm_free_sequence",
    "pa_bm_block_table",
    "pa_bm_num_tokens",
    "pa_bm_free_list",
    "pa_bm_add_sequence_tokens",
    "pa_bm_append_token_ids",
    "pa_bm_commit",
    "pa_bm_drop_version",
    "pa_bm_cached_blocks",
    "pa_bm_is_cached",
    "pa_bm_set_hash_bits",
    "pa_bm_block_size",
    "pa_sched_create",
    "pa_sched_destroy",
    "pa_sched_add_request",
    "pa_sched_schedule",
    "pa_sched_copies",
    "pa_sched_step",
    "pa_sched_state",
    "pa_sched_generated",
    "pa_sched_num_waiting",
    "pa_sched_num_active",
    "pa_status_string",
    "pa_version",
)


def lib() -> ctypes.CDLL:
    """Load libpa.so (built in-tree); raise if it is missing."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB_PATH):
        raise ImportError(
            f"{_LIB_PATH} is not built; run `python -m paged_kv_cache_326_amd.build` (hipcc, gfx950)"
        )
    L = ctypes.CDLL(_LIB_PATH)
    if os.environ.get("PA_LIB"):
        L = _Partial(L)
    vp, i32, i64p, i32p, f32, sz = ctypes.c_void_p, ctypes.c_int32, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_float, ctypes.c_size_t
    cache_p = ctypes.POINTER(pa_kv_cache)
    L.pa_slot_mapping.argtypes = [i32p, i32, i32p, i32p, i32, i32, i64p, i32, vp]
    L.pa_slot_mapping.restype = ctypes.c_int
    L.pa_reshape_and_cache.argtypes = [cache_p, vp, vp, i64p, i32, vp]
    L.pa_reshape_and_cache.restype = ctypes.c_int
    L.pa_append_kv.argtypes = [cache_p, vp, vp, i32p, i32, i32p, i32p, i32, i32, i64p, i32, vp]
    L.pa_append_kv.restype = ctypes.c_int
    L.pa_decode_auto_partition.argtypes = [i32, i32, i32, i32]
    L.pa_decode_auto_partition.restype = i32
    L.pa_decode_workspace_bytes.argtypes = [i32, i32, i32, i32, i32, i32, i32]
    L.pa_decode_workspace_bytes.restype = sz
    L.pa_decode.argtypes = [cache_p, vp, vp, i32p, i32, i32p, i32, i32, i32, f32, vp, sz, vp]
    L.pa_decode.restype = ctypes.c_int
    L.pa_decode_ex.argtypes = [cache_p, vp, vp, i32p, i32, i32p, i32, i32, i32, f32, vp, sz, i32, vp]
    L.pa_decode_ex.restype = ctypes.c_int
    L.pa_decode_noalloc.argtypes = [cache_p, vp, vp, i32p, i32, i32p, i32, i32, i32, f32, i32, vp]
    L.pa_decode_noalloc.restype = ctypes.c_int
    L.pa_decode_stage.argtypes = [cache_p, vp, vp, i32p, i32, i32p, i32, i32, i32, f32, vp, sz, i32, i32, vp]
    L.pa_decode_stage.restype = ctypes.c_int
    L.pa_decode_timed.argtypes = [cache_p, vp, vp, i32p, i32, i32p, i32, i32, i32, f32, vp, sz, i32, vp, vp, vp]
    L.pa_decode_timed.restype = ctypes.c_int
    L.pa_decode_append.argtypes = [cache_p, vp, vp, i64p, vp, vp, i32p, i32, i32p, i32, i32, i32, f32, vp, sz, i32, vp, vp,
                                   vp]
    L.pa_decode_append.restype = ctypes.c_int
    L.pa_decode_run.argtypes = [ctypes.POINTER(pa_decode_args), vp]
    L.pa_decode_run.restype = ctypes.c_int
    L.pa_decode_plan.argtypes = [vp, i32, i32, i32, vp, i32]
    L.pa_decode_plan.restype = i32
    L.pa_prefill_chunk.argtypes = [cache_p, vp, vp, i32p, i32p, i32p, i32, i32, i32, i32, f32, vp]
    L.pa_prefill_chunk.restype = ctypes.c_int
    for name in ("pa_copy_blocks",):
        getattr(L, name).argtypes = [cache_p, vp, vp, i32, vp]
        getattr(L, name).restype = ctypes.c_int
    for name in ("pa_gather_blocks", "pa_scatter_blocks"):
        getattr(L, name).argtypes = [cache_p, vp, i32, vp, vp, vp]
        getattr(L, name).restype = ctypes.c_int
    bm = ctypes.c_void_p
    i64 = ctypes.c_int64
    L.pa_bm_create.argtypes = [i32, i32, vp]
    L.pa_bm_create.restype = bm
    L.pa_bm_destroy.argtypes = [bm]
    L.pa_bm_destroy.restype = None
    L.pa_bm_available.argtypes = [bm]
    L.pa_bm_available.restype = i32
    L.pa_bm_refcount.argtypes = [bm, i32]
    L.pa_bm_refcount.restype = i32
    L.pa_bm_add_sequence.argtypes = [bm, i64, i32]
    L.pa_bm_add_sequence.restype = ctypes.c_int
    L.pa_bm_fork.argtypes = [bm, i64, i64]
    L.pa_bm_fork.restype = ctypes.c_int
    L.pa_bm_append_tokens.argtypes = [bm, i64, i32, vp, vp, vp]
    L.pa_bm_append_tokens.restype = ctypes.c_int
    L.pa_bm_free_sequence.argtypes = [bm, i64]
    L.pa_bm_free_sequence.restype = ctypes.c_int
    L.pa_bm_block_table.argtypes = [bm, i64, vp, i32]
    L.pa_bm_block_table.restype = i32
    L.pa_bm_num_tokens.argtypes = [bm, i64]
    L.pa_bm_num_tokens.restype = i64
    L.pa_bm_free_list.argtypes = [bm, vp, i32]
    L.pa_bm_free_list.restype = i32
    u64 = ctypes.c_uint64
    L.pa_bm_add_sequence_tokens.argtypes = [bm, i64, vp, i32, u64, vp]
    L.pa_bm_add_sequence_tokens.restype = ctypes.c_int
    L.pa_bm_append_token_ids.argtypes = [bm, i64, vp, i32, vp, vp, vp]
    L.pa_bm_append_token_ids.restype = ctypes.c_int
    L.pa_bm_commit.argtypes = [bm, i64, i32]
    L.pa_bm_commit.restype = ctypes.c_int
    L.pa_bm_drop_version.argtypes = [bm, u64]
    L.pa_bm_drop_version.restype = i32
    L.pa_bm_cached_blocks.argtypes = [bm]
    L.pa_bm_cached_blocks.restype = i32
    L.pa_bm_is_cached.argtypes = [bm, i32]
    L.pa_bm_is_cached.restype = i32
    L.pa_bm_set_hash_bits.argtypes = [bm, i32]
    L.pa_bm_set_hash_bits.restype = ctypes.c_int
    L.pa_bm_block_size.argtypes = [bm]
    L.pa_bm_block_size.restype = i32
    sc = ctypes.c_void_p
    L.pa_sched_create.argtypes = [bm, i32]
    L.pa_sched_create.restype = sc
    L.pa_sched_destroy.argtypes = [sc]
    L.pa_sched_destroy.restype = None
    L.pa_sched_add_request.argtypes = [sc, i64, i32, i32]
    L.pa_sched_add_request.restype = ctypes.c_int
    L.pa_sched_schedule.argtypes = [sc, vp, i32, vp]
    L.pa_sched_schedule.restype = ctypes.c_int
    L.pa_sched_copies.argtypes = [sc, vp, vp, i32]
    L.pa_sched_copies.restype = i32
    L.pa_sched_step.argtypes = [sc, i64]
    L.pa_sched_step.restype = ctypes.c_int
    for name in ("pa_sched_state", "pa_sched_generated"):
        getattr(L, name).argtypes = [sc, i64]
        getattr(L, name).restype = i32
    for name in ("pa_sched_num_waiting", "pa_sched_num_active"):
        getattr(L, name).argtypes = [sc]
        getattr(L, name).restype = i32
    L.pa_stream_read.argtypes = [vp, sz, i32, i32, vp, vp]
    L.pa_stream_read.restype = ctypes.c_int
    L.pa_status_string.argtypes = [ctypes.c_int]
    L.pa_status_string.restype = ctypes.c_char_p
    L.pa_version.argtypes = []
    L.pa_version.restype = ctypes.c_char_p
    _lib = L
    return L


def _stream(stream: Optional[torch.cuda.Stream]) -> int:
    s = stream if stream is not None else torch.cuda.current_stream()
    return s.cuda_stream


def _need(t: torch.Tensor, name: str, dtype=None):
    if not t.is_cuda:
        raise ValueError(f"{name} must be a GPU tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if dtype is not None and t.dtype != dtype:
        raise ValueError(f"{name} must be {dtype}, got {t.dtype}")


def key_shape(num_blocks: int, num_kv_heads: int, block_size: int, head_dim: int, dtype: torch.dtype):
    """Shape of a key pool: each (block, KV head) tile's block_size rows cut
    into column chunks of 64 bytes of elements,
    [num_blocks, num_kv_heads, head_dim // kc, block_size, kc]."""
    kc = 64 // dtype.itemsize
    if head_dim % kc:
        raise ValueError(f"head_dim {head_dim} is not a multiple of the {kc}-element key chunk")
    return (num_blocks, num_kv_heads, head_dim // kc, block_size, kc)


def value_shape(key_shape):
    """Shape of the value pool that goes with a key pool of ``key_shape``."""
    NB, H, NC, B, KC = key_shape
    return (NB, H, NC * KC, B)


def is_fp8(key_cache: torch.Tensor) -> bool:
    return _DTYPE.get(key_cache.dtype) == PA_FP8_E4M3


def io_dtype(key_cache: torch.Tensor) -> torch.dtype:
    """dtype of the queries, outputs and new K/V rows that go with a pool."""
    return torch.float16 if is_fp8(key_cache) else key_cache.dtype


def kv_cache(key_cache: torch.Tensor, value_cache: torch.Tensor, scales=None) -> pa_kv_cache:
    """Describe a pool: keys [num_blocks, num_kv_heads, head_dim // kc,
    block_size, kc] (key_shape: 64-byte column chunks of each key tile),
    values [num_blocks, num_kv_heads, head_dim, block_size] (each value tile
    transposed).

    ``scales`` = (k_scale, v_scale) is required for an FP8 pool: a code c
    stands for value(c) * scale."""
    _need(key_cache, "key_cache")
    _need(value_cache, "value_cache", key_cache.dtype)
    if key_cache.dtype not in _DTYPE:
        raise ValueError(f"unsupported cache dtype {key_cache.dtype}")
    ok = key_cache.dim() == 5 and value_cache.dim() == 4
    if ok:
        NB, H, NC, B, KC = key_cache.shape
        ok = key_cache.shape == key_shape(NB, H, B, NC * KC, key_cache.dtype) and \
            value_cache.shape == value_shape(key_cache.shape)
    if not ok:
        raise ValueError("key_cache must be [num_blocks, num_kv_heads, head_dim // kc, block_size, kc] with kc = 64 "
                         "bytes of elements, and value_cache [num_blocks, num_kv_heads, head_dim, block_size]")
    if is_fp8(key_cache) and scales is None:
        raise ValueError("an FP8 pool needs scales=(k_scale, v_scale)")
    ks, vs = (1.0, 1.0) if scales is None else (float(scales[0]), float(scales[1]))
    return pa_kv_cache(key_cache.data_ptr(), value_cache.data_ptr(), NB, H, NC * KC, B, _DTYPE[key_cache.dtype], ks, vs)


def debug_enabled() -> bool:
    """PA_DEBUG=1: before each launch the binding copies the device-resident
    contents the kernels trust (block tables, lengths, slots, chunk offsets,
    block lists) to the host and checks them, raising ValueError instead of
    launching.  The copies wait for the stream: a debugging aid, not for
    timed runs.  Without it those contents are the caller's contract (the
    kernels skip block ids outside the pool and negative slots, and clamp
    lengths, but compute nothing meaningful from them)."""
    return os.environ.get("PA_DEBUG", "0") not in ("", "0")


def _host(t):
    import numpy as np

    return t.detach().cpu().numpy() if torch.is_tensor(t) else np.asarray(t)


def debug_check_tables(block_tables, seq_lens, num_blocks: int, block_size: int, max_seq_len: int, what: str):
    """Every length in [0, max_seq_len] and within its table row; every
    block id a sequence reads (its first ceil(L / block_size) entries) in
    [0, num_blocks)."""
    import numpy as np

    bt, L = _host(block_tables), _host(seq_lens).astype(np.int64)
    bad = np.nonzero((L < 0) | (L > max_seq_len))[0]
    if bad.size:
        raise ValueError(f"{what}: seq_lens[{bad[0]}] = {L[bad[0]]} outside [0, max_seq_len = {max_seq_len}]")
    need = -(-L // block_size)
    bad = np.nonzero(need > bt.shape[1])[0]
    if bad.size:
        raise ValueError(f"{what}: sequence {bad[0]} needs {need[bad[0]]} blocks, its table row holds {bt.shape[1]}")
    used = np.arange(bt.shape[1])[None, :] < need[:, None]
    s, i = np.nonzero(used & ((bt < 0) | (bt >= num_blocks)))
    if s.size:
        raise ValueError(f"{what}: block_tables[{s[0]}][{i[0]}] = {bt[s[0], i[0]]} outside the pool [0, {num_blocks})")


def debug_check_slots(slot_mapping, num_tokens: int, num_blocks: int, block_size: int, what: str):
    """The first num_tokens slots: negative (skip) or in the pool, and no
    slot written twice."""
    import numpy as np

    sl = _host(slot_mapping)[:num_tokens].astype(np.int64)
    bad = np.nonzero(sl >= (np.int64(num_blocks) * block_size))[0]
    if bad.size:
        raise ValueError(f"{what}: slot_mapping[{bad[0]}] = {sl[bad[0]]} beyond the pool ({num_blocks} x {block_size})")
    live = np.sort(sl[sl >= 0])
    dup = np.nonzero(live[1:] == live[:-1])[0]
    if dup.size:
        raise ValueError(f"{what}: slot {live[dup[0]]} is written by two tokens")


def debug_check_chunks(cu_q_lens, seq_lens, max_q_len: int, num_tokens: int, what: str):
    """Chunk offsets start at 0, never decrease and stay within the token
    rows; every chunk fits max_q_len and its sequence's length."""
    import numpy as np

    cu, L = _host(cu_q_lens).astype(np.int64), _host(seq_lens).astype(np.int64)
    q = np.diff(cu)
    if cu.size == 0 or cu[0] != 0:
        raise ValueError(f"{what}: cu_q_lens must start at 0")
    bad = np.nonzero(q < 0)[0]
    if bad.size:
        raise ValueError(f"{what}: cu_q_lens decreases at sequence {bad[0]}")
    if cu[-1] > num_tokens:
        raise ValueError(f"{what}: cu_q_lens ends at {cu[-1]}, beyond the {num_tokens} token rows")
    bad = np.nonzero(q > max_q_len)[0]
    if bad.size:
        raise ValueError(f"{what}: chunk {bad[0]} has {q[bad[0]]} tokens, more than max_q_len = {max_q_len}")
    bad = np.nonzero(q > L)[0]
    if bad.size:
        raise ValueError(f"{what}: chunk {bad[0]} has {q[bad[0]]} tokens but seq_lens[{bad[0]}] = {L[bad[0]]}")


def debug_check_blocks(ids, num_blocks: int, what: str, distinct: bool = False, other=None):
    """Block ids in [0, num_blocks); with ``distinct`` none twice, and none
    also in ``other`` (a copy's sources)."""
    import numpy as np

    b = _host(ids).astype(np.int64).ravel()
    bad = np.nonzero((b < 0) | (b >= num_blocks))[0]
    if bad.size:
        raise ValueError(f"{what}: block id {b[bad[0]]} outside the pool [0, {num_blocks})")
    if distinct:
        sb = np.sort(b)
        if (sb[1:] == sb[:-1]).any():
            raise ValueError(f"{what}: a destination block appears twice")
        if other is not None and np.intersect1d(b, _host(other)).size:
            raise ValueError(f"{what}: a block is both a source and a destination")


def _check(status: int, what: str):
    if status != 0:
        raise PaError(status, what)


def pa_slot_mapping(block_tables, seq_lens, cu_q_lens, block_size: int, slot_mapping=None, num_tokens=None, stream=None):
    _need(block_tables, "block_tables", torch.int32)
    _need(seq_lens, "seq_lens", torch.int32)
    _need(cu_q_lens, "cu_q_lens", torch.int32)
    S = seq_lens.shape[0]
    if num_tokens is None:
        num_tokens = int(cu_q_lens[-1].item()) if slot_mapping is None else slot_mapping.shape[0]
    if slot_mapping is None:
        slot_mapping = torch.empty(num_tokens, dtype=torch.int64, device=block_tables.device)
    _need(slot_mapping, "slot_mapping", torch.int64)
    if debug_enabled():
        MB = block_tables.shape[1]
        debug_check_tables(block_tables, seq_lens, 2**31 - 1, block_size, MB * block_size, "pa_slot_mapping")
        debug_check_chunks(cu_q_lens, seq_lens, MB * block_size, num_tokens, "pa_slot_mapping")
    st = lib().pa_slot_mapping(block_tables.data_ptr(), block_tables.shape[1], seq_lens.data_ptr(), cu_q_lens.data_ptr(),
                               S, block_size, slot_mapping.data_ptr(), num_tokens, _stream(stream))
    _check(st, "pa_slot_mapping")
    return slot_mapping


def pa_reshape_and_cache(key_cache, value_cache, key, value, slot_mapping, stream=None, scales=None):
    c = kv_cache(key_cache, value_cache, scales)
    _need(key, "key", io_dtype(key_cache))
    _need(value, "value", io_dtype(key_cache))
    _need(slot_mapping, "slot_mapping", torch.int64)
    T = key.shape[0]
    if key.shape != (T, c.num_kv_heads, c.head_dim) or value.shape != key.shape or slot_mapping.shape[0] < T:
        raise ValueError("key/value must be [num_tokens, num_kv_heads, head_dim] with one slot per token")
    if debug_enabled():
        debug_check_slots(slot_mapping, T, c.num_blocks, c.block_size, "pa_reshape_and_cache")
    st = lib().pa_reshape_and_cache(ctypes.byref(c), key.data_ptr(), value.data_ptr(), slot_mapping.data_ptr(), T, _stream(stream))
    _check(st, "pa_reshape_and_cache")


def _append_kv_call(key_cache, value_cache, key, value, block_tables, seq_lens, cu_q_lens, max_q_len, slot_mapping,
                    stream, scales):
    """Checks and marshals the arguments of pa_append_kv: returns the pool
    descriptor, the argument tuple and the slot mapping."""
    c = kv_cache(key_cache, value_cache, scales)
    io = io_dtype(key_cache)
    _need(key, "key", io)
    _need(value, "value", io)
    _need(block_tables, "block_tables", torch.int32)
    _need(seq_lens, "seq_lens", torch.int32)
    _need(cu_q_lens, "cu_q_lens", torch.int32)
    T = key.shape[0]
    S = seq_lens.shape[0]
    if key.shape != (T, c.num_kv_heads, c.head_dim) or value.shape != key.shape or cu_q_lens.shape[0] != S + 1:
        raise ValueError("key/value must be [num_tokens, num_kv_heads, head_dim]; cu_q_lens [num_seqs + 1]")
    if slot_mapping is None:
        slot_mapping = torch.empty(T, dtype=torch.int64, device=key.device)
    _need(slot_mapping, "slot_mapping", torch.int64)
    args = (ctypes.byref(c), key.data_ptr(), value.data_ptr(), block_tables.data_ptr(), block_tables.shape[1],
            seq_lens.data_ptr(), cu_q_lens.data_ptr(), S, int(max_q_len), slot_mapping.data_ptr(), T, _stream(stream))
    return c, args, slot_mapping


def _debug_append(c, key, block_tables, seq_lens, cu_q_lens, max_q_len):
    debug_check_tables(block_tables, seq_lens, c.num_blocks, c.block_size, block_tables.shape[1] * c.block_size,
                       "pa_append_kv")
    debug_check_chunks(cu_q_lens, seq_lens, int(max_q_len), key.shape[0], "pa_append_kv")


def pa_append_kv(key_cache, value_cache, key, value, block_tables, seq_lens, cu_q_lens, max_q_len: int,
                 slot_mapping=None, stream=None, scales=None):
    c, args, slot_mapping = _append_kv_call(key_cache, value_cache, key, value, block_tables, seq_lens, cu_q_lens,
                                            max_q_len, slot_mapping, stream, scales)
    if debug_enabled():
        _debug_append(c, key, block_tables, seq_lens, cu_q_lens, max_q_len)
    _check(lib().pa_append_kv(*args), "pa_append_kv")
    return slot_mapping


def _prepared(name, args, keep, check):
    """A function that calls library entry point `name` again with the
    arguments marshalled once (numbers converted to their C types here)."""
    fn = getattr(lib(), name)
    types = getattr(fn, "argtypes", None)
    if types:
        args = tuple(t(a) if isinstance(a, (int, float)) else a for t, a in zip(types, args))
    debug = debug_enabled()

    def launch():
        if debug:
            check()
        st = fn(*args)
        if st:
            raise PaError(st, name)

    launch.buffers = keep  # the tensors the marshalled pointers refer to stay alive with the function
    return launch


def prepare_append_kv(key_cache, value_cache, key, value, block_tables, seq_lens, cu_q_lens, max_q_len: int,
                      slot_mapping=None, stream=None, scales=None):
    """pa_append_kv with its arguments checked and marshalled once (see
    prepare_decode_append): the returned function launches it again on the
    same buffers."""
    c, args, slot_mapping = _append_kv_call(key_cache, value_cache, key, value, block_tables, seq_lens, cu_q_lens,
                                            max_q_len, slot_mapping, stream, scales)
    keep = (c, key_cache, value_cache, key, value, block_tables, seq_lens, cu_q_lens, slot_mapping)
    return _prepared("pa_append_kv", args, keep,
                     lambda: _debug_append(c, key, block_tables, seq_lens, cu_q_lens, max_q_len))


def pa_decode_auto_partition(num_seqs: int, num_kv_heads: int, max_seq_len: int, block_size: int) -> int:
    return int(lib().pa_decode_auto_partition(num_seqs, num_kv_heads, max_seq_len, block_size))


def pa_decode_workspace_bytes(num_seqs, num_heads, num_kv_heads, head_dim, block_size, max_seq_len, partition_size=0) -> int:
    return int(lib().pa_decode_workspace_bytes(num_seqs, num_heads, num_kv_heads, head_dim, block_size, max_seq_len, partition_size))


def decode_workspace(query, key_cache, max_seq_len: int, partition_size: int = 0) -> torch.Tensor:
    """Allocate (with torch) the scratch pa_decode needs for these shapes."""
    S, Hq, D = query.shape
    n = pa_decode_workspace_bytes(S, Hq, key_cache.shape[1], D, key_cache.shape[3], max_seq_len, partition_size)
    return torch.empty(max(n, 1), dtype=torch.uint8, device=query.device)


def pa_decode(out, query, key_cache, value_cache, block_tables, seq_lens, scale: float, max_seq_len: int,
              workspace: Optional[torch.Tensor] = None, partition_size: int = 0, stream=None, scales=None,
              stage: int = 0):
    """Decode attention; ``stage`` 1 or 2 runs only the partition kernel or
    only the merge (pa_decode_stage), 0 both (pa_decode_ex)."""
    c = kv_cache(key_cache, value_cache, scales)
    _need(query, "query", io_dtype(key_cache))
    _need(out, "out", io_dtype(key_cache))
    _need(block_tables, "block_tables", torch.int32)
    _need(seq_lens, "seq_lens", torch.int32)
    S, Hq, D = query.shape
    if out.shape != query.shape or D != c.head_dim or block_tables.shape[0] != S or seq_lens.shape[0] != S:
        raise ValueError("shape mismatch between query/out/block_tables/seq_lens and the cache")
    if workspace is None:
        workspace = decode_workspace(query, key_cache, max_seq_len, partition_size)
    _need(workspace, "workspace")
    ws_bytes = workspace.numel() * workspace.element_size()
    if debug_enabled():
        debug_check_tables(block_tables, seq_lens, c.num_blocks, c.block_size, int(max_seq_len), "pa_decode")
    args = (ctypes.byref(c), out.data_ptr(), query.data_ptr(), block_tables.data_ptr(), block_tables.shape[1],
            seq_lens.data_ptr(), S, Hq, int(max_seq_len), float(scale), workspace.data_ptr(), ws_bytes, int(partition_size))
    if stage:
        st = lib().pa_decode_stage(*args, int(stage), _stream(stream))
    else:
        st = lib().pa_decode_ex(*args, _stream(stream))
    _check(st, "pa_decode")
    return out


# Scratch bytes pa_decode_noalloc has on each GPU (PA_NOALLOC_SCRATCH_BYTES).
NOALLOC_SCRATCH_BYTES = 16 << 20


def pa_decode_noalloc(out, query, key_cache, value_cache, block_tables, seq_lens, scale: float, max_seq_len: int,
                      partition_size: int = 0, stream=None, scales=None):
    """Decode attention with the library's fixed per-GPU scratch instead of a
    workspace (pa_decode_noalloc): nothing is allocated, here or in the
    library.  Calls that overlap in time on one GPU share that scratch and
    race."""
    c = kv_cache(key_cache, value_cache, scales)
    _need(query, "query", io_dtype(key_cache))
    _need(out, "out", io_dtype(key_cache))
    _need(block_tables, "block_tables", torch.int32)
    _need(seq_lens, "seq_lens", torch.int32)
    S, Hq, D = query.shape
    if out.shape != query.shape or D != c.head_dim or block_tables.shape[0] != S or seq_lens.shape[0] != S:
        raise ValueError("shape mismatch between query/out/block_tables/seq_lens and the cache")
    if debug_enabled():
        debug_check_tables(block_tables, seq_lens, c.num_blocks, c.block_size, int(max_seq_len), "pa_decode_noalloc")
    st = lib().pa_decode_noalloc(ctypes.byref(c), out.data_ptr(), query.data_ptr(), block_tables.data_ptr(),
                                 block_tables.shape[1], seq_lens.data_ptr(), S, Hq, int(max_seq_len), float(scale),
                                 int(partition_size), _stream(stream))
    _check(st, "pa_decode_noalloc")
    return out


def _event_handle(ev) -> int:
    """Raw HIP event of a torch.cuda.Event (which must have been recorded
    once, so that it exists) or an integer handle."""
    h = ev if isinstance(ev, int) else ev.cuda_event
    if not h:
        raise ValueError("record the event once before passing it (torch creates events lazily)")
    return int(h)


def pa_decode_timed(out, query, key_cache, value_cache, block_tables, seq_lens, scale: float, max_seq_len: int,
                    kernel_start, kernel_stop, workspace: Optional[torch.Tensor] = None, partition_size: int = 0,
                    stream=None, scales=None):
    """pa_decode whose partition kernel records its own start and end into
    the two events (torch.cuda.Event or raw handles)."""
    c = kv_cache(key_cache, value_cache, scales)
    _need(query, "query", io_dtype(key_cache))
    _need(out, "out", io_dtype(key_cache))
    _need(block_tables, "block_tables", torch.int32)
    _need(seq_lens, "seq_lens", torch.int32)
    S, Hq, D = query.shape
    if out.shape != query.shape or D != c.head_dim or block_tables.shape[0] != S or seq_lens.shape[0] != S:
        raise ValueError("shape mismatch between query/out/block_tables/seq_lens and the cache")
    if workspace is None:
        workspace = decode_workspace(query, key_cache, max_seq_len, partition_size)
    _need(workspace, "workspace")
    if debug_enabled():
        debug_check_tables(block_tables, seq_lens, c.num_blocks, c.block_size, int(max_seq_len), "pa_decode_timed")
    st = lib().pa_decode_timed(ctypes.byref(c), out.data_ptr(), query.data_ptr(), block_tables.data_ptr(),
                               block_tables.shape[1], seq_lens.data_ptr(), S, Hq, int(max_seq_len), float(scale),
                               workspace.data_ptr(), workspace.numel() * workspace.element_size(), int(partition_size),
                               _event_handle(kernel_start), _event_handle(kernel_stop), _stream(stream))
    _check(st, "pa_decode_timed")
    return out


def _decode_append_call(out, query, key_cache, value_cache, new_key, new_value, block_tables, seq_lens, scale,
                        max_seq_len, slot_mapping, workspace, partition_size, kernel_start, kernel_stop, stream, scales):
    """Checks and marshals the arguments of pa_decode_append: returns the
    pool descriptor (which the argument tuple points to), the tuple and the
    slot mapping."""
    c = kv_cache(key_cache, value_cache, scales)
    io = io_dtype(key_cache)
    _need(query, "query", io)
    _need(out, "out", io)
    _need(new_key, "new_key", io)
    _need(new_value, "new_value", io)
    _need(block_tables, "block_tables", torch.int32)
    _need(seq_lens, "seq_lens", torch.int32)
    S, Hq, D = query.shape
    if out.shape != query.shape or D != c.head_dim or block_tables.shape[0] != S or seq_lens.shape[0] != S:
        raise ValueError("shape mismatch between query/out/block_tables/seq_lens and the cache")
    if new_key.shape != (S, c.num_kv_heads, D) or new_value.shape != new_key.shape:
        raise ValueError("new_key/new_value must be [num_seqs, num_kv_heads, head_dim]")
    if slot_mapping is None:
        slot_mapping = torch.empty(S, dtype=torch.int64, device=query.device)
    _need(slot_mapping, "slot_mapping", torch.int64)
    if workspace is None:
        workspace = decode_workspace(query, key_cache, max_seq_len, partition_size)
    _need(workspace, "workspace")
    ev0 = None if kernel_start is None else _event_handle(kernel_start)
    ev1 = None if kernel_stop is None else _event_handle(kernel_stop)
    args = (ctypes.byref(c), new_key.data_ptr(), new_value.data_ptr(), slot_mapping.data_ptr(), out.data_ptr(),
            query.data_ptr(), block_tables.data_ptr(), block_tables.shape[1], seq_lens.data_ptr(), S, Hq,
            int(max_seq_len), float(scale), workspace.data_ptr(), workspace.numel() * workspace.element_size(),
            int(partition_size), ev0, ev1, _stream(stream))
    return c, args, slot_mapping


def pa_decode_append(out, query, key_cache, value_cache, new_key, new_value, block_tables, seq_lens, scale: float,
                     max_seq_len: int, slot_mapping=None, workspace: Optional[torch.Tensor] = None,
                     partition_size: int = 0, kernel_start=None, kernel_stop=None, stream=None, scales=None):
    """One decode step: each sequence's new token (position seq_lens[s]-1)
    written into the pool, then decode attention, in the partition kernel."""
    c, args, slot_mapping = _decode_append_call(out, query, key_cache, value_cache, new_key, new_value, block_tables,
                                                seq_lens, scale, max_seq_len, slot_mapping, workspace, partition_size,
                                                kernel_start, kernel_stop, stream, scales)
    if debug_enabled():
        debug_check_tables(block_tables, seq_lens, c.num_blocks, c.block_size, int(max_seq_len), "pa_decode_append")
    _check(lib().pa_decode_append(*args), "pa_decode_append")
    return slot_mapping


def prepare_decode_append(out, query, key_cache, value_cache, new_key, new_value, block_tables, seq_lens,
                          scale: float, max_seq_len: int, slot_mapping=None, workspace: Optional[torch.Tensor] = None,
                          partition_size: int = 0, kernel_start=None, kernel_stop=None, stream=None, scales=None):
    """pa_decode_append with its arguments checked and marshalled once: the
    returned function launches the step again on the same buffers (whose
    contents, such as lengths, tables, queries and new rows, may change
    between launches; the buffers themselves, the stream and max_seq_len may
    not).  For a serving loop that keeps its step buffers in place, it takes
    the binding's per-call checks (more than 10 us of Python) off the host's
    path to the launch.  PA_DEBUG is read once, here: with it set, every
    launch checks the tables first."""
    c, args, slot_mapping = _decode_append_call(out, query, key_cache, value_cache, new_key, new_value, block_tables,
                                                seq_lens, scale, max_seq_len, slot_mapping, workspace, partition_size,
                                                kernel_start, kernel_stop, stream, scales)
    keep = (c, out, query, key_cache, value_cache, new_key, new_value, block_tables, seq_lens, slot_mapping, workspace)
    return _prepared("pa_decode_append", args, keep,
                     lambda: debug_check_tables(block_tables, seq_lens, c.num_blocks, c.block_size, int(max_seq_len),
                                                "pa_decode_append"))


def decode_plan(seq_lens_host, max_seq_len: int, partition_size: int, device="cuda") -> torch.Tensor:
    """pa_decode_plan on a host copy of seq_lens; the list, uploaded."""
    import numpy as np

    lens = np.ascontiguousarray(seq_lens_host, dtype=np.int32)
    L = lib()
    n = L.pa_decode_plan(lens.ctypes.data, len(lens), int(max_seq_len), int(partition_size), None, 0)
    if n < 0:
        raise ValueError("pa_decode_plan rejected its arguments")
    work = np.empty(max(n, 1), dtype=np.int32)
    L.pa_decode_plan(lens.ctypes.data, len(lens), int(max_seq_len), int(partition_size), work.ctypes.data, n)
    return torch.from_numpy(work[:n]).to(device)


def pa_decode_run(out, query, key_cache, value_cache, block_tables, seq_lens, scale: float, max_seq_len: int,
                  workspace: Optional[torch.Tensor] = None, partition_size: int = 0, stage: int = 0,
                  new_key=None, new_value=None, slot_mapping=None, work: Optional[torch.Tensor] = None,
                  kernel_start=None, kernel_stop=None, stream=None, scales=None):
    """Every decode option in one call (pa_decode_run)."""
    c = kv_cache(key_cache, value_cache, scales)
    _need(query, "query", io_dtype(key_cache))
    _need(out, "out", io_dtype(key_cache))
    _need(block_tables, "block_tables", torch.int32)
    _need(seq_lens, "seq_lens", torch.int32)
    S, Hq, D = query.shape
    if out.shape != query.shape or D != c.head_dim or block_tables.shape[0] != S or seq_lens.shape[0] != S:
        raise ValueError("shape mismatch between query/out/block_tables/seq_lens and the cache")
    if workspace is None:
        workspace = decode_workspace(query, key_cache, max_seq_len, partition_size)
    _need(workspace, "workspace")
    if debug_enabled():
        debug_check_tables(block_tables, seq_lens, c.num_blocks, c.block_size, int(max_seq_len), "pa_decode_run")
    d = pa_decode_args()
    d.cache = ctypes.pointer(c)
    d.out, d.query = out.data_ptr(), query.data_ptr()
    d.block_tables, d.max_blocks_per_seq = block_tables.data_ptr(), block_tables.shape[1]
    d.seq_lens, d.num_seqs, d.num_heads, d.max_seq_len = seq_lens.data_ptr(), S, Hq, int(max_seq_len)
    d.scale = float(scale)
    d.workspace, d.workspace_bytes = workspace.data_ptr(), workspace.numel() * workspace.element_size()
    d.partition_size, d.stage = int(partition_size), int(stage)
    if new_key is not None:
        _need(new_key, "new_key", io_dtype(key_cache))
        _need(new_value, "new_value", io_dtype(key_cache))
        _need(slot_mapping, "slot_mapping", torch.int64)
        if new_key.shape != (S, c.num_kv_heads, D) or new_value.shape != new_key.shape or slot_mapping.shape != (S,):
            raise ValueError("new_key/new_value [num_seqs, num_kv_heads, head_dim], slot_mapping [num_seqs]")
        d.new_key, d.new_value, d.slot_mapping = new_key.data_ptr(), new_value.data_ptr(), slot_mapping.data_ptr()
    if work is not None:
        _need(work, "work", torch.int32)
        d.work, d.num_work = work.data_ptr(), work.numel()
    if kernel_start is not None:
        d.kernel_start = _event_handle(kernel_start)
    if kernel_stop is not None:
        d.kernel_stop = _event_handle(kernel_stop)
    _check(lib().pa_decode_run(ctypes.byref(d), _stream(stream)), "pa_decode_run")
    return out


def pa_prefill_chunk(out, query, key_cache, value_cache, cu_q_lens, seq_lens, block_tables, scale: float,
                     max_q_len: int, stream=None, scales=None):
    c = kv_cache(key_cache, value_cache, scales)
    _need(query, "query", io_dtype(key_cache))
    _need(out, "out", io_dtype(key_cache))
    _need(cu_q_lens, "cu_q_lens", torch.int32)
    _need(seq_lens, "seq_lens", torch.int32)
    _need(block_tables, "block_tables", torch.int32)
    S = seq_lens.shape[0]
    T, Hq, D = query.shape
    if out.shape != query.shape or D != c.head_dim or cu_q_lens.shape[0] != S + 1 or block_tables.shape[0] != S:
        raise ValueError("shape mismatch between query/out/cu_q_lens/seq_lens/block_tables and the cache")
    if debug_enabled():
        debug_check_tables(block_tables, seq_lens, c.num_blocks, c.block_size, block_tables.shape[1] * c.block_size,
                           "pa_prefill_chunk")
        debug_check_chunks(cu_q_lens, seq_lens, int(max_q_len), T, "pa_prefill_chunk")
    st = lib().pa_prefill_chunk(ctypes.byref(c), out.data_ptr(), query.data_ptr(), cu_q_lens.data_ptr(), seq_lens.data_ptr(),
                                block_tables.data_ptr(), block_tables.shape[1], S, Hq, int(max_q_len), float(scale),
                                _stream(stream))
    _check(st, "pa_prefill_chunk")
    return out


def pa_copy_blocks(key_cache, value_cache, src, dst, stream=None):
    """Pool block src[i] -> pool block dst[i] (device int32 tensors)."""
    c = kv_cache(key_cache, value_cache, (1.0, 1.0))  # bit copies: scales unused
    _need(src, "src", torch.int32)
    _need(dst, "dst", torch.int32)
    if src.shape != dst.shape:
        raise ValueError("src and dst must have the same length")
    if debug_enabled():
        debug_check_blocks(src, c.num_blocks, "pa_copy_blocks")
        debug_check_blocks(dst, c.num_blocks, "pa_copy_blocks", distinct=True, other=src)
    _check(lib().pa_copy_blocks(ctypes.byref(c), src.data_ptr(), dst.data_ptr(), src.numel(), _stream(stream)), "pa_copy_blocks")


def _buf_ok(t, pool, n, name):
    if t.dtype != pool.dtype or not t.is_contiguous() or tuple(t.shape) != (n, *pool.shape[1:]):
        raise ValueError(f"{name} must be contiguous [{n}, *block shape of its pool] in the cache dtype")
    if not (t.is_cuda or t.is_pinned()):
        raise ValueError(f"{name} must be device memory or pinned host memory")


def pa_gather_blocks(key_cache, value_cache, block_ids, key_out, value_out, stream=None):
    c = kv_cache(key_cache, value_cache, (1.0, 1.0))  # bit copies: scales unused
    _need(block_ids, "block_ids", torch.int32)
    n = block_ids.numel()
    _buf_ok(key_out, key_cache, n, "key_out")
    _buf_ok(value_out, value_cache, n, "value_out")
    if debug_enabled():
        debug_check_blocks(block_ids, c.num_blocks, "pa_gather_blocks")
    _check(lib().pa_gather_blocks(ctypes.byref(c), block_ids.data_ptr(), n, key_out.data_ptr(), value_out.data_ptr(),
                                  _stream(stream)), "pa_gather_blocks")


def pa_scatter_blocks(key_cache, value_cache, block_ids, key_in, value_in, stream=None):
    c = kv_cache(key_cache, value_cache, (1.0, 1.0))  # bit copies: scales unused
    _need(block_ids, "block_ids", torch.int32)
    n = block_ids.numel()
    _buf_ok(key_in, key_cache, n, "key_in")
    _buf_ok(value_in, value_cache, n, "value_in")
    if debug_enabled():
        debug_check_blocks(block_ids, c.num_blocks, "pa_scatter_blocks", distinct=True)
    _check(lib().pa_scatter_blocks(ctypes.byref(c), block_ids.data_ptr(), n, key_in.data_ptr(), value_in.data_ptr(),
                                   _stream(stream)), "pa_scatter_blocks")


class BlockManager:
    """The library's host-side block manager (FIFO pool, refcounts, copy-on-write, prefix cache)."""

    def __init__(self, num_blocks: int, block_size: int, free_order=None):
        L = lib()
        self._order = None
        ptr = None
        if free_order is not None:
            import numpy as np

            self._order = np.ascontiguousarray(free_order, dtype=np.int32)
            ptr = self._order.ctypes.data
        self._h = L.pa_bm_create(int(num_blocks), int(block_size), ptr)
        if not self._h:
            raise ValueError("pa_bm_create rejected its arguments")
        self.num_blocks, self.block_size = int(num_blocks), int(block_size)

    def close(self):
        h = getattr(self, "_h", None)
        self._h = None
        if h and _lib is not None:  # at interpreter exit the library may already be gone
            _lib.pa_bm_destroy(h)

    __del__ = close

    def available(self) -> int:
        return int(lib().pa_bm_available(self._h))

    def refcount(self, block: int) -> int:
        return int(lib().pa_bm_refcount(self._h, int(block)))

    def add_sequence(self, seq_id: int, num_tokens: int):
        _check(lib().pa_bm_add_sequence(self._h, int(seq_id), int(num_tokens)), "pa_bm_add_sequence")

    def fork(self, parent: int, child: int):
        _check(lib().pa_bm_fork(self._h, int(parent), int(child)), "pa_bm_fork")

    def append_tokens(self, seq_id: int, num_new: int):
        """Returns the (src, dst) block pairs to copy before scattering."""
        src, dst, n = ctypes.c_int32(), ctypes.c_int32(), ctypes.c_int32()
        _check(lib().pa_bm_append_tokens(self._h, int(seq_id), int(num_new), ctypes.addressof(src), ctypes.addressof(dst),
                                         ctypes.addressof(n)), "pa_bm_append_tokens")
        return [(src.value, dst.value)] if n.value else []

    def free_sequence(self, seq_id: int):
        _check(lib().pa_bm_free_sequence(self._h, int(seq_id)), "pa_bm_free_sequence")

    def block_table(self, seq_id: int):
        L = lib()
        n = L.pa_bm_block_table(self._h, int(seq_id), None, 0)
        if n < 0:
            raise PaError(7, "pa_bm_block_table")
        buf = (ctypes.c_int32 * max(n, 1))()
        L.pa_bm_block_table(self._h, int(seq_id), buf, n)
        return list(buf[:n])

    def num_tokens(self, seq_id: int) -> int:
        return int(lib().pa_bm_num_tokens(self._h, int(seq_id)))

    def free_list(self):
        L = lib()
        n = L.pa_bm_free_list(self._h, None, 0)
        buf = (ctypes.c_int32 * max(n, 1))()
        L.pa_bm_free_list(self._h, buf, n)
        return list(buf[:n])

    # Prefix cache
    @staticmethod
    def _ids(token_ids):
        arr = (ctypes.c_int32 * max(len(token_ids), 1))(*[int(x) for x in token_ids])
        return arr, len(token_ids)

    def add_sequence_tokens(self, seq_id: int, token_ids, version: int = 0) -> int:
        """New sequence with token ids; returns how many leading tokens were found cached."""
        arr, n = self._ids(token_ids)
        hit = ctypes.c_int32()
        _check(lib().pa_bm_add_sequence_tokens(self._h, int(seq_id), arr, n, int(version), ctypes.addressof(hit)),
               "pa_bm_add_sequence_tokens")
        return hit.value

    def append_token_ids(self, seq_id: int, token_ids):
        arr, n = self._ids(token_ids)
        src, dst, k = ctypes.c_int32(), ctypes.c_int32(), ctypes.c_int32()
        _check(lib().pa_bm_append_token_ids(self._h, int(seq_id), arr, n, ctypes.addressof(src), ctypes.addressof(dst),
                                            ctypes.addressof(k)), "pa_bm_append_token_ids")
        return [(src.value, dst.value)] if k.value else []

    def commit(self, seq_id: int, num_computed_tokens: int):
        _check(lib().pa_bm_commit(self._h, int(seq_id), int(num_computed_tokens)), "pa_bm_commit")

    def drop_version(self, version: int) -> int:
        return int(lib().pa_bm_drop_version(self._h, int(version)))

    def cached_blocks(self) -> int:
        return int(lib().pa_bm_cached_blocks(self._h))

    def is_cached(self, block: int) -> bool:
        return lib().pa_bm_is_cached(self._h, int(block)) == 1

    def set_hash_bits(self, bits: int):
        _check(lib().pa_bm_set_hash_bits(self._h, int(bits)), "pa_bm_set_hash_bits")


class Scheduler:
    """The library's continuous-batching step arithmetic over a BlockManager
    (request ids are the manager's sequence ids)."""

    WAITING, DECODING, FINISHED = 0, 1, 2

    def __init__(self, manager: BlockManager, max_batch_size: int):
        self._bm = manager  # keeps the manager alive while the scheduler uses it
        self._h = lib().pa_sched_create(manager._h, int(max_batch_size))
        if not self._h:
            raise ValueError("pa_sched_create rejected its arguments")

    def close(self):
        h = getattr(self, "_h", None)
        self._h = None
        if h and _lib is not None:
            _lib.pa_sched_destroy(h)

    __del__ = close

    def add_request(self, request_id: int, prompt_len: int, max_tokens: int):
        _check(lib().pa_sched_add_request(self._h, int(request_id), int(prompt_len), int(max_tokens)),
               "pa_sched_add_request")

    def schedule(self):
        """One iteration; returns the scheduled request ids in order."""
        L = lib()
        n = ctypes.c_int32()
        cap = max(L.pa_sched_num_active(self._h) + L.pa_sched_num_waiting(self._h), 1)
        buf = (ctypes.c_int64 * cap)()
        _check(L.pa_sched_schedule(self._h, buf, cap, ctypes.addressof(n)), "pa_sched_schedule")
        return list(buf[: n.value])

    def copies(self):
        """Copy-on-write (old, new) block pairs of the last schedule() call."""
        L = lib()
        n = L.pa_sched_copies(self._h, None, None, 0)
        if n <= 0:
            return []
        src, dst = (ctypes.c_int32 * n)(), (ctypes.c_int32 * n)()
        L.pa_sched_copies(self._h, src, dst, n)
        return list(zip(src, dst))

    def step(self, request_id: int):
        _check(lib().pa_sched_step(self._h, int(request_id)), "pa_sched_step")

    def state(self, request_id: int) -> int:
        return int(lib().pa_sched_state(self._h, int(request_id)))

    def generated(self, request_id: int) -> int:
        return int(lib().pa_sched_generated(self._h, int(request_id)))

    def num_waiting(self) -> int:
        return int(lib().pa_sched_num_waiting(self._h))

    def num_active(self) -> int:
        return int(lib().pa_sched_num_active(self._h))


def pa_stream_read(src: torch.Tensor, workgroups: int, threads: int, sink: torch.Tensor, stream=None):
    """Measurement helper: a plain streaming read of ``src`` (all its bytes)
    at the given launch shape; ``sink`` is a uint32/int32 device tensor of at
    least ``workgroups`` words (XOR-ed)."""
    _need(src, "src")
    _need(sink, "sink")
    if sink.numel() < workgroups or sink.element_size() != 4:
        raise ValueError("sink needs one 32-bit word per workgroup")
    nbytes = src.numel() * src.element_size()
    _check(lib().pa_stream_read(src.data_ptr(), nbytes, int(workgroups), int(threads), sink.data_ptr(),
                                _stream(stream)), "pa_stream_read")


def version() -> str:
    return lib().pa_version().decode()
