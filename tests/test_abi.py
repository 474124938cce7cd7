"""The C ABI library loads, exports everything include/pa.h declares, and
rejects bad arguments on the host before any launch.  CPU only: no call here
reaches a kernel."""

import ctypes
import os
import re

import pytest

from tests import harness

ROOT = harness.ROOT


@pytest.fixture(scope="module")
def L():
    harness.build_if_missing()
    from paged_kv_cache_326_amd import pa

    return pa.lib()


def _declared():
    txt = open(os.path.join(ROOT, "include", "pa.h")).read()
    txt = re.sub(r"/\*.*?\*/", "", txt, flags=re.S)
    return sorted(set(re.findall(r"\b(pa_[a-z0-9_]+)\s*\(", txt)))


def test_exports_every_declared_symbol(L):
    names = _declared()
    assert "pa_decode" in names and "pa_reshape_and_cache" in names
    for n in names:
        assert hasattr(L, n), f"libpa.so does not export {n}"
    from paged_kv_cache_326_amd import pa

    assert set(pa.EXPORTS) <= set(names)


def test_version_and_status_strings(L):
    assert b"gfx950" in L.pa_version()
    for s in range(9):
        assert L.pa_status_string(s)


def _cache(pa, **kw):
    c = pa.pa_kv_cache(0x1000, 0x2000, 64, 2, 64, 16, pa.PA_F16)
    for k, v in kw.items():
        setattr(c, k, v)
    return c


def _decode(L, pa, c, **kw):
    a = dict(out=0x3000, query=0x4000, bt=0x5000, mb=4, sl=0x6000, S=4, Hq=8, maxL=50, scale=0.125,
             ws=0x7000, wsb=1 << 20, P=0)
    a.update(kw)
    return L.pa_decode_ex(ctypes.byref(c), a["out"], a["query"], a["bt"], a["mb"], a["sl"], a["S"], a["Hq"], a["maxL"],
                          a["scale"], a["ws"], a["wsb"], a["P"], None)


def test_decode_argument_errors(L):
    from paged_kv_cache_326_amd import pa

    assert _decode(L, pa, _cache(pa, key_cache=0)) == 1  # NULL cache array
    assert _decode(L, pa, _cache(pa), query=0) == 1
    assert _decode(L, pa, _cache(pa, head_dim=96)) == 3  # unsupported head_dim
    assert _decode(L, pa, _cache(pa, block_size=8)) == 3
    assert _decode(L, pa, _cache(pa, dtype=7)) == 3
    assert _decode(L, pa, _cache(pa), Hq=7) == 2  # not a multiple of num_kv_heads
    assert _decode(L, pa, _cache(pa), Hq=32) == 3  # group of 16 not built
    assert _decode(L, pa, _cache(pa), maxL=65) == 2  # beyond max_blocks_per_seq * block_size
    assert _decode(L, pa, _cache(pa), P=24) == 2  # not a multiple of block_size
    assert _decode(L, pa, _cache(pa), P=8192) == 2  # above the 4096-token maximum
    assert _decode(L, pa, _cache(pa), P=16, ws=0) == 4  # needs a workspace
    assert _decode(L, pa, _cache(pa), P=16, wsb=100) == 4
    assert _decode(L, pa, _cache(pa), S=0) == 0  # nothing to do, nothing launched


def test_workspace_size_formula(L):
    # 4 sequences x 8 heads x ceil(50/16)=4 partitions: m and l rows (float32,
    # 256-byte aligned) plus head_dim floats per row.
    rows = 4 * 8 * 4
    al = lambda x: (x + 255) // 256 * 256  # noqa: E731
    assert L.pa_decode_workspace_bytes(4, 8, 2, 64, 16, 50, 16) == 2 * al(rows * 4) + al(rows * 64 * 4)
    assert L.pa_decode_workspace_bytes(4, 8, 2, 64, 16, 50, 64) == 0  # one partition: written directly
    # 16 x 8 = 128 pairs: two 2048-token parts each, one workgroup per compute unit
    assert L.pa_decode_auto_partition(16, 8, 4096, 16) == 2048
    assert L.pa_decode_auto_partition(32, 8, 1280, 16) == 1280  # 256 pairs fill the chip alone
    assert L.pa_decode_auto_partition(64, 8, 7852, 16) == 1024  # 512 pairs: 1024-token partitions
    assert L.pa_decode_auto_partition(4, 2, 50, 16) == 16  # tiny: rounded up to one block
    assert L.pa_decode_auto_partition(1, 1, 10**6, 32) == 3936  # 10^6 / 256 parts, rounded up to blocks
    assert L.pa_decode_auto_partition(1, 1, 10**7, 32) == 4096  # capped


def test_scatter_and_slot_argument_errors(L):
    from paged_kv_cache_326_amd import pa

    c = _cache(pa)
    assert L.pa_reshape_and_cache(ctypes.byref(c), 0, 0x10, 0x20, 4, None) == 1
    assert L.pa_reshape_and_cache(ctypes.byref(c), 0x10, 0x10, 0x20, -1, None) == 2
    assert L.pa_reshape_and_cache(ctypes.byref(c), 0x10, 0x10, 0x20, 0, None) == 0
    assert L.pa_reshape_and_cache(ctypes.byref(_cache(pa, num_blocks=0)), 0x10, 0x10, 0x20, 4, None) == 2
    assert L.pa_slot_mapping(0x10, 4, 0x20, 0x30, 4, 0, 0x40, 4, None) == 2
    assert L.pa_slot_mapping(0x10, 4, 0, 0x30, 4, 16, 0x40, 4, None) == 1
    assert L.pa_slot_mapping(0x10, 4, 0x20, 0x30, 0, 16, 0x40, 0, None) == 0


def test_block_move_argument_errors(L):
    from paged_kv_cache_326_amd import pa

    c = _cache(pa)
    assert L.pa_copy_blocks(ctypes.byref(c), 0x10, 0, 4, None) == 1  # no dst
    assert L.pa_copy_blocks(ctypes.byref(c), 0x10, 0x20, -1, None) == 2
    assert L.pa_copy_blocks(ctypes.byref(c), 0x10, 0x20, 0, None) == 0  # nothing to do
    assert L.pa_copy_blocks(ctypes.byref(_cache(pa, head_dim=96)), 0x10, 0x20, 4, None) == 3
    assert L.pa_gather_blocks(ctypes.byref(c), 0x10, 4, 0, 0x30, None) == 1
    assert L.pa_scatter_blocks(ctypes.byref(c), 0, 4, 0x20, 0x30, None) == 1
    assert L.pa_scatter_blocks(ctypes.byref(c), 0x10, 0, 0x20, 0x30, None) == 0


def test_decode_stage_argument_errors(L):
    from paged_kv_cache_326_amd import pa

    c = _cache(pa)
    args = (ctypes.byref(c), 0x3000, 0x4000, 0x5000, 4, 0x6000, 4, 8, 50, 0.125, 0x7000, 1 << 20, 0)
    assert L.pa_decode_stage(*args, 3, None) == 2  # no such stage
    assert L.pa_decode_stage(*args, 0, None) == 2
    c0 = _cache(pa, key_cache=0)
    assert L.pa_decode_stage(ctypes.byref(c0), *args[1:], 1, None) == 1


def _plan(L, lens, maxL, P):
    import numpy as np

    arr = np.ascontiguousarray(lens, dtype=np.int32)
    n = L.pa_decode_plan(arr.ctypes.data, len(arr), maxL, P, None, 0)
    out = np.zeros(max(n, 1), np.int32)
    assert L.pa_decode_plan(arr.ctypes.data, len(arr), maxL, P, out.ctypes.data, n) == n
    return n, out[:n]


def test_decode_plan_lists_live_partitions_longest_first(L):
    import numpy as np

    rng = np.random.default_rng(0)
    for trial in range(50):
        S = int(rng.integers(1, 40))
        maxL = int(rng.integers(1, 5000))
        P = int(rng.choice([16, 64, 256, 1024]))
        lens = rng.integers(-3, maxL + 50, size=S)
        n, work = _plan(L, lens, maxL, P)
        np_ = -(-maxL // P)
        # brute force: every (s, part) with a token, plus partition 0 of empty sequences
        units = []
        for s, l in enumerate(lens):
            l = min(max(int(l), 0), maxL)
            parts = -(-l // P) if l > 0 else 1
            units += [(min(P, l - q * P), s, q) for q in range(parts)]
        assert n == len(units)
        got = [(int(x) // np_, int(x) % np_) for x in work]
        assert sorted(got) == sorted((s, q) for _, s, q in units)
        sizes = {(s, q): z for z, s, q in units}
        seq = [sizes[u] for u in got]
        assert all(a >= b for a, b in zip(seq, seq[1:]))  # longest first
        for i in range(1, len(got)):  # ties keep sequence order
            if seq[i] == seq[i - 1]:
                assert got[i] > got[i - 1]
    assert L.pa_decode_plan(None, 3, 10, 16, None, 0) == -1
    assert L.pa_decode_plan(None, 0, 10, 16, None, 0) == 0
    assert L.pa_decode_plan(None, 0, 10, 0, None, 0) == -1


def test_decode_run_argument_errors(L):
    from paged_kv_cache_326_amd import pa

    c = _cache(pa)
    d = pa.pa_decode_args()
    d.cache = ctypes.pointer(c)
    d.out, d.query, d.block_tables, d.max_blocks_per_seq, d.seq_lens = 0x3000, 0x4000, 0x5000, 4, 0x6000
    d.num_seqs, d.num_heads, d.max_seq_len, d.scale = 4, 8, 50, 0.125
    d.workspace, d.workspace_bytes = 0x7000, 1 << 20
    assert L.pa_decode_run(None, None) == 1
    d.stage = 3
    assert L.pa_decode_run(ctypes.byref(d), None) == 2
    d.stage = 0
    d.new_key = 0x8000  # fused append needs all three of key, value, slot_mapping
    assert L.pa_decode_run(ctypes.byref(d), None) == 1
    d.new_key = 0
    d.work, d.num_work = 0x9000, 0  # a plan always lists something
    assert L.pa_decode_run(ctypes.byref(d), None) == 2
    d.num_work = -1
    assert L.pa_decode_run(ctypes.byref(d), None) == 2


def test_decode_noalloc_refuses_oversize_batches_on_the_host(L):
    # Partials beyond the fixed scratch (64 x 32 heads x 500 partitions of
    # D = 128) are refused before anything touches a device; so are bad caches.
    from paged_kv_cache_326_amd import pa

    c = _cache(pa, num_blocks=40000, num_kv_heads=8, head_dim=128)
    assert L.pa_decode_workspace_bytes(64, 32, 8, 128, 16, 8000, 16) > pa.NOALLOC_SCRATCH_BYTES
    assert L.pa_decode_noalloc(ctypes.byref(c), 0x3000, 0x4000, 0x5000, 500, 0x6000, 64, 32, 8000, 0.1, 16,
                               None) == pa.PA_ERR_WORKSPACE
    assert L.pa_decode_noalloc(None, 0x3000, 0x4000, 0x5000, 500, 0x6000, 64, 32, 8000, 0.1, 16, None) == 1
    assert L.pa_decode_noalloc(ctypes.byref(_cache(pa, head_dim=96)), 0x3000, 0x4000, 0x5000, 4, 0x6000, 4, 8, 50,
                               0.1, 0, None) == 3


def test_stream_read_rejects_bad_shapes_on_the_host(L):
    # The measurement helper checks its launch shape before launching.
    assert L.pa_stream_read(0x1000, 1 << 20, 0, 256, 0x2000, None) == 2   # no workgroups
    assert L.pa_stream_read(0x1000, 1 << 20, 4, 100, 0x2000, None) == 2   # not whole waves
    assert L.pa_stream_read(0x1000, 1 << 20, 4, 2048, 0x2000, None) == 2  # over 1024 threads
    assert L.pa_stream_read(0x1000, 1000, 4, 256, 0x2000, None) == 2      # not 16-byte pieces
    assert L.pa_stream_read(0x1008, 1 << 20, 4, 256, 0x2000, None) == 2   # misaligned
    assert L.pa_stream_read(0, 1 << 20, 4, 256, 0x2000, None) == 1
    assert L.pa_stream_read(0x1000, 1 << 20, 4, 256, 0, None) == 1
    assert L.pa_stream_read(0x1000, 0, 4, 256, 0x2000, None) == 0         # nothing to read
