"""Parity of the HIP path (through the C ABI) with the CPU oracle: slot
mapping and the KV scatter bit-exact, decode attention within tolerance, on
the five seeded configs at full size plus shape/partition sweeps and edge
cases.  GPU only."""

import numpy as np
import pytest

import oracle
from paged_kv_cache_326_amd import synth

from tests import harness

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    import torch

    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    harness.build_if_missing()
    yield
    torch.cuda.synchronize()


def _sync():
    import torch

    torch.cuda.synchronize()


def _as64(t, dt):
    return oracle.to_float64(harness.from_device(t, dt), dt)


def _assert_close(got, ref, dt, what):
    ok, maxerr, nbad = harness.tolerance_ok(got, ref, dt)
    print(f"{what}: max abs err {maxerr:.3e}, {nbad} outside tolerance", flush=True)
    assert ok, f"{what}: {nbad} elements outside tolerance (max err {maxerr:.3e})"


@pytest.mark.parametrize("k", [1, 2, 3, 4, 5])
def test_slot_mapping_and_scatter_bitexact(k):
    w = synth.config(k)
    gw = harness.GpuWorkload(w)
    slots = gw.slots()
    gw.scatter()
    _sync()
    ref_slots, ref_kc, ref_vc = harness.oracle_scatter_storage(w)
    np.testing.assert_array_equal(slots.cpu().numpy(), ref_slots)
    # Whole pool, byte for byte: target slots hold the new tokens, every other
    # byte (including the NaN poison) is untouched.
    for got, ref in ((gw.key_cache, ref_kc), (gw.value_cache, ref_vc)):
        g = harness.from_device(got, w.dtype)
        assert np.array_equal(np.ascontiguousarray(g).view(np.uint8), np.ascontiguousarray(ref).view(np.uint8))


@pytest.mark.parametrize("k", [1, 2, 3, 4, 5])
def test_append_kv_bitexact(k):
    # Slot mapping + scatter fused in one launch: same slots, same pool bytes.
    w = synth.config(k)
    gw = harness.GpuWorkload(w)
    slots = gw.append()
    _sync()
    ref_slots, ref_kc, ref_vc = harness.oracle_scatter_storage(w)
    np.testing.assert_array_equal(slots.cpu().numpy(), ref_slots)
    for got, ref in ((gw.key_cache, ref_kc), (gw.value_cache, ref_vc)):
        g = harness.from_device(got, w.dtype)
        assert np.array_equal(np.ascontiguousarray(g).view(np.uint8), np.ascontiguousarray(ref).view(np.uint8))


def test_scatter_skips_negative_slots():
    import torch

    w = synth.config(1)
    gw = harness.GpuWorkload(w)
    gw.slots()
    gw.slot_mapping[1] = -1
    gw.slot_mapping[3] = -5
    gw.scatter()
    _sync()
    slots = gw.slot_mapping.cpu().numpy()
    kc, vc = w.key_cache.copy(), w.value_cache.copy()
    oracle.reshape_and_cache(kc, vc, w.new_key, w.new_value, slots)
    assert np.array_equal(harness.from_device(gw.key_cache, w.dtype).view(np.uint8), kc.view(np.uint8))
    assert np.array_equal(harness.from_device(gw.value_cache, w.dtype).view(np.uint8), vc.view(np.uint8))
    del torch


@pytest.mark.parametrize("k", [1, 2, 3, 4])
def test_decode_parity_full_config(k):
    w = synth.config(k)
    gw = harness.GpuWorkload(w)
    out = gw.step()
    _sync()
    _, _, _, ref = harness.oracle_step(w)
    _assert_close(_as64(out, w.dtype), ref, w.dtype, f"config {k} decode")


def test_decode_parity_mixed_batch_decode_part():
    w = synth.config(5)
    gw = harness.GpuWorkload(w)
    gw.slots()
    gw.scatter()  # all 2096 new tokens, chunk and decode alike
    _, dec = synth.prefill_decode_split(w)
    wd = w.subset(dec)
    gd = harness.GpuWorkload(wd)
    gd.key_cache, gd.value_cache = gw.key_cache, gw.value_cache
    out = gd.decode()
    _sync()
    slots, kc, vc, _ = harness.oracle_step(w, seqs=[])
    ref = oracle.decode_attention(oracle.to_float64(wd.query, w.dtype), kc, vc, wd.block_tables, wd.seq_lens, w.scale)
    _assert_close(_as64(out, w.dtype), ref, w.dtype, "config 5 decode sequences")


@pytest.mark.parametrize("partition", [16, 32, 64, 128, 256, 512, 1024, 2048, 4096, 0])
def test_decode_partition_sweep(partition):
    w = synth.config(3, scale_down=4)
    gw = harness.GpuWorkload(w)
    out = gw.step(partition_size=partition)
    _sync()
    _, _, _, ref = harness.oracle_step(w)
    _assert_close(_as64(out, w.dtype), ref, w.dtype, f"config 3/4 P={partition}")


@pytest.mark.parametrize("dt", ["f16", "bf16"])
@pytest.mark.parametrize("partition", [0, 512, 1024, 4096])
def test_decode_eight_wave_workgroups_and_long_partitions(dt, partition):
    # 8 sequences x 4 KV heads: with 1024- or 4096-token partitions (and the
    # automatic choice) the workgroups fit one round of the chip and run 8
    # waves each; with 512 they do not and run 4.  Lengths straddle the
    # partition and block boundaries.
    w = synth.custom(seed=77, dtype=dt, num_heads=32, num_kv_heads=4, head_dim=128, block_size=16,
                     seq_lens=[1, 17, 1000, 2049, 4096, 4097, 6000, 8191])
    gw = harness.GpuWorkload(w)
    out = gw.step(partition_size=partition)
    _sync()
    _, _, _, ref = harness.oracle_step(w)
    _assert_close(_as64(out, w.dtype), ref, w.dtype, f"8-wave case {dt} P={partition}")


def test_decode_two_stages_match_the_single_call():
    import torch
    from paged_kv_cache_326_amd import pa

    w = synth.config(3, scale_down=4)
    gw = harness.GpuWorkload(w)
    gw.append()
    one = gw.decode().clone()
    ws = pa.decode_workspace(gw.query, gw.key_cache, w.max_seq_len)
    two = torch.full_like(one, float("nan"))
    for stage in (1, 2):
        pa.pa_decode(two, gw.query, gw.key_cache, gw.value_cache, gw.block_tables, gw.seq_lens, w.scale,
                     w.max_seq_len, workspace=ws, stage=stage)
    _sync()
    assert torch.equal(one.view(torch.int16), two.view(torch.int16))


def test_decode_timed_matches_and_times_the_partition_kernel():
    import torch
    from paged_kv_cache_326_amd import pa

    w = synth.config(4, scale_down=2)
    gw = harness.GpuWorkload(w)
    gw.append()
    one = gw.decode().clone()
    t0, t1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t0.record()
    t1.record()
    two = torch.full_like(one, float("nan"))
    pa.pa_decode_timed(two, gw.query, gw.key_cache, gw.value_cache, gw.block_tables, gw.seq_lens, w.scale,
                       w.max_seq_len, t0, t1)
    _sync()
    assert torch.equal(one.view(torch.int16), two.view(torch.int16))
    ms = t0.elapsed_time(t1)
    assert 0.0 < ms < 100.0


@pytest.mark.parametrize("k,partition", [(1, 0), (2, 0), (2, 512), (3, 0), (3, 64), (4, 0)])
def test_fused_append_decode_matches_append_then_decode(k, partition):
    # One call (the partition kernel writes each sequence's new token) against
    # pa_append_kv followed by pa_decode: the same pool bytes, slots and
    # outputs, bit for bit; and the output against the oracle.
    import torch
    from paged_kv_cache_326_amd import pa

    w = synth.config(k, scale_down=4 if k in (2, 3) else 1)
    ref_w = harness.GpuWorkload(w)
    ref_w.append()
    ref_out = ref_w.decode(partition_size=partition).clone()
    gw = harness.GpuWorkload(w)
    slots = torch.full((w.num_seqs,), -7, dtype=torch.int64, device="cuda")
    pa.pa_decode_append(gw.out, gw.query, gw.key_cache, gw.value_cache, gw.new_key, gw.new_value, gw.block_tables,
                        gw.seq_lens, w.scale, w.max_seq_len, slot_mapping=slots, partition_size=partition)
    _sync()
    assert torch.equal(slots, ref_w.slot_mapping)
    for a_, b_ in ((gw.key_cache, ref_w.key_cache), (gw.value_cache, ref_w.value_cache), (gw.out, ref_out)):
        assert np.array_equal(harness.from_device(a_, w.dtype).view(np.uint8), harness.from_device(b_, w.dtype).view(np.uint8))
    _, _, _, ref = harness.oracle_step(w)
    _assert_close(_as64(gw.out, w.dtype), ref, w.dtype, f"fused append + decode, config {k}")


@pytest.mark.parametrize("k,partition", [(1, 0), (3, 64)])
def test_prepared_decode_append_matches_the_plain_call(k, partition):
    # prepare_decode_append marshals the arguments once; its launches must
    # match pa_decode_append bit for bit, also after the buffers' contents
    # (queries, new rows) change in place between launches.
    import torch
    from paged_kv_cache_326_amd import pa

    w = synth.config(k, scale_down=4 if k == 3 else 1)
    ref, gw = harness.GpuWorkload(w), harness.GpuWorkload(w)
    launch = pa.prepare_decode_append(gw.out, gw.query, gw.key_cache, gw.value_cache, gw.new_key, gw.new_value,
                                      gw.block_tables, gw.seq_lens, w.scale, w.max_seq_len,
                                      slot_mapping=gw.slot_mapping, partition_size=partition)
    g = torch.Generator(device="cuda").manual_seed(77)
    for rnd in range(2):
        if rnd:
            for t in ("query", "new_key", "new_value"):
                fresh = torch.randn(getattr(gw, t).shape, generator=g, device="cuda").to(getattr(gw, t).dtype)
                getattr(gw, t).copy_(fresh)
                getattr(ref, t).copy_(fresh)
        pa.pa_decode_append(ref.out, ref.query, ref.key_cache, ref.value_cache, ref.new_key, ref.new_value,
                            ref.block_tables, ref.seq_lens, w.scale, w.max_seq_len, slot_mapping=ref.slot_mapping,
                            partition_size=partition)
        gw.out.fill_(float("nan"))
        launch()
        _sync()
        assert torch.equal(gw.slot_mapping, ref.slot_mapping)
        for a_, b_ in ((gw.key_cache, ref.key_cache), (gw.value_cache, ref.value_cache), (gw.out, ref.out)):
            assert np.array_equal(harness.from_device(a_, w.dtype).view(np.uint8),
                                  harness.from_device(b_, w.dtype).view(np.uint8)), f"launch {rnd}"


def _planned_vs_plain(w, partition=0, append=False):
    import torch
    from paged_kv_cache_326_amd import pa

    P = partition or pa.pa_decode_auto_partition(w.num_seqs, w.num_kv_heads, w.max_seq_len, w.block_size)
    work = pa.decode_plan(w.seq_lens, w.max_seq_len, P)
    plain, planned = harness.GpuWorkload(w), harness.GpuWorkload(w)
    if not append:
        plain.append()
        planned.append()
        plain.decode(partition_size=P)
        pa.pa_decode_run(planned.out, planned.query, planned.key_cache, planned.value_cache, planned.block_tables,
                         planned.seq_lens, w.scale, w.max_seq_len, partition_size=P, work=work)
    else:
        for g, wk in ((plain, None), (planned, work)):
            pa.pa_decode_run(g.out, g.query, g.key_cache, g.value_cache, g.block_tables, g.seq_lens, w.scale,
                             w.max_seq_len, partition_size=P, new_key=g.new_key, new_value=g.new_value,
                             slot_mapping=g.slot_mapping, work=wk)
    _sync()
    for a_, b_ in ((plain.out, planned.out), (plain.key_cache, planned.key_cache), (plain.value_cache, planned.value_cache)):
        assert np.array_equal(harness.from_device(a_, w.dtype).view(np.uint8), harness.from_device(b_, w.dtype).view(np.uint8))
    _, _, _, ref = harness.oracle_step(w)
    _assert_close(_as64(planned.out, w.dtype), ref, w.dtype, f"planned decode {w.name} P={P}")


@pytest.mark.parametrize("partition", [0, 256])
def test_planned_decode_matches_the_full_grid_mixed_lengths(partition):
    _planned_vs_plain(synth.config(3), partition)


def test_planned_decode_with_fused_append_and_empty_sequences():
    w = synth.custom(seed=91, dtype="bf16", num_heads=16, num_kv_heads=4, head_dim=128, block_size=16,
                     seq_lens=[1, 4096, 2, 1024, 1025, 3000, 17], pool_factor=1.3)
    _planned_vs_plain(w, 1024, append=True)
    _planned_vs_plain(w, 512)
    # zero-length sequences: planned partition 0 still writes their zeros
    import torch
    from paged_kv_cache_326_amd import pa

    wz = synth.custom(seed=92, dtype="f16", num_heads=8, num_kv_heads=2, head_dim=64, block_size=16,
                      seq_lens=[1, 700, 3, 33], pool_factor=1.2)
    gz = harness.GpuWorkload(wz)
    gz.append()
    _, kc, vc, _ = harness.oracle_step(wz, seqs=[])
    lens = wz.seq_lens.copy()
    lens[0] = 0
    lens[2] = 0
    gz.seq_lens.copy_(gz.seq_lens.new_tensor(lens))
    gz.out.fill_(float("nan"))
    pa.pa_decode_run(gz.out, gz.query, gz.key_cache, gz.value_cache, gz.block_tables, gz.seq_lens, wz.scale,
                     wz.max_seq_len, partition_size=256, work=pa.decode_plan(lens, wz.max_seq_len, 256))
    _sync()
    got = _as64(gz.out, wz.dtype)
    assert np.all(got[0] == 0) and np.all(got[2] == 0)
    ref = oracle.decode_attention(oracle.to_float64(wz.query, wz.dtype), kc, vc, wz.block_tables, lens, wz.scale)
    _assert_close(got, ref, wz.dtype, "planned decode with zero-length sequences")


@pytest.mark.parametrize("num_seqs", [64, 65])
def test_decode_device_order_covers_every_partition(num_seqs):
    # Without a host plan, batches of at most 64 sequences take their units
    # in a longest-first order computed by every workgroup on the device (65
    # sequences keep the full grid).  Lengths hit the cases of that order:
    # empty sequences, exact multiples of the partition (no partial unit),
    # one token past one, single-partition sequences, several full
    # partitions, and the eighths the partial units are ordered by.
    rng = np.random.default_rng(num_seqs)
    P = 32
    special = [0, 1, P - 1, P, P + 1, 2 * P, 2 * P + 1, 5 * P, 5 * P + 7, 8, P // 8, P // 8 + 1, 0, 3 * P - 1]
    lens = special + list(rng.integers(1, 6 * P, num_seqs - len(special)))
    w = synth.custom(seed=300 + num_seqs, dtype="f16", num_heads=8, num_kv_heads=2, head_dim=64, block_size=16,
                     seq_lens=[max(int(x), 1) for x in lens], pool_factor=1.3)
    gw = harness.GpuWorkload(w)
    gw.append()
    _, kc, vc, _ = harness.oracle_step(w, seqs=[])
    import torch
    from paged_kv_cache_326_amd import pa

    lens = np.asarray([int(x) for x in lens], dtype=np.int32)
    gw.seq_lens.copy_(torch.from_numpy(lens).to(gw.seq_lens.device))
    gw.out.fill_(float("nan"))
    pa.pa_decode_run(gw.out, gw.query, gw.key_cache, gw.value_cache, gw.block_tables, gw.seq_lens, w.scale,
                     w.max_seq_len, partition_size=P)
    _sync()
    got = _as64(gw.out, w.dtype)
    assert np.all(got[lens == 0] == 0)
    ref = oracle.decode_attention(oracle.to_float64(w.query, w.dtype), kc, vc, w.block_tables, lens, w.scale)
    _assert_close(got, ref, w.dtype, f"device-ordered decode, {num_seqs} sequences")


@pytest.mark.parametrize("num_seqs", [17, 64])
def test_decode_device_order_unit_bound_is_tight(num_seqs):
    # Workgroups whose rank is at least the batch size first test it against
    # a bound on the unit count, (sum of max(L, 1) + n (P - 1)) // P, and
    # leave when past it.  With every length k P + 1 (or 0) the bound equals
    # the count, so the last unit's workgroups sit right below it; 17
    # sequences also take the lengths past the last whole 16.
    rng = np.random.default_rng(500 + num_seqs)
    P = 32
    lens = np.asarray([int(k) * P + 1 for k in rng.integers(0, 7, num_seqs)], dtype=np.int32)
    lens[0] = 6 * P + 1
    lens[3] = 0
    lens[-1] = 0
    units = int(sum(max(1, -(-int(L) // P)) for L in lens))
    assert (int(np.maximum(lens, 1).sum()) + num_seqs * (P - 1)) // P == units
    w = synth.custom(seed=500 + num_seqs, dtype="bf16", num_heads=8, num_kv_heads=2, head_dim=64, block_size=16,
                     seq_lens=[max(int(x), 1) for x in lens], pool_factor=1.2)
    gw = harness.GpuWorkload(w)
    gw.append()
    _, kc, vc, _ = harness.oracle_step(w, seqs=[])
    import torch
    from paged_kv_cache_326_amd import pa

    gw.seq_lens.copy_(torch.from_numpy(lens).to(gw.seq_lens.device))
    gw.out.fill_(float("nan"))
    pa.pa_decode_run(gw.out, gw.query, gw.key_cache, gw.value_cache, gw.block_tables, gw.seq_lens, w.scale,
                     w.max_seq_len, partition_size=P)
    _sync()
    got = _as64(gw.out, w.dtype)
    assert np.all(got[lens == 0] == 0)
    ref = oracle.decode_attention(oracle.to_float64(w.query, w.dtype), kc, vc, w.block_tables, lens, w.scale)
    _assert_close(got, ref, w.dtype, f"device-ordered decode at the unit bound, {num_seqs} sequences")


@pytest.mark.parametrize("partition", [16, 32, 0])
def test_decode_tiny_config_partitions(partition):
    w = synth.config(1)
    gw = harness.GpuWorkload(w)
    out = gw.step(partition_size=partition)
    _sync()
    _, _, _, ref = harness.oracle_step(w)
    _assert_close(_as64(out, w.dtype), ref, w.dtype, f"config 1 P={partition}")


SHAPES = [(dt, D, B, G) for dt in ("f32", "f16", "bf16") for D in (64, 128) for B in (16, 32) for G in (1, 2, 4, 8)]


@pytest.mark.parametrize("dt,D,B,G", SHAPES)
def test_decode_shapes_and_ragged_lengths(dt, D, B, G):
    Hkv = 2
    lens = [1, B - 1, B, B + 1, 3 * B + 5, 200, 7 * B]
    w = synth.custom(seed=D * 1000 + B * 10 + G, dtype=dt, num_heads=G * Hkv, num_kv_heads=Hkv, head_dim=D,
                     block_size=B, seq_lens=lens, pool_factor=1.5, max_blocks_per_seq=16)
    gw = harness.GpuWorkload(w)
    gw.slots()
    gw.scatter()
    _, kc, vc, _ = harness.oracle_step(w, seqs=[])
    for P in (B, 4 * B, 0):
        out = gw.decode(partition_size=P)
        _sync()
        ref = oracle.decode_attention(oracle.to_float64(w.query, dt), kc, vc, w.block_tables, w.seq_lens, w.scale)
        _assert_close(_as64(out, dt), ref, dt, f"{dt} D{D} B{B} G{G} P{P}")


def test_decode_zero_length_sequence_gives_zeros():
    w = synth.custom(seed=3, dtype="f16", num_heads=8, num_kv_heads=2, head_dim=128, block_size=16,
                     seq_lens=[40, 1, 700, 3], pool_factor=1.2)
    gw = harness.GpuWorkload(w)
    gw.slots()
    gw.scatter()
    _, kc, vc, _ = harness.oracle_step(w, seqs=[])
    lens = w.seq_lens.copy()
    lens[1] = 0
    lens[3] = 0
    gw.seq_lens.copy_(gw.seq_lens.new_tensor(lens))
    for P in (16, 0):
        out = gw.decode(partition_size=P)
        _sync()
        got = _as64(out, w.dtype)
        assert np.all(got[1] == 0) and np.all(got[3] == 0)
        ref = oracle.decode_attention(oracle.to_float64(w.query, w.dtype), kc, vc, w.block_tables, lens, w.scale)
        _assert_close(got, ref, w.dtype, f"zero-length P={P}")


def test_decode_max_length_sequence():
    # A sequence that fills its whole table row, longer than the largest partition.
    B = 16
    w = synth.custom(seed=9, dtype="bf16", num_heads=32, num_kv_heads=8, head_dim=128, block_size=B,
                     seq_lens=[8192, 8000, 17], max_blocks_per_seq=512)
    gw = harness.GpuWorkload(w)
    out = gw.step()
    _sync()
    _, _, _, ref = harness.oracle_step(w)
    _assert_close(_as64(out, w.dtype), ref, w.dtype, "max-length")


@pytest.mark.parametrize("partition", [0, 1024])
def test_decode_long_context_many_partitions(partition):
    # A 131 072-token context beside two short sequences: 32 (automatic) or
    # 128 partitions, ordered on the device, merged from that many partials.
    w = synth.custom(seed=13, dtype="f16", num_heads=32, num_kv_heads=8, head_dim=128, block_size=16,
                     seq_lens=[131072, 300, 1], pool_factor=1.0, poison_unused=False)
    gw = harness.GpuWorkload(w)
    out = gw.step(partition_size=partition)
    _sync()
    _, _, _, ref = harness.oracle_step(w)
    _assert_close(_as64(out, w.dtype), ref, w.dtype, f"131072-token context, partition {partition}")


def _relabel(w, seed):
    rng = np.random.default_rng(seed)
    perm = rng.permutation(w.num_blocks)
    kc = np.empty_like(w.key_cache)
    vc = np.empty_like(w.value_cache)
    kc[perm] = w.key_cache
    vc[perm] = w.value_cache
    import dataclasses

    return dataclasses.replace(w, key_cache=kc, value_cache=vc, block_tables=perm[w.block_tables].astype(np.int32))


def test_decode_bit_identical_under_block_permutation():
    w = synth.config(3, scale_down=4)
    a = harness.GpuWorkload(w).step()
    b = harness.GpuWorkload(_relabel(w, 5)).step()
    c = harness.GpuWorkload(synth.identity_tables(w)).step()
    _sync()
    ha, hb, hc = (harness.from_device(t, w.dtype) for t in (a, b, c))
    assert np.array_equal(ha.view(np.uint8), hb.view(np.uint8))
    assert np.array_equal(ha.view(np.uint8), hc.view(np.uint8))


def test_decode_shared_prefix_bit_identical_to_private_copies():
    import dataclasses

    w = synth.config(4)
    B = w.block_size
    nb = oracle.blocks_needed(int(w.seq_lens[0]), B)
    S = w.num_seqs
    kc = np.concatenate([w.key_cache[w.block_tables[s, :nb]] for s in range(S)])
    vc = np.concatenate([w.value_cache[w.block_tables[s, :nb]] for s in range(S)])
    priv = dataclasses.replace(w, key_cache=kc, value_cache=vc, num_blocks=S * nb,
                               block_tables=np.arange(S * nb, dtype=np.int32).reshape(S, nb),
                               refcounts=np.ones(S * nb, np.int32))
    # The shared pool gets the new tokens once per sample (private tail blocks),
    # exactly as in the private layout.
    a = harness.GpuWorkload(w).step()
    b = harness.GpuWorkload(priv).step()
    _sync()
    assert np.array_equal(harness.from_device(a, w.dtype).view(np.uint8), harness.from_device(b, w.dtype).view(np.uint8))


@pytest.mark.parametrize("dt", ["f32", "f16", "bf16"])
@pytest.mark.parametrize("slope", [0.02, 0.15, 1.5])
@pytest.mark.parametrize("partition", [0, 512])
def test_decode_growing_logits(dt, slope, partition):
    # Logits rise along the tokens: per 32-token step by less than the lazy
    # rescale threshold (the reference maximum stays, probabilities grow
    # towards 2^8), by about it, and by far more (a rescale every step);
    # with 512-token partitions the split partials carry stale references.
    w = synth.custom(seed=21, dtype=dt, num_heads=16, num_kv_heads=2, head_dim=128, block_size=16,
                     seq_lens=[40, 700, 3000])
    w = harness.ramped_keys(w, slope / w.scale, seed=5)
    gw = harness.GpuWorkload(w)
    out = gw.step(partition_size=partition)
    _sync()
    _, _, _, ref = harness.oracle_step(w)
    _assert_close(_as64(out, w.dtype), ref, w.dtype, f"decode {dt} ramp {slope} P={partition}")


@pytest.mark.parametrize("dt,G,P", [("f16", 8, 0), ("bf16", 4, 32), ("f32", 2, 16)])
def test_decode_skips_table_entries_outside_the_pool(dt, G, P):
    # The library skips a table entry outside [0, num_blocks): its positions
    # hold no key.  Entries -1 and num_blocks + 3 are planted after the step's
    # tokens are written (one sequence loses every block); the oracle drops
    # the same keys.  Missing blocks' slots are NaN-poisoned in the pool, so a
    # kernel that read them would fail.
    import torch

    w = synth.custom(seed=41, dtype=dt, num_heads=2 * G, num_kv_heads=2, head_dim=128, block_size=16,
                     seq_lens=[70, 300, 33, 129], pool_factor=1.5)
    gw = harness.GpuWorkload(w)
    gw.slots()
    gw.scatter()
    _, kc, vc, _ = harness.oracle_step(w, seqs=[])
    tables = w.block_tables.copy()
    tables[0, 1] = -1
    tables[1, 2] = w.num_blocks + 3
    tables[1, 10] = -7
    tables[2, :3] = -1
    tables[3, 8] = -1  # the last (one-token) block
    gw.block_tables = torch.from_numpy(tables).cuda()
    out = gw.decode(partition_size=P)
    _sync()
    q = oracle.to_float64(w.query, dt)
    ref = oracle.decode_attention(q, kc, vc, tables, w.seq_lens, w.scale, drop_missing_blocks=True)
    got = _as64(out, dt)
    assert (got[2] == 0).all()
    _assert_close(got, ref, dt, f"decode with missing blocks {dt} G={G} P={P}")
