"""PA_DEBUG=1 on the GPU: the binding checks the device-resident contents on
the host before each launch.  Valid contents give the same bytes as without
the checks; a bad block id, an over-long chunk or a repeated slot raises
ValueError and launches nothing (the output keeps its sentinel)."""

import numpy as np
import pytest

from paged_kv_cache_326_amd import pa, synth
from tests import harness

pytestmark = pytest.mark.gpu


def _workload(chunks=True):
    return synth.custom(seed=11, dtype="bf16", num_heads=16, num_kv_heads=2, head_dim=128, block_size=16,
                        seq_lens=[70, 33], q_lens=[20, 9] if chunks else None, pool_factor=1.2)


@pytest.mark.parametrize("chunks", [True, False], ids=["prefill", "decode"])
def test_debug_checks_pass_valid_contents_unchanged(monkeypatch, chunks):
    import torch

    w = _workload(chunks)
    outs = []
    for flag in ("0", "1"):
        monkeypatch.setenv("PA_DEBUG", flag)
        g = harness.GpuWorkload(w)
        g.append()
        out = g.prefill() if chunks else g.decode()
        torch.cuda.synchronize()
        outs.append(harness.from_device(out, w.dtype).copy())
    assert np.array_equal(outs[0].view(np.uint8), outs[1].view(np.uint8))


def test_debug_checks_reject_bad_contents_before_launch(monkeypatch):
    import torch

    wd, w = _workload(False), _workload(True)
    gd, g = harness.GpuWorkload(wd), harness.GpuWorkload(w)
    gd.append()
    g.append()
    torch.cuda.synchronize()
    monkeypatch.setenv("PA_DEBUG", "1")
    for x in (gd, g):
        x.out.fill_(7.0)
    sentinels = (gd.out.clone(), g.out.clone())

    bad = gd.block_tables.clone()
    bad[1, 0] = wd.num_blocks  # the first block sequence 1 reads
    with pytest.raises(ValueError, match=r"block_tables\[1\]\[0\]"):
        pa.pa_decode(gd.out, gd.query, gd.key_cache, gd.value_cache, bad, gd.seq_lens, wd.scale, wd.max_seq_len)
    with pytest.raises(ValueError, match="more than max_q_len"):
        g.prefill(max_q_len=int(w.q_lens.max()) - 1)
    torch.cuda.synchronize()
    assert torch.equal(gd.out, sentinels[0]) and torch.equal(g.out, sentinels[1])

    slots = g.slot_mapping.clone()
    slots[1] = slots[0]
    kc = g.key_cache.clone()
    with pytest.raises(ValueError, match="written by two tokens"):
        pa.pa_reshape_and_cache(g.key_cache, g.value_cache, g.new_key, g.new_value, slots)
    torch.cuda.synchronize()
    assert torch.equal(g.key_cache.view(torch.int16), kc.view(torch.int16))  # bytes: the pool holds NaN poison
