"""The prepared calls (prepare_decode_append, prepare_append_kv) check their
arguments the way the plain calls do, once, before anything reaches the
library (CPU)."""

import pytest
import torch

from paged_kv_cache_326_amd import pa


def _args(device="cpu", new_rows=8):
    kc = torch.empty(pa.key_shape(4, 2, 16, 64, torch.float16), dtype=torch.float16, device=device)
    vc = torch.empty(pa.value_shape(kc.shape), dtype=torch.float16, device=device)
    q = torch.empty(3, 4, 64, dtype=torch.float16, device=device)
    return dict(out=torch.empty_like(q), query=q, key_cache=kc, value_cache=vc,
                new_key=torch.empty(3, 2, new_rows * 8, dtype=torch.float16, device=device),
                new_value=torch.empty(3, 2, new_rows * 8, dtype=torch.float16, device=device),
                block_tables=torch.zeros(3, 4, dtype=torch.int32, device=device),
                seq_lens=torch.ones(3, dtype=torch.int32, device=device), scale=0.125, max_seq_len=64)


def test_prepared_step_refuses_host_tensors():
    with pytest.raises(ValueError, match="must be a GPU tensor"):
        pa.prepare_decode_append(**_args())


def test_key_chunk_follows_the_element_size():
    # 64-byte key chunks: 16 float32, 32 float16 or bfloat16, 64 FP8 codes.
    for dt, kc in ((torch.float32, 16), (torch.float16, 32), (torch.bfloat16, 32), (torch.float8_e4m3fn, 64)):
        assert pa.key_shape(5, 2, 16, 128, dt) == (5, 2, 128 // kc, 16, kc)
    with pytest.raises(ValueError, match="not a multiple"):
        pa.key_shape(5, 2, 16, 48, torch.float16)


def test_prepared_append_refuses_host_tensors():
    a = _args()
    with pytest.raises(ValueError, match="must be a GPU tensor"):
        pa.prepare_append_kv(a["key_cache"], a["value_cache"], a["new_key"], a["new_value"], a["block_tables"],
                             a["seq_lens"], torch.zeros(4, dtype=torch.int32), 1)
