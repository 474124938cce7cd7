"""CPU oracle for paged-attention decode, chunked prefill and the KV-cache
scatter.  TEST INFRASTRUCTURE ONLY: the test suite, the smoke check and the
benchmark's CPU-baseline leg may import it; the product path never does.

It is a plain, slow, obviously correct float64 implementation of what the
paged path computes: gather each sequence's K/V through its block table into
contiguous arrays, then run dense softmax attention.  It shares no code with
the HIP library or its binding; the only module both sides use is the seeded
input generator (``paged_kv_cache_326_amd.synth``), which holds none of the
method's arithmetic.

Sources (web pages on paged KV caches):
  [P1] "大模型推理内存优化从 KV Cache 分页到连续批处理的工程实践"
       (seekfood.cn/news/1660747)
  [P2] "KV Cache管理优化：大模型推理显存瓶颈突破"
       (intelliparadigm.com/article/weixin_33178839/2255646)
  [P3] "大语言模型KV Cache内存优化与PagedAttention实践"
       (intelliparadigm.com/article/weixin_30558697/2223113)

Pins (tests/test_oracle_*.py, run with ``-m "not gpu"``):
  kv_cache_bytes       the worked LLaMA-2-70B values printed on [P1]
  preallocation_waste  the waste percentages printed on [P1] for requests
                       against a 4096-slot reservation, and the overflow
  paged_waste          brute force: at most one partly filled block
  blocks_needed        brute-force count of distinct blocks touched
  slot_mapping         brute-force page-table walk + injectivity/ordering
  reshape_and_cache    round trip, untouched-slot sentinel, skip/duplicate rules
  decode_attention     torch SDPA (float64) on an identity-layout pool, closed
                       forms, block-permutation and shared-prefix invariance;
                       with drop_missing_blocks, SDPA over the dense K/V with
                       the missing blocks' rows deleted by index
  prefill_attention    torch SDPA causal / explicit-mask special cases, the
                       same with missing blocks (mask built from positions),
                       a row that sees no present key -> zeros, a row that
                       sees one key -> that key's value
  copy_blocks          hand-built pools whose values name block and position:
                       destination = old source, sources and bystanders
                       untouched, one source to several destinations,
                       repeated or aliased destinations refused with the
                       pool intact, out-of-pool and src == dst pairs skipped
  gather_blocks        rows in id order, out-of-pool rows untouched
  scatter_blocks       only the named blocks written, repeated id refused,
                       gather -> wipe -> scatter restores the pool, swap out,
                       swap in elsewhere and copy back lands the bytes
  BlockPoolModel       FIFO order and conservation of blocks, reference
                       counts under sharing, brute-force block counts; the
                       prefix cache against the page's shared-system-prompt
                       claims, and a prompt of whole cached blocks keeping
                       its last block private
  SchedulerModel       hand-worked iterations of the three scheduling steps
                       (admission, head-of-line wait, preemption, release),
                       conservation, batch limit and block-need invariants,
                       a forked request's copy-on-write pair worked by hand
  fp8 (E4M3 codes)     torch float8_e4m3fn values and rounding, hand-worked
                       values, exact midpoints, brute-force nearest,
                       saturation and quantisation error bounds
Every function above has at least one pin that does not come from the
oracle itself; none is "parity unpinned".
"""

from .storage import to_float64, round_to_storage  # noqa: F401
from .paging import (  # noqa: F401
    blocks_needed,
    kv_cache_bytes,
    preallocation_waste,
    paged_waste,
    slot_mapping,
    reshape_and_cache,
    gather_kv,
    key_rows,
    key_tiles,
)
from .attention import decode_attention, prefill_attention  # noqa: F401
from .block_pool import BlockPoolModel, NoBlocks, copy_blocks, gather_blocks, scatter_blocks  # noqa: F401
from .scheduler import SchedulerModel  # noqa: F401
from .fp8 import (  # noqa: F401
    FP8_MAX,
    E4M3_VALUES,
    fp8_value,
    fp8_encode,
    fp8_quantize,
    fp8_dequantize,
    reshape_and_cache_fp8,
)
