"""Oracle: a plain, slow, fp64 CPU implementation of the paged KV-cache hot path.

TEST INFRASTRUCTURE ONLY.  Nothing in the product (``paged_kv_cache_134_amd``)
may import, call or execute anything in this package; only ``tests/``,
``__graft_entry__.smoke()`` and ``bench.py``'s CPU-baseline leg use it.  It
shares no code with the HIP path: it is NumPy only and imports nothing from
the product package.

Sources (web pages, cited by title and section):

* [k4i]    "Paged attention" post, k4i.top -- sections "block table"
  (#the-block-table), "block manager" (#the-block-manager), "attention over
  non-contiguous blocks" (#paged-attention-kernel), "copy-on-write" (#cow),
  "prefix caching" (#prefix-caching), "memory utilization".
* [vllm]   "PagedAttention 在 vLLM 中的实现分析" (blog.chen3feng.top) -- §3.1
  block table, §3.2 slot mapping, §3.3 KV cache layout, §4.1 block pool data
  structures, §5.4 CommonAttentionMetadata, §6.2 forward, §6.3 cache update,
  §7.3 V1 vs V2, §7.4 cache-write kernel.
* [atb]    ATB "PagedAttention + virtual memory" article (2048ai.net) --
  reference counting and copy-on-write sections.
* [tut]    vLLM long-sequence guide, ch. 3 "PagedAttention原理" -- §3.3.2
  allocation and release, §3.4 (paging leaves the attention math unchanged).
* [packed] cann-recipes-infer Paged KV Cache + Packed Sequence notes
  (m.xxqk.cn) -- §2.3 packed sequences, §3.2 packed index.

Modules
-------
``attention``  cache write, per-token gather, decode and causal packed
               prefill as plain definitions, plus the block-wise online-softmax
               and split-K merge written out as cross-checks.
``fp8``        FP8 (OCP E4M3) KV cache: code table, quantising write
               (x / scale in fp32, nearest with ties to even, saturated) and
               read-back (code value times scale).
``allocator``  step-by-step block-manager model (free queue, reference counts,
               fork, append with copy-on-write, free).
``state``      derives block tables, slot mappings and the host pool of a
               seeded workload with the two modules above.

Every function here is pinned by ``tests/test_oracle_*.py`` against worked
examples printed on the pages, closed forms, invariants or brute force.
"""
from .attention import (  # noqa: F401
    attention_dense, bits_to_f64, decode_ref, gather_seq, merge_partitions,
    online_softmax_blocks, partition_stats, prefill_ref, write_ref, write_ref_fp8, NHD, HND,
)
from .allocator import BlockManagerModel, OutOfBlocks  # noqa: F401
