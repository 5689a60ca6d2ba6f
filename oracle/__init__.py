"""CPU oracle for paged decode attention — TEST INFRASTRUCTURE ONLY.

This package is the slow, plain, obviously-correct statement of what the paged
decode path computes.  It exists to check the HIP library, never to stand in for
it: only the test suite, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg
of ``bench.py`` may import it.  The product path (``paged_kv_cache_355_amd``)
never imports, links or calls anything here, and this package never imports the
product path.  The two share nothing except the seeded input generators in
``workloads/``, which hold none of the method's arithmetic.

Pages cited (titles as printed; a citation names the page key and the section):

* [P1] "Paged Attention：大模型推理显存优化的核心方案" (learnblockchain.cn,
  a translated article).  Sections are its headings: "KV Cache 快速回顾",
  "内存浪费的两种形式", "Paged Attention 的工作原理" (the worked example),
  "块表（Block Table）", "为什么 Paged Attention 如此高效",
  "跨请求的内存共享".
* [P2] "PagedAttention：操作系统级 KV 缓存虚拟内存管理" (freeguideonline.com
  tutorial).  Numbered sections §1.1 (the attention formula) … §8.
* [P3] "PagedAttention 和 vLLM" (aiunderstanding.org).  Sections "深入探讨",
  "技术洞察".

Modules:

* ``numerics``      — exact storage-dtype → float64 decoding (fp32/fp16/bf16).
* ``block_manager`` — FIFO free list, refcounts, fork, copy-on-write, slots.
* ``kv_ops``        — bitwise slot-mapped KV write and block copy.
* ``attention``     — paged single-query decode attention in float64.
* ``accounting``    — memory-utilisation accounting (paged vs contiguous).

Parity status: every function here is pinned by ``tests/test_oracle_*.py``
against values the pages print, closed forms, library special cases and brute
force; none is "parity unpinned".
"""
