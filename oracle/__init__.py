"""CPU oracle for the paged decode hot path -- TEST INFRASTRUCTURE ONLY.

A plain, slow, obviously-correct implementation of what the path computes,
written from the pages' definitions.  Only ``tests/``,
``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of ``bench.py`` may
import it.  It shares no code with the HIP library (``paged_attention_slot_amd``)
and never imports it; the product path never imports this package.

Floating point is evaluated in float64 from the exact stored input bits.

Pages cited (titles as they appear on each page):

* [KVM]  "19.2 KV Cache 系统化管理" -- book chapter, sections 19.2.1-19.2.6,
  figures 19-5..19-8, and the simplified implementation with its self-check in
  section 19.2.3.
* [KVX]  "KV Cache：长上下文为什么吃显存，PagedAttention 怎么救" -- explainer,
  numbered sections 00-07 (section 01: the new-token attention equation;
  section 02: memory formula and the GQA ratio).
* [SLOT] "推理与 KV Cache 02:分页、共享与回收如何协作" -- blog post; sections
  "从一个位置找到缓存块" (locate: logical block / offset equations, block-table
  example, token-slot equation), "按整块分配,会多占多少空间" (whole-block
  allocation table), "请求结束后,缓存会立刻消失吗" (release / refcounts).
* [PFX]  "学习大模型推理的显存优化：PagedAttention 与前缀缓存" -- blog post;
  sections "PagedAttention 原理" (principle) and "前缀缓存" (prefix).
* [ENG]  the PagedAttention engineering article served under the page title
  "企业官网建设流程全解析"; numbered sections 1.1-8.3.

Modules:
  block_manager  free list, refcounts, block tables, fork, prefix sharing, CoW
  cache_ops      slot-scatter write and whole-block copy
  attention      decode attention: plain definition, contiguous brute force,
                 block-wise online softmax, split-KV with log-sum-exp merge
  replay         drives a ``workloads.Workload`` through the above

Parity status: every function is pinned by ``tests/test_oracle_*.py``; none is
"parity unpinned".
"""
