"""CPU oracle for paged KV-cache attention.

TEST INFRASTRUCTURE, NOT PRODUCT CODE.  This package is a plain, slow,
deliberately obvious CPU statement of what the paged-attention path
computes.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import it.  The HIP library under
``paged_kv_cache_plan_amd/`` never imports, links or calls anything here,
and nothing here imports that package: the two share no code, no constants
and no helpers.  The only module both sides use is ``workloads`` (seeded
synthetic inputs, which holds none of the method's arithmetic).

Sources.  Three web pages describe the method; every function cites the
page title and the section it follows:

* "Deep Dive - FlashInfer" (leetllm.com) -- worked 3-request example,
  length contract, bottom-right causal mask, base-2 state merge, plan/run.
* "FlashInfer 中的 KV-Cache 布局" (KV-Cache layouts, docs.flashinfer.cn) --
  ragged tensors, CSR page table, NHD/HND shapes, MLA paged cache.
* "GPU attention backends: FlashInfer and FlashAttention" (mini-sglang from
  Scratch, Stage 4) -- page-size-1 token tables and page-number tables.

Modules
-------
metadata   plain-int metadata: lengths, validation, addresses, mask, append
           slot map, token-table -> page-table conversion.
planner    the work-partition specification (our reading; the pages give the
           trade-offs but no algorithm).
attention  numpy float64 paged attention (GQA, NHD/HND, causal) and MLA.
merge      base-2 log-sum-exp state merge, pairwise and multi-way.
cascade    multi-level cascade attention: per-level states over one paged
           cache, merged per query row.
mask       ragged KV and the 2-D ragged custom mask (offsets, little-endian
           bit packing, attention over ragged keys).
brute      pure-Python ``math`` attention for tiny inputs; pins ``attention``.

Pin status (see the tests under ``tests/test_oracle_*.py``): every function
here is pinned by values the pages print, closed forms, invariants, brute
force or an independent library routine (torch SDPA in float64), except
where a docstring says "parity unpinned".
"""
