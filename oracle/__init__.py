"""Plain, slow CPU oracle for the MoonEP data-parallel hot path.

TEST INFRASTRUCTURE ONLY.  Nothing in the product path may import, call or
link this package: only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` use it.  It shares no code, table or
helper with the HIP library in ``moe_expert_load_amd/``; the only thing both
sides consume is the seeded input generator in ``workloads/``.

Sources (the pages this oracle is written from):

* [K3-blog] "Kimi K3 模型结构（8）：训练并行，MoonEP 与四类等待"
  (blog.javazero.top) -- headings "MoonEP：从「完全平衡」这个目标出发",
  "定理 1", "定理 2", "在线规划、零拷贝、静态 shape", "rank 内部".
* [MoonEP-news] "Moonshot AI 开源 MoonEP：为 MoE 训练打造的完美均衡专家并行库"
  (feinterview) -- sections "MoonEP 针对的问题" (maxvio), "核心思想：动态冗余专家"
  (the [E+B, H, H'] weight contract, cu_seqlens, prefetch_weight, reduce_grad,
  B policy).
* [MoonEP-fr] "MoonEP : l'équilibrage parfait" (mkdocs.reaper.mx) -- "Le
  théorème" (Théorème 1 and its lemma, Théorème 2), "La planification en
  ligne" (offline ILP as the yardstick).
* [TSR] "TRAINING_SYSTEMS_RESEARCH" (llm-atlas), the page titled
  "大规模 LLM 训练系统研究账本" -- §6.1 (router -> dispatch -> expert GEMM ->
  combine -> weighted sum), §6.4 (proof structure) and §9.5 (the MoE
  backward stays on the permuted layout; dispatch is redone to restore the
  GEMM input).

Modules:

* :mod:`oracle.bf16`     -- bf16 round-to-nearest-even from its definition.
* :mod:`oracle.plan`     -- histogram, stable slot ranks, the deterministic
  Theorem-1 construction, cu_seqlens and the route map.
* :mod:`oracle.dataflow` -- dispatch, prefetch, grouped GEMM, combine,
  weight-grad GEMM and reduce_grad, and the data backward (combine_backward,
  dgrad, dispatch_backward), in float64.
* :mod:`oracle.swiglu`   -- the two-projection SwiGLU expert: first
  projection fused with the activation, and the activation's backward.
* :mod:`oracle.optimum`  -- minimum achievable max-redundancy on tiny inputs
  (brute force with a Hall-condition feasibility test, and a SciPy MILP), the
  per-rank lower bound and the Theorem-2 bound.
* :mod:`oracle.metrics`  -- maxvio.

Parity status of each function is stated in its docstring; every function
here is pinned by a ``-m "not gpu"`` test in ``tests/test_oracle_*.py``.
"""
