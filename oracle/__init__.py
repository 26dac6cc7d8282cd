"""Plain CPU oracle for the FP4 KV-cache decode path.

TEST INFRASTRUCTURE ONLY. This package is imported by ``tests/``, by
``__graft_entry__.smoke()`` and by the CPU-baseline leg of ``bench.py``.
The product path (``fp4_kv_cache_amd`` and its HIP library) never imports,
calls or links anything here, and nothing here imports the product path.
The only module both sides share is the seeded input generator
``fp4_kv_cache_amd.workloads``, which holds random draws and shapes only.

Sources cited throughout (by page title and section):

* [Abstract] "BitDecoding-FP4: Native FP4 KV Cache Decoding via
  Algorithm-System Co-Design", section "Article Summary" (the arXiv abstract).
* [Blog/New] "FP4 KV Cache Done Right: What BitDecoding-FP4 Changes for
  Long-Context Serving", section "What is actually new in BitDecoding-FP4?".
* [Blog/Why] same page, section "Why does the KV cache matter so much for
  long-context serving?".
* [Explainer/Analyse] "BitDecoding-FP4 : décodage natif du KV cache FP4",
  section "Analyse approfondie".
* [Explainer/Contexte] same page, section "Contexte".
* [Editorial/Three] "BitDecoding-FP4 tests native 4-bit attention for long
  contexts", section "How BitDecoding-FP4 addresses three errors".
* [OCP-MX] OCP Microscaling Formats (MX) Specification v1.0 (E2M1 element,
  E8M0 shared scale, 32-element blocks) -- public spec the pages name by
  format only.
* [OCP-FP8] OCP 8-bit Floating Point Specification (E4M3 "FN" variant).
* [NVFP4] NVIDIA's public NVFP4 description: 16-element blocks, E4M3 block
  scale, one FP32 per-tensor scale.

The pages give the method's steps in prose only; every place where they
leave a step open is resolved by a stated reading (R-numbers in the
docstrings), collected in the repository's design notes.

Parity status per function is stated in each module header.  Every public
function is pinned by at least one ``-m "not gpu"`` test against the
mathematics or the formats' definitions, except where a header says
"parity unpinned".
"""
