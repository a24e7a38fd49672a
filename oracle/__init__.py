"""Plain, slow, float64 CPU oracle for the rotated-basis ternary projection.

TEST INFRASTRUCTURE ONLY.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import or call anything in this
package.  The product (the HIP library and its Python binding) never routes
through it, and this package imports nothing from the product: the two share
no code, no tables and no helpers.

What it computes, and where the pages define it (page titles are given in
full once here and abbreviated below):

* [ninfer-skill]  "ninfer 三元制品：容器格式与几何" (ninfer ternary artifact:
  container format and geometry), jindage.com skill bonsaiGGUF2ninfer.
  §2 ternary numeric formats, §3 row-split plane geometry, §4 block <-> plane
  slices, §6 constants.
* [gguf-explainer]  "GGUF 完整讲解" (GGUF explained), huashanblogllm.xyz.
  §4.3 ternary restore (2-bit code semantics), §4.4 dot product identity.
* [ninfer-v3]  "artifact-container.md" (NInfer v3 artifact container).
  §6.1 numeric formats, §6.2 layouts, §8 ``hadamard_signs`` auxiliary.
* [tensorsharp]  "从 TensorSharp 视角解读 Ternary Bonsai 2 27B：当 1.72 比特的
  权重遇上 Hadamard 变换" (Ternary Bonsai 2 27B through TensorSharp's eyes),
  cloud.tencent.com article 2751622.  §4.2 transform contract, §4.4 network
  flow.

Modules:

* :mod:`oracle.geometry`   -- the 16-field row-split geometry record.
* :mod:`oracle.codec`      -- trit <-> byte encoders/decoders, plane packing.
* :mod:`oracle.transform`  -- dense Sylvester Hadamard, signed forward/inverse.
* :mod:`oracle.projection` -- dequantisation, float64 projection, embedding
  rows, and the acceptance bounds.

Parity status: every function here is pinned by a ``-m "not gpu"`` test to
values the pages print, closed forms, invariants, library routines or brute
force, except the PTQ1_0_G128 trit packing, whose bit order the pages do not
give: it follows this project's own documented convention and is pinned to
that convention (bijections and hand-computed bytes), not to the pages.
"""
