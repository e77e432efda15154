"""Oracle: a plain, slow CPU definition of the hybrid compressed attention path.

TEST INFRASTRUCTURE ONLY. Nothing on the product path may import, call or link
this package: only the test suite, the smoke check of the graft entry point and
the ``cpu_baseline`` leg of the benchmark use it. It shares no code with the
HIP library and does not import it.

Arithmetic is numpy float64. Where a floating-point value decides an integer
(a quantised code, a top-k membership) the decision is taken on the float32
value, which is the precision the kernels take it in.

Sources (web pages; cited by site, title and section):

* [webconsulting] webconsulting.at, "DeepSeek V4-Pro: Architektur,
  KV-Cache-Kompression und Hyper-Connections im Detail", sections
  "Das Wichtigste" and "Kompression und Selektion".
* [framia] framia.pro, "DeepSeek V4 Modellarchitektur: Hybrid Attention, mHC
  und MoE erklärt", section "2. Hybrid Attention Architektur: CSA + HCA".
* [chaosnode] chaosnode.de, "DeepSeek-V4: 1 Million Token Context endlich
  nutzbar", section "Hybrid Attention: CSA und HCA".
* [golem] golem.de, "Chinas KI-Unabhängigkeit?: Bei Deepseek V4 haben kleine
  Änderungen große Wirkung", sections "Komprimierte Erinnerung für längere
  Kontexte" and the introduction (MXFP4).
* Number formats follow the public OCP specifications: "OCP 8-bit Floating
  Point Specification (OFP8)" rev 1.0 (E4M3) and "OCP Microscaling Formats (MX)
  Specification" v1.0 (E2M1 elements, E8M0 shared scale, section 6.3 scale
  rule). The pages name FP8, BF16, FP4 and MXFP4 but do not define them.

Parity status of each function is stated in its module. The indexer score
formula (``indexer.index_scores``) is a reading: the pages say only that a
learned low-precision indexer scores compressed entries per query and keeps the
top k. Its implementation is pinned (brute force, exact integer dot products),
but the formula itself is not fixed by the pages.
"""

from . import formats, rope, compress, indexer, attention, model  # noqa: F401
